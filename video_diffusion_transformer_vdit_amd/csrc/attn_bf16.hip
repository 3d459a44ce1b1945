// bf16 flash-style attention forward for gfx950 (MI355X).
//
// Computes O = softmax(scale * Q K^T) V per (batch, head) without storing the
// S x S score matrix: the full spatiotemporal self-attention of a video DiT
// (VC-Attention article (aikraft.ru), section 01) with the FlashAttention
// tiling the FLOPS article (sudonull.com, "Optymalizacje") credits with
// removing the 75K x 75K matrix.
//
// Design (one workgroup = 8 waves = 256 queries, one workgroup per CU, so
// every SIMD runs two waves that share each K/V tile in LDS):
//  * Each wave owns 32 queries.  Its Q slice stays in registers for the whole
//    key loop as the B operand of v_mfma_f32_32x32x16_bf16.
//  * Scores are produced transposed, S^T = K Q^T, so lane (q, half) holds one
//    query and 16 keys of every 32-key block: row max / row sum are in-lane,
//    plus one v_permlane32_swap for the max.
//  * K/V tiles of 64 keys go straight from global memory to LDS
//    (global_load_lds_dwordx4, no register staging) into a two-deep ring; one
//    barrier per tile.  K is stored chunk-major ([16-byte chunk][key]), so the
//    K operand of every MFMA is one 16-byte read at a linear offset and
//    consecutive lanes read consecutive bytes.  V is stored row-major with
//    its 16-byte chunks XOR-swizzled (chunk ^ 4*(row & 3)) and read with
//    ds_read_b64_tr_b16, which hands each lane 4 keys of one channel; both
//    reads are free of bank conflicts.
//  * Software pipeline: while the exponentials of tile j are computed, the
//    MFMAs of S(j+1) = K(j+1) Q^T and of O^T += V(j)^T P(j)^T are in flight.
//  * Online softmax in the log2 domain with an integer running reference
//    m (ceil of the running maximum of scale*log2(e)*s): P = 2^(c s - m) <= 1,
//    and the accumulator is rescaled (by an exact power of two) only in the
//    rare tiles where some row's maximum exceeds its reference.  P is rounded
//    to bf16 once; the row sum adds exactly those rounded weights.
//  * Ragged tails: rows of the last K/V tile past S are read from row S-1
//    (finite data), scored -inf, and so weigh exactly 0; queries >= S are
//    computed on zeros and not stored.
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kWaves = 8;
constexpr int kBr = 32 * kWaves;       // queries per workgroup
constexpr int kBc = 64;                // keys per K/V tile
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerWave = 16 / kWaves;  // 1 KB DMA loads per wave per tile
constexpr int kRowBytes = kHeadDim * 2;
constexpr int kTileBytes = kBc * kRowBytes;  // 16 KB

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

__device__ __forceinline__ lds_void* lds_ptr(void* p) { return (lds_void*)p; }

// 8 keys x 1 channel for the V^T operand: two transposing 64-bit reads.
__device__ __forceinline__ bf16x8 read_v_operand(const char* p0, const char* p1) {
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  const s16x8_t v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(kThreads, 8 / kWaves) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, int S, int n_qtiles, float c) {
  // Four separate LDS objects (not one indexed array): the compiler can then
  // tell that a DMA into one buffer does not alias reads of the other, and
  // does not wait for the in-flight tile before reading the current one.
  __shared__ __attribute__((aligned(1024))) char lds_k0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[kTileBytes];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const size_t base = (size_t)bh * S * kHeadDim;
  const char* Kh = reinterpret_cast<const char*>(K + base);
  const char* Vh = reinterpret_cast<const char*>(V + base);
  uint16_t* Oh = O + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qt * kBr + wave * 32 + col;
  const int nkt = (S + kBc - 1) / kBc;
  const bool tail = (S % kBc) != 0;

  // ---- per-lane constant offsets ----
  // V loads: wave w, load i covers tile rows 8w + 4i + lane/16; lane writes
  // physical chunk lane%16 of its row, so it fetches the logical chunk that
  // the swizzle maps there.  K loads: load i of wave w fills chunk row
  // c = 2w + i (1 KB) with chunk c of all 64 keys (lane = key).
  const int lrow0 = 4 * kLoadsPerWave * wave + (lane >> 4);   // + 4i
  const int pchunk = lane & 15;
  int kgo[kLoadsPerWave], vgo[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int r = lrow0 + 4 * i;
    kgo[i] = lane * kRowBytes + 16 * (kLoadsPerWave * wave + i);
    vgo[i] = r * kRowBytes + 16 * (pchunk ^ (4 * (r & 3)));
  }
  // K operand: lane (key = 32kb + col, half) reads chunk 2kk + half of its key
  const int kbase = half * 1024 + col * 16;
  // V operand: 16-lane group g = lane/16, s = lane%16 reads row
  // 16kc + 8r + 4(g>>1) + s/4, channels 32mb + 16(g&1) + 4(s%4) .. +3.
  const int g = lane >> 4, s16 = lane & 15;
  const int vrow = 4 * (g >> 1) + (s16 >> 2);
  const int vx = 2 * (g & 1) + ((s16 >> 1) & 1);
  int voff[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
    voff[mb] = vrow * kRowBytes + 16 * (4 * (mb ^ (s16 >> 2)) + vx) + 8 * (s16 & 1);

  auto issue_k = [&](int t, char* buf) {
    const int key0 = t * kBc;
    const char* src = Kh + (size_t)key0 * kRowBytes;
    char* dst = buf + 4 * kLoadsPerWave * wave * kRowBytes;
    if (tail && t == nkt - 1) {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int row = min(key0 + lane, S - 1);
        const int go = (row - key0) * kRowBytes + 16 * (kLoadsPerWave * wave + i);
        __builtin_amdgcn_global_load_lds(src + go, lds_ptr(dst + i * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i)
        __builtin_amdgcn_global_load_lds(src + kgo[i], lds_ptr(dst + i * 1024), 16, 0, 0);
    }
  };
  auto issue_v = [&](int t, char* buf) {
    const int key0 = t * kBc;
    const char* src = Vh + (size_t)key0 * kRowBytes;
    char* dst = buf + 4 * kLoadsPerWave * wave * kRowBytes;
    if (tail && t == nkt - 1) {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int r = lrow0 + 4 * i;
        const int row = min(key0 + r, S - 1);
        const int go = (row - key0) * kRowBytes + 16 * (pchunk ^ (4 * (r & 3)));
        __builtin_amdgcn_global_load_lds(src + go, lds_ptr(dst + i * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i)
        __builtin_amdgcn_global_load_lds(src + vgo[i], lds_ptr(dst + i * 1024), 16, 0, 0);
    }
  };

  // ---- Q operand (registers for the whole loop) ----
  bf16x8 qf[8];
  {
    const uint16_t* Qr = Q + base + (size_t)min(qrow, S - 1) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 w = *reinterpret_cast<const u32x4*>(Qr + 16 * kk + 8 * half);
      if (qrow >= S) w = u32x4{0u, 0u, 0u, 0u};
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  auto qk = [&](const char* Kb, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + 2048 * kk + 512 * kb + kbase);
        s[kb] = mfma32x32x16_bf16(a, qf[kk], s[kb]);
      }
  };
  auto mask_tail = [&](int t, f32x16* s) {
    // keeps the compiler from turning this once-per-workgroup branch into
    // selects executed on every tile
    asm volatile("" ::: "memory");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t * kBc + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key >= S) s[kb][i] = -INFINITY;
      }
  };

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_ref = -INFINITY;  // integer-valued log2-domain reference
  // this lane's share of the row sum, in four independent partial sums so
  // that the additions do not form one long dependency chain
  float l4[4] = {0.f, 0.f, 0.f, 0.f};

  // Row maximum of a score tile, reference update and (rare) rescale.
  auto update_max = [&](const f32x16* s) {
    // balanced tree over the 32 scores (depth 4 instead of a chain of 16)
    float t8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      t8[u] = fmaxf(fmaxf(s[u >> 2][4 * (u & 3)], s[u >> 2][4 * (u & 3) + 1]),
                    fmaxf(s[u >> 2][4 * (u & 3) + 2], s[u >> 2][4 * (u & 3) + 3]));
    const float mx = fmaxf(fmaxf(fmaxf(t8[0], t8[1]), fmaxf(t8[2], t8[3])),
                           fmaxf(fmaxf(t8[4], t8[5]), fmaxf(t8[6], t8[7])));
    const float mnew = max_halves(mx) * c;
    if (__ballot(mnew > m_ref) != 0ull) {
      // rare: keep it a real branch rather than 64 multiplies per tile
      asm volatile("" ::: "memory");
      const float mnext = mnew > m_ref ? ceilf(mnew) : m_ref;
      const float alpha = exp2_fast(m_ref - mnext);
#pragma unroll
      for (int u = 0; u < 4; ++u) l4[u] *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
      m_ref = mnext;
    }
  };

  // P = bf16(2^(c s - m)) packed in S^T register order; l += sum of P.
  auto softmax_p = [&](const f32x16* s, uint32_t (*pk)[8]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float p0 = exp2_fast(fmaf(s[kb][2 * p], c, -m_ref));
        const float p1 = exp2_fast(fmaf(s[kb][2 * p + 1], c, -m_ref));
        pk[kb][p] = pack_bf16x2(p0, p1);
        l4[p & 3] = sum_bf16x2(pk[kb][p], l4[p & 3]);
      }
  };

  // O^T += V^T P^T over four 16-key chunks (keys 16kc + 4half + {0..3} and
  // 16kc + 8 + 4half + {0..3}, matching the S^T register order of P).
  auto pv = [&](const char* Vb, uint32_t (*pk)[8]) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1, cc = kc & 1;
      const u32x4 pw = {pk[kb][4 * cc], pk[kb][4 * cc + 1], pk[kb][4 * cc + 2], pk[kb][4 * cc + 3]};
      const bf16x8 b = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const char* p0 = Vb + (16 * kc) * kRowBytes + voff[mb];
        const bf16x8 a = read_v_operand(p0, p0 + 8 * kRowBytes);
        acc[mb] = mfma32x32x16_bf16(a, b, acc[mb]);
      }
    }
  };

  auto wait_loads_and_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
  };

  // ---- prologue: K(0), V(0), K(1) in flight; S(0) ----
  issue_k(0, lds_k0);
  issue_v(0, lds_v0);
  if (nkt > 1) issue_k(1, lds_k1);
  wait_loads_and_sync();
  f32x16 s_cur[2];
  qk(lds_k0, s_cur);
  if (tail && nkt == 1) mask_tail(0, s_cur);
  update_max(s_cur);
  // every wave has read lds_k0 before anyone refills it
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();

  // One pipelined step for tile j (which has a successor): tile j+1's K is in
  // k_next, tile j's V in v_cur; V(j+1) goes to v_fill and K(j+2) to k_fill.
  // s_in holds S(j); S(j+1) is written to s_out (the two register sets swap
  // roles from one step to the next, so nothing is copied).
  auto step = [&](int j, const char* k_next, const char* v_cur, char* v_fill, char* k_fill,
                  f32x16* s_in, f32x16* s_out) {
    issue_v(j + 1, v_fill);
    if (j + 2 < nkt) issue_k(j + 2, k_fill);
    uint32_t pk[2][8];
    softmax_p(s_in, pk);
    qk(k_next, s_out);
    pv(v_cur, pk);
    if (tail && j + 2 == nkt) mask_tail(j + 1, s_out);
    update_max(s_out);
    wait_loads_and_sync();
  };

  // ---- main loop, unrolled by two so every LDS buffer and score register
  // set is named statically ----
  f32x16 s_alt[2];
  int j = 0;
  for (; j + 2 < nkt; j += 2) {
    step(j, lds_k1, lds_v0, lds_v1, lds_k0, s_cur, s_alt);
    step(j + 1, lds_k0, lds_v1, lds_v0, lds_k1, s_alt, s_cur);
  }
  bool in_alt = false;
  if (j + 1 < nkt) {
    step(j, lds_k1, lds_v0, lds_v1, lds_k0, s_cur, s_alt);
    in_alt = true;
    ++j;
  }

  // ---- last tile (j = nkt - 1); every register set is named statically ----
  auto last_tile = [&](const f32x16* s_last) {
    uint32_t pk[2][8];
    softmax_p(s_last, pk);
    if (j & 1)
      pv(lds_v1, pk);
    else
      pv(lds_v0, pk);
  };
  if (in_alt)
    last_tile(s_alt);
  else
    last_tile(s_cur);

  const float inv = 1.0f / sum_halves((l4[0] + l4[1]) + (l4[2] + l4[3]));
  if (qrow < S) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 w;
        w.x = pack_bf16x2(acc[mb][4 * gq] * inv, acc[mb][4 * gq + 1] * inv);
        w.y = pack_bf16x2(acc[mb][4 * gq + 2] * inv, acc[mb][4 * gq + 3] * inv);
        *reinterpret_cast<u32x2*>(Oh + (size_t)qrow * kHeadDim + 32 * mb + 8 * gq + 4 * half) = w;
      }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o,
                                int B, int H, int S, float scale, hipStream_t stream) {
  const int n_qtiles = (S + kBr - 1) / kBr;
  const long long blocks = (long long)B * H * n_qtiles;
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), S, n_qtiles,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace vdit
