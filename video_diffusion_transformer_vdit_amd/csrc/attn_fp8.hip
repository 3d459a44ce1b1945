// fp8 (E4M3) flash-style attention forward for gfx950 on the pre-pass
// outputs (quant_fp8.hip).
//
// Low-bit attention after the VC-Attention article (aikraft.ru): QK^T and PV
// on 8-bit tensor instructions (section 01; FP8 doubles throughput per the
// FLOPS article's "Optymalizacje"), softmax in fp32, V-Smooth restore of the
// value mean in the epilogue from the online-softmax row sum with no second
// pass (section 02, Restore).
//
// Scores of query i and key j (key block b = j / 64):
//   s_ij = q_scale_i k_scale_b (q8_i . k8_j) + q_hat_i . k_mean_b
// The second term restores the K mean.  q_hat . k_mean = q_scale (dec(q8) .
// k_mean) where dec(q8) is exact in bf16 and k_mean is split into a bf16 high
// part and a bf16 residual, so two bf16 MFMAs per 16 channels give it to
// about 2^-16 relative.  With one mean per 64-token block it is computed for
// 32 blocks at a time and parked in LDS; with one global mean it is computed
// once.  It is applied even when it is constant along a row: a constant shift
// does not change the softmax but it does move the fp8 grid P is rounded on.
// Softmax runs in the log2 domain with an integer running reference m
// (the ceiling of the running row maximum): p = 2^(t - m) <= 1.  P is
// quantised as E4M3(448 p) for the fp8 PV product; the row sum takes the fp32
// 448 p; because m only moves by whole powers of two, the quantised weights
// equal those taken against the final row maximum (outside the subnormal
// range).  Epilogue: o = v_scale (sum_j P8_ij v8_j) / l_i + v_mean.
//
// Layout of the work: one workgroup = 4 waves x 32 queries; K/V tiles of 64
// keys (= one scale block) staged through registers into a double-buffered
// LDS ring; scores are produced transposed (S^T = K Q^T) so each lane owns
// one query; V is transposed at staging time so that the P^T operand is the
// S^T accumulator registers in order.
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kBr = 128;
constexpr int kBc = 64;
constexpr int kThreads = 256;
constexpr int kKStride = kHeadDim + 16;  // bytes per K8 row in LDS (144)
constexpr int kVStride = kBc + 16;       // bytes per V8^T row in LDS (80)
constexpr int kKBuf = kBc * kKStride;
constexpr int kVBuf = kHeadDim * kVStride;
constexpr int kCompBlocks = 32;          // K-mean blocks per compensation batch
constexpr float kLog2P8 = 8.807354922057604f;  // log2(448)

__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // operand formats 0/0 = E4M3 x E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const uint8_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

__device__ __forceinline__ u32x2 ld8(const uint8_t* p, bool ok) {
  u32x2 z = {0u, 0u};
  return ok ? *reinterpret_cast<const u32x2*>(p) : z;
}

struct Staged {
  u32x4 k[2];  // K8 row t/4, bytes 32*(t%4) .. +31
  u32x2 v[4];  // V8 rows 4*(t/16) .. +3, bytes 8*(t%16) .. +7
  float ks;    // k_scale of the tile
};

__device__ __forceinline__ void load_tile(Staged& st, const uint8_t* K8h, const uint8_t* V8h,
                                          const float* ksh, int j, int S, int tid) {
  const int key0 = j * kBc;
  const int kr = key0 + (tid >> 2);
  const int kc = (tid & 3) * 32;
  st.k[0] = ld16(K8h + (size_t)kr * kHeadDim + kc, kr < S);
  st.k[1] = ld16(K8h + (size_t)kr * kHeadDim + kc + 16, kr < S);
  const int vc = (tid & 15) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int vr = key0 + 4 * (tid >> 4) + i;
    st.v[i] = ld8(V8h + (size_t)vr * kHeadDim + vc, vr < S);
  }
  st.ks = ksh[j];
}

// Byte e of lane half h in the PV operand is key 32(e/16) + 8((e%16)/4) + 4h + e%4
// of the tile; V8^T keeps keys in that order: key bits [5|4:3|2|1:0] = a,b,h,r
// go to position bits [5|4|3:2|1:0] = h,a,b,r.
__device__ __forceinline__ int vpos(int key) {
  return ((key >> 2) & 1) << 5 | ((key >> 5) & 1) << 4 | ((key >> 3) & 3) << 2 | (key & 3);
}

__device__ __forceinline__ void store_tile(const Staged& st, uint8_t* Ks, uint8_t* Vs, int tid) {
  uint8_t* kd = Ks + (tid >> 2) * kKStride + (tid & 3) * 32;
  *reinterpret_cast<u32x4*>(kd) = st.k[0];
  *reinterpret_cast<u32x4*>(kd + 16) = st.k[1];
  const int g = tid >> 4, c = tid & 15;
  const int pos = vpos(4 * g);
  // 4 keys x 8 channels -> 8 dwords of 4 keys each
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t a0 = st.v[0][w], a1 = st.v[1][w], a2 = st.v[2][w], a3 = st.v[3][w];
    const uint32_t lo01 = __byte_perm(a0, a1, 0x5140);  // a0.b0 a1.b0 a0.b1 a1.b1
    const uint32_t hi01 = __byte_perm(a0, a1, 0x7362);  // a0.b2 a1.b2 a0.b3 a1.b3
    const uint32_t lo23 = __byte_perm(a2, a3, 0x5140);
    const uint32_t hi23 = __byte_perm(a2, a3, 0x7362);
    const uint32_t d0 = __byte_perm(lo01, lo23, 0x5410);  // channel 4w+0: keys 0..3
    const uint32_t d1 = __byte_perm(lo01, lo23, 0x7632);  // channel 4w+1
    const uint32_t d2 = __byte_perm(hi01, hi23, 0x5410);  // channel 4w+2
    const uint32_t d3 = __byte_perm(hi01, hi23, 0x7632);  // channel 4w+3
    const int ch = 8 * c + 4 * w;
    *reinterpret_cast<uint32_t*>(Vs + (ch + 0) * kVStride + pos) = d0;
    *reinterpret_cast<uint32_t*>(Vs + (ch + 1) * kVStride + pos) = d1;
    *reinterpret_cast<uint32_t*>(Vs + (ch + 2) * kVStride + pos) = d2;
    *reinterpret_cast<uint32_t*>(Vs + (ch + 3) * kVStride + pos) = d3;
  }
}

// E4M3 code (from the OCP format: bias 7, 3 mantissa bits, subnormals 2^-9)
// -> float; used to build the bf16 q_hat of the compensation term.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? (float)m * 0.001953125f
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// kBlockMean: one K mean per 64-token block (else one mean per head)
template <bool kBlockMean>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    const float* __restrict__ k_mean, const float* __restrict__ v_mean,
    const float* __restrict__ v_scale, uint16_t* __restrict__ O, int S, int n_qtiles, float c) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2 * kKBuf];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2 * kVBuf];
  __shared__ float lds_comp[4][kCompBlocks][32];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const size_t base = (size_t)bh * S * kHeadDim;
  const int nb = (S + kBc - 1) / kBc;
  const uint8_t* Q8h = Q8 + base;
  const uint8_t* K8h = K8 + base;
  const uint8_t* V8h = V8 + base;
  const float* ksh = k_scale + (size_t)bh * nb;
  uint16_t* Oh = O + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qt * kBr + wave * 32 + col;
  const bool qok = qrow < S;

  i32x8 qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const uint8_t* p = Q8h + (size_t)qrow * kHeadDim + 64 * kk + 32 * half;
    const u32x4 lo = ld16(p, qok), hi = ld16(p + 16, qok);
    qf[kk] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  // all 32 queries of a wave sit in one 64-token scale block
  const float qsc = q_scale[(size_t)bh * nb + min(qrow, S - 1) / kBc] * c;

  // dec(q8) in bf16 (exact) as the B operand of the K-mean MFMAs (lane:
  // query col, channels 16kk + 8half .. +7).
  bf16x8 qh[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const u32x2 w = ld8(Q8h + (size_t)qrow * kHeadDim + 16 * kk + 8 * half, qok);
#pragma unroll
    for (int e = 0; e < 8; ++e) qh[kk][e] = (__bf16)e4m3_value((w[e >> 2] >> (8 * (e & 3))) & 255u);
  }
  const int nbm = kBlockMean ? nb : 1;
  const float* kmh = k_mean + (size_t)bh * nbm * kHeadDim;
  // dec(q8_i) . k_mean_b for b = b0 .. b0+31 (clamped to the last block),
  // written to this wave's LDS slots lds_comp[wave][b - b0][query].
  auto kmean_batch = [&](int b0) {
    f32x16 cm;
#pragma unroll
    for (int i = 0; i < 16; ++i) cm[i] = 0.f;
    const float* km = kmh + (size_t)min(b0 + col, nbm - 1) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(km + 16 * kk + 8 * half);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(km + 16 * kk + 8 * half + 4);
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? a0[e] : a1[e - 4];
        hi[e] = (__bf16)x;
        lo[e] = (__bf16)(x - (float)hi[e]);
      }
      cm = mfma32x32x16_bf16(hi, qh[kk], cm);
      cm = mfma32x32x16_bf16(lo, qh[kk], cm);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) lds_comp[wave][8 * (i >> 2) + 4 * half + (i & 3)][col] = cm[i];
  };
  // Each wave reads only its own slots, after its own writes (LDS operations
  // of one wave complete in order), so no barrier is needed around them.
  float cb_global = 0.f;
  if (!kBlockMean) {
    kmean_batch(0);
    cb_global = lds_comp[wave][0][col] * qsc;
  }

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_ref = -INFINITY;
  float l = 0.f;

  const int nkt = nb;
  Staged st;
  load_tile(st, K8h, V8h, ksh, 0, S, tid);
  store_tile(st, lds_k, lds_v, tid);
  float ks_cur = st.ks;
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (kBlockMean && (j % kCompBlocks) == 0) kmean_batch(j);
    if (j + 1 < nkt) load_tile(st, K8h, V8h, ksh, j + 1, S, tid);
    const uint8_t* Ks = lds_k + buf * kKBuf;
    const uint8_t* Vs = lds_v + buf * kVBuf;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint8_t* p = Ks + (32 * kb + col) * kKStride + 64 * kk + 32 * half;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
        const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        s[kb] = mfma32x32x64_fp8(a, qf[kk], s[kb]);
      }
    }
    if (j == nkt - 1 && (S % kBc) != 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j * kBc + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          if (key >= S) s[kb][i] = -INFINITY;
        }
    }
    // t = a * dot + cb (log2 domain); a >= 0, so the row max of t is at the
    // row max of dot.
    const float a = qsc * ks_cur;
    const float cb = kBlockMean ? lds_comp[wave][j % kCompBlocks][col] * qsc : cb_global;
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    float mnew = fmaf(mx, a, cb);
    mnew = fmaxf(mnew, swap_halves(mnew));
    if (__ballot(mnew > m_ref) != 0ull) {
      const float mnext = mnew > m_ref ? ceilf(mnew) : m_ref;
      const float alpha = exp2_fast(m_ref - mnext);
      l *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
      m_ref = mnext;
    }
    const float bias = cb + kLog2P8 - m_ref;
    uint32_t pk[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          e[u] = fminf(exp2_fast(fmaf(s[kb][4 * p + u], a, bias)), 448.0f);
          l += e[u];
        }
        uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
        pk[4 * kb + p] = w;
      }
    const i32x8 pb = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3],
                      (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint8_t* p = Vs + (32 * mb + col) * kVStride + 32 * half;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
      const i32x8 av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      acc[mb] = mfma32x32x64_fp8(av, pb, acc[mb]);
    }

    if (j + 1 < nkt) {
      store_tile(st, lds_k + (buf ^ 1) * kKBuf, lds_v + (buf ^ 1) * kVBuf, tid);
      ks_cur = st.ks;
    }
    __syncthreads();
  }

  const float inv = 1.0f / (l + swap_halves(l));
  if (qok) {
    const float* vsh = v_scale + (size_t)bh * kHeadDim;
    const float* vmh = v_mean + (size_t)bh * kHeadDim;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * half;
        const f32x4 vs = *reinterpret_cast<const f32x4*>(vsh + d0);
        const f32x4 vm = *reinterpret_cast<const f32x4*>(vmh + d0);
        u32x2 w;
        w.x = pack_bf16x2(fmaf(acc[mb][4 * g] * inv, vs[0], vm[0]),
                          fmaf(acc[mb][4 * g + 1] * inv, vs[1], vm[1]));
        w.y = pack_bf16x2(fmaf(acc[mb][4 * g + 2] * inv, vs[2], vm[2]),
                          fmaf(acc[mb][4 * g + 3] * inv, vs[3], vm[3]));
        *reinterpret_cast<u32x2*>(Oh + (size_t)qrow * kHeadDim + d0) = w;
      }
  }
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                               const float* q_scale, const float* k_scale, const float* k_mean,
                               int k_mean_blocks, const float* v_mean, const float* v_scale,
                               void* o, int B, int H, int S, float scale, hipStream_t stream) {
  const int n_qtiles = (S + kBr - 1) / kBr;
  const unsigned blocks = (unsigned)((long long)B * H * n_qtiles);
  const int nb = (S + kBc - 1) / kBc;
  const bool block_mean = k_mean_blocks == nb && nb > 1;
  const uint8_t* q = static_cast<const uint8_t*>(q8);
  const uint8_t* k = static_cast<const uint8_t*>(k8);
  const uint8_t* v = static_cast<const uint8_t*>(v8);
  uint16_t* out = static_cast<uint16_t*>(o);
  const float c = scale * kLog2e;
  if (block_mean)
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, q, k, v,
                       q_scale, k_scale, k_mean, v_mean, v_scale, out, S, n_qtiles, c);
  else
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, q, k,
                       v, q_scale, k_scale, k_mean, v_mean, v_scale, out, S, n_qtiles, c);
  return hipGetLastError();
}

}  // namespace vdit
