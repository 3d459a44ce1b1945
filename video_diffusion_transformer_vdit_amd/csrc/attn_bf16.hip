// bf16 flash-style attention forward for gfx950 (MI355X).
//
// Computes O = softmax(scale * Q K^T) V per (batch, head) without storing the
// S x S score matrix: the full spatiotemporal self-attention of a video DiT
// (VC-Attention article (aikraft.ru), section 01) with the FlashAttention
// tiling the FLOPS article (sudonull.com, "Optymalizacje") credits with
// removing the 75K x 75K matrix.
//
// Design (one workgroup = 4 waves = 128 queries; two workgroups per CU):
//  * Each wave owns 32 queries.  Its Q slice stays in registers for the whole
//    key loop as the B operand of v_mfma_f32_32x32x16_bf16.
//  * Scores are produced transposed, S^T = K Q^T, so lane (q, half) holds one
//    query and 16 keys of every 32-key block: row max / row sum are in-lane,
//    plus one exchange with lane ^ 32 for the max.
//  * K/V tiles of 64 keys are staged through registers into a double-buffered
//    LDS ring (one barrier per tile).  K is stored row-major; V is stored
//    transposed (V^T, keys contiguous) by a register transpose at staging
//    time so that O^T += V^T P^T reads 16-byte A operands.  Inside every
//    16-key chunk, key bits 2 and 3 are swapped in V^T so that the P^T
//    operand is exactly the S^T accumulator registers in order.
//  * Online softmax in the log2 domain with an integer running reference
//    m (ceil of the running maximum of scale*log2(e)*s): P = 2^(c s - m) <= 1,
//    and the accumulator is rescaled (by an exact power of two) only in the
//    rare tiles where some row's maximum exceeds its reference.
//  * Row padding: keys >= S are zero-filled and scored -inf in the last tile;
//    queries >= S are computed on zeros and not stored.
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kBr = 128;                 // queries per workgroup
constexpr int kBc = 64;                  // keys per K/V tile
constexpr int kThreads = 256;            // 4 waves
constexpr int kKStride = kHeadDim + 8;   // bf16 per K row in LDS (272 B)
constexpr int kVStride = kBc + 8;        // bf16 per V^T row in LDS (144 B)
constexpr int kKBuf = kBc * kKStride;
constexpr int kVBuf = kHeadDim * kVStride;

struct Staged {
  u32x4 k[4];
  u32x4 v[4];
};

__device__ __forceinline__ u32x4 load16(const uint16_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

// Thread t stages K rows {p*16 + t/16} (p = 0..3), 16-byte chunk t%16, and V
// rows 4*(t/16) .. +3 of the same chunk (all coalesced 16-byte loads).
__device__ __forceinline__ void load_tile(Staged& st, const uint16_t* Kh, const uint16_t* Vh,
                                          int key0, int S, int tid) {
  const int c8 = (tid & 15) * 8;
  const int r = tid >> 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = key0 + p * 16 + r;
    st.k[p] = load16(Kh + (size_t)row * kHeadDim + c8, row < S);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = key0 + 4 * r + i;
    st.v[i] = load16(Vh + (size_t)row * kHeadDim + c8, row < S);
  }
}

__device__ __forceinline__ void store_tile(const Staged& st, uint16_t* Ks, uint16_t* Vs, int tid) {
  const int c = tid & 15;
  const int g = tid >> 4;
#pragma unroll
  for (int p = 0; p < 4; ++p)
    *reinterpret_cast<u32x4*>(Ks + (p * 16 + g) * kKStride + c * 8) = st.k[p];
  // keys 4g..4g+3 land at position 16*(g>>2) + 8*(g&1) + 4*((g>>1)&1)
  const int pos = 16 * (g >> 2) + 8 * (g & 1) + 4 * ((g >> 1) & 1);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    u32x2 lo, hi;
    lo.x = __byte_perm(st.v[0][w], st.v[1][w], 0x5410);
    lo.y = __byte_perm(st.v[2][w], st.v[3][w], 0x5410);
    hi.x = __byte_perm(st.v[0][w], st.v[1][w], 0x7632);
    hi.y = __byte_perm(st.v[2][w], st.v[3][w], 0x7632);
    *reinterpret_cast<u32x2*>(Vs + (c * 8 + 2 * w) * kVStride + pos) = lo;
    *reinterpret_cast<u32x2*>(Vs + (c * 8 + 2 * w + 1) * kVStride + pos) = hi;
  }
}

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, int S, int n_qtiles, float c) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2 * kKBuf];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2 * kVBuf];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const size_t base = (size_t)bh * S * kHeadDim;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  uint16_t* Oh = O + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qt * kBr + wave * 32 + col;

  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8, load16(Qh + (size_t)qrow * kHeadDim + 16 * kk + 8 * half, qrow < S));

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_ref = -INFINITY;  // integer-valued log2-domain reference
  float l = 0.f;            // this lane's share of the row sum

  const int nkt = (S + kBc - 1) / kBc;
  Staged st;
  load_tile(st, Kh, Vh, 0, S, tid);
  store_tile(st, lds_k, lds_v, tid);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkt) load_tile(st, Kh, Vh, (j + 1) * kBc, S, tid);
    const uint16_t* Ks = lds_k + buf * kKBuf;
    const uint16_t* Vs = lds_v + buf * kVBuf;

    // S^T[key][query] for two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (32 * kb + col) * kKStride + 16 * kk + 8 * half);
        s[kb] = mfma32x32x16_bf16(a, qf[kk], s[kb]);
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

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, swap_halves(mx));
    const float mnew = mx * c;
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

    uint32_t pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float p0 = exp2_fast(fmaf(s[kb][2 * p], c, -m_ref));
        const float p1 = exp2_fast(fmaf(s[kb][2 * p + 1], c, -m_ref));
        l += p0;
        l += p1;
        pk[kb][p] = pack_bf16x2(p0, p1);
      }

    // O^T[d][query] += V^T P^T over four 16-key chunks.
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1, cc = kc & 1;
      u32x4 pw = {pk[kb][4 * cc], pk[kb][4 * cc + 1], pk[kb][4 * cc + 2], pk[kb][4 * cc + 3]};
      const bf16x8 b = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + (32 * mb + col) * kVStride + 16 * kc + 8 * half);
        acc[mb] = mfma32x32x16_bf16(a, b, acc[mb]);
      }
    }

    if (j + 1 < nkt) store_tile(st, lds_k + (buf ^ 1) * kKBuf, lds_v + (buf ^ 1) * kVBuf, tid);
    __syncthreads();
  }

  const float inv = 1.0f / (l + swap_halves(l));
  if (qrow < S) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w.x = pack_bf16x2(acc[mb][4 * g] * inv, acc[mb][4 * g + 1] * inv);
        w.y = pack_bf16x2(acc[mb][4 * g + 2] * inv, acc[mb][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(Oh + (size_t)qrow * kHeadDim + 32 * mb + 8 * g + 4 * half) = w;
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
