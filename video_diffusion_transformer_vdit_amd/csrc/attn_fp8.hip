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
// 32 blocks at a time and parked in LDS (the fp32 means of a batch reach LDS
// by DMA a few tiles ahead and are split once per workgroup); with one
// global mean it is computed once.  It is applied even when it is constant along a row: a constant shift
// does not change the softmax but it does move the fp8 grid P is rounded on.
// Softmax runs in the log2 domain with an integer running reference m
// (the ceiling of the running row maximum): p = 2^(t - m) <= 1.  P is
// quantised as P8 = E4M3(448 p) for the fp8 PV product; because m only moves
// by whole powers of two, the quantised weights equal those taken against
// the final row maximum (outside the subnormal range).  The row sum is that
// of the quantised weights, formed by one 16x16x128 fp8 MFMA per tile (half
// the cycles of a 32x32x64 one) against a 0/1 selection operand, so the
// weights of a row sum to exactly one and the mean restore is exact.
// Epilogue: o = v_scale (sum_j P8_ij v8_j) / (sum_j P8_ij) + v_mean.
//
// With V block means (the article's Demean over 128-token hardware blocks)
// the restore runs inside the key loop instead: the row sum is a 32x32x64
// MFMA against a one-hot operand whose single row of ones is the block's slot, so it
// accumulates each block's weight sum in its own row (16 blocks = 32 tiles
// per batch); after each batch two bf16 MFMAs per 32 channels (the exact
// bf16 means against the high and low bf16 parts of the sums, about 2^-16
// relative) give sum_b (sum_{j in b} P8_ij) v_mean_b, which is added to the
// code-unit accumulator divided by v_scale, and the batch's sums join the
// row sum.  Epilogue: o = v_scale acc / l.
//
// Work layout (the bf16 kernel's): one workgroup = 8 waves x 32 queries, one
// workgroup per CU; scores transposed (S^T = K Q^T) so each lane owns one
// query; K tiles (row-major, 16-byte chunks XOR-swizzled by key & 7) and V
// tiles (already transposed and permuted by the pre-pass) go global -> LDS by
// DMA into four-deep rings; waves 0-3 and
// 4-7 run the exponential phase and the MFMA phase of each tile one phase
// apart (ping-pong).  The block-causal and block-sparse key masks follow the
// bf16 kernel's schedules.
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kWaves = 8;
constexpr int kBr = 32 * kWaves;  // 256 queries per workgroup
constexpr int kBc = 64;           // keys per tile = one scale block
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = kBc * kHeadDim;  // 8 KB of codes
constexpr int kCompBlocks = 32;             // K-mean blocks per compensation batch
constexpr float kLog2P8 = 8.807354922057604f;  // log2(448)
// ExpCast-FP8: the E4M3 byte of a value v, read as an integer, is about
// 8 log2(v) + 56 (VC-Attention article, section 03); with the article's
// centring constant -0.35 and P scaled by 448, the byte position of 448 p
// with log2 p = t - m is z = 8 (t - m) + 8 log2(448) + 55.65.  A normal byte
// 8 e + m stands for 2^(e - 7) (1 + m / 8); the same rule at a real position
// z is the fp32 value whose bit pattern is z 2^20 + 120 2^23 (exponent field
// floor(z / 8) + 120, mantissa (z mod 8) 2^20).  The kernel forms that
// pattern with one FMA per weight and lets the hardware E4M3 convert round
// it: in the normal range (z >= 7.5) the code is rne(z), the article's byte;
// below it, where bytes 1-7 are subnormals (m 2^-9) rather than points of
// the log map, it is the subnormal nearest the map's value, within one code
// of the exact cast, so the weights scale by exact powers of two with the
// online reference just as exp-then-cast weights do.
constexpr float kExpCastOffset = 8.0f * 8.807354922057604f + 56.0f - 0.35f;
constexpr float kTwo20 = 1048576.0f;       // 2^20: one byte position in fp32 bits
constexpr float kBias120 = 1006632960.0f;  // 120 2^23: exponent field of byte 0's octave

// fp32 -> u32, saturating: negative values and -inf give 0 (v_cvt_u32_f32).
// Written as asm: the C++ conversion of a negative value is undefined.
__device__ __forceinline__ uint32_t cvt_u32_sat(float x) {
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // operand formats 0/0 = E4M3 x E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x128_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const uint8_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// E4M3 code (from the OCP format: bias 7, 3 mantissa bits, subnormals 2^-9)
// -> float; used to build the bf16 q_hat of the compensation term.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? (float)m * 0.001953125f
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// Key masks (as in the bf16 kernel): kDense, kCausal (query i sees key j iff
// j / chunk <= i / chunk) or kSparse (block_mask[b,h,i/128,j/64] != 0).
constexpr int kDense = 0, kCausal = 1, kSparse = 2;
constexpr int kMaxSparseTiles = 16384;

// Matrix-phase schedule of the V-block-mean ExpCast instance: every operand
// read (two 16-byte reads for each of the 4 QK^T and 4 PV MFMAs; none for
// the row-sum MFMA, the ninth) issued L MFMAs ahead of its use.  That
// instance's matrix phase is the long one and runs 2.6% faster with L = 2;
// the other instances are faster with the default schedule.
template <int L, int I = 0>
__device__ __forceinline__ void sched_reads_ahead() {
  constexpr auto reads = [](int i) { return i < 8 ? 2 : 0; };
  if constexpr (I == 0) {
    constexpr int pre = [] {
      int n = 0;
      for (int j = 0; j < L; ++j) n += j < 8 ? 2 : 0;
      return n;
    }();
    __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);
  }
  if constexpr (I < 9) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I + L < 9 && reads(I + L) > 0) __builtin_amdgcn_sched_group_barrier(0x100, reads(I + L), 0);
    sched_reads_ahead<L, I + 1>();
  }
}

// kBlockMean: one K mean per 64-token block (else one mean per head);
// kExpCast: P8 bytes written directly from the log domain (else exp2, then
// an E4M3 conversion); kVBlock: V means per 128-token block (v_bmean, bf16,
// [bh][channel][nbv_pad]) restored in the loop (else one v_mean per channel;
// kVBlock is only built for kDense); kMode: the key mask.
template <bool kBlockMean, bool kExpCast, bool kVBlock, int kMode>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    const float* __restrict__ k_mean, const float* __restrict__ v_mean,
    const uint16_t* __restrict__ v_bmean, int nbv_pad, const float* __restrict__ v_scale,
    uint16_t* __restrict__ O, int S, int n_qtiles, float c, int chunk,
    const uint8_t* __restrict__ block_mask, int nqb) {
  // four-deep rings of K and V tiles, one LDS object per buffer
  constexpr int kRing = 4;
  __shared__ __attribute__((aligned(1024))) char lds_k0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v3[kTileBytes];
  __shared__ float lds_comp[kWaves][kCompBlocks][32];
  constexpr bool kStageKm = kBlockMean;
  __shared__ __attribute__((aligned(1024))) char lds_km[kStageKm ? kCompBlocks * 512 : 1];
  __shared__ __attribute__((aligned(16))) float lds_ivs[kHeadDim];  // 1 / v_scale (V block means only)

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  // block-causal: heaviest query tiles first
  const int qt = kMode == kCausal ? n_qtiles - 1 - (tile - bh * n_qtiles) : tile - bh * n_qtiles;
  const size_t base = (size_t)bh * S * kHeadDim;
  const int nkt_all = (S + kBc - 1) / kBc;
  const uint8_t* Q8h = Q8 + base;
  const char* K8h = reinterpret_cast<const char*>(K8 + base);
  // V codes: nkt_all tiles of 8 KB per head
  const char* V8h = reinterpret_cast<const char*>(V8) + (size_t)bh * nkt_all * kTileBytes;
  const float* ksh = k_scale + (size_t)bh * nkt_all;
  uint16_t* Oh = O + base;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qt * kBr + wave * 32 + col;
  const bool qok = qrow < S;
  const bool tail = (S % kBc) != 0;

  // ---- key masks: the tiles this workgroup visits (nkt loop steps) ----
  auto key_limit = [&](int row) { return kMode == kCausal ? min(S, (row / chunk + 1) * chunk) : S; };
  const int lim = key_limit(min(qrow, S - 1));
  const int wave_lim = key_limit(min(qt * kBr + wave * 32, S - 1));
  int nkt = (key_limit(min(qt * kBr + kBr - 1, S - 1)) + kBc - 1) / kBc;
  // block-sparse: the union of the tiles allowed to the workgroup's two
  // 128-query blocks, ascending, entry kt | (blocks allowing it) << 14
  __shared__ uint16_t lds_list[kMode == kSparse ? kMaxSparseTiles : 1];
  __shared__ int lds_cnt[kWaves];
  const uint32_t wbit = wave < 4 ? 1u : 2u;
  if (kMode == kSparse) {
    const uint8_t* m0 = block_mask + ((size_t)bh * nqb + 2 * qt) * nkt_all;
    const bool has1 = 2 * qt + 1 < nqb;
    int nvis = 0;
    for (int c0 = 0; c0 < nkt_all; c0 += kThreads) {
      const int kt = c0 + tid;
      uint32_t f = 0;
      if (kt < nkt_all) f = (m0[kt] ? 1u : 0u) | ((has1 && m0[nkt_all + kt]) ? 2u : 0u);
      const unsigned long long bal = __ballot(f != 0);
      if (lane == 0) lds_cnt[wave] = __popcll(bal);
      __syncthreads();
      int off = nvis;
      for (int w = 0; w < wave; ++w) off += lds_cnt[w];
      if (f) lds_list[off + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)(kt | (f << 14));
      for (int w = 0; w < kWaves; ++w) nvis += lds_cnt[w];
      __syncthreads();
    }
    nkt = __builtin_amdgcn_readfirstlane(nvis);
    if (nkt == 0) {  // no allowed key for any row of this workgroup: zeros
      if (qok)
        for (int d = 0; d < kHeadDim; d += 8)
          *reinterpret_cast<u32x4*>(Oh + (size_t)qrow * kHeadDim + d) = u32x4{0u, 0u, 0u, 0u};
      return;
    }
  }
  // key tile of loop step t (clamped: steps past the end reload the last one)
  auto tile_of = [&](int t) __attribute__((always_inline)) {
    t = min(t, nkt - 1);
    return kMode == kSparse ? __builtin_amdgcn_readfirstlane((int)(lds_list[t] & 0x3fffu)) : t;
  };
  // block-sparse: the list entries that the matrix phase of step t needs (the
  // tiles of K(t+kRing) and V(t+kRing-1), the mask of step t+1, which is
  // also the K-scale tile of the next exponential phase), read in the
  // exponential phase before it
  uint32_t pre_k = 0, pre_v = 0, pre_m = 0;

  // ---- DMA: one 1 KB load per wave per tile and tensor ----
  // K: wave w fills tile rows 8w .. 8w+7; lane i writes physical chunk i%8 of
  // row 8w + i/8 and fetches the logical chunk the swizzle maps there.
  const int krow = 8 * wave + (lane >> 3);
  const int kgo = krow * kHeadDim + 16 * ((lane & 7) ^ (krow & 7));
  const uint32_t wslice = (uint32_t)wave * 1024;
  // DMA of key tile t (an index into K and V, not a loop step)
  auto issue_k = [&](int t, const void* buf) __attribute__((always_inline)) {
    const int key0 = t * kBc;
    const char* src = K8h + (size_t)key0 * kHeadDim;
    int go = kgo;
    if (tail && t == nkt_all - 1) go = (min(key0 + krow, S - 1) - key0) * kHeadDim + 16 * ((lane & 7) ^ (krow & 7));
    dma16(src, (uint32_t)go, lds_addr(buf) + wslice);
  };
  auto issue_v = [&](int t, const void* buf) __attribute__((always_inline)) {
    dma16(V8h + (size_t)t * kTileBytes, (uint32_t)(wslice + 16 * lane), lds_addr(buf) + wslice);
  };
  // K operand of key block kb, channel step kk: lane (key 32kb + col, half)
  // reads logical chunks 4kk + 2half + {0, 1} of its key row.
  int koff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) koff[kk][h2] = col * kHeadDim + 16 * ((4 * kk + 2 * half + h2) ^ (col & 7));
  // V^T operand of channel block mb: lane (channel 32mb + col, half) reads
  // key slots 32half .. +31 = logical chunks 2half + {0, 1} of its row.
  int voff[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) voff[h2] = col * kBc + 16 * ((2 * half + h2) ^ ((col >> 2) & 3));

  // ---- Q operand (registers for the whole loop) ----
  i32x8 qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const uint8_t* p = Q8h + (size_t)qrow * kHeadDim + 64 * kk + 32 * half;
    qf[kk] = join(ld16(p, qok), ld16(p + 16, qok));
  }
  // all 32 queries of a wave sit in one 64-token scale block
  const float qsc = q_scale[(size_t)bh * nkt_all + min(qrow, S - 1) / kBc] * c;

  // dec(q8) in bf16 (exact: every E4M3 value is a bf16 value) as the B
  // operand of the K-mean MFMAs (lane: query col, channels 16kk + 8half ..
  // +7).  Held in 32 registers, except with V block means: there the
  // restore needs those registers, so it is rebuilt from the (L2-resident) Q
  // codes at each batch by the hardware E4M3 convert (v_cvt_pk_f32_fp8, the
  // OCP format of the codes), which keeps LDS free for the staged K means
  // and the fourth ring buffer.
  const uint8_t* q8row = Q8h + (size_t)min(qrow, S - 1) * kHeadDim + 8 * half;
  auto load_q8 = [&](u32x2 (&w)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      w[kk] = qok ? *reinterpret_cast<const u32x2*>(q8row + 16 * kk) : u32x2{0u, 0u};
  };
  auto dec_q8 = [&](const u32x2& w) __attribute__((always_inline)) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const f32x2 c2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    const bf16x8 r = {(__bf16)a[0], (__bf16)a[1], (__bf16)b[0], (__bf16)b[1],
                      (__bf16)c2[0], (__bf16)c2[1], (__bf16)d[0], (__bf16)d[1]};
    return r;
  };
  bf16x8 qh_reg[8];
  if (!kVBlock) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint8_t* p = Q8h + (size_t)qrow * kHeadDim + 16 * kk + 8 * half;
      const u32x2 w = qok ? *reinterpret_cast<const u32x2*>(p) : u32x2{0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) qh_reg[kk][e] = (__bf16)e4m3_value((w[e >> 2] >> (8 * (e & 3))) & 255u);
    }
  }
  const int nbm = kBlockMean ? nkt_all : 1;
  const float* kmh = k_mean + (size_t)bh * nbm * kHeadDim;
  // dec(q8_i) . k_mean_b for b = b0 .. b0+31 (clamped to the last block),
  // written to this wave's LDS slots lds_comp[wave][b - b0][query].  Each
  // wave reads only its own slots, after its own writes (LDS operations of
  // one wave complete in order), so no barrier is needed around them.
  // lane col: the K block of loop step b0 + col (the one mean of the head
  // without block means)
  auto kmean_block = [&](int step) __attribute__((always_inline)) {
    return !kBlockMean         ? 0
           : kMode == kSparse ? (int)(lds_list[min(step, nkt - 1)] & 0x3fffu)
                              : min(step, nbm - 1);
  };
  // Staged block means (block means without V block means): the fp32 means
  // of a batch's 32 blocks arrive in lds_km by DMA a few steps ahead (block
  // b in bytes 512b .. 512b+511); each wave then rewrites its four blocks in
  // place as bf16 hi and lo halves (x ~ hi + lo to 2^-16), 16-byte chunk c of
  // each at chunk c ^ (b % 16) of the block's first and second 256 bytes, so
  // that the MFMA operand reads of 32 blocks hit distinct banks.
  auto km_issue = [&](int b0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = 4 * wave + 2 * i;
      const int kb = kmean_block(b0 + blk + (lane >> 5));
      dma16(reinterpret_cast<const char*>(kmh), (uint32_t)(kb * kHeadDim + 4 * (lane & 31)) * 4u,
            lds_addr(lds_km) + (uint32_t)blk * 512u);
    }
  };
  auto km_convert = [&]() __attribute__((always_inline)) {
    const int b = 4 * wave + (lane >> 4), c = lane & 15;
    char* row = lds_km + b * 512;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(row + 32 * c);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(row + 32 * c + 16);
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = e < 4 ? x0[e] : x1[e - 4];
      hi[e] = (__bf16)x;
      lo[e] = (__bf16)(x - (float)hi[e]);
    }
    // the wave's reads above complete before these writes (one wave's LDS
    // operations are done in order), so rewriting in place is safe
    *reinterpret_cast<bf16x8*>(row + 16 * (c ^ (b & 15))) = hi;
    *reinterpret_cast<bf16x8*>(row + 256 + 16 * (c ^ (b & 15))) = lo;
  };
  auto kmean_batch = [&](int b0) __attribute__((always_inline)) {
    f32x16 cm;
#pragma unroll
    for (int i = 0; i < 16; ++i) cm[i] = 0.f;
    u32x2 q8w[8];
    if (kVBlock) load_q8(q8w);
    const float* km = kmh + (size_t)kmean_block(b0 + col) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8 hi, lo;
      if (kStageKm) {
        const char* row = lds_km + col * 512 + 16 * ((2 * kk + half) ^ (col & 15));
        hi = *reinterpret_cast<const bf16x8*>(row);
        lo = *reinterpret_cast<const bf16x8*>(row + 256);
      } else {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(km + 16 * kk + 8 * half);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(km + 16 * kk + 8 * half + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e < 4 ? a0[e] : a1[e - 4];
          hi[e] = (__bf16)x;
          lo[e] = (__bf16)(x - (float)hi[e]);
        }
      }
      const bf16x8 qh = kVBlock ? dec_q8(q8w[kk]) : qh_reg[kk];
      cm = mfma32x32x16_bf16(hi, qh, cm);
      cm = mfma32x32x16_bf16(lo, qh, cm);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) lds_comp[wave][8 * (i >> 2) + 4 * half + (i & 3)][col] = cm[i];
  };
  float cb_global = 0.f;
  if (!kBlockMean) {
    kmean_batch(0);
    cb_global = lds_comp[wave][0][col] * qsc;
  }

  f32x16 s[2];  // S^T of one tile: key block kb, lane (q, half): keys 32kb + 8(i/4) + 4half + i%4
  auto qk = [&](const char* Kb) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const char* p = Kb + kb * 32 * kHeadDim;
        const i32x8 a = join(*reinterpret_cast<const u32x4*>(p + koff[kk][0]),
                             *reinterpret_cast<const u32x4*>(p + koff[kk][1]));
        s[kb] = mfma32x32x64_fp8(a, qf[kk], s[kb]);
      }
    }
  };
  auto mask_tail = [&](int t) __attribute__((always_inline)) {
    // keeps the compiler from turning this once-per-workgroup branch into
    // selects executed on every tile
    asm volatile("" ::: "memory");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t * kBc + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key >= lim) s[kb][i] = -INFINITY;
      }
  };
  // block-sparse: step t's scores -inf where this wave's query block does not
  // allow the tile (or t is past the list), keys past S in the ragged tile
  auto mask_sparse = [&](uint32_t e) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    e = __builtin_amdgcn_readfirstlane(e);
    const int kt = (int)(e & 0x3fffu);
    if (((e >> 14) & wbit) == 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = -INFINITY;
    } else if (tail && kt == nkt_all - 1) {
      mask_tail(kt);
    }
  };
  // (block-sparse: e is the list entry of step t, 0 past the list)
  auto mask_step = [&](int t, uint32_t e) __attribute__((always_inline)) {
    if (kMode == kSparse)
      mask_sparse(e);
    else if (t * kBc + kBc > wave_lim)
      mask_tail(t);
  };

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  // with V block means: per-block weight sums (see pv below)
  f32x16 lacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) lacc[i] = 0.f;
  // Row sum of the quantised weights on a 16x16x128 MFMA whose B operand is
  // the P registers of the 32x32x64 PV product as they stand: lane l then
  // stands for column l % 16 and k-group l / 16, i.e. query l % 16 + 16 (g % 2)
  // with keys 32 (g / 2) .. + 31 of the tile (g = l / 16).  Rows 0 and 8 of
  // the selection operand take k-groups 0 and 2 (queries 0-15), rows 4 and 12
  // groups 1 and 3 (queries 16-31), so element 0 of lane l's output (row
  // 4 (l / 16), column l % 16) is the weight sum of the lane's own query.
  f32x4 rsum = {0.f, 0.f, 0.f, 0.f};
  const int sel_row = lane & 15, sel_grp = lane >> 4;
  const bool sel_on =
      (sel_grp & 1) ? (sel_row == 4 || sel_row == 12) : (sel_row == 0 || sel_row == 8);
  const int sel_b = sel_on ? 0x38383838 : 0;  // E4M3 1.0 or 0
  i32x8 sel = {sel_b, sel_b, sel_b, sel_b, sel_b, sel_b, sel_b, sel_b};
  // opaque from here on: kept in its eight registers rather than rebuilt
  // before every row-sum MFMA
  if (!kVBlock) asm volatile("" : "+v"(sel));
  // finite when block-sparse: tiles scored entirely -inf before a row's first
  // allowed key then give weight 0, not NaN
  float m_ref = kMode == kSparse ? -1e30f : -INFINITY;
  // V block means: row sum of the drained batches; 1 / v_scale per channel
  // in LDS (it scales the means into code units for the restore MFMA)
  float l_tot = 0.f;
  const uint16_t* vbmh = v_bmean + (size_t)bh * kHeadDim * nbv_pad;
  if (kVBlock && tid < kHeadDim) lds_ivs[tid] = 1.0f / v_scale[(size_t)bh * kHeadDim + tid];
  // Restore of batch `batch` (128-token blocks 16 batch .. +15): lane (query
  // col, half) holds the weight sums of blocks 16 batch + 8 half + j in
  // lacc[j] (the one-hot rows below put them there), which is exactly the B
  // operand of a 32x32x16 bf16 MFMA over those 16 blocks.
  // The batch's means (16 bytes per lane and 32-channel block) are loaded in
  // the exponential phase before the drain, so their latency overlaps it.
  u32x4 vbm_pre[4];
  auto vload = [&](int batch) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      vbm_pre[mb] = *reinterpret_cast<const u32x4*>(vbmh + (size_t)(32 * mb + col) * nbv_pad +
                                                     16 * batch + 8 * half);
  };
  auto vdrain = [&]() __attribute__((always_inline)) {
    bf16x8 bhi, blo;
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ls += lacc[j];
      bhi[j] = (__bf16)lacc[j];
      blo[j] = (__bf16)(lacc[j] - (float)bhi[j]);
    }
    l_tot += sum_halves(ls);
    // r = means x sums in value units (the bf16 means are exact operands),
    // then acc += r / v_scale row by row
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const bf16x8 vm = __builtin_bit_cast(bf16x8, vbm_pre[mb]);
      f32x16 r;
#pragma unroll
      for (int i = 0; i < 16; ++i) r[i] = 0.f;
      r = mfma32x32x16_bf16(vm, bhi, r);
      r = mfma32x32x16_bf16(vm, blo, r);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 iv = *reinterpret_cast<const f32x4*>(&lds_ivs[32 * mb + 8 * g + 4 * half]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mb][4 * g + e] = fmaf(r[4 * g + e], iv[e], acc[mb][4 * g + e]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) lacc[i] = 0.f;
  };

  // P8 of tile t: t = a dot + cb in the log2 domain (a >= 0, so the row max
  // of t is at the row max of dot); reference update and (rare) rescale;
  // e = 2^(t - m) * 448 <= 448 up to the last bit of exp2, packed as E4M3.
  uint32_t pk[8];
  auto softmax_p = [&](int t) __attribute__((always_inline)) {
    // (block-sparse: pre_m holds step t's list entry here)
    const float a = qsc * ksh[kMode == kSparse ? __builtin_amdgcn_readfirstlane((int)(pre_m & 0x3fffu))
                                               : min(t, nkt - 1)];
    const float cb = kBlockMean ? lds_comp[wave][t % kCompBlocks][col] * qsc : cb_global;
    const float mx = max_of_32(s[0], s[1]);
    const float mnew = fmaf(mx, a, cb);
    if (__ballot(mnew > m_ref) != 0ull) {
      // rare: keep it a real branch rather than 80 multiplies per tile
      asm volatile("" ::: "memory");
      const float mq = max_halves(mnew);
      const float mnext = mq > m_ref ? ceilf(mq) : m_ref;
      const float alpha = exp2_fast(m_ref - mnext);
      if (kVBlock) {
        lacc *= alpha;
        l_tot *= alpha;
      } else {
        rsum *= alpha;
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] *= alpha;
      m_ref = mnext;
    }
    if (kExpCast) {
      // bits of the byte map's value at z = 8 (t - m) + offset: one FMA to
      // z 2^20 + 120 2^23 (an integer-valued float, exact to 2^-14 in z), a
      // saturating convert to u32 (masked keys, -inf, give 0), the E4M3
      // rounding by the hardware convert.  t <= m keeps z <= 126.1, so the
      // code is at most 126, the code of 448.
      const float a20 = (8.0f * kTwo20) * a;
      const float b20 = fmaf(8.0f * (cb - m_ref) + kExpCastOffset, kTwo20, kBias120);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float v0 = __uint_as_float(cvt_u32_sat(fmaf(s[kb][4 * p], a20, b20)));
          const float v1 = __uint_as_float(cvt_u32_sat(fmaf(s[kb][4 * p + 1], a20, b20)));
          const float v2 = __uint_as_float(cvt_u32_sat(fmaf(s[kb][4 * p + 2], a20, b20)));
          const float v3 = __uint_as_float(cvt_u32_sat(fmaf(s[kb][4 * p + 3], a20, b20)));
          // the second convert fills the high half: start from v0's bits
          uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, (int)__float_as_uint(v0), false);
          pk[4 * kb + p] = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
        }
    } else {
      const float bias = cb + kLog2P8 - m_ref;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float e0 = exp2_fast(fmaf(s[kb][4 * p], a, bias));
          const float e1 = exp2_fast(fmaf(s[kb][4 * p + 1], a, bias));
          const float e2 = exp2_fast(fmaf(s[kb][4 * p + 2], a, bias));
          const float e3 = exp2_fast(fmaf(s[kb][4 * p + 3], a, bias));
          // the second convert fills the high half: start from e0's bits, not a zeroed register
          uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, (int)__float_as_uint(e0), false);
          pk[4 * kb + p] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
        }
    }
  };
  // O^T += V^T P^T (one 32x32x64 MFMA per 32-channel block) and the row sum
  // (with V block means: the weight sum of tile t's 128-token block, in the
  // output row of its slot k = (t / 2) % 16, row 4(k / 8) + 8((k % 8) / 4) +
  // k % 4, which lane (query, k / 8) holds in lacc[k % 8])
  auto pv = [&](const char* Vb, int t) __attribute__((always_inline)) {
    const i32x8 pb = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3],
                      (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const char* p = Vb + mb * 32 * kBc;
      const i32x8 av = join(*reinterpret_cast<const u32x4*>(p + voff[0]),
                            *reinterpret_cast<const u32x4*>(p + voff[1]));
      acc[mb] = mfma32x32x64_fp8(av, pb, acc[mb]);
    }
    if (kVBlock) {
      const int k = (t >> 1) & 15;
      const int r = 4 * (k >> 3) + 8 * ((k & 7) >> 2) + (k & 3);
      const int o = col == r ? 0x38383838 : 0;
      const i32x8 onehot = {o, o, o, o, o, o, o, o};
      lacc = mfma32x32x64_fp8(onehot, pb, lacc);
    } else {
      rsum = mfma16x16x128_fp8(sel, pb, rsum);
    }
  };

  // workgroup barrier that the compiler moves no memory access across
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- two wave groups in ping-pong (as in the bf16 kernel) ----
  // Phase P1(t): P8 of tile t (VALU); phase P2(t): S of tile t+1 and
  // O += P8(t) V(t) (MFMA), plus the K-mean batch for the next 32 tiles when
  // tile t+1 starts one.  Waves 4-7 run one phase behind waves 0-3; a barrier
  // ends every phase.  At the start of P2(t) every wave issues its share of
  // K(t+kRing) and V(t+kRing-1), into the buffers of K(t) and V(t-1), which
  // both groups have finished reading by then; every wave waits for all but
  // its newest kRing - 2 batches before each barrier, so a load has
  // 2 kRing - 3 phases to land.
  const bool group_a = wave < 4;
  // all but the newest kRing - 2 batches (two loads each): a batch issued in
  // phase 2 of step t is first read in phase 2 of step t + kRing - 1
  auto wait_loads = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4)
  };
  // exp-then-cast instances: the matrix phase's wave runs at a raised issue
  // priority (1.2% faster; ExpCast, whose exponential phase is shorter, runs
  // 0.7% slower with it and keeps one priority)
  auto phase1 = [&](int t) __attribute__((always_inline)) {
    if (!kExpCast) __builtin_amdgcn_s_setprio(0);
    if (kVBlock && (t % 32) == 0 && t > 0) vload((t >> 5) - 1);
    softmax_p(t);
    // consume P here: otherwise the exponentials are moved to their use
    // after the barrier, into the MFMA phase
    asm volatile("" ::"v"(pk[0]), "v"(pk[1]), "v"(pk[2]), "v"(pk[3]), "v"(pk[4]), "v"(pk[5]),
                 "v"(pk[6]), "v"(pk[7]));
    // (after the softmax, which reads step t's entry from pre_m)
    if (kMode == kSparse) {
      pre_k = lds_list[min(t + kRing, nkt - 1)];
      pre_v = lds_list[min(t + kRing - 1, nkt - 1)];
      pre_m = t + 1 < nkt ? (uint32_t)lds_list[t + 1] : 0u;
    }
    wait_loads();
    __builtin_amdgcn_sched_barrier(0);
    barrier();
  };
  auto phase2 = [&](int t, const char* kn, const char* vc, const void* kfill, const void* vfill)
                    __attribute__((always_inline)) {
    if (!kExpCast) __builtin_amdgcn_s_setprio(2);
    // batch t/32 - 1 is complete (its last P.V ran in the previous phase 2)
    if (kVBlock && (t % 32) == 0 && t > 0) {
      vdrain();
      __builtin_amdgcn_sched_barrier(0);
    }
    // block means of the batch that starts at step t + 4
    if (kStageKm && ((t + 4) % kCompBlocks) == 0 && t + 4 < nkt) km_issue(t + 4);
    // steps past the end reload the last tile into a free buffer
    issue_k(kMode == kSparse ? __builtin_amdgcn_readfirstlane((int)(pre_k & 0x3fffu)) : tile_of(t + kRing),
            kfill);
    issue_v(kMode == kSparse ? __builtin_amdgcn_readfirstlane((int)(pre_v & 0x3fffu))
                             : tile_of(t + kRing - 1),
            vfill);
    __builtin_amdgcn_sched_barrier(0);
    qk(kn);
    pv(vc, t);
    if constexpr (kVBlock && kExpCast) sched_reads_ahead<2>();
    // keys past the row limits (the ragged last tile, or the tile after the
    // last, whose scores come from reloaded data and must weigh nothing)
    mask_step(t + 1, pre_m);
    // (staged means: loaded by the end of phase 2 of step t - 1 and its
    // barrier, converted here two steps before their batch, read after the
    // next barrier)
    if (kStageKm && ((t + 2) % kCompBlocks) == 0 && t + 2 < nkt) km_convert();
    if (kBlockMean && ((t + 1) % kCompBlocks) == 0 && t + 1 < nkt) kmean_batch(t + 1);
    wait_loads();
    __builtin_amdgcn_sched_barrier(0);
    barrier();
  };

  // ---- prologue: K(0..kRing-1), V(0..kRing-2) in flight; S(0) ----
  issue_k(tile_of(0), lds_k0);
  issue_v(tile_of(0), lds_v0);
  issue_k(tile_of(1), lds_k1);
  issue_v(tile_of(1), lds_v1);
  issue_k(tile_of(2), lds_k2);
  issue_v(tile_of(2), lds_v2);
  issue_k(tile_of(3), lds_k3);
  if (kStageKm) km_issue(0);
  if (kBlockMean && !kStageKm) kmean_batch(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  barrier();
  if (kStageKm) {
    km_convert();
    barrier();
    kmean_batch(0);
  }
  qk(lds_k0);
  if (kMode == kSparse) pre_m = lds_list[0];
  mask_step(0, pre_m);
  if (!group_a) barrier();  // group B starts one phase later

  // kRing tiles per iteration, so every ring buffer is named statically.
  // Step t reads K(t+1) and V(t) and refills the buffers of K(t) and V(t-1)
  // with K(t+kRing) and V(t+kRing-1).
  int t = 0;
  for (; t + 4 <= nkt; t += 4) {
    phase1(t);
    phase2(t, lds_k1, lds_v0, lds_k0, lds_v3);
    phase1(t + 1);
    phase2(t + 1, lds_k2, lds_v1, lds_k1, lds_v0);
    phase1(t + 2);
    phase2(t + 2, lds_k3, lds_v2, lds_k2, lds_v1);
    phase1(t + 3);
    phase2(t + 3, lds_k0, lds_v3, lds_k3, lds_v2);
  }
  if (t < nkt) {
    phase1(t);
    phase2(t, lds_k1, lds_v0, lds_k0, lds_v3);
  }
  if (t + 1 < nkt) {
    phase1(t + 1);
    phase2(t + 1, lds_k2, lds_v1, lds_k1, lds_v0);
  }
  if (t + 2 < nkt) {
    phase1(t + 2);
    phase2(t + 2, lds_k3, lds_v2, lds_k2, lds_v1);
  }
  if (group_a) barrier();  // matches group B's extra one
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  if (kVBlock) {
    vload((nkt - 1) >> 5);
    vdrain();
  }
  const float lsum = kVBlock ? l_tot : rsum[0];
  // a row with no allowed key (block-sparse) has l = 0 and outputs zeros
  const bool empty_row = kMode == kSparse && lsum == 0.f;
  const float inv = empty_row ? 0.f : 1.0f / lsum;
  if (qok && kVBlock) {
    const float* vsh = v_scale + (size_t)bh * kHeadDim;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * half;
        const f32x4 vs = *reinterpret_cast<const f32x4*>(vsh + d0);
        u32x2 w;
        w.x = pack_bf16x2(acc[mb][4 * g] * inv * vs[0], acc[mb][4 * g + 1] * inv * vs[1]);
        w.y = pack_bf16x2(acc[mb][4 * g + 2] * inv * vs[2], acc[mb][4 * g + 3] * inv * vs[3]);
        *reinterpret_cast<u32x2*>(Oh + (size_t)qrow * kHeadDim + d0) = w;
      }
  } else if (qok) {
    const float* vsh = v_scale + (size_t)bh * kHeadDim;
    const float* vmh = v_mean + (size_t)bh * kHeadDim;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * half;
        const f32x4 vs = *reinterpret_cast<const f32x4*>(vsh + d0);
        f32x4 vm = *reinterpret_cast<const f32x4*>(vmh + d0);
        if (empty_row) vm = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x2 w;
        w.x = pack_bf16x2(fmaf(acc[mb][4 * g] * inv, vs[0], vm[0]),
                          fmaf(acc[mb][4 * g + 1] * inv, vs[1], vm[1]));
        w.y = pack_bf16x2(fmaf(acc[mb][4 * g + 2] * inv, vs[2], vm[2]),
                          fmaf(acc[mb][4 * g + 3] * inv, vs[3], vm[3]));
        *reinterpret_cast<u32x2*>(Oh + (size_t)qrow * kHeadDim + d0) = w;
      }
  }
}

template <bool kExpCast, bool kVBlock, int kMode>
void launch_fp8(bool block_mean, unsigned blocks, hipStream_t stream, const uint8_t* q,
                const uint8_t* k, const uint8_t* v, const float* q_scale, const float* k_scale,
                const float* k_mean, const float* v_mean, const uint16_t* v_bmean, int nbv_pad,
                const float* v_scale, uint16_t* out, int S, int n_qtiles, float c, int chunk,
                const uint8_t* mask, int nqb) {
  if (block_mean)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, kExpCast, kVBlock, kMode>), dim3(blocks),
                       dim3(kThreads), 0, stream, q, k, v, q_scale, k_scale, k_mean, v_mean,
                       v_bmean, nbv_pad, v_scale, out, S, n_qtiles, c, chunk, mask, nqb);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, kExpCast, kVBlock, kMode>), dim3(blocks),
                       dim3(kThreads), 0, stream, q, k, v, q_scale, k_scale, k_mean, v_mean,
                       v_bmean, nbv_pad, v_scale, out, S, n_qtiles, c, chunk, mask, nqb);
}

template <bool kExpCast>
void launch_fp8_mode(bool block_mean, bool vblock, int chunk, const uint8_t* mask, unsigned blocks,
                     hipStream_t stream, const uint8_t* q, const uint8_t* k, const uint8_t* v,
                     const float* q_scale, const float* k_scale, const float* k_mean,
                     const float* v_mean, const uint16_t* v_bmean, int nbv_pad,
                     const float* v_scale, uint16_t* out, int S, int n_qtiles, float c, int nqb) {
  if (vblock)
    launch_fp8<kExpCast, true, kDense>(block_mean, blocks, stream, q, k, v, q_scale, k_scale, k_mean,
                                       v_mean, v_bmean, nbv_pad, v_scale, out, S, n_qtiles, c, 0,
                                       nullptr, nqb);
  else if (mask)
    launch_fp8<kExpCast, false, kSparse>(block_mean, blocks, stream, q, k, v, q_scale, k_scale,
                                         k_mean, v_mean, v_bmean, nbv_pad, v_scale, out, S,
                                         n_qtiles, c, 0, mask, nqb);
  else if (chunk > 0)
    launch_fp8<kExpCast, false, kCausal>(block_mean, blocks, stream, q, k, v, q_scale, k_scale,
                                         k_mean, v_mean, v_bmean, nbv_pad, v_scale, out, S,
                                         n_qtiles, c, chunk, nullptr, nqb);
  else
    launch_fp8<kExpCast, false, kDense>(block_mean, blocks, stream, q, k, v, q_scale, k_scale,
                                        k_mean, v_mean, v_bmean, nbv_pad, v_scale, out, S, n_qtiles,
                                        c, 0, nullptr, nqb);
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                               const float* q_scale, const float* k_scale, const float* k_mean,
                               int k_mean_blocks, const float* v_mean, const void* v_bmean,
                               const float* v_scale, void* o, int B, int H, int S, float scale,
                               bool expcast, int chunk, const void* block_mask,
                               hipStream_t stream) {
  const int n_qtiles = (S + kBr - 1) / kBr;
  const unsigned blocks = (unsigned)((long long)B * H * n_qtiles);
  const int nb = (S + kBc - 1) / kBc;
  const bool block_mean = k_mean_blocks == nb && nb > 1;
  const uint8_t* q = static_cast<const uint8_t*>(q8);
  const uint8_t* k = static_cast<const uint8_t*>(k8);
  const uint8_t* v = static_cast<const uint8_t*>(v8);
  uint16_t* out = static_cast<uint16_t*>(o);
  const float c = scale * kLog2e;
  const uint16_t* vbm = static_cast<const uint16_t*>(v_bmean);
  const uint8_t* mask = static_cast<const uint8_t*>(block_mask);
  const int nbv_pad = vsmooth_blocks_padded(S);
  const int nqb = (S + 127) / 128;
  if (expcast)
    launch_fp8_mode<true>(block_mean, vbm != nullptr, chunk, mask, blocks, stream, q, k, v, q_scale,
                          k_scale, k_mean, v_mean, vbm, nbv_pad, v_scale, out, S, n_qtiles, c, nqb);
  else
    launch_fp8_mode<false>(block_mean, vbm != nullptr, chunk, mask, blocks, stream, q, k, v,
                           q_scale, k_scale, k_mean, v_mean, vbm, nbv_pad, v_scale, out, S,
                           n_qtiles, c, nqb);
  return hipGetLastError();
}

}  // namespace vdit
