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
//  * Ping-pong between the two waves of a SIMD.  Per 64-key tile a wave runs
//    an exponential phase (reference update, P = 2^(c s - m), VALU) and a
//    matrix phase (S of the next tile and O += P V, MFMA).  Waves 0-3 and
//    4-7 run one phase apart, so each SIMD overlaps one wave's exponentials
//    with the other wave's MFMAs; a workgroup barrier ends every phase.
//    Within a matrix phase every LDS operand read is issued six MFMAs ahead
//    of its use, and the wave runs at a raised issue priority (s_setprio) so
//    that the other wave's exponentials fill the MFMA wave's gaps rather than
//    delaying its MFMAs.
//  * K/V tiles go straight from global memory to LDS (global_load_lds_dwordx4,
//    no register staging) into three-deep rings.  Each load instruction
//    covers four whole 256-byte rows, so global reads are fully coalesced.
//    K is stored row-major with its 16-byte chunks XOR-swizzled by
//    (row & 15): the 16 lanes that the LDS serves together read 16 different
//    rows at 16 different bank groups.  V is stored row-major with its chunks
//    XOR-swizzled by 4*(row & 3) and read with ds_read_b64_tr_b16, which
//    hands each lane 4 keys of one channel; both reads are free of bank
//    conflicts.  The swizzles are applied by choosing which global chunk each
//    lane fetches, since the DMA writes 16 consecutive bytes per lane.
//  * Online softmax in the log2 domain with an integer running reference
//    m (ceil of the running maximum of scale*log2(e)*s): P = 2^(c s - m) <= 1,
//    and the accumulator is rescaled (by an exact power of two) only in the
//    rare tiles where some row's maximum exceeds its reference.  P is rounded
//    to bf16 once; the row sum adds exactly those rounded weights.
//  * Block-causal instance (chunk > 0): query i attends to key j iff
//    j / chunk <= i / chunk, i.e. to keys below lim(i) = min(S, (i/chunk + 1)
//    chunk).  A workgroup visits only the key tiles below the largest limit
//    of its rows; keys at or past a row's limit score -inf.  Query tiles are
//    dealt heaviest first.
//  * Ragged tails: rows of the last K/V tile past S are read from row S-1
//    (finite data), scored -inf, and so weigh exactly 0; queries >= S are
//    computed on zeros and not stored.
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kWaves = 8;
constexpr int kBr = 32 * kWaves;        // 256 queries per workgroup
constexpr int kBc = 64;                 // keys per K/V tile
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerWave = 16 / kWaves;  // 1 KB DMA loads per wave per tile and tensor
constexpr int kRowBytes = kHeadDim * 2;
constexpr int kTileBytes = kBc * kRowBytes;  // 16 KB

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// 8 keys x 1 channel for the V^T operand: two transposing 64-bit reads.
__device__ __forceinline__ bf16x8 read_v_operand(const char* p0, const char* p1) {
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  const s16x8_t v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// kMode: kDense (full attention), kCausal (block-causal by chunks of `chunk`
// tokens) or kSparse (block-sparse: block_mask[b,h,qb,kt] != 0 lets the 128
// queries of block qb see the 64 keys of tile kt; nqb = ceil(S / 128)).
constexpr int kDense = 0, kCausal = 1, kSparse = 2;
constexpr int kSparseQBlock = 128;
constexpr int kMaxSparseTiles = 16384;  // key tiles per head (S <= 1,048,576)

// Matrix-phase schedule: the reads of the first kLead operands, then MFMA i
// followed by the reads of operand i + kLead (operands 0-15 are one K read
// each, 16-31 two V reads each), then the last kLead MFMAs.
constexpr int kLead = 6;
constexpr int reads_of(int op) { return op < 16 ? 1 : 2; }
constexpr int reads_before(int n) { return n <= 0 ? 0 : reads_of(n - 1) + reads_before(n - 1); }
template <int L, int I = 0>
__device__ __forceinline__ void sched_reads_ahead() {
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, reads_before(L), 0);
  if constexpr (I < 32 - L) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, reads_of(I + L), 0);
    sched_reads_ahead<L, I + 1>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, L, 0);
  }
}

template <int kMode>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, int S, int n_qtiles, float c,
    int chunk, const uint8_t* __restrict__ block_mask, int nqb) {
  // three-deep rings of K and V tiles, one LDS object per buffer
  __shared__ __attribute__((aligned(1024))) char lds_k0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v2[kTileBytes];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  // heaviest query tiles first (they see the most keys when block-causal)
  const int qt = n_qtiles - 1 - (tile - bh * n_qtiles);
  const size_t base = (size_t)bh * S * kHeadDim;
  const char* Kh = reinterpret_cast<const char*>(K + base);
  const char* Vh = reinterpret_cast<const char*>(V + base);
  uint16_t* Oh = O + base;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qt * kBr + wave * 32 + col;
  const int nkt_all = (S + kBc - 1) / kBc;
  const bool tail = (S % kBc) != 0;
  // key limits: this lane's row, this wave's first (smallest) row, and the
  // workgroup's last valid row (the largest)
  // (a run-time test on chunk, not on kMode: the dense instance compiled from
  // the compile-time form schedules its loop worse and runs 1-4% slower)
  auto key_limit = [&](int row) { return chunk > 0 ? min(S, (row / chunk + 1) * chunk) : S; };
  const int lim = key_limit(min(qrow, S - 1));
  const int wave_lim = key_limit(min(qt * kBr + wave * 32, S - 1));
  int nkt = (key_limit(min(qt * kBr + kBr - 1, S - 1)) + kBc - 1) / kBc;

  // Block-sparse: the key tiles this workgroup visits, in ascending order:
  // the union of the tiles allowed to its two 128-query blocks, each entry
  // kt | (query blocks allowing it) << 14.  A wave (32 rows, one query block)
  // scores a tile its block does not allow as -inf.
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
      if (qrow < S)
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
  // tiles of K(t+3) and V(t+2), the mask of step t+1), read in the
  // exponential phase before it so that the matrix phase does not wait on LDS
  uint32_t pre_k = 0, pre_v = 0, pre_m = 0;
  auto prefetch_list = [&](int t) __attribute__((always_inline)) {
    if (kMode == kSparse) {
      pre_k = lds_list[min(t + 3, nkt - 1)];
      pre_v = lds_list[min(t + 2, nkt - 1)];
      pre_m = t + 1 < nkt ? (uint32_t)lds_list[t + 1] : 0u;
    }
  };

  // ---- per-lane constant offsets ----
  // K and V loads: wave w, load i covers tile rows 8w + 4i + lane/16; lane
  // writes physical chunk lane%16 of its row, so it fetches the logical chunk
  // that the row's swizzle maps there.
  const int lrow0 = 4 * kLoadsPerWave * wave + (lane >> 4);  // + 4i
  const int pchunk = lane & 15;
  int kgo[kLoadsPerWave], vgo[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int r = lrow0 + 4 * i;
    kgo[i] = r * kRowBytes + 16 * (pchunk ^ (r & 15));
    vgo[i] = r * kRowBytes + 16 * (pchunk ^ (4 * (r & 3)));
  }
  // K operand: lane (key = 32kb + col, half) reads chunk 2kk + half of its
  // key, stored at physical chunk (2kk + half) ^ (key & 15)
  int koff[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = col * kRowBytes + 16 * ((2 * kk + half) ^ (col & 15));
  // V operand: 16-lane group g = lane/16, s = lane%16 reads row
  // 16kc + 8r + 4(g>>1) + s/4, channels 32mb + 16(g&1) + 4(s%4) .. +3.
  const int g = lane >> 4, s16 = lane & 15;
  const int vrow = 4 * (g >> 1) + (s16 >> 2);
  const int vx = 2 * (g & 1) + ((s16 >> 1) & 1);
  int voff[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
    voff[mb] = vrow * kRowBytes + 16 * (4 * (mb ^ (s16 >> 2)) + vx) + 8 * (s16 & 1);

  const uint32_t wslice = (uint32_t)wave * (4 * kLoadsPerWave * kRowBytes);
  // DMA of key tile t (an index into K and V, not a loop step)
  auto issue_k = [&](int t, const void* buf) __attribute__((always_inline)) {
    const int key0 = t * kBc;
    const char* src = Kh + (size_t)key0 * kRowBytes;
    const uint32_t dst = lds_addr(buf) + wslice;
    if (tail && t == nkt_all - 1) {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int r = lrow0 + 4 * i;
        const int row = min(key0 + r, S - 1);
        const int go = (row - key0) * kRowBytes + 16 * (pchunk ^ (r & 15));
        dma16(src, (uint32_t)go, dst + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) dma16(src, (uint32_t)kgo[i], dst + i * 1024);
    }
  };
  auto issue_v = [&](int t, const void* buf) __attribute__((always_inline)) {
    const int key0 = t * kBc;
    const char* src = Vh + (size_t)key0 * kRowBytes;
    const uint32_t dst = lds_addr(buf) + wslice;
    if (tail && t == nkt_all - 1) {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int r = lrow0 + 4 * i;
        const int row = min(key0 + r, S - 1);
        const int go = (row - key0) * kRowBytes + 16 * (pchunk ^ (4 * (r & 3)));
        dma16(src, (uint32_t)go, dst + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) dma16(src, (uint32_t)vgo[i], dst + i * 1024);
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

  f32x16 s[2];  // S^T of one tile: key block kb, lane (q, half): keys 32kb + 8(i/4) + 4half + i%4
  auto qk = [&](const char* Kb) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + 32 * kRowBytes * kb + koff[kk]);
        s[kb] = mfma32x32x16_bf16(a, qf[kk], s[kb]);
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

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  // integer-valued log2-domain reference (finite when block-sparse, so that
  // tiles scored entirely -inf before a row's first allowed key give 0, not NaN)
  float m_ref = kMode == kSparse ? -1e30f : -INFINITY;
  float l4[4] = {0.f, 0.f, 0.f, 0.f};

  // Reference update and (rare) rescale.  In the common case only the
  // lane-local maximum is formed and compared with the reference.
  auto update_max = [&]() __attribute__((always_inline)) {
    const float mx = max_of_32(s[0], s[1]) * c;
    if (__ballot(mx > m_ref) != 0ull) {
      // rare: keep it a real branch rather than 64 multiplies per tile
      asm volatile("" ::: "memory");
      const float mq = max_halves(mx);
      const float mnext = mq > m_ref ? ceilf(mq) : m_ref;
      const float alpha = exp2_fast(m_ref - mnext);
#pragma unroll
      for (int u = 0; u < 4; ++u) l4[u] *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] *= alpha;
      m_ref = mnext;
    }
  };

  // P = bf16(2^(c s - m)) packed in S^T register order; l += sum of P.
  uint32_t pk[2][8];
  auto softmax_p = [&]() __attribute__((always_inline)) {
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
  auto pv = [&](const char* Vb) __attribute__((always_inline)) {
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

  // workgroup barrier that the compiler moves no instruction across (the
  // exponentials of the next phase would otherwise be hoisted above it)
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- two wave groups in ping-pong ----
  // Waves 0-3 (group A, one per SIMD) and 4-7 (group B) run the same
  // sequence of phases, B one phase behind A, so that while one wave of a
  // SIMD is in its exponential phase (VALU) the other is in its matrix phase
  // (MFMA).  Phase P1(t): reference update and P = 2^(c s - m) of tile t;
  // phase P2(t): S of tile t+1 (QK^T) and O += P(t) V(t).  A barrier ends
  // every phase.  K and V tiles live in three-deep rings; at the start of
  // P2(t) every wave issues its share of K(t+3) and V(t+2), into the
  // buffers of K(t) and V(t-1), which both groups have finished reading by
  // then.  Each wave waits for all but its newest batch of loads before
  // every barrier, so a load has at least two phases to land before the
  // barrier that precedes its first use.
  const bool group_a = wave < 4;
  auto phase1 = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
    prefetch_list(t);
    update_max();
    softmax_p();
    // consume P here: otherwise the exponentials are moved to their use
    // after the barrier, into the MFMA phase
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      asm volatile("" ::"v"(pk[kb][0]), "v"(pk[kb][1]), "v"(pk[kb][2]), "v"(pk[kb][3]), "v"(pk[kb][4]),
                   "v"(pk[kb][5]), "v"(pk[kb][6]), "v"(pk[kb][7]));
    __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4): all but the newest batch
    __builtin_amdgcn_sched_barrier(0);
    barrier();
  };
  auto phase2 = [&](int t, const char* kn, const char* vc, const void* kfill, const void* vfill)
                    __attribute__((always_inline)) {
    // the matrix phase's wave takes the SIMD's issue slots first: 1.5%
    // faster dense, 7% block-sparse (the reverse order: 1.4% slower)
    __builtin_amdgcn_s_setprio(2);
    // steps past the end reload the last tile into a free buffer
    issue_k(kMode == kSparse ? __builtin_amdgcn_readfirstlane((int)(pre_k & 0x3fffu)) : tile_of(t + 3),
            kfill);
    issue_v(kMode == kSparse ? __builtin_amdgcn_readfirstlane((int)(pre_v & 0x3fffu)) : tile_of(t + 2),
            vfill);
    __builtin_amdgcn_sched_barrier(0);
    qk(kn);
    pv(vc);
    // Keep every operand read kLead MFMAs ahead of its use across the 32
    // MFMAs of the phase (16 K operands of one read, then 16 V operands of
    // two): the default schedule reads each operand just before its MFMA,
    // which leaves a lone wave waiting on LDS latency.
    sched_reads_ahead<kLead>();
    // keys past S (the ragged last tile, or the tile after the last, whose
    // scores come from reloaded data and must weigh nothing)
    if (kMode == kSparse)
      mask_sparse(pre_m);
    else if ((t + 1) * kBc + kBc > wave_lim)
      mask_tail(t + 1);
    __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4)
    __builtin_amdgcn_sched_barrier(0);
    barrier();
  };

  // ---- prologue: K(0..2), V(0..1) in flight; S(0) ----
  issue_k(tile_of(0), lds_k0);
  issue_v(tile_of(0), lds_v0);
  issue_k(tile_of(1), lds_k1);
  issue_v(tile_of(1), lds_v1);
  issue_k(tile_of(2), lds_k2);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  barrier();
  qk(lds_k0);
  if (kMode == kSparse)
    mask_sparse(lds_list[0]);
  else if (kBc > wave_lim)
    mask_tail(0);
  if (!group_a) barrier();  // group B starts one phase later

  // three tiles per iteration, so every ring buffer is named statically
  int t = 0;
  for (; t + 3 <= nkt; t += 3) {
    phase1(t);
    phase2(t, lds_k1, lds_v0, lds_k0, lds_v2);
    phase1(t + 1);
    phase2(t + 1, lds_k2, lds_v1, lds_k1, lds_v0);
    phase1(t + 2);
    phase2(t + 2, lds_k0, lds_v2, lds_k2, lds_v1);
  }
  if (t < nkt) {
    phase1(t);
    phase2(t, lds_k1, lds_v0, lds_k0, lds_v2);
  }
  if (t + 1 < nkt) {
    phase1(t + 1);
    phase2(t + 1, lds_k2, lds_v1, lds_k1, lds_v0);
  }
  if (group_a) barrier();  // matches group B's extra one
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  const float lsum = sum_halves((l4[0] + l4[1]) + (l4[2] + l4[3]));
  // a row with no allowed key (block-sparse) has l = 0 and outputs zeros
  const float inv = (kMode == kSparse && lsum == 0.f) ? 0.f : 1.0f / lsum;
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
                                int B, int H, int S, float scale, int chunk,
                                const void* block_mask, hipStream_t stream) {
  const int n_qtiles = (S + kBr - 1) / kBr;
  const long long blocks = (long long)B * H * n_qtiles;
  const int nqb = (S + kSparseQBlock - 1) / kSparseQBlock;
  auto kernel = block_mask  ? attn_fwd_bf16_kernel<kSparse>
                : chunk > 0 ? attn_fwd_bf16_kernel<kCausal>
                            : attn_fwd_bf16_kernel<kDense>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), S, n_qtiles,
                     scale * kLog2e, chunk, static_cast<const uint8_t*>(block_mask), nqb);
  return hipGetLastError();
}

int bf16_sparse_max_tiles() { return kMaxSparseTiles; }

}  // namespace vdit
