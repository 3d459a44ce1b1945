// fp8 pre-pass: quantise and smooth bf16 Q, K, V into E4M3 codes, scales and
// means for the fp8 attention kernel.
//
// V-Smooth (VC-Attention article (aikraft.ru), section 02): subtract a mean,
// quantise only the residual per channel in E4M3; the mean is added back in
// the attention epilogue.  Q/K smoothing before the low-bit QK^T (section 01):
// K loses the mean of each 64-token block (or one mean per head), Q and the
// K residual get one E4M3 scale per 64-token block.  The article fuses its
// pre-processing into one kernel (section 04); here it is three HBM-bound
// launches because the V statistics span the whole sequence:
//   1. per (b,h, 64-token block): Q codes + scale; K block mean, residual
//      codes + scale (block mode) or K partial sums (global mode); V partial
//      sum / min / max per channel  -> workspace
//   2. per (b,h) and 16 channels: reduce the V (and global K) partials ->
//      v_mean, v_scale, 1/scale (workspace), k_mean (global mode)
//   3. per (b,h) and run of 4 blocks: V residual codes; K residual codes
//      (global mode)
//
// With block means for V (the article's own Demean: one mean per channel
// and hardware block of 128 tokens) launch 2 forms, per 128-token block, the
// mean from the two 64-token partial sums, rounds it to bf16 (the 16-bit
// mean: 0.125 bit per value element) and the block's residual range from its
// minima and maxima; the per-channel scale covers the residual over the whole
// sequence.  Launch 3 subtracts each token's block mean.  The means are
// written channel-major, [b,h][channel][block], padded with zeros to a
// multiple of 16 blocks: the attention kernel restores them 16 blocks at a
// time.
//
// V codes are written as the attention kernel reads them: per (b,h) and
// 64-token block one 8 KB tile of 128 channel rows x 64 key slots, slot s of
// a row holding key 32((s>>4)&1) + 8((s>>2)&3) + 4(s>>5) + (s&3) of the block
// (the order of the P^T operand of the 32x32x64 fp8 MFMA), with the four
// 16-byte chunks of a row XOR-swizzled by (channel >> 2) & 3 so that the
// kernel's LDS reads are free of bank conflicts.  Keys past S are code 0.
//
// Integer-valued decisions are taken in a stated precision so they can be
// checked bit for bit: sums of bf16 values in fp64 (exact for these inputs),
// mean = fp32(sum / n), residual = fp32(x - mean), scale = fp32(amax / 448)
// and inv = fp32(448 / amax) from fp64 quotients (1 and 0 when amax = 0),
// code = E4M3 round-to-nearest-even of clamp(fp32(r * inv), +-448) (by the
// hardware convert: the same codes as a software encoder of that rule on
// every tie, subnormal and zero tried); the
// 16-bit V block mean is bf16(fp32 mean), nearest even, and the residual is
// taken against it.
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kBlock = 64;     // tokens per block
constexpr int kThreads = 256;  // 16 row groups x 16 chunks of 8 channels

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 (one 16-byte chunk) -> 8 floats
__device__ __forceinline__ void unpack8(u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

// E4M3 codes of four values (|x| <= 448), low byte first: the hardware
// OCP E4M3 convert, round to nearest even, subnormals on the 2^-9 grid, the
// sign kept on zero (-0 and negatives that round to zero give 0x80)
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)lo, true);
}

// 8 codes of f[0..7] * inv -> two packed dwords
__device__ __forceinline__ u32x2 encode8(const float* f, float inv) {
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = clamp448(__fmul_rn(f[i], inv));
  u32x2 r;
  r.x = e4m3x4(c[0], c[1], c[2], c[3]);
  r.y = e4m3x4(c[4], c[5], c[6], c[7]);
  return r;
}

// float -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// max over the workgroup of a per-thread value (all threads get it)
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ void scales_from_amax(float amax, float* scale, float* inv) {
  if (amax == 0.0f) {
    *scale = 1.0f;
    *inv = 0.0f;
  } else {
    *scale = (float)((double)amax / 448.0);
    *inv = (float)(448.0 / (double)amax);
  }
}

struct Workspace {
  double* v_sum;  // [BH][nb][D]
  float* v_min;   // [BH][nb][D]
  float* v_max;   // [BH][nb][D]
  float* v_inv;   // [BH][D]
  double* k_sum;  // [BH][nb][D] (global K mean only)
};

// Launch 1: one workgroup per (bh, block).
__global__ __launch_bounds__(kThreads) void quant_blocks_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint8_t* __restrict__ Q8, uint8_t* __restrict__ K8, float* __restrict__ q_scale,
    float* __restrict__ k_scale, float* __restrict__ k_mean, Workspace ws, int S, int nb,
    int k_global) {
  __shared__ double red_d[16][kHeadDim];
  __shared__ float red_f[2][16][kHeadDim];
  __shared__ float mean_s[kHeadDim];
  __shared__ float red[4];

  const int bh = blockIdx.x / nb;
  const int blk = blockIdx.x - bh * nb;
  const int tid = threadIdx.x;
  const int c = tid & 15, rg = tid >> 4;
  const int row0 = blk * kBlock;
  const int nvalid = min(kBlock, S - row0);
  const size_t head = (size_t)bh * S * kHeadDim;

  float q[4][8], k[4][8], v[4][8];
  bool ok[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = rg + 16 * p;
    ok[p] = r < nvalid;
    const size_t off = head + (size_t)(row0 + r) * kHeadDim + 8 * c;
    unpack8(ld16(Q + off, ok[p]), q[p]);
    unpack8(ld16(K + off, ok[p]), k[p]);
    unpack8(ld16(V + off, ok[p]), v[p]);
  }

  // ---- V partial statistics over this block's valid rows ----
  {
    double s[8];
    float mn[8], mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s[i] = 0.0;
      mn[i] = INFINITY;
      mx[i] = -INFINITY;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (ok[p]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          s[i] += (double)v[p][i];
          mn[i] = fminf(mn[i], v[p][i]);
          mx[i] = fmaxf(mx[i], v[p][i]);
        }
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      red_d[rg][8 * c + i] = s[i];
      red_f[0][rg][8 * c + i] = mn[i];
      red_f[1][rg][8 * c + i] = mx[i];
    }
    __syncthreads();
    if (tid < kHeadDim) {
      double ts = 0.0;
      float tmn = INFINITY, tmx = -INFINITY;
      for (int g = 0; g < 16; ++g) {
        ts += red_d[g][tid];
        tmn = fminf(tmn, red_f[0][g][tid]);
        tmx = fmaxf(tmx, red_f[1][g][tid]);
      }
      const size_t o = ((size_t)bh * nb + blk) * kHeadDim + tid;
      ws.v_sum[o] = ts;
      ws.v_min[o] = tmn;
      ws.v_max[o] = tmx;
    }
    __syncthreads();
  }

  // ---- K: block mean (block mode) or partial sums (global mode) ----
  {
    double s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.0;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (ok[p]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += (double)k[p][i];
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) red_d[rg][8 * c + i] = s[i];
    __syncthreads();
    if (tid < kHeadDim) {
      double ts = 0.0;
      for (int g = 0; g < 16; ++g) ts += red_d[g][tid];
      if (k_global) {
        ws.k_sum[((size_t)bh * nb + blk) * kHeadDim + tid] = ts;
      } else {
        const float m = (float)(ts / (double)nvalid);
        mean_s[tid] = m;
        k_mean[((size_t)bh * nb + blk) * kHeadDim + tid] = m;
      }
    }
    __syncthreads();
  }

  // ---- Q codes (no smoothing) ----
  {
    float a = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, ok[p] ? fabsf(q[p][i]) : 0.f);
    const float amax = block_max(a, red);
    float sc, inv;
    scales_from_amax(amax, &sc, &inv);
    if (tid == 0) q_scale[(size_t)bh * nb + blk] = sc;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (ok[p])
        *reinterpret_cast<u32x2*>(Q8 + head + (size_t)(row0 + rg + 16 * p) * kHeadDim + 8 * c) =
            encode8(q[p], inv);
  }

  // ---- K residual codes (block mode) ----
  if (!k_global) {
    float a = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        k[p][i] = __fsub_rn(k[p][i], mean_s[8 * c + i]);
        a = fmaxf(a, ok[p] ? fabsf(k[p][i]) : 0.f);
      }
    const float amax = block_max(a, red);
    float sc, inv;
    scales_from_amax(amax, &sc, &inv);
    if (tid == 0) k_scale[(size_t)bh * nb + blk] = sc;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (ok[p])
        *reinterpret_cast<u32x2*>(K8 + head + (size_t)(row0 + rg + 16 * p) * kHeadDim + 8 * c) =
            encode8(k[p], inv);
  }
}

// Launch 2: one workgroup per (bh, group of kReduceChans channels), of
// kReduceParts x kReduceChans threads; thread (part, channel) folds the
// channel over the blocks b = part (mod kReduceParts), and the threads of
// part 0 combine the parts in part order.  The fp64 sums of bf16 values are
// exact, so the grouping does not change them.
// With v_bmean (block mode) thread (part, channel) handles the 128-token
// blocks b = part (mod kReduceParts): mean, its bf16 rounding, and the
// block's residual range.
constexpr int kReduceChans = 16;
constexpr int kReduceParts = 64;
__global__ __launch_bounds__(kReduceParts * kReduceChans) void quant_reduce_kernel(
    float* __restrict__ v_mean, float* __restrict__ v_scale, float* __restrict__ k_mean,
    uint16_t* __restrict__ v_bmean, int nbv_pad, Workspace ws, int S, int nb, int k_global) {
  __shared__ float ram[kReduceParts][kReduceChans];
  __shared__ double rs[kReduceParts][kReduceChans];
  __shared__ double rk[kReduceParts][kReduceChans];
  __shared__ float rmn[kReduceParts][kReduceChans], rmx[kReduceParts][kReduceChans];
  constexpr int kGroups = kHeadDim / kReduceChans;
  const int bh = blockIdx.x / kGroups;
  const int dl = threadIdx.x % kReduceChans, part = threadIdx.x / kReduceChans;
  const int d = (blockIdx.x - bh * kGroups) * kReduceChans + dl;
  double s = 0.0, sk = 0.0;
  float mn = INFINITY, mx = -INFINITY;
  for (int b = part; b < nb; b += kReduceParts) {
    const size_t o = ((size_t)bh * nb + b) * kHeadDim + d;
    s += ws.v_sum[o];
    mn = fminf(mn, ws.v_min[o]);
    mx = fmaxf(mx, ws.v_max[o]);
    if (k_global) sk += ws.k_sum[o];
  }
  rs[part][dl] = s;
  rk[part][dl] = sk;
  rmn[part][dl] = mn;
  rmx[part][dl] = mx;
  if (v_bmean) {
    const int nbv = (S + 2 * kBlock - 1) / (2 * kBlock);
    uint16_t* vb = v_bmean + ((size_t)bh * kHeadDim + d) * nbv_pad;
    float am = 0.0f;
    for (int b = part; b < nbv_pad; b += kReduceParts) {
      if (b >= nbv) {
        vb[b] = 0;
        continue;
      }
      const size_t o = ((size_t)bh * nb + 2 * b) * kHeadDim + d;
      const bool two = 2 * b + 1 < nb;
      const double bs = ws.v_sum[o] + (two ? ws.v_sum[o + kHeadDim] : 0.0);
      const float lo = two ? fminf(ws.v_min[o], ws.v_min[o + kHeadDim]) : ws.v_min[o];
      const float hi = two ? fmaxf(ws.v_max[o], ws.v_max[o + kHeadDim]) : ws.v_max[o];
      const int n = min(2 * kBlock, S - 2 * kBlock * b);
      const uint32_t mb = bf16_bits_rne((float)(bs / (double)n));
      const float m16 = __uint_as_float(mb << 16);
      vb[b] = (uint16_t)mb;
      am = fmaxf(am, fmaxf(fabsf(__fsub_rn(hi, m16)), fabsf(__fsub_rn(lo, m16))));
    }
    ram[part][dl] = am;
  }
  __syncthreads();
  if (part != 0) return;
  double ssum = 0.0, sksum = 0.0;
  float lo = INFINITY, hi = -INFINITY, amb = 0.0f;
  for (int p = 0; p < kReduceParts; ++p) {
    ssum += rs[p][dl];
    sksum += rk[p][dl];
    lo = fminf(lo, rmn[p][dl]);
    hi = fmaxf(hi, rmx[p][dl]);
    if (v_bmean) amb = fmaxf(amb, ram[p][dl]);
  }
  if (k_global) k_mean[(size_t)bh * kHeadDim + d] = (float)(sksum / (double)S);
  float sc, inv;
  if (v_bmean) {
    scales_from_amax(amb, &sc, &inv);
  } else {
    const float mean = (float)(ssum / (double)S);
    // fp32 subtraction is monotone, so this is max_j |fp32(v_j - mean)|
    const float amax = fmaxf(fabsf(__fsub_rn(hi, mean)), fabsf(__fsub_rn(lo, mean)));
    scales_from_amax(amax, &sc, &inv);
    v_mean[(size_t)bh * kHeadDim + d] = mean;
  }
  v_scale[(size_t)bh * kHeadDim + d] = sc;
  ws.v_inv[(size_t)bh * kHeadDim + d] = inv;
}

// Launch 3: one workgroup per (bh, run of kResidualRun blocks): V residual
// codes, and K residual codes + scale when K uses one global mean.  The
// workgroup walks its blocks in order with the next block's V rows already
// in flight, and the channel-major tile alternates between two LDS buffers,
// so one barrier per block separates its writes from its reads.
constexpr int kResidualRun = 4;
__global__ __launch_bounds__(kThreads) void quant_residual_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, uint8_t* __restrict__ K8,
    uint8_t* __restrict__ V8, float* __restrict__ k_scale, const float* __restrict__ k_mean,
    const float* __restrict__ v_mean, const uint16_t* __restrict__ v_bmean, int nbv_pad,
    Workspace ws, int S, int nb, int k_global) {
  __shared__ float red[4];
  // codes channel-major, [channel][key], rows padded to 68 bytes so that the
  // transposing reads below spread over the banks
  constexpr int kRowT = kBlock + 4;
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kHeadDim * kRowT];
  const int runs = (nb + kResidualRun - 1) / kResidualRun;
  const int bh = blockIdx.x / runs;
  const int blk0 = (blockIdx.x - bh * runs) * kResidualRun;
  const int blk_end = min(nb, blk0 + kResidualRun);
  const int tid = threadIdx.x;
  const int c = tid & 15, rg = tid >> 4;
  const size_t head = (size_t)bh * S * kHeadDim;
  float vm[8], vi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    vm[i] = v_bmean ? 0.f : v_mean[(size_t)bh * kHeadDim + 8 * c + i];
    vi[i] = ws.v_inv[(size_t)bh * kHeadDim + 8 * c + i];
  }
  // thread (row group rg, chunk c): keys 4rg .. 4rg+3 of channels 8c .. 8c+7
  // (keys past S: zero rows)
  auto load_v = [&](int blk, u32x4* w) __attribute__((always_inline)) {
    const int nvalid = min(kBlock, S - blk * kBlock);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 4 * rg + p;
      w[p] = ld16(V + head + (size_t)(blk * kBlock + r) * kHeadDim + 8 * c, r < nvalid);
    }
  };
  u32x4 cur[4], nxt[4] = {};
  load_v(blk0, cur);
  for (int blk = blk0, buf = 0; blk < blk_end; ++blk, buf ^= 1) {
    if (blk + 1 < blk_end) load_v(blk + 1, nxt);
    const int nvalid = min(kBlock, S - blk * kBlock);
    // (a V block mean spans two 64-token blocks)
    if (v_bmean && ((blk & 1) == 0 || blk == blk0)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vm[i] = __uint_as_float((uint32_t)v_bmean[((size_t)bh * kHeadDim + 8 * c + i) * nbv_pad + (blk >> 1)]
                                << 16);
    }
    // residual codes, one 4-key word per channel (keys past S: +0, code 0)
    float rv[4][8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool ok = 4 * rg + p < nvalid;
      float f[8];
      unpack8(cur[p], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[p][i] = ok ? clamp448(__fmul_rn(__fsub_rn(f[i], vm[i]), vi[i])) : 0.0f;
    }
    uint8_t* tl = tile[buf];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint32_t*>(&tl[(8 * c + i) * kRowT + 4 * rg]) =
          e4m3x4(rv[0][i], rv[1][i], rv[2][i], rv[3][i]);
    __syncthreads();
    // transpose into the kernel's tile: thread -> (channel d, physical chunk pc)
    {
      uint8_t* V8t = V8 + ((size_t)bh * nb + blk) * (kBlock * kHeadDim);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int idx = tid + kThreads * h;  // 0 .. 511
        const int d = idx >> 2, pc = idx & 3;
        const int lc = pc ^ ((d >> 2) & 3);
        // slots 16lc + 4q + b hold keys 32(lc & 1) + 8q + 4(lc >> 1) + b: four
        // consecutive keys, one aligned word of the channel-major tile
        uint32_t wd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          wd[q] = *reinterpret_cast<const uint32_t*>(&tl[d * kRowT + 32 * (lc & 1) + 8 * q + 4 * (lc >> 1)]);
        *reinterpret_cast<u32x4*>(V8t + d * kBlock + 16 * pc) = u32x4{wd[0], wd[1], wd[2], wd[3]};
      }
    }
    if (k_global) {
      const int row0 = blk * kBlock;
      float km[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) km[i] = k_mean[(size_t)bh * kHeadDim + 8 * c + i];
      float k[4][8];
      float a = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = rg + 16 * p;
        const bool ok = r < nvalid;
        unpack8(ld16(K + head + (size_t)(row0 + r) * kHeadDim + 8 * c, ok), k[p]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          k[p][i] = __fsub_rn(k[p][i], km[i]);
          a = fmaxf(a, ok ? fabsf(k[p][i]) : 0.f);
        }
      }
      const float amax = block_max(a, red);
      float sc, inv;
      scales_from_amax(amax, &sc, &inv);
      if (tid == 0) k_scale[(size_t)bh * nb + blk] = sc;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (rg + 16 * p < nvalid)
          *reinterpret_cast<u32x2*>(K8 + head + (size_t)(row0 + rg + 16 * p) * kHeadDim + 8 * c) =
              encode8(k[p], inv);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) cur[p] = nxt[p];
  }
}

Workspace carve(void* base, int BH, int nb, int k_global) {
  const size_t n = (size_t)BH * nb * kHeadDim;
  char* p = static_cast<char*>(base);
  Workspace ws;
  ws.v_sum = reinterpret_cast<double*>(p);
  p += n * sizeof(double);
  ws.k_sum = k_global ? reinterpret_cast<double*>(p) : nullptr;
  if (k_global) p += n * sizeof(double);
  ws.v_min = reinterpret_cast<float*>(p);
  p += n * sizeof(float);
  ws.v_max = reinterpret_cast<float*>(p);
  p += n * sizeof(float);
  ws.v_inv = reinterpret_cast<float*>(p);
  return ws;
}

}  // namespace

size_t quant_fp8_workspace_bytes(int B, int H, int S, int k_mean_blocks) {
  const int nb = (S + kBlock - 1) / kBlock;
  const int k_global = (k_mean_blocks == 1 && nb > 1) ? 1 : 0;
  const size_t n = (size_t)B * H * nb * kHeadDim;
  return n * sizeof(double) * (k_global ? 2 : 1) + n * sizeof(float) * 2 +
         (size_t)B * H * kHeadDim * sizeof(float);
}

hipError_t launch_quant_fp8(const void* q, const void* k, const void* v, void* q8, void* k8,
                            void* v8, float* q_scale, float* k_scale, float* k_mean,
                            int k_mean_blocks, float* v_mean, void* v_bmean, float* v_scale,
                            void* workspace, int B, int H, int S, hipStream_t stream) {
  const int nb = (S + kBlock - 1) / kBlock;
  const int BH = B * H;
  // With a single block the block mean is the global mean.
  const int k_global = (k_mean_blocks == 1 && nb > 1) ? 1 : 0;
  const Workspace ws = carve(workspace, BH, nb, k_global);
  const unsigned grid = (unsigned)((size_t)BH * nb);
  hipLaunchKernelGGL(quant_blocks_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint8_t*>(q8),
                     static_cast<uint8_t*>(k8), q_scale, k_scale, k_mean, ws, S, nb, k_global);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint16_t* vbm = static_cast<uint16_t*>(v_bmean);
  const int nbv_pad = vsmooth_blocks_padded(S);
  hipLaunchKernelGGL(quant_reduce_kernel, dim3((unsigned)BH * (kHeadDim / kReduceChans)),
                     dim3(kReduceParts * kReduceChans), 0, stream, v_mean, v_scale,
                     k_mean, vbm, nbv_pad, ws, S, nb, k_global);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int runs = (nb + kResidualRun - 1) / kResidualRun;
  hipLaunchKernelGGL(quant_residual_kernel, dim3((unsigned)((size_t)BH * runs)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<uint8_t*>(k8), static_cast<uint8_t*>(v8), k_scale, k_mean, v_mean,
                     vbm, nbv_pad, ws, S, nb, k_global);
  return hipGetLastError();
}

}  // namespace vdit
