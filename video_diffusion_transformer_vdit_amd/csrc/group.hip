// V-Smooth Group (VC-Attention article (aikraft.ru), section 02, Group):
// k-means of the value tokens of every (b,h), and the stable permutation
// that lists the tokens cluster by cluster.  Keys and values permuted by the
// same permutation leave non-causal attention unchanged, and the 128-token
// block means of the grouped values take out far more of the block energy
// than in sequence order, which is what the block demean of V-Smooth needs.
//
// Lloyd's algorithm with a fixed number of rounds, every step deterministic
// (no floating-point atomics; every sum in a fixed order):
//   init     centroid c = token floor(c * S / k)
//   assign   label = argmin_c |mu_c|^2 - 2 v . mu_c, ties to the lowest c.
//            v . mu_c on bf16 MFMAs: v is exact in bf16 and mu (fp32) is
//            split into a bf16 high part and a bf16 residual (about 2^-16).
//   sort     counting sort of the labels: per 1024-token chunk histograms
//            (integer LDS atomics), one scan per (b,h), then each chunk
//            places its tokens in token order, so the order is stable
//   update   mu_c = mean of the tokens of cluster c, summed in token order in
//            fp32 (an empty cluster keeps its centroid); |mu_c|^2 in fp32
// Rounds: init, then `rounds` x (assign, sort, update), then a final
// assign + sort, whose permutation and labels are returned with the last
// centroids.
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kChunk = 1024;      // tokens per histogram / placement chunk
constexpr int kAssignWaves = 8;   // 8 x 64 tokens per assignment workgroup

struct GroupWs {
  uint16_t* muh;  // [BH][kpad][2][128] bf16 high, residual
  float* m2;      // [BH][kpad] |mu|^2
  int* hist;      // [BH][nchunk][k]: counts, then placement bases
  int* seg;       // [BH][k] first position of each cluster
  int* cnt;       // [BH][k] tokens per cluster
};

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// |mu|^2 over 128 threads (one channel each), fixed reduction order
__device__ __forceinline__ float norm2_128(float x, float* red) {
  float s = x * x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  return red[0] + red[1];
}

// centroid c (fp32) -> output array, bf16 high/residual and |mu|^2
__device__ __forceinline__ void store_centroid(float mu, float* cent, GroupWs ws, int bh, int c,
                                               int k, int kpad, float* red) {
  const int d = threadIdx.x;
  cent[((size_t)bh * k + c) * kHeadDim + d] = mu;
  const uint16_t hi = bf16_bits(mu);
  const uint16_t lo = bf16_bits(mu - bf16_value(hi));
  uint16_t* m = ws.muh + (((size_t)bh * kpad + c) * 2) * kHeadDim;
  m[d] = hi;
  m[kHeadDim + d] = lo;
  const float n2 = norm2_128(mu, red);
  if (d == 0) ws.m2[(size_t)bh * kpad + c] = n2;
}

// grid (BH * k), 128 threads
__global__ __launch_bounds__(128) void group_init_kernel(const uint16_t* __restrict__ V,
                                                         float* __restrict__ cent, GroupWs ws,
                                                         int S, int k, int kpad) {
  __shared__ float red[2];
  const int bh = blockIdx.x / k, c = blockIdx.x - bh * k;
  const int tok = (int)(((long long)c * S) / k);
  const float mu = bf16_value(V[((size_t)bh * S + tok) * kHeadDim + threadIdx.x]);
  store_centroid(mu, cent, ws, bh, c, k, kpad, red);
}

// grid (BH * ceil(S / 512)), 512 threads: wave w scores tokens 64w .. 64w+63
// of the workgroup's 512 (two 32-token column blocks) against all centroids,
// 32 at a time.  Each chunk of centroids (bf16 high and residual rows, 16 KB,
// and their 32 squared norms) goes from global memory straight into LDS
// (global_load_lds_dwordx4), once for the 8 waves, into a three-deep ring
// filled two chunks ahead; one barrier per chunk.  LDS rows are
// [centroid][high | residual][16 chunks of 16 B], chunks XOR-swizzled by
// centroid & 15 so the 16 lanes the LDS serves together hit 16 bank groups
// (the DMA's source addresses apply the permutation).
constexpr int kAssignTokens = 64 * kAssignWaves;
__global__ __launch_bounds__(64 * kAssignWaves) void group_assign_kernel(
    const uint16_t* __restrict__ V, int* __restrict__ labels, GroupWs ws, int S, int k, int kpad,
    int ntiles) {
  __shared__ __attribute__((aligned(1024))) char lds_a[3][32 * 2 * 256];
  __shared__ __attribute__((aligned(16))) float lds_m2[3][32];
  const int bh = blockIdx.x / ntiles, tile = blockIdx.x - bh * ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  // B operands: tokens 64w + 32j + col, channels 16kk + 8half .. +7
  bf16x8 vb[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tok = tile * kAssignTokens + wave * 64 + 32 * j + col;
    const uint16_t* row = V + ((size_t)bh * S + min(tok, S - 1)) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      vb[j][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * kk + 8 * half));
  }
  const uint16_t* muh = ws.muh + (size_t)bh * kpad * 2 * kHeadDim;
  const float* m2 = ws.m2 + (size_t)bh * kpad;
  // DMA: wave w fills LDS slots L = 128w + 64u + lane (u = 0, 1) of 16 B,
  // slot L = (2 centroid + part) * 16 + (chunk ^ (centroid & 15)); the
  // arrays are padded to a multiple of 32 centroids, so every chunk is in
  // bounds (the padding is never selected).  Lanes 0-7 of every wave also
  // bring the chunk's 32 norms (the same bytes from each wave).
  uint32_t voff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int L = 128 * wave + 64 * u + lane;
    voff[u] = (uint32_t)((L >> 4) * 256 + 16 * ((L & 15) ^ ((L >> 5) & 15)));
  }
  const uint32_t a_base =
      __builtin_amdgcn_readfirstlane(lds_addr(&lds_a[0][0]) + (uint32_t)wave * 2048);
  const uint32_t m_base = lds_addr(&lds_m2[0][0]);
  auto issue = [&](int c0, int b) __attribute__((always_inline)) {
    const char* src = reinterpret_cast<const char*>(muh + (size_t)c0 * 2 * kHeadDim);
#pragma unroll
    for (int u = 0; u < 2; ++u) dma16(src, voff[u], a_base + (uint32_t)b * (32 * 2 * 256) + u * 1024);
    if (lane < 8) dma16(reinterpret_cast<const char*>(m2 + c0), 16u * lane, m_base + (uint32_t)b * 128);
  };
  const int nch = (k + 31) / 32;
  float best[2] = {INFINITY, INFINITY};
  int best_c[2] = {0x7fffffff, 0x7fffffff};
  // prologue: chunks 0 and 1 in flight; wait for chunk 0 (three loads per
  // wave per chunk)
  issue(0, 0);
  if (nch > 1) {
    issue(32, 1);
    __builtin_amdgcn_s_waitcnt(0x0f73);  // vmcnt(3)
  } else {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  }
  asm volatile("" ::: "memory");
  __syncthreads();
  for (int i = 0; i < nch; ++i) {
    const int c0 = 32 * i, b = i % 3;
    // buffer (i + 2) % 3 held chunk i - 1, which every wave finished before
    // the last barrier
    if (i + 2 < nch) issue(c0 + 64, (i + 2) % 3);
    f32x4 m2c[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) m2c[ii] = *reinterpret_cast<const f32x4*>(&lds_m2[b][8 * ii + 4 * half]);
    // A operand: centroid c0 + col, logical chunk 2kk + half of each part
    bf16x8 ah[8], al[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int pc = (2 * kk + half) ^ (col & 15);
      ah[kk] = *reinterpret_cast<const bf16x8*>(&lds_a[b][((col * 2) * 16 + pc) * 16]);
      al[kk] = *reinterpret_cast<const bf16x8*>(&lds_a[b][((col * 2 + 1) * 16 + pc) * 16]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x16 acc;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        acc = mfma32x32x16_bf16(ah[kk], vb[j][kk], acc);
        acc = mfma32x32x16_bf16(al[kk], vb[j][kk], acc);
      }
      // lane holds centroids c0 + 8(q/4) + 4half + q%4 of its token, in
      // increasing order: a strict < keeps the lowest index on ties
      if (c0 + 32 <= k) {  // a full chunk: every centroid is real
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float d = fmaf(-2.0f, acc[q], m2c[q >> 2][q & 3]);
          const bool take = d < best[j];
          best[j] = take ? d : best[j];
          best_c[j] = take ? c0 + 8 * (q >> 2) + 4 * half + (q & 3) : best_c[j];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int c = c0 + 8 * (q >> 2) + 4 * half + (q & 3);
          const float d = fmaf(-2.0f, acc[q], m2c[q >> 2][q & 3]);
          const bool take = (c < k) & (d < best[j]);
          best[j] = take ? d : best[j];
          best_c[j] = take ? c : best_c[j];
        }
      }
    }
    if (i + 1 < nch) {
      // chunk i + 1 landed (only chunk i + 2's loads may still be in flight)
      if (i + 2 < nch)
        __builtin_amdgcn_s_waitcnt(0x0f73);  // vmcnt(3)
      else
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      asm volatile("" ::: "memory");
      __syncthreads();
    }
  }
  // the other half of the wave holds the interleaved rows for the same token
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float ob = __shfl_xor(best[j], 32);
    const int oc = __shfl_xor(best_c[j], 32);
    int bc = best_c[j];
    if (ob < best[j] || (ob == best[j] && oc < bc)) bc = oc;
    const int tok = tile * kAssignTokens + wave * 64 + 32 * j + col;
    // (no centroid scored, only possible with non-finite inputs: cluster 0)
    if (half == 0 && tok < S) labels[(size_t)bh * S + tok] = bc < k ? bc : 0;
  }
}

// grid (BH * nchunk), 256 threads: label counts of one chunk
__global__ __launch_bounds__(256) void group_hist_kernel(const int* __restrict__ labels,
                                                         GroupWs ws, int S, int k, int nchunk) {
  extern __shared__ int cnt_s[];
  const int bh = blockIdx.x / nchunk, ch = blockIdx.x - bh * nchunk;
  for (int c = threadIdx.x; c < k; c += 256) cnt_s[c] = 0;
  __syncthreads();
  const int t0 = ch * kChunk, t1 = min(S, t0 + kChunk);
  for (int t = t0 + threadIdx.x; t < t1; t += 256) atomicAdd(&cnt_s[labels[(size_t)bh * S + t]], 1);
  __syncthreads();
  int* h = ws.hist + ((size_t)bh * nchunk + ch) * k;
  for (int c = threadIdx.x; c < k; c += 256) h[c] = cnt_s[c];
}

// grid BH, 256 threads: cluster offsets and per-chunk placement bases.
// Integer sums, so the grouping of the additions does not matter.
__global__ __launch_bounds__(256) void group_scan_kernel(GroupWs ws, int k, int nchunk) {
  extern __shared__ int tot_s[];
  __shared__ int part_s[256];
  const int bh = blockIdx.x;
  int* h = ws.hist + (size_t)bh * nchunk * k;
  // cluster totals over the chunks, eight loads in flight
  for (int c = threadIdx.x; c < k; c += 256) {
    int s = 0, ch = 0;
    for (; ch + 8 <= nchunk; ch += 8) {
      int x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = h[(size_t)(ch + u) * k + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += x[u];
    }
    for (; ch < nchunk; ++ch) s += h[(size_t)ch * k + c];
    tot_s[c] = s;
  }
  __syncthreads();
  // exclusive prefix over the clusters: thread t owns a run of `per`
  // consecutive clusters; the runs' sums are scanned in LDS
  const int per = (k + 255) / 256;
  const int c0 = min(k, (int)threadIdx.x * per), c1 = min(k, c0 + per);
  int run = 0;
  for (int c = c0; c < c1; ++c) run += tot_s[c];
  part_s[threadIdx.x] = run;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = threadIdx.x >= off ? part_s[threadIdx.x - off] : 0;
    __syncthreads();
    part_s[threadIdx.x] += add;
    __syncthreads();
  }
  int base = threadIdx.x > 0 ? part_s[threadIdx.x - 1] : 0;
  for (int c = c0; c < c1; ++c) {
    const int n = tot_s[c];
    ws.cnt[(size_t)bh * k + c] = n;
    ws.seg[(size_t)bh * k + c] = base;
    tot_s[c] = base;
    base += n;
  }
  __syncthreads();
  // each chunk's first position in each cluster (chunks in token order)
  for (int c = threadIdx.x; c < k; c += 256) {
    int b = tot_s[c], ch = 0;
    for (; ch + 8 <= nchunk; ch += 8) {
      int x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = h[(size_t)(ch + u) * k + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        h[(size_t)(ch + u) * k + c] = b;
        b += x[u];
      }
    }
    for (; ch < nchunk; ++ch) {
      const int n = h[(size_t)ch * k + c];
      h[(size_t)ch * k + c] = b;
      b += n;
    }
  }
}

// grid (BH * nchunk), 256 threads: the chunk's tokens go to their cluster's
// next positions in token order.  Wave w takes tokens 256w .. 256w+255 of
// the chunk; per-wave label counts give each wave its offset in each cluster
// within the chunk, and within a wave 64 tokens at a time are ranked among
// the earlier lanes with the same label, so the placement is stable.  The
// four waves' counts, then offsets (at most 1,024), are 16-bit halves of two
// words per cluster.
__global__ __launch_bounds__(256) void group_place_kernel(const int* __restrict__ labels,
                                                          int* __restrict__ perm, GroupWs ws, int S,
                                                          int k, int nchunk) {
  // [k] chunk bases, [2][k] packed per-wave counts / offsets, [kChunk] labels
  extern __shared__ int base_s[];
  uint32_t* pair_s = reinterpret_cast<uint32_t*>(base_s + k);
  uint16_t* off_s = reinterpret_cast<uint16_t*>(pair_s);
  int* lab_s = base_s + 3 * k;
  const int bh = blockIdx.x / nchunk, ch = blockIdx.x - bh * nchunk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int* h = ws.hist + ((size_t)bh * nchunk + ch) * k;
  for (int c = threadIdx.x; c < k; c += 256) {
    base_s[c] = h[c];
    pair_s[c] = 0u;
    pair_s[k + c] = 0u;
  }
  const int t0 = ch * kChunk, n = min(S - t0, kChunk);
  for (int t = threadIdx.x; t < kChunk; t += 256) lab_s[t] = t < n ? labels[(size_t)bh * S + t0 + t] : -1;
  __syncthreads();
  // wave w counts into half (w & 1) of word (w >> 1) * k + label
  for (int i = 0; i < kChunk / 256; ++i) {
    const int lab = lab_s[256 * wave + 64 * i + lane];
    if (lab >= 0) atomicAdd(&pair_s[(wave >> 1) * k + lab], 1u << (16 * (wave & 1)));
  }
  __syncthreads();
  for (int c = threadIdx.x; c < k; c += 256) {
    const uint32_t a = pair_s[c], b = pair_s[k + c];
    const uint32_t o1 = a & 0xffffu, o2 = o1 + (a >> 16), o3 = o2 + (b & 0xffffu);
    pair_s[c] = o1 << 16;
    pair_s[k + c] = o2 | (o3 << 16);
  }
  __syncthreads();
  uint16_t* wo = off_s + 2 * (wave >> 1) * k + (wave & 1);  // wave's offset of label c: wo[2c]
  int* p = perm + (size_t)bh * S;
  for (int i = 0; i < kChunk / 256; ++i) {
    const int t = 256 * wave + 64 * i + lane;
    const int lab = lab_s[t];
    int rank = 0, total = 0;
#pragma unroll 8
    for (int j = 0; j < 64; ++j) {
      const int eq = __builtin_amdgcn_readlane(lab, j) == lab;
      total += eq;
      rank += (j < lane) & eq;
    }
    if (lab >= 0) {
      const int o = wo[2 * lab];
      p[base_s[lab] + o + rank] = t0 + t;
      // the first lane of each label moves the wave's offset past the group
      if (rank == 0) wo[2 * lab] = (uint16_t)(o + total);
    }
  }
}

// grid (BH * k), 128 threads: new centroid = mean of the cluster's tokens;
// an empty cluster keeps its centroid.  Thread (g, c) = (tid / 16, tid % 16)
// sums channels 8c .. 8c+7 (one 16-byte load per token) over the members
// g, g + 8, g + 16, ... in order, four loads in flight; the eight partial
// sums are then added in g order, so the result is deterministic.
__global__ __launch_bounds__(128) void group_update_kernel(const uint16_t* __restrict__ V,
                                                           const int* __restrict__ perm,
                                                           float* __restrict__ cent, GroupWs ws,
                                                           int S, int k, int kpad) {
  __shared__ float red[2];
  __shared__ float part[8][kHeadDim];
  const int bh = blockIdx.x / k, c = blockIdx.x - bh * k;
  const int n = ws.cnt[(size_t)bh * k + c], s0 = ws.seg[(size_t)bh * k + c];
  const int d = threadIdx.x;
  float mu = cent[((size_t)bh * k + c) * kHeadDim + d];
  if (n > 0) {
    const int g = threadIdx.x >> 4, c8 = 8 * (threadIdx.x & 15);
    const int* p = perm + (size_t)bh * S + s0;
    const uint16_t* vh = V + (size_t)bh * S * kHeadDim + c8;
    float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j = g;
    for (; j + 24 < n; j += 32) {
      u32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const u32x4*>(vh + (size_t)p[j + 8 * u] * kHeadDim);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[2 * e] += __uint_as_float(x[u][e] << 16);
          sum[2 * e + 1] += __uint_as_float(x[u][e] & 0xffff0000u);
        }
    }
    for (; j < n; j += 8) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(vh + (size_t)p[j] * kHeadDim);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sum[2 * e] += __uint_as_float(x[e] << 16);
        sum[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[g][c8 + e] = sum[e];
  }
  __syncthreads();
  if (n > 0) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) t += part[q][d];
    mu = t / (float)n;
  }
  store_centroid(mu, cent, ws, bh, c, k, kpad, red);
}

// grid (BH * ceil(S / 16)), 256 threads: out row i = x row perm[i]
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint16_t* __restrict__ X,
                                                           const int* __restrict__ perm,
                                                           uint16_t* __restrict__ out, int S,
                                                           int nblk) {
  const int bh = blockIdx.x / nblk, blk = blockIdx.x - bh * nblk;
  const int i = blk * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
  if (i >= S) return;
  const int src = perm[(size_t)bh * S + i];
  const size_t head = (size_t)bh * S * kHeadDim;
  *reinterpret_cast<u32x4*>(out + head + (size_t)i * kHeadDim + 8 * c) =
      *reinterpret_cast<const u32x4*>(X + head + (size_t)src * kHeadDim + 8 * c);
}

GroupWs carve_group(void* base, int BH, int k, int kpad, int nchunk) {
  char* p = static_cast<char*>(base);
  GroupWs ws;
  ws.muh = reinterpret_cast<uint16_t*>(p);
  p += (size_t)BH * kpad * 2 * kHeadDim * sizeof(uint16_t);
  ws.m2 = reinterpret_cast<float*>(p);
  p += (size_t)BH * kpad * sizeof(float);
  ws.hist = reinterpret_cast<int*>(p);
  p += (size_t)BH * nchunk * k * sizeof(int);
  ws.seg = reinterpret_cast<int*>(p);
  p += (size_t)BH * k * sizeof(int);
  ws.cnt = reinterpret_cast<int*>(p);
  return ws;
}

}  // namespace

size_t group_workspace_bytes(int B, int H, int S, int k) {
  const size_t BH = (size_t)B * H;
  const int kpad = (k + 31) / 32 * 32, nchunk = (S + kChunk - 1) / kChunk;
  return BH * kpad * 2 * kHeadDim * sizeof(uint16_t) + BH * kpad * sizeof(float) +
         BH * nchunk * k * sizeof(int) + 2 * BH * k * sizeof(int) + 256;
}

hipError_t launch_vsmooth_group(const void* v, int* perm, int* labels, float* centroids,
                                void* workspace, int B, int H, int S, int k, int rounds,
                                hipStream_t stream) {
  const int BH = B * H;
  const int kpad = (k + 31) / 32 * 32, nchunk = (S + kChunk - 1) / kChunk;
  const int ntiles = (S + kAssignTokens - 1) / kAssignTokens;
  const GroupWs ws = carve_group(workspace, BH, k, kpad, nchunk);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  const size_t lds_k = (size_t)k * sizeof(int);
  hipLaunchKernelGGL(group_init_kernel, dim3(BH * k), dim3(128), 0, stream, V, centroids, ws, S,
                     k, kpad);
  for (int r = 0; r <= rounds; ++r) {
    hipLaunchKernelGGL(group_assign_kernel, dim3(BH * ntiles), dim3(64 * kAssignWaves), 0, stream,
                       V, labels, ws, S, k, kpad, ntiles);
    hipLaunchKernelGGL(group_hist_kernel, dim3(BH * nchunk), dim3(256), lds_k, stream, labels, ws,
                       S, k, nchunk);
    hipLaunchKernelGGL(group_scan_kernel, dim3(BH), dim3(256), lds_k, stream, ws, k, nchunk);
    hipLaunchKernelGGL(group_place_kernel, dim3(BH * nchunk), dim3(256),
                       3 * lds_k + kChunk * sizeof(int), stream, labels, perm, ws, S, k, nchunk);
    if (r < rounds)
      hipLaunchKernelGGL(group_update_kernel, dim3(BH * k), dim3(128), 0, stream, V, perm,
                         centroids, ws, S, k, kpad);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_permute_rows(const void* x, const int* perm, void* out, int B, int H, int S,
                               hipStream_t stream) {
  const int nblk = (S + 15) / 16;
  hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)((long long)B * H * nblk)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(x), perm, static_cast<uint16_t*>(out), S,
                     nblk);
  return hipGetLastError();
}

}  // namespace vdit
