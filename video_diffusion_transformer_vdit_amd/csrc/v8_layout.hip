// Conversions between E4M3 V codes in token-major [B,H,S,128] layout and the
// tiled layout the fp8 attention kernel loads (what the pre-pass writes).
//
// The tiled layout, per (b,h) and 64-token block: a [128 channel][64 slot]
// tile; slot `pos` of channel row d holds the key
//   key(sl) = 32((sl>>4)&1) + 8((sl>>2)&3) + 4(sl>>5) + (sl&3),
//   sl = 16((pos>>4) ^ ((d>>2)&3)) + (pos&15),
// i.e. the keys in the order of the P^T operand of the 32x32x64 fp8 MFMA,
// with the four 16-byte chunks of each row XOR-swizzled so that the kernel's
// operand reads hit distinct LDS banks.  Keys past S hold code 0.
//
// Both directions move one 8 KB block per workgroup through LDS: 16-byte
// global loads and stores on both sides, the byte permutation in LDS.  They
// are bound by HBM bandwidth (read + write the codes once).
#include "device_common.h"
#include "launchers.h"

namespace vdit {
namespace {

constexpr int kBlk = 64;
constexpr int kTile = kBlk * kHeadDim;  // 8 KB
constexpr int kThreads = kTile / 16;    // 512: one 16-byte chunk each

// slot of key k (0..63) in channel row d
__device__ __forceinline__ int slot_of(int k, int d) {
  const int sl = (k & 3) | (((k >> 3) & 3) << 2) | (((k >> 5) & 1) << 4) | (((k >> 2) & 1) << 5);
  return ((((sl >> 4) ^ ((d >> 2) & 3)) & 3) << 4) | (sl & 15);
}

// key held by slot pos of channel row d
__device__ __forceinline__ int key_of(int pos, int d) {
  const int sl = 16 * ((pos >> 4) ^ ((d >> 2) & 3)) + (pos & 15);
  return 32 * ((sl >> 4) & 1) + 8 * ((sl >> 2) & 3) + 4 * (sl >> 5) + (sl & 3);
}

// token-major [S][128] block -> tile [128][64]
__global__ __launch_bounds__(kThreads) void v8_to_tiles_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst, int S,
                                                              int nb) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTile];  // [key][channel]
  const int bh = blockIdx.x / nb, blk = blockIdx.x - bh * nb;
  const int tid = threadIdx.x;
  const int nvalid = min(kBlk, S - blk * kBlk);
  {
    const int key = tid >> 3, c16 = tid & 7;  // 16-byte chunk of a key's row
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < nvalid)
      w = *reinterpret_cast<const u32x4*>(src + ((size_t)bh * S + (size_t)blk * kBlk + key) * kHeadDim +
                                          16 * c16);
    *reinterpret_cast<u32x4*>(lds + key * kHeadDim + 16 * c16) = w;
  }
  __syncthreads();
  const int d = tid >> 2, p0 = 16 * (tid & 3);
  uint32_t out[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t x = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) x |= (uint32_t)lds[key_of(p0 + 4 * w + b, d) * kHeadDim + d] << (8 * b);
    out[w] = x;
  }
  *reinterpret_cast<u32x4*>(dst + ((size_t)bh * nb + blk) * kTile + d * kBlk + p0) =
      u32x4{out[0], out[1], out[2], out[3]};
}

// tile [128][64] -> token-major [S][128] block (keys < S only)
__global__ __launch_bounds__(kThreads) void v8_from_tiles_kernel(const uint8_t* __restrict__ src,
                                                                uint8_t* __restrict__ dst, int S,
                                                                int nb) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTile];  // [channel][slot]
  const int bh = blockIdx.x / nb, blk = blockIdx.x - bh * nb;
  const int tid = threadIdx.x;
  *reinterpret_cast<u32x4*>(lds + 16 * tid) =
      *reinterpret_cast<const u32x4*>(src + ((size_t)bh * nb + blk) * kTile + 16 * tid);
  __syncthreads();
  const int key = tid >> 3, c0 = 16 * (tid & 7);
  if (blk * kBlk + key >= S) return;
  uint32_t out[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t x = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int d = c0 + 4 * w + b;
      x |= (uint32_t)lds[d * kBlk + slot_of(key, d)] << (8 * b);
    }
    out[w] = x;
  }
  *reinterpret_cast<u32x4*>(dst + ((size_t)bh * S + (size_t)blk * kBlk + key) * kHeadDim + c0) =
      u32x4{out[0], out[1], out[2], out[3]};
}

}  // namespace

hipError_t launch_v8_layout(const void* src, void* dst, int B, int H, int S, bool to_tiles,
                            hipStream_t stream) {
  const int nb = (S + kBlk - 1) / kBlk;
  const unsigned grid = (unsigned)((size_t)B * H * nb);
  if (to_tiles)
    hipLaunchKernelGGL(v8_to_tiles_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), S, nb);
  else
    hipLaunchKernelGGL(v8_from_tiles_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), S, nb);
  return hipGetLastError();
}

}  // namespace vdit
