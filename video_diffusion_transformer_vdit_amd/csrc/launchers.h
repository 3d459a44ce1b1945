// Internal launch wrappers of libvdit_attn (host side).  Arguments have been
// validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>

namespace vdit {

// chunk > 0: block-causal; block_mask != nullptr: block-sparse
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o,
                                int B, int H, int S, float scale, int chunk,
                                const void* block_mask, hipStream_t stream);
int bf16_sparse_max_tiles();

size_t quant_fp8_workspace_bytes(int B, int H, int S, int k_mean_blocks);

// V-Smooth block means: one per channel and 128-token block, stored
// [b,h][channel][block] with the block count padded to a multiple of 16.
constexpr int kVSmoothBlock = 128;
inline int vsmooth_blocks_padded(int S) {
  const int nbv = (S + kVSmoothBlock - 1) / kVSmoothBlock;
  return (nbv + 15) / 16 * 16;
}

hipError_t launch_quant_fp8(const void* q, const void* k, const void* v,
                            void* q8, void* k8, void* v8, float* q_scale, float* k_scale,
                            float* k_mean, int k_mean_blocks, float* v_mean, void* v_bmean,
                            float* v_scale, void* workspace, int B, int H, int S,
                            hipStream_t stream);

// Allocation-free pre-pass: the library's own device scratch (noalloc.hip),
// its size, and its address on the current device (which the stream, if
// not null, must belong to).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(hipStream_t stream, void** out);

hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                               const float* q_scale, const float* k_scale,
                               const float* k_mean, int k_mean_blocks,
                               const float* v_mean, const void* v_bmean,
                               const float* v_scale, void* o, int B, int H, int S, float scale,
                               bool expcast, int chunk, const void* block_mask,
                               hipStream_t stream);

// E4M3 V codes between token-major [B,H,S,128] and the fp8 kernel's tiles
hipError_t launch_v8_layout(const void* src, void* dst, int B, int H, int S, bool to_tiles,
                            hipStream_t stream);

// V-Smooth Group: k-means of V tokens and the stable cluster permutation
constexpr int kGroupMaxClusters = 4096;
size_t group_workspace_bytes(int B, int H, int S, int k);
hipError_t launch_vsmooth_group(const void* v, int* perm, int* labels, float* centroids,
                                void* workspace, int B, int H, int S, int k, int rounds,
                                hipStream_t stream);
hipError_t launch_permute_rows(const void* x, const int* perm, void* out, int B, int H, int S,
                               hipStream_t stream);

}  // namespace vdit
