// C ABI of libvdit_attn: argument validation, error reporting and dispatch to
// the gfx950 kernels.  Every check runs before any HIP call, so the checks
// can be exercised on a machine without a GPU.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/vdit_attn.h"
#include "launchers.h"

namespace {

thread_local char g_last_error[512] = "";

vdit_status fail(vdit_status s, const char* fmt, const char* what) {
  std::snprintf(g_last_error, sizeof(g_last_error), fmt, what);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, const void* b, size_t bytes_a, size_t bytes_b) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bytes_b && y < x + bytes_a;
}

// Shape checks shared by every entry point.
vdit_status check_shape(int B, int H, int S, int D) {
  if (B < 1 || H < 1 || S < 1) return fail(VDIT_ERR_INVALID_ARG, "%s", "B, H and S must be >= 1");
  if (D != VDIT_HEAD_DIM) return fail(VDIT_ERR_UNSUPPORTED, "%s", "only D = 128 is supported");
  // token indices and limits (up to twice S for block-causal chunks) are
  // 32-bit in the kernels and in the size arithmetic below
  if (S > VDIT_MAX_SEQ) return fail(VDIT_ERR_UNSUPPORTED, "%s", "S must be <= 2^30");
  // grid = B*H*ceil(S/128) workgroups must fit a 32-bit grid dimension, and
  // per-head offsets are 64-bit.
  const long long tiles = (long long)B * H * (((long long)S + 127) / 128);
  if (tiles > 0x7fffffffLL || (long long)B * H > 0x7fffffffLL)
    return fail(VDIT_ERR_UNSUPPORTED, "%s", "problem too large for one launch");
  return VDIT_OK;
}

vdit_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(VDIT_ERR_INVALID_ARG, "null pointer: %s", name);
  if (!aligned16(p)) return fail(VDIT_ERR_INVALID_ARG, "pointer not 16-byte aligned: %s", name);
  return VDIT_OK;
}

vdit_status check_fptr(const void* p, const char* name) { return check_ptr(p, name); }

vdit_status hip_result(hipError_t e) {
  if (e == hipSuccess) {
    g_last_error[0] = '\0';
    return VDIT_OK;
  }
  return fail(VDIT_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
}

bool scale_ok(float scale) { return std::isfinite(scale) && scale > 0.f; }

#define VDIT_TRY(expr)                 \
  do {                                 \
    const vdit_status st_ = (expr);    \
    if (st_ != VDIT_OK) return st_;    \
  } while (0)

}  // namespace

extern "C" {

int vdit_abi_version(void) { return VDIT_ABI_VERSION; }

const char* vdit_status_str(int status) {
  switch (status) {
    case VDIT_OK: return "ok";
    case VDIT_ERR_INVALID_ARG: return "invalid argument";
    case VDIT_ERR_UNSUPPORTED: return "unsupported argument";
    case VDIT_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* vdit_last_error(void) { return g_last_error; }

static vdit_status fwd_bf16(const void* q, const void* k, const void* v, void* o, int B, int H,
                            int S, int D, float scale, int chunk, const void* block_mask,
                            int dtype, void* stream) {
  VDIT_TRY(check_ptr(q, "q"));
  VDIT_TRY(check_ptr(k, "k"));
  VDIT_TRY(check_ptr(v, "v"));
  VDIT_TRY(check_ptr(o, "o"));
  VDIT_TRY(check_shape(B, H, S, D));
  if (!scale_ok(scale)) return fail(VDIT_ERR_INVALID_ARG, "%s", "scale must be finite and > 0");
  if (dtype != VDIT_DTYPE_BF16) return fail(VDIT_ERR_UNSUPPORTED, "%s", "dtype must be VDIT_DTYPE_BF16");
  const size_t bytes = (size_t)B * H * S * D * 2;
  if (overlaps(o, q, bytes, bytes) || overlaps(o, k, bytes, bytes) || overlaps(o, v, bytes, bytes))
    return fail(VDIT_ERR_INVALID_ARG, "%s", "o overlaps an input");
  if (block_mask && (S + 63) / 64 > vdit::bf16_sparse_max_tiles())
    return fail(VDIT_ERR_UNSUPPORTED, "%s", "block-sparse attention supports S <= 1048576");
  return hip_result(vdit::launch_attn_fwd_bf16(q, k, v, o, B, H, S, scale, chunk, block_mask,
                                               static_cast<hipStream_t>(stream)));
}

vdit_status vdit_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H,
                          int S, int D, float scale, int dtype, void* stream) {
  return fwd_bf16(q, k, v, o, B, H, S, D, scale, 0, nullptr, dtype, stream);
}

vdit_status vdit_attn_fwd_block_causal(const void* q, const void* k, const void* v, void* o, int B,
                                       int H, int S, int D, float scale, int chunk, int dtype,
                                       void* stream) {
  if (chunk < 1) return fail(VDIT_ERR_INVALID_ARG, "%s", "chunk must be >= 1");
  return fwd_bf16(q, k, v, o, B, H, S, D, scale, chunk, nullptr, dtype, stream);
}

vdit_status vdit_attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, int B,
                                       int H, int S, int D, float scale, const void* block_mask,
                                       int dtype, void* stream) {
  if (!block_mask) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: block_mask");
  return fwd_bf16(q, k, v, o, B, H, S, D, scale, 0, block_mask, dtype, stream);
}

// use_scratch: the allocation-free entry point, whose workspace is the
// library's own device scratch instead of a caller argument.
static vdit_status quant_fp8(const void* q, const void* k, const void* v, void* q8, void* k8,
                             void* v8, float* q_scale, float* k_scale, float* k_mean,
                             int k_mean_blocks, float* v_mean, void* v_bmean, float* v_scale,
                             void* workspace, size_t workspace_bytes, int B, int H, int S, int D,
                             void* stream, bool use_scratch = false) {
  VDIT_TRY(check_ptr(q, "q"));
  VDIT_TRY(check_ptr(k, "k"));
  VDIT_TRY(check_ptr(v, "v"));
  VDIT_TRY(check_ptr(q8, "q8"));
  VDIT_TRY(check_ptr(k8, "k8"));
  VDIT_TRY(check_ptr(v8, "v8"));
  VDIT_TRY(check_fptr(q_scale, "q_scale"));
  VDIT_TRY(check_fptr(k_scale, "k_scale"));
  VDIT_TRY(check_fptr(k_mean, "k_mean"));
  if (v_bmean)
    VDIT_TRY(check_ptr(v_bmean, "v_bmean"));
  else
    VDIT_TRY(check_fptr(v_mean, "v_mean"));
  VDIT_TRY(check_fptr(v_scale, "v_scale"));
  if (!use_scratch) VDIT_TRY(check_ptr(workspace, "workspace"));
  VDIT_TRY(check_shape(B, H, S, D));
  const int nb = (S + VDIT_FP8_BLOCK - 1) / VDIT_FP8_BLOCK;
  if (k_mean_blocks != 1 && k_mean_blocks != nb)
    return fail(VDIT_ERR_UNSUPPORTED, "%s", "k_mean_blocks must be 1 or ceil(S/64)");
  const size_t need = vdit::quant_fp8_workspace_bytes(B, H, S, k_mean_blocks);
  if (use_scratch) {
    if (need > vdit::noalloc_scratch_bytes()) {
      char msg[160];
      std::snprintf(msg, sizeof(msg), "the pre-pass needs %zu bytes of scratch; the allocation-free "
                    "entry point holds %zu (use vdit_attn_quant_fp8 with a workspace)",
                    need, vdit::noalloc_scratch_bytes());
      return fail(VDIT_ERR_UNSUPPORTED, "%s", msg);
    }
    const hipError_t e = vdit::noalloc_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (e != hipSuccess) return hip_result(e);
  } else if (workspace_bytes < need) {
    return fail(VDIT_ERR_INVALID_ARG, "%s", "workspace too small");
  }
  return hip_result(vdit::launch_quant_fp8(q, k, v, q8, k8, v8, q_scale, k_scale, k_mean,
                                           k_mean_blocks, v_mean, v_bmean, v_scale, workspace, B,
                                           H, S, static_cast<hipStream_t>(stream)));
}

vdit_status vdit_attn_quant_fp8(const void* q, const void* k, const void* v, void* q8, void* k8,
                                void* v8, float* q_scale, float* k_scale, float* k_mean,
                                int k_mean_blocks, float* v_mean, float* v_scale, void* workspace,
                                size_t workspace_bytes, int B, int H, int S, int D,
                                void* stream) {
  if (!v_mean) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: v_mean");
  return quant_fp8(q, k, v, q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks, v_mean, nullptr,
                   v_scale, workspace, workspace_bytes, B, H, S, D, stream);
}

vdit_status vdit_attn_quant_fp8_noalloc(const void* q, const void* k, const void* v, void* q8,
                                        void* k8, void* v8, float* q_scale, float* k_scale,
                                        float* k_mean, int k_mean_blocks, float* v_mean,
                                        float* v_scale, int B, int H, int S, int D, void* stream) {
  if (!v_mean) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: v_mean");
  return quant_fp8(q, k, v, q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks, v_mean, nullptr,
                   v_scale, nullptr, 0, B, H, S, D, stream, true);
}

size_t vdit_attn_quant_fp8_noalloc_max_workspace(void) { return vdit::noalloc_scratch_bytes(); }

vdit_status vdit_attn_quant_fp8_vsmooth(const void* q, const void* k, const void* v, void* q8,
                                        void* k8, void* v8, float* q_scale, float* k_scale,
                                        float* k_mean, int k_mean_blocks, void* v_bmean,
                                        float* v_scale, void* workspace, size_t workspace_bytes,
                                        int B, int H, int S, int D, void* stream) {
  if (!v_bmean) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: v_bmean");
  return quant_fp8(q, k, v, q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks, nullptr, v_bmean,
                   v_scale, workspace, workspace_bytes, B, H, S, D, stream);
}

vdit_status vdit_attn_v8_relayout(const void* src, void* dst, int B, int H, int S, int D,
                                  int to_tiles, void* stream) {
  VDIT_TRY(check_ptr(src, "src"));
  VDIT_TRY(check_ptr(dst, "dst"));
  VDIT_TRY(check_shape(B, H, S, D));
  if (to_tiles != 0 && to_tiles != 1) return fail(VDIT_ERR_INVALID_ARG, "%s", "to_tiles must be 0 or 1");
  const size_t tokens = (size_t)B * H * S * D;
  const size_t tiles = (size_t)B * H * ((S + VDIT_FP8_BLOCK - 1) / VDIT_FP8_BLOCK) * VDIT_FP8_BLOCK * D;
  if (overlaps(src, dst, to_tiles ? tokens : tiles, to_tiles ? tiles : tokens))
    return fail(VDIT_ERR_INVALID_ARG, "%s", "src and dst overlap");
  return hip_result(vdit::launch_v8_layout(src, dst, B, H, S, to_tiles == 1,
                                           static_cast<hipStream_t>(stream)));
}

int vdit_attn_vsmooth_blocks(int S) {
  if (S < 1 || S > VDIT_MAX_SEQ) return 0;
  return vdit::vsmooth_blocks_padded(S);
}

size_t vdit_attn_quant_fp8_workspace_size(int B, int H, int S, int D, int k_mean_blocks) {
  if (check_shape(B, H, S, D) != VDIT_OK) return 0;
  const int nb = (S + VDIT_FP8_BLOCK - 1) / VDIT_FP8_BLOCK;
  if (k_mean_blocks != 1 && k_mean_blocks != nb) return 0;
  return vdit::quant_fp8_workspace_bytes(B, H, S, k_mean_blocks);
}

static vdit_status fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale,
                           const float* k_scale, const float* k_mean, int k_mean_blocks,
                           const float* v_mean, const void* v_bmean, const float* v_scale,
                           void* o, int B, int H, int S, int D, float scale, bool expcast,
                           void* stream, int chunk = 0, const void* block_mask = nullptr) {
  VDIT_TRY(check_ptr(q8, "q8"));
  VDIT_TRY(check_ptr(k8, "k8"));
  VDIT_TRY(check_ptr(v8, "v8"));
  VDIT_TRY(check_fptr(q_scale, "q_scale"));
  VDIT_TRY(check_fptr(k_scale, "k_scale"));
  VDIT_TRY(check_fptr(k_mean, "k_mean"));
  if (v_bmean)
    VDIT_TRY(check_ptr(v_bmean, "v_bmean"));
  else
    VDIT_TRY(check_fptr(v_mean, "v_mean"));
  VDIT_TRY(check_fptr(v_scale, "v_scale"));
  VDIT_TRY(check_ptr(o, "o"));
  VDIT_TRY(check_shape(B, H, S, D));
  if (!scale_ok(scale)) return fail(VDIT_ERR_INVALID_ARG, "%s", "scale must be finite and > 0");
  const int nb = (S + VDIT_FP8_BLOCK - 1) / VDIT_FP8_BLOCK;
  if (k_mean_blocks != 1 && k_mean_blocks != nb)
    return fail(VDIT_ERR_UNSUPPORTED, "%s", "k_mean_blocks must be 1 or ceil(S/64)");
  if (block_mask && (S + 63) / 64 > 16384)
    return fail(VDIT_ERR_UNSUPPORTED, "%s", "block-sparse attention supports S <= 1048576");
  // the bf16 output must not overlap the codes it is computed from
  const size_t codes = (size_t)B * H * S * D;
  const size_t tiles = (size_t)B * H * nb * VDIT_FP8_BLOCK * D;
  if (overlaps(o, q8, 2 * codes, codes) || overlaps(o, k8, 2 * codes, codes) ||
      overlaps(o, v8, 2 * codes, tiles))
    return fail(VDIT_ERR_INVALID_ARG, "%s", "o overlaps an input");
  return hip_result(vdit::launch_attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks,
                                              v_mean, v_bmean, v_scale, o, B, H, S, scale, expcast,
                                              chunk, block_mask, static_cast<hipStream_t>(stream)));
}

vdit_status vdit_attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                              const float* q_scale, const float* k_scale, const float* k_mean,
                              int k_mean_blocks, const float* v_mean, const float* v_scale,
                              void* o, int B, int H, int S, int D, float scale, void* stream) {
  if (!v_mean) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: v_mean");
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks, v_mean, nullptr, v_scale, o,
                 B, H, S, D, scale, false, stream);
}

vdit_status vdit_attn_fwd_fp8_expcast(const void* q8, const void* k8, const void* v8,
                                      const float* q_scale, const float* k_scale,
                                      const float* k_mean, int k_mean_blocks, const float* v_mean,
                                      const float* v_scale, void* o, int B, int H, int S, int D,
                                      float scale, void* stream) {
  if (!v_mean) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: v_mean");
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks, v_mean, nullptr, v_scale, o,
                 B, H, S, D, scale, true, stream);
}

vdit_status vdit_attn_fwd_fp8_masked(const void* q8, const void* k8, const void* v8,
                                     const float* q_scale, const float* k_scale,
                                     const float* k_mean, int k_mean_blocks, const float* v_mean,
                                     const float* v_scale, void* o, int B, int H, int S, int D,
                                     float scale, int chunk, const void* block_mask, int expcast,
                                     void* stream) {
  if (!v_mean) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: v_mean");
  if (chunk < 0) return fail(VDIT_ERR_INVALID_ARG, "%s", "chunk must be >= 0");
  if (chunk > 0 && block_mask)
    return fail(VDIT_ERR_INVALID_ARG, "%s", "give either chunk or block_mask, not both");
  if (expcast != 0 && expcast != 1) return fail(VDIT_ERR_INVALID_ARG, "%s", "expcast must be 0 or 1");
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks, v_mean, nullptr, v_scale, o,
                 B, H, S, D, scale, expcast == 1, stream, chunk, block_mask);
}

vdit_status vdit_attn_fwd_fp8_vsmooth(const void* q8, const void* k8, const void* v8,
                                      const float* q_scale, const float* k_scale,
                                      const float* k_mean, int k_mean_blocks, const void* v_bmean,
                                      const float* v_scale, void* o, int B, int H, int S, int D,
                                      float scale, int expcast, void* stream) {
  if (!v_bmean) return fail(VDIT_ERR_INVALID_ARG, "%s", "null pointer: v_bmean");
  if (expcast != 0 && expcast != 1) return fail(VDIT_ERR_INVALID_ARG, "%s", "expcast must be 0 or 1");
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, k_mean, k_mean_blocks, nullptr, v_bmean, v_scale, o,
                 B, H, S, D, scale, expcast == 1, stream);
}

static bool group_args_ok(int S, int n_clusters, int rounds) {
  return n_clusters >= 1 && n_clusters <= vdit::kGroupMaxClusters && n_clusters <= S &&
         rounds >= 0 && rounds <= 64;
}

size_t vdit_vsmooth_group_workspace_size(int B, int H, int S, int D, int n_clusters) {
  if (check_shape(B, H, S, D) != VDIT_OK || !group_args_ok(S, n_clusters, 0)) return 0;
  return vdit::group_workspace_bytes(B, H, S, n_clusters);
}

vdit_status vdit_vsmooth_group(const void* v, int* perm, int* labels, float* centroids, int B,
                               int H, int S, int D, int n_clusters, int rounds, void* workspace,
                               size_t workspace_bytes, void* stream) {
  VDIT_TRY(check_ptr(v, "v"));
  VDIT_TRY(check_ptr(perm, "perm"));
  VDIT_TRY(check_ptr(labels, "labels"));
  VDIT_TRY(check_fptr(centroids, "centroids"));
  VDIT_TRY(check_ptr(workspace, "workspace"));
  VDIT_TRY(check_shape(B, H, S, D));
  if (!group_args_ok(S, n_clusters, rounds))
    return fail(VDIT_ERR_INVALID_ARG, "%s", "need 1 <= n_clusters <= min(S, 4096), 0 <= rounds <= 64");
  if (workspace_bytes < vdit::group_workspace_bytes(B, H, S, n_clusters))
    return fail(VDIT_ERR_INVALID_ARG, "%s", "workspace too small");
  return hip_result(vdit::launch_vsmooth_group(v, perm, labels, centroids, workspace, B, H, S,
                                               n_clusters, rounds, static_cast<hipStream_t>(stream)));
}

vdit_status vdit_permute_tokens(const void* x, const int* perm, void* out, int B, int H, int S,
                                int D, void* stream) {
  VDIT_TRY(check_ptr(x, "x"));
  VDIT_TRY(check_ptr(perm, "perm"));
  VDIT_TRY(check_ptr(out, "out"));
  VDIT_TRY(check_shape(B, H, S, D));
  const size_t bytes = (size_t)B * H * S * D * 2;
  if (overlaps(out, x, bytes, bytes)) return fail(VDIT_ERR_INVALID_ARG, "%s", "out overlaps x");
  return hip_result(vdit::launch_permute_rows(x, perm, out, B, H, S, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
