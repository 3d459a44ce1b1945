/*
 * vdit_attn.h - C ABI of the MI355X (gfx950) spatiotemporal self-attention
 * forward library (libvdit_attn.so).
 *
 * The operation.  A video DiT flattens a clip into one sequence of S
 * spatiotemporal tokens and runs full, non-causal self-attention over all of
 * them in every layer (VC-Attention article (aikraft.ru), section 01); the
 * score matrix is quadratic in S and, with its projections, about 82% of a
 * Wan2.1-14B layer's FLOPs at S = 75,600 (real-time video generation FLOPS
 * article (sudonull.com), FLOP list).  For every batch b, head h and query i:
 *
 *     O[b,h,i,:] = sum_j softmax_j(scale * <Q[b,h,i,:], K[b,h,j,:]>) V[b,h,j,:]
 *
 * computed flash-style (the S x S matrix is never stored; same article,
 * "Optymalizacje", FlashAttention item).
 *
 * Conventions shared by every entry point:
 *  - Tensors are caller-owned DEVICE memory, layout [B, H, S, D], contiguous,
 *    D fastest.  D must be 128.  Pointers must be 16-byte aligned.
 *    1 <= S <= VDIT_MAX_SEQ (2^30) and B*H*ceil(S/128) < 2^31, else
 *    VDIT_ERR_UNSUPPORTED (block-sparse masks: S <= 2^20).
 *  - The library never allocates, frees or synchronises; work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and runs
 *    asynchronously.  Buffers must stay valid until the stream reaches it.
 *  - Arguments are validated before any HIP call.  Errors are returned, never
 *    thrown.  On VDIT_ERR_HIP the launch failed; vdit_last_error() gives the
 *    HIP error text of the calling thread's last failure.
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    order (the grouping's histograms use integer atomics, whose counts do
 *    not depend on order).
 */
#ifndef VDIT_ATTN_H
#define VDIT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VDIT_ABI_VERSION 1
#define VDIT_HEAD_DIM 128
#define VDIT_FP8_BLOCK 64 /* tokens per Q/K fp8 scale block and K mean block */
#define VDIT_MAX_SEQ (1 << 30) /* largest S any entry point accepts */

typedef enum vdit_status {
  VDIT_OK = 0,
  VDIT_ERR_INVALID_ARG = 1, /* null/misaligned pointer, B/H/S < 1, bad scale */
  VDIT_ERR_UNSUPPORTED = 2, /* D != 128, unknown dtype, too large, bad mode */
  VDIT_ERR_HIP = 3          /* a HIP launch or runtime call failed */
} vdit_status;

typedef enum vdit_dtype {
  VDIT_DTYPE_BF16 = 0 /* q, k, v, o are bfloat16 */
} vdit_dtype;

/* Version of this ABI (VDIT_ABI_VERSION the library was built with). */
int vdit_abi_version(void);

/* Static text for a status code ("unknown status" for other values). */
const char* vdit_status_str(int status);

/* Text of the calling thread's last error ("" if none). */
const char* vdit_last_error(void);

/*
 * bf16 attention forward.
 *   q, k, v : [B,H,S,D] bf16 inputs.   o : [B,H,S,D] bf16 output.
 *   scale   : softmax scale (usually 1/sqrt(D)); finite and > 0.
 *   dtype   : VDIT_DTYPE_BF16.
 * Softmax and accumulation are fp32; P is rounded to bf16 before the P.V
 * product and the row sum adds those rounded weights; O is rounded to bf16
 * (nearest even).  o may not alias q, k or v.
 */
vdit_status vdit_attn_fwd(const void* q, const void* k, const void* v, void* o,
                          int B, int H, int S, int D, float scale, int dtype,
                          void* stream);

/*
 * Block-causal variant of vdit_attn_fwd for chunk-wise (frame-block) video
 * generation: query i attends to key j iff floor(j / chunk) <= floor(i / chunk),
 * i.e. every token sees its own chunk and all earlier ones (the Wave Forcing
 * note on airadar.tv: later blocks read the context of earlier blocks; a
 * chunk is a group of latent frames, e.g. 3600 tokens per 720p latent frame).
 *   o[b,h,i,:] = sum_{j < lim(i)} softmax_j(scale * q_i . k_j) v_j,
 *   lim(i) = min(S, (floor(i / chunk) + 1) * chunk).
 * Key tiles past a workgroup's largest limit are not visited.  chunk >= S is
 * full attention.  Arguments, layouts and errors as vdit_attn_fwd, plus
 * VDIT_ERR_INVALID_ARG for chunk < 1.
 */
vdit_status vdit_attn_fwd_block_causal(const void* q, const void* k, const void* v, void* o,
                                       int B, int H, int S, int D, float scale, int chunk,
                                       int dtype, void* stream);

/*
 * fp8 pre-pass: quantise and smooth bf16 Q, K, V to E4M3 (OCP E4M3FN, max 448)
 * for vdit_attn_fwd_fp8.  Follows V-Smooth (VC-Attention article, section 02:
 * subtract a mean, quantise only the residual per channel in E4M3) and the
 * Q/K smoothing of section 01.  With nb = ceil(S / 64):
 *   q8, k8      : [B,H,S,D] uint8 E4M3 codes (out).
 *   v8          : [B,H,nb,D,64] uint8 E4M3 codes (out), the layout the fp8
 *                 attention kernel loads tile by tile: per 64-token block a
 *                 tile of D channel rows x 64 key slots; slot s of a row holds
 *                 key 32((s>>4)&1) + 8((s>>2)&3) + 4(s>>5) + (s&3) of the block,
 *                 the four 16-byte chunks of channel row d are XOR-swizzled by
 *                 (d >> 2) & 3, and keys past S hold code 0.  Note the size:
 *                 B*H*nb*64*D bytes, which exceeds B*H*S*D when S % 64 != 0.
 *   q_scale     : [B,H,nb] float, amax/448 of each 64-token Q block (out).
 *   k_mean      : [B,H,k_mean_blocks,D] float (out); k_mean_blocks = nb gives
 *                 one mean per 64-token block (valid tokens only), = 1 one
 *                 mean per channel over the whole sequence.
 *   k_scale     : [B,H,nb] float, amax/448 of each block of K - k_mean (out).
 *   v_mean      : [B,H,D] float, per-channel mean of V over the sequence (out).
 *   v_scale     : [B,H,D] float, per-channel amax/448 of V - v_mean (out).
 *   workspace   : caller-owned device scratch of at least
 *                 vdit_attn_quant_fp8_workspace_size(B,H,S,D,k_mean_blocks)
 *                 bytes, 16-byte aligned; holds the per-block V (and global
 *                 K) partial statistics between the three launches.  Its
 *                 contents on entry do not matter; calls that share one
 *                 workspace must be ordered on one stream.
 * Means are fp64 sums divided in fp64 and rounded once to fp32; residuals
 * are fp32; codes are E4M3 round-to-nearest-even of clamp(r * fp32(448/amax),
 * +-448); a block or channel with amax = 0 gets scale 1 and zero codes.
 * Float arrays must be 16-byte aligned.
 */
vdit_status vdit_attn_quant_fp8(const void* q, const void* k, const void* v,
                                void* q8, void* k8, void* v8,
                                float* q_scale, float* k_scale,
                                float* k_mean, int k_mean_blocks,
                                float* v_mean, float* v_scale,
                                void* workspace, size_t workspace_bytes,
                                int B, int H, int S, int D, void* stream);

/*
 * E4M3 V codes between the token-major layout [B,H,S,D] (uint8, the layout
 * of q8 and k8) and the tiled layout above (v8: [B,H,ceil(S/64),D,64]) that
 * vdit_attn_quant_fp8 writes and every fp8 attention entry point reads.
 *   to_tiles = 1: src [B,H,S,D] -> dst tiled (keys past S get code 0);
 *   to_tiles = 0: src tiled -> dst [B,H,S,D].
 * Both are caller-owned device buffers, 16-byte aligned, not overlapping.
 * The tiled layout is the fp8 MFMA's P^T key order with a bank swizzle;
 * keeping it at the boundary saves the attention call this pass (one read
 * and one write of the codes, bound by HBM bandwidth).  Errors as above.
 */
vdit_status vdit_attn_v8_relayout(const void* src, void* dst, int B, int H, int S, int D,
                                  int to_tiles, void* stream);

/* Bytes of workspace vdit_attn_quant_fp8 needs (0 for invalid shapes). */
size_t vdit_attn_quant_fp8_workspace_size(int B, int H, int S, int D, int k_mean_blocks);

/*
 * Allocation-free vdit_attn_quant_fp8, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, outputs and errors as
 * vdit_attn_quant_fp8 without the workspace: the per-block statistics live in
 * the library's own device scratch, a static array of
 * vdit_attn_quant_fp8_noalloc_max_workspace() bytes (128 MiB; the 720p
 * workload, 40 heads x 75,600 tokens with one K mean per 64-token block,
 * needs 96.9 MB) that every GPU the library runs on holds until the process
 * ends.  A shape whose vdit_attn_quant_fp8_workspace_size exceeds it gives
 * VDIT_ERR_UNSUPPORTED before any HIP call.  The call allocates nothing and
 * the scratch needs no clearing (every statistic it reads is written by the
 * same call).  The stream must belong to the current device (else
 * VDIT_ERR_HIP).  All calls on one GPU share its scratch: calls that overlap
 * in time on one GPU (different streams, or host threads) race and must be
 * ordered by the caller.
 */
vdit_status vdit_attn_quant_fp8_noalloc(const void* q, const void* k, const void* v,
                                        void* q8, void* k8, void* v8,
                                        float* q_scale, float* k_scale,
                                        float* k_mean, int k_mean_blocks,
                                        float* v_mean, float* v_scale,
                                        int B, int H, int S, int D, void* stream);

/* Size in bytes of the scratch behind vdit_attn_quant_fp8_noalloc. */
size_t vdit_attn_quant_fp8_noalloc_max_workspace(void);

/*
 * fp8 attention forward on the pre-pass outputs (same shapes and layouts as
 * above, v8 tiled).
 * Scores: s_ij = q_scale_b(i) k_scale_b(j) (q8_i . k8_j) + q_hat_i . k_mean_b(j)
 * (the second term restores the K mean; it is kept even when k_mean_blocks = 1
 * makes it constant along a row, because it moves the grid P is rounded on).
 * Softmax in the log2 domain with an integer running reference; P is
 * quantised as P8 = E4M3(448 * p) for the fp8 P.V product and the row sum is
 * that of the quantised weights, so the weights of a row sum to one and the
 * mean restore is exact (VC-Attention article, section 02, Restore):
 *   o = v_scale * (sum_j P8_ij v8_j) / (sum_j P8_ij) + v_mean, bf16 out.
 * Float arrays must be 16-byte aligned; o may not overlap q8, k8 or v8
 * (VDIT_ERR_INVALID_ARG).
 */
vdit_status vdit_attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                              const float* q_scale, const float* k_scale,
                              const float* k_mean, int k_mean_blocks,
                              const float* v_mean, const float* v_scale,
                              void* o, int B, int H, int S, int D, float scale,
                              void* stream);

/*
 * ExpCast-FP8 variant of vdit_attn_fwd_fp8 (VC-Attention article, section 03):
 * same arguments and result definition, except that the P8 byte is written
 * directly from the log domain instead of exp2 followed by an E4M3
 * conversion.  The E4M3 byte of v read as an integer is about 8 log2(v) + 56;
 * with the article's centring constant -0.35 and P scaled by 448, the byte
 * position of a weight is z_ij = 8 (t_ij - m_i) + 8 log2(448) + 55.65
 * (t <= m keeps it <= 126, the code of 448).  Where z >= 7.5 the code is
 * rne(z), the article's byte; below, where codes 1-7 are E4M3 subnormals
 * rather than points of the log map, it is the subnormal nearest the value
 * 2^(floor(z/8) - 7) (1 + (z mod 8)/8) that the same map gives to z, so a
 * weight is always within one code of the exact cast and scales by exact
 * powers of two with the reference.  One FMA and two converts per weight;
 * it agrees with the exact byte in about 79.6% of weights in the normal
 * range.
 */
vdit_status vdit_attn_fwd_fp8_expcast(const void* q8, const void* k8, const void* v8,
                                      const float* q_scale, const float* k_scale,
                                      const float* k_mean, int k_mean_blocks,
                                      const float* v_mean, const float* v_scale,
                                      void* o, int B, int H, int S, int D, float scale,
                                      void* stream);

/*
 * Block-sparse bf16 attention (sparse attention that skips unimportant token
 * pairs, after the FLOPS article's "Optymalizacje", block-sparse form):
 * query i sees key j iff block_mask[b,h,i/128,j/64] != 0.
 *   block_mask : [B,H,ceil(S/128),ceil(S/64)] uint8 device array (any
 *                alignment); nonzero = the 128 queries of the row block may
 *                attend to the 64 keys of the column tile.
 * Other arguments as vdit_attn_fwd.  Only tiles allowed for some query of a
 * 256-query workgroup are loaded and scored.  A query row with no allowed key
 * outputs zeros.  S > 1,048,576 is VDIT_ERR_UNSUPPORTED.
 */
vdit_status vdit_attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o,
                                       int B, int H, int S, int D, float scale,
                                       const void* block_mask, int dtype, void* stream);

/*
 * fp8 attention with a key mask, on the outputs of vdit_attn_quant_fp8
 * (per-channel V mean).  Scores, weights (expcast = 1: ExpCast bytes,
 * 0: exp2 then E4M3) and restore as vdit_attn_fwd_fp8, restricted to the
 * allowed keys of each query:
 *   chunk > 0        block-causal as vdit_attn_fwd_block_causal;
 *   block_mask != 0  block-sparse as vdit_attn_fwd_block_sparse (uint8
 *                    [B,H,ceil(S/128),ceil(S/64)], S <= 1,048,576);
 *   neither          full attention (vdit_attn_fwd_fp8).
 * Giving both is VDIT_ERR_INVALID_ARG; so is chunk < 0.  A query row with no
 * allowed key outputs zeros.
 */
vdit_status vdit_attn_fwd_fp8_masked(const void* q8, const void* k8, const void* v8,
                                     const float* q_scale, const float* k_scale,
                                     const float* k_mean, int k_mean_blocks,
                                     const float* v_mean, const float* v_scale,
                                     void* o, int B, int H, int S, int D, float scale,
                                     int chunk, const void* block_mask, int expcast,
                                     void* stream);

/*
 * V-Smooth with the VC-Attention article's own Demean (section 02): V loses
 * the per-channel mean of every hardware block of 128 tokens (valid tokens
 * only) instead of one mean over the sequence; the residual is quantised per
 * channel in E4M3 with one scale per channel over the sequence.  The mean is
 * stored in 16 bits (0.125 bit per value element, as the article counts it):
 *   v_bmean[b,h,d,blk] = bf16_rne(fp32(fp64 sum / n)), blk = token / 128,
 * and the residual fp32(v - v_bmean) is taken against that rounded mean, so
 * adding it back restores exactly what was subtracted.
 * Number of 128-token blocks, padded: nbv_pad = vdit_attn_vsmooth_blocks(S)
 * = 16 * ceil(ceil(S / 128) / 16); blocks past ceil(S / 128) are written as 0.
 */
int vdit_attn_vsmooth_blocks(int S);

/*
 * The fp8 pre-pass with V block means.  Arguments as vdit_attn_quant_fp8
 * except:
 *   v_bmean : [B,H,D,nbv_pad] bf16 (out), channel-major, 16-byte aligned;
 *   v_scale : [B,H,D] float, per-channel amax/448 of V - v_bmean (out).
 * The same workspace size (vdit_attn_quant_fp8_workspace_size) suffices.
 */
vdit_status vdit_attn_quant_fp8_vsmooth(const void* q, const void* k, const void* v,
                                        void* q8, void* k8, void* v8,
                                        float* q_scale, float* k_scale,
                                        float* k_mean, int k_mean_blocks,
                                        void* v_bmean, float* v_scale,
                                        void* workspace, size_t workspace_bytes,
                                        int B, int H, int S, int D, void* stream);

/*
 * fp8 attention on the outputs of vdit_attn_quant_fp8_vsmooth.  Scores and
 * weights as vdit_attn_fwd_fp8 (expcast = 1: ExpCast-FP8 bytes as in
 * vdit_attn_fwd_fp8_expcast, expcast = 0: exp2 then E4M3); the block means
 * are restored through the online softmax's row sums (section 02, Restore):
 *   o = (v_scale * sum_j P8_ij v8_j + sum_blk (sum_{j in blk} P8_ij) v_bmean_blk)
 *       / (sum_j P8_ij), bf16 out,
 * with no second pass: each block's weight sum is accumulated per tile and
 * multiplied into the output every 16 blocks.  expcast other than 0 or 1 is
 * VDIT_ERR_INVALID_ARG.
 */
vdit_status vdit_attn_fwd_fp8_vsmooth(const void* q8, const void* k8, const void* v8,
                                      const float* q_scale, const float* k_scale,
                                      const float* k_mean, int k_mean_blocks,
                                      const void* v_bmean, const float* v_scale,
                                      void* o, int B, int H, int S, int D, float scale,
                                      int expcast, void* stream);

/*
 * V-Smooth Group (VC-Attention article, section 02, Group): k-means of the
 * value tokens of every (b,h) and the permutation that lists the tokens
 * cluster by cluster.  Permuting K and V by it (vdit_permute_tokens) leaves
 * non-causal attention unchanged and gathers similar values into the same
 * 128-token blocks, so the block demean of vdit_attn_quant_fp8_vsmooth takes
 * out more of their energy.  The article reuses a permutation for several
 * denoising steps; so can the caller.
 * Lloyd's algorithm, deterministic: centroid c starts as token
 * floor(c * S / n_clusters); `rounds` times: assign every token to
 * argmin_c |mu_c|^2 - 2 v . mu_c (v . mu on bf16 MFMAs with mu split into
 * bf16 high and residual parts; ties to the lowest c), sort stably by
 * cluster, mu_c = fp32 mean of the cluster's tokens (empty: unchanged); then
 * a final assignment and sort.
 *   v         : [B,H,S,D] bf16 (in), D = 128
 *   perm      : [B,H,S] int32 (out): perm[i] = token placed at position i,
 *               tokens ordered by (cluster, token index)
 *   labels    : [B,H,S] int32 (out): cluster of every token (final assignment)
 *   centroids : [B,H,n_clusters,D] float (out): the last centroids
 *   1 <= n_clusters <= min(S, 4096) (ceil(S/128) gives one cluster per
 *   hardware block on average), 0 <= rounds <= 64; workspace of at least
 *   vdit_vsmooth_group_workspace_size() bytes, 16-byte aligned.
 */
size_t vdit_vsmooth_group_workspace_size(int B, int H, int S, int D, int n_clusters);
vdit_status vdit_vsmooth_group(const void* v, int* perm, int* labels, float* centroids,
                               int B, int H, int S, int D, int n_clusters, int rounds,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * out[b,h,i,:] = x[b,h,perm[b,h,i],:] for bf16 [B,H,S,D] rows (apply the
 * same perm to K and V).  perm must be a permutation of 0..S-1 per (b,h)
 * (not checked); out must not overlap x.
 */
vdit_status vdit_permute_tokens(const void* x, const int* perm, void* out,
                                int B, int H, int S, int D, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VDIT_ATTN_H */
