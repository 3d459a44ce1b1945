"""ctypes binding of libvdit_attn.so with the C ABI's names.

Argument marshalling only: every step of the attention runs in the HIP
library.  torch supplies device memory and the current HIP stream; nothing
here computes on the CPU, and a missing library raises instead of falling
back to anything else.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# VDIT_ATTN_LIB points the binding at another build of the same library
# (e.g. the host-instrumented one the sanitizer test builds)
LIB_PATH = os.environ.get("VDIT_ATTN_LIB") or os.path.join(PKG, "libvdit_attn.so")
HEAD_DIM = 128
FP8_BLOCK = 64
DTYPE_BF16 = 0

STATUS = {0: "VDIT_OK", 1: "VDIT_ERR_INVALID_ARG", 2: "VDIT_ERR_UNSUPPORTED", 3: "VDIT_ERR_HIP"}

# exported symbol -> (restype, argtypes)
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "vdit_abi_version": (_I, []),
    "vdit_status_str": (ctypes.c_char_p, [_I]),
    "vdit_last_error": (ctypes.c_char_p, []),
    "vdit_attn_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "vdit_attn_fwd_block_causal": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "vdit_attn_fwd_block_sparse": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _I, _P]),
    "vdit_attn_quant_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _Z,
                                 _I, _I, _I, _I, _P]),
    "vdit_attn_quant_fp8_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "vdit_attn_quant_fp8_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                         _I, _I, _I, _I, _P]),
    "vdit_attn_quant_fp8_noalloc_max_workspace": (_Z, []),
    "vdit_attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F, _P]),
    "vdit_attn_fwd_fp8_expcast": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F, _P]),
    "vdit_attn_quant_fp8_vsmooth": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _Z,
                                         _I, _I, _I, _I, _P]),
    "vdit_attn_vsmooth_blocks": (_I, [_I]),
    "vdit_attn_fwd_fp8_vsmooth": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F,
                                       _I, _P]),
    "vdit_attn_fwd_fp8_masked": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F,
                                      _I, _P, _I, _P]),
    "vdit_attn_v8_relayout": (_I, [_P, _P, _I, _I, _I, _I, _I, _P]),
    "vdit_vsmooth_group_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "vdit_vsmooth_group": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _Z, _P]),
    "vdit_permute_tokens": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
}

_lib = None


class VditError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load the library once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m video_diffusion_transformer_vdit_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        lib = load()
        raise VditError(status, lib.vdit_last_error().decode() or lib.vdit_status_str(status).decode())


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream):
    """Context for the tensors a call allocates (outputs, workspaces): on the
    stream the call launches on, so that torch's caching allocator, which
    tracks blocks per stream, does not hand them to other streams' work while
    the call's kernels are still queued.  Inert for the current stream."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(stream)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape4(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, S, D] tensors")
    return tuple(int(x) for x in q.shape)


def vdit_attn_fwd(q, k, v, o=None, scale=None, stream=None):
    """o = softmax(scale q k^T) v for bf16 [B, H, S, 128] tensors; returns o."""
    import torch
    B, H, S, D = _shape4(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if o is None:
        with _alloc_on(stream):
            o = torch.empty_like(q)
    scale = D ** -0.5 if scale is None else float(scale)
    lib = load()
    check(lib.vdit_attn_fwd(_dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"),
                            _dev(v, torch.bfloat16, "v"), _dev(o, torch.bfloat16, "o"),
                            B, H, S, D, scale, DTYPE_BF16, _stream(stream)))
    return o


def vdit_attn_fwd_block_causal(q, k, v, chunk, o=None, scale=None, stream=None):
    """Block-causal attention by chunks of ``chunk`` tokens (query i sees key
    j iff j // chunk <= i // chunk) for bf16 [B, H, S, 128]; returns o."""
    import torch
    B, H, S, D = _shape4(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if o is None:
        with _alloc_on(stream):
            o = torch.empty_like(q)
    scale = D ** -0.5 if scale is None else float(scale)
    lib = load()
    check(lib.vdit_attn_fwd_block_causal(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(o, torch.bfloat16, "o"), B, H, S, D, scale, int(chunk), DTYPE_BF16, _stream(stream)))
    return o


SPARSE_Q_BLOCK = 128
SPARSE_K_TILE = 64


def vdit_attn_fwd_block_sparse(q, k, v, block_mask, o=None, scale=None, stream=None):
    """Block-sparse attention for bf16 [B, H, S, 128]: query i sees key j iff
    block_mask[b, h, i // 128, j // 64] != 0; block_mask is a uint8 (or
    bool) device tensor [B, H, ceil(S/128), ceil(S/64)].  Returns o."""
    import torch
    B, H, S, D = _shape4(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    want = (B, H, -(-S // SPARSE_Q_BLOCK), -(-S // SPARSE_K_TILE))
    if tuple(block_mask.shape) != want:
        raise ValueError(f"block_mask must have shape {want}, not {tuple(block_mask.shape)}")
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if o is None:
        with _alloc_on(stream):
            o = torch.empty_like(q)
    scale = D ** -0.5 if scale is None else float(scale)
    lib = load()
    check(lib.vdit_attn_fwd_block_sparse(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(o, torch.bfloat16, "o"), B, H, S, D, scale,
        _dev(block_mask, torch.uint8, "block_mask"), DTYPE_BF16, _stream(stream)))
    return o


def quant_buffers(B, H, S, k_mean_blocks=None, device="cuda", v_mean="global"):
    """Allocate the pre-pass outputs and workspace (torch, on ``device``).
    ``v_mean="block"`` (V-Smooth Demean) replaces v_mean [B,H,128] by v_bmean,
    bf16 [B,H,128,nbv_pad]: per channel the mean of every 128-token block,
    nbv_pad = vdit_attn_vsmooth_blocks(S) (zero padded)."""
    import torch
    nb = -(-S // FP8_BLOCK)
    kmb = nb if k_mean_blocks is None else int(k_mean_blocks)
    lib = load()
    ws = int(lib.vdit_attn_quant_fp8_workspace_size(B, H, S, HEAD_DIM, kmb))
    if ws == 0:
        raise ValueError("invalid shape or k_mean_blocks for the fp8 pre-pass")
    f32 = dict(dtype=torch.float32, device=device)
    u8 = dict(dtype=torch.uint8, device=device)
    z = {
        "q8": torch.empty((B, H, S, HEAD_DIM), **u8),
        "k8": torch.empty((B, H, S, HEAD_DIM), **u8),
        # V codes in the attention kernel's layout: per 64-token block a
        # [128 channel][64 key slot] tile (see include/vdit_attn.h)
        "v8": torch.empty((B, H, nb, HEAD_DIM, FP8_BLOCK), **u8),
        "q_scale": torch.empty((B, H, nb), **f32),
        "k_scale": torch.empty((B, H, nb), **f32),
        "k_mean": torch.empty((B, H, kmb, HEAD_DIM), **f32),
        "v_scale": torch.empty((B, H, HEAD_DIM), **f32),
        "workspace": torch.empty(ws, **u8),
    }
    if v_mean == "global":
        z["v_mean"] = torch.empty((B, H, HEAD_DIM), **f32)
    elif v_mean == "block":
        nbv_pad = int(lib.vdit_attn_vsmooth_blocks(S))
        z["v_bmean"] = torch.empty((B, H, HEAD_DIM, nbv_pad), dtype=torch.bfloat16, device=device)
    else:
        raise ValueError(f"v_mean must be 'global' or 'block', not {v_mean!r}")
    return z


def vdit_attn_quant_fp8(q, k, v, k_mean_blocks=None, out=None, stream=None, v_mean="global"):
    """fp8 pre-pass on bf16 q, k, v; returns the dict of quant_buffers().
    With ``v_mean="block"`` (or an ``out`` holding v_bmean) V is smoothed by
    its 128-token block means (vdit_attn_quant_fp8_vsmooth)."""
    import torch
    B, H, S, D = _shape4(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if out is None:
        with _alloc_on(stream):
            z = quant_buffers(B, H, S, k_mean_blocks, q.device, v_mean)
    else:
        z = out
    kmb = int(z["k_mean"].shape[2])
    lib = load()
    if "v_bmean" in z:
        check(lib.vdit_attn_quant_fp8_vsmooth(
            _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
            _dev(z["q8"], torch.uint8, "q8"), _dev(z["k8"], torch.uint8, "k8"),
            _dev(z["v8"], torch.uint8, "v8"), _dev(z["q_scale"], torch.float32, "q_scale"),
            _dev(z["k_scale"], torch.float32, "k_scale"), _dev(z["k_mean"], torch.float32, "k_mean"),
            kmb, _dev(z["v_bmean"], torch.bfloat16, "v_bmean"),
            _dev(z["v_scale"], torch.float32, "v_scale"),
            _dev(z["workspace"], torch.uint8, "workspace"), z["workspace"].numel(),
            B, H, S, D, _stream(stream)))
        return z
    check(lib.vdit_attn_quant_fp8(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(z["q8"], torch.uint8, "q8"), _dev(z["k8"], torch.uint8, "k8"),
        _dev(z["v8"], torch.uint8, "v8"), _dev(z["q_scale"], torch.float32, "q_scale"),
        _dev(z["k_scale"], torch.float32, "k_scale"), _dev(z["k_mean"], torch.float32, "k_mean"),
        kmb, _dev(z["v_mean"], torch.float32, "v_mean"), _dev(z["v_scale"], torch.float32, "v_scale"),
        _dev(z["workspace"], torch.uint8, "workspace"), z["workspace"].numel(),
        B, H, S, D, _stream(stream)))
    return z


def vdit_attn_quant_fp8_noalloc(q, k, v, out, stream=None):
    """The fp8 pre-pass through the allocation-free entry point: the caller
    passes the outputs (``out``, a dict as from quant_buffers with v_mean;
    its workspace is not used) and the library's own device scratch holds
    the intermediate statistics.  Returns ``out``."""
    import torch
    B, H, S, D = _shape4(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    z = out
    lib = load()
    check(lib.vdit_attn_quant_fp8_noalloc(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        _dev(z["q8"], torch.uint8, "q8"), _dev(z["k8"], torch.uint8, "k8"),
        _dev(z["v8"], torch.uint8, "v8"), _dev(z["q_scale"], torch.float32, "q_scale"),
        _dev(z["k_scale"], torch.float32, "k_scale"), _dev(z["k_mean"], torch.float32, "k_mean"),
        int(z["k_mean"].shape[2]), _dev(z["v_mean"], torch.float32, "v_mean"),
        _dev(z["v_scale"], torch.float32, "v_scale"), B, H, S, D, _stream(stream)))
    return z


def vdit_attn_v8_to_tiles(v8_tokens, out=None, stream=None):
    """uint8 E4M3 V codes [B, H, S, 128] -> the fp8 kernels' tiled layout
    [B, H, ceil(S/64), 128, 64] (vdit_attn_v8_relayout)."""
    import torch
    B, H, S, D = _shape4(v8_tokens)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, H, -(-S // FP8_BLOCK), D, FP8_BLOCK), dtype=torch.uint8,
                              device=v8_tokens.device)
    lib = load()
    check(lib.vdit_attn_v8_relayout(_dev(v8_tokens, torch.uint8, "src"), _dev(out, torch.uint8, "dst"),
                                    B, H, S, D, 1, _stream(stream)))
    return out


def vdit_attn_v8_from_tiles(v8_tiles, S, out=None, stream=None):
    """The fp8 kernels' tiled V codes [B, H, ceil(S/64), 128, 64] ->
    token-major [B, H, S, 128] (vdit_attn_v8_relayout)."""
    import torch
    if v8_tiles.dim() != 5:
        raise ValueError("expected tiled codes [B, H, ceil(S/64), 128, 64]")
    B, H, nb, D, blk = (int(x) for x in v8_tiles.shape)
    if blk != FP8_BLOCK or nb != -(-int(S) // FP8_BLOCK):
        raise ValueError("tile count does not match S")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, H, int(S), D), dtype=torch.uint8, device=v8_tiles.device)
    lib = load()
    check(lib.vdit_attn_v8_relayout(_dev(v8_tiles, torch.uint8, "src"), _dev(out, torch.uint8, "dst"),
                                    B, H, int(S), D, 0, _stream(stream)))
    return out


def vdit_attn_fwd_fp8(z, scale=None, o=None, stream=None, expcast=False, chunk=0, block_mask=None):
    """fp8 attention on pre-pass outputs ``z`` (dict as from vdit_attn_quant_fp8);
    returns bf16 o [B, H, S, 128].  ``expcast`` selects the ExpCast-FP8 entry
    point (P bytes written directly from the log domain).  A ``z`` holding
    v_bmean (V block means) goes to vdit_attn_fwd_fp8_vsmooth; ``chunk`` > 0
    (block-causal) or ``block_mask`` (block-sparse, uint8 [B, H, ceil(S/128),
    ceil(S/64)]) go to vdit_attn_fwd_fp8_masked."""
    import torch
    B, H, S, D = _shape4(z["q8"])
    if o is None:
        with _alloc_on(stream):
            o = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=z["q8"].device)
    scale = D ** -0.5 if scale is None else float(scale)
    kmb = int(z["k_mean"].shape[2])
    lib = load()
    if chunk or block_mask is not None:
        if "v_bmean" in z:
            raise ValueError("key masks take the per-channel V mean pre-pass (v_mean)")
        if block_mask is not None:
            want = (B, H, -(-S // SPARSE_Q_BLOCK), -(-S // SPARSE_K_TILE))
            if tuple(block_mask.shape) != want:
                raise ValueError(f"block_mask must have shape {want}, not {tuple(block_mask.shape)}")
            if block_mask.dtype == torch.bool:
                block_mask = block_mask.view(torch.uint8)
        mask_ptr = _dev(block_mask, torch.uint8, "block_mask") if block_mask is not None else None
        check(lib.vdit_attn_fwd_fp8_masked(
            _dev(z["q8"], torch.uint8, "q8"), _dev(z["k8"], torch.uint8, "k8"),
            _dev(z["v8"], torch.uint8, "v8"), _dev(z["q_scale"], torch.float32, "q_scale"),
            _dev(z["k_scale"], torch.float32, "k_scale"), _dev(z["k_mean"], torch.float32, "k_mean"),
            kmb, _dev(z["v_mean"], torch.float32, "v_mean"), _dev(z["v_scale"], torch.float32, "v_scale"),
            _dev(o, torch.bfloat16, "o"), B, H, S, D, scale, int(chunk), mask_ptr,
            1 if expcast else 0, _stream(stream)))
        return o
    if "v_bmean" in z:
        check(lib.vdit_attn_fwd_fp8_vsmooth(
            _dev(z["q8"], torch.uint8, "q8"), _dev(z["k8"], torch.uint8, "k8"),
            _dev(z["v8"], torch.uint8, "v8"), _dev(z["q_scale"], torch.float32, "q_scale"),
            _dev(z["k_scale"], torch.float32, "k_scale"), _dev(z["k_mean"], torch.float32, "k_mean"),
            kmb, _dev(z["v_bmean"], torch.bfloat16, "v_bmean"),
            _dev(z["v_scale"], torch.float32, "v_scale"),
            _dev(o, torch.bfloat16, "o"), B, H, S, D, scale, 1 if expcast else 0, _stream(stream)))
        return o
    fn = lib.vdit_attn_fwd_fp8_expcast if expcast else lib.vdit_attn_fwd_fp8
    check(fn(
        _dev(z["q8"], torch.uint8, "q8"), _dev(z["k8"], torch.uint8, "k8"),
        _dev(z["v8"], torch.uint8, "v8"), _dev(z["q_scale"], torch.float32, "q_scale"),
        _dev(z["k_scale"], torch.float32, "k_scale"), _dev(z["k_mean"], torch.float32, "k_mean"),
        kmb, _dev(z["v_mean"], torch.float32, "v_mean"), _dev(z["v_scale"], torch.float32, "v_scale"),
        _dev(o, torch.bfloat16, "o"), B, H, S, D, scale, _stream(stream)))
    return o


def vdit_vsmooth_group(v, n_clusters=None, rounds=4, stream=None):
    """k-means grouping of the value tokens of bf16 v [B, H, S, 128]; returns
    (perm, labels, centroids): int32 [B, H, S], int32 [B, H, S] and float32
    [B, H, n_clusters, 128].  n_clusters defaults to ceil(S / 128)."""
    import torch
    B, H, S, D = _shape4(v)
    k = -(-S // 128) if n_clusters is None else int(n_clusters)
    lib = load()
    ws_bytes = int(lib.vdit_vsmooth_group_workspace_size(B, H, S, D, k))
    if ws_bytes == 0:
        raise ValueError("invalid shape or n_clusters for V-Smooth Group")
    with _alloc_on(stream):
        perm = torch.empty((B, H, S), dtype=torch.int32, device=v.device)
        labels = torch.empty((B, H, S), dtype=torch.int32, device=v.device)
        cent = torch.empty((B, H, k, D), dtype=torch.float32, device=v.device)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=v.device)
    check(lib.vdit_vsmooth_group(
        _dev(v, torch.bfloat16, "v"), _dev(perm, torch.int32, "perm"),
        _dev(labels, torch.int32, "labels"), _dev(cent, torch.float32, "centroids"),
        B, H, S, D, k, int(rounds), _dev(ws, torch.uint8, "workspace"), ws_bytes, _stream(stream)))
    return perm, labels, cent


def vdit_permute_tokens(x, perm, out=None, stream=None):
    """out[b, h, i] = x[b, h, perm[b, h, i]] for bf16 [B, H, S, 128]."""
    import torch
    B, H, S, D = _shape4(x)
    if tuple(perm.shape) != (B, H, S):
        raise ValueError("perm must have shape [B, H, S]")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty_like(x)
    lib = load()
    check(lib.vdit_permute_tokens(_dev(x, torch.bfloat16, "x"), _dev(perm, torch.int32, "perm"),
                                  _dev(out, torch.bfloat16, "out"), B, H, S, D, _stream(stream)))
    return out
