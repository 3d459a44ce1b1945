"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments before any HIP call (so this runs without a GPU)."""

import ctypes
import os
import re

import pytest

from video_diffusion_transformer_vdit_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vdit_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="library not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vdit_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["vdit_attn_fwd", "vdit_attn_quant_fp8", "vdit_attn_fwd_fp8", "vdit_status_str",
              "vdit_last_error", "vdit_abi_version", "vdit_attn_quant_fp8_workspace_size"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) <= set(binding.SIGNATURES)


def test_abi_version_and_status_strings():
    lib = binding.load()
    assert lib.vdit_abi_version() == 1
    assert lib.vdit_status_str(0) == b"ok"
    assert lib.vdit_status_str(1) == b"invalid argument"
    assert lib.vdit_status_str(2) == b"unsupported argument"
    assert lib.vdit_status_str(3) == b"HIP runtime error"
    assert lib.vdit_status_str(99) == b"unknown status"


A = 0x10000  # fake, 16-byte aligned addresses: validation never dereferences


def fwd(q=A, k=A * 2, v=A * 3, o=A * 4, B=1, H=1, S=16, D=128, scale=0.1, dtype=0):
    lib = binding.load()
    st = lib.vdit_attn_fwd(q, k, v, o, B, H, S, D, scale, dtype, None)
    return st, lib.vdit_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), 1, "null pointer: q"),
    (dict(o=None), 1, "null pointer: o"),
    (dict(k=A + 8), 1, "not 16-byte aligned: k"),
    (dict(B=0), 1, "B, H and S"),
    (dict(H=-1), 1, "B, H and S"),
    (dict(S=0), 1, "B, H and S"),
    (dict(D=64), 2, "D = 128"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(dtype=1), 2, "dtype"),
    (dict(o=A, q=A), 1, "overlaps"),
    (dict(B=1 << 16, H=1 << 16, S=1 << 10), 2, "too large"),
    (dict(S=(1 << 30) + 1), 2, "2^30"),
    (dict(S=(1 << 31) - 1), 2, "2^30"),
])
def test_fwd_validation(kw, status, msg):
    st, err = fwd(**kw)
    assert st == status and msg in err, (st, err)


def test_fp8_validation():
    lib = binding.load()
    S = 200
    nb = 4
    ws = lib.vdit_attn_quant_fp8_workspace_size(1, 2, S, 128, nb)
    assert ws > 0
    assert lib.vdit_attn_quant_fp8_workspace_size(1, 2, S, 128, 3) == 0
    assert lib.vdit_attn_quant_fp8_workspace_size(1, 2, S, 64, nb) == 0
    args = [A] * 9
    st = lib.vdit_attn_quant_fp8(*args[:9], nb, A, A, A, ws - 1, 1, 2, S, 128, None)
    assert st == 1 and b"workspace too small" in lib.vdit_last_error()
    st = lib.vdit_attn_quant_fp8(*args[:9], 2, A, A, A, ws, 1, 2, S, 128, None)
    assert st == 2 and b"k_mean_blocks" in lib.vdit_last_error()
    st = lib.vdit_attn_quant_fp8(*args[:9], nb, A, A, None, ws, 1, 2, S, 128, None)
    assert st == 1 and b"workspace" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8(A, A, A, A, A, A, nb, A, A, A, 1, 2, S, 128, 0.0, None)
    assert st == 1 and b"scale" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8(A, A, A, A, A, A, 5, A, A, A, 1, 2, S, 128, 0.1, None)
    assert st == 2 and b"k_mean_blocks" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8(A, A, A, A + 4, A, A, nb, A, A, A, 1, 2, S, 128, 0.1, None)
    assert st == 1 and b"q_scale" in lib.vdit_last_error()


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        binding.vdit_attn_fwd(x, x, x, o=x.clone())


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = binding._lib
    binding._lib = None
    try:
        return binding.load(path)
    finally:
        binding._lib = saved


def test_block_causal_and_expcast_validation():
    lib = binding.load()
    st = lib.vdit_attn_fwd_block_causal(A, A * 2, A * 3, A * 4, 1, 1, 16, 128, 0.1, 0, 0, None)
    assert st == 1 and b"chunk" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_block_causal(A, A * 2, A * 3, A * 4, 1, 1, 16, 64, 0.1, 4, 0, None)
    assert st == 2 and b"D = 128" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_block_causal(None, A * 2, A * 3, A * 4, 1, 1, 16, 128, 0.1, 4, 0, None)
    assert st == 1 and b"null pointer: q" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_expcast(A, A, A, A, A, A, 4, A, A, A, 1, 2, 200, 128, 0.0, None)
    assert st == 1 and b"scale" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_expcast(A, A, A, A, A, A, 5, A, A, A, 1, 2, 200, 128, 0.1, None)
    assert st == 2 and b"k_mean_blocks" in lib.vdit_last_error()


def test_vsmooth_validation():
    lib = binding.load()
    assert [lib.vdit_attn_vsmooth_blocks(s) for s in (0, 1, 128, 129, 2048, 2049, 75600)] == \
        [0, 16, 16, 16, 16, 32, 592]
    st = lib.vdit_attn_quant_fp8_vsmooth(A, A, A, A, A, A, A, A, A, 4, None, A, A, 1 << 30,
                                         1, 2, 200, 128, None)
    assert st == 1 and b"null pointer: v_bmean" in lib.vdit_last_error()
    st = lib.vdit_attn_quant_fp8_vsmooth(A, A, A, A, A, A, A, A, A, 5, A, A, A, 1 << 30,
                                         1, 2, 200, 128, None)
    assert st == 2 and b"k_mean_blocks" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_vsmooth(A, A, A, A, A, A, 4, A, A, A, 1, 2, 200, 128, 0.1, 2, None)
    assert st == 1 and b"expcast" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_vsmooth(A, A, A, A, A, A, 4, None, A, A, 1, 2, 200, 128, 0.1, 0, None)
    assert st == 1 and b"null pointer: v_bmean" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_vsmooth(A, A, A, A, A, A, 4, A + 2, A, A, 1, 2, 200, 128, 0.1, 0, None)
    assert st == 1 and b"aligned: v_bmean" in lib.vdit_last_error()


def test_block_sparse_validation():
    lib = binding.load()
    st = lib.vdit_attn_fwd_block_sparse(A, A * 2, A * 3, A * 4, 1, 1, 16, 128, 0.1, None, 0, None)
    assert st == 1 and b"null pointer: block_mask" in lib.vdit_last_error()
    # any alignment is fine for the mask; D is checked as for the dense call
    st = lib.vdit_attn_fwd_block_sparse(A, A * 2, A * 3, A * 4, 1, 1, 16, 64, 0.1, A + 1, 0, None)
    assert st == 2 and b"D = 128" in lib.vdit_last_error()
    far = 1 << 40  # fake buffers far enough apart not to overlap at this size
    st = lib.vdit_attn_fwd_block_sparse(A, A + far, A + 2 * far, A + 3 * far, 1, 1, 1048577, 128,
                                        0.1, A + 1, 0, None)
    assert st == 2 and b"1048576" in lib.vdit_last_error()


def test_vsmooth_group_validation():
    lib = binding.load()
    assert lib.vdit_vsmooth_group_workspace_size(1, 2, 75600, 128, 591) > 0
    assert lib.vdit_vsmooth_group_workspace_size(1, 2, 100, 128, 101) == 0   # more clusters than tokens
    assert lib.vdit_vsmooth_group_workspace_size(1, 2, 10 ** 6, 128, 4097) == 0
    st = lib.vdit_vsmooth_group(A, A, A, A, 1, 2, 100, 128, 0, 4, A, 1 << 30, None)
    assert st == 1 and b"n_clusters" in lib.vdit_last_error()
    st = lib.vdit_vsmooth_group(A, A, A, A, 1, 2, 100, 128, 10, 65, A, 1 << 30, None)
    assert st == 1 and b"rounds" in lib.vdit_last_error()
    st = lib.vdit_vsmooth_group(A, A, A, A, 1, 2, 100, 128, 10, 4, A, 16, None)
    assert st == 1 and b"workspace too small" in lib.vdit_last_error()
    st = lib.vdit_permute_tokens(A, A, A, 1, 1, 16, 128, None)
    assert st == 1 and b"overlaps" in lib.vdit_last_error()


def test_fp8_output_must_not_overlap_the_codes():
    lib = binding.load()
    far = 1 << 40
    S, nb = 200, 4
    ptrs = [A + i * far for i in range(10)]  # q8 k8 v8 q_scale k_scale k_mean v_mean v_scale o
    q8, k8, v8, qs, ks, km, vm, vs, o = ptrs[:9]
    for alias in (q8, k8, v8, v8 + 256 * 128):
        st = lib.vdit_attn_fwd_fp8(q8, k8, v8, qs, ks, km, nb, vm, vs, alias, 1, 2, S, 128, 0.1, None)
        assert st == 1 and b"o overlaps" in lib.vdit_last_error()


def test_fp8_masked_validation():
    lib = binding.load()
    args = (A, A, A, A, A, A, 4, A, A, A, 1, 2, 200, 128, 0.1)
    st = lib.vdit_attn_fwd_fp8_masked(*args, -1, None, 0, None)
    assert st == 1 and b"chunk" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_masked(*args, 64, A + 1, 0, None)
    assert st == 1 and b"not both" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_masked(*args, 0, None, 3, None)
    assert st == 1 and b"expcast" in lib.vdit_last_error()
    far = 1 << 40  # fake buffers far apart: no overlap at this size
    big = 1048577
    st = lib.vdit_attn_fwd_fp8_masked(A, A + far, A + 2 * far, A + 3 * far, A + 4 * far, A + 5 * far,
                                      -(-big // 64), A + 6 * far, A + 7 * far, A + 8 * far,
                                      1, 1, big, 128, 0.1, 0, A + 9 * far, 0, None)
    assert st == 2 and b"1048576" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_masked(*args[:7], None, *args[8:], 64, None, 0, None)
    assert st == 1 and b"v_mean" in lib.vdit_last_error()
    st = lib.vdit_attn_fwd_fp8_masked(*args[:6], 3, *args[7:], 64, None, 0, None)
    assert st == 2 and b"k_mean_blocks" in lib.vdit_last_error()


def test_fp8_masks_reject_block_v_means():
    import torch
    z = {"q8": torch.empty((1, 1, 64, 128), dtype=torch.uint8),
         "k_mean": torch.empty((1, 1, 1, 128)),
         "v_bmean": torch.empty((1, 1, 128, 16), dtype=torch.bfloat16)}
    with pytest.raises(ValueError, match="per-channel V mean"):
        binding.vdit_attn_fwd_fp8(z, chunk=32)


def test_sizes_refuse_sequences_past_the_limit():
    """No size query overflows 32-bit token arithmetic: S past 2^30 gives 0."""
    lib = binding.load()
    big = (1 << 31) - 1
    assert lib.vdit_attn_vsmooth_blocks(big) == 0
    assert lib.vdit_attn_vsmooth_blocks(1 << 30) == -(-(1 << 30) // 128)
    assert lib.vdit_attn_quant_fp8_workspace_size(1, 1, big, 128, 1) == 0
    assert lib.vdit_vsmooth_group_workspace_size(1, 1, big, 128, 16) == 0


def test_v8_relayout_validation():
    lib = binding.load()
    st = lib.vdit_attn_v8_relayout(A, A * 4, 1, 2, 200, 128, 2, None)
    assert st == 1 and b"to_tiles" in lib.vdit_last_error()
    st = lib.vdit_attn_v8_relayout(None, A * 4, 1, 2, 200, 128, 1, None)
    assert st == 1 and b"null pointer: src" in lib.vdit_last_error()
    st = lib.vdit_attn_v8_relayout(A, A + 8, 1, 2, 200, 128, 1, None)
    assert st == 1 and b"aligned: dst" in lib.vdit_last_error()
    st = lib.vdit_attn_v8_relayout(A, A + 16 * 1024, 1, 2, 200, 128, 0, None)
    assert st == 1 and b"overlap" in lib.vdit_last_error()
    st = lib.vdit_attn_v8_relayout(A, A * 1000, 1, 2, 200, 64, 0, None)
    assert st == 2 and b"D = 128" in lib.vdit_last_error()
