"""The allocation-free fp8 pre-pass (vdit_attn_quant_fp8_noalloc) against the
workspace entry point (vdit_attn_quant_fp8), through the C ABI.

Both run the same kernels; only where the intermediate statistics live
differs (the library's static device scratch, or the caller's workspace).
The pre-pass is integer work, so every output must agree bit for bit, on
two calls in a row, the second smaller than the first (the scratch keeps the
first call's contents).  The size limit is checked before any HIP call, so
that part runs without a GPU."""

import ctypes

import numpy as np
import pytest

from video_diffusion_transformer_vdit_amd import binding, inputs

from gpu_util import log, to_dev

A = 0x10000  # fake, 16-byte aligned addresses: validation never dereferences
KEYS = ["q8", "k8", "v8", "q_scale", "k_scale", "k_mean", "v_mean", "v_scale"]


def noalloc_status(B, H, S, k_mean_blocks):
    lib = binding.load()
    st = lib.vdit_attn_quant_fp8_noalloc(A, A, A, A, A, A, A, A, A, k_mean_blocks, A, A,
                                         B, H, S, 128, None)
    return st, lib.vdit_last_error().decode()


def test_noalloc_scratch_size_and_limit():
    lib = binding.load()
    cap = int(lib.vdit_attn_quant_fp8_noalloc_max_workspace())
    assert cap == 128 << 20
    # the 720p workload with one K mean per 64-token block fits ...
    need = int(lib.vdit_attn_quant_fp8_workspace_size(1, 40, 75600, 128, 1182))
    assert 0 < need <= cap
    # ... a larger problem is refused before any HIP call, naming the sizes
    big = int(lib.vdit_attn_quant_fp8_workspace_size(1, 64, 75600, 128, 1182))
    assert big > cap
    st, err = noalloc_status(1, 64, 75600, 1182)
    assert st == 2 and "allocation-free" in err and str(big) in err, (st, err)
    # the usual argument checks still apply
    st, err = noalloc_status(1, 1, 100, 3)
    assert st == 2 and "k_mean_blocks" in err
    st = lib.vdit_attn_quant_fp8_noalloc(None, A, A, A, A, A, A, A, A, 2, A, A, 1, 1, 100, 128, None)
    assert st == 1 and b"null pointer: q" in lib.vdit_last_error()


def rand_bits(shape, seed, scale=1.0, offset=0.0):
    g = np.random.default_rng(seed)
    return inputs.f32_to_bf16_bits((g.standard_normal(shape) * scale + offset).astype(np.float32))


@pytest.mark.gpu
def test_noalloc_prepass_matches_workspace_entry_point():
    """Two calls in a row through the allocation-free entry point, the 720p
    workload (40 heads x 75,600 tokens) and then a smaller, ragged problem
    (B = 2, H = 3, S = 1,000, one K mean per head), each bit-identical to the
    workspace entry point on the same inputs."""
    import torch
    w = inputs.get_workload("wan2.1-14b-720p-fp8")
    q, k, v = inputs.make_inputs(w)
    cases = [("720p", (q, k, v), None),
             ("B=2 H=3 S=1000 global K mean",
              (rand_bits((2, 3, 1000, 128), 1), rand_bits((2, 3, 1000, 128), 2, 2.0, 0.3),
               rand_bits((2, 3, 1000, 128), 3, 1.5, -4.0)), 1)]
    for name, (qb, kb, vb), kmb in cases:
        log(f"no-alloc pre-pass: {name}")
        qd, kd, vd = to_dev(qb), to_dev(kb), to_dev(vb)
        ref = binding.vdit_attn_quant_fp8(qd, kd, vd, k_mean_blocks=kmb)
        B, H, S, _ = qd.shape
        out = binding.quant_buffers(B, H, S, kmb, qd.device)
        for key in KEYS:                 # sentinels: every output must be written
            out[key].fill_(0x7F if out[key].dtype == torch.uint8 else float("nan"))
        got = binding.vdit_attn_quant_fp8_noalloc(qd, kd, vd, out)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], ref[key]), f"{name}: {key}"
        del ref, out, got, qd, kd, vd
        torch.cuda.empty_cache()
