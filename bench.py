#!/usr/bin/env python3
"""Benchmark of the spatiotemporal self-attention forward on one MI355X.

Default: the 720p Wan2.1-14B-shaped self-attention (B=1, H=40, S=75,600,
D=128, bf16, 4 outlier channels per head in K and V) through the C ABI
(vdit_attn_fwd), W warm-up launches then K timed launches bracketed by HIP
events on the launch stream.  Prints ONE JSON line with the throughput in
TFLOP/s (4 B H S^2 D per launch), the roofline of the attention kernel
against the dense bf16 MFMA peak, the fp8 path (pre-pass + fp8 attention on
the same tensors) timed the same way, and the fp64 CPU oracle timed on a
bounded row sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-fp8]
                  [--no-cpu-baseline] [--cpu-seconds T]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from video_diffusion_transformer_vdit_amd import binding, inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
HEADLINE = "wan2.1-14b-720p"
METRIC = "attention TFLOP/s & % of bf16 MFMA peak at S=75,600 H=40 D=128"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_launches(fn, steps, warmup, detail=False):
    """Average ms per launch over `steps` launches after `warmup` ones, with
    HIP events recorded on torch's current stream (the launch stream).

    With `detail`, an event also follows every launch, and while the launches
    run the host samples the graphics clock and the socket power from sysfs;
    it then returns (average ms, per-launch ms list, clock samples in MHz,
    power samples in W)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if detail else 2)]
    marks[0].record()
    for i in range(steps):
        fn()
        if detail:
            marks[i + 1].record()
    marks[-1].record()
    clocks, powers = [], []
    path = sclk_path() if detail else None
    ppath = power_path() if detail else None
    while (path or ppath) and not marks[-1].query():
        mhz = read_sclk(path) if path else None
        if mhz is not None:
            clocks.append(mhz)
        watts = read_power(ppath) if ppath else None
        if watts is not None:
            powers.append(watts)
        time.sleep(0.01)
    torch.cuda.synchronize()
    avg = marks[0].elapsed_time(marks[-1]) / steps
    if not detail:
        return avg
    return avg, [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)], clocks, powers


def sclk_path():
    """The sysfs file that lists the graphics clock levels of torch's device
    0, the current one marked with '*'; None if sysfs has no readable one."""
    import glob
    import torch
    p = torch.cuda.get_device_properties(0)
    path = "/sys/bus/pci/devices/%04x:%02x:%02x.0/pp_dpm_sclk" % (
        p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
    if os.access(path, os.R_OK):
        return path
    found = [f for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk") if os.access(f, os.R_OK)]
    return found[0] if len(found) == 1 else None


def power_path():
    """The hwmon file with the socket power of torch's device 0 (microwatts),
    or None if sysfs has no readable one."""
    import glob
    import torch
    p = torch.cuda.get_device_properties(0)
    dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
    for name in ("power1_average", "power1_input"):
        found = [f for f in glob.glob(os.path.join(dev, "hwmon", "hwmon*", name)) if os.access(f, os.R_OK)]
        if found and read_power(found[0]) is not None:
            return found[0]
    return None


def power_cap():
    """The socket power cap in W (hwmon power1_cap beside the power file), or None."""
    path = power_path()
    return read_power(os.path.join(os.path.dirname(path), "power1_cap")) if path else None


def read_power(path):
    """Socket power in W from a hwmon file in microwatts, or None."""
    try:
        with open(path) as f:
            uw = int(f.read().strip())
    except (OSError, ValueError):
        return None
    return uw / 1e6 if uw > 0 else None


def read_sclk(path):
    """Current graphics clock in MHz from a pp_dpm_sclk listing, or None."""
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    digits = "".join(c for c in line.split(":", 1)[1] if c.isdigit() or c == ".")
                    return float(digits) if digits else None
    except (OSError, IndexError, ValueError):
        return None
    return None


CSRC = os.path.join(ROOT, "video_diffusion_transformer_vdit_amd", "csrc")
KERNEL_SOURCE = os.path.join(CSRC, "attn_bf16.hip")
FP8_SOURCE = os.path.join(CSRC, "attn_fp8.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_kernel__wan2.1-14b-720p__hbm_traffic.txt")
COUNTER_FILE = os.path.join(ROOT, "profiles", "attn_kernels__wan2.1-14b-720p__valu_mfma_counters.txt")


def source_sha256(path=KERNEL_SOURCE):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_counters():
    """Per-kernel counter figures (clock, MFMA busy, VALU active, LDS active)
    from the committed counter summary, keyed by kernel name; only kernels
    whose source file still has the recorded sha256 are returned."""
    if not os.path.exists(COUNTER_FILE):
        return {}
    shas, rows = {}, {}
    cols = None
    with open(COUNTER_FILE) as f:
        for line in f:
            if line.startswith("# ") and "sha256:" in line:
                name, _, sha = line[2:].partition("sha256:")
                shas[name.strip()] = sha.strip()
            elif line.startswith("# kernel |"):
                cols = [c.strip() for c in line[2:].split("|")]
            elif cols and not line.startswith("#") and line.strip():
                parts = line.split()
                name = parts[0]
                if len(parts) == len(cols):
                    rows[name] = dict(zip(cols[1:], (float(x) for x in parts[1:])))
    ok = {"attn_fwd_bf16": shas.get("attn_bf16.hip") == source_sha256(KERNEL_SOURCE),
          "attn_fwd_fp8": shas.get("attn_fp8.hip") == source_sha256(FP8_SOURCE)}
    return {k: v for k, v in rows.items() if any(k.startswith(p) and good for p, good in ok.items())}


def measured_traffic():
    """HBM bytes per launch of the bf16 kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain-copy calibration);
    None when absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != source_sha256():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def calibration_copy(n_bytes=1 << 31, reps=3):
    """Plain device-to-device copy of a known size, for scaling FETCH_SIZE /
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    x = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n_bytes, "reps": reps}), flush=True)


def cpu_baseline(w, q, k, v, scale, seconds, gpu_head0=None):
    """fp64 oracle (as it stands) on head 0, 256-row chunks until `seconds`
    have elapsed; rate scaled to TFLOP/s of the same attention arithmetic.
    The oracle's matrix products run on numpy's BLAS threads, so `cores` is
    that thread count; the host's logical CPUs and the process's affinity
    set are reported beside it.  With `gpu_head0` (the timed kernel's bf16
    output bits of head 0, [S, D]) the rows the oracle computed also check
    that output: max-abs and L1 mean-rel against the oracle rounded to bf16,
    and how many elements exceed 1e-2 and by how many bf16 steps of their
    magnitude at most (outside the timed loop, which the comparison does not
    slow)."""
    from oracle import attention as oa
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = affinity
    rows_done = 0
    t0 = time.perf_counter()
    chunk = 256
    start = 0
    outs = []
    while True:
        rows = np.arange(start, min(w.S, start + chunk))
        ref = oa.attention_head(q[0, 0], k[0, 0], v[0, 0], scale, rows=rows)
        if gpu_head0 is not None and len(outs) * chunk < w.S:
            outs.append((rows, ref))
        rows_done += rows.size
        start = (start + chunk) % w.S
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    check = {}
    if gpu_head0 is not None and outs:
        num = den = 0.0
        worst = worst_steps = 0.0
        n = n_over = 0
        for rows, ref in outs:
            ref_b = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
            got = inputs.bf16_bits_to_f32(gpu_head0[rows]).astype(np.float64)
            err = np.abs(got - ref_b)
            num += float(err.sum())
            den += float(np.abs(ref_b).sum())
            worst = max(worst, float(err.max()))
            over = err > 1e-2
            n_over += int(over.sum())
            if over.any():
                # one bf16 step of the reference: 2^-7 relative
                worst_steps = max(worst_steps, float((err[over] / (2.0 ** -7 * np.abs(ref_b[over]))).max()))
            n += rows.size
        check = {"check_rows": n, "max_abs_vs_oracle": worst, "mean_rel_vs_oracle": num / den,
                 "elements_over_1e-2": n_over, "over_1e-2_max_bf16_steps": worst_steps}
    flop = rows_done * 4.0 * w.S * w.D
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "blas_threads": int(threads),
        "cpu_count": os.cpu_count(),
        "affinity_cpus": affinity,
        "kind": "oracle",
        "sample": (f"{rows_done} query rows of head 0 of {w.name} (S={w.S}), fp64 numpy, "
                   f"{dt:.1f} s; full call extrapolates to {w.flop / (flop / dt):.0f} s"),
        **check,
    }


CONFIGS = ("tiny-3x16x16", "wan2.1-1.3b-480p", "wan2.2-720p-16x")


def other_configs(steps, warmup, fp8=True):
    """bf16 attention (and the fp8 pre-pass + attention) on the workloads
    other than the headline, timed the same way: TFLOP/s and the fraction of
    the dense peak of the arithmetic's type."""
    import torch
    out = {}
    for name in CONFIGS:
        w = inputs.get_workload(name)
        scale = float(np.float32(1.0 / math.sqrt(w.D)))
        log(f"[bench] {name} {w.shape}")
        qb, kb, vb = inputs.make_inputs(w)
        q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for b in (qb, kb, vb))
        del qb, kb, vb
        o = torch.empty_like(q)
        # the tiny workload runs for microseconds: more launches to time
        n = steps * (50 if w.S < 4096 else 1)
        ms = time_launches(lambda: binding.vdit_attn_fwd(q, k, v, o=o, scale=scale), n, warmup)
        tf = w.flop / (ms * 1e-3) / 1e12
        r = {"shape": list(w.shape), "bf16_ms": round(ms, 4), "bf16_tflops": round(tf, 2),
             "bf16_peak_fraction": round(tf / PEAK_BF16_TFLOPS, 4)}
        if fp8:
            z = binding.vdit_attn_quant_fp8(q, k, v)
            ms_a = time_launches(lambda: binding.vdit_attn_fwd_fp8(z, scale=scale, o=o), n, warmup)
            ms_x = time_launches(lambda: binding.vdit_attn_fwd_fp8(z, scale=scale, o=o, expcast=True),
                                 n, warmup)
            for key, t in (("fp8", ms_a), ("fp8_expcast", ms_x)):
                tf8 = w.flop / (t * 1e-3) / 1e12
                r[key + "_ms"] = round(t, 4)
                r[key + "_tflops"] = round(tf8, 2)
                r[key + "_peak_fraction"] = round(tf8 / PEAK_FP8_TFLOPS, 4)
            del z
        out[name] = r
        del q, k, v, o
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the bf16/fp8 timings of the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a 2 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange inside attention).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy:
        calibration_copy()
        return
    binding.load()

    w = inputs.get_workload(args.workload)
    scale = float(np.float32(1.0 / math.sqrt(w.D)))
    log(f"[bench] generating {w.name} {w.shape}")
    qb, kb, vb = inputs.make_inputs(w)

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(qb), dev(kb), dev(vb)
    o = torch.empty_like(q)
    log("[bench] bf16 attention")
    ms, per_launch, clocks, powers = time_launches(lambda: binding.vdit_attn_fwd(q, k, v, o=o, scale=scale),
                                           args.steps, args.warmup, detail=True)
    # head 0 of the timed kernel's output, for the CPU leg's check
    head0 = o[0, 0].view(torch.int16).cpu().numpy().view(np.uint16)
    tflops = w.flop / (ms * 1e-3) / 1e12
    sclk = float(np.median(clocks)) if clocks else None
    headline = w.name == HEADLINE
    counters = measured_counters() if headline else {}
    cnt_bf16 = counters.get("attn_fwd_bf16_kernel<0>", {})
    traffic = measured_traffic() if headline else None
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q/K/V with the workload's structure; no model weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "structure": w.structure, "causal": False, "scale": scale},
        "peak_fraction": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_bf16_kernel<0>",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "hbm_gbs": round(traffic / (ms * 1e-3) / 1e9, 1) if traffic else None,
            "algorithmic_flop_per_launch": w.flop,
            "algorithmic_bytes_per_launch": 4 * w.B * w.H * w.S * w.D * 2,
            # from the committed counter pass on the same kernel source
            # (rocprofv3 --pmc; null once the source has changed)
            "mfma_busy": cnt_bf16.get("mfma_busy"),
            "valu_active": cnt_bf16.get("valu_active"),
            "counter_clock_ghz": cnt_bf16.get("clock_GHz"),
        },
        "launch_ms": {"median": round(float(np.median(per_launch)), 4),
                      "min": round(min(per_launch), 4), "max": round(max(per_launch), 4)},
        # one exponential per (query, key) score
        "exp2_per_s": float("%.4g" % (w.B * w.H * w.S * w.S / (ms * 1e-3))),
        # graphics clock sampled from sysfs while the timed launches ran, and
        # the dense bf16 peak rescaled from the 2.4 GHz nameplate to it
        "sclk_mhz": {"median": sclk, "min": min(clocks) if clocks else None,
                     "max": max(clocks) if clocks else None, "samples": len(clocks)},
        # socket power sampled the same way, with the cap beside it: the kernel
        # runs near the cap, where the power management holds the clock above
        "socket_power_w": {"median": round(float(np.median(powers)), 1) if powers else None,
                           "max": round(max(powers), 1) if powers else None, "samples": len(powers),
                           "cap": power_cap()},
        "peak_at_observed_clock": round(PEAK_BF16_TFLOPS * sclk / 2400.0, 1) if sclk else None,
        "frac_at_observed_clock": round(tflops / (PEAK_BF16_TFLOPS * sclk / 2400.0), 4) if sclk else None,
    }

    # block-causal variant, one chunk per latent frame; FLOP counts only the
    # scored (query, key) pairs: sum over rows of the row's key limit
    chunk = w.tokens_per_frame
    rows = np.arange(w.S, dtype=np.int64)
    pairs = int(np.minimum((rows // chunk + 1) * chunk, w.S).sum())
    causal_flop = 4 * w.B * w.H * pairs * w.D
    log("[bench] bf16 block-causal attention")
    ms_c = time_launches(lambda: binding.vdit_attn_fwd_block_causal(q, k, v, chunk, o=o, scale=scale),
                         args.steps, args.warmup)
    result["block_causal"] = {
        "chunk": chunk,
        "scored_pair_fraction": round(pairs / (w.S * w.S), 4),
        "ms": round(ms_c, 4),
        "tflops": round(causal_flop / (ms_c * 1e-3) / 1e12, 2),
        "peak_fraction": round(causal_flop / (ms_c * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }

    # block-sparse variant on a seeded 25% map (each 256-query group keeps a
    # quarter of the key tiles plus its own); FLOP over scored pairs only
    mask = inputs.make_block_mask(w.B, w.H, w.S, 0.25, seed=w.seed)
    rows_qb = np.minimum(128, w.S - 128 * np.arange(mask.shape[2]))
    keys_kt = np.minimum(64, w.S - 64 * np.arange(mask.shape[3]))
    sp_pairs = int((mask.astype(np.int64) * rows_qb[:, None] * keys_kt[None, :]).sum())
    sparse_flop = 4 * sp_pairs * w.D
    mask_dev = torch.from_numpy(mask).cuda()
    log("[bench] bf16 block-sparse attention")
    ms_s = time_launches(lambda: binding.vdit_attn_fwd_block_sparse(q, k, v, mask_dev, o=o, scale=scale),
                         args.steps, args.warmup)
    result["block_sparse"] = {
        "density": round(sp_pairs / (w.B * w.H * w.S * w.S), 4),
        "ms": round(ms_s, 4),
        "tflops": round(sparse_flop / (ms_s * 1e-3) / 1e12, 2),
        "peak_fraction": round(sparse_flop / (ms_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }

    if not args.no_fp8:
        log("[bench] fp8 pre-pass + attention")
        z = binding.vdit_attn_quant_fp8(q, k, v)
        o8 = torch.empty_like(q)
        ms_q = time_launches(lambda: binding.vdit_attn_quant_fp8(q, k, v, out=z), args.steps, args.warmup)
        ms_a = time_launches(lambda: binding.vdit_attn_fwd_fp8(z, scale=scale, o=o8), args.steps, args.warmup)
        ms_x = time_launches(lambda: binding.vdit_attn_fwd_fp8(z, scale=scale, o=o8, expcast=True),
                             args.steps, args.warmup)
        # reads Q, K, V (2 B each) and V again (2 B); writes three 1-byte code tensors
        prepass_bytes = w.B * w.H * w.S * w.D * (2 * 3 + 2 + 3)
        result["fp8"] = {
            "attention_ms": round(ms_a, 4),
            "attention_tflops": round(w.flop / (ms_a * 1e-3) / 1e12, 2),
            "attention_peak_fraction": round(w.flop / (ms_a * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "prepass_ms": round(ms_q, 4),
            "prepass_gbs": round(prepass_bytes / (ms_q * 1e-3) / 1e9, 1),
            "combined_tflops": round(w.flop / ((ms_a + ms_q) * 1e-3) / 1e12, 2),
            "expcast_attention_ms": round(ms_x, 4),
            "expcast_attention_tflops": round(w.flop / (ms_x * 1e-3) / 1e12, 2),
            "expcast_attention_peak_fraction": round(w.flop / (ms_x * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        }
        for key, kname in (("attention", "attn_fwd_fp8_kernel<true,false,false,0>"),
                           ("expcast_attention", "attn_fwd_fp8_kernel<true,true,false,0>")):
            c = counters.get(kname, {})
            result["fp8"][key + "_counters"] = {"mfma_busy": c.get("mfma_busy"),
                                                "valu_active": c.get("valu_active"),
                                                "clock_ghz": c.get("clock_GHz")} if c else None
        # the pre-pass writes V codes in the kernel's tiled layout; a boundary
        # taking token-major [B,H,S,D] codes would add this pass per call
        v8_tokens = binding.vdit_attn_v8_from_tiles(z["v8"], w.S)
        v8_tiles = torch.empty_like(z["v8"])
        ms_r = time_launches(lambda: binding.vdit_attn_v8_to_tiles(v8_tokens, out=v8_tiles),
                             args.steps, args.warmup)
        relayout_bytes = w.B * w.H * w.S * w.D + v8_tiles.numel()
        result["fp8"].update({
            "v8_to_tiles_ms": round(ms_r, 4),
            "v8_to_tiles_gbs": round(relayout_bytes / (ms_r * 1e-3) / 1e9, 1),
            "v8_to_tiles_share_of_attention": round(ms_r / ms_a, 4),
        })
        del v8_tokens, v8_tiles
        log("[bench] fp8 block-causal and block-sparse attention (same chunk and map as bf16)")
        for name, kw, flop in (("block_causal", {"chunk": chunk}, causal_flop),
                               ("block_sparse", {"block_mask": mask_dev}, sparse_flop)):
            ms_m = time_launches(lambda: binding.vdit_attn_fwd_fp8(z, scale=scale, o=o8, **kw),
                                 args.steps, args.warmup)
            ms_mx = time_launches(lambda: binding.vdit_attn_fwd_fp8(z, scale=scale, o=o8, expcast=True, **kw),
                                  args.steps, args.warmup)
            result["fp8"].update({
                f"{name}_attention_ms": round(ms_m, 4),
                f"{name}_attention_tflops": round(flop / (ms_m * 1e-3) / 1e12, 2),
                f"{name}_expcast_attention_ms": round(ms_mx, 4),
                f"{name}_expcast_attention_tflops": round(flop / (ms_mx * 1e-3) / 1e12, 2),
            })
        log("[bench] fp8 with V-Smooth block means (128-token blocks)")
        zv = binding.vdit_attn_quant_fp8(q, k, v, v_mean="block")
        ms_vq = time_launches(lambda: binding.vdit_attn_quant_fp8(q, k, v, out=zv), args.steps, args.warmup)
        ms_va = time_launches(lambda: binding.vdit_attn_fwd_fp8(zv, scale=scale, o=o8), args.steps, args.warmup)
        ms_vx = time_launches(lambda: binding.vdit_attn_fwd_fp8(zv, scale=scale, o=o8, expcast=True),
                              args.steps, args.warmup)
        result["fp8"].update({
            "vsmooth_prepass_ms": round(ms_vq, 4),
            "vsmooth_attention_ms": round(ms_va, 4),
            "vsmooth_attention_tflops": round(w.flop / (ms_va * 1e-3) / 1e12, 2),
            "vsmooth_expcast_attention_ms": round(ms_vx, 4),
            "vsmooth_expcast_attention_tflops": round(w.flop / (ms_vx * 1e-3) / 1e12, 2),
        })
        log("[bench] V-Smooth Group (k-means of V, 128-token clusters on average, 4 rounds)")
        ms_g = time_launches(lambda: binding.vdit_vsmooth_group(v), max(1, args.steps // 2), 1)
        perm, _, _ = binding.vdit_vsmooth_group(v)
        kp = torch.empty_like(k)
        ms_p = time_launches(lambda: binding.vdit_permute_tokens(k, perm, out=kp), args.steps, args.warmup)
        result["fp8"].update({
            "vsmooth_group_ms": round(ms_g, 4),
            "permute_tokens_ms": round(ms_p, 4),
        })
        del z, zv, o8, kp, perm
    del o, mask_dev, q, k, v
    torch.cuda.synchronize()

    if not args.no_configs and headline:
        result["configs"] = other_configs(args.steps, args.warmup, not args.no_fp8)

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, scale, args.cpu_seconds, head0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
