"""Host-side pieces of bench.py (no GPU): the sysfs clock and power readers,
the committed counter and traffic summaries it reads by kernel-source hash,
and the accuracy check its CPU-baseline leg applies to the timed output."""

import math

import numpy as np
import pytest

import bench
from video_diffusion_transformer_vdit_amd import inputs


def test_read_sclk_takes_the_starred_level(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("0: 500Mhz\n1: 1787Mhz *\n2: 2400Mhz\n")
    assert bench.read_sclk(str(p)) == 1787.0
    p.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk(str(p)) is None
    assert bench.read_sclk(str(tmp_path / "missing")) is None


def test_read_power_converts_microwatts(tmp_path):
    p = tmp_path / "power1_input"
    p.write_text("1329000000\n")
    assert bench.read_power(str(p)) == 1329.0
    p.write_text("0\n")
    assert bench.read_power(str(p)) is None
    p.write_text("n/a\n")
    assert bench.read_power(str(p)) is None
    assert bench.read_power(str(tmp_path / "missing")) is None


def test_committed_counters_match_the_kernel_sources():
    """The counter summary under profiles/ was taken on the kernels as they
    stand: every attention kernel is reported, with fractions in [0, 1]."""
    c = bench.measured_counters()
    assert any(k.startswith("attn_fwd_bf16_kernel") for k in c), sorted(c)
    assert any(k.startswith("attn_fwd_fp8_kernel") for k in c), sorted(c)
    for name, row in c.items():
        assert 0.0 < row["mfma_busy"] <= 1.0, name
        assert 0.0 < row["valu_active"] <= 1.0, name
        assert 1.0 < row["clock_GHz"] < 2.5, name
    t = bench.measured_traffic()
    assert t is not None and t > 4 * 40 * 75_600 * 128 * 2


def test_counters_are_dropped_for_a_changed_source(monkeypatch):
    monkeypatch.setattr(bench, "source_sha256", lambda path=bench.KERNEL_SOURCE: "0" * 64)
    assert bench.measured_counters() == {}
    assert bench.measured_traffic() is None


def _bf16_of(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_cpu_baseline_check_of_the_timed_output():
    """The CPU leg compares the rows it computes with the timed output: an
    output equal to the oracle rounded to bf16 scores zero error, and one
    element moved by one bf16 step is counted with its size in steps."""
    from oracle import attention as oa
    w = inputs.get_workload("tiny-3x16x16")
    q, k, v = inputs.make_inputs(w)
    scale = float(np.float32(1 / math.sqrt(w.D)))
    ref = oa.attention_head(q[0, 0], k[0, 0], v[0, 0], scale)
    head0 = _bf16_of(ref)
    r = bench.cpu_baseline(w, q, k, v, scale, 0.0, head0)
    assert r["check_rows"] >= 256
    assert r["max_abs_vs_oracle"] == 0.0 and r["mean_rel_vs_oracle"] == 0.0
    assert r["elements_over_1e-2"] == 0
    # move one element of row 3 by 0.05
    bad = head0.copy()
    moved = np.float32(inputs.bf16_bits_to_f32(head0[3:4, 7])[0] + 0.05)
    bad[3, 7] = _bf16_of([moved])[0]
    r = bench.cpu_baseline(w, q, k, v, scale, 0.0, bad)
    assert r["elements_over_1e-2"] == 1
    assert 0.04 < r["max_abs_vs_oracle"] < 0.06
    assert r["over_1e-2_max_bf16_steps"] > 1.0


@pytest.mark.parametrize("gpus", [2, 8])
def test_more_than_one_gpu_is_refused(gpus, monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", str(gpus)])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
