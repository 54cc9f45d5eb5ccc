"""Host-side logic (CPU only): the input recipe, the product/oracle separation, the
benchmark's single-GPU contract."""

import ast
import os
import subprocess
import sys

import numpy as np
import torch

from long_context_prefix_amd.workloads import WORKLOADS, make_inputs, ragged_kv_len, sample_rows

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_prefix_amd")


def test_pads_sit_exactly_past_each_prefix():
    lens = [5, 0, 12]
    q, k, v, kv = make_inputs(3, 2, 4, 12, 64, lens, "bf16", 1.0, seed=7)
    assert kv.tolist() == lens and kv.dtype == torch.int32
    for b, n in enumerate(lens):
        for t in (k, v):
            pad = t[b, :, n:].float()
            assert torch.all(pad.abs() == 9984.0), "pads are +-1e4 rounded to bf16"
            if n:
                assert torch.all(t[b, :, :n].float().abs() < 100.0)
    # NaN pads for the invariance tests
    _, k2, v2, _ = make_inputs(3, 2, 4, 12, 64, lens, "bf16", 1.0, seed=7, pad=float("nan"))
    assert torch.isnan(k2[0, :, 5:].float()).all() and not torch.isnan(k2[0, :, :5].float()).any()
    # the valid part does not depend on the pad value
    assert torch.equal(k2[0, :, :5], k[0, :, :5]) and torch.equal(v2[2, :, :12], v[2, :, :12])


def test_inputs_are_reproducible_and_per_sequence_draws_stand_alone():
    a = make_inputs(2, 1, 3, 8, 64, [8, 3], "f32", 0.5, seed=11)
    b = make_inputs(2, 1, 3, 8, 64, [8, 3], "f32", 0.5, seed=11)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    full = make_inputs(3, 1, 2, 8, 64, [8, 4, 2], "bf16", 1.0, seed=3, per_sequence=True)
    one = make_inputs(1, 1, 2, 8, 64, [4], "bf16", 1.0, seed=3 + 1 + 1, per_sequence=False)
    # element b of a per-sequence draw is the plain draw seeded seed + 1 + b
    assert torch.equal(full[0][1:2], one[0]) and torch.equal(full[1][1:2], one[1])


def test_ragged_lengths_force_both_ends():
    lens = ragged_kv_len(1003, 8, 32768)
    assert lens[0] == 1 and lens[-1] == 32768 and lens.min() >= 1 and lens.max() <= 32768
    assert np.array_equal(lens, WORKLOADS["ragged_32k"].lens())


def test_sampled_rows_hold_both_ends():
    rows = sample_rows(5, 1000, 17, 4)
    assert rows.shape == (4, 17)
    assert np.all(rows[:, 0] == 0) and np.all(rows[:, -1] == 999)
    assert all(len(set(r.tolist())) == 17 for r in rows)


def test_product_never_imports_the_oracle():
    """Only tests, the smoke check and the benchmark's CPU-baseline leg may use the oracle."""
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n == "oracle" or n.startswith("oracle.") for n in names), f"{f} imports the oracle"
    for f in os.listdir(os.path.join(PKG, "csrc")):
        assert "oracle" not in open(os.path.join(PKG, "csrc", f)).read(), f


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_bench_parity_gate():
    """A timed output outside the bf16 tolerance voids the bench line (value null, exit 1)."""
    sys.path.insert(0, ROOT)
    import bench

    ref = np.ones((2, 3))
    lse = np.array([1.0, -np.inf])
    good = bench.parity_stats(np, ref + 1e-3, lse, ref, lse)
    assert bench.parity_failures(good) == []
    assert len(bench.parity_failures(bench.parity_stats(np, ref + 3e-2, lse, ref, lse))) == 2  # max-abs and rel-L2
    assert len(bench.parity_failures(bench.parity_stats(np, ref, lse + np.array([2e-3, 0.0]), ref, lse))) == 1
    nan_out = ref.copy()
    nan_out[0, 0] = np.nan
    assert bench.parity_failures(bench.parity_stats(np, nan_out, lse, ref, lse))  # NaN never passes
    assert bench.parity_failures(bench.parity_stats(np, ref, np.array([1.0, 0.0]), ref, lse))  # -inf pattern


def test_bench_power_summary_uses_whole_refresh_intervals():
    """The power figures come only from firmware refreshes first seen inside the block:
    a block of 3.5 s at 1,300 W with refreshes every second, a refresh before the block
    and one after it (both at other powers) must not move the result."""
    sys.path.insert(0, ROOT)
    import bench

    t0, t1, watts = 10.0, 13.5, 1300.0
    samples = [{"t": 9.7, "ts": int(9.69e9), "E": 0.0, "accumulation_counter": 0, "ppt_residency_acc": 0, "clk": 158.0}]
    e, ticks, ppt = 50.0, 0, 0  # the refresh before the block saw an idle GPU
    for i, t in enumerate((10.3, 11.3, 12.3, 13.3)):
        if i:
            e += watts * 1.0
            ticks += 1000
            ppt += 750
        samples.append({"t": t, "ts": int((t - 0.001) * 1e9), "E": e, "accumulation_counter": ticks,
                        "ppt_residency_acc": ppt, "clk": 1800.0})
    samples.append({"t": 14.3, "ts": int(14.299e9), "E": e + 300.0, "accumulation_counter": ticks + 1000,
                    "ppt_residency_acc": ppt, "clk": 158.0})
    r = bench.power_summary(samples, t0, t1, 70, 1400.0)
    assert r["refresh_intervals"] == 3
    assert abs(r["mean_power_w"] - watts) < 0.5
    assert abs(r["joules_per_launch"] - watts * 3.5 / 70) < 1e-3
    assert r["power_limited_share"] == 0.75
    assert r["gfxclk_mhz_mean"] == 1800.0
    # fewer than two refreshes inside: no power figure rather than a wrong one
    r = bench.power_summary(samples[:2] + samples[-1:], t0, t1, 70, 1400.0)
    assert r["refresh_intervals"] == 0 and "mean_power_w" not in r
