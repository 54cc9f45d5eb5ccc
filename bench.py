#!/usr/bin/env python3
"""Benchmark of the prefix-masked attention path on one MI355X.

A timed step is one fused prefix-masked forward (work bounds, Q tile, K/V
stream, QK^T, online softmax, PV, epilogue) over the 121k-key ICL block:
B=1, H=8, D=256, T_q=131,072 queries, n=121,000 valid keys of S=131,072 slots,
bf16 inputs, fp32 softmax.  ``value`` counts only valid keys:
FLOP = 4 * D * H * T_q * sum_b n_b.

The split-KV rows (per-chunk partials plus the LSE merge) run in the same
process at their own workload -- 160 sequences x 4 heads, D=128, 128 queries,
100,000 valid keys of 102,400, 4,096-key chunks -- and are reported in the
``splitkv`` object in GB/s of algorithmic bytes (Q + valid K + valid V + out +
lse; the fp32 partial round trip is implementation overhead, not counted).

Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  Kernel durations come from HIP events on the stream the kernels are
launched on.  The CPU baseline times the fp64 oracle on a bounded sample of
query rows of the same workload, and the same rows check parity of the timed
output.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("long_context_prefix_amd/csrc/attn_kernels.hpp", "long_context_prefix_amd/csrc/attn_api.hip"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return float(m_bytes.group(1))


def blas_vendor() -> str:
    """BLAS library numpy calls (the oracle's matrix products run there)."""
    try:
        from threadpoolctl import threadpool_info

        libs = [f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)"
                for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            return "; ".join(libs)
    except Exception:  # pragma: no cover
        pass
    try:
        import numpy as np

        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        return f"{blas.get('name')} {blas.get('version')}"
    except Exception:  # pragma: no cover
        return "unknown"


BF16_TOL = {"out_max_abs": 2e-2, "out_rel_l2": 5e-3, "lse_max_abs": 1e-3}


def parity_stats(np, got_out, got_lse, ref_out, ref_lse) -> dict:
    d = got_out - ref_out
    fin = np.isfinite(ref_lse)
    return {
        "out_max_abs": float(np.abs(d).max()),
        "out_rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref_out)),
        "lse_max_abs": float(np.abs(got_lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0,
        "finite": bool(np.isfinite(got_out).all() and np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse))),
    }


def parity_failures(p: dict) -> list:
    bad = [f"{k} {p[k]:.3e} > {t:.0e}" for k, t in BF16_TOL.items() if not p[k] <= t]
    if not p["finite"]:
        bad.append("non-finite output or -inf pattern differs")
    return bad


def time_launches(fn, steps: int, torch):
    """Run fn() `steps` times with HIP events around each call on the current stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [s.elapsed_time(e) for s, e in evs]


class GpuMeter:
    """Power, clock and power-limit residency of the GPU that torch calls device 0,
    from the amdsmi library.  The firmware refreshes its energy and residency counters
    about once a second, so `measure` runs a launch back to back for a few seconds of its
    own (outside any timed region) while a thread records each refresh, and reports
    only whole refresh intervals inside that block.  Every figure is None where the
    library, the device match or a counter is unavailable; the meter never fails the run."""

    def __init__(self, torch):
        self.torch = torch
        self.smi = self.h = None
        self.power_cap_w = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            p = torch.cuda.get_device_properties(0)
            want = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}"
            for h in amdsmi.amdsmi_get_processor_handles():
                if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(want):
                    self.smi, self.h = amdsmi, h
            if self.h is None:
                log(f"energy: no amdsmi device at {want}")
                return
            cap = amdsmi.amdsmi_get_power_cap_info(self.h).get("power_cap")
            # the library reports the cap in microwatts
            self.power_cap_w = cap / 1e6 if isinstance(cap, (int, float)) and cap > 0 else None
        except Exception as e:  # pragma: no cover - depends on the machine
            log(f"energy: amdsmi unavailable ({type(e).__name__}: {e})")
            self.smi = self.h = None

    def _sample(self):
        e = self.smi.amdsmi_get_energy_count(self.h)
        r = {"t": time.perf_counter(), "ts": e["timestamp"],
             "E": e["energy_accumulator"] * e["counter_resolution"] * 1e-6}  # resolution in uJ
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
            for k in ("accumulation_counter", "ppt_residency_acc"):
                if isinstance(m.get(k), int):
                    r[k] = m[k]
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int)]
            if clks:
                r["clk"] = sum(clks) / len(clks)
        except Exception:  # pragma: no cover
            pass
        return r

    def measure(self, fn, seconds: float = 3.5, sync_every: int = 8):
        """Run fn() (one launch each) back to back for `seconds`; returns power (W), mean
        GFX clock over the XCDs (MHz), the share of the firmware's 1 ms ticks spent held
        at the package power limit, and energy per launch (J)."""
        if self.h is None:
            return None
        import threading

        torch = self.torch
        samples, stop = [], threading.Event()

        def poll():
            last = None
            while not stop.is_set():
                try:
                    r = self._sample()
                except Exception:  # pragma: no cover
                    return
                if last is None or r["ts"] != last:
                    samples.append(r)
                    last = r["ts"]
                time.sleep(0.002)

        th = threading.Thread(target=poll, daemon=True)
        torch.cuda.synchronize()
        th.start()
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(sync_every):
                fn()
            n += sync_every
            torch.cuda.synchronize()
        t1 = time.perf_counter()
        stop.set()
        th.join(timeout=5)
        return power_summary(samples, t0, t1, n, self.power_cap_w)


def power_summary(samples, t0: float, t1: float, launches: int, power_cap_w=None):
    """Power figures of a block [t0, t1] of `launches` back-to-back launches from the
    firmware refreshes a polling thread recorded (host time t of first sight, firmware
    timestamp ts in ns, energy E in J, 1 ms tick counter, power-limit ticks, clock).
    Only refreshes first seen inside the block count, so each pair of them bounds a
    whole firmware interval of the block's own work."""
    inside = [r for r in samples if t0 + 0.01 < r["t"] <= t1]
    out = {"power_cap_w": power_cap_w, "seconds": round(t1 - t0, 3), "launches": launches,
           "refresh_intervals": max(0, len(inside) - 1)}
    if len(inside) < 2 or inside[-1]["ts"] <= inside[0]["ts"]:
        return out
    a, b = inside[0], inside[-1]
    p = (b["E"] - a["E"]) / ((b["ts"] - a["ts"]) * 1e-9)
    out["mean_power_w"] = round(p, 1)
    out["joules_per_launch"] = round(p * (t1 - t0) / launches, 4)
    if "accumulation_counter" in a and "accumulation_counter" in b and "ppt_residency_acc" in a and "ppt_residency_acc" in b:
        ticks = b["accumulation_counter"] - a["accumulation_counter"]
        if ticks > 0:
            out["power_limited_share"] = round((b["ppt_residency_acc"] - a["ppt_residency_acc"]) / ticks, 3)
    clks = [r["clk"] for r in inside[1:] if "clk" in r]
    if clks:
        out["gfxclk_mhz_mean"] = round(sum(clks) / len(clks), 1)
    return out


def fetch_scaling(torch, _lib) -> int:
    """Fused launches at B=1, H=8, D=128, Tq=128 (one query tile per head, so each valid
    key row is fetched once) over S=131072 slots whose padded rows hold +-1e4, with
    n = S, S/2 and S/4.  Under a FETCH_SIZE counter run the bytes per dispatch should
    scale with n (2 * n * D * 2 bytes of K/V per head), showing that padded slots are
    never read."""
    from long_context_prefix_amd.workloads import make_inputs

    B, H, Tq, S, D = 1, 8, 128, 131072, 128
    res = []
    for n in (S, S // 2, S // 4):
        q, k, v, kv = make_inputs(B, H, Tq, S, D, [n], "bf16", 1.0, seed=4242, device="cuda")
        out = torch.empty_like(q)
        for _ in range(3):
            _lib.attn_prefix_fwd(q, k, v, kv, 1.0 / D ** 0.5, out=out)
        torch.cuda.synchronize()
        res.append({"n": n, "valid_kv_bytes_per_launch": 2 * H * n * D * 2, "launches": 3})
        log(f"fetch scaling: n={n} done")
        del q, k, v, out
    print(json.dumps({"fetch_scaling": res, "B": B, "H": H, "T_q": Tq, "S": S, "head_dim": D}), flush=True)
    return 0


def wave_forms(torch, _lib, rounds: int, copy_calibration: bool, meter=None) -> int:
    """The ragged 32k forward (B=8, H=8, D=128) in the 32-row kernel's two forms, four
    waves per workgroup (128 rows, two workgroups per CU) and eight (256 rows, one per
    CU), launched alternately in one process so that both see the same clock.  Prints
    each form's launch times from HIP events and checks that the two outputs are the
    same bits.  Under a counter run the two forms are told apart by the wave count in
    the kernel's name."""
    from long_context_prefix_amd.workloads import WORKLOADS, make_workload

    wb = WORKLOADS["ragged_32k"]
    q, k, v, kv = make_workload(wb, device="cuda")
    flop = 4.0 * wb.D * float(wb.H) * wb.Tq * float(wb.lens().sum())
    forms = ("128", "128x8")
    outs = {f: (torch.empty_like(q), torch.empty((wb.B, wb.H, wb.Tq), dtype=torch.float32, device="cuda"))
            for f in forms}
    prev = os.environ.get("ATTN_PREFIX_FWD_ROWS")

    def launch(form):
        os.environ["ATTN_PREFIX_FWD_ROWS"] = form
        _lib.attn_prefix_fwd(q, k, v, kv, wb.scale, out=outs[form][0], lse=outs[form][1])

    times = {f: [] for f in forms}
    try:
        for f in forms:
            launch(f)
        torch.cuda.synchronize()
        for r in range(rounds):
            for f in (forms if r % 2 == 0 else forms[::-1]):
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                launch(f)
                e.record()
                times[f].append((s, e))
            log(f"wave forms: round {r + 1}/{rounds} done")
        torch.cuda.synchronize()
        # power and clock: one block of a few seconds per form, in A B B A order
        blocks = {f: [] for f in forms}
        if meter is not None and meter.h is not None:
            for f in forms + forms[::-1]:
                blocks[f].append(meter.measure(lambda: launch(f)))
                log(f"wave forms: power block of {f} done")
    finally:
        if prev is None:
            os.environ.pop("ATTN_PREFIX_FWD_ROWS", None)
        else:
            os.environ["ATTN_PREFIX_FWD_ROWS"] = prev
    same = all(torch.equal(outs[forms[0]][i], outs[forms[1]][i]) for i in range(2))
    if copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written")
    res = {}
    for f in forms:
        ms = sorted(s.elapsed_time(e) for s, e in times[f])
        med = ms[len(ms) // 2]
        res[f] = {"waves_per_workgroup": 8 if f.endswith("x8") else 4, "ms_median": round(med, 4),
                  "ms_min": round(ms[0], 4), "tflops_median": round(flop / (med * 1e-3) / 1e12, 2)}
        if blocks[f]:
            res[f]["power_blocks"] = blocks[f]
    print(json.dumps({"wave_forms": res, "workload": wb.name, "B": wb.B, "H": wb.H, "head_dim": wb.D,
                      "T_q": wb.Tq, "S": wb.S, "kv_len": [int(x) for x in wb.lens()], "launches_each": rounds,
                      "same_bits": same}), flush=True)
    return 0 if same else 1


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-splitkv", action="store_true", help="skip the split-KV workload")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward workloads")
    ap.add_argument("--no-icl16k", action="store_true", help="skip the warm / MALL-scrubbed 16k ICL leg")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing and parity sample")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="oracle query rows per head for the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference kernel for HBM counter scaling)")
    ap.add_argument("--fetch-scaling", action="store_true",
                    help="only run the fused kernel on one query tile per head over S=131072 slots with "
                         "n = S, S/2, S/4 (for HBM fetch counters: bytes read must follow n, not S)")
    ap.add_argument("--wave-forms", type=int, default=0, metavar="R",
                    help="only run the ragged 32k forward R times in each of the 32-row kernel's "
                         "four- and eight-wave forms, alternately, and compare their times and bits")
    ap.add_argument("--energy", action="store_true",
                    help="after each timed leg (and per --wave-forms form), run its launch for a few more "
                         "seconds and report power, clock and power-limit residency from amdsmi")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from long_context_prefix_amd import _lib
    from long_context_prefix_amd.workloads import WORKLOADS, make_workload, sample_rows

    _lib.load()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)
    src_hash = kernel_source_hash()
    if args.fetch_scaling:
        return fetch_scaling(torch, _lib)
    if args.wave_forms:
        return wave_forms(torch, _lib, args.wave_forms, args.copy_calibration,
                          GpuMeter(torch) if args.energy else None)

    # ------------------------------------------------------------- fused path
    w = WORKLOADS["icl_121k"]
    log(f"generating {w.name}: B={w.B} H={w.H} D={w.D} Tq={w.Tq} S={w.S} kv_len={w.lens().tolist()}")
    q, k, v, kv = make_workload(w, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device="cuda")
    lens = w.lens()
    flops = 4.0 * w.D * w.H * w.Tq * float(lens.sum())

    def fused():
        _lib.attn_prefix_fwd(q, k, v, kv, w.scale, out=out, lse=lse)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    meter = GpuMeter(torch) if args.energy else None
    log(f"timing {args.steps} fused steps")
    wall, ms = time_launches(fused, args.steps, torch)
    ms_avg = sum(ms) / len(ms)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (ms_avg * 1e-3) / 1e12
    log(f"fused: {ms_avg:.3f} ms/launch (min {min(ms):.3f}), {achieved:.1f} TFLOP/s, wall {wall:.3f} s")

    traffic = traffic_from_profile("attn_fwd_icl_121k_traffic.md", src_hash)
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
        "kernel": "attn_fwd_wide_kernel<256,false,false> (64 query rows per wave)", "avg_launch_ms": round(ms_avg, 4),
        "algorithmic_flop_per_launch": flops,
    }

    result = {
        "metric": "prefix-masked attention TFLOP/s (valid keys, bf16, d=256) and % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normals, +-1e4 in padded key slots)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "head_dim": w.D, "T_q": w.Tq, "S": w.S,
                   "kv_len": [int(x) for x in lens], "scale": w.scale, "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": roofline,
        "kernel_source_sha256_16": src_hash,
    }
    if meter:
        en = meter.measure(fused, sync_every=2)
        if en and "joules_per_launch" in en:
            en["tflop_per_joule"] = round(flops / 1e12 / en["joules_per_launch"], 3)
        result["power"] = en
        log(f"power: {en}")

    invalid = []  # parity failures of timed outputs: the line then carries no value

    # -------------------------------------------------- CPU baseline + parity
    if not args.no_cpu_baseline:
        from oracle import ref_prefix_fwd  # test infrastructure: used only for this leg

        try:
            from threadpoolctl import threadpool_info

            blas_threads = max([p.get("num_threads", 0) for p in threadpool_info()] + [0])
        except Exception:  # pragma: no cover
            blas_threads = 0
        cores = len(os.sched_getaffinity(0))
        rows = sample_rows(w.seed, w.Tq, args.cpu_rows, w.B * w.H)
        log(f"oracle on {rows.shape[1]} rows x {w.B * w.H} heads (cores={cores}, blas_threads={blas_threads})")
        idx = torch.as_tensor(rows, device="cuda").view(w.B, w.H, -1)
        q_s = torch.gather(q, 2, idx[..., None].expand(-1, -1, -1, w.D)).float().cpu().numpy()
        k_h = k[:, :, : int(lens.max())].float().cpu().numpy()
        v_h = v[:, :, : int(lens.max())].float().cpu().numpy()
        t0 = time.perf_counter()
        ro, rl = ref_prefix_fwd(q_s, k_h, v_h, lens, w.scale)
        t_cpu = time.perf_counter() - t0
        sample_flops = 4.0 * w.D * rows.size * float(lens.max())
        result["cpu_baseline"] = {
            "value": round(sample_flops / t_cpu / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads or cores),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle on {rows.shape[1]} seeded query rows per head x {w.B * w.H} heads "
                      f"against all {int(lens.max())} valid keys ({sample_flops:.3e} FLOP in {t_cpu:.2f} s)",
            "blas": blas_vendor(),
            "host_cores": cores,
            "full_config_s_extrapolated": round(t_cpu * flops / sample_flops, 1),
            "extrapolation": "extrapolated, not measured: the sample's time scaled by the full launch's FLOP "
                             f"({flops:.4e} / {sample_flops:.4e})",
        }
        go = torch.gather(out, 2, idx[..., None].expand(-1, -1, -1, w.D)).double().cpu().numpy()
        gl = torch.gather(lse, 2, idx).double().cpu().numpy()
        par = parity_stats(np, go, gl, ro, rl)
        result["parity"] = dict(rows_checked=int(rows.size), **par,
                                tolerance="max_abs <= 2e-2 and rel_l2 <= 5e-3 (bf16), lse <= 1e-3")
        log(f"parity: {result['parity']}")
        invalid += [f"{w.name}: {m}" for m in parity_failures(par)]
        del k_h, v_h

    del q, k, v, out, lse
    torch.cuda.empty_cache()

    # ------------------------------------------------------------- split-KV
    if not args.no_splitkv:
        ws = WORKLOADS["inducing_splitkv"]
        log(f"generating {ws.name}: B={ws.B} H={ws.H} D={ws.D} Tq={ws.Tq} S={ws.S} n=100000 chunk={ws.chunk}")
        q, k, v, kv = make_workload(ws, device="cuda")
        C = -(-ws.S // ws.chunk)
        po = torch.empty((ws.B, ws.H, C, ws.Tq, ws.D), dtype=torch.float32, device="cuda")
        pl = torch.empty((ws.B, ws.H, C, ws.Tq), dtype=torch.float32, device="cuda")
        out = torch.empty_like(q)
        lse = torch.empty((ws.B, ws.H, ws.Tq), dtype=torch.float32, device="cuda")
        slens = ws.lens()
        esz = 2
        alg_bytes = float(ws.B * ws.H * (2 * ws.Tq * ws.D * esz + ws.Tq * 4)) + float(2 * ws.H * ws.D * esz * slens.sum())
        part_bytes = float(po.numel() * 4 + pl.numel() * 4)

        def partial():
            _lib.attn_splitkv_partial(q, k, v, kv, ws.chunk, ws.scale, part_out=po, part_lse=pl)

        def combine():
            _lib.attn_lse_combine(po, pl, torch.bfloat16, out=out, lse=lse)

        for _ in range(args.warmup):
            partial()
            combine()
        torch.cuda.synchronize()
        steps = max(1, args.steps)
        log(f"timing {steps} split-KV steps")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        for e0, e1, e2 in evs:
            e0.record()
            partial()
            e1.record()
            combine()
            e2.record()
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        t_part = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
        t_comb = sum(b.elapsed_time(c) for _, b, c in evs) / steps
        gbs = alg_bytes / ((t_part + t_comb) * 1e-3) / 1e9
        part_gbs = (alg_bytes - float(ws.B * ws.H * (ws.Tq * ws.D * esz + ws.Tq * 4)) + part_bytes) / (t_part * 1e-3) / 1e9
        log(f"split-KV: partial {t_part:.3f} ms, combine {t_comb:.3f} ms, {gbs:.0f} GB/s algorithmic")
        en_s = None
        if meter:
            def step_s():
                partial()
                combine()
            en_s = meter.measure(step_s)
            log(f"split-KV power: {en_s}")
        result["splitkv"] = {
            "workload": ws.name, "B": ws.B, "H": ws.H, "head_dim": ws.D, "T_q": ws.Tq, "S": ws.S, "n": int(slens[0]),
            "chunk": ws.chunk, "chunks": C,
            "value": round(gbs, 1), "unit": "GB/s (algorithmic: Q + valid K/V + out + lse)",
            "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "ms_per_step": round(wall_s / steps * 1e3, 4), "partial_ms": round(t_part, 4), "combine_ms": round(t_comb, 4),
            "alg_bytes": alg_bytes, "partial_roundtrip_bytes": 2 * part_bytes,
            "tflops_valid_keys": round(4.0 * ws.D * ws.H * ws.Tq * float(slens.sum()) / ((t_part + t_comb) * 1e-3) / 1e12, 2),
            "roofline_partial_kernel": {
                "bound": "hbm", "achieved": round(part_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(part_gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic_from_profile("attn_splitkv_partial_inducing_traffic.md", src_hash),
                "bytes_counted": "Q + valid K/V + fp32 partial write",
            },
        }
        if en_s is not None:
            result["splitkv"]["power"] = en_s
        if not args.no_cpu_baseline:
            # the oracle on whole sequences of the timed output (the first and a seeded one):
            # parity of the split-KV leg, and its CPU baseline in the same unit
            from oracle import ref_lse_combine, ref_splitkv_partial

            seqs = sorted({0, int(np.random.default_rng(ws.seed + 11).integers(1, ws.B))})
            t_cpu, pars = 0.0, []
            for b in seqs:
                n = int(slens[b])
                qb = q[b:b + 1].float().cpu().numpy().astype(np.float64)
                kb = k[b:b + 1].float().cpu().numpy().astype(np.float64)
                vb = v[b:b + 1].float().cpu().numpy().astype(np.float64)
                t0 = time.perf_counter()
                rpo, rpl = ref_splitkv_partial(qb, kb, vb, [n], ws.scale, ws.chunk)
                ro, rl = ref_lse_combine(rpo, rpl, axis=2)
                t_cpu += time.perf_counter() - t0
                pars.append(parity_stats(np, out[b:b + 1].double().cpu().numpy(), lse[b:b + 1].double().cpu().numpy(),
                                         ro, rl))
            seq_bytes = alg_bytes / ws.B * len(seqs)
            par = {kk: max(p[kk] for p in pars) for kk in BF16_TOL}
            par["finite"] = all(p["finite"] for p in pars)
            result["splitkv"]["parity"] = dict(sequences_checked=seqs, heads_rows="all 4 heads x 128 rows", **par)
            result["splitkv"]["cpu_baseline"] = {
                "value": round(seq_bytes / t_cpu / 1e9, 4), "unit": "GB/s (algorithmic)", "cores": int(len(os.sched_getaffinity(0))),
                "kind": "oracle",
                "sample": f"fp64 numpy oracle (chunk partials + LSE merge) on sequences {seqs}, all heads and rows "
                          f"({t_cpu:.2f} s)",
                "full_config_s_extrapolated": round(t_cpu * ws.B / len(seqs), 1),
            }
            log(f"split-KV parity: {result['splitkv']['parity']}")
            invalid += [f"{ws.name}: {m}" for m in parity_failures(par)]
        del q, k, v, po, pl, out, lse
        torch.cuda.empty_cache()

    # ------------------------------------------------- 16k ICL, warm and cold
    # Its 134 MB of K/V fits the 256 MB MALL: time it with the cache warm, and after a
    # 1 GiB write that evicts it (the event pair brackets the kernel only).
    if not args.no_icl16k:
        wi = WORKLOADS["icl_16k"]
        log(f"generating {wi.name}: B={wi.B} H={wi.H} D={wi.D} Tq={wi.Tq} S={wi.S}")
        q, k, v, kv = make_workload(wi, device="cuda")
        out = torch.empty_like(q)
        lse = torch.empty((wi.B, wi.H, wi.Tq), dtype=torch.float32, device="cuda")
        scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        fl16 = 4.0 * wi.D * wi.H * wi.Tq * float(wi.lens().sum())

        def icl16():
            _lib.attn_prefix_fwd(q, k, v, kv, wi.scale, out=out, lse=lse)

        icl16()
        torch.cuda.synchronize()
        reps = max(5, args.steps)
        warm, cold = [], []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            icl16()
            e1.record()
            torch.cuda.synchronize()
            warm.append(e0.elapsed_time(e1))
        for _ in range(reps):
            scrub.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            icl16()
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        mw, mc = sorted(warm)[len(warm) // 2], sorted(cold)[len(cold) // 2]
        log(f"icl_16k: warm {mw:.3f} ms, after a 1 GiB scrub {mc:.3f} ms")
        result["icl_16k"] = {
            "workload": wi.name, "B": wi.B, "H": wi.H, "head_dim": wi.D, "T_q": wi.Tq, "S": wi.S,
            "warm_ms_median": round(mw, 4), "scrubbed_ms_median": round(mc, 4),
            "warm_tflops": round(fl16 / (mw * 1e-3) / 1e12, 2), "scrubbed_tflops": round(fl16 / (mc * 1e-3) / 1e12, 2),
            "pct_mfma_peak_warm": round(100 * fl16 / (mw * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        }
        del q, k, v, out, lse, scrub
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- backward
    if not args.no_backward:
        wb = WORKLOADS["ragged_32k"]
        log(f"generating {wb.name}: B={wb.B} H={wb.H} D={wb.D} Tq={wb.Tq} S={wb.S} kv_len={wb.lens().tolist()}")
        q, k, v, kv = make_workload(wb, device="cuda")
        blens = wb.lens()
        pairs = float(wb.H) * wb.Tq * float(blens.sum())
        out = torch.empty_like(q)
        lse = torch.empty((wb.B, wb.H, wb.Tq), dtype=torch.float32, device="cuda")
        g = torch.Generator(device="cpu").manual_seed(wb.seed + 77)
        dout = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to("cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)

        def fwd_b():
            _lib.attn_prefix_fwd(q, k, v, kv, wb.scale, out=out, lse=lse)

        def bwd_b():
            _lib.attn_prefix_bwd(q, k, v, kv, out, dout, lse, wb.scale, dq=dq, dk=dk, dv=dv, delta=delta)

        for _ in range(args.warmup):
            fwd_b()
            bwd_b()
        torch.cuda.synchronize()
        steps = max(1, args.steps)
        log(f"timing {steps} forward + backward steps")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e0, e1, e2 in evs:
            e0.record()
            fwd_b()
            e1.record()
            bwd_b()
            e2.record()
        torch.cuda.synchronize()
        t_f = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
        t_b = sum(b.elapsed_time(c) for _, b, c in evs) / steps
        alg_b = 10.0 * wb.D * pairs  # dV, dP, dQ, dK and the recomputed S: five products of 2 D per pair
        log(f"backward: fwd {t_f:.3f} ms, bwd {t_b:.3f} ms, {alg_b / (t_b * 1e-3) / 1e12:.1f} TFLOP/s")
        en_b = None
        if meter:
            en_b = meter.measure(bwd_b, sync_every=4)
            log(f"backward power: {en_b}")
        result["backward"] = {
            "workload": wb.name, "B": wb.B, "H": wb.H, "head_dim": wb.D, "T_q": wb.Tq, "S": wb.S,
            "kv_len": [int(x) for x in blens],
            "forward_ms": round(t_f, 4), "backward_ms": round(t_b, 4),
            "forward_tflops": round(4.0 * wb.D * pairs / (t_f * 1e-3) / 1e12, 2),
            "value": round(alg_b / (t_b * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s (algorithmic: 10 D per (query, valid key) pair and head)",
            "pct_mfma_peak": round(100 * alg_b / (t_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "executed_tflops": round(14.0 * wb.D * pairs / (t_b * 1e-3) / 1e12, 2),
            "kernels": "bwd_delta_kernel, bwd_dq_slot_kernel (S, dP, dQ), bwd_dkdv_pipe_kernel (S, dP, dV, dK)",
        }
        if en_b is not None:
            result["backward"]["power"] = en_b
        del q, k, v, out, lse, dout, dq, dk, dv, delta
        torch.cuda.empty_cache()

        # the ICL head size, D = 256, at the 16k block
        wi = WORKLOADS["icl_16k"]
        log(f"generating {wi.name} backward: B={wi.B} H={wi.H} D={wi.D} Tq={wi.Tq} S={wi.S}")
        q, k, v, kv = make_workload(wi, device="cuda")
        ilens = wi.lens()
        ipairs = float(wi.H) * wi.Tq * float(ilens.sum())
        out = torch.empty_like(q)
        lse = torch.empty((wi.B, wi.H, wi.Tq), dtype=torch.float32, device="cuda")
        g = torch.Generator(device="cpu").manual_seed(wi.seed + 77)
        dout = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to("cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)
        _lib.attn_prefix_fwd(q, k, v, kv, wi.scale, out=out, lse=lse)

        def bwd_i():
            _lib.attn_prefix_bwd(q, k, v, kv, out, dout, lse, wi.scale, dq=dq, dk=dk, dv=dv, delta=delta)

        for _ in range(args.warmup):
            bwd_i()
        torch.cuda.synchronize()
        _, ms_i = time_launches(bwd_i, steps, torch)
        t_i = sum(ms_i) / len(ms_i)
        alg_i = 10.0 * wi.D * ipairs
        log(f"backward {wi.name}: {t_i:.3f} ms, {alg_i / (t_i * 1e-3) / 1e12:.1f} TFLOP/s")
        result["backward_d256"] = {
            "workload": wi.name, "B": wi.B, "H": wi.H, "head_dim": wi.D, "T_q": wi.Tq, "S": wi.S,
            "backward_ms": round(t_i, 4), "value": round(alg_i / (t_i * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s (algorithmic: 10 D per (query, valid key) pair and head)",
            "pct_mfma_peak": round(100 * alg_i / (t_i * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "kernels": "bwd_delta_kernel, bwd_dq_slot_kernel (S, dP, dQ), bwd_dkdv_slot_kernel (S, dP, dV, dK)",
        }
        del q, k, v, out, lse, dout, dq, dk, dv, delta
        torch.cuda.empty_cache()

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written")

    if invalid:
        # a timed output that misses the oracle's tolerance voids the measurement
        result["value"] = None
        result["invalid"] = invalid
        log(f"PARITY FAILED: {invalid}")
    print(json.dumps(result), flush=True)
    return 1 if invalid else 0


if __name__ == "__main__":
    sys.exit(main())
