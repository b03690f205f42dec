"""Benchmark: attention TFLOP/s and fraction of the MI355X bf16 MFMA peak on one GPU.

Headline (`value`): causal bf16 forward, B=1 H=32 N=32768 d=128 (the 32K x 128 case),
one step = one fa_fwd call over inputs already resident in HBM. The other workloads
(small dense head, 7B-like causal layer in (B,N,H,d), 128K block-sparse, causal
backward; grouped K/V heads, packed variable-length sequences, block-sparse backward,
fp8 inputs) are timed in the same run and reported under "workloads".

FLOP conventions: forward 4*B*H*N^2*d, halved for causal; backward 2.5x the forward
(five matrix products against two); block-sparse: listed 128x128 tiles x 4*128*128*d
("counting only unmasked tiles"), with the element-exact count alongside.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads all|headline|KEY,...]
                       [--no-cpu-baseline]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

N_CU = 256
BF16_FLOP_PER_CU_CLK = 4096
SPEC_CLOCK_GHZ = 2.4
PEAK_BF16_TFLOPS = N_CU * BF16_FLOP_PER_CU_CLK * SPEC_CLOCK_GHZ / 1e3   # 2516.6 (AMD quotes 2.5 PFLOP/s dense)
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS                                  # 5033.2 (AMD quotes 5.0 dense)
# The fp8 forward runs Q.K^T (half the FLOPs) on the fp8 matrix cores and P.V in bf16: at
# both peaks the time is F/2 / fp8 + F/2 / bf16, so its ceiling is the harmonic mean.
PEAK_FP8_MIXED_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)   # 3355.5
HBM_PEAK_GBS = 8000.0
CPU_WORKERS_MAX = 16          # the host-core share of a one-GPU job
HEADLINE = "causal_h32_n32k"


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_fwd_causal_h32_n32k.md")
COUNTER_PROFILE = os.path.join(ROOT, "profiles", "mfma_lds_counters_fwd_causal_h32_n32k.md")
FWD_SOURCE = os.path.join(ROOT, "exact_block_sparse_amd", "csrc", "fa_fwd.hip")


def _profile_json(path):
    """The JSON block of a committed rocprofv3 summary, or None when it is missing or the
    headline kernel's source has changed since the counters were taken."""
    import hashlib
    try:
        text = open(path).read()
        d = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        cur = hashlib.sha256(open(FWD_SOURCE, "rb").read()).hexdigest()[:16]
    except (OSError, IndexError, ValueError):
        return None
    return d if d.get("source_sha256_16") == cur else None


def measured_traffic():
    """HBM bytes per launch of the headline kernel (FETCH_SIZE + WRITE_SIZE, copy-calibrated)."""
    d = _profile_json(TRAFFIC_PROFILE)
    return int(d["traffic_bytes"]) if d else None


class LiveClock:
    """Shader clock and socket power read from the GPU's metrics table (amdsmi: the mean of the
    8 XCDs' current GFX clocks, MHz; socket power, W) every 20 ms on a host thread. The table
    trails the load by a fraction of a second, so the readings are taken over a window of
    back-to-back headline calls right after the timed ones, and the window's first second is
    left out. Reading the table touches no GPU work; where amdsmi is missing or refuses, the
    figures are None."""

    def __init__(self):
        self.samples, self._stop, self._th, self._h = [], None, None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:
            self._h = None

    def _loop(self):
        import time
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
                if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
                    clks = [m["current_gfxclk"]]
                pw = m.get("current_socket_power")
                if clks:
                    self.samples.append((time.perf_counter(), sum(clks) / len(clks),
                                         pw if isinstance(pw, (int, float)) else None))
            except Exception:
                return
            time.sleep(0.02)

    def __enter__(self):
        import threading
        import time
        self.t0 = time.perf_counter()
        if self._h is not None:
            self._stop = threading.Event()
            self._th = threading.Thread(target=self._loop, daemon=True)
            self._th.start()
        return self

    def __exit__(self, *exc):
        if self._th is not None:
            self._stop.set()
            self._th.join()
        return False

    def summary(self, skip_s: float = 1.0):
        kept = [(c, w) for ts, c, w in self.samples if ts >= self.t0 + skip_s]
        if not kept:
            return None, None
        ghz = sum(c for c, _ in kept) / len(kept) / 1e3
        pws = [w for _, w in kept if w is not None]
        return round(ghz, 4), (round(sum(pws) / len(pws), 1) if pws else None)


def measured_clock_ghz():
    """Shader clock of the headline kernel under load: GRBM_GUI_ACTIVE cycles (summed over
    the 8 XCDs, so divided by 8) per second of dispatch, from the committed counter run."""
    d = _profile_json(COUNTER_PROFILE)
    return float(d["clock_ghz"]) if d and d.get("clock_ghz") else None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def fwd_flops(w) -> float:
    """4*H*n^2*d per sequence of n rows (halved for causal), summed over the batch."""
    sq = sum(n * n for n in w.seqlens) if w.packed else w.B * w.N * w.N
    f = 4.0 * w.H * sq * w.d
    return f / 2 if w.causal else f


def sparse_flops(w, offsets, indices) -> tuple[float, float]:
    """(tile-count FLOPs, element-exact FLOPs) for the block-sparse forward."""
    import numpy as np
    blk = w.sparse["block"]
    tiles = int(offsets[-1])
    by_tiles = tiles * 4.0 * blk * blk * w.d * w.B * w.H
    nb = len(offsets) - 1
    elems = 0
    for q in range(nb):
        ks = indices[offsets[q]:offsets[q + 1]]
        full = int(np.sum(ks < q)) if w.causal else len(ks)
        elems += full * blk * blk
        if w.causal and q in ks:
            elems += blk * (blk + 1) // 2
    exact = elems * 4.0 * w.d * w.B * w.H
    return by_tiles, exact


def algorithmic_bytes(w, direction: str, nnz: int = 0) -> int:
    rows = w.total                              # B*N, or the packed row count
    es = 1 if w.dtype == "fp8_e4m3" else 2      # bytes per input element (O is always bf16)
    tq = rows * w.H * w.d * 2                   # one bf16 tensor with the query heads
    tk = rows * w.hkv * w.d * 2                 # one bf16 tensor with the K/V heads
    lse = rows * w.H * 4
    lists = 0 if not w.sparse else (len_off(w) + nnz) * 4
    if direction in ("bwd", "sparse_bwd"):
        # q k v o do read, dq dk dv written, lse read (+ both list forms)
        return 4 * tq + 4 * tk + lse + (2 * lists if w.sparse else 0)
    return (tq + 2 * tk) * es // 2 + tq + lse + lists   # q k v read, o written, lse written


def len_off(w) -> int:
    return (w.N + w.sparse["block"] - 1) // w.sparse["block"] + 1 if w.sparse else 0


class Timer:
    """HIP events on torch's current stream, where the library launches its kernels.

    The timed calls run back to back between two events (the mean per call is their
    distance over the number of calls), so the host's work for one call overlaps the GPU's
    work for the previous one, as in a stream of calls. A second pass with an event pair
    around every call gives the per-call median and minimum (there each call also waits
    for its own host-side preparation, which matters only for the smallest problems)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps: int, warmup: int):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        first.record()
        for _ in range(steps):
            fn()
        last.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total = first.elapsed_time(last)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            starts[i].record()
            fn()
            ends[i].record()
        torch.cuda.synchronize()
        per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
        return dict(mean_ms=total / steps, median_ms=per[len(per) // 2], min_ms=per[0], total_ms=total,
                    wall_s=wall, reps=steps)


def prepare(fa, W, torch, key, store_ds=None):
    w = W.WORKLOADS[key]
    log(f"[bench] preparing {key}: {w.describe()}")
    x = W.make_inputs(w)
    dev = {n: t.to("cuda") for n, t in x.items() if hasattr(t, "to")}
    info = dict(workload=w, x=x, dev=dev)
    # grouped heads, packed sequences and fp8 inputs go through the general entry points
    general = w.packed or w.hkv != w.H or w.dtype != "bf16"
    kw = dict(causal=w.causal, scale=w.scale)
    if w.dtype != "bf16":
        kw.update(q_descale=x["q_descale"], k_descale=x["k_descale"], v_descale=x["v_descale"])
    if w.packed:
        kw.update(cu_seqlens=torch.from_numpy(w.cu_seqlens()).to("cuda"), max_seqlen=w.N)
    if w.direction == "fwd":
        if general:
            info["fn"] = lambda: fa.attn_fwd(dev["q"], dev["k"], dev["v"], **kw)
        else:
            info["fn"] = lambda: fa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale)
        info["flops"] = fwd_flops(w)
        info["bytes"] = algorithmic_bytes(w, "fwd")
    elif w.direction == "sparse_bwd":
        nb = (w.N + w.sparse["block"] - 1) // w.sparse["block"]
        off, idx = fa.make_block_lists(nb, w.sparse["window"], w.sparse["stride"], causal=w.causal,
                                       rule=w.sparse["rule"])
        t_off, t_idx = fa.transpose_block_lists(off, idx, nb)
        lists = dict(kv_offsets=torch.from_numpy(off).to("cuda"), kv_indices=torch.from_numpy(idx).to("cuda"))
        tlists = dict(q_offsets=torch.from_numpy(t_off).to("cuda"), q_indices=torch.from_numpy(t_idx).to("cuda"))
        o, lse = fa.attn_fwd(dev["q"], dev["k"], dev["v"], **kw, **lists)
        info["fn"] = lambda: fa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], **kw, **lists, **tlists,
                                         store_ds=store_ds)
        fl, fl_exact = sparse_flops(w, off, idx)
        info["flops"], info["flops_exact"] = 2.5 * fl, 2.5 * fl_exact
        info["tiles_per_head"] = int(off[-1])
        info["bytes"] = algorithmic_bytes(w, "sparse_bwd", len(idx))
    elif w.direction == "sparse_fwd":
        nb = (w.N + w.sparse["block"] - 1) // w.sparse["block"]
        off, idx = fa.make_block_lists(nb, w.sparse["window"], w.sparse["stride"], causal=w.causal,
                                       rule=w.sparse["rule"])
        doff = torch.from_numpy(off).to("cuda")
        didx = torch.from_numpy(idx).to("cuda")
        info["fn"] = lambda: fa.sparse_fwd(dev["q"], dev["k"], dev["v"], doff, didx, causal=w.causal,
                                           scale=w.scale)
        info["flops"], info["flops_exact"] = sparse_flops(w, off, idx)
        info["tiles_per_head"] = int(off[-1])
        info["bytes"] = algorithmic_bytes(w, "sparse_fwd", len(idx))
    elif general:
        o, lse = fa.attn_fwd(dev["q"], dev["k"], dev["v"], **kw)
        info["fn"] = lambda: fa.attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], **kw, store_ds=store_ds)
        info["flops"] = 2.5 * fwd_flops(w)
        info["bytes"] = algorithmic_bytes(w, "bwd")
    else:
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale)
        info["fn"] = lambda: fa.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=w.causal,
                                    scale=w.scale, store_ds=store_ds)
        info["flops"] = 2.5 * fwd_flops(w)
        info["bytes"] = algorithmic_bytes(w, "bwd")
    return info


def summarize(info, t):
    ms = t["mean_ms"]
    tflops = info["flops"] / (ms * 1e-3) / 1e12
    out = dict(workload=info["workload"].describe(), ms_mean=round(ms, 4), ms_median=round(t["median_ms"], 4),
               ms_min=round(t["min_ms"], 4), reps=t["reps"], tflops=round(tflops, 2),
               pct_peak=round(100 * tflops / PEAK_BF16_TFLOPS, 2), flops=info["flops"],
               algorithmic_bytes=info["bytes"])
    if info["workload"].dtype == "fp8_e4m3":
        out["pct_of_mixed_fp8_bf16_peak"] = round(100 * tflops / PEAK_FP8_MIXED_TFLOPS, 2)
        out["mixed_fp8_bf16_peak"] = round(PEAK_FP8_MIXED_TFLOPS, 1)
    if "flops_exact" in info:
        out["flops_element_exact"] = info["flops_exact"]
        out["tflops_element_exact"] = round(info["flops_exact"] / (ms * 1e-3) / 1e12, 2)
        out["tiles_per_head"] = info["tiles_per_head"]
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_head(w, x):
    """Head (0, 0) of a workload's CPU inputs as fp64 numpy [1, 1, n, d] arrays (the first
    sequence when packed): the sample the CPU baseline times."""
    import torch
    out = {}
    for n in ("q", "k", "v", "do"):
        if n not in x:
            continue
        t = x[n]
        if w.packed:
            t = t[: int(w.seqlens[0]), 0:1].transpose(0, 1)[None]
        else:
            t = t[0:1, 0:1]
        t = t.to(torch.float64)
        if w.dtype == "fp8_e4m3":
            t = t * x[n + "_descale"]
        out[n] = t.contiguous().numpy()
    return out


def _sample_rows(w, n, kind, budget_flop, rng):
    """Random query rows of head (0, 0) until the oracle FLOP of the sample reach the budget;
    a row with J allowed keys costs 4*J*d FLOP forward and 6*J*d for a dQ row (scores, dP,
    dQ)."""
    import oracle
    ks = oracle.KeySets(n, w.causal, w.sparse)
    per = 6 if kind == "dq" else 4
    rows, flop = [], 0.0
    for r in rng.permutation(n):
        f = per * len(ks.keys(int(r))) * w.d
        if rows and flop + f > budget_flop:
            break
        rows.append(int(r))
        flop += f
    return sorted(rows), flop


def cpu_baseline(samples, seconds_target: float = 15.0, per_workload_seconds: float = 2.5):
    """The oracle as it stands, timed on the host cores over bounded samples of the workloads:
    whole query rows of head (0, 0) (forward rows; for a backward workload, the oracle's
    per-row dQ), spread over the sequence, one process per core (at most the 16-core share
    of a one-GPU job). The headline's sample is about `seconds_target` seconds of CPU work;
    the others about `per_workload_seconds` each. Reported as TFLOP/s over the FLOP the
    oracle performs for the sampled rows, and as rows/s."""
    import multiprocessing as mp
    import numpy as np

    cores = max(1, min(os.cpu_count() or 1, CPU_WORKERS_MAX))
    rate = 1.5e9   # rough per-core fp64 rate of the row-at-a-time oracle, to size the samples
    ctx = mp.get_context("fork")
    results = {}
    for key, (w, head) in samples.items():
        kind = "dq" if w.direction in ("bwd", "sparse_bwd") else "fwd"
        n = head["q"].shape[2]
        secs = seconds_target if key == HEADLINE else per_workload_seconds
        rows, flop = _sample_rows(w, n, kind, secs * rate * cores, np.random.default_rng(0))
        _CPU_STATE.clear()
        _CPU_STATE.update(w=w, x=head, kind=kind)
        with ctx.Pool(cores) as pool:
            t0 = time.perf_counter()
            pool.map(_cpu_rows, [rows[i::cores] for i in range(cores)])
            dt = time.perf_counter() - t0
        what = "per-row dQ of the backward" if kind == "dq" else "forward rows"
        results[key] = {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "rows": len(rows),
                        "rows_per_s": round(len(rows) / dt, 1), "seconds": round(dt, 2),
                        "sample": f"{len(rows)} random {what} of head (0,0) of {w.describe()}; "
                                  f"{flop:.3e} FLOP"}
    head = results[HEADLINE]
    return {"value": head["value"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": head["sample"] + f" in {head['seconds']} s (fp64 numpy, row at a time, one process "
                                       f"per core)",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "per_workload": results}


_CPU_STATE = {}


def _cpu_rows(rows):
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    import oracle
    w, x, kind = _CPU_STATE["w"], _CPU_STATE["x"], _CPU_STATE["kind"]
    if kind == "dq":
        oracle.backward_rows_dq(x["q"], x["k"], x["v"], x["do"], causal=w.causal, scale=w.scale, sparse=w.sparse,
                                rows=rows)
    else:
        oracle.attention_forward(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, sparse=w.sparse, rows=rows)
    return len(rows)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads", default="all",
                    help="all, headline, or a comma-separated list of workload keys (besides the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-schedule", choices=("auto", "stored", "recomputed"), default="auto",
                    help="backward: dS stored by the dK/dV pass for dQ (stored), dQ recomputing S and dP "
                         "(recomputed), or the library binding's default choice (auto)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (to scale "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 2
        src_t = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst_t = torch.empty_like(src_t)
        for _ in range(5):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 2 * n, "launches": 5}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (heads and sequence "
              "shards would be independent per GPU). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_block_sparse_amd as fa
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    timer = Timer(torch)

    head = prepare(fa, W, torch, HEADLINE)
    log(f"[bench] timing {HEADLINE}: warmup {args.warmup}, steps {args.steps}")
    t = timer.run(head["fn"], args.steps, args.warmup)
    live = LiveClock()
    with live:   # about 2.5 s of back-to-back headline calls, not timed
        end = time.perf_counter() + 2.5
        while time.perf_counter() < end:
            for _ in range(10):
                head["fn"]()
            torch.cuda.synchronize()
    live_ghz, live_w = live.summary()
    hs = summarize(head, t)
    log(f"[bench] {HEADLINE}: {hs['ms_mean']} ms, {hs['tflops']} TFLOP/s ({hs['pct_peak']}% of peak)")
    w = head["workload"]
    achieved = head["flops"] / (t["mean_ms"] * 1e-3) / 1e12
    # the CPU baseline times the oracle on head (0, 0) of the five benchmark configurations
    cpu_samples = {}
    want_cpu = not args.no_cpu_baseline
    if want_cpu:
        cpu_samples[HEADLINE] = (w, cpu_head(w, head["x"]))

    others = {}
    if args.workloads != "headline":
        keys = W.ORDER if args.workloads == "all" else [HEADLINE] + args.workloads.split(",")
        unknown = [k for k in keys if k not in W.WORKLOADS]
        if unknown:
            raise SystemExit(f"unknown workloads {unknown}; known: {W.ORDER}")
        del head["dev"]
        torch.cuda.empty_cache()
        for key in keys:
            if key == HEADLINE:
                others[key] = hs
                continue
            info = prepare(fa, W, torch, key, {"auto": None, "stored": True, "recomputed": False}[args.bwd_schedule])
            if want_cpu and key in W.BENCHMARK_CONFIGS:
                cpu_samples[key] = (info["workload"], cpu_head(info["workload"], info["x"]))
            reps = 50 if key == "dense_n512_d64" else max(20, args.steps)
            tt = timer.run(info["fn"], reps, 3)
            others[key] = summarize(info, tt)
            log(f"[bench] {key}: {others[key]['ms_mean']} ms, {others[key]['tflops']} TFLOP/s")
            del info
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: timing the oracle on host cores")
        del head["x"]
        cpu = cpu_baseline(cpu_samples)
        log(f"[bench] cpu_baseline: {cpu['value']} TFLOP/s on {cpu['cores']} cores ({cpu['cpu_model']}); "
            + ", ".join(f"{k} {v['rows_per_s']} rows/s" for k, v in cpu["per_workload"].items()))
    clock = measured_clock_ghz()

    line = {
        "metric": "attention TFLOP/s (bf16 fwd/bwd, causal & block-sparse) and % of MFMA peak on 1 GPU",
        "value": round(achieved, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["mean_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{HEADLINE}: {w.describe()}", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed, "sigma": w.sigma},
        "pct_of_peak": round(100 * achieved / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(), "algorithmic_bytes": head["bytes"],
                     "kernel": "fwd_pingpong_dma_kernel<causal>", "per_launch_flop": head["flops"],
                     "avg_launch_ms": round(t["mean_ms"], 4),
                     # the same achieved rate against the peak at the shader clock measured under
                     # this kernel's load (GRBM_GUI_ACTIVE, committed counter run), not 2.4 GHz
                     "clock_ghz_measured": clock,
                     "pct_of_measured_clock_peak": (round(100 * achieved / (N_CU * BF16_FLOP_PER_CU_CLK * clock / 1e3),
                                                          2) if clock else None),
                     # the clock and socket power read live during this run's timed headline calls
                     "clock_ghz_live": live_ghz,
                     "pct_of_live_clock_peak": (round(100 * achieved / (N_CU * BF16_FLOP_PER_CU_CLK * live_ghz / 1e3), 2)
                                                if live_ghz else None),
                     "socket_power_w_live": live_w},
        "cpu_baseline": cpu,
        "workloads": others,
        "bwd_schedule": args.bwd_schedule,
        "context": "pages' claim: FlashAttention-2 2-4x faster than cuDNN attention on one A100 beyond 8K "
                   "tokens (context only, other hardware)",
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
