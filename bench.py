"""Benchmark of the fused MoE forward on one MI355X.

One step = one call of the whole forward (routing, grouped gate/up GEMM with
SiLU, grouped down GEMM, combine; or the weight-streaming path for a single
decode token) on seeded synthetic inputs already resident in HBM. Inputs
follow the atrex-bench operator #009 "Input Generation" recipe on rows of its
"Shapes" table.

Timing protocol: before every timed call (and every warm-up call) a 512 MiB
buffer is read, more than the 256 MB last-level cache plus the L2s hold, so
no call finds the previous call's weights, tokens or intermediates in cache;
each call is timed on its own with HIP events on the stream it runs on; the
line reports mean, median, p10 and p90.

Prints one JSON line. The headline workload (default: the shapes-table row
T=15381, H=I=4096, E=8, top-2, the largest that fits one GPU) gives the
required top-level fields, ``roofline`` (the dominant kernel, the gate/up
GEMM, timed on its own the same way, plus the whole call's fraction of the
bound) and ``cpu_baseline`` (the CPU oracle on a bounded sample of the same
inputs, on this host's cores, extrapolated to the whole call; plus 1-core
figures). ``configs`` holds a record of the same kind for each of the other
workloads (tiny, prefill, decode, wide).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

import moe_topk_ids_amd as moe
from moe_topk_ids_amd.inputs import SHAPES, SHAPES_TABLE, bf16_bits, make_fp8_weights, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))
METRIC = "fused-MoE bf16 TFLOP/s and µs/call per shape; % of MFMA/HBM roofline at 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
FLUSH_BYTES = 512 * 2 ** 20
# atrex-bench #009 shapes table, T_Prod of the production kernel on its "XPU-A"
# hardware (another machine: context only), in microseconds.
PAGE_T_PROD_US = {"prefill": 1600.0, "decode": 116.9, "wide": 5690.0, "large": 18640.0}
PATHS = {
    "default": 0,
    "slot": moe.FLAG_FORCE_GROUPED,
    "atomic": moe.FLAG_FORCE_GROUPED | moe.FLAG_ATOMIC_COMBINE,
    "decode": moe.FLAG_FORCE_DECODE,
    "small_batch": moe.FLAG_FORCE_SMALL_BATCH,
    # the default path with the expert outputs kept fp32 / rounded to bf16
    "fp32_y": moe.FLAG_FP32_Y,
    "bf16_y": moe.FLAG_BF16_Y,
    # the default path with the down projection in one launch (no column-half tail)
    "no_tail": moe.FLAG_NO_TAIL_SPLIT,
}
PATH_NAMES = {moe.PATH_GROUPED: "grouped", moe.PATH_DECODE: "decode",
              moe.PATH_SMALL_BATCH: "small_batch"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(HERE, "moe_topk_ids_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source (else None)."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))[f"{kernel}:{workload}"]
    except (KeyError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(*rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


class Flusher:
    """Reads a 512 MiB device buffer: afterwards neither the L2s nor the
    last-level cache hold anything a timed call reads."""

    def __init__(self, enabled: bool):
        self.enabled = enabled
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") \
            if enabled else None
        self.sink = torch.empty(1, dtype=torch.float32, device="cuda")

    def __call__(self):
        if self.enabled:
            torch.sum(self.buf, dim=0, keepdim=True, out=self.sink)


def time_calls(fn, steps: int, warmup: int, flush: Flusher) -> np.ndarray:
    """Microseconds of each of `steps` calls of fn, each after a flush, each
    bracketed by its own pair of HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        flush()
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        flush()
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])


def summary(us: np.ndarray) -> dict:
    return {"mean": float(us.mean()), "median": float(np.median(us)),
            "p10": float(np.percentile(us, 10)), "p90": float(np.percentile(us, 90)),
            "min": float(us.min()), "max": float(us.max()), "n": int(us.size)}


def forward_caller(dev, out, flags, q, block):
    """A step function calling the C ABI with its arguments marshalled once
    (the binding checks every tensor on each call, about 15 us of host time,
    which would hide the GPU time of the small-T paths). One call through the
    Python binding first checks shapes and dtypes."""
    lib = moe.load_library()
    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    T, H = dev["hidden_states"].shape
    K = dev["topk_ids"].shape[1]
    fl = ctypes.c_uint32(flags)
    if q is not None:
        E, I2, _ = q["w1q"].shape
        moe.moe_forward_fp8(dev["hidden_states"], q["w1q"], q["w1s"], q["w2q"], q["w2s"], block,
                            dev["topk_weights"], dev["topk_ids"], out=out, flags=flags)
        args = (P(dev["hidden_states"]), P(q["w1q"]), P(q["w1s"]), P(q["w2q"]), P(q["w2s"]),
                block, P(dev["topk_weights"]), P(dev["topk_ids"]), T, H, I2 // 2, E, K,
                moe.ACT_SILU, ctypes.c_float(1.702), ctypes.c_float(7.0), None, None, P(out), fl,
                None, 0, cs)
        call = lib.moe_forward_fp8
    else:
        E, I2, _ = dev["w1"].shape
        moe.moe_forward(dev["hidden_states"], dev["w1"], dev["w2"], dev["topk_weights"],
                        dev["topk_ids"], out=out, flags=flags)
        args = (P(dev["hidden_states"]), P(dev["w1"]), P(dev["w2"]), P(dev["topk_weights"]),
                P(dev["topk_ids"]), T, H, I2 // 2, E, K, P(out), fl, None, 0, cs)
        call = lib.moe_forward_ex

    def step(_i):
        rc = call(*args)
        if rc != moe.MOE_OK:
            raise moe.MoeError(rc, lib.moe_last_error().decode())
    return step


def bench_workload(name: str, args, flush: Flusher):
    """Times the forward on one workload and its dominant kernel; returns
    (record, CPU inputs)."""
    s = SHAPES[name]
    flags = PATHS[args.path]
    fp8 = args.weights == "fp8"
    block = 256 if s.I % 256 == 0 else 128
    log(f"[bench] {name}: T={s.T} H={s.H} I={s.I} E={s.E} K={s.K}: generating inputs")
    d = make_inputs(s.T, s.H, s.I, s.E, s.K, seed=0)
    dev = {k: v.cuda() for k, v in d.items() if k != "router_logits"}
    q = None
    if fp8:
        qc = make_fp8_weights(d, block)
        q = {k: qc[k].cuda() for k in ("w1q", "w1s", "w2q", "w2s")}
        flags |= moe.FLAG_FP8_WEIGHTS
        del dev["w1"], dev["w2"]
    out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    step = forward_caller(dev, out, flags, q, block)
    t0 = time.perf_counter()
    us = time_calls(step, args.steps, args.warmup, flush)
    wall_s = time.perf_counter() - t0
    st = summary(us)
    path = PATH_NAMES[moe.moe_path(s.T, s.H, s.I, s.E, s.K, flags)]
    touched = int(len(np.unique(d["topk_ids"].numpy())))
    wbytes = 1 if fp8 else 2
    scale_bytes = touched * 3 * s.H * (s.I // block) * 4 if fp8 else 0
    alg_bytes = (touched * 3 * s.H * s.I * wbytes + scale_bytes + s.T * s.H * 2 + s.T * s.H * 4
                 + s.T * s.K * 8)
    flop = float(s.flop)
    mfma_bound = flop / (PEAK_BF16_TFLOPS * 1e12) >= alg_bytes / (PEAK_HBM_GBS * 1e9)
    log(f"[bench] {name}: path {path}, {st['median']:.1f} us/call median "
        f"(p10 {st['p10']:.1f}, p90 {st['p90']:.1f}, mean {st['mean']:.1f})")

    # ---- the dominant kernel, timed on its own (same flush protocol) ----
    if path == "grouped":
        M = moe.moe_m_tile(s.T, s.H, s.I, s.E, s.K)
        r = moe.moe_route(dev["topk_ids"], s.E, M)
        act = torch.empty((r["capacity"], s.I), dtype=torch.bfloat16, device="cuda")
        if fp8 and moe.moe_fp8_widens_in_gemm(s.T, s.H, s.I, s.E, s.K, block):
            kernel = "grouped_gemm_gate_up_silu_fp8"

            def gemm1(_i):
                moe.moe_gemm1_silu_fp8(dev["hidden_states"], q["w1q"], q["w1s"], block, r, s.K,
                                       M, act=act)
            w1_for = None
        else:
            # with FP8 weights widened first, the forward's GEMM1 is the bf16 one
            w1_for = d["w1"].cuda() if fp8 else dev["w1"]
            kernel = "grouped_gemm_gate_up_silu"

            def gemm1(_i):
                moe.moe_gemm1_silu(dev["hidden_states"], w1_for, r, s.K, M, act=act)
        kus = time_calls(gemm1, args.steps, min(args.warmup, 3), flush)
        ks = summary(kus)
        alg_flop = 4.0 * s.T * s.K * s.H * s.I
        achieved = alg_flop / (ks["mean"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": kernel, "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic_for(kernel, name), "algorithmic_flop": alg_flop,
                "avg_launch_us": ks["mean"], "launch_us": ks, "m_tile": M}
        log(f"[bench] {name}: {kernel} {ks['mean']:.1f} us/launch mean "
            f"({ks['median']:.1f} median), {achieved:.1f} TFLOP/s")
        del act, r, w1_for
    else:
        # the streaming paths: the whole call is the weight stream
        kernel = {"decode": "decode_path", "small_batch": "small_batch_path"}[path]
        kernel += "_fp8" if fp8 else ""
        achieved = alg_bytes / (st["mean"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": kernel + " (whole call)", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": traffic_for(kernel, name), "algorithmic_bytes": alg_bytes,
                "avg_launch_us": st["mean"], "launch_us": st}
    if mfma_bound:
        roof["call_frac"] = flop / (st["mean"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
        roof["call_bound"] = "mfma"
        roof["call_roofline_us"] = flop / (PEAK_BF16_TFLOPS * 1e6)
    else:
        roof["call_frac"] = alg_bytes / (st["mean"] * 1e-6) / 1e9 / PEAK_HBM_GBS
        roof["call_bound"] = "hbm"
        roof["call_roofline_us"] = alg_bytes / (PEAK_HBM_GBS * 1e3)
    rec = {
        "workload": f"{name}: T={s.T} H={s.H} I={s.I} E={s.E} top_k={s.K}",
        "path": path,
        "y_bf16": moe.moe_y_bf16(s.T, s.H, s.I, s.E, s.K, flags),
        "us_per_call": st,
        "tflops": flop / st["mean"] / 1e6,
        "algorithmic_gbs": alg_bytes / st["mean"] / 1e3,
        "algorithmic_flop": flop,
        "algorithmic_bytes": alg_bytes,
        "experts_touched": touched,
        "roofline": roof,
        "page_t_prod_us_xpu_a": PAGE_T_PROD_US.get(name),
        "timed_wall_s_incl_flush": wall_s,
    }
    del dev, out, q
    torch.cuda.empty_cache()
    return rec, d


def cpu_baseline(headline: str, d: dict, budget_s: float) -> dict:
    """The oracle as it stands on this host: a leading-token sample of the
    headline workload (about budget_s of work) on every core it uses, scaled
    to the whole call; plus 1-core figures on tiny, decode and a prefill
    sample."""
    import oracle

    s = SHAPES[headline]
    threads = oracle.omp_threads()

    def run(dd, n):
        x = bf16_bits(dd["hidden_states"][:n])
        t0 = time.perf_counter()
        oracle.moe_forward(x, bf16_bits(dd["w1"]), bf16_bits(dd["w2"]),
                           dd["topk_weights"][:n].numpy(), dd["topk_ids"][:n].numpy())
        return time.perf_counter() - t0

    per_tok = run(d, min(s.T, 8)) / min(s.T, 8)
    n = int(min(s.T, max(8, budget_s / max(per_tok, 1e-9))))
    dt = run(d, n)
    flop = 6.0 * n * s.K * s.H * s.I
    res = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": (f"first {n} of {s.T} tokens of the {headline} inputs, fp32 C oracle, "
                      f"{dt:.2f} s on {threads} threads"),
           "us_per_call_extrapolated": dt / n * s.T * 1e6,
           "extrapolated": n < s.T}
    one = {}
    oracle.set_omp_threads(1)
    try:
        for name, cap_s in (("tiny", None), ("decode", None), ("prefill", 2.0)):
            w = SHAPES[name]
            dd = make_inputs(w.T, w.H, w.I, w.E, w.K, seed=0)
            m = w.T
            if cap_s is not None:
                pt = run(dd, 4) / 4
                m = int(min(w.T, max(4, cap_s / pt)))
            t = run(dd, m)
            one[name] = {"tokens": m, "of": w.T, "s": t,
                         "us_per_call_extrapolated": t / m * w.T * 1e6,
                         "gflops": 6.0 * m * w.K * w.H * w.I / t / 1e9}
            del dd
    finally:
        oracle.set_omp_threads(threads)
    res["one_core"] = one
    return res


def bench_router(args, s):
    """The router (moe_topk_softmax) alone on the workload's router logits."""
    d = make_inputs(s.T, 128, 128, s.E, s.K, seed=0)  # only the logits are used
    logits = d["router_logits"].cuda()
    w = torch.empty((s.T, s.K), dtype=torch.float32, device="cuda")
    ids = torch.empty((s.T, s.K), dtype=torch.int32, device="cuda")
    flush = Flusher(not args.no_flush)
    us = time_calls(lambda _i: moe.moe_topk_softmax(logits, s.K, topk_weights=w, topk_ids=ids),
                    args.steps, args.warmup, flush)
    st = summary(us)
    nbytes = s.T * s.E * 4 + s.T * s.K * 8
    achieved = nbytes / st["mean"] / 1e3
    print(json.dumps({
        "metric": "router softmax->top-k->renormalise GB/s and µs/call", "value": achieved,
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": st["mean"] / 1e3, "us_per_call": st,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded fp32 N(0,1) router logits)",
        "config": {"workload": f"{s.name} router: T={s.T} E={s.E} top_k={s.K}", "T": s.T,
                   "E": s.E, "top_k": s.K},
        "roofline": {"bound": "hbm", "kernel": "topk_softmax_kernel", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "algorithmic_bytes": nbytes, "avg_launch_us": st["mean"], "traffic": None},
    }), flush=True)


def _time_rows(rows, H, I, E, K, flags, steps, flush):
    """us per call (median over `steps` flushed calls) of leading-token
    slices of one input set."""
    T_max = max(rows)
    d = make_inputs(T_max, H, I, E, K, seed=0)
    dev = {k: v.cuda() for k, v in d.items() if k != "router_logits"}
    res = {}
    for T in rows:
        sub = {k: (v[:T].contiguous() if k in ("hidden_states", "topk_weights", "topk_ids")
                   else v) for k, v in dev.items()}
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        for name, fl in flags.items():
            step = forward_caller(sub, out, fl, None, 0)
            res[(T, name)] = summary(time_calls(step, steps(T), 3, flush))["median"]
        del out
    del dev
    torch.cuda.empty_cache()
    return res


def bench_table(args):
    """Every row of the shapes table: us/call and TFLOP/s next to the page's
    T_SOL and T_Prod (measured there on its "XPU-A" hardware)."""
    flush = Flusher(not args.no_flush)
    groups = {}
    for row in SHAPES_TABLE:
        groups.setdefault(row[1:5], []).append(row)
    results = []
    for (H, I, E, K), rows in groups.items():
        log(f"[table] H={H} I={I} E={E} K={K}")
        steps = lambda T: int(max(5, min(50, 3e5 / max(6.0 * T * K * H * I / 5e14 * 1e6, 20.0))))
        us = _time_rows([r[0] for r in rows], H, I, E, K, {"default": PATHS[args.path]}, steps,
                        flush)
        for (T, _, _, _, _, t_sol, t_prod) in rows:
            u = us[(T, "default")]
            flop = 6.0 * T * K * H * I
            fl = PATHS[args.path]
            rec = {"T": T, "H": H, "I": I, "E": E, "top_k": K, "us_per_call": u,
                   "tflops": flop / u / 1e6, "path": PATH_NAMES[moe.moe_path(T, H, I, E, K, fl)],
                   "y_bf16": moe.moe_y_bf16(T, H, I, E, K, fl),
                   "page_t_sol_us": t_sol, "page_t_prod_us": t_prod,
                   "speedup_vs_page_t_prod": t_prod / u}
            results.append(rec)
            log(f"[table] T={T:6d} H={H} I={I} E={E:3d} K={K}: {u:9.1f} us {rec['tflops']:7.1f} "
                f"TFLOP/s  page T_Prod {t_prod:8.1f} us  x{t_prod / u:.2f}")
    print(json.dumps({"stage": "table", "rows": results}), flush=True)


def bench_small_t(args):
    """Crossover of the per-token and per-expert weight-streaming paths and
    the grouped path."""
    flush = Flusher(not args.no_flush)
    results = []
    for (H, I, E, K) in ((2048, 768, 128, 8), (2048, 2048, 8, 2), (4096, 384, 128, 8),
                         (4096, 4096, 8, 2)):
        Ts = [T for T in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512)
              if T * K <= 1024]
        paths = {"decode": moe.FLAG_FORCE_DECODE, "small_batch": moe.FLAG_FORCE_SMALL_BATCH,
                 "grouped": moe.FLAG_FORCE_GROUPED}
        us = _time_rows(Ts, H, I, E, K, paths, lambda T: 20, flush)
        for T in Ts:
            row = {"T": T, "H": H, "I": I, "E": E, "top_k": K,
                   "default_path": PATH_NAMES[moe.moe_path(T, H, I, E, K)]}
            for name, fl in paths.items():
                if PATH_NAMES[moe.moe_path(T, H, I, E, K, fl)] == name:
                    row[name + "_us"] = us[(T, name)]
            results.append(row)
            log(f"[small_t] {row}")
    print(json.dumps({"stage": "small_t", "rows": results}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large", choices=list(SHAPES),
                    help="headline workload (top-level fields of the line)")
    ap.add_argument("--configs", default="tiny,prefill,decode,wide",
                    help="comma-separated other workloads measured into the line's 'configs' "
                         "('' for none)")
    ap.add_argument("--path", default="default", choices=list(PATHS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of multi-core CPU oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the 512 MiB read before each call (warm-cache numbers)")
    ap.add_argument("--weights", default="bf16", choices=["bf16", "fp8"],
                    help="expert weights: bf16, or OCP FP8 E4M3 codes with an fp32 scale per "
                         "block of 256 (128 where I is not a multiple of 256) along the "
                         "contraction axis (moe_forward_fp8)")
    ap.add_argument("--stage", default="forward",
                    choices=["forward", "router", "copy", "table", "small_t"],
                    help="forward: the fused MoE forward (default); router: softmax/top-k "
                         "alone; copy: a plain 512 MiB device copy, the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes; "
                         "table: every row of the atrex-bench #009 shapes table; small_t: "
                         "decode path vs grouped path for T = 1..512")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(token data-parallel use runs it independently per GPU on each GPU's "
              "share of the tokens).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    moe.load_library()

    if args.stage == "router":
        return bench_router(args, SHAPES[args.workload])
    if args.stage == "table":
        return bench_table(args)
    if args.stage == "small_t":
        return bench_small_t(args)
    if args.stage == "copy":
        src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"stage": "copy", "bytes_read": FLUSH_BYTES,
                          "bytes_written": FLUSH_BYTES, "launches": max(args.steps, 1)}),
              flush=True)
        return None

    flush = Flusher(not args.no_flush)
    head, d = bench_workload(args.workload, args, flush)
    others = [c for c in args.configs.split(",") if c and c != args.workload]
    configs = {}
    for c in others:
        if c not in SHAPES:
            raise SystemExit(f"unknown workload {c!r}")
        configs[c], _ = bench_workload(c, args, flush)
    s = SHAPES[args.workload]
    st = head["us_per_call"]
    result = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": st["mean"] / 1e3,
        "us_per_call": st,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (PAGE_T_PROD_US[args.workload] / st["mean"]
                        if args.workload in PAGE_T_PROD_US else None),
        "vs_baseline_note": ("the page's production time for this shapes-table row, measured "
                             "on its own 'XPU-A' hardware, over this mean time per call "
                             "(context, not a target)"),
        "dtype": "bf16 (fp8-e4m3 expert weights)" if args.weights == "fp8" else "bf16",
        "data": "synthetic (seeded, atrex-bench #009 input recipe)",
        "config": {"workload": head["workload"], "T": s.T, "H": s.H, "I": s.I, "E": s.E,
                   "top_k": s.K, "path": head["path"], "weights": args.weights,
                   "flush_before_each_call_bytes": 0 if args.no_flush else FLUSH_BYTES,
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "configs": configs,
    }
    if args.cpu_budget > 0:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(args.workload, d, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
