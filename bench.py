"""Benchmark of the fused MoE forward on one MI355X.

One step = one call of the whole forward (routing, grouped gate/up GEMM with
SiLU, grouped down GEMM, combine; or the weight-streaming path for a single
decode token) on seeded synthetic inputs already resident in HBM. Inputs
follow the atrex-bench operator #009 "Input Generation" recipe; the default
workload is its shapes-table row T=4195, H=2048, I=2048, E=8, top-2.

To keep the weights from being served out of the 256 MB last-level cache
between steps, every step uses the next of R device copies of the expert
weights (R chosen so the copies together exceed 512 MB), as consecutive MoE
layers of a model would.

Prints one JSON line (rank 0, one GPU). Besides the required fields it
carries ``roofline`` for the dominant kernel (timed on its own with HIP
events on the stream it runs on) and ``cpu_baseline`` (the CPU oracle on a
bounded sample of the same inputs, on this host's cores).
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
# atrex-bench #009 shapes table, T_Prod of the production kernel on its "XPU-A"
# hardware (another machine: context only), in microseconds.
PAGE_T_PROD_US = {"prefill": 1600.0, "decode": 116.9, "wide": 5690.0, "large": 18640.0}
PATHS = {
    "default": None,
    "slot": moe.FLAG_FORCE_GROUPED,
    "atomic": moe.FLAG_FORCE_GROUPED | moe.FLAG_ATOMIC_COMBINE,
    "decode": moe.FLAG_FORCE_DECODE,
}


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


def cpu_baseline(d: dict, s, budget_s: float):
    """The oracle as it stands on a leading sample of tokens sized to ~budget_s."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    x = bf16_bits(d["hidden_states"])
    w1, w2 = bf16_bits(d["w1"]), bf16_bits(d["w2"])
    tw, ids = d["topk_weights"].numpy(), d["topk_ids"].numpy()
    calib = min(s.T, 8)
    t0 = time.perf_counter()
    oracle.moe_forward(x[:calib], w1, w2, tw[:calib], ids[:calib])
    per_tok = (time.perf_counter() - t0) / calib
    n = int(min(s.T, max(calib, budget_s / max(per_tok, 1e-9))))
    t0 = time.perf_counter()
    oracle.moe_forward(x[:n], w1, w2, tw[:n], ids[:n])
    dt = time.perf_counter() - t0
    flop = 6.0 * n * s.K * s.H * s.I
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {s.T} tokens (same inputs), fp32 C oracle, {dt:.2f} s",
            "us_per_call_extrapolated": dt / n * s.T * 1e6}


def bench_router(args, s):
    """The router (moe_topk_softmax) alone on the workload's router logits."""
    d = make_inputs(s.T, 128, 128, s.E, s.K, seed=0)  # only the logits are used
    logits = d["router_logits"].cuda()
    w = torch.empty((s.T, s.K), dtype=torch.float32, device="cuda")
    ids = torch.empty((s.T, s.K), dtype=torch.int32, device="cuda")
    for _ in range(args.warmup):
        moe.moe_topk_softmax(logits, s.K, topk_weights=w, topk_ids=ids)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        moe.moe_topk_softmax(logits, s.K, topk_weights=w, topk_ids=ids)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    us = (t1 - t0) * 1e6 / args.steps
    us_ev = ev0.elapsed_time(ev1) * 1e3 / args.steps
    nbytes = s.T * s.E * 4 + s.T * s.K * 8
    print(json.dumps({
        "metric": "router softmax->top-k->renormalise GB/s and µs/call", "value": nbytes / us / 1e3,
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": us / 1e3, "us_per_call": us, "us_per_call_events": us_ev,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded fp32 N(0,1) router logits)",
        "config": {"workload": f"{s.name} router: T={s.T} E={s.E} top_k={s.K}", "T": s.T,
                   "E": s.E, "top_k": s.K},
        "roofline": {"bound": "hbm", "kernel": "topk_softmax_kernel", "achieved": nbytes / us_ev / 1e3,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": nbytes / us_ev / 1e3 / PEAK_HBM_GBS,
                     "algorithmic_bytes": nbytes, "avg_launch_us": us_ev, "traffic": None},
    }), flush=True)


def _time_forward(dev, copies, w1s, w2s, out, flags, steps, warmup):
    """us per forward, rotating over the weight copies; HIP events. The
    timed calls go to the C ABI with pre-marshalled arguments (see main)."""
    moe.moe_forward(dev["hidden_states"], w1s[0], w2s[0], dev["topk_weights"], dev["topk_ids"],
                    out=out, flags=flags)  # checks shapes once
    lib = moe.load_library()
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    T, H = dev["hidden_states"].shape
    E, I2, _ = w1s[0].shape
    K = dev["topk_ids"].shape[1]
    argsets = [(P(dev["hidden_states"]), P(w1s[c]), P(w2s[c]), P(dev["topk_weights"]),
                P(dev["topk_ids"]), T, H, I2 // 2, E, K, P(out), ctypes.c_uint32(flags or 0),
                None, 0, ctypes.c_void_p(stream.cuda_stream)) for c in range(copies)]

    def step(i):
        rc = lib.moe_forward_ex(*argsets[i % copies])
        if rc != moe.MOE_OK:
            raise moe.MoeError(rc, lib.moe_last_error().decode())
    for i in range(warmup):
        step(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / steps


def _group_inputs(H, I, E, K, T_max):
    d = make_inputs(T_max, H, I, E, K, seed=0)
    return {k: v.cuda() for k, v in d.items()}


def _copies_for(ids_cpu, H, I):
    touched = len(np.unique(ids_cpu.numpy()))
    return max(1, min(8, -(-512 * 2 ** 20 // (touched * 3 * H * I * 2))))


_PATH_NAMES = {moe.PATH_GROUPED: "grouped", moe.PATH_DECODE: "decode",
               moe.PATH_SMALL_BATCH: "small_batch"}


def bench_table(args):
    """Every row of the shapes table: us/call and TFLOP/s next to the page's
    T_SOL and T_Prod (measured there on its "XPU-A" hardware)."""
    groups = {}
    for row in SHAPES_TABLE:
        groups.setdefault(row[1:5], []).append(row)
    results = []
    for (H, I, E, K), rows in groups.items():
        T_max = max(r[0] for r in rows)
        log(f"[table] H={H} I={I} E={E} K={K}: generating inputs for T={T_max}")
        dev = _group_inputs(H, I, E, K, T_max)
        for (T, _, _, _, _, t_sol, t_prod) in rows:
            sub = {k: (v[:T].contiguous() if k in ("hidden_states", "topk_weights", "topk_ids")
                       else v) for k, v in dev.items()}
            copies = _copies_for(sub["topk_ids"].cpu(), H, I)
            w1s = [sub["w1"]] + [sub["w1"].clone() for _ in range(copies - 1)]
            w2s = [sub["w2"]] + [sub["w2"].clone() for _ in range(copies - 1)]
            out = torch.empty((T, H), dtype=torch.float32, device="cuda")
            flop = 6.0 * T * K * H * I
            est = max(flop / 5e14 * 1e6, 20.0)
            steps = int(max(5, min(100, 3e5 / est)))
            us = _time_forward(sub, copies, w1s, w2s, out, None, steps, 3)
            rec = {"T": T, "H": H, "I": I, "E": E, "top_k": K, "us_per_call": us,
                   "tflops": flop / us / 1e6, "path": _PATH_NAMES[moe.moe_path(T, H, I, E, K)],
                   "page_t_sol_us": t_sol, "page_t_prod_us": t_prod,
                   "speedup_vs_page_t_prod": t_prod / us}
            results.append(rec)
            log(f"[table] T={T:6d} H={H} I={I} E={E:3d} K={K}: {us:9.1f} us {rec['tflops']:7.1f} "
                f"TFLOP/s  page T_Prod {t_prod:8.1f} us  x{t_prod / us:.2f}")
            del w1s, w2s, out
        del dev
        torch.cuda.empty_cache()
    print(json.dumps({"stage": "table", "rows": results}), flush=True)
    return None


def bench_small_t(args):
    """Crossover of the per-token and per-expert weight-streaming paths and
    the grouped path."""
    results = []
    for (H, I, E, K) in ((2048, 768, 128, 8), (2048, 2048, 8, 2), (4096, 384, 128, 8),
                         (4096, 4096, 8, 2)):
        dev = _group_inputs(H, I, E, K, 512)
        for T in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512):
            if T * K > 1024:
                continue
            sub = {k: (v[:T].contiguous() if k in ("hidden_states", "topk_weights", "topk_ids")
                       else v) for k, v in dev.items()}
            copies = _copies_for(sub["topk_ids"].cpu(), H, I)
            w1s = [sub["w1"]] + [sub["w1"].clone() for _ in range(copies - 1)]
            w2s = [sub["w2"]] + [sub["w2"].clone() for _ in range(copies - 1)]
            out = torch.empty((T, H), dtype=torch.float32, device="cuda")
            row = {"T": T, "H": H, "I": I, "E": E, "top_k": K}
            for name, fl in (("decode", moe.FLAG_FORCE_DECODE),
                             ("small_batch", moe.FLAG_FORCE_SMALL_BATCH),
                             ("grouped", moe.FLAG_FORCE_GROUPED)):
                if _PATH_NAMES[moe.moe_path(T, H, I, E, K, fl)] != name:
                    continue
                if name == "decode" and T * K > 256:
                    continue  # per-slot streaming: far off the pace by then
                row[name + "_us"] = _time_forward(sub, copies, w1s, w2s, out, fl, 30, 3)
            row["default_path"] = _PATH_NAMES[moe.moe_path(T, H, I, E, K)]
            results.append(row)
            log(f"[small_t] {row}")
            del w1s, w2s
        del dev
        torch.cuda.empty_cache()
    print(json.dumps({"stage": "small_t", "rows": results}), flush=True)
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill", choices=list(SHAPES))
    ap.add_argument("--path", default="default", choices=list(PATHS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--no-rotate", action="store_true", help="reuse one weight copy every step")
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
                         "decode path vs grouped path for T = 1..64")
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

    s = SHAPES[args.workload]
    if args.stage == "router":
        return bench_router(args, s)
    if args.stage == "table":
        return bench_table(args)
    if args.stage == "small_t":
        return bench_small_t(args)
    if args.stage == "copy":
        n = 512 * 2 ** 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"stage": "copy", "bytes_read": n, "bytes_written": n,
                          "launches": max(args.steps, 1)}), flush=True)
        return None
    flags = PATHS[args.path]
    log(f"[bench] workload {s} path {args.path}: generating inputs")
    d = make_inputs(s.T, s.H, s.I, s.E, s.K, seed=0)
    dev = {k: v.cuda() for k, v in d.items()}
    touched = len(np.unique(d["topk_ids"].numpy()))
    fp8 = args.weights == "fp8"
    block = 256 if s.I % 256 == 0 else 128
    wbytes_per_elem = 1 if fp8 else 2
    wbytes_touched = touched * 3 * s.H * s.I * wbytes_per_elem
    copies = 1 if args.no_rotate else max(1, min(8, -(-512 * 2 ** 20 // wbytes_touched)))
    out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    # The timed loop calls the C ABI with its arguments marshalled once
    # (the binding checks every tensor on each call, about 15 us of host
    # time, which would hide the GPU time of the small-T paths). One call
    # through the Python binding first checks the shapes and the result.
    lib = moe.load_library()
    cs = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    fl = ctypes.c_uint32(flags or 0)
    if fp8:
        q = make_fp8_weights(d, block)
        qs = [{k: q[k].cuda() for k in ("w1q", "w1s", "w2q", "w2s")}]
        qs += [{k: v.clone() for k, v in qs[0].items()} for _ in range(copies - 1)]
        w1s = [torch.empty(0, device="cuda")] * copies  # unused on this path
        w2s = w1s
        flags = (flags or 0) | moe.FLAG_FP8_WEIGHTS
        moe.moe_forward_fp8(dev["hidden_states"], qs[0]["w1q"], qs[0]["w1s"], qs[0]["w2q"],
                            qs[0]["w2s"], block, dev["topk_weights"], dev["topk_ids"], out=out,
                            flags=flags)
        argsets = [(P(dev["hidden_states"]), P(c["w1q"]), P(c["w1s"]), P(c["w2q"]), P(c["w2s"]),
                    block, P(dev["topk_weights"]), P(dev["topk_ids"]), s.T, s.H, s.I, s.E, s.K,
                    moe.ACT_SILU, ctypes.c_float(1.702), ctypes.c_float(7.0), None, None, P(out),
                    fl, None, 0, cs) for c in qs]
        call = lib.moe_forward_fp8
    else:
        w1s = [dev["w1"]] + [dev["w1"].clone() for _ in range(copies - 1)]
        w2s = [dev["w2"]] + [dev["w2"].clone() for _ in range(copies - 1)]
        moe.moe_forward(dev["hidden_states"], w1s[0], w2s[0], dev["topk_weights"],
                        dev["topk_ids"], out=out, flags=flags)
        argsets = [(P(dev["hidden_states"]), P(w1s[c]), P(w2s[c]), P(dev["topk_weights"]),
                    P(dev["topk_ids"]), s.T, s.H, s.I, s.E, s.K, P(out), fl, None, 0, cs)
                   for c in range(copies)]
        call = lib.moe_forward_ex

    def step(i):
        rc = call(*argsets[i % copies])
        if rc != moe.MOE_OK:
            raise moe.MoeError(rc, lib.moe_last_error().decode())

    log(f"[bench] warmup {args.warmup} (weight copies: {copies})")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_wall = (t1 - t0) * 1e3 / args.steps
    ms_event = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] {args.steps} steps: {ms_wall * 1e3:.1f} us/step wall, {ms_event * 1e3:.1f} us/step events")

    # ---- dominant kernel, timed on its own ----
    uses_decode = moe.moe_uses_decode_path(s.T, s.H, s.I, s.E, s.K, flags or 0)
    if uses_decode:
        kernel = "decode_path_fp8" if fp8 else "decode_path"
        scale_bytes = touched * 3 * s.H * (s.I // block) * 4 if fp8 else 0
        alg_bytes = (touched * 3 * s.H * s.I * wbytes_per_elem + scale_bytes + s.T * s.H * 2
                     + s.T * s.H * 4 + s.T * s.K * 8)
        dur_ms = ms_event
        achieved = alg_bytes / (dur_ms * 1e-3) / 1e9
        roof = {"bound": "hbm",
                "kernel": ("decode_gateup_q+decode_down_q (whole decode path, fp8 weights)" if fp8
                           else "decode_gateup+decode_down (whole decode path)"),
                "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS,
                "algorithmic_bytes": alg_bytes, "avg_launch_us": dur_ms * 1e3}
    else:
        M = moe.moe_m_tile(s.T, s.H, s.I, s.E, s.K)
        r = moe.moe_route(dev["topk_ids"], s.E, M)
        act = torch.empty((r["capacity"], s.I), dtype=torch.bfloat16, device="cuda")
        if fp8 and moe.moe_fp8_widens_in_gemm(s.T, s.H, s.I, s.E, s.K, block):
            # the forward's GEMM1 reads the FP8 codes and widens them in registers
            kernel = "grouped_gemm_gate_up_silu_fp8"

            def gemm1(i):
                c = qs[i % copies]
                moe.moe_gemm1_silu_fp8(dev["hidden_states"], c["w1q"], c["w1s"], block, r, s.K,
                                       M, act=act)
        else:
            if fp8:  # the forward widens the weights first; its GEMM1 is the bf16 one
                w1s = [dev["w1"]]
                copies = 1
            kernel = "grouped_gemm_gate_up_silu"

            def gemm1(i):
                moe.moe_gemm1_silu(dev["hidden_states"], w1s[i % copies], r, s.K, M, act=act)
        for i in range(3):
            gemm1(i)
        reps = max(args.steps, 20)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(reps):
            gemm1(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        dur_ms = ev0.elapsed_time(ev1) / reps
        alg_flop = 4.0 * s.T * s.K * s.H * s.I
        achieved = alg_flop / (dur_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kernel, "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "algorithmic_flop": alg_flop, "avg_launch_us": dur_ms * 1e3}
        log(f"[bench] {kernel}: {dur_ms * 1e3:.1f} us/launch, {achieved:.1f} TFLOP/s")
    roof["traffic"] = traffic_for(kernel, args.workload)

    flop = float(s.flop)
    value = flop / (ms_wall * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_wall,
        "us_per_call": ms_wall * 1e3,
        "us_per_call_events": ms_event * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (PAGE_T_PROD_US[args.workload] / (ms_wall * 1e3)
                        if args.workload in PAGE_T_PROD_US else None),
        "vs_baseline_note": ("page's production time on its own 'XPU-A' hardware for this "
                             "shapes-table row (context, not a target)"),
        "dtype": "bf16 (fp8-e4m3 expert weights)" if fp8 else "bf16",
        "data": "synthetic (seeded, atrex-bench #009 input recipe)",
        "config": {"workload": f"{s.name}: T={s.T} H={s.H} I={s.I} E={s.E} top_k={s.K}",
                   "T": s.T, "H": s.H, "I": s.I, "E": s.E, "top_k": s.K,
                   "path": args.path, "weights": args.weights, "weight_copies": copies,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if args.cpu_budget > 0:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(d, s, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
