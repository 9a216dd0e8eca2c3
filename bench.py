"""Throughput of the KVSculpt optimizer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]

Default (the compress row): the long-context Qwen2.5-7B-shaped cache, all
112 (layer, KV-head) problems, N = 32768, n = 17920 training queries per
problem.  The run is the whole method: the 60-iteration pilot at uniform k0,
the budget reallocation, reference attention and Select+Fit at the new
ragged k, then the 150-iteration main run.  A step is one block of 5 main-run
iterations of every problem (direction, Armijo trials, loss and gradient,
history update, then the ridge value re-solve and the loss/gradient after
it), driven through kvs_compress_begin / kvs_compress_advance.  W blocks are
warm-up, the next K are timed (inputs resident in HBM, synchronised before
and after), the rest finish the main run; the metric is problem-iterations
per second, P * 5 * K / (wall time of the K blocks).  The whole-model
compress latency (pilot through iteration T) is measured in the same run.
--config 0..3 runs the other workloads the same way (configs 0 and 1 have
no pilot).

The roofline comes from HIP events on the library's stream around every
launch of the timed kernels during the timed blocks (kvs_profile_enable):
the contraction kernel with the most time is the dominant one.  The float64
oracle is timed on a bounded sample on the host CPU (one block of problem 0).

With --row queries the step is instead one kvs_build_queries call over the
workload's problems: retain queries copied and synthetic future queries
re-embedded from context queries sampled uniformly over the context (the
step just before the optimizer); the metric is training queries built per
second.  With --row use it is one kvs_use_eval call: held-out future
queries over the full and the compressed cache (the step just after the
optimizer); the metric is held-out queries evaluated per second.  Both
default to the 56-problem full-cache workload (--config 2), as does --row
solve: one standalone kvs_value_solve at the Select+Fit keys (Gram,
Cholesky, triangular solves, the refinement step).  --row adam runs
the schedule with Adam on the keys and reports its final output MSE over
L-BFGS's; --row restarts runs R random restarts of one problem as one batch
(kvs_compress_from_keys) and reports the single Select+Fit run's final loss
over the best restart's.  Each row times its own oracle on a bounded sample
beside it.  --row alloc
times the value-norm signal kernel on a llama3-8b-shaped zone and compares
the main run's final MSE under uniform, pilot (flat, two-level, alpha 1)
and value-norm allocations of the same total budget.  --row vector runs 25
iterations on a 64-problem slice of the llama3-8b-shaped cache, large enough
for the vector and reduction kernels' HBM rates to be read from a trace.
These rows time whole calls and take a second, event-timed pass for their
roofline.
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
sys.path.insert(0, ROOT)

# MI355X published dense peaks
PEAK_FP32_MFMA = 157.3e12
PEAK_FP64_MFMA = 78.6e12
PEAK_INT8_MFMA = 5.0e15
PEAK_BF16_MFMA = 2.5e15
PEAK_HBM = 8.0e12
# the Gram's 128x128 tiles: bf16 MFMA products per multiply-add (every operand
# split exactly into three bf16 pieces, the six piece products of weight <= 2)
GRAM_SPLIT_PRODUCTS = 6
PEAK_GRAM_SPLIT = PEAK_BF16_MFMA / GRAM_SPLIT_PRODUCTS
# the integer scores of the loss forward: digit products per score (five
# base-128 digits per element, the pairs of weight s + t <= 5)
INT8_PRODUCTS = 19


def log(*a):
    print(*a, file=sys.stderr, flush=True)


LOGIT_NOTES = {
    "int8": "exact integer products of five base-128 digits per element on int8 MFMA "
            f"({INT8_PRODUCTS} products, int32 sums), shifted in fp64, stored fp32",
    "fp64": "fp64 MFMA, shifted in fp64, stored fp32",
    "fp32": "fp32 MFMA, shifted in fp64, stored fp32"}


def logit_mode():
    """Score arithmetic of the library's loss forwards (KVS_LOGITS, default int8)."""
    m = os.environ.get("KVS_LOGITS", "int8")
    return m if m in ("fp32", "fp64") else "int8"


def score_time_per_flop(mode):
    """Seconds at peak per algorithmic flop of Q Kc^T: fp32 or fp64 MFMA, or
    INT8_PRODUCTS int8 digit products per multiply-add."""
    if mode == "fp64":
        return 1.0 / PEAK_FP64_MFMA
    if mode == "fp32":
        return 1.0 / PEAK_FP32_MFMA
    return INT8_PRODUCTS / PEAK_INT8_MFMA


def mixed_fwd_peak(mode=None):
    """Forward kernel: half its algorithmic flops (Q Kc^T) on the score
    arithmetic's unit, half (A Vc) on fp32 MFMA; the peak is the harmonic
    mix (the MFMA pipes are shared)."""
    return 1.0 / (0.5 * score_time_per_flop(mode or logit_mode()) + 0.5 / PEAK_FP32_MFMA)


# HBM bytes per launch of a kernel on one workload (bench row), from
# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE, each scaled by the ratio of a
# plain copy's known bytes to what the same counter reads for it.  Valid only
# for that kernel source (sha256 of the file) and that workload: other
# workloads report null.
MEASURED_TRAFFIC = {
    # long-context default bench, the timed blocks' dispatches:
    # loss-mode forward (integer scores): FETCH 3393086.5 KiB x 1.99980 + WRITE 18157940.8 KiB x 1.00000 per dispatch
    ("attn_fwd", "qwen2.5-7b-long-context"):
        {"bytes": 25542077627, "source": "attn_fwd.hip", "sha": "d786fa10287fbda0"},
    # Gram, 256x256 tiles on split bf16 products: FETCH 141733727.5 KiB x 1.99980 + WRITE 2765207.7 KiB x 1.00000 per dispatch
    ("gram_split", "qwen2.5-7b-long-context"):
        {"bytes": 293073219537, "source": "gram.hip", "sha": "8175c6117de39252"},
    # L-BFGS vector passes and the merge of the same runs (each operand streamed once):
    # inner products FETCH 1552134.5 KiB x 1.99980 + WRITE 377476.8 KiB, direction FETCH
    # 1085940.2 KiB x 1.99980 + WRITE 220762.4 KiB, merge FETCH 754083.2 KiB x 1.99980 +
    # WRITE 764748.1 KiB per dispatch
    ("hist_dots", "qwen2.5-7b-long-context"):
        {"bytes": 3564989822, "source": "lbfgs.hip", "sha": "f883507a64090751"},
    ("direction", "qwen2.5-7b-long-context"):
        {"bytes": 2449843827, "source": "lbfgs.hip", "sha": "f883507a64090751"},
    ("merge", "qwen2.5-7b-long-context"):
        {"bytes": 2327310012, "source": "attn_fwd.hip", "sha": "d786fa10287fbda0"},
    # training queries: FETCH 53517.7 KiB x 1.99978 + WRITE 107520.0 KiB x 1.00000 per dispatch
    ("build_queries", "qwen2.5-1.5b-full-cache"):
        {"bytes": 219692476, "source": "queries.hip", "sha": "b2221c837c63d711"},
    # loss-mode forward (integer scores): FETCH 10318.44 KiB x 1.99980 + WRITE 48582.10 KiB x 1.00000 per dispatch
    ("attn_fwd", "qwen2.5-1.5b-one-layer"):
        {"bytes": 70878108, "source": "attn_fwd.hip", "sha": "d786fa10287fbda0"},
    # standalone value solve, 128x128 Gram tiles on split bf16 products:
    # FETCH 2628652.75 KiB x 1.99980 + WRITE 134400.0 KiB x 1.00000 per dispatch
    ("gram_split", "qwen2.5-1.5b-full-cache solve"):
        {"bytes": 5520568084, "source": "gram.hip", "sha": "8175c6117de39252"},
}


def source_sha(name):
    import hashlib
    path = os.path.join(ROOT, "attention_distillation_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel, workload):
    t = MEASURED_TRAFFIC.get((kernel, workload))
    if t is None or source_sha(t["source"]) != t["sha"]:
        return None
    return t["bytes"]


def copy_probe(torch, mib):
    """Plain device-to-device copies of a known size (counter calibration)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {mib} MiB three times")


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return os.cpu_count() or 1


def _blas():
    """The BLAS library NumPy/SciPy use, its version and thread pool size."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                         for i in libs) or None
    except Exception:
        return None


def timed_pass(torch, step, steps):
    """Wall time of `steps` calls with nothing recorded on the stream."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def event_pass(torch, K, ctx, kernels, step, steps):
    """The same calls again with a HIP event pair on the library's stream around
    every launch of `kernels`: their launch counts and durations.  Kept out of
    the throughput pass because each event pair costs about 2 us per launch."""
    K.kvs_profile_enable(ctx, True, kernels=kernels)
    torch.cuda.synchronize()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    stats = K.kvs_profile_read(ctx)
    K.kvs_profile_enable(ctx, False)
    return stats


def cpu_queries(w, b, seconds):
    """Float64 oracle of the training-query construction on whole problems."""
    from oracle import kvsculpt as O
    P = b["Qctx"].shape[0]
    done, rows, t0 = 0, 0, time.perf_counter()
    while True:
        p = done % P
        Qo = O.training_queries(b["Qctx"][p], b["src"][p], w.m, w.theta)
        rows += Qo.shape[0]
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": rows / el, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{w.name}: {done} problems' training queries "
                      f"({rows} rows of d={w.d}), float64 NumPy"}


def bench_queries(args, torch, K):
    """Training-query construction alone: one launch per step."""
    from synth import WORKLOADS, make_context_batch
    w = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] generating context queries of {w.name}: P={w.P} g={w.g} N={w.N} d={w.d}")
    b = make_context_batch(w, 0)
    P, g, N, d = b["Qctx"].shape
    F, m = b["src"].shape[2], w.m
    n = g * (m + F)
    Qctx = torch.from_numpy(b["Qctx"]).to(dev)
    src = torch.from_numpy(b["src"]).to(dev)
    Q = torch.empty((P, n, d), dtype=torch.float32, device=dev)
    ctx = K.Context()

    def step():
        K.kvs_build_queries(ctx, P, g, N, m, F, d, w.theta, Qctx, src, Q, None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    elapsed = timed_pass(torch, step, args.steps)
    st = event_pass(torch, K, ctx, ["build_queries"], step, args.steps)["build_queries"]
    avg_s = st["ms"] / st["launches"] / 1e3
    bytes_launch = st["bytes"] / st["launches"]
    achieved = bytes_launch / avg_s
    roofline = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                "traffic": traffic_for("build_queries", w.name), "kernel": "build_queries",
                "launches": st["launches"], "avg_us": round(avg_s * 1e6, 2)}
    cpu = None if args.no_cpu_baseline else cpu_queries(w, b, min(args.cpu_seconds, 10.0))
    out = {
        "metric": "training queries built/sec (retain copies + De-RoPE/RoPE future queries)",
        "value": round(P * n * args.steps / elapsed, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (angles f64)", "data": "synthetic",
        "config": {"workload": w.name, "row": "queries", "problems": P, "g": g, "N": N, "m": m,
                   "F": F, "d": d, "theta": w.theta},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_use(w, u, Kc, Vc, k, seconds):
    """Float64 oracle of the use-side evaluation on whole problems."""
    from oracle import kvsculpt as O
    P = u["Qh"].shape[0]
    done, rows, t0 = 0, 0, time.perf_counter()
    while True:
        p = done % P
        O.use_side_outputs(u["Qh"][p], u["Kz"][p], u["Vz"][p], u["Kr"][p], u["Vr"][p],
                           Kc[p * k:(p + 1) * k], Vc[p * k:(p + 1) * k], u["scale"])
        rows += u["Qh"].shape[1]
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": rows / el, "unit": "queries/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{w.name}: {done} problems' use-side outputs ({rows} held-out queries "
                      f"over Z={w.Z} + m={w.m} and k={k} + m keys), float64 NumPy"}


def bench_use(args, torch, K):
    """Use-side evaluation alone: held-out queries over the full and the compressed cache."""
    from synth import WORKLOADS, make_use_batch
    w = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] generating held-out queries of {w.name}: P={w.P} g={w.g} per head {w.F}")
    u = make_use_batch(w, 0)
    P, n, d = u["Qh"].shape
    k = w.k0
    rng = np.random.default_rng(0)
    idx = [np.sort(rng.choice(w.Z, size=k, replace=False)) for _ in range(P)]
    Kc = np.concatenate([u["Kz"][p, idx[p]] for p in range(P)])
    Vc = np.concatenate([u["Vz"][p, idx[p]] for p in range(P)])
    g = {key: torch.from_numpy(u[key]).to(dev) for key in ("Qh", "Kz", "Vz", "Kr", "Vr")}
    Kcg, Vcg = torch.from_numpy(Kc).to(dev), torch.from_numpy(Vc).to(dev)
    bt = K.Batch(P, d, w.Z, n, k=[k] * P, scale=u["scale"])
    ws = torch.empty(K.use_eval_workspace_bytes(bt, w.m), dtype=torch.uint8, device=dev)
    mse = torch.empty(P, dtype=torch.float32, device=dev)
    rl = torch.empty(P, dtype=torch.float32, device=dev)
    ctx = K.Context()

    def step():
        K.kvs_use_eval(ctx, bt, w.m, g["Qh"], g["Kz"], g["Vz"], g["Kr"], g["Vr"], Kcg, Vcg, None,
                       None, mse, rl, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    elapsed = timed_pass(torch, step, args.steps)
    st = event_pass(torch, K, ctx, ["use_attn_fwd"], step, args.steps)["use_attn_fwd"]
    avg_s = st["ms"] / st["launches"] / 1e3
    achieved = st["flops"] / st["launches"] / avg_s
    # the use-side forwards form their scores on fp64 MFMA (fp32 if asked)
    peak = mixed_fwd_peak("fp32" if logit_mode() == "fp32" else "fp64")
    roofline = {"bound": "mfma", "achieved": round(achieved / 1e12, 3), "peak": round(peak / 1e12, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic_for("use_attn_fwd", w.name), "kernel": "use_attn_fwd",
                "launches": st["launches"], "avg_us": round(avg_s * 1e6, 2)}
    log(f"[bench] use-side rel error per problem: {rl.cpu().numpy()[:8].tolist()} ...")
    cpu = None if args.no_cpu_baseline else cpu_use(w, u, Kc, Vc, k, min(args.cpu_seconds, 10.0))
    out = {
        "metric": "held-out queries evaluated/sec over the full and the compressed cache",
        "value": round(P * n * args.steps / elapsed, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (scores f64)", "data": "synthetic",
        "config": {"workload": w.name, "row": "use", "problems": P, "n_heldout": n, "Z": w.Z,
                   "m": w.m, "k": k, "d": d},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_solve(w, hb, Kc, k, seconds):
    """Float64 oracle of the ridge value solve on whole problems."""
    from oracle import kvsculpt as O
    P = hb["Q"].shape[0]
    done, t0 = 0, time.perf_counter()
    while True:
        p = done % P
        O.ridge_values(hb["Q"][p], hb["Y"][p], Kc[p * k:(p + 1) * k], hb["scale"])
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": done / el, "unit": "problem-solves/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{w.name}: {done} problems' ridge solves (n={hb['Q'].shape[1]}, k={k}, "
                      f"d={w.d}), float64 NumPy/SciPy"}


def bench_solve(args, torch, K):
    """The standalone ridge value solve at the Select+Fit keys: scores, Gram with the
    A^T Y rows, Cholesky, back substitution and the refinement step."""
    from synth import WORKLOADS, make_batch
    w = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}: P={w.P} n={w.n} Z={w.Z} d={w.d} k0={w.k0}")
    b = make_batch(w, 0)
    P, n, d = b["Q"].shape
    Z, k = b["Kz"].shape[1], w.k0
    Q = torch.from_numpy(b["Q"]).to(dev)
    Kz = torch.from_numpy(b["Kz"]).to(dev)
    Vz = torch.from_numpy(b["Vz"]).to(dev)
    ctx = K.Context()
    bt = K.Batch(P, d, Z, n, k=[k] * P, scale=b["scale"])
    ws = torch.empty(K.workspace_bytes(bt), dtype=torch.uint8, device=dev)
    Y = torch.empty((P, n, d), dtype=torch.float32, device=dev)
    lse = torch.empty((P, n), dtype=torch.float32, device=dev)
    K.kvs_reference_attn(ctx, bt, Q, Kz, Vz, Y, lse, ws)
    idx = torch.empty(P * k, dtype=torch.int32, device=dev)
    Kc = torch.empty((P * k, d), dtype=torch.float32, device=dev)
    Vc = torch.empty((P * k, d), dtype=torch.float32, device=dev)
    flags = torch.zeros(P, dtype=torch.int32, device=dev)
    K.kvs_init_topk(ctx, bt, Q, Kz, Y, lse, idx, Kc, Vc, flags, ws)
    log("[bench] Select+Fit keys ready")

    def step():
        K.kvs_value_solve(ctx, bt, Q, Y, lse, Kc, Vc, flags, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    elapsed = timed_pass(torch, step, args.steps)
    ev = event_pass(torch, K, ctx, ["gram", "gram_split"], step, args.steps)
    gname = gram_kernel_of(ev)
    st = ev[gname]
    avg_s = st["ms"] / st["launches"] / 1e3
    achieved = st["flops"] / st["launches"] / avg_s
    peak, peak_note = contraction_peak(gname)
    roofline = {"bound": "mfma", "achieved": round(achieved / 1e12, 3),
                "peak": round(peak / 1e12, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "frac_fp32_mfma": round(achieved / PEAK_FP32_MFMA, 4),
                "traffic": traffic_for(gname, w.name + " solve"), "kernel": gname, "peak_kind": peak_note,
                "launches": st["launches"], "avg_us": round(avg_s * 1e6, 2)}
    log(f"[bench] flags {int(flags.ne(0).sum().item())} of {P} problems set")
    cpu = None
    if not args.no_cpu_baseline:
        hb = {"Q": b["Q"], "Y": Y.cpu().numpy(), "scale": b["scale"]}
        cpu = cpu_solve(w, hb, Kc.cpu().numpy(), k, min(args.cpu_seconds, 15.0))
    out = {
        "metric": "ridge value solves/sec (Gram, Cholesky, triangular solves, one refinement step)",
        "value": round(P * args.steps / elapsed, 2), "unit": "problem-solves/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (scores " + {"int8": "exact int8 digit products", "fp64": "f64",
                                     "fp32": "f32"}[logit_mode()] + ", residual f64)",
        "data": "synthetic",
        "config": {"workload": w.name, "row": "solve", "problems": P, "n": n, "Z": Z, "k": k, "d": d,
                   "keys": "Select+Fit"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def _fwd_roofline(stats, workload):
    st = stats["attn_fwd"]
    avg_s = st["ms"] / st["launches"] / 1e3
    achieved = st["flops"] / st["launches"] / avg_s
    peak = mixed_fwd_peak()
    return {"bound": "mfma", "achieved": round(achieved / 1e12, 3), "peak": round(peak / 1e12, 1),
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": traffic_for("attn_fwd", workload),
            "kernel": "attn_fwd", "launches": st["launches"], "avg_us": round(avg_s * 1e6, 2)}


def cpu_adam(w, b, seconds, lr):
    """Float64 oracle of the Adam schedule on problem 0 (bounded iterations)."""
    from oracle import kvsculpt as O
    Q, Kz, Vz, s = b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"]
    Y, l = O.reference_attention(Q, Kz, Vz, s)
    t0 = time.perf_counter()
    O.compress_problem_adam(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=5), O.AdamOptions(lr=lr),
                            Y=Y, lse=l)
    t5 = time.perf_counter() - t0
    iters = int(max(5, min(w.T, 5 * round(seconds / max(t5, 1e-3)))))
    t0 = time.perf_counter()
    O.compress_problem_adam(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=iters),
                            O.AdamOptions(lr=lr), Y=Y, lse=l)
    el = time.perf_counter() - t0
    return {"value": iters / el, "unit": "problem-iterations/s", "cores": _threads(),
            "kind": "oracle", "sample": f"{w.name} problem 0, {iters} Adam iterations with value "
                                        f"solves every 5 (Select+Fit init included), float64"}


def cpu_restart(w, b, K0, seconds):
    """Float64 oracle of one restart (the schedule from given keys) on problem 0."""
    from oracle import kvsculpt as O
    Q, Kz, Vz, s = b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"]
    Y, l = O.reference_attention(Q, Kz, Vz, s)
    t0 = time.perf_counter()
    O.compress_problem(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=5), Y=Y, lse=l, init=K0,
                       init_keys=True)
    t5 = time.perf_counter() - t0
    iters = int(max(5, min(w.T, 5 * round(seconds / max(t5, 1e-3)))))
    t0 = time.perf_counter()
    O.compress_problem(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=iters), Y=Y, lse=l, init=K0,
                       init_keys=True)
    el = time.perf_counter() - t0
    return {"value": iters / el, "unit": "problem-iterations/s", "cores": _threads(),
            "kind": "oracle", "sample": f"{w.name} problem 0, one restart of {iters} L-BFGS "
                                        f"iterations from random keys, float64"}


def bench_adam(args, torch, K):
    """The schedule with Adam on the keys, and its final MSE against L-BFGS's."""
    from synth import WORKLOADS, make_batch
    w = WORKLOADS[args.config]
    T = w.T if args.iters is None else args.iters
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}: P={w.P} n={w.n} Z={w.Z} k={w.k0} T={T}")
    b = make_batch(w, 0)
    P, n, d = b["Q"].shape
    Q, Kz, Vz = (torch.from_numpy(b[key]).to(dev) for key in ("Q", "Kz", "Vz"))
    bt = K.Batch(P, d, w.Z, n, k=[w.k0] * P, scale=b["scale"])
    o = K.opts(iters=T)
    a = K.adam_opts(lr=args.adam_lr)
    ws = torch.empty(K.workspace_bytes(bt, o), dtype=torch.uint8, device=dev)
    Kc = torch.empty((w.k0 * P, d), dtype=torch.float32, device=dev)
    Vc = torch.empty_like(Kc)
    loss, mse, l0 = (torch.empty(P, dtype=torch.float32, device=dev) for _ in range(3))
    flags = torch.zeros(P, dtype=torch.int32, device=dev)
    ctx = K.Context()

    def step():
        K.kvs_compress_adam(ctx, bt, o, a, 0, Q, Kz, Vz, Kc, Vc, loss, mse, l0, flags, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    elapsed = timed_pass(torch, step, args.steps)
    stats = event_pass(torch, K, ctx, ["attn_fwd"], step, args.steps)
    mse_adam, fl = mse.cpu().numpy().copy(), flags.cpu().numpy().copy()
    K.kvs_compress(ctx, bt, o, Q, Kz, Vz, Kc, Vc, loss, mse, l0, flags, ws)
    mse_lb = mse.cpu().numpy().copy()
    ratio = [float(x) for x in mse_adam / mse_lb]
    log(f"[bench] final output MSE Adam {mse_adam.tolist()} L-BFGS {mse_lb.tolist()} flags {fl.tolist()}")
    cpu = None if args.no_cpu_baseline else cpu_adam(w, b, min(args.cpu_seconds, 15.0), args.adam_lr)
    out = {
        "metric": "Adam-on-keys schedule: problem-iterations/sec (ablation of L-BFGS)",
        "value": round(P * T * args.steps / elapsed, 2), "unit": "problem-iterations/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "row": "adam", "problems": P, "n": n, "Z": w.Z,
                   "k": w.k0, "iters": T, "vc_every": 5, "lr": args.adam_lr,
                   "mse_adam_over_lbfgs": [round(r, 3) for r in ratio]},
        "roofline": _fwd_roofline(stats, w.name),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_restarts(args, torch, K):
    """A search over random restarts of one problem, batched, against one run."""
    from synth import WORKLOADS, make_batch
    w = WORKLOADS[args.config]
    T = w.T if args.iters is None else args.iters
    R = args.restarts
    dev = torch.device("cuda:0")
    b = make_batch(w, 0, problems=[0])
    _, n, d = b["Q"].shape
    log(f"[bench] {R} restarts of {w.name} problem 0: n={n} Z={w.Z} k={w.k0} T={T}")
    rng = np.random.default_rng(0)
    draws = [np.sort(rng.choice(w.Z, w.k0, replace=False)) for _ in range(R)]
    Kc0 = np.concatenate([b["Kz"][0][ix] for ix in draws])
    rep = {key: torch.from_numpy(b[key]).to(dev).expand(R, -1, -1).contiguous()
           for key in ("Q", "Kz", "Vz")}
    bt = K.Batch(R, d, w.Z, n, k=[w.k0] * R, scale=b["scale"])
    o = K.opts(iters=T)
    ws = torch.empty(K.workspace_bytes(bt, o), dtype=torch.uint8, device=dev)
    Kc0g = torch.from_numpy(Kc0).to(dev)
    Kc = torch.empty_like(Kc0g)
    Vc = torch.empty_like(Kc0g)
    loss, mse, l0 = (torch.empty(R, dtype=torch.float32, device=dev) for _ in range(3))
    flags = torch.zeros(R, dtype=torch.int32, device=dev)
    ctx = K.Context()

    def step():
        Kc.copy_(Kc0g)
        K.kvs_compress_from_keys(ctx, bt, o, rep["Q"], rep["Kz"], rep["Vz"], Kc, Vc, loss, mse, l0,
                                 flags, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    elapsed = timed_pass(torch, step, args.steps)
    stats = event_pass(torch, K, ctx, ["attn_fwd"], step, args.steps)
    lr_ = loss.cpu().numpy().copy()
    # the single Select+Fit run of the same problem
    b1 = K.Batch(1, d, w.Z, n, k=[w.k0], scale=b["scale"])
    K.kvs_compress(ctx, b1, o, rep["Q"][:1], rep["Kz"][:1], rep["Vz"][:1], Kc[:w.k0], Vc[:w.k0],
                   loss[:1], mse[:1], l0[:1], flags[:1], ws)
    single = float(loss[:1].cpu().numpy()[0])
    best = float(lr_.min())
    log(f"[bench] restart losses min {best:.6g} median {float(np.median(lr_)):.6g} "
        f"max {float(lr_.max()):.6g}; single Select+Fit run {single:.6g}")
    cpu = None if args.no_cpu_baseline else cpu_restart(w, b, b["Kz"][0][draws[0]],
                                                        min(args.cpu_seconds, 15.0))
    out = {
        "metric": "random-restart search: problem-iterations/sec over R restarts batched",
        "value": round(R * T * args.steps / elapsed, 2), "unit": "problem-iterations/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "row": "restarts", "problem": 0, "restarts": R, "n": n,
                   "Z": w.Z, "k": w.k0, "iters": T,
                   "single_run_over_best_restart": round(single / best, 4)},
        "roofline": _fwd_roofline(stats, f"{w.name} x{R} restarts"),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_alloc(args, torch, K):
    """Allocation variants: the value-norm signal kernel timed on a large zone,
    then the main run's final output MSE under each allocation of the budget."""
    from synth import WORKLOADS, make_batch
    dev = torch.device("cuda:0")
    # timed: the static signal over a llama3-8b-shaped compress zone, N(0, 1)
    # values (the generator's value distribution) drawn on the device
    w3 = WORKLOADS[3]
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    V = torch.randn((w3.P, w3.Z, w3.d), generator=gen, device=dev, dtype=torch.float32)
    sig = torch.empty(w3.P, dtype=torch.float64, device=dev)
    ws = torch.empty(K.value_norms_workspace_bytes(w3.P, w3.Z), dtype=torch.uint8, device=dev)
    ctx = K.Context()
    for _ in range(args.warmup):
        K.kvs_value_norms(ctx, w3.P, w3.Z, w3.d, V, sig, ws)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(args.steps, 10)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(reps):
        K.kvs_value_norms(ctx, w3.P, w3.Z, w3.d, V, sig, ws)
    e1.record(st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg_s = e0.elapsed_time(e1) / reps / 1e3
    nbytes = float(w3.P) * w3.Z * w3.d * 4
    roofline = {"bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(nbytes / avg_s / PEAK_HBM, 4),
                "traffic": traffic_for("value_norms", "llama3-8b zone"), "kernel": "value_norms (+ final sum)",
                "launches": reps, "avg_us": round(avg_s * 1e6, 2)}
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle signal on problems of the same zone, copied to the host
        from oracle import kvsculpt as O
        Vh = V[: min(w3.P, 16)].cpu().numpy()
        done, t0c = 0, time.perf_counter()
        while time.perf_counter() - t0c < min(args.cpu_seconds, 10.0):
            O.value_norm_signal(Vh[done % Vh.shape[0]])
            done += 1
        elc = time.perf_counter() - t0c
        cpu = {"value": round(done * w3.Z / elc, 1), "unit": "rows/s", "cores": _threads(),
               "kind": "oracle", "sample": f"{done} problems' value-norm signals ({w3.Z} x {w3.d} "
                                           f"zones), float64 NumPy"}
    del V
    # quality: pilot at uniform k, then the main run under each allocation
    w = WORKLOADS[args.config]
    T = w.T if args.iters is None else args.iters
    log(f"[bench] generating {w.name}: P={w.P} layers={w.layers} heads={w.kv_heads}")
    b = make_batch(w, 0)
    P, n, d = b["Q"].shape
    Q, Kz, Vz = (torch.from_numpy(b[key]).to(dev) for key in ("Q", "Kz", "Vz"))
    K_total = w.k0 * P
    bt0 = K.Batch(P, d, w.Z, n, k=[w.k0] * P, scale=b["scale"])
    pm = torch.empty(P, dtype=torch.float32, device=dev)
    o = K.opts(iters=T)
    need = max(K.workspace_bytes(K.Batch(P, d, w.Z, n, k=[w.Z] * P, scale=b["scale"]), o), 256)
    wsm = torch.empty(need, dtype=torch.uint8, device=dev)
    K.kvs_pilot_allocate(ctx, bt0, K.opts(iters=w.pilot or 60), w.pilot or 60, 0.5, 1, w.Z, Q, Kz,
                         Vz, pm, wsm)
    pilot = pm.cpu().numpy().astype(np.float64)
    wsn = torch.empty(K.value_norms_workspace_bytes(P, w.Z), dtype=torch.uint8, device=dev)
    vsig = torch.empty(P, dtype=torch.float64, device=dev)
    K.kvs_value_norms(ctx, P, w.Z, d, Vz, vsig, wsn)
    allocs = {
        "uniform": np.full(P, w.k0, dtype=np.int32),
        "pilot_sqrt_flat": K.kvs_allocate_budget(pilot, K_total, 0.5, 1, w.Z),
        "pilot_sqrt_two_level": K.kvs_allocate_budget_two_level(pilot, w.layers, w.kv_heads,
                                                                K_total, 0.5, 1, w.Z),
        "pilot_mse_flat_alpha1": K.kvs_allocate_budget(pilot, K_total, 1.0, 1, w.Z),
        "value_norm_static": K.kvs_allocate_budget(vsig.cpu().numpy(), K_total, 1.0, 1, w.Z),
    }
    # held-out queries for the use-side error of each allocation
    from synth import make_use_batch
    u = make_use_batch(w, 0, per_head=128)
    nh = u["Qh"].shape[1]
    Qh, Kr, Vr = (torch.from_numpy(u[key]).to(dev) for key in ("Qh", "Kr", "Vr"))
    umse = torch.empty(P, dtype=torch.float32, device=dev)
    urel = torch.empty(P, dtype=torch.float32, device=dev)
    quality = {}
    for name, ks in allocs.items():
        bt = K.Batch(P, d, w.Z, n, k=ks, scale=b["scale"])
        Kc = torch.empty((int(ks.sum()), d), dtype=torch.float32, device=dev)
        Vc = torch.empty_like(Kc)
        loss, mse, l0 = (torch.empty(P, dtype=torch.float32, device=dev) for _ in range(3))
        flags = torch.zeros(P, dtype=torch.int32, device=dev)
        K.kvs_compress(ctx, bt, o, Q, Kz, Vz, Kc, Vc, loss, mse, l0, flags, wsm)
        m = mse.cpu().numpy().astype(np.float64)
        bu = K.Batch(P, d, w.Z, nh, k=ks, scale=b["scale"])
        wsu = torch.empty(K.use_eval_workspace_bytes(bu, w.m), dtype=torch.uint8, device=dev)
        K.kvs_use_eval(ctx, bu, w.m, Qh, Kz, Vz, Kr, Vr, Kc, Vc, None, None, umse, urel, wsu)
        um = umse.cpu().numpy().astype(np.float64)
        quality[name] = {"mean_mse": float(m.mean()), "max_mse": float(m.max()),
                         "use_mean_mse": float(um.mean()),
                         "use_mean_rel": float(urel.cpu().numpy().astype(np.float64).mean()),
                         "k_min": int(ks.min()), "k_max": int(ks.max())}
        log(f"[bench] {name:22s} mean final MSE {m.mean():.4e} max {m.max():.4e}; held-out "
            f"use-side MSE {um.mean():.4e}; k in [{ks.min()}, {ks.max()}]")
        del wsu
    base = quality["uniform"]["mean_mse"]
    ubase = quality["uniform"]["use_mean_mse"]
    out = {
        "metric": "value-norm allocation signal: zone rows reduced/sec (HBM); allocation variants' final MSE",
        "value": round(w3.P * w3.Z * reps / elapsed, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": reps, "warmup": args.warmup, "ms_per_step": round(1e3 * elapsed / reps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32 (sums f64)",
        "data": "synthetic",
        "config": {"workload": f"signal: {w3.name} zone ({w3.P} x {w3.Z} x {w3.d}); quality: {w.name}",
                   "row": "alloc", "iters": T,
                   "mean_mse_over_uniform": {k: round(v["mean_mse"] / base, 4) for k, v in quality.items()},
                   "use_mse_over_uniform": {k: round(v["use_mean_mse"] / ubase, 4)
                                            for k, v in quality.items()},
                   "quality": quality},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_vector(args, torch, K):
    """The schedule on a 64-problem slice of the llama3-8b-shaped cache: one key
    chunk and one query split, so the merge, history and direction kernels move
    hundreds of MB per launch (their HBM fractions come from a kernel trace)."""
    from synth import WORKLOADS, make_batch
    w = WORKLOADS[3]
    P = 64
    T = 25 if args.iters is None else args.iters
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name} problems 0..{P - 1}: n={w.n} Z={w.Z} k={w.k0} T={T}")
    b = make_batch(w, 0, problems=list(range(P)))
    _, n, d = b["Q"].shape
    Q, Kz, Vz = (torch.from_numpy(b[key]).to(dev) for key in ("Q", "Kz", "Vz"))
    bt = K.Batch(P, d, w.Z, n, k=[w.k0] * P, scale=b["scale"])
    o = K.opts(iters=T)
    ws = torch.empty(K.workspace_bytes(bt, o), dtype=torch.uint8, device=dev)
    Kc = torch.empty((w.k0 * P, d), dtype=torch.float32, device=dev)
    Vc = torch.empty_like(Kc)
    loss, mse, l0 = (torch.empty(P, dtype=torch.float32, device=dev) for _ in range(3))
    flags = torch.zeros(P, dtype=torch.int32, device=dev)
    ctx = K.Context()

    def step():
        K.kvs_compress(ctx, bt, o, Q, Kz, Vz, Kc, Vc, loss, mse, l0, flags, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    elapsed = timed_pass(torch, step, args.steps)
    stats = event_pass(torch, K, ctx, ["attn_fwd"], step, args.steps)
    out = {
        "metric": "L-BFGS problem-iterations/sec on a 64-problem llama3-8b slice (vector-kernel sizing run)",
        "value": round(P * T * args.steps / elapsed, 2), "unit": "problem-iterations/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name} problems 0..{P - 1}", "row": "vector", "n": n,
                   "Z": w.Z, "k": w.k0, "iters": T},
        "roofline": _fwd_roofline(stats, f"{w.name} slice of {P}"),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


# kernels whose launches are timed with HIP events during the timed blocks
TIMED_KERNELS = ["attn_fwd", "attn_bwd", "attn_bwd_split", "gram", "gram_split", "attn_pv", "potrf_panel",
                 "back_subst",
                 "merge", "hist_dots", "direction", "key_digits", "resid_rhs", "resid_rhs_split",
                 "fwd_subst"]
# contraction kernels (MFMA roofline) and their peaks: the loss forward forms
# its scores on the score arithmetic's unit (half its flops) and A Vc on fp32
# MFMA (the other half); the split-product Gram, refinement residual and
# backward run on bf16 MFMA, six products per multiply-add; the others are
# fp32 MFMA only
CONTRACTIONS = ("attn_fwd", "attn_bwd", "attn_bwd_split", "gram", "gram_split", "attn_pv", "resid_rhs",
                "resid_rhs_split")
SPLIT_KERNELS = ("gram_split", "resid_rhs_split", "attn_bwd_split")


def gram_kernel_of(stats):
    """The Gram's profile name in these stats: the split-product kernel when
    its launches ran (large batches), else the fp32 one."""
    return "gram_split" if stats.get("gram_split", {}).get("launches", 0) else "gram"


def contraction_peak(name):
    """(peak flop rate, description) of a contraction kernel other than the
    loss forward."""
    if name in SPLIT_KERNELS:
        return PEAK_GRAM_SPLIT, (f"bf16 MFMA over {GRAM_SPLIT_PRODUCTS} products per multiply-add "
                                 f"(exact three-piece bf16 splits of both operands)")
    return PEAK_FP32_MFMA, "fp32 MFMA"


def kernel_rows(stats):
    """Per-kernel time, launches and roofline fractions from event totals."""
    rows = {}
    for name, st in stats.items():
        if st["launches"] == 0:
            continue
        sec = st["ms"] / 1e3
        row = {"launches": st["launches"], "ms": round(st["ms"], 3),
               "avg_us": round(1e6 * sec / st["launches"], 2)}
        if name in CONTRACTIONS and st["flops"] > 0:
            fl = st["flops"]
            row["tflops"] = round(fl / sec / 1e12, 2)
            if name == "attn_fwd":
                # t_min = (fl/2) on the score unit + (fl/2)/fp32 peak, the MFMA pipes being shared
                mode = logit_mode()
                ts = 0.5 * fl * score_time_per_flop(mode)
                row["frac_mfma_mixed"] = round((ts + 0.5 * fl / PEAK_FP32_MFMA) / sec, 4)
                row[f"frac_{mode}_scores_part"] = round(ts / sec, 4)
                row["frac_fp32_part"] = round(0.5 * fl / sec / PEAK_FP32_MFMA, 4)
                # the algorithmic rate against the fp32 MFMA peak
                row["frac_fp32_mfma"] = round(fl / sec / PEAK_FP32_MFMA, 4)
            else:
                if name in SPLIT_KERNELS:
                    row["frac_split_bf16_mfma"] = round(fl / sec / PEAK_GRAM_SPLIT, 4)
                row["frac_fp32_mfma"] = round(fl / sec / PEAK_FP32_MFMA, 4)
        rows[name] = row
    return rows


def contractions_note(stats):
    parts = []
    if gram_kernel_of(stats) == "gram_split":
        parts.append("the Gram's large tiles")
    if stats.get("resid_rhs_split", {}).get("launches", 0):
        parts.append("the refinement residual A^T G")
    if stats.get("attn_bwd_split", {}).get("launches", 0):
        parts.append("the backward (G Vc^T, dS^T Q)")
    if not parts:
        return "fp32 MFMA"
    return (f"fp32 MFMA; {' and '.join(parts)} on bf16 MFMA over exact three-piece bf16 splits "
            f"({GRAM_SPLIT_PRODUCTS} products per multiply-add, fp32 accumulation)")


def cpu_baseline_block(w, b):
    """The float64 oracle on problem 0 of the workload, timed on one block of
    the main run: 5 L-BFGS iterations at uniform k0 from the Select+Fit start,
    the value re-solve and the loss/gradient after it (the unit the GPU's
    step is made of).  The reference attention, Select+Fit and the loss at
    the start are set-up, not timed.  Then the work of one iteration (a
    trial loss and a loss/gradient) with the BLAS pool held to one thread."""
    from oracle import kvsculpt as O
    threads = _threads()
    Q, Kz, Vz, s = b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"]
    t0 = time.perf_counter()
    Y, l = O.reference_attention(Q, Kz, Vz, s)
    idx, Kc, Vc, ok = O.init_select_fit(Q, Kz, Y, l, w.k0, s)
    t_setup = time.perf_counter() - t0
    log(f"[bench] oracle set-up (reference attention, Select+Fit) {t_setup:.1f} s")
    t0 = time.perf_counter()
    O.loss_grad(Q, Y, l, Kc, Vc, s)
    t_eval = time.perf_counter() - t0
    t0 = time.perf_counter()
    r = O.compress_problem(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=5), Y=Y, lse=l, init=(Kc, Vc))
    t_blk = time.perf_counter() - t0 - t_eval       # less the start's loss/gradient
    log(f"[bench] oracle block of 5 iterations {t_blk:.1f} s on {threads} threads")
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.loss(Q, Y, l, r["Kc"], r["Vc"], s)
            t_f1 = time.perf_counter() - t0
            t0 = time.perf_counter()
            O.loss_grad(Q, Y, l, r["Kc"], r["Vc"], s)
            t_g1 = time.perf_counter() - t0
        one = {"value": round(1.0 / (t_f1 + t_g1), 4), "unit": "problem-iterations/s", "cores": 1,
               "sample": f"{w.name} problem 0 at the block's end point, BLAS held to 1 thread: one "
                         f"trial loss ({t_f1:.2f} s) plus one loss and gradient ({t_g1:.2f} s), the "
                         f"work of an iteration whose first trial is accepted, without the value "
                         f"re-solve's share"}
        log(f"[bench] oracle iteration work on 1 thread {t_f1 + t_g1:.2f} s")
    except Exception as e:  # threadpoolctl missing: report the multi-thread figure only
        log(f"[bench] one-thread oracle run skipped: {e}")
    return {"value": round(5.0 / t_blk, 4), "unit": "problem-iterations/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{w.name} problem 0 at k0={w.k0}: one block of 5 L-BFGS iterations "
                      f"with its value re-solve and the loss/gradient after it, from the Select+Fit start, float64 NumPy/SciPy; "
                      f"reference attention and Select+Fit ({t_setup:.0f} s) not timed",
            "host_cpus": os.cpu_count(), "blas": _blas(),
            "one_thread": one}


def bench_compress(args, torch, K):
    """The optimizer on a whole cache: pilot, reallocation, then the main run
    at ragged k, timed in blocks of 5 iterations (one step = one block for
    all problems, ending with the value re-solve and the loss/gradient after
    it).  The whole-model compress latency (pilot, reallocation, reference
    attention, Select+Fit, all T iterations) is measured in the same run."""
    from synth import WORKLOADS, make_batch
    w = WORKLOADS[args.config]
    if args.ratio is not None:
        w = w.with_ratio(args.ratio)
    T = w.T if args.iters is None else args.iters
    VC = 5
    if T % VC:
        raise SystemExit("--iters must be a multiple of 5 (a step is a block of 5 iterations)")
    W, Kst = args.warmup, args.steps
    nblk_T = T // VC
    nblk = max(nblk_T, W + Kst)
    workers = min(16, os.cpu_count() or 1)
    log(f"[bench] generating {w.name}: P={w.P} n={w.n} Z={w.Z} d={w.d} k0={w.k0} T={T} "
        f"pilot={w.pilot} ({workers} processes)")
    t0 = time.perf_counter()
    b = make_batch(w, 0, workers=workers if w.P > 8 else 1)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    P, n, d = b["Q"].shape
    Z = b["Kz"].shape[1]
    Q = torch.from_numpy(b["Q"]).to(dev)
    Kz = torch.from_numpy(b["Kz"]).to(dev)
    Vz = torch.from_numpy(b["Vz"]).to(dev)
    ctx = K.Context()
    o = K.opts(iters=T)
    pilot = w.pilot or 0
    loss, mse, l0 = (torch.empty(P, dtype=torch.float32, device=dev) for _ in range(3))
    flags = torch.zeros(P, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs in HBM ({(b['Q'].nbytes + 2 * b['Kz'].nbytes) / 2**30:.2f} GiB)")

    # ---- whole-model compress: everything from here to the end of iteration T
    t_start = time.perf_counter()
    ks = [w.k0] * P
    t_pilot = 0.0
    if pilot:
        bt0 = K.Batch(P, d, Z, n, k=ks, scale=b["scale"])
        ws0 = torch.empty(K.workspace_bytes(bt0, K.opts(iters=pilot)), dtype=torch.uint8, device=dev)
        pm = torch.empty(P, dtype=torch.float32, device=dev)
        ks = list(K.kvs_pilot_allocate(ctx, bt0, K.opts(iters=pilot), pilot, 0.5, 1, Z, Q, Kz, Vz, pm,
                                       ws0))
        t_pilot = time.perf_counter() - t_start
        del ws0
        log(f"[bench] pilot ({pilot} iterations) + reallocation {t_pilot:.2f} s: k in "
            f"[{min(ks)}, {max(ks)}], sum {sum(ks)}")
    bt = K.Batch(P, d, Z, n, k=ks, scale=b["scale"])
    ws = torch.empty(K.workspace_bytes(bt, o), dtype=torch.uint8, device=dev)
    Kc = torch.empty((sum(ks), d), dtype=torch.float32, device=dev)
    Vc = torch.empty_like(Kc)
    t_b = time.perf_counter()
    K.kvs_compress_begin(ctx, bt, o, Q, Kz, Vz, 0, Kc, Vc, l0, ws)
    torch.cuda.synchronize()
    t_begin = time.perf_counter() - t_b
    log(f"[bench] reference attention + Select+Fit at the new k: {t_begin:.2f} s; main run: "
        f"{nblk} blocks of {VC} (warmup {W}, timed {Kst})")
    t_timed = t_latency = None
    stats = None
    for i in range(nblk):
        if i == W:
            torch.cuda.synchronize()
            K.kvs_profile_enable(ctx, True, kernels=TIMED_KERNELS)
            t1 = time.perf_counter()
        K.kvs_compress_advance(ctx, bt, o, Q, VC * i, VC * (i + 1), Kc, Vc, loss, mse, flags, ws)
        if i == W + Kst - 1:
            torch.cuda.synchronize()
            t_timed = time.perf_counter() - t1
            stats = K.kvs_profile_read(ctx)
            K.kvs_profile_enable(ctx, False)
        if i == nblk_T - 1:
            torch.cuda.synchronize()
            t_latency = time.perf_counter() - t_start
        if i % 5 == 4 or i == nblk - 1:
            log(f"[bench] block {i + 1}/{nblk} done ({time.perf_counter() - t_start:.1f} s since the "
                f"pilot started)")
    torch.cuda.synchronize()
    lg, l0g, fg = loss.cpu().numpy(), l0.cpu().numpy(), flags.cpu().numpy()
    log(f"[bench] final/start loss ratio: median {np.median(lg / l0g):.4f} min {np.min(lg / l0g):.4f} "
        f"max {np.max(lg / l0g):.4f}; flagged problems {int(np.count_nonzero(fg))}")

    value = P * VC * Kst / t_timed
    rows = kernel_rows(stats)
    name = max((k for k in rows if k in CONTRACTIONS), key=lambda k: rows[k]["ms"])
    st = stats[name]
    avg_s = st["ms"] / st["launches"] / 1e3
    fl_launch = st["flops"] / st["launches"]
    achieved = fl_launch / avg_s
    if name == "attn_fwd":
        peak = mixed_fwd_peak()
        peak_note = {"fp64": "harmonic mix of the fp64 (scores) and fp32 (A Vc) MFMA peaks",
                     "fp32": "fp32 MFMA",
                     "int8": f"harmonic mix of the int8 MFMA peak over {INT8_PRODUCTS} digit products "
                             f"(scores) and the fp32 MFMA peak (A Vc)"}[logit_mode()]
    else:
        peak, peak_note = contraction_peak(name)
    tot_ms = sum(r["ms"] for r in rows.values())
    for k2, r in sorted(rows.items(), key=lambda kv: -kv[1]["ms"]):
        log(f"[bench] {k2:12s} launches={r['launches']:6d} ms={r['ms']:10.2f} avg_us={r['avg_us']:9.1f} "
            + " ".join(f"{kk}={vv}" for kk, vv in r.items() if kk.startswith(("tflops", "frac"))))
    roofline = {"bound": "mfma", "achieved": round(achieved / 1e12, 3), "peak": round(peak / 1e12, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic_for(name, w.name if args.ratio is None else None),
                "kernel": name, "peak_kind": peak_note, "launches": st["launches"],
                "avg_us": round(avg_s * 1e6, 2),
                "timed": f"HIP events on the library stream around every launch of the timed "
                         f"kernels during the {Kst} timed blocks ({tot_ms / Kst:.1f} ms of "
                         f"event-timed kernels per {1e3 * t_timed / Kst:.1f} ms step)"}
    # HBM rate of the L-BFGS vector passes and the merge (measured bytes per
    # dispatch over the event-timed average)
    vec = {}
    for nm in ("hist_dots", "direction", "merge"):
        r = rows.get(nm)
        if not r:
            continue
        bts = traffic_for(nm, w.name if args.ratio is None else None)
        e = {"launches": r["launches"], "avg_us": r["avg_us"], "bytes_per_launch": bts}
        if bts:
            rate = bts / (r["avg_us"] * 1e-6)
            e["GB/s"] = round(rate / 1e9, 1)
            e["frac_hbm"] = round(rate / PEAK_HBM, 4)
        vec[nm] = e
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host")
        cpu = cpu_baseline_block(w, b)
    out = {
        "metric": "KVSculpt L-BFGS iterations/sec over all layer×KV-head problems; % fp32 MFMA",
        "value": round(value, 2), "unit": "problem-iterations/s", "n_gpus": 1,
        "steps": Kst, "warmup": W, "ms_per_step": round(1e3 * t_timed / Kst, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "problems": P, "d": d, "n": n, "Z": Z, "k0": w.k0,
                   "k_range": [int(min(ks)), int(max(ks))], "k_total": int(sum(ks)),
                   "iters": T, "vc_every": VC, "history": 10, "pilot": pilot,
                   "step": f"one block of {VC} L-BFGS iterations of all {P} problems with the value "
                           f"re-solve and loss/gradient after it (main run at the pilot's ragged k)",
                   "logits": LOGIT_NOTES[logit_mode()], "contractions": contractions_note(stats)},
        "latency": {"whole_model_compress_s": round(t_latency, 3), "pilot_and_allocation_s": round(t_pilot, 3),
                    "reference_and_select_fit_s": round(t_begin, 3),
                    "note": f"pilot ({pilot} iterations at k0) + reallocation + reference attention + "
                            f"Select+Fit at the new k + {T} main-run iterations, wall clock, inputs in HBM"},
        "kernels": rows,
        "roofline": roofline,
        "vector_phases": {"kernels": vec, "peak_GB/s": PEAK_HBM / 1e9,
                          "bytes": "HBM bytes per dispatch measured by FETCH_SIZE / WRITE_SIZE over the timed "
                                   "blocks (copy-calibrated; null once the kernel source changed); these "
                                   "kernels stream each operand once"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (compress: blocks of 5 iterations, default 20; other rows: 5)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (compress 5, others 1)")
    ap.add_argument("--config", type=int, default=None,
                    help="workload (compress: default 4, the long-context cache; 2 for the "
                         "queries / use / solve / alloc rows)")
    ap.add_argument("--ratio", type=float, default=None, help="compression ratio r (configs 2..4)")
    ap.add_argument("--iters", type=int, default=None, help="override T (profiling runs only)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row", choices=["compress", "queries", "use", "solve", "adam", "restarts",
                                      "alloc", "vector"],
                    default="compress",
                    help="compress: the optimizer (default); queries: training-query "
                         "construction; use: use-side evaluation; solve: the standalone "
                         "ridge value solve; adam / restarts: the "
                         "optimizer ablations; alloc: allocation variants; vector: the "
                         "schedule on a 64-problem llama3-8b slice (vector-kernel sizing)")
    ap.add_argument("--adam-lr", type=float, default=1e-2)
    ap.add_argument("--restarts", type=int, default=100)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run plain device copies of this size (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.config is None:
        args.config = {"compress": 4, "adam": 1, "restarts": 1, "vector": 3}.get(args.row, 2)
    if args.steps is None:
        args.steps = 20 if args.row == "compress" else 5
    if args.warmup is None:
        args.warmup = 5 if args.row == "compress" else 1
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU: the problems of a batch are independent and the library "
            "runs them all on a single MI355X; multi-GPU runs are not supported (use --gpus 1).")
        sys.exit(2)

    import torch
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
        return
    import attention_distillation_amd as K
    from synth import WORKLOADS, make_batch
    if args.row == "queries":
        bench_queries(args, torch, K)
        return
    if args.row == "use":
        bench_use(args, torch, K)
        return
    if args.row == "solve":
        bench_solve(args, torch, K)
        return
    if args.row == "adam":
        bench_adam(args, torch, K)
        return
    if args.row == "restarts":
        bench_restarts(args, torch, K)
        return
    if args.row == "alloc":
        bench_alloc(args, torch, K)
        return
    if args.row == "vector":
        bench_vector(args, torch, K)
        return

    bench_compress(args, torch, K)


if __name__ == "__main__":
    main()
