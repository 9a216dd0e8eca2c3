"""Write oracle-only expected values for the long end-to-end GPU checks.

Every number stored here comes from ``oracle/`` (float64) run on the seeded
synthetic inputs of ``synth``; nothing is read from the GPU path.

    python tests/golden/make_golden.py qwen2.5-1.5b-one-layer    # 300 iterations
    python tests/golden/make_golden.py states     # one-layer iterates at t = 5 and t = 300
    python tests/golden/make_golden.py pilot      # full-cache pilot, r = 0.3 / 0.5 / 0.7
    python tests/golden/make_golden.py e2e-llama  # llama3-8b problem 0, k = 2381 and 4680
    python tests/golden/make_golden.py e2e-long   # long-context problem 0, k = 3226
    python tests/golden/make_golden.py e2e-ragged # llama3-8b, 8 seeded problems at ragged k

The pilot set runs its 168 problems in a process pool (one BLAS thread each).
Each run is stored with the final loss of the same schedule run with its
keys kept at float32 (the oracle's sensitivity variant); ``--reuse`` keeps
the plain runs of an existing file and computes only those.
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import kvsculpt as O  # noqa: E402
from synth import WORKLOADS, make_batch  # noqa: E402


def golden_compress(cid: int, iters: int | None = None, seed: int = 0):
    w = WORKLOADS[cid]
    b = make_batch(w, seed)
    T = w.T if iters is None else iters
    opt = O.CompressOptions(iters=T)
    out = {"config": cid, "workload": w.name, "seed": seed, "iters": T, "k": w.k0, "problems": []}
    for p in range(b["Q"].shape[0]):
        t0 = time.time()
        r = O.compress_problem(b["Q"][p], b["Kz"][p], b["Vz"][p], w.k0, b["scale"], opt, record=True)
        out["problems"].append({
            "p": p, "init_loss": r["init_loss"], "final_loss": r["loss"], "mse": r["mse"],
            "flags": r["flags"], "idx": [int(i) for i in r["idx"]],
            "traj": [float(v) for v in r["traj"]], "seconds": time.time() - t0})
        print(f"{w.name} problem {p}: {r['init_loss']:.6g} -> {r['loss']:.6g} "
              f"({time.time() - t0:.1f} s)", flush=True)
    return out


def golden_states(seed: int = 0, stops=(5, 300)):
    """The oracle's iterates (Kc, Vc) of both one-layer problems after t
    iterations of the schedule, rounded to float32 (the per-call parity
    tests feed them to both sides), with the oracle's loss there."""
    import numpy as np
    w = WORKLOADS[1]
    b = make_batch(w, seed)
    arrays, meta = {}, {"workload": w.name, "seed": seed, "k": w.k0, "stops": list(stops), "loss": {}}
    for p in range(b["Q"].shape[0]):
        for t in stops:
            t0 = time.time()
            r = O.compress_problem(b["Q"][p], b["Kz"][p], b["Vz"][p], w.k0, b["scale"],
                                   O.CompressOptions(iters=t))
            arrays[f"Kc_t{t}_p{p}"] = r["Kc"].astype(np.float32)
            arrays[f"Vc_t{t}_p{p}"] = r["Vc"].astype(np.float32)
            meta["loss"][f"t{t}_p{p}"] = r["loss"]
            print(f"{w.name} p={p} t={t}: loss {r['loss']:.6g} ({time.time() - t0:.1f} s)", flush=True)
    return arrays, meta


def _pilot_one(args):
    ratio, p, seed, plain = args
    w = WORKLOADS[2].with_ratio(ratio)
    b = make_batch(w, seed, problems=[p])
    Y, l = O.reference_attention(b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"])
    r32 = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], w.k0, b["scale"],
                             O.CompressOptions(iters=w.pilot, keys_f32=True), Y=Y, lse=l)
    if plain is not None:
        return ratio, p, plain[0], plain[1], plain[2], r32["loss"]
    r = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], w.k0, b["scale"],
                           O.CompressOptions(iters=w.pilot), Y=Y, lse=l)
    return ratio, p, r["mse"], r["flags"], r["loss"], r32["loss"]


def golden_pilot(seed: int = 0, ratios=(0.3, 0.5, 0.7), workers: int = 6, previous=None):
    """The oracle's 60-iteration pilot on every full-cache problem at each
    ratio: final loss and output MSE per problem, the oracle's own
    allocation, and the final loss of the same run with its keys kept at
    float32 (the sensitivity variant).  ``previous``: a stored result whose
    plain runs are reused (only the float32-key runs are computed)."""
    import concurrent.futures as cf
    w0 = WORKLOADS[2]
    def plain(r, p):
        if previous is None:
            return None
        g = previous["ratios"][str(r)]
        return (g["mse"][p], g["flags"][p], g["loss"][p])
    jobs = [(r, p, seed, plain(r, p)) for r in ratios for p in range(w0.P)]
    res = {}
    with cf.ProcessPoolExecutor(workers) as ex:
        for i, (r, p, mse, fl, loss, loss32) in enumerate(ex.map(_pilot_one, jobs)):
            res[(r, p)] = (mse, fl, loss, loss32)
            if i % 8 == 7:
                print(f"pilot {i + 1}/{len(jobs)}", flush=True)
    out = {"workload": w0.name, "seed": seed, "pilot_iters": w0.pilot, "alpha": 0.5, "ratios": {}}
    for r in ratios:
        w = w0.with_ratio(r)
        mse = [res[(r, p)][0] for p in range(w.P)]
        ks = O.allocate_budget(mse, w.k0 * w.P, 0.5, 1, w.Z)
        out["ratios"][str(r)] = {"k0": w.k0, "mse": mse, "flags": [res[(r, p)][1] for p in range(w.P)],
                                 "loss": [res[(r, p)][2] for p in range(w.P)],
                                 "loss_f32keys": [res[(r, p)][3] for p in range(w.P)], "k": ks}
    return out


def golden_e2e(cid: int, p: int, ks, seed: int = 0, previous=None):
    """The oracle's whole schedule (Select+Fit, T iterations) on one problem
    of a large workload at each given k, and the final loss of the same run
    with its keys kept at float32.  ``previous``: a stored result whose plain
    runs are reused."""
    w = WORKLOADS[cid]
    b = make_batch(w, seed, problems=[p])
    Y, l = O.reference_attention(b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"])
    out = {"workload": w.name, "seed": seed, "problem": p, "iters": w.T, "runs": []}
    for k in ks:
        t0 = time.time()
        old = next((x for x in (previous or {}).get("runs", []) if x["k"] == k), None)
        if old is None:
            r = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], k, b["scale"],
                                   O.CompressOptions(iters=w.T), Y=Y, lse=l, record=True)
            old = {"k": k, "init_loss": r["init_loss"], "final_loss": r["loss"], "mse": r["mse"],
                   "flags": r["flags"], "traj": [float(v) for v in r["traj"]], "seconds": time.time() - t0}
        r32 = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], k, b["scale"],
                                 O.CompressOptions(iters=w.T, keys_f32=True), Y=Y, lse=l)
        old["final_loss_f32keys"] = r32["loss"]
        out["runs"].append(old)
        r = {"init_loss": old["init_loss"], "loss": old["final_loss"]}
        print(f"{w.name} p={p} k={k}: {r['init_loss']:.6g} -> {r['loss']:.6g} (float32 keys "
              f"{old['final_loss_f32keys']:.6g}; {time.time() - t0:.1f} s)", flush=True)
    return out


def ragged_budgets(P: int, lo: int, hi: int, seed: int):
    """Seeded ragged budgets, log-uniform in [lo, hi]: test inputs with the
    spread a reallocation produces (on the llama3-8b cache the pilot hands out
    about 700 to 4700 pairs), independent of either side's pilot."""
    import numpy as np
    rng = np.random.default_rng(np.random.SeedSequence([seed, 8317]))
    return [int(round(float(np.exp(v)))) for v in rng.uniform(np.log(lo), np.log(hi), size=P)]


def _ragged_one(args):
    cid, p, k, seed, f32 = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        w = WORKLOADS[cid]
        b = make_batch(w, seed, problems=[p])
        t0 = time.time()
        r = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], k, b["scale"],
                               O.CompressOptions(iters=w.T, keys_f32=f32))
        return p, f32, r["init_loss"], r["loss"], r["flags"], time.time() - t0


def golden_ragged(cid: int = 3, seed: int = 0, nsample: int = 8, workers: int = 8):
    """The oracle's whole schedule (Select+Fit at the problem's budget, T
    iterations) on a seeded sample of problems of a large workload whose
    problems all have seeded ragged budgets, plain and with the keys kept at
    float32 (the sensitivity variant)."""
    import concurrent.futures as cf
    import numpy as np
    w = WORKLOADS[cid]
    ks = ragged_budgets(w.P, 700, 4680, seed)
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4471]))
    sample = sorted(int(p) for p in rng.choice(w.P, size=nsample, replace=False))
    jobs = [(cid, p, ks[p], seed, f32) for p in sample for f32 in (False, True)]
    res = {}
    with cf.ProcessPoolExecutor(workers) as ex:
        for p, f32, l0, loss, flags, sec in ex.map(_ragged_one, jobs):
            res[(p, f32)] = (l0, loss, flags)
            print(f"{w.name} p={p} k={ks[p]} {'float32 keys' if f32 else 'float64'}: {l0:.6g} -> {loss:.6g} "
                  f"({sec:.0f} s)", flush=True)
    runs = [{"p": p, "k": ks[p], "init_loss": res[(p, False)][0], "final_loss": res[(p, False)][1],
             "flags": res[(p, False)][2], "final_loss_f32keys": res[(p, True)][1]} for p in sample]
    return {"workload": w.name, "seed": seed, "iters": w.T, "k": ks, "runs": runs}


if __name__ == "__main__":
    name = sys.argv[1] if len(sys.argv) > 1 else "qwen2.5-1.5b-one-layer"
    if name == "states":
        import numpy as np
        arrays, meta = golden_states()
        np.savez_compressed(os.path.join(HERE, "oracle_states_qwen2.5-1.5b-one-layer.npz"), **arrays)
        with open(os.path.join(HERE, "oracle_states_qwen2.5-1.5b-one-layer.json"), "w") as f:
            json.dump(meta, f, indent=1)
        sys.exit(0)
    reuse = "--reuse" in sys.argv
    if name == "pilot":
        path = os.path.join(HERE, "oracle_pilot_qwen2.5-1.5b-full-cache.json")
        res = golden_pilot(previous=json.load(open(path)) if reuse else None)
        with open(os.path.join(HERE, "oracle_pilot_qwen2.5-1.5b-full-cache.json"), "w") as f:
            json.dump(res, f, indent=1)
        sys.exit(0)
    if name in ("e2e-llama", "e2e-long"):
        cid, ks = (3, [2381, 4680]) if name == "e2e-llama" else (4, [3226])
        path = os.path.join(HERE, f"oracle_compress_{WORKLOADS[cid].name}_p0.json")
        res = golden_e2e(cid, 0, ks, previous=json.load(open(path)) if reuse else None)
        with open(os.path.join(HERE, f"oracle_compress_{WORKLOADS[cid].name}_p0.json"), "w") as f:
            json.dump(res, f, indent=1)
        sys.exit(0)
    if name == "e2e-ragged":
        res = golden_ragged()
        with open(os.path.join(HERE, f"oracle_compress_{WORKLOADS[3].name}_ragged.json"), "w") as f:
            json.dump(res, f, indent=1)
        sys.exit(0)
    cid = next(c for c, w in WORKLOADS.items() if w.name == name)
    res = golden_compress(cid)
    path = os.path.join(HERE, f"oracle_compress_{name}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print("wrote", path)
