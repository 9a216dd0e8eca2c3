"""Write oracle-only expected values for the long end-to-end GPU checks.

Every number stored here comes from ``oracle/`` (float64) run on the seeded
synthetic inputs of ``synth``; nothing is read from the GPU path.

    python tests/golden/make_golden.py qwen2.5-1.5b-one-layer    # 300 iterations
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


if __name__ == "__main__":
    name = sys.argv[1] if len(sys.argv) > 1 else "qwen2.5-1.5b-one-layer"
    cid = next(c for c, w in WORKLOADS.items() if w.name == name)
    res = golden_compress(cid)
    path = os.path.join(HERE, f"oracle_compress_{name}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print("wrote", path)
