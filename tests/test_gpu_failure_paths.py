"""GPU failure paths and run-to-run determinism, through the C ABI.

- A NaN value row (an input value only: every index and size stays valid)
  makes one problem's reference output NaN.  Its flags must equal the
  oracle's (non-finite at the start, then every search fails), its keys stay
  at the Select+Fit choice, and the other problem of the batch is untouched.
- Armijo constant 0.999 with a single trial per search: the first trial of
  every iteration is rejected (by a margin of about 2% of the loss on the
  single-head workload, far above float32 rounding), so every search fails.
  This runs the failed-search branch of the device schedule (no move,
  history cleared, flag 4, the re-forward before each value solve of a
  problem whose last search failed).  Flags, keys and loss against the
  oracle under the same options.
- kvs_compress and kvs_pilot_allocate run twice on the same inputs give the
  same bits (fixed-order reductions, no float atomics).
"""
import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from synth import WORKLOADS, make_batch
from tests.gpu_common import empty, host, say, to_gpu, workspace

pytestmark = pytest.mark.gpu


def _run_compress(b, ks, o, Vz=None):
    P, n, d = b["Q"].shape
    Z = b["Kz"].shape[1]
    bt = K.Batch(P, d, Z, n, k=ks, scale=b["scale"])
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt, o))
    kt = sum(ks)
    Kc, Vc = empty((kt, d)), empty((kt, d))
    loss, mse, l0 = empty((P,)), empty((P,)), empty((P,))
    flags = to_gpu(np.zeros(P, np.int32))
    K.kvs_compress(ctx, bt, o, to_gpu(b["Q"]), to_gpu(b["Kz"]), to_gpu(b["Vz"] if Vz is None else Vz),
                   Kc, Vc, loss, mse, l0, flags, ws)
    return dict(Kc=host(Kc), Vc=host(Vc), loss=host(loss), mse=host(mse), l0=host(l0), flags=host(flags))


def test_nonfinite_value_row_flags_match_oracle():
    w = WORKLOADS[0]
    b = make_batch(w, 0)
    # two copies of the single-head problem; the second gets one NaN value row
    b2 = {"Q": np.concatenate([b["Q"], b["Q"]]), "Kz": np.concatenate([b["Kz"], b["Kz"]]),
          "Vz": np.concatenate([b["Vz"], b["Vz"]]), "scale": b["scale"]}
    Vz = b2["Vz"].copy()
    Vz[1, 7, :] = np.nan
    T = 10
    say(f"[nonfinite] two single-head problems, NaN in problem 1's value row 7, T={T}")
    g = _run_compress(b2, [w.k0, w.k0], K.opts(iters=T), Vz=Vz)
    opt = O.CompressOptions(iters=T)
    r0 = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], w.k0, b["scale"], opt)
    r1 = O.compress_problem(b["Q"][0], b["Kz"][0], Vz[1], w.k0, b["scale"], opt)
    say(f"   flags gpu={g['flags'].tolist()} oracle={[r0['flags'], r1['flags']]}; "
        f"loss gpu={g['loss'].tolist()} oracle={[r0['loss'], r1['loss']]}")
    assert g["flags"].tolist() == [r0["flags"], r1["flags"]] == [0, K.KVS_FLAG_NONFINITE | K.KVS_FLAG_LINESEARCH]
    assert abs(g["loss"][0] - r0["loss"]) <= 0.02 * r0["loss"]
    assert np.isnan(g["loss"][1]) and np.isnan(g["l0"][1])
    np.testing.assert_array_equal(g["Kc"][w.k0:], b["Kz"][0][r1["idx"]])
    assert np.all(np.isfinite(g["Kc"][:w.k0])) and np.all(np.isfinite(g["Vc"][:w.k0]))


def test_forced_line_search_failure_matches_oracle():
    w = WORKLOADS[0]
    b = make_batch(w, 0)
    T = 10
    o = K.opts(iters=T, max_backtracks=1, c1=0.999)
    say(f"[line-search failure] single-head, c1=0.999, one trial per search, T={T}")
    g = _run_compress(b, [w.k0], o)
    opt = O.CompressOptions(iters=T, lbfgs=O.LbfgsOptions(c1=0.999, max_backtracks=1))
    r = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], w.k0, b["scale"], opt, record=True)
    say(f"   flags gpu={g['flags'][0]} oracle={r['flags']}; init gpu={g['l0'][0]:.7g} oracle="
        f"{r['init_loss']:.7g}; final gpu={g['loss'][0]:.7g} oracle={r['loss']:.7g}")
    assert r["flags"] == K.KVS_FLAG_LINESEARCH and g["flags"][0] == K.KVS_FLAG_LINESEARCH
    assert all(v == r["init_loss"] for v in r["traj"])        # the oracle never moves either
    np.testing.assert_array_equal(g["Kc"], b["Kz"][0][r["idx"]])
    assert abs(g["l0"][0] - r["init_loss"]) <= 1e-4 * r["init_loss"]
    # the value re-solves at unmoved keys reproduce the start's values
    assert abs(g["loss"][0] - g["l0"][0]) <= 1e-5 * g["l0"][0]


def test_compress_runs_twice_bitwise():
    w = WORKLOADS[1]
    b = make_batch(w, 0)
    o = K.opts(iters=20)
    say("[determinism] qwen2.5-1.5b-one-layer kvs_compress T=20, twice")
    a = _run_compress(b, [w.k0] * 2, o)
    c = _run_compress(b, [w.k0] * 2, o)
    for key in a:
        assert a[key].tobytes() == c[key].tobytes(), key


def test_pilot_runs_twice_bitwise():
    w = WORKLOADS[2]
    b = make_batch(w, 0)
    P, n, d = b["Q"].shape
    Z = b["Kz"].shape[1]
    pilot = 60
    o = K.opts(iters=pilot)
    bt = K.Batch(P, d, Z, n, k=[w.k0] * P, scale=b["scale"])
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt, o))
    Q, Kz, Vz = to_gpu(b["Q"]), to_gpu(b["Kz"]), to_gpu(b["Vz"])
    say(f"[determinism] {w.name} pilot ({P} problems, k={w.k0}, {pilot} iterations), twice")
    out = []
    for _ in range(2):
        pm = empty((P,))
        k_out = K.kvs_pilot_allocate(ctx, bt, o, pilot, 0.5, 1, Z, Q, Kz, Vz, pm, ws)
        out.append((host(pm).tobytes(), list(k_out)))
    assert out[0] == out[1]
