"""GPU parity: training-query construction through the C ABI.

Bar: retain rows are bit-exact copies.  Each element of a future row lies
within 1e-6 of the float64 oracle, relative to the norm of its channel
plane.  The device turns each plane once, in float32, after reducing the
angle in float64.  The error budget is:
  * the reduced angle rounded to float32: <= 2.4e-7 rad at |r| <= pi;
  * float32 sine and cosine: ~1e-7;
  * the two products and their sum: <= 3 float32 roundings, ~1.8e-7 of the
    plane norm.
Together that is <= 6e-7 of the plane norm.
"""
import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from synth import WORKLOADS, make_context_batch, tiny_workload
from tests.gpu_common import empty, host, rel, say, to_gpu, workspace

pytestmark = pytest.mark.gpu
PLANE_TOL = 1e-6


def _cases():
    return {
        "single-head-d64": (WORKLOADS[0], None),
        "qwen-one-layer-d128": (WORKLOADS[1], None),
        "long-context-d128": (WORKLOADS[4], [0]),
        "tiny-d8": (tiny_workload(d=8, N=40, m=8, g=2, F=6, layers=2, kv_heads=2), None),
        "tiny-d256-ragged": (tiny_workload(d=256, N=70, m=3, g=5, F=13, layers=1, kv_heads=3),
                             None),
    }


def _build_gpu(w, b, src=None, flags=None):
    P, g, N, d = b["Qctx"].shape
    F = b["src"].shape[2]
    ctx = K.Context()
    Q = empty((P, g * (w.m + F), d))
    K.kvs_build_queries(ctx, P, g, N, w.m, F, d, w.theta, to_gpu(b["Qctx"]),
                        to_gpu(b["src"] if src is None else src), Q, flags)
    return host(Q)


def _check(w, b, Qg, p):
    g, N, d = b["Qctx"].shape[1:]
    m, F = w.m, b["src"].shape[2]
    Qo = O.training_queries(b["Qctx"][p], b["src"][p], m, w.theta)
    assert np.array_equal(Qg[p, :g * m], b["Qctx"][p, :, N - m:].reshape(g * m, d))
    h = d // 2
    fut_o, fut_g = Qo[g * m:], Qg[p, g * m:].astype(np.float64)
    plane = np.hypot(fut_o[:, :h], fut_o[:, h:])
    plane = np.concatenate([plane, plane], axis=1)
    err = np.abs(fut_g - fut_o) / np.maximum(plane, 1e-30)
    worst = float(err.max()) if err.size else 0.0
    say(f"   p={p} worst plane-relative error {worst:.2e}  rel={rel(fut_g, fut_o):.2e}")
    assert worst <= PLANE_TOL


@pytest.mark.parametrize("name", list(_cases()))
def test_build_queries_matches_oracle(name):
    w, probs = _cases()[name]
    b = make_context_batch(w, 0, probs)
    P, g, N, d = b["Qctx"].shape
    say(f"[queries] case={name} P={P} g={g} N={N} m={w.m} F={w.F} d={d} theta={w.theta:g}")
    Qg = _build_gpu(w, b)
    for p in range(P):
        _check(w, b, Qg, p)


def test_invalid_source_gives_zero_row_and_flag():
    w = tiny_workload(d=64, N=50, m=5, g=2, F=7, layers=1, kv_heads=3)
    b = make_context_batch(w, 1)
    src = b["src"].copy()
    src[1, 0, 3] = w.N          # one past the context
    src[2, 1, 6] = -1
    say("[queries] invalid sources at (p=1, h=0, j=3) and (p=2, h=1, j=6)")
    flags = to_gpu(np.zeros(3, dtype=np.int32))
    Qg = _build_gpu(w, b, src=src, flags=flags)
    assert host(flags).tolist() == [0, K.KVS_FLAG_BADINDEX, K.KVS_FLAG_BADINDEX]
    g, m, F = 2, w.m, w.F
    bad = {(1, g * m + 0 * F + 3), (2, g * m + 1 * F + 6)}
    for p, r in bad:
        assert not Qg[p, r].any()
    good = dict(b)
    good["src"] = np.where(src < 0, 0, np.where(src >= w.N, 0, src))
    for p in range(3):
        Qo = O.training_queries(b["Qctx"][p], good["src"][p], m, w.theta)
        for r in range(Qo.shape[0]):
            if (p, r) in bad:
                continue
            np.testing.assert_allclose(Qg[p, r], Qo[r], rtol=0, atol=2e-6 * np.abs(Qo[r]).max())


def test_built_queries_drive_reference_attention():
    """The built queries feed the path unchanged: the compress zone's reference
    attention from device-built queries matches the oracle's from its own."""
    w = WORKLOADS[1]
    b = make_context_batch(w, 2)
    P, g, N, d = b["Qctx"].shape
    say(f"[queries->ref-attn] P={P} n={g * (w.m + w.F)} Z={w.Z} d={d}")
    ctx = K.Context()
    n = g * (w.m + w.F)
    Q = empty((P, n, d))
    K.kvs_build_queries(ctx, P, g, N, w.m, w.F, d, w.theta, to_gpu(b["Qctx"]), to_gpu(b["src"]),
                        Q, None)
    bt = K.Batch(P, d, w.Z, n)
    ws = workspace(K.workspace_bytes(bt))
    Y, lse = empty((P, n, d)), empty((P, n))
    K.kvs_reference_attn(ctx, bt, Q, to_gpu(b["Kz"]), to_gpu(b["Vz"]), Y, lse, ws)
    Yg, lg = host(Y), host(lse)
    for p in range(P):
        Qo = O.training_queries(b["Qctx"][p], b["src"][p], w.m, w.theta)
        Yo, lo = O.reference_attention(Qo.astype(np.float32), b["Kz"][p], b["Vz"][p], b["scale"])
        ey, el = rel(Yg[p], Yo), rel(lg[p], lo)
        say(f"   p={p} relY={ey:.2e} rel_lse={el:.2e}")
        assert ey <= 1e-4 and el <= 1e-4


def test_degenerate_query_shapes():
    """No synthetic queries (src NULL) and no retain queries."""
    import torch
    rng = np.random.default_rng(9)
    P, g, N, d = 3, 2, 37, 64
    Qctx = rng.standard_normal((P, g, N, d)).astype(np.float32)
    ctx = K.Context()
    # F = 0: the retain block only, bit-exact copies
    Q = empty((P, g * 5, d))
    say("[queries] degenerate F=0 (src NULL), m=5")
    K.kvs_build_queries(ctx, P, g, N, 5, 0, d, 1e4, to_gpu(Qctx), None, Q, None)
    Qg = host(Q)
    for p in range(P):
        assert np.array_equal(Qg[p], Qctx[p, :, N - 5:].reshape(-1, d))
    # m = 0: the future block only, one source per head at the first and last position
    src = np.zeros((P, g, 2), dtype=np.int32)
    src[:, :, 1] = N - 1
    Q = empty((P, g * 2, d))
    say("[queries] degenerate m=0, sources 0 and N-1")
    K.kvs_build_queries(ctx, P, g, N, 0, 2, d, 1e4, to_gpu(Qctx), to_gpu(src), Q, None)
    Qg = host(Q).astype(np.float64)
    for p in range(P):
        Qo = O.training_queries(Qctx[p], src[p], 0, 1e4)
        assert np.abs(Qg[p] - Qo).max() <= 1e-6 * np.abs(Qo).max()
    torch.cuda.synchronize()
