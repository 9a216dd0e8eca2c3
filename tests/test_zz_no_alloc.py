"""The allocation-free entry point kvs_value_norms_noalloc (its scratch is a
static device array, no workspace argument, nothing allocated) against
kvs_value_norms with a caller workspace: the same kernels, so the same bits.
Two calls in a row, the second with a smaller batch (the array keeps the
first call's partials; each call writes every partial it reads).  The
result is also within 1e-12 of the oracle's float64 value-norm signal."""
import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from tests.gpu_common import host, say, to_gpu, torch_dev, workspace

pytestmark = pytest.mark.gpu


def test_noalloc_value_norms_equals_workspace_call():
    torch, dev = torch_dev()
    ctx = K.Context()
    rng = np.random.default_rng(17)
    for P, Z, d in ((256, 2000, 128), (7, 333, 64)):
        say(f"[noalloc] value norms P={P} Z={Z} d={d}")
        V = (rng.standard_normal((P, Z, d)) * np.exp(rng.normal(0, 1, (P, 1, 1)))).astype(np.float32)
        Vg = to_gpu(V)
        a = torch.full((P,), float("nan"), dtype=torch.float64, device=dev)
        b = torch.full((P,), float("nan"), dtype=torch.float64, device=dev)
        ws = workspace(K.value_norms_workspace_bytes(P, Z))
        K.kvs_value_norms(ctx, P, Z, d, Vg, a, ws)
        K.kvs_value_norms_noalloc(ctx, P, Z, d, Vg, b)
        ha, hb = host(a), host(b)
        assert ha.tobytes() == hb.tobytes()
        want = np.array([O.value_norm_signal(V[p]) for p in range(P)])
        err = float(np.max(np.abs(hb - want) / want))
        say(f"   bit-identical to the workspace call; max rel err vs oracle {err:.2e}")
        assert err <= 1e-12
    with pytest.raises(K.KvsError):
        K.kvs_value_norms_noalloc(ctx, 200000, 64, 64, Vg, b)
