"""GPU parity of the allocation variants through the C ABI.

- kvs_value_norms: within 1e-12 relative of the oracle's float64 mean row
  norm.  Both sides accumulate the same float32 values in float64, in
  different orders.
- The static allocation (kvs_allocate_budget, alpha = 1, on the device
  signal) equals the oracle allocator fed the oracle's signal, integer for
  integer.
The two-level split is pure host code, checked bit for bit against the
oracle in the CPU suite.
"""
import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from synth import WORKLOADS, make_batch, tiny_workload
from tests.gpu_common import host, say, to_gpu, workspace

pytestmark = pytest.mark.gpu


def _norms_gpu(Vz):
    import torch
    P, Z, d = Vz.shape
    out = torch.full((P,), float("nan"), dtype=torch.float64, device="cuda:0")
    ws = workspace(K.value_norms_workspace_bytes(P, Z))
    K.kvs_value_norms(K.Context(), P, Z, d, to_gpu(Vz), out, ws)
    return host(out)


CASES = {
    "qwen-full-cache": (WORKLOADS[2], None),
    "tiny-d64-short-zone": (tiny_workload(d=64, N=40, m=8, g=1, F=4, layers=3, kv_heads=2), None),
    "long-context-2-problems": (WORKLOADS[4], [0, 57]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_value_norms_match_oracle(name):
    w, probs = CASES[name]
    b = make_batch(w, 0, probs)
    P, Z, d = b["Vz"].shape
    say(f"[value-norms] case={name} P={P} Z={Z} d={d}")
    got = _norms_gpu(b["Vz"])
    want = np.array([O.value_norm_signal(b["Vz"][p]) for p in range(P)])
    err = np.abs(got - want) / want
    say(f"   max relative error {err.max():.2e}")
    assert err.max() <= 1e-12


def test_static_allocation_from_the_device_signal():
    w = WORKLOADS[2]
    b = make_batch(w, 0)
    P = b["Vz"].shape[0]
    sig = _norms_gpu(b["Vz"])
    want_sig = [O.value_norm_signal(b["Vz"][p]) for p in range(P)]
    K_total = w.k0 * P
    got = K.kvs_allocate_budget(sig, K_total, 1.0, 1, w.Z)
    want = O.allocate_budget(want_sig, K_total, 1.0, 1, w.Z)
    say(f"[value-norms] static allocation k in [{got.min()}, {got.max()}], sum {got.sum()}")
    assert got.tolist() == want
