"""Host-side checks of the C ABI (no GPU): exports, argument errors, allocator."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import kvsculpt as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    import attention_distillation_amd as K
    K.load()
    return K


def _declared():
    text = open(os.path.join(ROOT, "include", "kvsculpt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point(K):
    names = _declared()
    assert len(names) >= 16
    lib = ctypes.CDLL(K._lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(K.ENTRY_POINTS) == set(names)


def test_workspace_and_state_sizes(K):
    b = K.Batch(2, 128, 1920, 3840, k=[960, 960])
    o = K.opts()
    ws = K.workspace_bytes(b, o)
    st = K.lbfgs_state_bytes(b, o)
    # stored scores alone are k * n floats per problem
    assert ws > 2 * 960 * 3840 * 4
    assert st >= 2 * (2 + 2 * 11) * 960 * 128 * 4
    bad = K.Batch(2, 96, 1920, 3840, k=[960, 960])   # d must be 64 or 128
    assert K.workspace_bytes(bad, o) == 0
    bad2 = K.Batch(2, 128, 100, 64, k=[10, 101])     # k > Z
    assert K.workspace_bytes(bad2, o) == 0
    # n past 2^21: tile rows are addressed with 32-bit byte ranges and offsets
    assert K.workspace_bytes(K.Batch(1, 128, 100, 1 << 21, k=[10]), o) > 0
    assert K.workspace_bytes(K.Batch(1, 128, 100, (1 << 21) + 1, k=[10]), o) == 0


def test_argument_errors_are_reported_before_any_launch(K):
    lib = K.load()
    ctx = ctypes.c_void_p()
    assert lib.kvs_create(ctypes.byref(ctx), None) == 0
    b = K.Batch(1, 64, 224, 96, k=[64])
    # NULL pointers -> invalid; misaligned -> align; small workspace -> workspace
    st = lib.kvs_loss_grad(ctx, ctypes.byref(b.c), None, None, None, None, None, None, None, None,
                           None, 0)
    assert st == -1 and b"NULL" in lib.kvs_last_error(ctx)
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    st = lib.kvs_loss_grad(ctx, ctypes.byref(b.c), odd, fake, fake, fake, fake, fake, None, None,
                           fake, 1 << 30)
    assert st == -2
    st = lib.kvs_loss_grad(ctx, ctypes.byref(b.c), fake, fake, fake, fake, fake, fake, None, None,
                           fake, 16)
    assert st == -3 and b"workspace" in lib.kvs_last_error(ctx)
    o = K.opts(max_backtracks=0)
    st = lib.kvs_compress(ctx, ctypes.byref(b.c), ctypes.byref(o), fake, fake, fake, fake, fake, fake,
                          None, None, None, fake, 1 << 30)
    assert st == -1 and b"max_backtracks" in lib.kvs_last_error(ctx)
    assert lib.kvs_destroy(ctx) == 0


def test_build_queries_argument_errors(K):
    lib = K.load()
    ctx = ctypes.c_void_p()
    assert lib.kvs_create(ctypes.byref(ctx), None) == 0
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    G = K._lib.KvsQueryGeom

    def call(geom, qctx=fake, src=fake, q=fake):
        return lib.kvs_build_queries(ctx, ctypes.byref(geom), qctx, src, q, None)

    # bad sizes, head dims and bases are refused with a message
    for geom, word in [(G(0, 6, 2048, 128, 512, 128, 1e6), b"sizes"),
                       (G(2, 6, 2048, 2049, 512, 128, 1e6), b"sizes"),
                       (G(2, 6, 2048, 128, -1, 128, 1e6), b"sizes"),
                       (G(2, 6, 2048, 128, 512, 96, 1e6), b"power of two"),
                       (G(2, 6, 2048, 128, 512, 128, 1.0), b"theta"),
                       (G(2, 6, 2048, 0, 0, 128, 1e6), b"no queries")]:
        assert call(geom) == -1 and word in lib.kvs_last_error(ctx), geom
    good = G(2, 6, 2048, 128, 512, 128, 1e6)
    assert call(good, qctx=None) == -1
    assert call(good, src=None) == -1 and b"src" in lib.kvs_last_error(ctx)
    assert call(good, q=odd) == -2
    assert lib.kvs_build_queries(ctx, None, fake, fake, fake, None) == -1
    assert lib.kvs_destroy(ctx) == 0


def test_use_eval_workspace_and_argument_errors(K):
    b = K.Batch(2, 128, 1920, 3072, k=[960, 700])
    ws = K.use_eval_workspace_bytes(b, 128)
    # two merged outputs alone are 2 * P * n * d floats; partials add more
    assert ws > 2 * 2 * 3072 * 128 * 4
    assert K.use_eval_workspace_bytes(b, -1) == 0
    assert K.use_eval_workspace_bytes(K.Batch(2, 96, 1920, 3072, k=[960, 700]), 128) == 0
    lib = K.load()
    ctx = ctypes.c_void_p()
    assert lib.kvs_create(ctypes.byref(ctx), None) == 0
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    args = [fake] * 6
    # retain zone pointers are required when m > 0
    st = lib.kvs_use_eval(ctx, ctypes.byref(b.c), 128, fake, fake, fake, None, None, fake, fake,
                          None, None, fake, None, fake, 1 << 40)
    assert st == -1 and b"Kr" in lib.kvs_last_error(ctx)
    st = lib.kvs_use_eval(ctx, ctypes.byref(b.c), 0, fake, fake, fake, None, None, fake, fake,
                          None, None, None, None, fake, 1 << 40)
    assert st == -1 and b"mse" in lib.kvs_last_error(ctx)
    st = lib.kvs_use_eval(ctx, ctypes.byref(b.c), 128, fake, fake, fake, fake, fake, fake, fake,
                          odd, None, fake, None, fake, 1 << 40)
    assert st == -2
    st = lib.kvs_use_eval(ctx, ctypes.byref(b.c), 128, *args, fake, None, None, fake, None,
                          fake, ws - 256)
    assert st == -3 and b"workspace" in lib.kvs_last_error(ctx)
    assert lib.kvs_destroy(ctx) == 0


def test_ablation_and_signal_argument_errors(K):
    lib = K.load()
    ctx = ctypes.c_void_p()
    assert lib.kvs_create(ctypes.byref(ctx), None) == 0
    fake = ctypes.c_void_p(0x1000)
    b = K.Batch(1, 64, 224, 96, k=[64])
    o = K.opts()
    big = 1 << 40
    # Adam: options checked before anything else
    st = lib.kvs_compress_adam(ctx, ctypes.byref(b.c), ctypes.byref(o), None, 0, fake, fake, fake,
                               fake, fake, fake, None, None, fake, fake, big)
    assert st == -1 and b"adam" in lib.kvs_last_error(ctx)
    for bad in (K.adam_opts(lr=0.0), K.adam_opts(beta1=1.0), K.adam_opts(beta2=-0.1),
                K.adam_opts(eps=0.0)):
        st = lib.kvs_compress_adam(ctx, ctypes.byref(b.c), ctypes.byref(o), ctypes.byref(bad), 0,
                                   fake, fake, fake, fake, fake, fake, None, None, fake, fake, big)
        assert st == -1 and b"lr" in lib.kvs_last_error(ctx)
    # flags are required for Adam
    good = K.adam_opts()
    st = lib.kvs_compress_adam(ctx, ctypes.byref(b.c), ctypes.byref(o), ctypes.byref(good), 0, fake,
                               fake, fake, fake, fake, fake, None, None, None, fake, big)
    assert st == -1 and b"flags" in lib.kvs_last_error(ctx)
    # restarts: the same checks as kvs_compress
    st = lib.kvs_compress_from_keys(ctx, ctypes.byref(b.c), None, fake, fake, fake, fake, fake, fake,
                                    None, None, fake, fake, big)
    assert st == -1 and b"opts" in lib.kvs_last_error(ctx)
    st = lib.kvs_compress_from_keys(ctx, ctypes.byref(b.c), ctypes.byref(o), fake, fake, fake, fake,
                                    fake, fake, None, None, fake, fake, 16)
    assert st == -3
    # value norms: sizes, pointers, workspace
    assert lib.kvs_value_norms(ctx, 2, 100, 96, fake, fake, fake, big) == -1
    assert lib.kvs_value_norms(ctx, 2, 100, 64, fake, None, fake, big) == -1
    assert lib.kvs_value_norms(ctx, 2, 100, 64, fake, fake, fake, 8) == -3
    d = K.adam_opts.__defaults__
    dflt = K._lib.KvsAdamOpts()
    lib.kvs_default_adam_opts(ctypes.byref(dflt))
    assert (dflt.lr, dflt.beta1, dflt.beta2, dflt.eps) == d
    assert lib.kvs_destroy(ctx) == 0


def test_allocator_cpp_equals_oracle_bit_for_bit(K):
    rng = np.random.default_rng(20)
    for it in range(10000):
        P = int(rng.integers(1, 60))
        scale = rng.choice([1e-6, 1.0, 1e3])
        mse = np.exp(rng.normal(0, 3, size=P)) * scale
        if it % 7 == 0:
            mse[rng.integers(0, P)] = 0.0
        kmax = int(rng.integers(1, 4000))
        kmin = int(rng.integers(1, kmax + 1))
        K_total = int(rng.integers(P * kmin, P * kmax + 1))
        alpha = [0.5, 1.0, 0.75][it % 3]
        want = O.allocate_budget(list(mse), K_total, alpha, kmin, kmax)
        got = K.kvs_allocate_budget(mse, K_total, alpha, kmin, kmax)
        assert got.tolist() == want, (it, P, kmin, kmax, K_total)


def test_two_level_allocator_cpp_equals_oracle_bit_for_bit(K):
    rng = np.random.default_rng(21)
    for it in range(3000):
        L, H = int(rng.integers(1, 33)), int(rng.integers(1, 9))
        P = L * H
        mse = np.exp(rng.normal(0, 3, size=P)) * rng.choice([1e-6, 1.0, 1e3])
        if it % 5 == 0:
            mse[rng.integers(0, P)] = 0.0
        kmax = int(rng.integers(1, 4000))
        kmin = int(rng.integers(1, kmax + 1))
        K_total = int(rng.integers(P * kmin, P * kmax + 1))
        alpha = [0.5, 1.0, 0.75][it % 3]
        want = O.allocate_budget_two_level(list(mse), L, H, K_total, alpha, kmin, kmax)
        got = K.kvs_allocate_budget_two_level(mse, L, H, K_total, alpha, kmin, kmax)
        assert got.tolist() == want, (it, L, H, kmin, kmax, K_total)
    with pytest.raises(K.KvsError):
        K.kvs_allocate_budget_two_level([1.0, 2.0, 3.0, 4.0], 2, 2, 100, 0.5, 1, 4)
    assert K.value_norms_workspace_bytes(0, 10) == 0 and K.value_norms_workspace_bytes(4, 100) >= 32


def test_allocator_rejects_bad_requests(K):
    with pytest.raises(K.KvsError):
        K.kvs_allocate_budget([1.0, 2.0], 10, 0.5, 1, 4)
    with pytest.raises(K.KvsError):
        K.kvs_allocate_budget([1.0, float("nan")], 4, 0.5, 1, 4)
    assert K.kvs_allocate_budget([0.0, 0.0, 0.0], 7).tolist() == [3, 2, 2]


def test_noalloc_value_norms_limit_is_checked_on_the_host(K):
    """The allocation-free value-norm call states its static scratch size and
    rejects a batch whose chunk partials would not fit, before any launch."""
    lib = K.load()
    assert K.value_norms_noalloc_max_bytes() == 1 << 20
    ctx = ctypes.c_void_p()
    assert lib.kvs_create(ctypes.byref(ctx), None) == 0
    fake = ctypes.c_void_p(0x1000)
    # 200000 problems of one chunk each: 1.6 MB of float64 partials > 1 MiB
    assert K.value_norms_workspace_bytes(200000, 64) > (1 << 20)
    st = lib.kvs_value_norms_noalloc(ctx, 200000, 64, 64, fake, fake)
    assert st == -1 and b"static array" in lib.kvs_last_error(ctx)
    assert lib.kvs_value_norms_noalloc(ctx, 4, 64, 96, fake, fake) == -1      # d
    assert lib.kvs_value_norms_noalloc(ctx, 4, 64, 64, None, fake) == -1      # Vz NULL
    assert lib.kvs_destroy(ctx) == 0
