"""ctypes binding of libkvsculpt.so (argument marshalling only).

Every function here forwards to the C entry point of the same name; all
computation runs in the HIP library.  Tensors are torch tensors on the GPU
(float32 / int32, contiguous); only their data pointers and the current HIP
stream are passed.  A missing library raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_double, c_int32, c_int64, c_size_t, c_void_p, c_char_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvsculpt.so")

KVS_FLAG_NONFINITE = 1
KVS_FLAG_CHOLESKY = 2
KVS_FLAG_LINESEARCH = 4
KVS_FLAG_NONDESCENT = 8
KVS_FLAG_BADINDEX = 16

__all__ = [
    "ENTRY_POINTS",
    "KVS_FLAG_BADINDEX",
    "KVS_FLAG_CHOLESKY",
    "KVS_FLAG_LINESEARCH",
    "KVS_FLAG_NONDESCENT",
    "KVS_FLAG_NONFINITE",
    "Batch",
    "Context",
    "KvsBatch",
    "KvsError",
    "KvsAdamOpts",
    "KvsOpts",
    "KvsQueryGeom",
    "adam_opts",
    "kvs_allocate_budget",
    "kvs_allocate_budget_two_level",
    "kvs_value_norms",
    "value_norms_workspace_bytes",
    "kvs_build_queries",
    "kvs_compress",
    "kvs_compress_adam",
    "kvs_compress_from_keys",
    "kvs_compress_begin",
    "kvs_compress_advance",
    "kvs_value_norms_noalloc",
    "value_norms_noalloc_max_bytes",
    "kvs_init_topk",
    "kvs_lbfgs_init",
    "kvs_lbfgs_step",
    "kvs_loss_grad",
    "kvs_pilot_allocate",
    "kvs_profile_enable",
    "kvs_profile_read",
    "kvs_reference_attn",
    "kvs_use_eval",
    "kvs_value_solve",
    "lbfgs_state_bytes",
    "load",
    "opts",
    "use_eval_workspace_bytes",
    "workspace_bytes",
]

ENTRY_POINTS = (
    "kvs_create", "kvs_destroy", "kvs_status_string", "kvs_last_error", "kvs_default_opts",
    "kvs_workspace_bytes", "kvs_lbfgs_state_bytes", "kvs_reference_attn", "kvs_init_topk",
    "kvs_loss_grad", "kvs_value_solve", "kvs_lbfgs_init", "kvs_lbfgs_step", "kvs_compress",
    "kvs_pilot_allocate", "kvs_allocate_budget", "kvs_build_queries", "kvs_use_eval_workspace_bytes",
    "kvs_use_eval", "kvs_compress_from_keys", "kvs_default_adam_opts", "kvs_compress_adam",
    "kvs_allocate_budget_two_level", "kvs_value_norms_workspace_bytes", "kvs_value_norms",
    "kvs_profile_enable", "kvs_profile_read", "kvs_compress_begin", "kvs_compress_advance",
    "kvs_value_norms_noalloc_max_bytes", "kvs_value_norms_noalloc",
)


class KvsError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


class KvsBatch(ctypes.Structure):
    _fields_ = [("P", c_int32), ("d", c_int32), ("Z", c_int32), ("n", c_int32),
                ("k", POINTER(c_int32)), ("scale", c_double), ("lambda_", c_double),
                ("ridge_rel", c_double)]


class KvsAdamOpts(ctypes.Structure):
    _fields_ = [("lr", c_double), ("beta1", c_double), ("beta2", c_double), ("eps", c_double)]


class KvsQueryGeom(ctypes.Structure):
    _fields_ = [("P", c_int32), ("g", c_int32), ("N", c_int32), ("m", c_int32), ("F", c_int32),
                ("d", c_int32), ("theta", c_double)]


class KvsKernelStats(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", c_int64), ("total_ms", c_double),
                ("flops", c_double), ("bytes", c_double)]


class KvsOpts(ctypes.Structure):
    _fields_ = [("iters", c_int32), ("vc_every", c_int32), ("history", c_int32),
                ("max_backtracks", c_int32), ("c1", c_double), ("shrink", c_double)]


_lib = None


def load(path: str | None = None):
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own HIP runtime with the same soname as /opt/rocm's; it
    # must be loaded first so that this library binds to that one copy.
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m attention_distillation_amd.build`")
    lib = ctypes.CDLL(p)
    B, O = POINTER(KvsBatch), POINTER(KvsOpts)
    V = c_void_p
    sig = {
        "kvs_create": (c_int32, [POINTER(c_void_p), V]),
        "kvs_destroy": (c_int32, [V]),
        "kvs_status_string": (c_char_p, [c_int32]),
        "kvs_last_error": (c_char_p, [V]),
        "kvs_default_opts": (None, [O]),
        "kvs_workspace_bytes": (c_size_t, [B, O]),
        "kvs_lbfgs_state_bytes": (c_size_t, [B, O]),
        "kvs_reference_attn": (c_int32, [V, B, V, V, V, V, V, V, c_size_t]),
        "kvs_init_topk": (c_int32, [V, B, V, V, V, V, V, V, V, V, V, c_size_t]),
        "kvs_loss_grad": (c_int32, [V, B, V, V, V, V, V, V, V, V, V, c_size_t]),
        "kvs_value_solve": (c_int32, [V, B, V, V, V, V, V, V, V, c_size_t]),
        "kvs_lbfgs_init": (c_int32, [V, B, O, V, V, V, V, V, c_int32, V, V, V, c_size_t, V, c_size_t]),
        "kvs_lbfgs_step": (c_int32, [V, B, O, V, V, V, V, V, V, V, V, c_size_t, V, c_size_t]),
        "kvs_compress": (c_int32, [V, B, O, V, V, V, V, V, V, V, V, V, V, c_size_t]),
        "kvs_pilot_allocate": (c_int32, [V, B, O, c_int32, c_double, c_int32, c_int32, V, V, V, V,
                                         V, V, c_size_t]),
        "kvs_allocate_budget": (c_int32, [POINTER(c_double), c_int32, c_int64, c_double, c_int32,
                                          c_int32, POINTER(c_int32)]),
        "kvs_build_queries": (c_int32, [V, POINTER(KvsQueryGeom), V, V, V, V]),
        "kvs_use_eval_workspace_bytes": (c_size_t, [B, c_int32]),
        "kvs_allocate_budget_two_level": (c_int32, [POINTER(c_double), c_int32, c_int32, c_int64,
                                                    c_double, c_int32, c_int32, POINTER(c_int32)]),
        "kvs_value_norms_workspace_bytes": (c_size_t, [c_int32, c_int32]),
        "kvs_value_norms": (c_int32, [V, c_int32, c_int32, c_int32, V, V, V, c_size_t]),
        "kvs_compress_from_keys": (c_int32, [V, B, O, V, V, V, V, V, V, V, V, V, V, c_size_t]),
        "kvs_default_adam_opts": (None, [POINTER(KvsAdamOpts)]),
        "kvs_compress_adam": (c_int32, [V, B, O, POINTER(KvsAdamOpts), c_int32, V, V, V, V, V, V, V,
                                        V, V, V, c_size_t]),
        "kvs_use_eval": (c_int32, [V, B, c_int32, V, V, V, V, V, V, V, V, V, V, V, V, c_size_t]),
        "kvs_compress_begin": (c_int32, [V, B, O, V, V, V, c_int32, V, V, V, V, c_size_t]),
        "kvs_compress_advance": (c_int32, [V, B, O, V, c_int32, c_int32, V, V, V, V, V, V,
                                           c_size_t]),
        "kvs_value_norms_noalloc_max_bytes": (c_size_t, []),
        "kvs_value_norms_noalloc": (c_int32, [V, c_int32, c_int32, c_int32, V, V]),
        "kvs_profile_enable": (c_int32, [V, c_int32]),
        "kvs_profile_read": (c_int32, [V, POINTER(KvsKernelStats), c_int32, POINTER(c_int32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Context:
    """A library context bound to the current torch HIP stream."""

    def __init__(self, stream=None):
        lib = load()
        h = ctypes.c_void_p()
        s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_handle()
        st = lib.kvs_create(ctypes.byref(h), s)
        if st != 0:
            raise KvsError("kvs_create", st, "")
        self.handle = h
        self.lib = lib

    def close(self):
        if self.handle:
            self.lib.kvs_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def check(self, fn, status):
        if status != 0:
            raise KvsError(fn, status, self.lib.kvs_last_error(self.handle).decode())


class Batch:
    """Holds a KvsBatch and the host k array it points to."""

    def __init__(self, P, d, Z, n, k=None, scale=None, lam=1.0, ridge_rel=1e-3):
        import numpy as np
        self.karr = np.ascontiguousarray(
            np.full(P, Z, dtype=np.int32) if k is None else np.asarray(k, dtype=np.int32))
        if self.karr.shape != (P,):
            raise ValueError("k must have P entries")
        self.c = KvsBatch(P, d, Z, n, self.karr.ctypes.data_as(POINTER(c_int32)),
                          1.0 / math.sqrt(d) if scale is None else scale, lam, ridge_rel)

    @property
    def ktot(self):
        return int(self.karr.sum())

    @property
    def P(self):
        return self.c.P


def opts(iters=20, vc_every=5, history=10, max_backtracks=30, c1=1e-4, shrink=0.5):
    return KvsOpts(iters, vc_every, history, max_backtracks, c1, shrink)


def workspace_bytes(batch: Batch, o: KvsOpts | None = None) -> int:
    return load().kvs_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(o) if o else None)


def lbfgs_state_bytes(batch: Batch, o: KvsOpts | None = None) -> int:
    return load().kvs_lbfgs_state_bytes(ctypes.byref(batch.c), ctypes.byref(o) if o else None)


def _ws(ws):
    return _ptr(ws), ws.numel() * ws.element_size()


def kvs_reference_attn(ctx, batch, Q, Kz, Vz, Y, lse, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_reference_attn", ctx.lib.kvs_reference_attn(
        ctx.handle, ctypes.byref(batch.c), _ptr(Q), _ptr(Kz), _ptr(Vz), _ptr(Y), _ptr(lse), w, nb))


def kvs_init_topk(ctx, batch, Q, Kz, Y, lse, idx, Kc, Vc, flags, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_init_topk", ctx.lib.kvs_init_topk(
        ctx.handle, ctypes.byref(batch.c), _ptr(Q), _ptr(Kz), _ptr(Y), _ptr(lse), _ptr(idx),
        _ptr(Kc), _ptr(Vc), _ptr(flags), w, nb))


def kvs_loss_grad(ctx, batch, Q, Y, lse, Kc, Vc, loss, grad, mse, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_loss_grad", ctx.lib.kvs_loss_grad(
        ctx.handle, ctypes.byref(batch.c), _ptr(Q), _ptr(Y), _ptr(lse), _ptr(Kc), _ptr(Vc),
        _ptr(loss), _ptr(grad), _ptr(mse), w, nb))


def kvs_value_solve(ctx, batch, Q, Y, lse, Kc, Vc, flags, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_value_solve", ctx.lib.kvs_value_solve(
        ctx.handle, ctypes.byref(batch.c), _ptr(Q), _ptr(Y), _ptr(lse), _ptr(Kc), _ptr(Vc),
        _ptr(flags), w, nb))


def kvs_lbfgs_init(ctx, batch, o, Q, Y, lse, Kc, Vc, clear_history, loss, flags, state, ws):
    w, nb = _ws(ws)
    s, sb = _ws(state)
    ctx.check("kvs_lbfgs_init", ctx.lib.kvs_lbfgs_init(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), _ptr(Q), _ptr(Y), _ptr(lse), _ptr(Kc),
        _ptr(Vc), int(clear_history), _ptr(loss), _ptr(flags), s, sb, w, nb))


def kvs_lbfgs_step(ctx, batch, o, Q, Y, lse, Kc, Vc, loss, flags, state, ws):
    w, nb = _ws(ws)
    s, sb = _ws(state)
    ctx.check("kvs_lbfgs_step", ctx.lib.kvs_lbfgs_step(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), _ptr(Q), _ptr(Y), _ptr(lse), _ptr(Kc),
        _ptr(Vc), _ptr(loss), _ptr(flags), s, sb, w, nb))


def kvs_compress(ctx, batch, o, Q, Kz, Vz, Kc, Vc, loss, mse, init_loss, flags, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_compress", ctx.lib.kvs_compress(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), _ptr(Q), _ptr(Kz), _ptr(Vz), _ptr(Kc),
        _ptr(Vc), _ptr(loss), _ptr(mse), _ptr(init_loss), _ptr(flags), w, nb))


def kvs_compress_from_keys(ctx, batch, o, Q, Kz, Vz, Kc, Vc, loss, mse, init_loss, flags, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_compress_from_keys", ctx.lib.kvs_compress_from_keys(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), _ptr(Q), _ptr(Kz), _ptr(Vz), _ptr(Kc),
        _ptr(Vc), _ptr(loss), _ptr(mse), _ptr(init_loss), _ptr(flags), w, nb))


def kvs_compress_begin(ctx, batch, o, Q, Kz, Vz, keys_given, Kc, Vc, init_loss, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_compress_begin", ctx.lib.kvs_compress_begin(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), _ptr(Q), _ptr(Kz), _ptr(Vz),
        int(keys_given), _ptr(Kc), _ptr(Vc), _ptr(init_loss), w, nb))


def kvs_compress_advance(ctx, batch, o, Q, t_begin, t_end, Kc, Vc, loss, mse, flags, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_compress_advance", ctx.lib.kvs_compress_advance(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), _ptr(Q), int(t_begin), int(t_end),
        _ptr(Kc), _ptr(Vc), _ptr(loss), _ptr(mse), _ptr(flags), w, nb))


def adam_opts(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8):
    return KvsAdamOpts(lr, beta1, beta2, eps)


def kvs_compress_adam(ctx, batch, o, a, keys_given, Q, Kz, Vz, Kc, Vc, loss, mse, init_loss,
                      flags, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_compress_adam", ctx.lib.kvs_compress_adam(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), ctypes.byref(a), int(keys_given),
        _ptr(Q), _ptr(Kz), _ptr(Vz), _ptr(Kc), _ptr(Vc), _ptr(loss), _ptr(mse), _ptr(init_loss),
        _ptr(flags), w, nb))


def kvs_pilot_allocate(ctx, batch, o, pilot_iters, alpha, k_min, k_max, Q, Kz, Vz, pilot_mse, ws):
    import numpy as np
    k_out = np.zeros(batch.P, dtype=np.int32)
    w, nb = _ws(ws)
    ctx.check("kvs_pilot_allocate", ctx.lib.kvs_pilot_allocate(
        ctx.handle, ctypes.byref(batch.c), ctypes.byref(o), int(pilot_iters), float(alpha),
        int(k_min), int(k_max), _ptr(Q), _ptr(Kz), _ptr(Vz), _ptr(pilot_mse),
        k_out.ctypes.data_as(c_void_p), w, nb))
    return k_out


def kvs_allocate_budget(mse, K_total, alpha=0.5, k_min=1, k_max=1 << 30):
    import numpy as np
    m = np.ascontiguousarray(np.asarray(mse, dtype=np.float64))
    out = np.zeros(m.size, dtype=np.int32)
    st = load().kvs_allocate_budget(m.ctypes.data_as(POINTER(c_double)), m.size, int(K_total),
                                    float(alpha), int(k_min), int(k_max),
                                    out.ctypes.data_as(POINTER(c_int32)))
    if st != 0:
        raise KvsError("kvs_allocate_budget", st, "invalid budget request")
    return out


def kvs_build_queries(ctx, P, g, N, m, F, d, theta, Qctx, src, Q, flags=None):
    geom = KvsQueryGeom(P, g, N, m, F, d, float(theta))
    ctx.check("kvs_build_queries", ctx.lib.kvs_build_queries(
        ctx.handle, ctypes.byref(geom), _ptr(Qctx), _ptr(src), _ptr(Q), _ptr(flags)))


def use_eval_workspace_bytes(batch: Batch, m: int) -> int:
    return load().kvs_use_eval_workspace_bytes(ctypes.byref(batch.c), int(m))


def kvs_use_eval(ctx, batch, m, Qh, Kz, Vz, Kr, Vr, Kc, Vc, Ofull, Ocomp, mse, rel, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_use_eval", ctx.lib.kvs_use_eval(
        ctx.handle, ctypes.byref(batch.c), int(m), _ptr(Qh), _ptr(Kz), _ptr(Vz), _ptr(Kr),
        _ptr(Vr), _ptr(Kc), _ptr(Vc), _ptr(Ofull), _ptr(Ocomp), _ptr(mse), _ptr(rel), w, nb))


def kvs_allocate_budget_two_level(mse, layers, heads, K_total, alpha=0.5, k_min=1, k_max=1 << 30):
    import numpy as np
    m = np.ascontiguousarray(np.asarray(mse, dtype=np.float64))
    out = np.zeros(m.size, dtype=np.int32)
    st = load().kvs_allocate_budget_two_level(m.ctypes.data_as(POINTER(c_double)), int(layers),
                                              int(heads), int(K_total), float(alpha), int(k_min),
                                              int(k_max), out.ctypes.data_as(POINTER(c_int32)))
    if st != 0:
        raise KvsError("kvs_allocate_budget_two_level", st, "invalid budget request")
    return out


def value_norms_workspace_bytes(P, Z):
    return load().kvs_value_norms_workspace_bytes(int(P), int(Z))


def kvs_value_norms(ctx, P, Z, d, Vz, signal, ws):
    w, nb = _ws(ws)
    ctx.check("kvs_value_norms", ctx.lib.kvs_value_norms(ctx.handle, int(P), int(Z), int(d),
                                                         _ptr(Vz), _ptr(signal), w, nb))


PROFILE_CLASSES = ("attn_fwd", "attn_bwd", "gram", "potrf_panel", "trailing", "back_subst",
                   "hist_dots", "direction", "importance", "ref_attn_fwd", "merge",
                   "build_queries", "use_attn_fwd", "attn_pv", "key_digits", "resid_rhs", "fwd_subst",
                   "gram_split", "resid_rhs_split", "attn_bwd_split")


def value_norms_noalloc_max_bytes():
    return int(load().kvs_value_norms_noalloc_max_bytes())


def kvs_value_norms_noalloc(ctx, P, Z, d, Vz, signal):
    ctx.check("kvs_value_norms_noalloc", ctx.lib.kvs_value_norms_noalloc(
        ctx.handle, int(P), int(Z), int(d), _ptr(Vz), _ptr(signal)))


def kvs_profile_enable(ctx, enable=True, kernels=None):
    """Enable per-kernel event timing (all kernels, or the named ones)."""
    mask = 0
    if enable:
        mask = -1 if kernels is None else sum(1 << PROFILE_CLASSES.index(k) for k in kernels)
    ctx.check("kvs_profile_enable", ctx.lib.kvs_profile_enable(ctx.handle, mask))


def kvs_profile_read(ctx):
    """Per-kernel totals since the last enable: {name: dict(launches, ms, flops, bytes)}."""
    arr = (KvsKernelStats * 32)()
    cnt = c_int32(0)
    ctx.check("kvs_profile_read", ctx.lib.kvs_profile_read(ctx.handle, arr, 32, ctypes.byref(cnt)))
    return {arr[i].name.decode(): dict(launches=int(arr[i].launches), ms=float(arr[i].total_ms),
                                       flops=float(arr[i].flops), bytes=float(arr[i].bytes))
            for i in range(cnt.value)}
