"""Seeded synthetic KVSculpt workloads.

This module only builds inputs: RoPE'd compress-zone keys and values, the
training queries and the per-head budgets.  It holds none of the optimizer's
arithmetic (no attention, loss, gradient, value solve, L-BFGS or allocation),
so the float64 oracle and the HIP path can both read its arrays without
sharing any of the method.

Source of each choice (KVSculpt: KV Cache Compression as Distillation, the
gist.science page, section 2 "Methodology"):

* Problem formulation: the oldest N-m pairs form the compress zone, the most
  recent m pairs the retain zone.
* Training query construction: retain queries are the real queries of the
  recent context; synthetic future queries are query content taken from the
  context by undoing RoPE at its own position and re-applying RoPE at a future
  position, with the source positions drawn uniformly over the context.

Shapes and distributions are the five workload presets below (single head;
one Qwen2.5-1.5B-shaped layer; the full Qwen2.5-1.5B-shaped cache; a
Llama-3-8B-shaped cache; a long-context Qwen2.5-7B-shaped cache).  Real model
caches and text are not used; these synthetic heads stand in for them.

Generation is float64 NumPy, rounded to float32 once at the end.  RoPE uses
half-split channel pairs (c, c + d/2) with angle pos * base**(-2c/d) and
0-based positions.  Per KV head the random stream is
``default_rng(SeedSequence([seed, config, layer, head]))``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload preset (all sizes per KV head unless stated)."""

    cid: int
    name: str
    layers: int
    kv_heads: int
    d: int
    N: int
    m: int
    g: int            # query heads per KV head (GQA group)
    F: int            # synthetic future queries per query head
    theta: float      # RoPE base
    ratio: float      # compression ratio r (k0 = round(r * Z))
    T: int            # main-run L-BFGS iterations
    pilot: int        # pilot iterations (0 = no pilot)
    outliers: int     # key channels whose scale is multiplied by 10
    student_t: bool   # heavy-tailed (Student-t, nu=3) key content
    temp_range: tuple | None = None   # per-layer temperature, log-uniform
    k0_override: int | None = None

    @property
    def P(self) -> int:
        return self.layers * self.kv_heads

    @property
    def Z(self) -> int:
        return self.N - self.m

    @property
    def n(self) -> int:
        return self.g * (self.m + self.F)

    @property
    def k0(self) -> int:
        if self.k0_override is not None:
            return self.k0_override
        # round half up, so 0.3*7936 = 2380.8 -> 2381 and 0.1*32256 -> 3226
        return int(math.floor(self.ratio * self.Z + 0.5))

    def with_ratio(self, r: float) -> "Workload":
        return dataclasses.replace(self, ratio=r, k0_override=None)


WORKLOADS = {
    0: Workload(0, "single-head-d64", layers=1, kv_heads=1, d=64, N=256, m=32,
                g=1, F=64, theta=1e4, ratio=64 / 224, T=20, pilot=0,
                outliers=0, student_t=False, k0_override=64),
    1: Workload(1, "qwen2.5-1.5b-one-layer", layers=1, kv_heads=2, d=128,
                N=2048, m=128, g=6, F=512, theta=1e6, ratio=0.5, T=300,
                pilot=0, outliers=4, student_t=False),
    2: Workload(2, "qwen2.5-1.5b-full-cache", layers=28, kv_heads=2, d=128,
                N=2048, m=128, g=6, F=512, theta=1e6, ratio=0.5, T=300,
                pilot=60, outliers=4, student_t=False, temp_range=(0.5, 4.0)),
    3: Workload(3, "llama3-8b-cache", layers=32, kv_heads=8, d=128, N=8192,
                m=256, g=4, F=1024, theta=5e5, ratio=0.3, T=200, pilot=60,
                outliers=4, student_t=False),
    4: Workload(4, "qwen2.5-7b-long-context", layers=28, kv_heads=4, d=128,
                N=32768, m=512, g=7, F=2048, theta=1e6, ratio=0.1, T=150,
                pilot=60, outliers=8, student_t=True),
}


def tiny_workload(d=8, N=40, m=8, g=2, F=6, k0=5, theta=1e4, outliers=0,
                  layers=1, kv_heads=1, T=10, student_t=False, name="tiny"):
    """A small preset with the same construction, for fast tests."""
    return Workload(99, name, layers=layers, kv_heads=kv_heads, d=d, N=N, m=m,
                    g=g, F=F, theta=theta, ratio=k0 / (N - m), T=T, pilot=0,
                    outliers=outliers, student_t=student_t, k0_override=k0)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate channel pairs (c, c+d/2) of rows of ``x`` by pos * theta**(-2c/d)."""
    d = x.shape[-1]
    h = d // 2
    inv = theta ** (-2.0 * np.arange(h, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def unrope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Inverse rotation of :func:`rope` (the De-RoPE step)."""
    return rope(x, -np.asarray(pos, dtype=np.float64), theta)


def layer_temperatures(w: Workload, seed: int = 0) -> np.ndarray:
    """Per-layer attention temperature, log-uniform over ``temp_range``."""
    if w.temp_range is None:
        return np.ones(w.layers)
    rng = np.random.default_rng(np.random.SeedSequence([seed, w.cid, 7919]))
    lo, hi = np.log(w.temp_range[0]), np.log(w.temp_range[1])
    return np.exp(rng.uniform(lo, hi, size=w.layers))


def _head_base(w: Workload, rng) -> dict:
    """Draws shared by every view of one KV head, in a fixed order: channel
    scales, key content (with outlier channels), values, the mean key
    direction and the future queries' source positions."""
    d, N, g, F = w.d, w.N, w.g, w.F
    sigma = np.exp(0.5 * rng.standard_normal(d))
    sigma_k = sigma.copy()
    if w.outliers:
        ch = rng.choice(d, size=w.outliers, replace=False)
        sigma_k[ch] *= 10.0
    if w.student_t:
        kc = rng.standard_t(3.0, size=(N, d)) * sigma_k
    else:
        kc = rng.standard_normal((N, d)) * sigma_k
    vals = rng.standard_normal((N, d))
    mean_dir = kc.mean(axis=0)
    mean_dir = mean_dir / np.linalg.norm(mean_dir)
    fut_src = rng.integers(0, N, size=(g, F))
    return dict(sigma=sigma, kc=kc, vals=vals, mean_dir=mean_dir, fut_src=fut_src)


def make_head(w: Workload, layer: int, head: int, seed: int = 0,
              temperature: float = 1.0) -> dict:
    """Build one KV head's problem in float64 (rounded to float32 by callers).

    Returns a dict with
      Kz, Vz   [Z, d]  compress zone (RoPE'd keys, plain values)
      Kr, Vr   [m, d]  retain zone
      Q        [n, d]  training queries: query head 0..g-1 retain rows, then
                       query head 0..g-1 future rows
      n_retain         number of retain rows (g*m)
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, w.cid, layer, head]))
    d, N, m, Z, g, F = w.d, w.N, w.m, w.Z, w.g, w.F
    base = _head_base(w, rng)
    sigma, kc, vals = base["sigma"], base["kc"], base["vals"]
    mean_dir, fut_src = base["mean_dir"], base["fut_src"]
    pos_all = np.arange(N)
    keys = rope(kc, pos_all, w.theta)

    retain_rows, future_rows = [], []
    for h in range(g):
        need = np.union1d(np.arange(Z, N), fut_src[h])
        content = 0.5 * mean_dir + rng.standard_normal((need.size, d)) * sigma
        content = content / temperature
        roped = rope(content, need, w.theta)            # the context's queries
        where = {int(p): i for i, p in enumerate(need)}
        retain_rows.append(roped[[where[p] for p in range(Z, N)]])
        src = fut_src[h]
        q_src = roped[[where[int(p)] for p in src]]
        back = unrope(q_src, src, w.theta)              # De-RoPE at source
        future_rows.append(rope(back, N + np.arange(F), w.theta))  # future pos
    Q = np.concatenate(retain_rows + future_rows, axis=0)
    return dict(Kz=keys[:Z], Vz=vals[:Z], Kr=keys[Z:], Vr=vals[Z:], Q=Q,
                n_retain=g * m)


def make_context(w: Workload, layer: int, head: int, seed: int = 0,
                 temperature: float = 1.0) -> dict:
    """One KV head's context queries, for building training queries on device.

    Keys, values and source positions are those of :func:`make_head` (same
    stream, same draw order); the query content is then drawn at every
    context position.  Returns
      Qctx  [g, N, d]  RoPE'd queries of the g query heads at positions 0..N-1
      src   [g, F]     source positions of the synthetic future queries,
                       uniform over [0, N)
      Kz, Vz, Kr, Vr   as in :func:`make_head`
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, w.cid, layer, head]))
    d, N, Z, g = w.d, w.N, w.Z, w.g
    base = _head_base(w, rng)
    keys = rope(base["kc"], np.arange(N), w.theta)
    vals = base["vals"]
    qctx = np.empty((g, N, d))
    for h in range(g):
        content = 0.5 * base["mean_dir"] + rng.standard_normal((N, d)) * base["sigma"]
        qctx[h] = rope(content / temperature, np.arange(N), w.theta)
    return dict(Qctx=qctx, src=base["fut_src"], Kz=keys[:Z], Vz=vals[:Z], Kr=keys[Z:],
                Vr=vals[Z:])


def make_context_batch(w: Workload, seed: int = 0,
                       problems: Sequence[int] | None = None) -> dict:
    """Stack :func:`make_context` over problems: Qctx [P, g, N, d] float32,
    src [P, g, F] int32, Kz/Vz [P, Z, d] float32."""
    temps = layer_temperatures(w, seed)
    plist = problem_list(w, problems)
    out = {k: [] for k in ("Qctx", "src", "Kz", "Vz")}
    for p in plist:
        layer, head = divmod(p, w.kv_heads)
        hd = make_context(w, layer, head, seed, float(temps[layer]))
        for k in out:
            out[k].append(hd[k])
    res = {k: np.ascontiguousarray(np.stack(v).astype(np.int32 if k == "src" else np.float32))
           for k, v in out.items()}
    res["problems"] = np.array(plist, dtype=np.int64)
    res["scale"] = 1.0 / math.sqrt(w.d)
    return res


def make_use_batch(w: Workload, seed: int = 0, problems: Sequence[int] | None = None,
                   per_head: int | None = None) -> dict:
    """Held-out future queries with the caches of :func:`make_batch`.

    Keys and values are those of :func:`make_head` (same stream, same draw
    order).  The held-out queries come from a stream of their own: per query
    head, ``per_head`` (default F) fresh query contents of the same
    distribution as the context's (0.5 * mean key direction + N(0, sigma^2),
    over the layer temperature), RoPE'd at the future positions N, N+1, ...
    Returns Qh [P, g*per_head, d], Kz/Vz [P, Z, d], Kr/Vr [P, m, d] float32.
    """
    temps = layer_temperatures(w, seed)
    plist = problem_list(w, problems)
    per = w.F if per_head is None else int(per_head)
    out = {k: [] for k in ("Qh", "Kz", "Vz", "Kr", "Vr")}
    for p in plist:
        layer, head = divmod(p, w.kv_heads)
        rng = np.random.default_rng(np.random.SeedSequence([seed, w.cid, layer, head]))
        base = _head_base(w, rng)
        keys = rope(base["kc"], np.arange(w.N), w.theta)
        hrng = np.random.default_rng(np.random.SeedSequence([seed, w.cid, layer, head, 2]))
        rows = []
        for _ in range(w.g):
            content = 0.5 * base["mean_dir"] + hrng.standard_normal((per, w.d)) * base["sigma"]
            rows.append(rope(content / float(temps[layer]), w.N + np.arange(per), w.theta))
        out["Qh"].append(np.concatenate(rows, axis=0))
        out["Kz"].append(keys[:w.Z])
        out["Vz"].append(base["vals"][:w.Z])
        out["Kr"].append(keys[w.Z:])
        out["Vr"].append(base["vals"][w.Z:])
    res = {k: np.ascontiguousarray(np.stack(v).astype(np.float32)) for k, v in out.items()}
    res["problems"] = np.array(plist, dtype=np.int64)
    res["scale"] = 1.0 / math.sqrt(w.d)
    return res


def problem_list(w: Workload, problems: Iterable[int] | None = None) -> list:
    P = w.P
    return list(range(P)) if problems is None else [int(p) for p in problems]


def _heads_f32(args):
    """Worker of :func:`make_batch`: float32 arrays of some problems."""
    w, seed, plist, keys = args
    temps = layer_temperatures(w, seed)
    out = {k: [] for k in keys}
    for p in plist:
        layer, head = divmod(p, w.kv_heads)
        hd = make_head(w, layer, head, seed, float(temps[layer]))
        for k in keys:
            out[k].append(hd[k].astype(np.float32))
    return out


def make_batch(w: Workload, seed: int = 0, problems: Sequence[int] | None = None,
               with_retain: bool = False, workers: int = 1) -> dict:
    """Stack problems p = layer * kv_heads + head into float32 arrays.

    Q [P, n, d], Kz [P, Z, d], Vz [P, Z, d] (+ Kr, Vr [P, m, d] if asked).
    ``workers`` > 1 builds the heads in that many processes (same arrays:
    every head has its own seeded stream).
    """
    temps = layer_temperatures(w, seed)
    plist = problem_list(w, problems)
    if workers > 1 and len(plist) > 1:
        import concurrent.futures as cf
        keys = ("Q", "Kz", "Vz") + (("Kr", "Vr") if with_retain else ())
        nw = min(workers, len(plist))
        chunks = [plist[i::nw] for i in range(nw)]
        res = {k: [None] * len(plist) for k in keys}
        where = {p: i for i, p in enumerate(plist)}
        with cf.ProcessPoolExecutor(nw) as ex:
            for chunk, part in zip(chunks, ex.map(_heads_f32, [(w, seed, c, keys) for c in chunks])):
                for k in keys:
                    for p, a in zip(chunk, part[k]):
                        res[k][where[p]] = a
        out = {}
        for k in keys:
            arr = np.empty((len(plist),) + res[k][0].shape, dtype=np.float32)
            for i, a in enumerate(res[k]):
                arr[i] = a
                res[k][i] = None
            out[k] = arr
        out["problems"] = np.array(plist, dtype=np.int64)
        out["scale"] = 1.0 / math.sqrt(w.d)
        return out
    out = {k: [] for k in ("Q", "Kz", "Vz", "Kr", "Vr")}
    for p in plist:
        layer, head = divmod(p, w.kv_heads)
        hd = make_head(w, layer, head, seed, float(temps[layer]))
        for k in out:
            out[k].append(hd[k])
    res = {k: np.ascontiguousarray(np.stack(v).astype(np.float32)) for k, v in out.items()
           if with_retain or k in ("Q", "Kz", "Vz")}
    res["problems"] = np.array(plist, dtype=np.int64)
    res["scale"] = 1.0 / math.sqrt(w.d)
    return res


def uniform_budget(w: Workload, P: int | None = None) -> np.ndarray:
    return np.full(w.P if P is None else P, w.k0, dtype=np.int32)
