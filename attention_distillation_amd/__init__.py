"""KVSculpt cache-distillation optimizer for MI355X (gfx950).

The compute lives in libkvsculpt.so (hand-written HIP kernels behind a C
ABI, declared in include/kvsculpt.h); this package is the thin ctypes
binding with the same entry-point names.  Importing it does not touch the
GPU; calling an entry point needs the built library and a GPU.
"""
from ._lib import (ENTRY_POINTS, KVS_FLAG_BADINDEX, KVS_FLAG_CHOLESKY, KVS_FLAG_LINESEARCH,
                   KVS_FLAG_NONDESCENT, KVS_FLAG_NONFINITE, Batch, Context, KvsBatch, KvsError,
                   KvsAdamOpts, KvsOpts, KvsQueryGeom, adam_opts, kvs_allocate_budget,
                   kvs_allocate_budget_two_level, kvs_value_norms, value_norms_workspace_bytes,
                   kvs_build_queries, kvs_compress, kvs_compress_adam, kvs_compress_from_keys,
                   kvs_init_topk, kvs_lbfgs_init, kvs_lbfgs_step, kvs_loss_grad,
                   kvs_pilot_allocate, kvs_profile_enable, kvs_profile_read, kvs_reference_attn,
                   kvs_use_eval, kvs_value_solve, lbfgs_state_bytes, load, opts,
                   use_eval_workspace_bytes, workspace_bytes)

__all__ = [
    "ENTRY_POINTS", "KVS_FLAG_BADINDEX", "KVS_FLAG_CHOLESKY", "KVS_FLAG_LINESEARCH",
    "KVS_FLAG_NONDESCENT", "KVS_FLAG_NONFINITE", "Batch", "Context", "KvsBatch", "KvsError",
    "KvsAdamOpts", "KvsOpts", "KvsQueryGeom", "adam_opts", "kvs_allocate_budget",
    "kvs_allocate_budget_two_level", "kvs_value_norms", "value_norms_workspace_bytes",
    "kvs_build_queries", "kvs_compress", "kvs_compress_adam", "kvs_compress_from_keys",
    "kvs_init_topk", "kvs_lbfgs_init", "kvs_lbfgs_step", "kvs_loss_grad", "kvs_pilot_allocate",
    "kvs_profile_enable", "kvs_profile_read", "kvs_reference_attn", "kvs_use_eval",
    "kvs_value_solve", "lbfgs_state_bytes", "load", "opts", "use_eval_workspace_bytes",
    "workspace_bytes",
]
