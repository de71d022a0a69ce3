"""ctypes binding of libsparsepr.so: the C ABI of include/sparsepr.h under the same names.

Argument marshalling only. Every step of the call runs in the library's HIP kernels;
PyTorch provides device memory and the current HIP stream. If the library is missing
the import fails loudly -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparsepr.so")

SPARSEPR_OK = 0
SPARSEPR_ERR_INVALID_ARG = 1
SPARSEPR_ERR_UNSUPPORTED = 2
SPARSEPR_ERR_WORKSPACE = 3
SPARSEPR_ERR_HIP = 4
SPARSEPR_ERR_NUMERICAL = 5
SPARSEPR_ERR_STATE = 6
SPARSEPR_ERR_TOO_LARGE = 7

# include/sparsepr.h SPARSEPR_STATIC_WORKSPACE_BYTES
STATIC_WORKSPACE_BYTES = 128 << 20

SPARSEPR_F32 = 0
SPARSEPR_BF16 = 1

EXPORT = dict(SAMPLED=0, KEY_LABELS=1, QUERY_LABELS=2, KEY_PERM=3, QUERY_PERM=4, KEY_OFFSETS=5,
              QUERY_OFFSETS=6, ROUTE_ROWPTR=7, ROUTE_COLS=8, PROBES=9, PROBE_WEIGHTS=10, GROUP_MASS=11,
              KEY_CENTROIDS=12, KEY_SEEDS=13, QUERY_SEEDS=14)


class sparsepr_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("n_sampled", ctypes.c_int32), ("n_key_groups", ctypes.c_int32),
                ("n_query_groups", ctypes.c_int32), ("n_probes", ctypes.c_int32), ("density", ctypes.c_double),
                ("kmeans_max_iter", ctypes.c_int32), ("kmeans_tol", ctypes.c_float),
                ("ridge_lambda", ctypes.c_float), ("penalize_bias", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("assign_precision", ctypes.c_int32), ("warm_iters", ctypes.c_int32),
                ("partition", ctypes.c_int32), ("correction", ctypes.c_int32), ("probe_selector", ctypes.c_int32),
                ("key_rank", ctypes.c_int32), ("attn_tile_rows", ctypes.c_int32), ("output_rank", ctypes.c_int32)]


class sparsepr_head_info(ctypes.Structure):
    _fields_ = [("key_groups", ctypes.c_int32), ("query_groups", ctypes.c_int32), ("key_iters", ctypes.c_int32),
                ("query_iters", ctypes.c_int32), ("executed_pairs", ctypes.c_int64), ("budget", ctypes.c_int64),
                ("tau", ctypes.c_int64), ("budget_exceeded", ctypes.c_int32), ("status", ctypes.c_int32)]


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SIGS = {
    "sparsepr_plan_create": (ctypes.c_int, [ctypes.POINTER(sparsepr_config), ctypes.POINTER(_P)]),
    "sparsepr_plan_destroy": (None, [_P]),
    "sparsepr_workspace_bytes": (_SZ, [_P]),
    "sparsepr_plan": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _P]),
    "sparsepr_plan_warm": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _P]),
    "sparsepr_plan_static": (ctypes.c_int, [_P, _P, _P, _P]),
    "sparsepr_plan_set_probes": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _P]),
    "sparsepr_plan_from_labels": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sparsepr_attend": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "sparsepr_fit_residual": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "sparsepr_apply": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "sparsepr_dense_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sparsepr_plan_info": (ctypes.c_int, [_P, ctypes.POINTER(sparsepr_head_info), ctypes.c_int32, _P]),
    "sparsepr_export_bytes": (_SZ, [_P, ctypes.c_int32]),
    "sparsepr_plan_export": (ctypes.c_int, [_P, ctypes.c_int32, _P, _SZ, _P]),
    "sparsepr_set_stage_timing": (ctypes.c_int, [_P, ctypes.c_int32]),
    "sparsepr_stage_times": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), ctypes.c_int32]),
    "sparsepr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}
STAGES = ("plan", "permute", "sparse", "probes", "fit", "apply")
SYMBOLS = tuple(_SIGS)


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"SparsePR HIP library not built: {path} is missing "
                          "(run python -m free_block_sparse_response_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


class SparsePRError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().sparsepr_status_string(status).decode()
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def _check(fn, status):
    if status != SPARSEPR_OK:
        raise SparsePRError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# --------------------------------------------------------------------------- same names
def make_config(batch, heads, seq_len, head_dim, dtype, n_sampled, n_key_groups, n_query_groups, n_probes,
                density, kmeans_max_iter=25, kmeans_tol=1e-4, ridge_lambda=1e-3, penalize_bias=0, seed=0,
                softmax_scale=0.0, assign_precision=0, warm_iters=2, partition=0, correction=0,
                probe_selector=0, key_rank=0, attn_tile_rows=0, output_rank=0):
    c = sparsepr_config()
    c.batch, c.heads, c.seq_len, c.head_dim = batch, heads, seq_len, head_dim
    c.dtype = {"f32": SPARSEPR_F32, "bf16": SPARSEPR_BF16}.get(dtype, dtype)
    c.softmax_scale = softmax_scale
    c.n_sampled, c.n_key_groups, c.n_query_groups, c.n_probes = n_sampled, n_key_groups, n_query_groups, n_probes
    c.density = density
    c.kmeans_max_iter, c.kmeans_tol = kmeans_max_iter, kmeans_tol
    c.ridge_lambda, c.penalize_bias, c.seed = ridge_lambda, penalize_bias, seed
    c.assign_precision = assign_precision
    c.warm_iters = warm_iters
    c.partition, c.correction, c.probe_selector = partition, correction, probe_selector
    c.key_rank = key_rank
    c.attn_tile_rows = attn_tile_rows
    c.output_rank = output_rank
    return c


def sparsepr_plan_create(cfg):
    h = _P()
    _check("sparsepr_plan_create", lib().sparsepr_plan_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def sparsepr_plan_destroy(plan):
    lib().sparsepr_plan_destroy(plan)


def sparsepr_workspace_bytes(plan):
    return lib().sparsepr_workspace_bytes(plan)


def sparsepr_plan(plan, q, k, workspace, stream=None):
    _check("sparsepr_plan", lib().sparsepr_plan(plan, _ptr(q), _ptr(k), _ptr(workspace),
                                                workspace.numel() * workspace.element_size(), _stream(stream)))


def sparsepr_plan_static(plan, q, k, stream=None):
    _check("sparsepr_plan_static", lib().sparsepr_plan_static(plan, _ptr(q), _ptr(k), _stream(stream)))


def sparsepr_plan_warm(plan, q, k, workspace, stream=None):
    _check("sparsepr_plan_warm", lib().sparsepr_plan_warm(plan, _ptr(q), _ptr(k), _ptr(workspace),
                                                          workspace.numel() * workspace.element_size(),
                                                          _stream(stream)))


def sparsepr_plan_set_probes(plan, probes, weights, workspace, stream=None):
    _check("sparsepr_plan_set_probes", lib().sparsepr_plan_set_probes(plan, _ptr(probes), _ptr(weights), _ptr(workspace),
                                                                      workspace.numel() * workspace.element_size(),
                                                                      _stream(stream)))


def sparsepr_plan_from_labels(plan, q, k, key_labels, query_labels, group_mass, workspace, stream=None):
    _check("sparsepr_plan_from_labels",
           lib().sparsepr_plan_from_labels(plan, _ptr(q), _ptr(k), _ptr(key_labels), _ptr(query_labels),
                                           _ptr(group_mass), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))


def sparsepr_attend(plan, q, k, v, o_sparse, o_probe_sparse, o_probe_dense, stream=None):
    _check("sparsepr_attend", lib().sparsepr_attend(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(o_sparse),
                                                    _ptr(o_probe_sparse), _ptr(o_probe_dense), _stream(stream)))


def sparsepr_fit_residual(plan, o_probe_sparse, o_probe_dense, probe_weights, coeffs, stream=None):
    _check("sparsepr_fit_residual",
           lib().sparsepr_fit_residual(plan, _ptr(o_probe_sparse), _ptr(o_probe_dense), _ptr(probe_weights),
                                       _ptr(coeffs), _stream(stream)))


def sparsepr_apply(plan, o_sparse, o_probe_dense, coeffs, out, stream=None):
    _check("sparsepr_apply", lib().sparsepr_apply(plan, _ptr(o_sparse), _ptr(o_probe_dense), _ptr(coeffs),
                                                  _ptr(out), _stream(stream)))


def sparsepr_dense_attention(plan, q, k, v, out, workspace, stream=None):
    _check("sparsepr_dense_attention",
           lib().sparsepr_dense_attention(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream)))


def sparsepr_plan_info(plan, n_heads, stream=None):
    arr = (sparsepr_head_info * n_heads)()
    _check("sparsepr_plan_info", lib().sparsepr_plan_info(plan, arr, n_heads, _stream(stream)))
    return [{f: getattr(a, f) for f, _ in sparsepr_head_info._fields_} for a in arr]


def sparsepr_export_bytes(plan, which):
    return lib().sparsepr_export_bytes(plan, EXPORT.get(which, which))


def sparsepr_plan_export(plan, which, dst, stream=None):
    w = EXPORT.get(which, which)
    _check("sparsepr_plan_export", lib().sparsepr_plan_export(plan, w, _ptr(dst), dst.numel() * dst.element_size(),
                                                              _stream(stream)))


def sparsepr_set_stage_timing(plan, enable):
    _check("sparsepr_set_stage_timing", lib().sparsepr_set_stage_timing(plan, int(enable)))


def sparsepr_stage_times(plan):
    arr = (ctypes.c_float * len(STAGES))()
    _check("sparsepr_stage_times", lib().sparsepr_stage_times(plan, arr, len(STAGES)))
    return dict(zip(STAGES, list(arr)))


def sparsepr_status_string(status):
    return lib().sparsepr_status_string(status).decode()
