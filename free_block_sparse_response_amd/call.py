"""The SparsePR call as one object: owns the plan handle and the torch-allocated buffers.

Device memory comes from PyTorch; every step runs in libsparsepr.so (see _lib).
"""
from __future__ import annotations

import math

import torch

from . import _lib as L

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
_EXPORT_DTYPE = {"PROBE_WEIGHTS": torch.float32, "GROUP_MASS": torch.int64, "KEY_CENTROIDS": torch.float32}


def check_tensor(t, name, shapes, dtype, device_type="cuda"):
    """Refuses a tensor the library cannot read as the layout it documents.

    The kernels take raw device pointers, so a tensor on another device, of another
    element type, non-contiguous (a transposed [B, N, H, d] view, say) or of another
    shape would be misread or read out of bounds. ``shapes`` lists the accepted shapes.
    Raises ValueError; checks only, no arithmetic.
    """
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != device_type:
        raise ValueError(f"{name}: expected a {device_type} tensor, got one on {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) not in [tuple(s) for s in shapes]:
        raise ValueError(f"{name}: expected shape {' or '.join(str(tuple(s)) for s in shapes)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor (row-major {tuple(t.shape)})")
    return t


class SparsePR:
    """One SparsePR configuration: shapes, planner sizes, density and ridge settings.

    ``cfg`` keys: batch, heads, seq_len, head_dim, dtype ("f32" / "bf16"), n_sampled,
    n_key_groups, n_query_groups, n_probes, density, ridge_lambda, seed and optionally
    kmeans_max_iter, kmeans_tol, penalize_bias, softmax_scale, assign_precision, warm_iters,
    partition, correction, probe_selector (comparison settings; 0 = the method), key_rank,
    attn_tile_rows (128 / 256; 0 = chosen by the size of the call), output_rank (residual fit
    truncated to that many probe-residual directions; 0 = none).
    """

    def __init__(self, cfg, device="cuda"):
        self.cfg = dict(cfg)
        c = self.cfg
        self.BH = c["batch"] * c["heads"]
        self.N, self.d, self.M = c["seq_len"], c["head_dim"], c["n_probes"]
        self.dtype = _DT[c["dtype"]]
        self._cc = L.make_config(c["batch"], c["heads"], c["seq_len"], c["head_dim"], c["dtype"], c["n_sampled"],
                                 c["n_key_groups"], c["n_query_groups"], c["n_probes"], c["density"],
                                 c.get("kmeans_max_iter", 25), c.get("kmeans_tol", 1e-4), c.get("ridge_lambda", 1e-3),
                                 c.get("penalize_bias", 0), c.get("seed", 0), c.get("softmax_scale", 0.0),
                                 c.get("assign_precision", 0), c.get("warm_iters", 2), c.get("partition", 0),
                                 c.get("correction", 0), c.get("probe_selector", 0), c.get("key_rank", 0),
                                 c.get("attn_tile_rows", 0), c.get("output_rank", 0))
        self.plan_h = L.sparsepr_plan_create(self._cc)
        self.ws = torch.empty(L.sparsepr_workspace_bytes(self.plan_h), dtype=torch.uint8, device=device)
        shape = (c["batch"], c["heads"], self.N, self.d)
        self.o_sparse = torch.empty(shape, dtype=self.dtype, device=device)
        pshape = (c["batch"], c["heads"], max(self.M, 1), self.d)
        self.o_probe = torch.empty(pshape, dtype=torch.float32, device=device)
        self.o_probe_sparse = torch.empty(pshape, dtype=torch.float32, device=device)
        self.coeffs = torch.empty((c["batch"], c["heads"], self.d + 1, self.d), dtype=torch.float32, device=device)
        self.out = torch.empty(shape, dtype=self.dtype, device=device)
        self._shape = shape
        self._dev = torch.device(device).type

    def close(self):
        """Releases the plan handle: stage timing off first (its HIP events are destroyed
        while the runtime is certainly alive), then the handle. Later calls raise; a second
        close() and the finaliser do nothing."""
        h = getattr(self, "plan_h", None)
        if h is not None:
            self.plan_h = None
            L.sparsepr_set_stage_timing(h, 0)
            L.sparsepr_plan_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown: the binding may already be gone
            pass

    def _handle(self):
        if self.plan_h is None:
            raise RuntimeError("SparsePR: the plan was closed")
        return self.plan_h

    def _qkv(self, *ts):
        for name, t in zip("qkv", ts):
            check_tensor(t, name, [self._shape], self.dtype, self._dev)

    def _rows(self, t, name, width, dtype):
        c = self.cfg
        return check_tensor(t, name, [(self.BH, width), (c["batch"], c["heads"], width)], dtype, self._dev)

    # the four stages
    def plan(self, q, k, key_labels=None, query_labels=None, group_mass=None, warm=False):
        self._qkv(q, k)
        h = self._handle()
        if warm:
            L.sparsepr_plan_warm(h, q, k, self.ws)
        elif key_labels is None:
            L.sparsepr_plan(h, q, k, self.ws)
        else:
            c = self.cfg
            self._rows(key_labels, "key_labels", self.N, torch.int32)
            self._rows(query_labels, "query_labels", self.N, torch.int32)
            if group_mass is not None:
                check_tensor(group_mass, "group_mass", [(self.BH, c["n_query_groups"], c["n_key_groups"]),
                                                        (c["batch"], c["heads"], c["n_query_groups"],
                                                         c["n_key_groups"])], torch.int64, self._dev)
            L.sparsepr_plan_from_labels(h, q, k, key_labels, query_labels, group_mass, self.ws)

    def set_probes(self, probes, weights=None):
        """Replace the current plan's probe rows ([B*H, M] int32 device; unit weights if None)."""
        self._rows(probes, "probes", self.M, torch.int32)
        if weights is not None:
            self._rows(weights, "weights", self.M, torch.float32)
        L.sparsepr_plan_set_probes(self._handle(), probes, weights, self.ws)

    def attend(self, q, k, v):
        self._qkv(q, k, v)
        m = self.M > 0
        L.sparsepr_attend(self._handle(), q, k, v, self.o_sparse, self.o_probe_sparse if m else None,
                          self.o_probe if m else None)

    def fit_residual(self, probe_weights=None):
        if probe_weights is not None:
            self._rows(probe_weights, "probe_weights", self.M, torch.float32)
        m = self.M > 0
        L.sparsepr_fit_residual(self._handle(), self.o_probe_sparse if m else None, self.o_probe if m else None,
                                probe_weights, self.coeffs)

    def apply(self, out=None):
        if out is not None:
            check_tensor(out, "out", [self._shape], self.dtype, self._dev)
        L.sparsepr_apply(self._handle(), self.o_sparse, self.o_probe if self.M else None, self.coeffs,
                         self.out if out is None else out)

    def __call__(self, q, k, v, warm=False):
        """One call; warm=True starts the planner from the previous call's groups."""
        self.plan(q, k, warm=warm)
        self.attend(q, k, v)
        self.fit_residual()
        self.apply()
        return self.out

    def dense(self, q, k, v, out):
        self._qkv(q, k, v)
        check_tensor(out, "out", [self._shape], self.dtype, self._dev)
        L.sparsepr_dense_attention(self._handle(), q, k, v, out, self.ws)
        return out

    # read-back helpers (synchronise)
    def info(self):
        return L.sparsepr_plan_info(self._handle(), self.BH)

    def export(self, which):
        n = L.sparsepr_export_bytes(self._handle(), which)
        dt = _EXPORT_DTYPE.get(which, torch.int32)
        esz = torch.tensor([], dtype=dt).element_size()
        dst = torch.empty(max(n // esz, 1), dtype=dt, device=self.ws.device)
        L.sparsepr_plan_export(self._handle(), which, dst)
        return dst[: n // esz].reshape(self.BH, -1)


def config_from_workload(w, **over):
    """Library config of a workload description (configs.CONFIGS entry)."""
    from .configs import KMEANS_MAX_ITER, KMEANS_TOL, seq_len

    c = dict(batch=w["batch"], heads=w["heads"], seq_len=seq_len(w), head_dim=w["head_dim"], dtype=w["dtype"],
             n_sampled=w["n_sampled"], n_key_groups=w["n_key_groups"], n_query_groups=w["n_query_groups"],
             n_probes=w["n_probes"], density=w["density"], ridge_lambda=w["ridge_lambda"], seed=w["seed"],
             kmeans_max_iter=KMEANS_MAX_ITER, kmeans_tol=KMEANS_TOL,
             softmax_scale=w.get("scale", 1.0 / math.sqrt(w["head_dim"])))
    for key in ("partition", "correction", "probe_selector", "key_rank", "attn_tile_rows", "output_rank"):
        if key in w:
            c[key] = w[key]
    c.update(over)
    return c
