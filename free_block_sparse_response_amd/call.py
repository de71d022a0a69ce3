"""The SparsePR call as one object: owns the plan handle and the torch-allocated buffers.

Device memory comes from PyTorch; every step runs in libsparsepr.so (see _lib).
"""
from __future__ import annotations

import math

import torch

from . import _lib as L

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
_EXPORT_DTYPE = {"PROBE_WEIGHTS": torch.float32, "GROUP_MASS": torch.int64, "KEY_CENTROIDS": torch.float32}


class SparsePR:
    """One SparsePR configuration: shapes, planner sizes, density and ridge settings.

    ``cfg`` keys: batch, heads, seq_len, head_dim, dtype ("f32" / "bf16"), n_sampled,
    n_key_groups, n_query_groups, n_probes, density, ridge_lambda, seed and optionally
    kmeans_max_iter, kmeans_tol, penalize_bias, softmax_scale, assign_precision, warm_iters,
    partition, correction, probe_selector (comparison settings; 0 = the method), key_rank.
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
                                 c.get("correction", 0), c.get("probe_selector", 0), c.get("key_rank", 0))
        self.plan_h = L.sparsepr_plan_create(self._cc)
        self.ws = torch.empty(L.sparsepr_workspace_bytes(self.plan_h), dtype=torch.uint8, device=device)
        shape = (c["batch"], c["heads"], self.N, self.d)
        self.o_sparse = torch.empty(shape, dtype=self.dtype, device=device)
        pshape = (c["batch"], c["heads"], max(self.M, 1), self.d)
        self.o_probe = torch.empty(pshape, dtype=torch.float32, device=device)
        self.o_probe_sparse = torch.empty(pshape, dtype=torch.float32, device=device)
        self.coeffs = torch.empty((c["batch"], c["heads"], self.d + 1, self.d), dtype=torch.float32, device=device)
        self.out = torch.empty(shape, dtype=self.dtype, device=device)

    def __del__(self):
        h = getattr(self, "plan_h", None)
        if h is not None:
            L.sparsepr_plan_destroy(h)
            self.plan_h = None

    # the four stages
    def plan(self, q, k, key_labels=None, query_labels=None, group_mass=None, warm=False):
        if warm:
            L.sparsepr_plan_warm(self.plan_h, q, k, self.ws)
        elif key_labels is None:
            L.sparsepr_plan(self.plan_h, q, k, self.ws)
        else:
            L.sparsepr_plan_from_labels(self.plan_h, q, k, key_labels, query_labels, group_mass, self.ws)

    def set_probes(self, probes, weights=None):
        """Replace the current plan's probe rows ([B*H, M] int32 device; unit weights if None)."""
        L.sparsepr_plan_set_probes(self.plan_h, probes, weights, self.ws)

    def attend(self, q, k, v):
        m = self.M > 0
        L.sparsepr_attend(self.plan_h, q, k, v, self.o_sparse, self.o_probe_sparse if m else None,
                          self.o_probe if m else None)

    def fit_residual(self, probe_weights=None):
        m = self.M > 0
        L.sparsepr_fit_residual(self.plan_h, self.o_probe_sparse if m else None, self.o_probe if m else None,
                                probe_weights, self.coeffs)

    def apply(self, out=None):
        L.sparsepr_apply(self.plan_h, self.o_sparse, self.o_probe if self.M else None, self.coeffs,
                         self.out if out is None else out)

    def __call__(self, q, k, v, warm=False):
        """One call; warm=True starts the planner from the previous call's groups."""
        self.plan(q, k, warm=warm)
        self.attend(q, k, v)
        self.fit_residual()
        self.apply()
        return self.out

    def dense(self, q, k, v, out):
        L.sparsepr_dense_attention(self.plan_h, q, k, v, out, self.ws)
        return out

    # read-back helpers (synchronise)
    def info(self):
        return L.sparsepr_plan_info(self.plan_h, self.BH)

    def export(self, which):
        n = L.sparsepr_export_bytes(self.plan_h, which)
        dt = _EXPORT_DTYPE.get(which, torch.int32)
        esz = torch.tensor([], dtype=dt).element_size()
        dst = torch.empty(max(n // esz, 1), dtype=dt, device=self.ws.device)
        L.sparsepr_plan_export(self.plan_h, which, dst)
        return dst[: n // esz].reshape(self.BH, -1)


def config_from_workload(w, **over):
    """Library config of a workload description (configs.CONFIGS entry)."""
    from .configs import KMEANS_MAX_ITER, KMEANS_TOL, seq_len

    c = dict(batch=w["batch"], heads=w["heads"], seq_len=seq_len(w), head_dim=w["head_dim"], dtype=w["dtype"],
             n_sampled=w["n_sampled"], n_key_groups=w["n_key_groups"], n_query_groups=w["n_query_groups"],
             n_probes=w["n_probes"], density=w["density"], ridge_lambda=w["ridge_lambda"], seed=w["seed"],
             kmeans_max_iter=KMEANS_MAX_ITER, kmeans_tol=KMEANS_TOL,
             softmax_scale=w.get("scale", 1.0 / math.sqrt(w["head_dim"])))
    for key in ("partition", "correction", "probe_selector", "key_rank"):
        if key in w:
            c[key] = w[key]
    c.update(over)
    return c
