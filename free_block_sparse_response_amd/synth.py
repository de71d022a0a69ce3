"""Seeded synthetic video-token inputs for the SparsePR call.

This module holds no step of the method: it only draws Q, K, V. Both the oracle tests
and the GPU path consume what it returns, so that the two sides see identical inputs.

The pages measure on real activations of four video models; those are not available,
so clustered spatio-temporal mixtures stand in for them, with the models' sequence
lengths (Table C.2 of the paper lists N_q = 75,600 for Wan2.2 and 118,800 for
HunyuanVideo).

Recipe, per (batch, head) substream of ``numpy.random.SeedSequence(seed)``:
  * token n of a (T, H, W) grid is (t, h, w) in raster order; its mixture cell is
    ((t*cT//T)*cH + h*cH//H)*cW + w*cW//W for cell counts (cT, cH, cW);
  * each cell c draws a direction u_c uniform on the unit sphere; Q and K share the
    cell mean 3*u_c (so a query attends most to keys of its own cell), V uses an
    independent mean 3*u'_c;
  * with ``drift`` the Q/K mean moves linearly over time from 3*u_c to 3*u''_c;
  * every token adds N(0, 0.5^2 I) noise independently to Q, K and V;
  * ``sink_frac`` of the tokens, picked by the same generator, get their K scaled x3;
  * ``text_tokens`` extra tokens are appended with Q, K, V i.i.d. uniform on (-1, 1).
Values are drawn in float64 and cast once to the workload dtype; every consumer reads
the cast values.
"""
from __future__ import annotations

import numpy as np

MEAN_NORM = 3.0
NOISE_SIGMA = 0.5


def _unit_rows(rng, n, d):
    u = rng.standard_normal((n, d))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def cell_labels(grid, cells):
    T, H, W = grid
    cT, cH, cW = cells
    t = np.arange(T)[:, None, None] * cT // T
    h = np.arange(H)[None, :, None] * cH // H
    w = np.arange(W)[None, None, :] * cW // W
    return ((t * cH + h) * cW + w).reshape(-1)


def head_inputs(cfg, rng):
    """Q, K, V float64 arrays [N, d] of one head, drawn from ``rng``."""
    T, H, W = cfg["grid"]
    d = cfg["head_dim"]
    cells = cfg["cells"]
    ncell = cells[0] * cells[1] * cells[2]
    lab = cell_labels(cfg["grid"], cells)
    nv = T * H * W
    u = _unit_rows(rng, ncell, d)
    uv = _unit_rows(rng, ncell, d)
    if cfg.get("drift", False):
        u2 = _unit_rows(rng, ncell, d)
        t = (np.arange(nv) // (H * W)).astype(np.float64)
        f = (t / max(T - 1, 1))[:, None]
        mean_qk = MEAN_NORM * ((1.0 - f) * u[lab] + f * u2[lab])
    else:
        mean_qk = MEAN_NORM * u[lab]
    q = mean_qk + NOISE_SIGMA * rng.standard_normal((nv, d))
    k = mean_qk + NOISE_SIGMA * rng.standard_normal((nv, d))
    v = MEAN_NORM * uv[lab] + NOISE_SIGMA * rng.standard_normal((nv, d))
    sf = cfg.get("sink_frac", 0.0)
    if sf > 0:
        sinks = rng.choice(nv, size=int(round(sf * nv)), replace=False)
        k[sinks] *= 3.0
    nt = cfg.get("text_tokens", 0)
    if nt:
        q = np.concatenate([q, rng.uniform(-1.0, 1.0, (nt, d))])
        k = np.concatenate([k, rng.uniform(-1.0, 1.0, (nt, d))])
        v = np.concatenate([v, rng.uniform(-1.0, 1.0, (nt, d))])
    return q, k, v


def head_streams(cfg):
    ss = np.random.SeedSequence(cfg["seed"])
    return [np.random.default_rng(s) for s in ss.spawn(cfg["batch"] * cfg["heads"])]


def make_inputs(cfg, heads=None):
    """Float64 Q, K, V of shape [B*H_sel, N, d] for the selected flat head ids.

    ``heads`` (default: all B*H) picks flat (batch*H + head) ids; each head's values
    depend only on the seed and its id, so a subset equals the same slice of the whole.
    """
    rngs = head_streams(cfg)
    sel = range(len(rngs)) if heads is None else heads
    out = [head_inputs(cfg, rngs[h]) for h in sel]
    return tuple(np.stack([o[i] for o in out]) for i in range(3))


def cast_to_dtype(x, dtype):
    """Round a float64 array to the workload dtype; returns (torch tensor, float64 copy)."""
    import torch

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(x)).to(tdt)
    return t, t.to(torch.float64).numpy()
