"""Shared GPU-test plumbing: seeded inputs, the oracle's per-head results, GPU exports."""
import math
import sys

import numpy as np
import torch

from free_block_sparse_response_amd import configs, synth
from free_block_sparse_response_amd.call import SparsePR, config_from_workload
from oracle import sparsepr_oracle as O

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(w, heads=None):
    """Torch device tensors [1, H, N, d] in the workload dtype and float64 copies [H, N, d]."""
    q, k, v = synth.make_inputs(w, heads)
    out = []
    for x in (q, k, v):
        t, x64 = synth.cast_to_dtype(x, w["dtype"])
        out.append((t.unsqueeze(0).contiguous().to(DEV), x64))
    return out


def oracle_heads(w, q64, k64, v64, head_ids, labels_only=False, **over):
    p = O.call_params(w)
    p.update(over)
    res = []
    # the library hashes with the flat head index of the launched batch, 0..len-1
    for i, _ in enumerate(head_ids):
        hp = O.plan_head(q64[i], k64[i], p, i, 25, 1e-4)
        res.append(hp if labels_only else O.attend_fit_apply(q64[i], k64[i], v64[i], p, hp))
    return res


def gpu_from_labels(w, tq, tk, tv, plans, **over):
    cfg = config_from_workload(w, heads=len(plans), **over)
    sp = SparsePR(cfg, device=DEV)
    kl = torch.from_numpy(np.stack([p.key_labels for p in plans]).astype(np.int32)).to(DEV)
    ql = torch.from_numpy(np.stack([p.query_labels for p in plans]).astype(np.int32)).to(DEV)
    Ck, Cq = cfg["n_key_groups"], cfg["n_query_groups"]
    u = np.zeros((len(plans), Cq, Ck), dtype=np.int64)
    for i, p in enumerate(plans):
        u[i, :p.u.shape[0], :p.u.shape[1]] = p.u
    sp.plan(tq, tk, kl, ql, torch.from_numpy(u).to(DEV))
    sp.attend(tq, tk, tv)
    sp.fit_residual()
    sp.apply()
    torch.cuda.synchronize()
    return sp


def np_(t):
    return t.detach().to(torch.float64).cpu().numpy() if t.is_floating_point() else t.cpu().numpy()


def check_integer_plan(sp, plans):
    """Bit-exact comparison of every integer product of the plan with the oracle's."""
    ex = {k: np_(sp.export(k)) for k in ("KEY_LABELS", "QUERY_LABELS", "KEY_PERM", "QUERY_PERM", "KEY_OFFSETS",
                                         "QUERY_OFFSETS", "ROUTE_ROWPTR", "ROUTE_COLS", "PROBES", "PROBE_WEIGHTS")}
    info = sp.info()
    for i, p in enumerate(plans):
        assert info[i]["key_groups"] == p.Ck and info[i]["query_groups"] == p.Cq
        assert np.array_equal(ex["KEY_LABELS"][i], p.key_labels)
        assert np.array_equal(ex["QUERY_LABELS"][i], p.query_labels)
        assert np.array_equal(ex["KEY_PERM"][i], p.k_perm)
        assert np.array_equal(ex["QUERY_PERM"][i], p.q_perm)
        assert np.array_equal(ex["KEY_OFFSETS"][i][:p.Ck + 1], p.k_off)
        assert np.array_equal(ex["QUERY_OFFSETS"][i][:p.Cq + 1], p.q_off)
        assert np.array_equal(ex["ROUTE_ROWPTR"][i][:p.Cq + 1], p.route.row_ptr)
        assert np.array_equal(ex["ROUTE_COLS"][i][:p.route.row_ptr[-1]], p.route.cols)
        assert info[i]["tau"] == p.route.tau and info[i]["budget"] == p.route.budget
        assert info[i]["budget_exceeded"] == int(p.route.budget_exceeded)
        assert info[i]["executed_pairs"] == p.pairs
        assert np.array_equal(ex["PROBES"][i], p.probes)
        np.testing.assert_allclose(ex["PROBE_WEIGHTS"][i], p.weights, rtol=1e-6)
    return info


def max_rel(a, b):
    return float(O.rel_l2(a, b).max()) if len(a) else 0.0
