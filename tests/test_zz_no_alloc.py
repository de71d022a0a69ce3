"""sparsepr_plan_static (plan state in the library's static device array, no allocation)
against sparsepr_plan with a caller workspace, through the C ABI: two calls in a row on
one GPU, the second with a smaller input, each compared output for output."""
import numpy as np
import pytest
import torch

from free_block_sparse_response_amd import _lib as L
from free_block_sparse_response_amd import configs
from free_block_sparse_response_amd.call import config_from_workload

from gpu_helpers import DEV, inputs, say

pytestmark = pytest.mark.gpu

KINDS = ("KEY_LABELS", "QUERY_LABELS", "KEY_PERM", "QUERY_PERM", "ROUTE_ROWPTR", "ROUTE_COLS", "PROBES",
         "PROBE_WEIGHTS", "GROUP_MASS")


def _handle(c):
    return L.sparsepr_plan_create(L.make_config(
        c["batch"], c["heads"], c["seq_len"], c["head_dim"], c["dtype"], c["n_sampled"], c["n_key_groups"],
        c["n_query_groups"], c["n_probes"], c["density"], c["kmeans_max_iter"], c["kmeans_tol"],
        c["ridge_lambda"], 0, c["seed"], c["softmax_scale"]))


def _outputs(c, tq):
    B, H, N, d, M = c["batch"], c["heads"], c["seq_len"], c["head_dim"], max(c["n_probes"], 1)
    return dict(o_sparse=torch.empty_like(tq), o_psp=torch.empty((B, H, M, d), dtype=torch.float32, device=DEV),
                o_pdn=torch.empty((B, H, M, d), dtype=torch.float32, device=DEV),
                coeffs=torch.empty((B, H, d + 1, d), dtype=torch.float32, device=DEV), out=torch.empty_like(tq))


def _rest_of_call(h, tq, tk, tv, o):
    L.sparsepr_attend(h, tq, tk, tv, o["o_sparse"], o["o_psp"], o["o_pdn"])
    L.sparsepr_fit_residual(h, o["o_psp"], o["o_pdn"], None, o["coeffs"])
    L.sparsepr_apply(h, o["o_sparse"], o["o_pdn"], o["coeffs"], o["out"])


_DT = {"PROBE_WEIGHTS": torch.float32, "GROUP_MASS": torch.int64}


def _exports(h, c, info):
    """The defined part of each plan export, per head (exports are sized for the requested
    group counts; entries past the realised groups and selected cells are not written)."""
    res = {}
    for k in KINDS:
        dt = _DT.get(k, torch.int32)
        n = L.sparsepr_export_bytes(h, k) // torch.tensor([], dtype=dt).element_size()
        dst = torch.empty(n, dtype=dt, device=DEV)
        L.sparsepr_plan_export(h, k, dst)
        res[k] = dst.reshape(c["heads"], -1)
    rows = []
    for i, inf in enumerate(info):
        ck, cq = inf["key_groups"], inf["query_groups"]
        rp = res["ROUTE_ROWPTR"][i][:cq + 1]
        mass = res["GROUP_MASS"][i].reshape(c["n_query_groups"], c["n_key_groups"])[:cq, :ck]
        rows.append([res[k][i] for k in ("KEY_LABELS", "QUERY_LABELS", "KEY_PERM", "QUERY_PERM", "PROBES",
                                         "PROBE_WEIGHTS")] + [rp, res["ROUTE_COLS"][i][:int(rp[-1])], mass])
    return rows


def _compare(w, label):
    c = config_from_workload(w)
    hs, hw = _handle(c), _handle(c)
    try:
        say(f"case: static-workspace plan vs caller workspace, {label} ({L.sparsepr_workspace_bytes(hs) >> 20} MiB)")
        (tq, _), (tk, _), (tv, _) = inputs(w)
        os_, ow = _outputs(c, tq), _outputs(c, tq)
        L.sparsepr_plan_static(hs, tq, tk)
        _rest_of_call(hs, tq, tk, tv, os_)
        ws = torch.empty(L.sparsepr_workspace_bytes(hw), dtype=torch.uint8, device=DEV)
        L.sparsepr_plan(hw, tq, tk, ws)
        _rest_of_call(hw, tq, tk, tv, ow)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: bit-identical plans and outputs
        info_s, info_w = L.sparsepr_plan_info(hs, c["heads"]), L.sparsepr_plan_info(hw, c["heads"])
        assert info_s == info_w and all(i["status"] == 0 for i in info_s)
        for i, (a, b) in enumerate(zip(_exports(hs, c, info_s), _exports(hw, c, info_w))):
            for k, (x, y) in enumerate(zip(a, b)):
                assert torch.equal(x, y), (i, k)
        for k in ("o_sparse", "o_psp", "o_pdn", "coeffs", "out"):
            assert torch.equal(os_[k], ow[k]), k
        say(f"  identical: {len(KINDS)} plan exports, 5 outputs; iterations {[(i['key_iters'], i['query_iters']) for i in info_s]}")
    finally:
        L.sparsepr_plan_destroy(hs)
        L.sparsepr_plan_destroy(hw)


def test_static_workspace_plan_matches_caller_workspace_twice():
    # first the 8-head, 16,384-token workload (110 MiB of plan state), then a smaller call on
    # the same array, which still holds the first call's contents
    _compare(configs.CONFIGS["c2"], "8 x 16,384")
    _compare(configs.with_overrides("c2", heads=3, grid=(6, 20, 24), n_key_groups=40, n_query_groups=24,
                                    n_sampled=128, n_probes=96, density=0.25), "3 x 2,880")


def test_static_workspace_refuses_a_larger_plan():
    c = config_from_workload(configs.CONFIGS["c3"])
    h = _handle(c)
    try:
        assert L.sparsepr_workspace_bytes(h) > L.STATIC_WORKSPACE_BYTES
        x = torch.empty((1, 1), dtype=torch.bfloat16, device=DEV)   # never read: refused on the host
        with pytest.raises(L.SparsePRError) as e:
            L.sparsepr_plan_static(h, x, x)
        assert e.value.status == L.SPARSEPR_ERR_TOO_LARGE
    finally:
        L.sparsepr_plan_destroy(h)
