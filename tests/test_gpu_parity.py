"""GPU parity: the HIP path against the CPU oracle, element by element.

Integer products (labels, permutations, offsets, route, probes) must match bit for bit
given the oracle's partition; float outputs must match per query within rel-L2 1e-4
(fp32) or 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

from free_block_sparse_response_amd import _lib as L
from free_block_sparse_response_amd import configs
from free_block_sparse_response_amd.call import SparsePR, config_from_workload
from oracle import sparsepr_oracle as O

from gpu_helpers import (DEV, check_integer_plan, gpu_from_labels, inputs, max_rel, np_, oracle_heads, say)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _parity_from_labels(w, heads, **over):
    say(f"case: from-labels {w['dtype']} N={configs.seq_len(w)} d={w['head_dim']} heads={heads} {over}")
    (tq, q64), (tk, k64), (tv, v64) = inputs(w, heads)
    refs = oracle_heads(w, q64, k64, v64, heads, **over)
    sp = gpu_from_labels(w, tq, tk, tv, [r.plan for r in refs], **over)
    check_integer_plan(sp, [r.plan for r in refs])
    tol = TOL[w["dtype"]]
    o_sp = np_(sp.o_sparse[0])
    o_pr = np_(sp.o_probe[0])
    o_psp = np_(sp.o_probe_sparse[0])
    out = np_(sp.out[0])
    for i, r in enumerate(refs):
        M = len(r.plan.probes)
        e_sp = max_rel(o_sp[i], r.o_sparse)
        e_pr = max_rel(o_pr[i][:M], r.o_probe_dense)
        e_psp = max_rel(o_psp[i][:M], r.o_sparse[r.plan.probes])
        e_out = max_rel(out[i], r.out)
        say(f"  head {heads[i]}: o_sparse {e_sp:.2e} probe sparse {e_psp:.2e} probe dense {e_pr:.2e} "
            f"out {e_out:.2e}")
        assert e_sp <= tol and e_pr <= tol and e_out <= tol and e_psp <= tol
        # probe rows carry their exact dense output (bit-equal to the probe buffer)
        assert np.array_equal(out[i][r.plan.probes], o_pr[i][:M].astype(out.dtype)) or w["dtype"] == "bf16"
    return sp, refs


def test_c1_fp32_from_labels():
    _parity_from_labels(configs.CONFIGS["c1"], [0])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_tiny_sequence(dtype, d):
    # 42 tokens: fewer than one 64-key tile, one 128-row Lloyd block and one attention tile,
    # ragged everywhere; the oracle's partition given, then the library's own plan
    w = configs.with_overrides("c1", grid=(2, 3, 7), head_dim=d, heads=2, dtype=dtype, n_sampled=8,
                               n_key_groups=4, n_query_groups=4, n_probes=3, density=0.5)
    sp, refs = _parity_from_labels(w, [0, 1])
    sp.close()
    (tq, q64), (tk, k64), (tv, v64) = inputs(w, [0, 1])
    sp = SparsePR(config_from_workload(w), device=DEV)
    sp(tq, tk, tv)
    torch.cuda.synchronize()
    out, info = np_(sp.out[0]), sp.info()
    p = O.call_params(w)
    for i, r in enumerate(refs):
        dn = O.dense_attention(q64[i], k64[i], v64[i], p["scale"])
        e_g, e_o = O.rel_l2(out[i], dn).mean(), O.rel_l2(r.out, dn).mean()
        say(f"  own plan head {i}: groups {info[i]['key_groups']}/{info[i]['query_groups']} (oracle "
            f"{r.plan.Ck}/{r.plan.Cq}), mean error {e_g:.4f} (oracle's own plan {e_o:.4f})")
        assert np.isfinite(out[i]).all()
        # the two k-means part only on near ties: as for the larger own-plan tests, the mean
        # error within 5% of the oracle's own plan's (measured: within 0.1%, same groups)
        assert abs(e_g - e_o) <= 0.05 * e_o
    sp.close()


def test_c1_fp32_d128_ragged():
    w = configs.with_overrides("c1", grid=(3, 15, 17), head_dim=128, heads=2)
    _parity_from_labels(w, [0, 1])


def test_c2_bf16_two_heads_from_labels():
    w = configs.CONFIGS["c2"]
    _parity_from_labels(w, [0, 5])


def test_bf16_d64_ragged_small():
    w = configs.with_overrides("c2", grid=(5, 13, 19), head_dim=64, heads=3, n_sampled=64, n_key_groups=24,
                               n_query_groups=20, n_probes=40, density=0.3)
    _parity_from_labels(w, [0, 1, 2])


def test_full_density_is_dense():
    w = configs.CONFIGS["c1"]
    N = configs.seq_len(w)
    sp, refs = _parity_from_labels(w, [0], density=1.0 + w["n_probes"] / N)
    dn = O.dense_attention(*[x for x in _dense_inputs(w)], 1 / 8.0)
    assert max_rel(np_(sp.o_sparse[0][0]), dn) <= 1e-4


def _dense_inputs(w):
    (_, q64), (_, k64), (_, v64) = inputs(w, [0])
    return q64[0], k64[0], v64[0]


def test_tight_budget_keeps_top1_and_flags():
    w = configs.CONFIGS["c1"]
    sp, refs = _parity_from_labels(w, [0], density=0.02)
    assert refs[0].plan.route.budget_exceeded
    assert sp.info()[0]["budget_exceeded"] == 1


def test_single_groups_equal_dense():
    w = configs.with_overrides("c1", n_key_groups=1, n_query_groups=1)
    sp, refs = _parity_from_labels(w, [0])
    q, k, v = _dense_inputs(w)
    assert max_rel(np_(sp.o_sparse[0][0]), O.dense_attention(q, k, v, 1 / 8.0)) <= 1e-4


def test_dense_entry_point_matches_oracle():
    for w in (configs.CONFIGS["c1"], configs.with_overrides("c2", heads=2, grid=(4, 16, 16))):
        say(f"case: dense {w['dtype']}")
        (tq, q64), (tk, k64), (tv, v64) = inputs(w, [0, 1][: w["heads"]])
        from free_block_sparse_response_amd.call import SparsePR, config_from_workload

        sp = SparsePR(config_from_workload(w), device=DEV)
        out = torch.empty_like(tq)
        sp.dense(tq, tk, tv, out)
        torch.cuda.synchronize()
        o = np_(out[0])
        for i in range(w["heads"]):
            ref = O.dense_attention(q64[i], k64[i], v64[i], 1 / np.sqrt(w["head_dim"]))
            e = max_rel(o[i], ref)
            say(f"  head {i}: dense rel-L2 {e:.2e}")
            assert e <= TOL[w["dtype"]] / 2


# ------------------------------------------------------------- probe selectors and corrections
@pytest.mark.parametrize("selector", [1, 2])
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_plain_probe_selectors_from_labels(name, selector):
    # random (smallest probe hash over all tokens) and uniform raster-order probes, unit
    # weights: probes bit-exact, outputs within tolerance
    w = configs.CONFIGS[name]
    _parity_from_labels(w, [0] if name == "c1" else [0, 2], probe_selector=selector)


@pytest.mark.parametrize("correction", [1, 2])
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_corrections_from_labels(name, correction):
    w = configs.CONFIGS[name]
    sp, refs = _parity_from_labels(w, [0] if name == "c1" else [1, 4], correction=correction)
    th = np_(sp.coeffs)
    d = w["head_dim"]
    for i, r in enumerate(refs):
        assert np.all(th[0, i, :d] == 0.0)
        # the bias is a mean of probe residuals: its error is bounded by that of the probe rows
        scale = np.abs(r.o_probe_dense).max()
        np.testing.assert_allclose(th[0, i, d], r.theta[d], rtol=0, atol=TOL[w["dtype"]] * scale)
    if correction == 2:
        out, osp = sp.out[0], sp.o_sparse[0]
        for i, r in enumerate(refs):
            un = torch.ones(out.shape[1], dtype=torch.bool, device=out.device)
            un[torch.from_numpy(r.plan.probes).to(out.device)] = False
            assert torch.equal(out[i][un], osp[i][un].to(out.dtype))


def test_caller_probes_from_labels():
    # probe rows given by the caller (any order, unit weights): the oracle's plan with the
    # same injected rows; out-of-range and repeated rows are refused before any launch
    w = configs.CONFIGS["c2"]
    heads = [0, 6]
    say(f"case: caller probes, c2 heads {heads}")
    (tq, q64), (tk, k64), (tv, v64) = inputs(w, heads)
    plans = oracle_heads(w, q64, k64, v64, heads, labels_only=True)
    N, M = configs.seq_len(w), w["n_probes"]
    rng = np.random.default_rng(9)
    inj = [rng.choice(N, M, replace=False) for _ in heads]
    p = O.call_params(w)
    refs = []
    for i, hp in enumerate(plans):
        hp2 = O.finish_plan(q64[i], k64[i], p, i, hp, u=hp.u, probes=inj[i])
        refs.append(O.attend_fit_apply(q64[i], k64[i], v64[i], p, hp2))
    sp = gpu_from_labels(w, tq, tk, tv, plans)
    bad = torch.from_numpy(np.stack(inj).astype(np.int32)).to(DEV)
    bad[1, 3] = bad[1, 7]
    with pytest.raises(L.SparsePRError):
        sp.set_probes(bad)
    bad[1, 3] = N
    with pytest.raises(L.SparsePRError):
        sp.set_probes(bad)
    sp.set_probes(torch.from_numpy(np.stack(inj).astype(np.int32)).to(DEV))
    sp.attend(tq, tk, tv)
    sp.fit_residual()
    sp.apply()
    torch.cuda.synchronize()
    assert np.array_equal(np_(sp.export("PROBES")), np.stack(inj))
    out, o_pr = np_(sp.out[0]), np_(sp.o_probe[0])
    for i, r in enumerate(refs):
        e_out, e_pr = max_rel(out[i], r.out), max_rel(o_pr[i], r.o_probe_dense)
        say(f"  head {heads[i]}: out {e_out:.2e} probe dense {e_pr:.2e}")
        assert e_out <= TOL["bf16"] and e_pr <= TOL["bf16"]


# ------------------------------------------------------------- attention tile heights
@pytest.mark.parametrize("rows", [128, 256])
@pytest.mark.parametrize("case", ["c2", "d64 ragged"])
def test_both_attention_tile_heights(case, rows):
    # 4-wave (128-row) and 8-wave (256-row) block-sparse tiles: the library picks one by the
    # size of the call; both must give the oracle's output (groups larger than a tile, last
    # tiles partly filled, ragged key runs)
    if case == "c2":
        w, heads = configs.CONFIGS["c2"], [2, 7]
    else:
        w = configs.with_overrides("c2", grid=(5, 13, 19), head_dim=64, heads=3, n_sampled=64, n_key_groups=24,
                                   n_query_groups=6, n_probes=40, density=0.3)
        heads = [0, 1, 2]
    _parity_from_labels(w, heads, attn_tile_rows=rows)


# ------------------------------------------------------------- output truncation ([D.2](a))
@pytest.mark.parametrize("name,rank", [("c1", 4), ("c1", 16), ("c2", 8), ("c2", 32)])
def test_output_truncation_from_labels(name, rank):
    # the fitted map's predicted residual projected on the probe residuals' `rank` leading
    # directions (Jacobi in float on the GPU, eigh in the oracle): outputs and coefficients
    # within the workload tolerance; the cut falls in a spectral gap (else the subspace, and
    # with it the reference, is not unique)
    w = configs.CONFIGS[name]
    heads = [0] if name == "c1" else [1, 6]
    sp, refs = _parity_from_labels(w, heads, output_rank=rank)
    th = np_(sp.coeffs[0])
    for i, r in enumerate(refs):
        hp = r.plan
        R = r.o_probe_dense - r.o_sparse[hp.probes]
        ev = np.sort(np.linalg.eigvalsh(R.T @ (hp.weights[:, None] * R)))[::-1]
        say(f"  head {heads[i]}: eigenvalues at the cut {ev[rank - 1]:.4g} / {ev[rank]:.4g}")
        assert ev[rank - 1] > 1.05 * ev[rank]
        scale = np.abs(r.theta).max()
        err = np.abs(th[i] - r.theta).max() / scale
        say(f"  head {heads[i]}: max |Theta - Theta_oracle| / max |Theta_oracle| = {err:.2e}")
        assert err <= TOL[w["dtype"]]
        # the map's output lies in the truncated subspace: Theta P = Theta
        P = O.residual_projector(r.o_sparse[hp.probes], r.o_probe_dense, hp.weights, rank)
        assert np.abs(r.theta - r.theta @ P).max() <= 1e-9 * scale
