"""sparsepr_fit_residual on given probe outputs against the oracle's weighted ridge (float64
normal equations solved by Cholesky), through the C ABI.

The probe buffers are filled with seeded data (a planted affine residual plus noise), so the
comparison covers the Gram build and the solve alone: both sides start from the same float32
values, so the coefficients may differ only by float64 rounding in the solve and the final
rounding to float32.
"""
import numpy as np
import pytest
import torch

from free_block_sparse_response_amd import configs
from free_block_sparse_response_amd.call import SparsePR, config_from_workload
from oracle import sparsepr_oracle as O

from gpu_helpers import DEV, inputs, np_, say

pytestmark = pytest.mark.gpu

# (head_dim, probes, lambda, penalize bias): fewer probes than unknowns (the ridge term makes
# the system definite), more, a ragged probe count over several 32-probe chunks, a
# penalised bias
CASES = [(64, 32, 1e-3, 0), (64, 200, 1e-3, 0), (128, 96, 0.1, 1), (128, 333, 1e-3, 0), (128, 1024, 1e-3, 0)]


def _probe_data(heads, M, d, seed):
    rng = np.random.default_rng(seed)
    o_sp = rng.standard_normal((heads, M, d)).astype(np.float32)
    theta = rng.standard_normal((heads, d + 1, d)) / np.sqrt(d)
    o_dn = (o_sp.astype(np.float64) + np.einsum("hmi,hij->hmj", o_sp.astype(np.float64), theta[:, :d])
            + theta[:, d][:, None, :] + 0.1 * rng.standard_normal((heads, M, d))).astype(np.float32)
    w = rng.uniform(0.5, 2.0, (heads, M)).astype(np.float32)
    return o_sp, o_dn, w


@pytest.mark.parametrize("d,M,lam,pen", CASES)
def test_fit_matches_oracle_ridge(d, M, lam, pen):
    heads = 3
    say(f"case: fit d={d} M={M} lambda={lam} penalize_bias={pen} heads={heads}")
    w = configs.with_overrides("c1", head_dim=d, heads=heads, grid=(4, 16, 32), n_probes=M, density=0.9)
    cfg = config_from_workload(w, ridge_lambda=lam, penalize_bias=pen)
    sp = SparsePR(cfg, device=DEV)
    (tq, _), (tk, _), _ = inputs(w)
    sp.plan(tq, tk)
    o_sp, o_dn, wt = _probe_data(heads, M, d, 1234 + d + M)
    sp.o_probe_sparse.copy_(torch.from_numpy(o_sp).reshape(sp.o_probe_sparse.shape))
    sp.o_probe.copy_(torch.from_numpy(o_dn).reshape(sp.o_probe.shape))
    sp.fit_residual(torch.from_numpy(wt).to(DEV))
    torch.cuda.synchronize()
    th = np_(sp.coeffs[0])
    assert all(i["status"] == 0 for i in sp.info())
    for h in range(heads):
        ref = O.ridge_fit(o_sp[h].astype(np.float64), o_dn[h].astype(np.float64), wt[h], lam, penalize_bias=bool(pen))
        err = np.abs(th[h] - ref).max() / np.abs(ref).max()
        say(f"  head {h}: max |theta - ref| / max |ref| = {err:.2e}")
        assert err <= 2e-6
    sp.close()
