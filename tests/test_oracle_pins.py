"""Pins of the CPU oracle against facts fixed outside itself.

Each test ties one oracle function to a published value, a closed form, a library
routine on a special case, or brute force on tiny inputs, chosen so that a plausible
slip (a dropped term, a wrong sign or index, a transposed operand) fails.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import sparsepr_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(path):
    with open(os.path.join(GOLD, path)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- hash and selection
def test_splitmix64_published_vector():
    want = [int(r[0]) for r in _rows("splitmix64_seed1234567.txt")]
    g = 0x9E3779B97F4A7C15
    states = np.array([(1234567 + n * g) % 2 ** 64 for n in range(5)], dtype=np.uint64)
    with np.errstate(over="ignore"):
        got = [int(x) for x in O.splitmix64(states)]
    assert got == want


def test_token_hash_is_nested_splitmix():
    # h(stream, head, i) built from scalar Python big-int arithmetic, independently.
    M64 = 2 ** 64 - 1

    def sm(x):
        z = (x + 0x9E3779B97F4A7C15) & M64
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
        return z ^ (z >> 31)

    for seed, stream, head, i in [(0, 1, 0, 0), (7, 4, 39, 118799), (2 ** 63 + 5, 2, 3, 17)]:
        want = sm(sm(sm(seed ^ stream) ^ head) ^ i)
        assert int(O.token_hash(seed, stream, head, [i])[0]) == want


def test_select_smallest_brute_force():
    cand = np.array([3, 5, 8, 13, 21, 34, 55, 89])
    for m in range(0, 9):
        got = O.select_smallest(11, 2, 5, cand, m)
        h = [int(x) for x in O.token_hash(11, 2, 5, cand)]
        ranked = sorted(zip(h, cand.tolist()))[:m]
        assert got.tolist() == sorted(c for _, c in ranked)


def test_select_smallest_is_uniform_without_replacement():
    # Every candidate is chosen with probability m/n; check over many heads.
    n, m, heads = 40, 10, 2000
    hits = np.zeros(n)
    for h in range(heads):
        s = O.select_smallest(3, 1, h, np.arange(n), m)
        assert len(set(s.tolist())) == m
        hits[s] += 1
    freq = hits / heads
    assert np.all(np.abs(freq - m / n) < 5 * math.sqrt(0.25 * 0.75 / heads))


# ---------------------------------------------------------------- attention
def test_dense_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((37, 16)) for _ in range(3))
    scale = 0.3
    got = O.dense_attention(q, k, v, scale, chunk=8)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=scale)[0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def _tiny_partition(rng, N, Cq, Ck):
    ql = rng.integers(0, Cq, N)
    kl = rng.integers(0, Ck, N)
    ql[:Cq] = np.arange(Cq)
    kl[:Ck] = np.arange(Ck)
    return ql, kl


def test_block_sparse_equals_masked_dense():
    rng = np.random.default_rng(1)
    N, d, Cq, Ck = 50, 8, 4, 5
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    ql, kl = _tiny_partition(rng, N, Cq, Ck)
    sel = rng.random((Cq, Ck)) < 0.5
    sel[np.arange(Cq), rng.integers(0, Ck, Cq)] = True
    qp, qo, _ = O.group_permutation(ql, Cq)
    kp, ko, _ = O.group_permutation(kl, Ck)
    cols = [np.flatnonzero(sel[a]) for a in range(Cq)]
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])])
    got = O.block_sparse_attention(q, k, v, 0.5, qp, qo, kp, ko, rp, np.concatenate(cols))
    # brute force: -inf mask per (query, key) pair from the selected cells
    logits = 0.5 * q @ k.T
    mask = sel[ql][:, kl]
    logits[~mask] = -np.inf
    p = np.exp(logits - logits.max(1, keepdims=True))
    want = (p / p.sum(1, keepdims=True)) @ v
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_block_sparse_all_cells_is_dense():
    rng = np.random.default_rng(2)
    N, d = 40, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    ql, kl = _tiny_partition(rng, N, 3, 4)
    qp, qo, _ = O.group_permutation(ql, 3)
    kp, ko, _ = O.group_permutation(kl, 4)
    rp = np.array([0, 4, 8, 12])
    cols = np.tile(np.arange(4), 3)
    got = O.block_sparse_attention(q, k, v, 0.7, qp, qo, kp, ko, rp, cols)
    np.testing.assert_allclose(got, O.dense_attention(q, k, v, 0.7), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- k-means
def test_sq_dists_matches_direct_differences():
    rng = np.random.default_rng(3)
    x, c = rng.standard_normal((9, 5)), rng.standard_normal((4, 5))
    direct = np.array([[np.sum((xi - cj) ** 2) for cj in c] for xi in x])
    np.testing.assert_allclose(O.sq_dists(x, c), direct, rtol=1e-12, atol=1e-12)


def _lloyd_loops(x, init, max_iter, tol):
    """Textbook Lloyd written with explicit loops (no vector algebra), for tiny inputs."""
    cent = [list(x[i]) for i in init]
    prev, labels, t = None, None, 0
    for t in range(1, max_iter + 1):
        labels, inertia = [], 0.0
        for row in x:
            ds = [sum((a - b) ** 2 for a, b in zip(row, c)) for c in cent]
            j = min(range(len(ds)), key=lambda i: (ds[i], i))
            labels.append(j)
            inertia += ds[j]
        if prev is not None and prev - inertia <= tol * prev:
            break
        if t == max_iter:
            break
        for c in range(len(cent)):
            mem = [x[i] for i in range(len(x)) if labels[i] == c]
            if mem:
                cent[c] = [sum(col) / len(mem) for col in zip(*mem)]
        prev = inertia
    return labels, t


def test_lloyd_matches_loop_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(5):
        x = rng.standard_normal((30, 3)) + rng.integers(0, 3, (30, 1)) * 2.0
        init = rng.choice(30, 4, replace=False)
        r = O.lloyd(x, init, 25, 1e-4)
        lab, it = _lloyd_loops(x, init, 25, 1e-4)
        assert r.labels.tolist() == lab and r.iterations == it


def test_lloyd_inertia_non_increasing_and_fixed_point():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((400, 6))
    r = O.lloyd(x, np.arange(12), 200, 0.0)
    assert all(b <= a * (1 + 1e-12) for a, b in zip(r.inertia, r.inertia[1:]))
    # converged with tol 0: one more update + assignment changes nothing
    cent = O.group_means(x, r.labels, 12)
    assert np.array_equal(np.argmin(O.sq_dists(x, cent), axis=1), r.labels)


def test_lloyd_recovers_planted_partition():
    rng = np.random.default_rng(6)
    C, per, d = 5, 40, 8
    means = rng.standard_normal((C, d)) * 20
    truth = np.repeat(np.arange(C), per)
    x = means[truth] + rng.standard_normal((C * per, d))
    init = [np.flatnonzero(truth == c)[0] for c in range(C)]
    r = O.lloyd(x, init, 25, 1e-4)
    assert np.array_equal(r.labels, truth)


def test_lloyd_stops_on_tolerance_and_cap():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((200, 4))
    assert O.lloyd(x, np.arange(6), 3, 0.0).iterations == 3
    r = O.lloyd(x, np.arange(6), 50, 1e-4)
    i = r.inertia
    assert i[-2] - i[-1] <= 1e-4 * i[-2]
    assert all(a - b > 1e-4 * a for a, b in zip(i[:-2], i[1:-1]))


def test_metric_form_of_key_kmeans_is_exact():
    """Lloyd on R_K = s K Q_S^T equals Lloyd on K under the metric G = s^2 Q_S^T Q_S.

    Every centroid is a mean of response rows, hence s m Q_S^T for a key-space mean m,
    so |R_K,j - c|^2 = (k_j - m) G (k_j - m)^T: both runs choose the same labels.
    """
    rng = np.random.default_rng(8)
    N, d, S, C, s = 300, 6, 10, 7, 0.4
    k = rng.standard_normal((N, d)) + rng.integers(0, 4, (N, 1))
    qs = rng.standard_normal((S, d))
    init = rng.choice(N, C, replace=False)
    lit = O.lloyd(O.key_responses(k, qs, s), init, 25, 1e-4)
    G = s * s * qs.T @ qs
    # metric Lloyd in key space written out directly
    cent = k[init].copy()
    prev, lab = None, None
    for t in range(1, 26):
        diff = k[:, None, :] - cent[None, :, :]
        dist = np.einsum("ncd,de,nce->nc", diff, G, diff)
        lab = dist.argmin(1)
        inertia = dist[np.arange(N), lab].sum()
        if prev is not None and prev - inertia <= 1e-4 * prev:
            break
        if t == 25:
            break
        for c in range(C):
            if np.any(lab == c):
                cent[c] = k[lab == c].mean(0)
        prev = inertia
    assert np.array_equal(lab, lit.labels) and t == lit.iterations


def test_compact_and_permutation_invariants():
    labels = np.array([5, 2, 5, 0, 2, 2, 7])
    c, Cc = O.compact_labels(labels, 9)
    assert Cc == 4 and c.tolist() == [2, 1, 2, 0, 1, 1, 3]
    perm, off, cnt = O.group_permutation(c, Cc)
    assert sorted(perm.tolist()) == list(range(7))
    assert perm.tolist() == [3, 1, 4, 5, 0, 2, 6]          # stable by token id
    assert off.tolist() == [0, 1, 4, 6, 7] and cnt.tolist() == [1, 3, 2, 1]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(7)
    assert np.array_equal(perm[inv], np.arange(7))


# ---------------------------------------------------------------- responses and masses
def test_query_features_rms_normalised():
    rng = np.random.default_rng(9)
    q, c = rng.standard_normal((20, 4)), rng.standard_normal((6, 4))
    q[3] = 0.0
    L, F = O.query_features(q, c, 0.5)
    assert np.allclose(L, 0.5 * np.einsum("id,bd->ib", q, c))
    rms = np.sqrt((F ** 2).mean(1))
    assert np.allclose(np.delete(rms, 3), 1.0) and np.all(F[3] == 0)
    # scale invariance of F: multiplying a query by 7 leaves its features unchanged
    _, F7 = O.query_features(q * 7.0, c, 0.5)
    assert np.allclose(F7, F)


def test_group_masses_closed_forms():
    # equal logits: p_i(b) = n_k[b] / N (softmax of log sizes)
    n_k = np.array([3, 1, 4, 2])
    L = np.zeros((6, 4))
    P, u = O.group_masses(L, n_k, np.array([0, 1, 0, 1, 1, 0]), 2)
    assert np.allclose(P, np.tile(n_k / n_k.sum(), (2, 1)))
    # hand value: two groups of one key, logits (ln 3, 0) -> masses (3/4, 1/4)
    P, u = O.group_masses(np.array([[math.log(3.0), 0.0]]), np.array([1, 1]), np.array([0]), 1)
    assert np.allclose(P, [[0.75, 0.25]]) and u.tolist() == [[3 * 2 ** 30, 2 ** 30]]
    rng = np.random.default_rng(10)
    L = rng.standard_normal((50, 7)) * 3
    P, u = O.group_masses(L, rng.integers(1, 9, 7), rng.integers(0, 3, 50), 3)
    assert np.allclose(P.sum(1), 1.0)
    assert np.all(np.abs(u.sum(1) - 2 ** 32) <= 7)


# ---------------------------------------------------------------- routing
def _route_brute(u, n_q, n_k, N, M, rho):
    """Scan every candidate selection implied by the sorted rows; keep the cheapest-fitting max."""
    Cq, Ck = u.shape
    budget = O.pair_budget(N, M, rho)
    orders = [sorted(range(Ck), key=lambda b: (-u[a, b], b)) for a in range(Cq)]
    # the thresholds that matter are 0, each prefix mass, each prefix mass + 1, and the top
    pts = {0, 2 ** 32 + Ck}
    for a in range(Cq):
        c = 0
        for b in orders[a]:
            c += int(u[a, b])
            pts.update({c, c + 1})
    best = None
    for tau in sorted(pts):
        if tau > 2 ** 32 + Ck:
            continue
        js, cost = [], 0
        for a in range(Cq):
            c, j = 0, 0
            for j, b in enumerate(orders[a], 1):
                c += int(u[a, b])
                if c >= tau:
                    break
            js.append(max(j, 1))
            cost += int(n_q[a]) * sum(int(n_k[b]) for b in orders[a][:js[-1]])
        if cost <= budget:
            best = [sorted(orders[a][:js[a]]) for a in range(Cq)]
    if best is None:
        return [[orders[a][0]] for a in range(Cq)], True
    return best, False


def test_route_matches_brute_force_threshold_scan():
    rng = np.random.default_rng(11)
    for trial in range(40):
        Cq, Ck = rng.integers(1, 5), rng.integers(1, 6)
        n_q = rng.integers(1, 9, Cq)
        n_k = rng.integers(1, 9, Ck)
        N = int(max(n_q.sum(), n_k.sum()))
        P = rng.dirichlet(np.ones(Ck) * 0.5, Cq)
        u = np.rint(P * 2 ** 32).astype(np.int64)
        if trial % 5 == 0:
            u[:, -1] = u[:, 0]            # exact ties between groups
        M = int(rng.integers(0, 3))
        rho = float(rng.uniform(0.02, 1.2))
        rt = O.route(u, n_q, n_k, N, M, rho)
        want, flag = _route_brute(u, n_q, n_k, N, M, rho)
        got = [rt.cols[rt.row_ptr[a]:rt.row_ptr[a + 1]].tolist() for a in range(Cq)]
        assert got == want and rt.budget_exceeded == flag


def test_route_invariants():
    rng = np.random.default_rng(12)
    Cq, Ck, N, M = 12, 15, 600, 6
    n_q = rng.multinomial(N - Cq, np.ones(Cq) / Cq) + 1
    n_k = rng.multinomial(N - Ck, np.ones(Ck) / Ck) + 1
    u = np.rint(rng.dirichlet(np.ones(Ck), Cq) * 2 ** 32).astype(np.int64)
    prev = None
    for rho in [0.05, 0.1, 0.2, 0.4, 0.8, 1.0 + M / N]:
        rt = O.route(u, n_q, n_k, N, M, rho)
        sel = {(a, b) for a in range(Cq) for b in rt.cols[rt.row_ptr[a]:rt.row_ptr[a + 1]]}
        assert all(rt.row_ptr[a + 1] > rt.row_ptr[a] for a in range(Cq))
        pairs = O.executed_pairs(rt, n_q, n_k, N, M)
        assert rt.budget_exceeded or pairs <= math.floor(rho * N * N)
        if prev is not None:
            assert prev <= sel                      # monotone in the budget
        prev = sel
    assert len(prev) == Cq * Ck                     # rho = 1 + M/N keeps every cell
    rt = O.route(u, n_q, n_k, N, M, 1e-4)
    assert rt.budget_exceeded and np.all(np.diff(rt.row_ptr) == 1)
    assert all(rt.cols[a] == np.lexsort((np.arange(Ck), -u[a]))[0] for a in range(Cq))


# ---------------------------------------------------------------- probes
def test_allocate_probes_largest_remainder_brute_force():
    for n_q, M in [([5, 3, 2], 4), ([1, 1, 1, 1], 2), ([7, 7, 7], 5), ([10, 1, 4, 9], 24), ([3], 1)]:
        n_q = np.array(n_q)
        N = int(n_q.sum())
        got = O.allocate_probes(n_q, M, N)
        quotas = [M * n / N for n in n_q]
        base = [math.floor(x) for x in quotas]
        rema = sorted(range(len(n_q)), key=lambda a: (-(quotas[a] - base[a]), a))
        for a in rema[:M - sum(base)]:
            base[a] += 1
        assert got.tolist() == base and got.sum() == M and np.all(got <= n_q)


def test_select_probes_stratified_weights():
    rng = np.random.default_rng(13)
    N, C, M = 300, 9, 20
    lab = rng.integers(0, C, N)
    perm, off, cnt = O.group_permutation(lab, C)
    idx, w = O.select_probes(0, 2, perm, off, cnt, M, N)
    m = O.allocate_probes(cnt, M, N)
    assert len(idx) == M and len(set(idx.tolist())) == M
    assert np.isclose(w.sum(), M)
    pos = 0
    for a in range(C):
        members = set(perm[off[a]:off[a + 1]].tolist())
        chunk = idx[pos:pos + m[a]]
        assert set(chunk.tolist()) <= members and np.all(np.diff(chunk) > 0)
        if m[a]:
            assert np.allclose(w[pos:pos + m[a]] * m[a] / cnt[a], w[pos] * m[a] / cnt[a])
        pos += m[a]


def test_select_probes_group_weight_is_the_group_share_of_queries():
    # [T4] "query group stratified" probes with a weighted ridge: each group's probes
    # together stand for that group's share of the queries, so a group's total weight
    # w_a * m_a is proportional to its size n_q[a] (here groups whose size-to-probe ratio
    # n_q[a] / m_a differs, so an inverted ratio m_a / n_q[a] would fail)
    sizes = np.array([120, 7, 33, 61, 3, 250, 26])
    N, M = int(sizes.sum()), 17
    rng = np.random.default_rng(31)
    lab = rng.permutation(np.repeat(np.arange(len(sizes)), sizes))
    perm, off, cnt = O.group_permutation(lab, len(sizes))
    m = O.allocate_probes(cnt, M, N)
    covered = m > 0
    ratio = cnt[covered] / m[covered]
    assert ratio.max() > 1.2 * ratio.min()            # the ratio really varies
    idx, w = O.select_probes(0, 3, perm, off, cnt, M, N)
    assert np.isclose(w.sum(), M)
    group_of = lab[idx]
    total = np.array([w[group_of == a].sum() for a in range(len(sizes))])
    assert np.all(total[~covered] == 0)
    # total weight of a group / all weight == its queries / all queries of covered groups
    np.testing.assert_allclose(total[covered] / M, cnt[covered] / cnt[covered].sum(), rtol=1e-12)
    # and every probe of a group weighs the same
    for a in np.flatnonzero(covered):
        assert np.ptp(w[group_of == a]) == 0


# ---------------------------------------------------------------- ridge
def test_ridge_matches_lstsq_on_augmented_system():
    rng = np.random.default_rng(14)
    for M, d, lam, pb in [(40, 6, 0.3, False), (5, 8, 1e-3, False), (30, 4, 2.0, True)]:
        o_sp = rng.standard_normal((M, d))
        o_dn = o_sp + rng.standard_normal((M, d)) * 0.2
        w = rng.uniform(0.5, 2.0, M)
        th = O.ridge_fit(o_sp, o_dn, w, lam, pb)
        Z = np.hstack([o_sp, np.ones((M, 1))])
        reg = np.sqrt(lam) * np.eye(d + 1)
        if not pb:
            reg = reg[:d]
        A = np.vstack([np.sqrt(w)[:, None] * Z, reg])
        B = np.vstack([np.sqrt(w)[:, None] * (o_dn - o_sp), np.zeros((reg.shape[0], d))])
        want = np.linalg.lstsq(A, B, rcond=None)[0]
        np.testing.assert_allclose(th, want, rtol=1e-8, atol=1e-10)


def test_ridge_recovers_planted_affine_map():
    rng = np.random.default_rng(15)
    M, d = 60, 8
    o_sp = rng.standard_normal((M, d))
    theta = rng.standard_normal((d + 1, d))
    o_dn = o_sp + o_sp @ theta[:d] + theta[d]
    got = O.ridge_fit(o_sp, o_dn, rng.uniform(0.5, 2, M), 1e-12)
    np.testing.assert_allclose(got, theta, atol=1e-9)


def test_planted_affine_residual_is_removed_end_to_end():
    # [abstract]: the residual of every unprobed row is predicted by the affine map fitted
    # on the probes. Dense outputs planted as o + o A + b (A not symmetric, so a transposed
    # map fails) are recovered for every row through ridge_fit then apply_residual, and the
    # probe rows return their given dense rows exactly.
    rng = np.random.default_rng(32)
    N, d, M = 400, 12, 40
    o_sp = rng.standard_normal((N, d))
    A = rng.standard_normal((d, d))
    assert np.abs(A - A.T).max() > 1.0
    b = rng.standard_normal(d)
    o_dn = np.empty_like(o_sp)
    for i in range(N):                     # the planted map, row by row
        for j in range(d):
            o_dn[i, j] = o_sp[i, j] + sum(o_sp[i, kk] * A[kk, j] for kk in range(d)) + b[j]
    probes = np.sort(rng.choice(N, M, replace=False))
    theta = O.ridge_fit(o_sp[probes], o_dn[probes], rng.uniform(0.5, 2.0, M), 1e-12)
    out = O.apply_residual(o_sp, probes, o_dn[probes], theta)
    np.testing.assert_allclose(out, o_dn, rtol=0, atol=1e-9)
    assert np.array_equal(out[probes], o_dn[probes])
    # the map is not the identity correction: without it the error is large
    assert np.abs(o_sp - o_dn).max() > 1.0


def test_ridge_interpolates_when_underdetermined():
    rng = np.random.default_rng(16)
    M, d = 6, 10
    o_sp = rng.standard_normal((M, d))
    o_dn = rng.standard_normal((M, d))
    th = O.ridge_fit(o_sp, o_dn, np.ones(M), 1e-10)
    fitted = o_sp @ th[:d] + th[d]
    np.testing.assert_allclose(fitted, o_dn - o_sp, atol=1e-6)
    # the prediction at any point lies in the span of the probe residuals (any lambda;
    # a well-conditioned lambda keeps the check at round-off level)
    R = o_dn - o_sp
    th = O.ridge_fit(o_sp, o_dn, np.ones(M), 0.1)
    pred = rng.standard_normal((4, d)) @ th[:d] + th[d]
    coef = np.linalg.lstsq(R.T, pred.T, rcond=None)[0]
    np.testing.assert_allclose(R.T @ coef, pred.T, atol=1e-8)


def test_ridge_large_lambda_is_mean_only_correction():
    # Table 4's mean-only family: with the bias unpenalised and lambda -> inf the map
    # keeps only the weighted mean residual.
    rng = np.random.default_rng(17)
    M, d = 25, 5
    o_sp = rng.standard_normal((M, d))
    o_dn = rng.standard_normal((M, d))
    w = rng.uniform(0.2, 3.0, M)
    th = O.ridge_fit(o_sp, o_dn, w, 1e12)
    assert np.abs(th[:d]).max() < 1e-9
    np.testing.assert_allclose(th[d], (w[:, None] * (o_dn - o_sp)).sum(0) / w.sum(), atol=1e-9)


def test_ridge_singular_system_is_a_numerical_error():
    rng = np.random.default_rng(18)
    o_sp = rng.standard_normal((4, 8))
    with pytest.raises(O.NumericalError):
        O.ridge_fit(o_sp, o_sp + 1, np.ones(4), 0.0)
    assert np.all(O.ridge_fit(np.zeros((0, 8)), np.zeros((0, 8)), np.zeros(0), 1.0) == 0)


def test_cholesky_matches_numpy():
    rng = np.random.default_rng(19)
    X = rng.standard_normal((20, 9))
    A = X.T @ X + np.eye(9)
    np.testing.assert_allclose(O.cholesky(A), np.linalg.cholesky(A), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- metric and pages' numbers
def test_rel_l2_formula():
    out = np.array([[3.0, 4.0], [1.0, 1.0]])
    ref = np.array([[0.0, 0.0], [1.0, 1.0]])
    e = O.rel_l2(out, ref)
    assert np.isclose(e[0], 5.0 / 1e-8) and e[1] == 0.0
    e = O.rel_l2(np.array([[1.0, 2.0, 2.0]]), np.array([[0.0, 0.0, 0.0]]) + np.array([[1.0, 0.0, 0.0]]))
    assert np.isclose(e[0], math.sqrt(8.0) / (1.0 + 1e-8))


def test_error_stats_excludes_probes_and_uses_linear_p99():
    ref = np.ones((101, 2))
    out = ref.copy()
    out[:, 0] += np.arange(101) / 100 * math.sqrt(2)      # e_i = i / 100
    out[50, 0] += 100.0                                     # probe row: excluded
    mean, p99 = O.error_stats(out, ref, [50])
    rest = np.delete(np.arange(101) / 100, 50)
    assert np.isclose(mean, rest.mean()) and np.isclose(p99, np.percentile(rest, 99))


def test_table_c2_probe_fractions():
    for _, n, pct in _rows("table_c2_probe_fraction.txt"):
        assert round(100 * O.probe_fraction(64, int(n)), 3) == float(pct)


def test_table2_error_reduction_matches_abstract_range():
    rows = _rows("table2_error_reduction.txt")
    reds = []
    for r in rows:
        if r[0] == "RANGE":
            lo, hi = float(r[1]), float(r[2])
            continue
        red = round(100 * O.error_reduction(float(r[1]), float(r[2])), 1)
        assert red == float(r[3])
        reds.append(red)
    assert (min(reds), max(reds)) == (lo, hi)


# ---------------------------------------------------------------- whole call
def _tiny_cfg(N=96, d=8):
    return dict(scale=1 / math.sqrt(d), seed=0, n_sampled=12, n_key_groups=6, n_query_groups=5,
                n_probes=7, density=0.3, ridge_lambda=1e-3)


def test_full_density_call_is_dense_everywhere():
    rng = np.random.default_rng(20)
    N, d = 96, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    p = _tiny_cfg(N, d)
    p["density"] = 1.0 + p["n_probes"] / N
    r = O.sparsepr_head(q, k, v, p, head=0)
    dn = O.dense_attention(q, k, v, p["scale"])
    np.testing.assert_allclose(r.o_sparse, dn, rtol=1e-12, atol=1e-12)
    assert np.abs(r.theta).max() < 1e-12          # residuals are round-off only
    np.testing.assert_allclose(r.out, dn, rtol=1e-12, atol=1e-12)


def test_probe_rows_return_exact_dense_output():
    rng = np.random.default_rng(21)
    N, d = 96, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    p = _tiny_cfg(N, d)
    r = O.sparsepr_head(q, k, v, p, head=3)
    dn = O.dense_attention(q, k, v, p["scale"])
    assert len(r.plan.probes) == p["n_probes"]
    assert np.array_equal(r.out[r.plan.probes], dn[r.plan.probes])
    assert r.plan.pairs <= math.floor(p["density"] * N * N) or r.plan.route.budget_exceeded


def test_single_group_partition_is_dense():
    rng = np.random.default_rng(22)
    N, d = 64, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    p = dict(_tiny_cfg(N, d), n_key_groups=1, n_query_groups=1, density=0.1)
    r = O.sparsepr_head(q, k, v, p, head=0)
    np.testing.assert_allclose(r.o_sparse, O.dense_attention(q, k, v, p["scale"]), rtol=1e-12, atol=1e-12)


def test_row_subset_entry_matches_whole_call():
    rng = np.random.default_rng(23)
    N, d = 96, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    p = _tiny_cfg(N, d)
    r = O.sparsepr_head(q, k, v, p, head=1)
    rows = np.array([0, 5, 17, 40, 95] + list(r.plan.probes[:2]))
    sub = O.attend_fit_apply_rows(q, k, v, p, r.plan, rows)
    np.testing.assert_allclose(sub["o_sparse"], r.o_sparse[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sub["theta"], r.theta, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(sub["out"], r.out[rows], rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- warm-started planning
def _clustered(rng, N, d, C, sep=4.0):
    means = sep * rng.standard_normal((C, d)) / math.sqrt(d)
    lab = rng.integers(0, C, N)
    return means[lab] + 0.3 * rng.standard_normal((N, d))


def test_warm_key_init_is_the_group_mean_of_responses():
    # a key group's response centroid is the response of its mean key (responses are linear)
    rng = np.random.default_rng(30)
    N, d, S = 200, 8, 12
    q, k = _clustered(rng, N, d, 5), _clustered(rng, N, d, 5)
    p = dict(_tiny_cfg(N, d), n_sampled=S)
    hp = O.plan_head(q, k, p, head=0, max_iter=25, tol=1e-4)
    qs = q[hp.sampled]
    RK = O.key_responses(k, qs, p["scale"])
    np.testing.assert_allclose(O.key_responses(hp.key_centroids, qs, p["scale"]),
                               O.group_means(RK, hp.key_labels, hp.Ck), rtol=1e-10, atol=1e-12)


def test_warm_query_init_is_the_group_mean_of_features():
    # F_i = (s / RMS_i) q_i C_k^T, so a query group's feature mean is its representative times C_k^T
    rng = np.random.default_rng(31)
    N, d = 200, 8
    q, k = _clustered(rng, N, d, 5), _clustered(rng, N, d, 5)
    p = _tiny_cfg(N, d)
    hp = O.plan_head(q, k, p, head=2, max_iter=25, tol=1e-4)
    _, F = O.query_features(q, hp.key_centroids, p["scale"])
    np.testing.assert_allclose(hp.query_reps @ hp.key_centroids.T, O.group_means(F, hp.query_labels, hp.Cq),
                               rtol=1e-10, atol=1e-12)


def test_warm_start_from_a_fixed_point_keeps_the_partition():
    # cold k-means run to a fixed point (tol 0); warm-starting on the same inputs must
    # reproduce both partitions exactly, stopping after the second assignment (the warm
    # centroids equal the final ones up to rounding, hence a round-off tolerance)
    rng = np.random.default_rng(32)
    N, d = 240, 8
    q, k = _clustered(rng, N, d, 6), _clustered(rng, N, d, 6)
    p = _tiny_cfg(N, d)
    cold = O.plan_head(q, k, p, head=1, max_iter=500, tol=0.0)
    warm = O.plan_head_warm(q, k, p, head=1, prev=cold, max_iter=25, tol=1e-12)
    assert np.array_equal(warm.key_labels, cold.key_labels)
    assert np.array_equal(warm.query_labels, cold.query_labels)
    assert (warm.Ck, warm.Cq) == (cold.Ck, cold.Cq)
    assert warm.key_iters == 2 and warm.query_iters == 2
    assert np.array_equal(warm.probes, cold.probes)


def test_warm_start_obeys_its_iteration_limit_and_drops_empty_groups():
    rng = np.random.default_rng(33)
    N, d = 240, 8
    q, k = _clustered(rng, N, d, 6), _clustered(rng, N, d, 6)
    p = _tiny_cfg(N, d)
    cold = O.plan_head(q, k, p, head=0, max_iter=25, tol=1e-4)
    q2 = q + 0.8 * rng.standard_normal(q.shape)
    k2 = k + 0.8 * rng.standard_normal(k.shape)
    warm = O.plan_head_warm(q2, k2, p, head=0, prev=cold, max_iter=2, tol=1e-4)
    assert warm.key_iters <= 2 and warm.query_iters <= 2
    assert warm.Ck <= cold.Ck and warm.Cq <= cold.Cq
    for lab, C in ((warm.key_labels, warm.Ck), (warm.query_labels, warm.Cq)):
        assert set(np.unique(lab)) == set(range(C))
    # the two iterations are those of lloyd_from on the mapped centroids
    qs = q2[warm.sampled]
    RK = O.key_responses(k2, qs, p["scale"])
    ref = O.lloyd_from(RK, O.key_responses(cold.key_centroids, qs, p["scale"]), 2, 1e-4)
    assert np.array_equal(O.compact_labels(ref.labels, cold.Ck)[0], warm.key_labels)


# ---------------------------------------------------------------- comparison settings (Tables 2, 4)
def _planted_same_as(labels, planted):
    """True iff two labelings induce the same partition."""
    pairs = set(zip(labels.tolist(), planted.tolist()))
    return len(pairs) == len(set(labels.tolist())) == len(set(planted.tolist()))


def _hidden_key_clusters(rng, N, d, C):
    # queries live in the first half of the coordinates; the planted key clusters differ only
    # in the second half, so every key response s q k^T is blind to them
    h = d // 2
    q = np.zeros((N, d))
    q[:, :h] = rng.standard_normal((N, h))
    lab = np.arange(N) % C
    means = np.zeros((C, d))
    means[:, h:] = 6.0 * rng.standard_normal((C, d - h))
    k = means[lab] + 0.05 * rng.standard_normal((N, d))
    k[:, :h] = rng.standard_normal((N, h))
    return q, k, lab


def test_semantic_partition_clusters_raw_keys_and_queries():
    # [T2] semantic baseline: k-means on raw K and raw Q. Planted raw clusters invisible to
    # the key responses are recovered by the semantic partition and not by the response one.
    rng = np.random.default_rng(40)
    N, d, C = 240, 8, 3
    q, k, lab = _hidden_key_clusters(rng, N, d, C)
    qlab = rng.integers(0, C, N)
    qmeans = np.zeros((C, d))
    qmeans[:, : d // 2] = 6.0 * rng.standard_normal((C, d // 2))
    q = qmeans[qlab] + 0.05 * rng.standard_normal((N, d))
    q[:, d // 2:] = 0.0
    p = dict(_tiny_cfg(N, d), n_key_groups=C, n_query_groups=C, n_sampled=24)
    # Forgy rows vary with the head; Lloyd finds the planted clusters from a good start
    sem_k = sem_q = rsp_k = 0
    for head in range(20):
        sem = O.plan_head(q, k, dict(p, partition=O.PARTITION_SEMANTIC), head, 50, 0.0)
        rsp = O.plan_head(q, k, dict(p, partition=O.PARTITION_RESPONSE), head, 50, 0.0)
        sem_k += _planted_same_as(sem.key_labels, lab)
        sem_q += _planted_same_as(sem.query_labels, qlab)
        rsp_k += _planted_same_as(rsp.key_labels, lab)
    assert sem_k >= 2 and sem_q >= 2 and rsp_k == 0


def test_key_response_partition_mixes_the_two_sides():
    # [T2] second row: K/V groups of the response-coupled partition, query groups of the
    # semantic one (both Lloyd runs start from the same Forgy rows in every mode)
    rng = np.random.default_rng(41)
    N, d = 200, 8
    q, k = rng.standard_normal((N, d)), _clustered(rng, N, d, 5)
    p = _tiny_cfg(N, d)
    plans = {m: O.plan_head(q, k, dict(p, partition=m), 1, 25, 1e-4)
             for m in (O.PARTITION_RESPONSE, O.PARTITION_SEMANTIC, O.PARTITION_KEY_RESPONSE)}
    mix = plans[O.PARTITION_KEY_RESPONSE]
    assert np.array_equal(mix.key_labels, plans[O.PARTITION_RESPONSE].key_labels)
    assert np.array_equal(mix.query_labels, plans[O.PARTITION_SEMANTIC].query_labels)
    assert not np.array_equal(plans[O.PARTITION_RESPONSE].query_labels, mix.query_labels)
    # semantic query representatives are plain member means of q
    np.testing.assert_allclose(mix.query_reps[0], q[mix.query_labels == 0].mean(axis=0), rtol=1e-12)


def test_random_probes_are_the_smallest_hashes_over_all_tokens():
    # [T4] random probes: M tokens uniformly without replacement, by brute force over the hashes
    N, M, seed, head = 150, 9, 5, 3
    got = O.select_probes_plain(seed, head, N, M, O.PROBES_RANDOM)
    h = [int(x) for x in O.token_hash(seed, O.STREAM_PROBES, head, np.arange(N))]
    assert got.tolist() == sorted(i for _, i in sorted(zip(h, range(N)))[:M])


def test_uniform_probes_take_one_token_per_equal_bin():
    # [T4] uniform spatiotemporal probes: evenly spaced in the raster order. Bins at least two
    # tokens wide each hold exactly one probe; gaps differ by at most one token; the set is
    # mirror-symmetric about the middle of the sequence (centres c and N - c).
    for N, M in [(100, 7), (96, 12), (5, 5), (1000, 1), (37, 36), (75600, 2268)]:
        got = O.select_probes_plain(0, 0, N, M, O.PROBES_UNIFORM)
        assert len(got) == M and np.all(np.diff(got) > 0) and got[0] >= 0 and got[-1] < N
        if N >= 2 * M:
            for b, t in enumerate(got.tolist()):
                assert b * N <= t * M < (b + 1) * N
        gaps = np.diff(got)
        if M > 1:
            assert gaps.max() - gaps.min() <= 1 and gaps.min() >= N // M - 1
        assert set((got + got[::-1]).tolist()) <= {N - 1, N}
    assert O.select_probes_plain(0, 0, 96, 12, O.PROBES_UNIFORM).tolist() == list(range(4, 96, 8))


def test_plain_selectors_weigh_every_probe_one():
    rng = np.random.default_rng(42)
    N, d = 96, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    for sel in (O.PROBES_RANDOM, O.PROBES_UNIFORM):
        p = dict(_tiny_cfg(N, d), probe_selector=sel)
        r = O.sparsepr_head(q, k, v, p, head=0)
        assert np.array_equal(r.plan.probes, O.select_probes_plain(p["seed"], 0, N, p["n_probes"], sel))
        assert np.all(r.plan.weights == 1.0)
        assert np.array_equal(r.out[r.plan.probes], O.dense_attention(q, k, v, p["scale"])[r.plan.probes])


def test_mean_only_correction_is_the_infinite_lambda_ridge():
    # [T4] mean-only: unprobed rows shift by the weighted mean probe residual, which is the
    # lam -> inf limit of the ridge with an unpenalised bias
    rng = np.random.default_rng(43)
    N, d = 96, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    p = _tiny_cfg(N, d)
    mo = O.sparsepr_head(q, k, v, dict(p, correction=O.CORRECTION_MEAN_ONLY), head=2)
    big = O.sparsepr_head(q, k, v, dict(p, ridge_lambda=1e12), head=2)
    np.testing.assert_allclose(mo.out, big.out, rtol=0, atol=1e-9)
    pr, w = mo.plan.probes, mo.plan.weights
    resid = O.dense_attention(q, k, v, p["scale"])[pr] - mo.o_sparse[pr]
    assert np.abs((w[:, None] * (resid - mo.theta[-1])).sum(axis=0)).max() < 1e-12
    assert np.all(mo.theta[:-1] == 0.0)


def test_disabled_correction_keeps_the_sparse_output():
    rng = np.random.default_rng(44)
    N, d = 96, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    p = dict(_tiny_cfg(N, d), correction=O.CORRECTION_NONE)
    r = O.sparsepr_head(q, k, v, p, head=1)
    un = np.setdiff1d(np.arange(N), r.plan.probes)
    assert np.array_equal(r.out[un], r.o_sparse[un])
    assert np.array_equal(r.out[r.plan.probes], O.dense_attention(q, k, v, p["scale"])[r.plan.probes])


# ---------------------------------------------------------------- key response rank ([C.1] r_K)
def test_reduced_key_features_are_the_rank_r_metric():
    # distances between reduced key features equal (k_i - k_j) G_r (k_i - k_j)^T, with G_r the
    # rank-r truncation of G = s^2 Q_S^T Q_S from its own eigendecomposition (eigh, not svd)
    rng = np.random.default_rng(50)
    N, d, S, r = 40, 8, 24, 3
    k, qs = rng.standard_normal((N, d)), rng.standard_normal((S, d)) * np.linspace(3, 0.5, d)
    s = 0.7
    Y = O.key_features(k, qs, s, r)
    assert Y.shape == (N, r)
    lam, U = np.linalg.eigh(s * s * qs.T @ qs)
    Gr = (U[:, -r:] * lam[-r:]) @ U[:, -r:].T
    D = k[:, None, :] - k[None, :, :]
    want = np.einsum("ija,ab,ijb->ij", D, Gr, D)
    got = ((Y[:, None, :] - Y[None, :, :]) ** 2).sum(-1)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-9)


def test_key_rank_at_or_above_d_is_the_full_response():
    rng = np.random.default_rng(51)
    N, d = 120, 8
    q, k = _clustered(rng, N, d, 4), _clustered(rng, N, d, 4)
    p = _tiny_cfg(N, d)
    full = O.plan_head(q, k, p, 0, 25, 1e-4)
    for r in (d, d + 5):
        same = O.plan_head(q, k, dict(p, key_rank=r), 0, 25, 1e-4)
        assert np.array_equal(same.key_labels, full.key_labels)
        assert np.array_equal(same.query_labels, full.query_labels)


def test_low_key_rank_drops_weak_response_directions():
    # key clusters separated only along the direction the sampled queries barely probe: the
    # full response separates them, a rank that keeps only the strong directions cannot
    rng = np.random.default_rng(52)
    N, d, C = 240, 8, 3
    q = rng.standard_normal((N, d))
    q[:, -1] *= 0.05                      # the last coordinate is barely probed
    lab = np.arange(N) % C
    k = rng.standard_normal((N, d))
    k[:, -1] = 80.0 * np.array([-1.0, 0.0, 1.0])[lab]
    p = dict(_tiny_cfg(N, d), n_key_groups=C, n_sampled=64)
    full_ok = low_ok = 0
    for head in range(12):
        full_ok += _planted_same_as(O.plan_head(q, k, p, head, 50, 0.0).key_labels, lab)
        low_ok += _planted_same_as(O.plan_head(q, k, dict(p, key_rank=d - 1), head, 50, 0.0).key_labels, lab)
    assert full_ok >= 2 and low_ok == 0


# ---------------------------------------------------------------- output truncation ([D.2](a))
def _probe_fit_case(rng, M, d, noise=0.3):
    o_sp = rng.standard_normal((M, d))
    o_dn = o_sp + noise * rng.standard_normal((M, d))
    w = rng.uniform(0.5, 2.0, M)
    return o_sp, o_dn, w


def test_residual_projector_is_the_leading_right_singular_subspace():
    # a different routine: the top right singular vectors of diag(sqrt w) R (SVD, not eigh)
    rng = np.random.default_rng(41)
    o_sp, o_dn, w = _probe_fit_case(rng, 50, 12)
    R = o_dn - o_sp
    for r in (1, 3, 7):
        P = O.residual_projector(o_sp, o_dn, w, r)
        V = np.linalg.svd(np.sqrt(w)[:, None] * R)[2][:r].T
        np.testing.assert_allclose(P, V @ V.T, atol=1e-10)
        np.testing.assert_allclose(P @ P, P, atol=1e-10)
        assert abs(np.trace(P) - r) < 1e-10


def test_truncation_at_or_above_the_residual_rank_is_the_plain_ridge():
    # fewer probes than dimensions: the residuals span M <= d directions, so any rank >= M
    # keeps the whole observed span and the prediction is unchanged
    rng = np.random.default_rng(42)
    d = 10
    for M in (6, 30):
        o_sp, o_dn, w = _probe_fit_case(rng, M, d)
        p = dict(ridge_lambda=0.1, penalize_bias=False)
        plain = O.fit_correction(o_sp, o_dn, w, p)
        for r in (min(M, d), d):
            cut = O.fit_correction(o_sp, o_dn, w, dict(p, output_rank=r))
            np.testing.assert_allclose(cut, plain, atol=1e-9)
        assert np.abs(O.fit_correction(o_sp, o_dn, w, dict(p, output_rank=2)) - plain).max() > 1e-3


def test_truncation_to_rank_zero_is_no_repair():
    rng = np.random.default_rng(43)
    N, d, M = 80, 6, 20
    o_sp_all = rng.standard_normal((N, d))
    probes = np.sort(rng.choice(N, M, replace=False))
    o_dn = o_sp_all[probes] + 0.5 * rng.standard_normal((M, d))
    w = np.ones(M)
    th = O.ridge_fit(o_sp_all[probes], o_dn, w, 0.1) @ O.residual_projector(o_sp_all[probes], o_dn, w, 0)
    assert np.all(th == 0)
    out = O.apply_residual(o_sp_all, probes, o_dn, th)
    none = O.apply_residual(o_sp_all, probes, o_dn, O.fit_correction(o_sp_all[probes], o_dn, w,
                                                                      dict(correction=O.CORRECTION_NONE)))
    np.testing.assert_array_equal(out, none)


def test_truncated_prediction_stays_in_the_planted_residual_subspace():
    # residuals confined to a planted 3-dimensional subspace U plus weak noise: rank 3 finds U
    # and every predicted residual lies in it
    rng = np.random.default_rng(44)
    M, d, r = 60, 16, 3
    U = np.linalg.qr(rng.standard_normal((d, r)))[0]
    o_sp = rng.standard_normal((M, d))
    o_dn = o_sp + (rng.standard_normal((M, r)) * [3.0, 2.0, 1.5]) @ U.T + 1e-4 * rng.standard_normal((M, d))
    w = rng.uniform(0.5, 2.0, M)
    P = O.residual_projector(o_sp, o_dn, w, r)
    np.testing.assert_allclose(P, U @ U.T, atol=1e-3)
    th = O.fit_correction(o_sp, o_dn, w, dict(ridge_lambda=1e-3, output_rank=r))
    pred = rng.standard_normal((5, d)) @ th[:d] + th[d]
    np.testing.assert_allclose(pred - pred @ P, 0.0, atol=1e-9)            # in the fitted subspace
    np.testing.assert_allclose(pred - pred @ U @ U.T, 0.0, atol=1e-3 * np.abs(pred).max())  # ~ planted
