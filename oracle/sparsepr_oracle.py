"""CPU oracle of the SparsePR attention call -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run this module. The product path (the HIP library and
its Python binding) never touches it, and this module imports nothing from that path.

It is a plain, slow, float64 NumPy statement of what the call computes, step by step,
in the order the pages give it. Sources ("the pages"):
  [abstract]  the paper's abstract (listing page and arXiv abstract page of
              "Partition the Support, Reconstruct the Residual", 2608.18484);
  [method]    the project website, Method section: stages 01 sample responses,
              02 partition support, 03 execute sparse routes, 04 reconstruct residual,
              and its RCP / PFRR panels;
  [results]   the project website, Results section (density convention);
  [C.1]       paper Table C.1, method configuration (iteration limits, tolerance);
  [D.1]       paper Table D.1, query RMS normalisation ablation and the error metric;
  [T2], [T4]  paper Tables 2 and 4 (error aggregation, stratified probes, weighted
              ridge, mean-only family).

Where the pages leave a step open the reading taken is named in the docstring
("Reading: ..."). Every function here is pinned by a CPU test against a closed form,
a library routine on a special case, brute force on tiny inputs or the pages' printed
values; none is "parity unpinned".

Notation, per head: N tokens, head dim d, scale s, S sampled queries, C_k / C_q
requested groups (realised C_k', C_q' after dropping empty clusters), M probes,
density rho, ridge strength lambda.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------------
# Counter-based hash: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
# number generators", OOPSLA 2014; public-domain reference by S. Vigna). h(x) is the
# first output of a SplitMix64 generator whose state is x.
# ----------------------------------------------------------------------------------
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

STREAM_SAMPLED = 1
STREAM_KEY_INIT = 2
STREAM_QUERY_INIT = 3
STREAM_PROBES = 4


def splitmix64(x):
    z = np.asarray(x, dtype=np.uint64) + _GOLDEN
    z = (z ^ (z >> np.uint64(30))) * _MIX1
    z = (z ^ (z >> np.uint64(27))) * _MIX2
    return z ^ (z >> np.uint64(31))


def token_hash(seed, stream, head, idx):
    """h(stream, head, i) = sm(sm(sm(seed ^ stream) ^ head) ^ i), vectorised over i."""
    with np.errstate(over="ignore"):
        a = splitmix64(np.array([np.uint64(seed) ^ np.uint64(stream)], dtype=np.uint64))
        b = splitmix64(a ^ np.uint64(head))
        return splitmix64(b ^ np.asarray(idx, dtype=np.uint64))


def select_smallest(seed, stream, head, candidates, m):
    """The m candidates with the smallest (hash, index), listed in ascending index order.

    Reading: the pages fix only budgets (S sampled queries per head [C.1], M probes);
    a seeded uniform choice without replacement is taken, made reproducible on any
    device by ranking a counter-based hash.
    """
    cand = np.asarray(candidates, dtype=np.int64)
    if m <= 0:
        return np.zeros(0, dtype=np.int64)
    h = token_hash(seed, stream, head, cand)
    order = np.lexsort((cand, h))
    return np.sort(cand[order[:m]])


# ----------------------------------------------------------------------------------
# Dense and block-sparse softmax attention
# ----------------------------------------------------------------------------------
def dense_attention(q, k, v, scale, chunk=2048):
    """O_i = sum_j softmax_j(s q_i.k_j) v_j over all keys (the dense reference)."""
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], chunk):
        logits = scale * (q[r0:r0 + chunk] @ k.T)
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r0 + chunk] = p @ v
    return out


def block_sparse_attention(q, k, v, scale, q_perm, q_off, k_perm, k_off, row_ptr, cols):
    """Softmax attention of each query group over the union of its selected key groups.

    [abstract], [method] stage 03: attention is computed only between selected
    (query group, key group) cells, and softmax is taken over the retained keys only.
    """
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    for a in range(len(q_off) - 1):
        rows = q_perm[q_off[a]:q_off[a + 1]]
        if len(rows) == 0:
            continue
        keys = np.concatenate([k_perm[k_off[b]:k_off[b + 1]] for b in cols[row_ptr[a]:row_ptr[a + 1]]])
        out[rows] = dense_attention(q[rows], k[keys], v[keys], scale)
    return out


def block_sparse_rows(q, k, v, scale, rows, q_labels, k_perm, k_off, row_ptr, cols):
    """block_sparse_attention restricted to the query rows ``rows`` (same definition)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    groups = q_labels[rows]
    for a in np.unique(groups):
        sel = np.flatnonzero(groups == a)
        keys = np.concatenate([k_perm[k_off[b]:k_off[b + 1]] for b in cols[row_ptr[a]:row_ptr[a + 1]]])
        out[sel] = dense_attention(q[rows[sel]], k[keys], v[keys], scale)
    return out


# ----------------------------------------------------------------------------------
# Lloyd k-means ([abstract]: keys grouped by their responses, queries grouped by
# responses to key-group centroids; [C.1]: 25 initial iterations, tolerance 1e-4)
# ----------------------------------------------------------------------------------
def sq_dists(x, c):
    """Squared Euclidean distances ||x_i - c_b||^2, expanded as |x|^2 - 2 x.c + |c|^2."""
    return (x * x).sum(1)[:, None] - 2.0 * (x @ c.T) + (c * c).sum(1)[None, :]


@dataclass
class LloydResult:
    labels: np.ndarray
    iterations: int
    inertia: list = field(default_factory=list)


def lloyd(x, init_rows, max_iter, tol):
    """Lloyd's algorithm with Forgy initialisation from the rows ``init_rows`` of x.

    Reading (the pages give only the iteration limit and tolerance [C.1]): one
    iteration is an assignment (nearest centroid, ties to the lower cluster id)
    followed by an update (member mean; an empty cluster keeps its centroid). The
    loop stops after the assignment of iteration t when t == max_iter or when the
    inertia decrease from iteration t-1 is at most tol times the previous inertia.
    The labels returned are those of the last assignment.
    """
    return lloyd_from(x, x[np.asarray(init_rows)], max_iter, tol)


def lloyd_from(x, init_centroids, max_iter, tol):
    """The iterations of ``lloyd`` started from explicit centroids (rows of init_centroids)."""
    cent = np.array(init_centroids, dtype=np.float64, copy=True)
    C = cent.shape[0]
    prev = None
    hist = []
    labels = None
    t = 0
    for t in range(1, max_iter + 1):
        dist = sq_dists(x, cent)
        labels = np.argmin(dist, axis=1)
        inertia = float(dist[np.arange(x.shape[0]), labels].sum())
        hist.append(inertia)
        if prev is not None and prev - inertia <= tol * prev:
            break
        if t == max_iter:
            break
        sums = np.zeros_like(cent)
        np.add.at(sums, labels, x)
        cnt = np.bincount(labels, minlength=C)
        nz = cnt > 0
        cent[nz] = sums[nz] / cnt[nz, None]
        prev = inertia
    return LloydResult(labels=labels.astype(np.int64), iterations=t, inertia=hist)


def compact_labels(labels, C):
    """Drop empty clusters and renumber the rest in ascending order of their old id.

    Reading: the groups of [C.1] are "requested", so the realised count may be lower.
    """
    cnt = np.bincount(labels, minlength=C)
    new_id = np.cumsum(cnt > 0) - 1
    return new_id[labels].astype(np.int64), int((cnt > 0).sum())


def group_permutation(labels, C):
    """Stable counting sort by label: perm[pos] = token, offsets[g] = first position."""
    perm = np.argsort(labels, kind="stable").astype(np.int64)
    counts = np.bincount(labels, minlength=C).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return perm, offsets, counts


def group_means(x, labels, C):
    sums = np.zeros((C, x.shape[1]), dtype=np.float64)
    np.add.at(sums, labels, x)
    cnt = np.bincount(labels, minlength=C)
    return sums / np.maximum(cnt, 1)[:, None]


# ----------------------------------------------------------------------------------
# Response-Coupled Partitioning ([abstract]; [method] stages 01-02 and RCP panel)
# ----------------------------------------------------------------------------------
def key_responses(k, q_sampled, scale):
    """R_K[j, t] = s q_t . k_j: how key j responds to sampled query t.

    Reading: the response is the scaled logit, not a probability.
    """
    return scale * (k @ q_sampled.T)


def response_basis(q_sampled, rank):
    """Top-`rank` principal directions of the sampled queries' response space.

    [C.1] gives a key response rank r_K = 48 and nothing more. Reading: a key's response
    vector s q_S k^T (one entry per sampled query) is represented by its coordinates on
    the `rank` leading left singular vectors of Q_S (the directions in which the sampled
    queries respond most), so the key k-means runs on a rank-`rank` image of R_K. Returns
    the S x rank orthonormal basis, or None when rank is 0 or not below the rank of Q_S
    (no reduction).
    """
    if rank <= 0 or rank >= min(q_sampled.shape):
        return None
    U, _, _ = np.linalg.svd(q_sampled, full_matrices=False)
    return U[:, :rank]


def key_features(k, q_sampled, scale, rank=0):
    """The rows the key k-means clusters: R_K, or R_K on the response basis when reduced."""
    RK = key_responses(k, q_sampled, scale)
    A = response_basis(q_sampled, rank)
    return RK if A is None else RK @ A


def query_features(q, key_centroids, scale):
    """Logits L = s Q C_k^T and their per-query RMS-normalised rows F.

    [abstract]: key-group centroids give query-response coordinates. [D.1]: per-query
    RMS normalisation (no centring) is the reference choice. A row with zero RMS maps
    to zero.
    """
    L = scale * (q @ key_centroids.T)
    rms = np.sqrt((L * L).mean(axis=1))
    F = np.zeros_like(L)
    nz = rms > 0
    F[nz] = L[nz] / rms[nz, None]
    return L, F


def group_masses(L, n_k, q_labels, Cq):
    """Estimated attention mass P[a, b] of query group a on key group b, and u = rint(P 2^32).

    Reading (the pages only say that cells are selected, [method] stage 03): a query's
    mass on key group b is the softmax over groups of its centroid logit plus the log
    of the group size (each of the n_k[b] keys stands in for the centroid); P[a, b] is
    the mean over the members of a. Rounding to integers (half to even) makes routing
    an exact integer function of u.
    """
    z = L + np.log(n_k.astype(np.float64))[None, :]
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    P = group_means(p, q_labels, Cq)
    u = np.rint(P * 2.0 ** 32).astype(np.int64)
    return P, u


# ----------------------------------------------------------------------------------
# Group-level routing under the executed-pair budget ([abstract]; [results]: density
# counts routed cells and exact probe rows)
# ----------------------------------------------------------------------------------
@dataclass
class Route:
    row_ptr: np.ndarray
    cols: np.ndarray
    tau: int
    budget: int
    cost: int
    budget_exceeded: bool


def pair_budget(N, M, rho):
    """floor(rho N^2) - M N: cell pairs left after the M exact probe rows."""
    return int(math.floor(rho * float(N * N))) - M * N


def route(u, n_q, n_k, N, M, rho):
    """Cells chosen by one global cumulative-mass threshold tau.

    Reading: each query group ranks key groups by (-u, b); j_a(tau) is the shortest
    prefix (at least one group) whose integer mass reaches tau, or all groups if none
    does; tau* is the largest integer in [0, 2^32 + C_k'] whose total cost
    sum_a n_q[a] * (keys in the prefix) fits the budget. If even one group per row
    does not fit, the top group of every row is kept and the overrun is flagged.
    """
    Cq, Ck = u.shape
    budget = pair_budget(N, M, rho)
    orders, cums, costs = [], [], []
    for a in range(Cq):
        order = np.lexsort((np.arange(Ck), -u[a]))
        orders.append(order)
        cums.append(np.cumsum(u[a, order]))
        costs.append(int(n_q[a]) * np.cumsum(n_k[order]))

    def take(tau):
        return [min(max(int(np.searchsorted(c, tau, side="left")) + 1, 1), Ck) for c in cums]

    def cost(tau):
        return sum(int(costs[a][j - 1]) for a, j in enumerate(take(tau)))

    hi = 2 ** 32 + Ck
    exceeded = False
    if cost(0) > budget:
        tau, exceeded = 0, True
    elif cost(hi) <= budget:
        tau = hi
    else:
        lo = 0
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if cost(mid) <= budget:
                lo = mid
            else:
                hi = mid
        tau = lo
    js = take(tau)
    cols = [np.sort(orders[a][:js[a]]) for a in range(Cq)]
    row_ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int64)
    return Route(row_ptr=row_ptr, cols=np.concatenate(cols).astype(np.int64), tau=int(tau),
                 budget=budget, cost=cost(tau), budget_exceeded=exceeded)


def executed_pairs(rt, n_q, n_k, N, M):
    pairs = M * N
    for a in range(len(rt.row_ptr) - 1):
        pairs += int(n_q[a]) * int(n_k[rt.cols[rt.row_ptr[a]:rt.row_ptr[a + 1]]].sum())
    return pairs


# ----------------------------------------------------------------------------------
# Probe rows ([T4]: query-group stratified probes, weighted ridge)
# ----------------------------------------------------------------------------------
def allocate_probes(n_q, M, N):
    """m_a = floor(M n_q[a] / N) plus one for the largest remainders (ties: lower a).

    With M <= N every m_a <= n_q[a], so no cap is ever needed.
    """
    n_q = np.asarray(n_q, dtype=np.int64)
    base = (M * n_q) // N
    rem = (M * n_q) % N
    left = M - int(base.sum())
    order = np.lexsort((np.arange(len(n_q)), -rem))
    base[order[:left]] += 1
    return base


def select_probes(seed, head, q_perm, q_off, n_q, M, N):
    """Stratified probe rows (group-major, ascending token id) and their weights.

    Reading: w_p = n_q[a] / m_a (each probe stands for its group's share of queries),
    rescaled so the weights sum to M.
    """
    m = allocate_probes(n_q, M, N)
    idx, wt = [], []
    covered = int(n_q[m > 0].sum())
    for a in range(len(n_q)):
        if m[a] == 0:
            continue
        members = np.sort(q_perm[q_off[a]:q_off[a + 1]])
        pick = select_smallest(seed, STREAM_PROBES, head, members, int(m[a]))
        idx.append(pick)
        wt.append(np.full(len(pick), (n_q[a] / m[a]) * (M / covered)))
    if not idx:
        return np.zeros(0, dtype=np.int64), np.zeros(0)
    return np.concatenate(idx).astype(np.int64), np.concatenate(wt)


PROBES_STRATIFIED = 0  # query-group stratified (the method, [T4])
PROBES_RANDOM = 1      # [T4] "Random probes"
PROBES_UNIFORM = 2     # [T4] "Uniform spatiotemporal probes"


def select_probes_plain(seed, head, N, M, selector):
    """The comparison probe sets of [T4], ascending token id, all weights 1 (reading).

    Random: the M tokens with the smallest probe hash (uniform without replacement).
    Uniform spatiotemporal: tokens floor((p + 1/2) N / M), p = 0..M-1, evenly spaced in
    the raster order of the latent grid (reading: the pages name the set only).
    """
    if M == 0:
        return np.zeros(0, dtype=np.int64)
    if selector == PROBES_RANDOM:
        return select_smallest(seed, STREAM_PROBES, head, np.arange(N), M).astype(np.int64)
    return ((2 * np.arange(M, dtype=np.int64) + 1) * N // (2 * M)).astype(np.int64)


# ----------------------------------------------------------------------------------
# Probe-Fitted Residual Reconstruction ([abstract]; [method] PFRR panel)
# ----------------------------------------------------------------------------------
class NumericalError(RuntimeError):
    pass


PIVOT_RTOL = 1e-12


def cholesky(A):
    """Lower-triangular L with L L^T = A; a pivot <= 1e-12 max(diag A) is a failure."""
    n = A.shape[0]
    L = np.zeros_like(A)
    floor = PIVOT_RTOL * float(np.max(np.diag(A))) if n else 0.0
    for j in range(n):
        piv = A[j, j] - L[j, :j] @ L[j, :j]
        if not piv > floor:
            raise NumericalError(f"non-positive pivot {piv} at column {j}")
        L[j, j] = math.sqrt(piv)
        L[j + 1:, j] = (A[j + 1:, j] - L[j + 1:, :j] @ L[j, :j]) / L[j, j]
    return L


def solve_lower(L, B):
    X = np.zeros_like(B)
    for i in range(L.shape[0]):
        X[i] = (B[i] - L[i, :i] @ X[:i]) / L[i, i]
    return X


def solve_upper(U, B):
    n = U.shape[0]
    X = np.zeros_like(B)
    for i in range(n - 1, -1, -1):
        X[i] = (B[i] - U[i, i + 1:] @ X[i + 1:]) / U[i, i]
    return X


def ridge_fit(o_sp_probe, o_dn_probe, weights, lam, penalize_bias=False):
    """Theta [(d+1), d] minimising sum_p w_p |r_p - [o_p, 1] Theta|^2 + lam |A|_F^2.

    r_p = O_dense_p - O_sparse_p is the probe residual (the abstract fits the
    difference between dense and sparse outputs). The normal equations
    (Z^T W Z + Lambda) Theta = Z^T W R, Z = [O_sp_P, 1], Lambda = diag(lam 1_d, 0)
    (bias unpenalised unless asked), are solved by Cholesky. The prediction
    [o, 1] Theta = [o, 1] (Z^T W Z + Lambda)^-1 Z^T W R is a combination of the rows of
    R, so it stays in the span of the observed probe residuals. No probes: Theta = 0.
    """
    M, d = o_sp_probe.shape
    if M == 0:
        return np.zeros((d + 1, d))
    Z = np.concatenate([o_sp_probe, np.ones((M, 1))], axis=1)
    R = o_dn_probe - o_sp_probe
    w = np.asarray(weights, dtype=np.float64)[:, None]
    A = Z.T @ (w * Z)
    A[np.arange(d), np.arange(d)] += lam
    if penalize_bias:
        A[d, d] += lam
    B = Z.T @ (w * R)
    L = cholesky(A)
    return solve_upper(L.T, solve_lower(L, B))


def residual_projector(o_sp_probe, o_dn_probe, weights, rank):
    """Orthogonal projector (d x d) onto the `rank` leading directions of the probe residuals.

    [method] PFRR panel: the affine correction acts in a low-rank probe-residual subspace;
    [D.2](a) holds "no output truncation" fixed, so truncation is a setting. Reading: the
    subspace is spanned by the `rank` eigenvectors of largest eigenvalue (ties: lower index)
    of the weighted residual second moment R^T W R (R = O_dense - O_sparse on the probes,
    W = diag(w), uncentred, the ridge's own weighting); the fitted map's predicted residual
    is projected onto it. rank >= rank(R) keeps the whole observed span (the untruncated
    fit); rank 0 removes the correction.
    """
    R = np.asarray(o_dn_probe, dtype=np.float64) - np.asarray(o_sp_probe, dtype=np.float64)
    d = R.shape[1]
    w = np.asarray(weights, dtype=np.float64)[:, None]
    C = R.T @ (w * R)
    evals, evecs = np.linalg.eigh(C)
    order = np.lexsort((np.arange(d), -evals))[:max(0, min(rank, d))]
    U = evecs[:, order]
    return U @ U.T


CORRECTION_RIDGE = 0      # full weighted ridge (the method)
CORRECTION_MEAN_ONLY = 1  # [T4] "Mean-only": add the weighted mean probe residual
CORRECTION_NONE = 2       # repair disabled ([T2] partition rows): sparse output kept


def fit_correction(o_sp_probe, o_dn_probe, weights, p):
    """Theta of the correction family p["correction"] (ridge by default).

    With p["output_rank"] = r > 0 the ridge's prediction is truncated to the r leading
    directions of the probe residuals (residual_projector); 0 or absent: no truncation.
    Mean-only is the lam -> infinity limit of the ridge with the bias unpenalised:
    Theta = [0; sum_p w_p r_p / sum_p w_p]. With repair disabled Theta = 0, so unprobed
    rows keep their sparse output (probe rows still return the exact output).
    """
    mode = p.get("correction", CORRECTION_RIDGE)
    M, d = o_sp_probe.shape
    if mode == CORRECTION_RIDGE:
        theta = ridge_fit(o_sp_probe, o_dn_probe, weights, p["ridge_lambda"], p.get("penalize_bias", False))
        r = p.get("output_rank", 0)
        if r and M > 0:
            # output truncation: the predicted residual [o, 1] Theta projected on the probe
            # residuals' r leading directions
            theta = theta @ residual_projector(o_sp_probe, o_dn_probe, weights, r)
        return theta
    theta = np.zeros((d + 1, d))
    if mode == CORRECTION_MEAN_ONLY and M > 0:
        w = np.asarray(weights, dtype=np.float64)
        theta[d] = (w[:, None] * (o_dn_probe - o_sp_probe)).sum(axis=0) / w.sum()
    return theta


def apply_residual(o_sp, probes, o_dn_probe, theta):
    """out_i = o_i + [o_i, 1] Theta for unprobed rows; probe rows keep their exact output."""
    out = o_sp + o_sp @ theta[:-1] + theta[-1][None, :]
    out[probes] = o_dn_probe
    return out


# ----------------------------------------------------------------------------------
# Error metric ([D.1] formula; [T2] mean / p99 over unprobed rows)
# ----------------------------------------------------------------------------------
def rel_l2(out, ref):
    """|O_i - O_i^dense|_2 / (|O_i^dense|_2 + 1e-8) per row."""
    return np.linalg.norm(out - ref, axis=1) / (np.linalg.norm(ref, axis=1) + 1e-8)


def error_stats(out, ref, probes):
    mask = np.ones(out.shape[0], dtype=bool)
    mask[np.asarray(probes, dtype=np.int64)] = False
    e = rel_l2(out[mask], ref[mask])
    return float(e.mean()), float(np.percentile(e, 99))


def error_reduction(err_before, err_after):
    return 1.0 - err_after / err_before


def probe_fraction(M, N):
    return M / N


# ----------------------------------------------------------------------------------
# The whole call, per head
# ----------------------------------------------------------------------------------
@dataclass
class HeadPlan:
    sampled: np.ndarray = None
    key_labels: np.ndarray = None
    key_iters: int = 0
    Ck: int = 0
    k_perm: np.ndarray = None
    k_off: np.ndarray = None
    n_k: np.ndarray = None
    key_centroids: np.ndarray = None
    query_reps: np.ndarray = None
    query_labels: np.ndarray = None
    query_iters: int = 0
    Cq: int = 0
    q_perm: np.ndarray = None
    q_off: np.ndarray = None
    n_q: np.ndarray = None
    P: np.ndarray = None
    u: np.ndarray = None
    route: Route = None
    probes: np.ndarray = None
    weights: np.ndarray = None
    pairs: int = 0


PARTITION_RESPONSE = 0   # response-coupled: key responses, then query responses (the method)
PARTITION_SEMANTIC = 1   # k-means on the raw keys and on the raw queries ([T2] "Semantic partition")
PARTITION_KEY_RESPONSE = 2  # key-response K/V groups, semantic query groups ([T2] second row)


def plan_head(q, k, p, head, max_iter, tol):
    """Response-Coupled Partitioning, masses, routing and probes for one head.

    p["partition"] selects the partition of [T2]: the method's response-coupled one
    (default), the semantic baseline (Lloyd on raw K and raw Q), or key-response K/V
    groups with semantic query groups. Everything after the two partitions is the same.
    """
    N = q.shape[0]
    s = p["scale"]
    mode = p.get("partition", PARTITION_RESPONSE)
    hp = HeadPlan()
    hp.sampled = select_smallest(p["seed"], STREAM_SAMPLED, head, np.arange(N), p["n_sampled"])
    RK = k if mode == PARTITION_SEMANTIC else key_features(k, q[hp.sampled], s, p.get("key_rank", 0))
    kinit = select_smallest(p["seed"], STREAM_KEY_INIT, head, np.arange(N), p["n_key_groups"])
    res = lloyd(RK, kinit, max_iter, tol)
    hp.key_iters = res.iterations
    hp.key_labels, hp.Ck = compact_labels(res.labels, p["n_key_groups"])
    if mode == PARTITION_RESPONSE:
        _, F = query_features(q, group_means(k, hp.key_labels, hp.Ck), s)
    else:
        F = q
    qinit = select_smallest(p["seed"], STREAM_QUERY_INIT, head, np.arange(N), p["n_query_groups"])
    res = lloyd(F, qinit, max_iter, tol)
    hp.query_iters = res.iterations
    hp.query_labels, hp.Cq = compact_labels(res.labels, p["n_query_groups"])
    return finish_plan(q, k, p, head, hp)


def query_representatives(q, L, scale, q_labels, Cq):
    """Query-group centroids as d-dimensional means of x_i = (s / RMS_i) q_i.

    F_i = x_i C_k^T (query_features), so the mean of F over a group is its
    representative times C_k^T; a warm start maps it through the new key centroids.
    """
    rms = np.sqrt((L * L).mean(axis=1))
    a = np.where(rms > 0, scale / np.where(rms > 0, rms, 1.0), 0.0)
    return group_means(a[:, None] * q, q_labels, Cq)


def plan_head_warm(q, k, p, head, prev, max_iter=2, tol=1e-4):
    """Planning started from the centroids of a previous plan (prev, a HeadPlan).

    [C.1] gives 25 iterations for the first k-means and 2 for subsequent ones.
    Reading: "subsequent" calls start from the previous call's final centroids, kept
    as d-dimensional means (key groups: mean of the member keys; query groups: the
    query_representatives), mapped into this call's response spaces: key centroids
    s m_b Q_S^T for the current sampled queries, query centroids z_a C_k^T for the
    current key centroids. The groups the previous call realised are the requested
    ones; groups left empty are dropped again.
    """
    N = q.shape[0]
    s = p["scale"]
    hp = HeadPlan()
    hp.sampled = select_smallest(p["seed"], STREAM_SAMPLED, head, np.arange(N), p["n_sampled"])
    mode = p.get("partition", PARTITION_RESPONSE)
    qs = q[hp.sampled]
    if mode == PARTITION_SEMANTIC:
        res = lloyd_from(k, prev.key_centroids, max_iter, tol)
    else:
        r = p.get("key_rank", 0)
        res = lloyd_from(key_features(k, qs, s, r), key_features(prev.key_centroids, qs, s, r), max_iter, tol)
    hp.key_iters = res.iterations
    hp.key_labels, hp.Ck = compact_labels(res.labels, prev.Ck)
    kc = group_means(k, hp.key_labels, hp.Ck)
    if mode == PARTITION_RESPONSE:
        _, F = query_features(q, kc, s)
        res = lloyd_from(F, prev.query_reps @ kc.T, max_iter, tol)
    else:
        res = lloyd_from(q, prev.query_reps, max_iter, tol)
    hp.query_iters = res.iterations
    hp.query_labels, hp.Cq = compact_labels(res.labels, prev.Cq)
    return finish_plan(q, k, p, head, hp)


def finish_plan(q, k, p, head, hp, u=None, probes=None):
    """Everything downstream of the two label vectors (also the labels-given entry).

    Labels in [0, C) are compacted first (empty groups dropped); an injected mass
    matrix u is indexed by the compacted ids; injected probe rows get unit weights.
    """
    N = q.shape[0]
    M = p["n_probes"]
    hp.key_labels, hp.Ck = compact_labels(np.asarray(hp.key_labels, dtype=np.int64), p["n_key_groups"])
    hp.query_labels, hp.Cq = compact_labels(np.asarray(hp.query_labels, dtype=np.int64), p["n_query_groups"])
    hp.k_perm, hp.k_off, hp.n_k = group_permutation(hp.key_labels, hp.Ck)
    hp.q_perm, hp.q_off, hp.n_q = group_permutation(hp.query_labels, hp.Cq)
    hp.key_centroids = group_means(k, hp.key_labels, hp.Ck)
    L, _ = query_features(q, hp.key_centroids, p["scale"])
    if p.get("partition", PARTITION_RESPONSE) == PARTITION_RESPONSE:
        hp.query_reps = query_representatives(q, L, p["scale"], hp.query_labels, hp.Cq)
    else:
        hp.query_reps = group_means(q, hp.query_labels, hp.Cq)
    if u is None:
        hp.P, hp.u = group_masses(L, hp.n_k, hp.query_labels, hp.Cq)
    else:
        hp.u = np.asarray(u, dtype=np.int64)
    hp.route = route(hp.u, hp.n_q, hp.n_k, N, M, p["density"])
    sel = p.get("probe_selector", PROBES_STRATIFIED)
    if probes is None and sel == PROBES_STRATIFIED:
        hp.probes, hp.weights = select_probes(p["seed"], head, hp.q_perm, hp.q_off, hp.n_q, M, N)
    elif probes is None:
        hp.probes = select_probes_plain(p["seed"], head, N, M, sel)
        hp.weights = np.ones(len(hp.probes))
    else:
        hp.probes = np.asarray(probes, dtype=np.int64)
        hp.weights = np.ones(len(hp.probes))
    hp.pairs = executed_pairs(hp.route, hp.n_q, hp.n_k, N, M)
    return hp


@dataclass
class HeadResult:
    plan: HeadPlan
    o_sparse: np.ndarray
    o_probe_dense: np.ndarray
    theta: np.ndarray
    out: np.ndarray


def attend_fit_apply(q, k, v, p, hp):
    s = p["scale"]
    o_sp = block_sparse_attention(q, k, v, s, hp.q_perm, hp.q_off, hp.k_perm, hp.k_off,
                                  hp.route.row_ptr, hp.route.cols)
    o_dn = dense_attention(q[hp.probes], k, v, s)
    theta = fit_correction(o_sp[hp.probes], o_dn, hp.weights, p)
    out = apply_residual(o_sp, hp.probes, o_dn, theta)
    return HeadResult(plan=hp, o_sparse=o_sp, o_probe_dense=o_dn, theta=theta, out=out)


def attend_fit_apply_rows(q, k, v, p, hp, rows):
    """The call's output on the query rows ``rows`` only (probe rows are always computed)."""
    s = p["scale"]
    rt = hp.route
    o_sp_pr = block_sparse_rows(q, k, v, s, hp.probes, hp.query_labels, hp.k_perm, hp.k_off, rt.row_ptr, rt.cols)
    o_dn = dense_attention(q[hp.probes], k, v, s)
    theta = fit_correction(o_sp_pr, o_dn, hp.weights, p)
    o_sp = block_sparse_rows(q, k, v, s, rows, hp.query_labels, hp.k_perm, hp.k_off, rt.row_ptr, rt.cols)
    out = o_sp + o_sp @ theta[:-1] + theta[-1][None, :]
    slot = {int(t): j for j, t in enumerate(hp.probes)}
    for r, t in enumerate(np.asarray(rows)):
        if int(t) in slot:
            out[r] = o_dn[slot[int(t)]]
    return dict(o_sparse=o_sp, o_probe_sparse=o_sp_pr, o_probe_dense=o_dn, theta=theta, out=out)


def call_params(cfg):
    """Oracle parameters from a workload description (scale 1/sqrt(d) unless given)."""
    d = cfg["head_dim"]
    return dict(scale=cfg.get("scale", 1.0 / math.sqrt(d)), seed=cfg["seed"],
                n_sampled=cfg["n_sampled"], n_key_groups=cfg["n_key_groups"],
                n_query_groups=cfg["n_query_groups"], n_probes=cfg["n_probes"],
                density=cfg["density"], ridge_lambda=cfg["ridge_lambda"],
                penalize_bias=cfg.get("penalize_bias", False),
                partition=cfg.get("partition", PARTITION_RESPONSE),
                correction=cfg.get("correction", CORRECTION_RIDGE),
                probe_selector=cfg.get("probe_selector", PROBES_STRATIFIED),
                key_rank=cfg.get("key_rank", 0), output_rank=cfg.get("output_rank", 0))


def sparsepr_head(q, k, v, p, head, max_iter=25, tol=1e-4):
    """One head of the full call: plan, block-sparse attention, probes, fit, apply."""
    hp = plan_head(q, k, p, head, max_iter, tol)
    return attend_fit_apply(q, k, v, p, hp)
