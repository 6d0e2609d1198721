"""Oracle diagnostics of the pages' structural observations (test
infrastructure, float64 NumPy, CPU only; nothing in the HIP path uses it).

* Pooled support [paperlayer.ai s3.1, O1]: the support of a query at mass
  alpha is the smallest set of keys whose attention probabilities, taken
  largest first, sum to at least alpha; pooling a few queries that share a
  route takes the union of their supports.  Per-query support fraction
  |S_t| / N against pooled fraction |U S_t| / N shows how much a shared route
  must grow because the queries' supports overlap only partly.
* Affine-explainable residual [paperlayer.ai s3.1, O3]: the residual
  R = O_dense - O_sparse of all rows splits into its best least-squares
  affine approximation from the sparse output, [1, X] beta, and the
  orthogonal rest; the explained fraction is 1 - ||rest||^2 / ||R||^2.  This
  needs every dense row, so it is a diagnostic, not part of sparse execution.

* Near ties and eigen-gaps (rounding-sensitivity reports, not parts of the
  method): k-means points whose best and second-best squared distances, in
  the expanded form the assignment evaluates, differ by less than 1e-9 of the
  best; route cells whose score equals the deciding cell's score to 1e-12
  relative (a row's best two cells, the cell at the budget cut, the k-th and
  (k+1)-th cells of a row); the gap of the eigenvalues of M_K at r_k relative
  to the largest.  A label or route that differs between two float64
  evaluations is explained only if it falls on such a tie.

Readings (the pages give the definitions, not these details): a pool is
`pool` members of one query group at evenly spaced ranks of the group-major
order (groups smaller than the pool are skipped); the affine fit is
unweighted over all rows of a head.
"""
import numpy as np

from . import sparsepr_oracle as o


def support_size(p: np.ndarray, alpha: float) -> np.ndarray:
    """Indices of the smallest key set whose probabilities (largest first,
    ties to the lower key index) sum to at least alpha."""
    order = np.lexsort((np.arange(len(p)), -p))
    mass = np.cumsum(p[order])
    k = int(np.searchsorted(mass, alpha * mass[-1] * (1.0 - 1e-15))) + 1
    return order[:min(k, len(p))]


def pooled_support(Q, K, part: "o.HeadPartition", scale: float, alpha: float = 0.9, pool: int = 8):
    """Per-query and pooled support fractions over the query groups of a
    partition.  Returns (per_query [n_pools * pool], pooled [n_pools])."""
    N = K.shape[0]
    per, pooled = [], []
    for a in range(len(part.q_off) - 1):
        b, e = int(part.q_off[a]), int(part.q_off[a + 1])
        if e - b < pool:
            continue
        members = part.q_perm[b + (2 * np.arange(pool) + 1) * (e - b) // (2 * pool)]
        union = set()
        for t in members:
            s = scale * (K @ Q[t])
            p = np.exp(s - s.max())
            p /= p.sum()
            sup = support_size(p, alpha)
            per.append(len(sup) / N)
            union.update(sup.tolist())
        pooled.append(len(union) / N)
    return np.asarray(per), np.asarray(pooled)


def affine_residual_split(X: np.ndarray, R: np.ndarray):
    """Best least-squares affine approximation of R from X (rows are
    samples): returns (explained fraction, orthogonal energy ||R - [1,X]b||^2,
    residual energy ||R||^2)."""
    A = np.hstack([np.ones((X.shape[0], 1)), X])
    beta, *_ = np.linalg.lstsq(A, R, rcond=None)
    rest = R - A @ beta
    tot = float(np.sum(R * R))
    orth = float(np.sum(rest * rest))
    return (1.0 - orth / tot if tot > 0 else 0.0), orth, tot


def head_diagnostics(Q, K, V, cfg, alpha: float = 0.9, pool: int = 8):
    """Both diagnostics for one head under cfg's partition: routing and the
    renormalised hard drop as in the method, every row."""
    s = cfg.softmax_scale
    part = o.partition_head(Q, K, cfg)
    route = o.route_head(part, cfg, Q.shape[0])
    O_sp, _ = o.sparse_attention(Q, K, V, part, route, s)
    O_dn, _ = o.dense_attention(Q, K, V, s)
    per, pooled = pooled_support(Q, K, part, s, alpha, pool)
    frac, orth, tot = affine_residual_split(O_sp, O_dn - O_sp)
    return {"per_query_support_median": float(np.median(per)), "pooled_support_median": float(np.median(pooled)),
            "affine_explained": frac, "orthogonal_energy": orth / float(np.sum(O_dn * O_dn)),
            "residual_energy": tot / float(np.sum(O_dn * O_dn)),
            "density": o.executed_pair_density(route.routed_pairs, cfg.M, Q.shape[0])}


NEAR_TIE_KMEANS = 1e-9
NEAR_TIE_ROUTE = 1e-12


def assignment_near_ties(X: np.ndarray, C: np.ndarray, rel: float = NEAR_TIE_KMEANS) -> np.ndarray:
    """Points of X whose two smallest squared distances to the centres C
    (||x||^2 - 2 x.c + ||c||^2, float64) differ by less than rel (best + 1e-300);
    returns their indices."""
    if C.shape[0] < 2:
        return np.zeros(0, dtype=np.int64)
    d2 = np.einsum("ij,ij->i", X, X)[:, None] - 2.0 * (X @ C.T) + np.einsum("ij,ij->i", C, C)[None, :]
    s = np.sort(d2, axis=1)
    return np.flatnonzero(s[:, 1] - s[:, 0] < rel * (np.abs(s[:, 0]) + 1e-300))


def kmeans_near_ties(X: np.ndarray, G: int, T: int, rel: float = NEAR_TIE_KMEANS) -> np.ndarray:
    """Near ties of the last of T Lloyd assignments (o.kmeans rules): the
    centres it uses are those after T - 1 rounds (the strided start rows for
    T = 1)."""
    if T > 1:
        _, C = o.kmeans(X, G, T - 1)
    else:
        n = X.shape[0]
        C = X[(2 * np.arange(G, dtype=np.int64) + 1) * n // (2 * G)]
    return assignment_near_ties(X, C, rel)


def eigen_gap(M_K: np.ndarray, r_k: int) -> float:
    """(lambda_{r_k} - lambda_{r_k + 1}) / lambda_1 of M_K (descending, clamped at
    0); 1 when r_k covers every direction, 0 for a zero matrix."""
    lam = np.sort(np.maximum(np.linalg.eigvalsh(M_K), 0.0))[::-1]
    if lam[0] <= 0.0:
        return 0.0
    if r_k >= len(lam):
        return 1.0
    return float((lam[r_k - 1] - lam[r_k]) / lam[0])


def route_near_ties(P: np.ndarray, q_sizes, kv_sizes, budget: int = None, k: int = 0,
                    rel: float = NEAR_TIE_ROUTE) -> dict:
    """Cells whose choice hinges on a score tie to rel: per nonempty query
    group its best two cells ("mandatory"); in top-k mode the k-th and
    (k+1)-th cells of a row ("topk"); in budget mode the cells, other than the
    kept best ones, whose score equals to rel that of the first cell that does
    not fit ("budget_cut"; o.select_cells_budget's scan).  Returns the counts."""
    q_sizes, kv_sizes = np.asarray(q_sizes), np.asarray(kv_sizes)
    valid = np.flatnonzero(kv_sizes > 0)
    out = {"mandatory": 0, "topk": 0, "budget_cut": 0}
    best = {}
    for a in np.flatnonzero(q_sizes > 0):
        row = P[a, valid]
        order = valid[np.argsort(-row, kind="stable")]
        best[a] = order[0]
        if len(order) > 1 and P[a, order[0]] - P[a, order[1]] <= rel * P[a, order[0]]:
            out["mandatory"] += 1
        if k > 0 and len(order) > k and P[a, order[k - 1]] - P[a, order[k]] <= rel * P[a, order[k - 1]]:
            out["topk"] += 1
    if budget is not None and k == 0:
        used = sum(int(q_sizes[a]) * int(kv_sizes[b]) for a, b in best.items())
        cells = sorted((-P[a, b], a, b) for a in best for b in valid if b != best[a])
        for neg, a, b in cells:
            c = int(q_sizes[a]) * int(kv_sizes[b])
            if used + c > budget:
                pc = -neg
                out["budget_cut"] = int(sum(1 for n2, a2, b2 in cells if abs(-n2 - pc) <= rel * pc)) - 1
                break
            used += c
    return out


def partition_near_ties(Q: np.ndarray, K: np.ndarray, cfg) -> dict:
    """Near ties of the final K/V and query labels of o.partition_head and the
    eigen-gap of M_K at r_k, for one head (float64 inputs)."""
    M_K = o.key_response_metric(Q, cfg.M_s)
    U_r, w, _ = o.eigen_weighted_basis(M_K, cfg.r_k, cfg.eig_weight_power)
    Z = o.key_response_coords(K, U_r, w)
    kv_label, _ = o.kmeans(Z, cfg.G_k, cfg.iters_kv)
    kv_mu, kv_sizes = o.group_means(K, kv_label, cfg.G_k)
    Y = o.query_response_coords(Q, kv_mu, kv_sizes, cfg.softmax_scale)
    return {"kv_near_ties": kmeans_near_ties(Z, cfg.G_k, cfg.iters_kv),
            "q_near_ties": kmeans_near_ties(Y, cfg.G_q, cfg.iters_q),
            "eigen_gap": eigen_gap(M_K, cfg.r_k)}
