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
