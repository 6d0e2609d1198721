"""SparsePR attention call -- plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path (no kernels, helpers, tables or pre/post-processing); both sides
only consume the same seeded inputs.

Source: "Partition the Support, Reconstruct the Residual: Training-Free Sparse
Attention for Video Generation and World Models" (Taghavi, Langari, Pandey,
arXiv:2608.18484).  Citations name the page and its section:
  [abstract]  the English abstract (paperdance.org card / paperlayer.ai)
  [PL s3]     paperlayer.ai summary, section 3 (formulation, observations)
  [PL s4]     paperlayer.ai summary, section 4 (method)
  [PL A.x]    paperlayer.ai summary, appendix A.1-A.3 (probe reconstruction)
  [PL B.x]    paperlayer.ai summary, appendix B.1-B.2 (partitioning)
  [PL C.x]    paperlayer.ai summary, appendix C.1-C.3 (implementation, timing)
  [gist-nl 2] gist.science Dutch technical summary, section 2 (methodology)

The method is an approximation computed by a procedure, so each function
takes the procedure's steps in the pages' order, in float64, with NumPy
primitives (matmul, eigh, svd, cholesky, argsort) as single steps and no
blocking or fusion beyond looping over query groups.  Where the pages leave a
step open, the reading taken is stated in the function's docstring (the
design notes list all of them).

Parity status: every public function is pinned by a CPU test
(tests/test_oracle_pins.py) against closed forms, invariants, brute force or
hand-worked fixtures; the *quality* of the correction (whether it lowers the
error against dense attention) is reported only and is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# numerical-rank cut for the probe-residual subspace: singular values at or
# below RANK_TOL * sigma_1 are treated as zero
RANK_TOL = 1e-6


# --------------------------------------------------------------------------
# Stage 1: response-coupled partition  [gist-nl 2A], [PL s4], [PL B.1], [PL B.2]
# --------------------------------------------------------------------------

def sampled_query_indices(N: int, M_s: int) -> np.ndarray:
    """Deterministic sampled queries [PL B.1].  The pages say only that the
    sampled queries are deterministic; reading: centred stride,
    idx_j = floor((2j+1) N / (2 M_s))."""
    j = np.arange(M_s, dtype=np.int64)
    return (2 * j + 1) * N // (2 * M_s)


def key_response_metric(Q: np.ndarray, M_s: int) -> np.ndarray:
    """M_K = Q_s^T Q_s / M_s over the sampled queries [gist-nl 2A]."""
    Qs = Q[sampled_query_indices(Q.shape[0], M_s)]
    return Qs.T @ Qs / M_s


def eigen_weighted_basis(M_K: np.ndarray, r_k: int, power: float = 0.5):
    """Leading eigendirections of M_K weighted by normalised eigenvalues
    [PL B.1].  Eigenvalues sorted descending (stable), clamped at 0,
    normalised by their sum; weight = (lambda_i / sum lambda)^power.
    Reading: power 1/2, so coordinate distances equal sampled-query
    response-profile distances up to one constant.  Each eigenvector's
    largest-magnitude entry is made positive (signs do not affect distances).
    Returns (U_r [d, r_k], w [r_k], lam [d] sorted)."""
    lam, U = np.linalg.eigh(M_K)
    order = np.argsort(-lam, kind="stable")
    lam = np.maximum(lam[order], 0.0)
    U = U[:, order]
    for i in range(U.shape[1]):
        j = int(np.argmax(np.abs(U[:, i])))
        if U[j, i] < 0:
            U[:, i] = -U[:, i]
    tot = lam.sum()
    w = (lam / tot) ** power if tot > 0 else np.zeros_like(lam)
    return U[:, :r_k], w[:r_k], lam


def key_response_coords(K: np.ndarray, U_r: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Key-response coordinates Z = K U_r diag(w) [PL B.1]."""
    return (K @ U_r) * w[None, :]


def kmeans(X: np.ndarray, G: int, T: int, init_labels: np.ndarray = None):
    """Lloyd's k-means with the fixed rules both sides use [PL C.1 names GPU
    k-means; the rules are readings]: centres start at rows
    floor((2g+1) n / (2G)); T rounds of (assign to the nearest centre, ties to
    the lowest index; replace each centre by the mean of its members, an empty
    centre keeps its value).  Squared distance in expanded form
    ||x||^2 - 2 x.c + ||c||^2.  Returns (labels of the last assignment,
    centres after the last update).

    Warm start [PL C.1 "warm-started GPU k-means" across diffusion steps]:
    with init_labels (the previous call's labels; values clamped into
    [0, G)), each group that has members starts at the mean of its members'
    current coordinates instead (an empty one at its centred-stride row);
    the T rounds are unchanged.  Labels carry over between calls where
    centres would not: the coordinates themselves are rebuilt every call."""
    n = X.shape[0]
    C = X[(2 * np.arange(G, dtype=np.int64) + 1) * n // (2 * G)].copy()
    if init_labels is not None:
        lab0 = np.clip(np.asarray(init_labels, dtype=np.int64), 0, G - 1)
        for g in range(G):
            members = X[lab0 == g]
            if members.shape[0] > 0:
                C[g] = members.mean(axis=0)
    xx = np.einsum("ij,ij->i", X, X)
    labels = np.zeros(n, dtype=np.int64)
    for _ in range(T):
        d2 = xx[:, None] - 2.0 * (X @ C.T) + np.einsum("ij,ij->i", C, C)[None, :]
        labels = np.argmin(d2, axis=1)
        for g in range(G):
            members = X[labels == g]
            if members.shape[0] > 0:
                C[g] = members.mean(axis=0)
    return labels, C


def group_means(X: np.ndarray, labels: np.ndarray, G: int):
    """Per-group mean of rows of X (zeros for empty groups) and group sizes."""
    sizes = np.bincount(labels, minlength=G)
    means = np.zeros((G, X.shape[1]))
    for g in range(G):
        if sizes[g] > 0:
            means[g] = X[labels == g].mean(axis=0)
    return means, sizes


def query_response_coords(Q: np.ndarray, kv_means: np.ndarray, kv_sizes: np.ndarray, scale: float):
    """Query-response coordinates [PL B.2], [gist-nl 2A]: pre-softmax logits
    of each query against the equally weighted, centred, nonempty K/V-group
    centroids, y_t = s q_t [mu_g - mean_g mu_g], then RMS-normalised per query
    [PL C.1] (a zero vector stays zero).  Centroids are key-space means of the
    raw keys; values do not enter [PL B].  -> Yhat [n, G']"""
    mu = kv_means[kv_sizes > 0]
    C = (mu - mu.mean(axis=0)).T
    Y = scale * (Q @ C)
    rms = np.sqrt(np.mean(Y * Y, axis=1))
    out = np.zeros_like(Y)
    nz = rms > 0
    out[nz] = Y[nz] / rms[nz, None]
    return out


def stable_group_permutation(labels: np.ndarray, G: int):
    """Group-major layout [PL s4 Sparse Execution]: perm[slot] = original index,
    stable (ascending original index inside a group); offsets = exclusive
    prefix sum of group sizes."""
    perm = np.argsort(labels, kind="stable").astype(np.int64)
    off = np.zeros(G + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.bincount(labels, minlength=G))
    return perm, off


@dataclass
class HeadPartition:
    kv_label: np.ndarray
    q_label: np.ndarray
    kv_perm: np.ndarray
    q_perm: np.ndarray
    kv_off: np.ndarray
    q_off: np.ndarray
    kv_centroid: np.ndarray      # [G_k, d] raw-key means (0 for empty)
    q_centroid: np.ndarray       # [G_q, d] raw-query means (0 for empty)
    q_dist: np.ndarray           # [N] squared distance to own query-coordinate centre
    key_coords: np.ndarray = field(repr=False, default=None)
    query_coords: np.ndarray = field(repr=False, default=None)
    eigvals: np.ndarray = field(repr=False, default=None)


def partition_head(Q, K, cfg, prev=None) -> HeadPartition:
    """Response-coupled partition of one head, one asymmetric pass (K/V
    first, then queries; no alternation) [PL s4, PL B.2].  With
    cfg.partition == "semantic", the semantic baseline instead.  prev =
    (kv_label, q_label) of the previous call warm-starts both k-means."""
    kv0, q0 = prev if prev is not None else (None, None)
    if getattr(cfg, "partition", "response") == "semantic":
        return semantic_partition_head(Q, K, cfg, prev)
    s = cfg.softmax_scale
    M_K = key_response_metric(Q, cfg.M_s)
    U_r, w, lam = eigen_weighted_basis(M_K, cfg.r_k, cfg.eig_weight_power)
    Z = key_response_coords(K, U_r, w)
    kv_label, _ = kmeans(Z, cfg.G_k, cfg.iters_kv, kv0)       # V inherits the key's label
    kv_mu, kv_n = group_means(K, kv_label, cfg.G_k)
    Yhat = query_response_coords(Q, kv_mu, kv_n, s)
    q_label, q_centres = kmeans(Yhat, cfg.G_q, cfg.iters_q, q0)
    diff = Yhat - q_centres[q_label]
    q_dist = np.einsum("ij,ij->i", diff, diff)
    q_mu, _ = group_means(Q, q_label, cfg.G_q)
    kv_perm, kv_off = stable_group_permutation(kv_label, cfg.G_k)
    q_perm, q_off = stable_group_permutation(q_label, cfg.G_q)
    return HeadPartition(kv_label, q_label, kv_perm, q_perm, kv_off, q_off, kv_mu, q_mu, q_dist,
                         Z, Yhat, lam)


def semantic_partition_head(Q, K, cfg, prev=None) -> HeadPartition:
    """Semantic-partition baseline, the comparator of the pages' ablations
    [PL s3.1 O3, appendix D]: K/V groups by k-means on the raw keys and query
    groups by k-means on the raw queries, with the same k-means rules, group
    counts and iterations as the method; q_dist is the squared distance of a
    query to its own centre in raw query space.  Routing, attention, probes
    and the fit downstream are unchanged (matched group counts, routing and
    density, as the pages compare)."""
    kv0, q0 = prev if prev is not None else (None, None)
    kv_label, _ = kmeans(K, cfg.G_k, cfg.iters_kv, kv0)
    kv_mu, _ = group_means(K, kv_label, cfg.G_k)
    q_label, q_centres = kmeans(Q, cfg.G_q, cfg.iters_q, q0)
    diff = Q - q_centres[q_label]
    q_dist = np.einsum("ij,ij->i", diff, diff)
    q_mu, _ = group_means(Q, q_label, cfg.G_q)
    kv_perm, kv_off = stable_group_permutation(kv_label, cfg.G_k)
    q_perm, q_off = stable_group_permutation(q_label, cfg.G_q)
    return HeadPartition(kv_label, q_label, kv_perm, q_perm, kv_off, q_off, kv_mu, q_mu, q_dist, K, Q, None)


# --------------------------------------------------------------------------
# Stage 2: routing under a pair budget  [PL s4 Sparse Execution], [abstract]
# --------------------------------------------------------------------------

def pair_budget(density: float, N: int, M: int) -> int:
    """Routed-pair budget: the executed-pair target includes probe rows
    [PL s5 Implementation details, PL C.3], so budget = floor(rho * N^2) - M N."""
    return int(math.floor(density * float(N * N))) - M * N


def cell_scores(q_mu, q_sizes, kv_mu, kv_sizes, scale):
    """Cell score P_ab = softmax over nonempty b of (s qbar_a . mu_b + ln n_b):
    the group-centroid estimate of the attention mass query group a puts on
    K/V group b (reading; the pages say only that centroids induce the
    coordinates used for shared routing [abstract]).  Rows of empty query
    groups and columns of empty K/V groups are absent (0)."""
    Gq, Gk = len(q_sizes), len(kv_sizes)
    P = np.zeros((Gq, Gk))
    A = np.flatnonzero(q_sizes > 0)
    B = np.flatnonzero(kv_sizes > 0)
    L = scale * (q_mu[A] @ kv_mu[B].T) + np.log(kv_sizes[B].astype(np.float64))[None, :]
    L = L - L.max(axis=1, keepdims=True)
    E = np.exp(L)
    P[np.ix_(A, B)] = E / E.sum(axis=1, keepdims=True)
    return P


def select_cells_budget(P, q_sizes, kv_sizes, budget):
    """Select cells under a query-key pair budget using true cell costs
    n_a n_b [PL s4 Sparse Execution].  Reading: every nonempty query group
    keeps its best cell; the remaining cells are visited by (P desc, a asc,
    b asc) and added while the total stays within budget, stopping at the
    first cell that does not fit (so each query group's route is a prefix of
    its own ranking).  Returns a boolean [G_q, G_k] mask."""
    Gq, Gk = P.shape
    sel = np.zeros((Gq, Gk), dtype=bool)
    used = 0
    for a in range(Gq):
        if q_sizes[a] == 0:
            continue
        valid = np.flatnonzero(kv_sizes > 0)
        b = valid[np.argmax(P[a, valid])]
        sel[a, b] = True
        used += int(q_sizes[a]) * int(kv_sizes[b])
    cells = [(-P[a, b], a, b) for a in range(Gq) for b in range(Gk)
             if q_sizes[a] > 0 and kv_sizes[b] > 0 and not sel[a, b]]
    cells.sort()
    for _, a, b in cells:
        c = int(q_sizes[a]) * int(kv_sizes[b])
        if used + c > budget:
            break
        sel[a, b] = True
        used += c
    return sel


def select_cells_topk(P, q_sizes, kv_sizes, k):
    """Fixed top-k routing: the k largest P_ab per nonempty query group,
    ties to the smaller b."""
    Gq, Gk = P.shape
    sel = np.zeros((Gq, Gk), dtype=bool)
    valid = np.flatnonzero(kv_sizes > 0)
    for a in range(Gq):
        if q_sizes[a] == 0:
            continue
        order = valid[np.argsort(-P[a, valid], kind="stable")]
        sel[a, order[:k]] = True
    return sel


@dataclass
class HeadRoute:
    row_ptr: np.ndarray     # [G_q+1]
    col_idx: np.ndarray     # [nnz] ascending per row
    routed_pairs: int
    P: np.ndarray = field(repr=False, default=None)
    mask: np.ndarray = field(repr=False, default=None)


def route_head(part: HeadPartition, cfg, N: int) -> HeadRoute:
    q_sizes = np.diff(part.q_off)
    kv_sizes = np.diff(part.kv_off)
    P = cell_scores(part.q_centroid, q_sizes, part.kv_centroid, kv_sizes, cfg.softmax_scale)
    if cfg.top_k > 0:
        sel = select_cells_topk(P, q_sizes, kv_sizes, cfg.top_k)
    else:
        sel = select_cells_budget(P, q_sizes, kv_sizes, pair_budget(cfg.density, N, cfg.M))
    row_ptr = np.zeros(len(q_sizes) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(sel.sum(axis=1))
    col_idx = np.concatenate([np.flatnonzero(sel[a]) for a in range(len(q_sizes))]).astype(np.int64) \
        if sel.any() else np.zeros(0, dtype=np.int64)
    pairs = int((q_sizes[:, None] * kv_sizes[None, :])[sel].sum())
    return HeadRoute(row_ptr, col_idx, pairs, P, sel)


def executed_pair_density(routed_pairs: int, M: int, N: int) -> float:
    """Executed-pair density counts routed cells plus the exact probe rows
    [PL C.3 Density accounting]: (routed + M N) / N^2."""
    return (routed_pairs + M * N) / float(N * N)


# --------------------------------------------------------------------------
# Stage 3: sparse attention with renormalised hard drop  [PL s4], [PL A.1]
# --------------------------------------------------------------------------

def dense_attention(Q, K, V, scale, rows=None):
    """Full softmax attention (non-causal, full sequence [PL s2])."""
    q = Q if rows is None else Q[rows]
    S = scale * (q @ K.T)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return (E @ V) / l, (m + np.log(l))[:, 0]


def allowed_keys(part: HeadPartition, route: HeadRoute, a: int) -> np.ndarray:
    """Original indices of the keys in the K/V groups routed to query group a."""
    cols = route.col_idx[route.row_ptr[a]:route.row_ptr[a + 1]]
    if len(cols) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([part.kv_perm[part.kv_off[b]:part.kv_off[b + 1]] for b in cols])


def sparse_attention(Q, K, V, part: HeadPartition, route: HeadRoute, scale, rows=None):
    """Renormalised hard drop [PL s4 Sparse Execution]: a query in group a
    takes the softmax over only the keys of its routed K/V groups, so the
    retained weights are renormalised and skipped interactions contribute
    nothing.  Loops over query groups.  Returns (O [n, d], lse [n]) for the
    requested original row indices (all rows by default)."""
    N = Q.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    O = np.zeros((len(rows), V.shape[1]))
    lse = np.full(len(rows), -np.inf)
    lab = part.q_label[rows]
    for a in np.unique(lab):
        pos = np.flatnonzero(lab == a)
        keys = allowed_keys(part, route, a)
        if len(keys) == 0:
            continue
        O[pos], lse[pos] = dense_attention(Q[rows[pos]], K[keys], V[keys], scale)
    return O, lse


def masked_attention_bruteforce(Q, K, V, mask, scale):
    """Explicit-mask attention in pure Python floats (tiny inputs only):
    row t takes the softmax over keys u with mask[t][u] true."""
    n, d = len(Q), len(Q[0])
    out = []
    for t in range(n):
        logits = []
        for u in range(len(K)):
            if mask[t][u]:
                logits.append((u, scale * sum(Q[t][i] * K[u][i] for i in range(d))))
        m = max(v for _, v in logits)
        wts = [(u, math.exp(v - m)) for u, v in logits]
        z = sum(w for _, w in wts)
        out.append([sum(w * V[u][j] for u, w in wts) / z for j in range(len(V[0]))])
    return out


# --------------------------------------------------------------------------
# Stage 4: query-group-stratified exact probes  [PL A.2], [PL s4]
# --------------------------------------------------------------------------

def probe_allocation(q_sizes: np.ndarray, M: int) -> np.ndarray:
    """Probes per query group, stratified across query groups [PL s4].
    Reading: if M is below the number of nonempty groups, the M largest
    groups (ties to the smaller index) get one each; otherwise every nonempty
    group gets one and the other M - |A| are shared in proportion to group
    size by largest remainder (integer quotients, remainders ranked
    descending, ties to the smaller index), never more than a group's size;
    what a cap leaves over is shared again over the uncapped groups."""
    G = len(q_sizes)
    m = np.zeros(G, dtype=np.int64)
    A = [a for a in range(G) if q_sizes[a] > 0]
    if M == 0 or not A:
        return m
    if M < len(A):
        for a in sorted(A, key=lambda a: (-int(q_sizes[a]), a))[:M]:
            m[a] = 1
        return m
    for a in A:
        m[a] = 1
    left = M - len(A)
    active = list(A)
    while left > 0:
        S = sum(int(q_sizes[a]) for a in active)
        share = {a: (left * int(q_sizes[a])) // S for a in active}
        rem = {a: (left * int(q_sizes[a])) % S for a in active}
        extra = dict(share)
        spare = left - sum(share.values())
        for a in sorted(active, key=lambda a: (-rem[a], a))[:spare]:
            extra[a] += 1
        left = 0
        still = []
        for a in active:
            room = int(q_sizes[a]) - int(m[a])
            take = min(extra[a], room)
            m[a] += take
            left += extra[a] - take
            if m[a] < q_sizes[a]:
                still.append(a)
        active = still
    return m


DIST_RANK_BITS = 30


def distance_rank_key(x: float) -> float:
    """The distance a probe ranking compares: the float64 distance rounded to
    DIST_RANK_BITS significant bits (round half up on the magnitude).
    Distances that are equal in exact arithmetic -- the two members of a
    two-point group, for one -- come out a few ulps apart depending on the
    order of summation; compared at 2^-30 they are equal and the original
    index decides (reading: the pages fix no tie rule)."""
    b = np.array([x], dtype=np.float64).view(np.uint64)[0]
    drop = 64 - 12 - (DIST_RANK_BITS - 1)            # low mantissa bits cleared
    b = (int(b) + (1 << (drop - 1))) & ~((1 << drop) - 1)
    return float(np.array([b], dtype=np.uint64).view(np.float64)[0])


def probe_select(part: HeadPartition, M: int):
    """Probe rows and coverage weights [PL A.2], chosen from query partitions
    and query-response coordinates without looking at any residual.  Inside a
    group the members are ranked by (distance to their query-coordinate
    centre compared at 2^-30, original index; see distance_rank_key) and
    ranks floor((2j+1) n_a / (2 m_a)) are taken
    (reading: quantiles of the distance).  Weight of a probe in group a:
    (n_a / m_a) / sum over probed groups of n_a (inverse inclusion rate,
    summing to 1; reading of "coverage weighting" [PL s4]).
    Returns (probe_idx ascending, weights aligned)."""
    q_sizes = np.diff(part.q_off)
    m = probe_allocation(q_sizes, M)
    total = int(q_sizes[m > 0].sum())
    idx, wts = [], []
    for a in np.flatnonzero(m > 0):
        members = np.flatnonzero(part.q_label == a)
        order = sorted(members.tolist(), key=lambda t: (distance_rank_key(part.q_dist[t]), t))
        n_a, m_a = int(q_sizes[a]), int(m[a])
        for j in range(m_a):
            idx.append(order[(2 * j + 1) * n_a // (2 * m_a)])
            wts.append((n_a / m_a) / total)
    o = np.argsort(idx, kind="stable")
    return np.asarray(idx, dtype=np.int64)[o], np.asarray(wts)[o]


# --------------------------------------------------------------------------
# Stage 5: probe-fitted affine residual correction  [PL A.1], [PL A.3], [PL s4]
# --------------------------------------------------------------------------

@dataclass
class HeadFit:
    r_bar: np.ndarray      # [d]
    x_bar: np.ndarray      # [d]
    B_r: np.ndarray        # [d, r_eff]
    V_r: np.ndarray        # [d, r_eff]
    rank_eff: int
    sing: np.ndarray = field(repr=False, default=None)


def fit_residual(X: np.ndarray, R: np.ndarray, w: np.ndarray, rank: int, lam: float) -> HeadFit:
    """Weighted ridge affine fit R ~ b + x B from probe rows [gist-nl 2B],
    [PL A.3]; regressor = the sparse output only (query coordinates are not
    features [PL A]).  Weighted centring gives the intercept (unpenalised);
    the feature-dependent part is restricted to the span V_r of the leading
    right singular vectors of the weighted, centred probe-residual matrix
    [PL s4], r_eff = min(rank, #{sigma_i > RANK_TOL sigma_1}):
        B_r = (Xt^T Xt + lam I)^-1 Xt^T Rt V_r   (Cholesky),
    Xt = sqrt(w)(X - xbar), Rt = sqrt(w)(R - rbar).  If the ridge matrix is
    not positive definite (only possible with lam = 0), the feature term is
    dropped (r_eff = 0)."""
    d = X.shape[1]
    x_bar = w @ X
    r_bar = w @ R
    sw = np.sqrt(w)[:, None]
    Xt = sw * (X - x_bar)
    Rt = sw * (R - r_bar)
    _, sing, Vt = np.linalg.svd(Rt, full_matrices=False)
    if len(sing) == 0 or sing[0] <= 0:
        r_eff = 0
    else:
        r_eff = int(min(rank, np.count_nonzero(sing > RANK_TOL * sing[0])))
    V_r = Vt[:r_eff].T.copy()
    if r_eff == 0:
        return HeadFit(r_bar, x_bar, np.zeros((d, 0)), V_r, 0, sing)
    A = Xt.T @ Xt + lam * np.eye(d)
    try:
        L = np.linalg.cholesky(A)
    except np.linalg.LinAlgError:
        return HeadFit(r_bar, x_bar, np.zeros((d, 0)), np.zeros((d, 0)), 0, sing)
    rhs = Xt.T @ (Rt @ V_r)
    y = np.linalg.solve(L, rhs)          # forward substitution
    B_r = np.linalg.solve(L.T, y)        # back substitution
    return HeadFit(r_bar, x_bar, B_r, V_r, r_eff, sing)


def apply_correction(X: np.ndarray, fit: HeadFit) -> np.ndarray:
    """Corrected rows O = x + rbar + (x - xbar) B_r V_r^T [gist-nl 2B]: the
    fitted map's residual estimate is added to the sparse output; only the
    feature-dependent part is confined to span(V_r) [PL s4 Takeaways]."""
    return X + fit.r_bar[None, :] + ((X - fit.x_bar[None, :]) @ fit.B_r) @ fit.V_r.T


# --------------------------------------------------------------------------
# The whole call, one head
# --------------------------------------------------------------------------

@dataclass
class HeadResult:
    part: HeadPartition
    route: HeadRoute
    O_sparse: np.ndarray       # [N or len(rows), d], original order, rows as requested
    lse: np.ndarray
    probe_idx: np.ndarray
    probe_w: np.ndarray
    O_probe: np.ndarray        # exact dense rows at probe_idx
    fit: HeadFit
    O: np.ndarray              # final output rows (original order), float64 before the cast
    rows: np.ndarray
    X_probe: np.ndarray = field(repr=False, default=None)   # sparse output at probe_idx (the fit's regressor)


def sparsepr_head(Q, K, V, cfg, rows=None, prev=None) -> HeadResult:
    """One SparsePR attention call for one head, Q/K/V float64 [N, d] in
    original order.  `rows` restricts the sparse and final outputs to some
    original rows (the probe rows are always computed); the output covers the
    pipeline from response-coordinate construction to output restoration
    [PL C.3]."""
    N = Q.shape[0]
    s = cfg.softmax_scale
    part = partition_head(Q, K, cfg, prev)
    route = route_head(part, cfg, N)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    O_sp, lse = sparse_attention(Q, K, V, part, route, s, rows)
    probe_idx, probe_w = probe_select(part, cfg.M)
    if len(probe_idx):
        X, _ = sparse_attention(Q, K, V, part, route, s, probe_idx)
        O_dn, _ = dense_attention(Q, K, V, s, probe_idx)
        fit = fit_residual(X, O_dn - X, probe_w, cfg.rank, cfg.lam)
        O = apply_correction(O_sp, fit)
        where = {int(t): j for j, t in enumerate(probe_idx)}
        for i, t in enumerate(rows):
            j = where.get(int(t))
            if j is not None:
                O[i] = O_dn[j]
    else:
        X = O_dn = np.zeros((0, Q.shape[1]))
        fit = HeadFit(np.zeros(Q.shape[1]), np.zeros(Q.shape[1]), np.zeros((Q.shape[1], 0)),
                      np.zeros((Q.shape[1], 0)), 0)
        O = O_sp.copy()
    return HeadResult(part, route, O_sp, lse, probe_idx, probe_w, O_dn, fit, O, rows, X)


def sparsepr_call(Q, K, V, cfg, heads=None, rows=None):
    """The SparsePR call over heads (float64 arrays [H, N, d], original
    order); heads are independent.  Returns a list of HeadResult."""
    heads = range(Q.shape[0]) if heads is None else heads
    return [sparsepr_head(Q[h], K[h], V[h], cfg, rows) for h in heads]
