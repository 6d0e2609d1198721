"""Pins for the fp64 CPU oracle: closed forms, invariants, brute force and
hand-worked fixtures, each chosen so that a plausible slip in the oracle (a
dropped term, a wrong sign, index or power, a transposed operand) fails.

Pages: "Partition the Support, Reconstruct the Residual" (arXiv:2608.18484);
section names refer to the paperlayer.ai summary unless stated.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import sparsepr_oracle as o
from synth import get_config, make_qkv, as_f64, with_overrides

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _small_cfg(**kw):
    base = dict(H=1, N=512, d=16, dtype="fp32", frames=1, lat_h=16, lat_w=32, generator="clusters",
                G_k=6, G_q=5, M_s=32, r_k=8, iters_kv=5, iters_q=5, top_k=2, density=1.0, M=24,
                rank=4, lam=1e-3)
    base.update(kw)
    return with_overrides(get_config(0), **base)


# ---------------------------------------------------------------- stage 1

def test_sampled_query_indices_hand_worked():
    # appendix B.1: deterministic sampled queries (centred stride reading)
    for c in _gold("sampled_queries.json")["cases"]:
        assert o.sampled_query_indices(c["N"], c["M_s"]).tolist() == c["idx"]


def test_key_metric_on_basis_rows():
    # rows e_i repeated: M_K = diag(counts) / M_s, exactly
    d, M_s = 5, 10
    Q = np.zeros((M_s, d))
    rows = [0, 0, 1, 3, 3, 3, 4, 2, 2, 2]
    for t, i in enumerate(rows):
        Q[t, i] = 1.0
    M_K = o.key_response_metric(Q, M_s)
    assert np.array_equal(M_K, np.diag(np.bincount(rows, minlength=d) / M_s))


def test_key_coords_distance_identity_full_rank():
    # appendix B.1 with r_k = d and power 1/2: coordinate distances equal the
    # sampled-query response-profile distance ||Q_s (k_i - k_j)||^2 / (M_s tr M_K)
    rng = np.random.default_rng(1)
    N, d, M_s = 200, 12, 40
    Q = rng.standard_normal((N, d)) * np.linspace(0.3, 2.0, d)
    K = rng.standard_normal((30, d))
    M_K = o.key_response_metric(Q, M_s)
    U, w, lam = o.eigen_weighted_basis(M_K, d, 0.5)
    Z = o.key_response_coords(K, U, w)
    Qs = Q[o.sampled_query_indices(N, M_s)]
    for i, j in [(0, 1), (3, 17), (29, 5)]:
        lhs = np.sum((Z[i] - Z[j]) ** 2)
        rhs = np.sum((Qs @ (K[i] - K[j])) ** 2) / (M_s * np.trace(M_K))
        assert lhs == pytest.approx(rhs, rel=1e-11)


def test_key_coords_truncation_and_order():
    # diagonal metric: eigenvectors are basis vectors, largest first; Z keeps
    # the r_k heaviest coordinates scaled by sqrt(lambda / sum lambda)
    d, r = 6, 3
    a = np.array([1.0, 3.0, 0.5, 2.0, 4.0, 1.5])
    Q = np.diag(a)                                   # N = M_s = d: every row sampled
    M_K = o.key_response_metric(Q, d)
    U, w, lam = o.eigen_weighted_basis(M_K, r, 0.5)
    order = [4, 1, 3]
    assert np.allclose(lam, np.sort(a ** 2 / d)[::-1])
    assert np.allclose(U, np.eye(d)[:, order])
    assert np.allclose(w, np.sqrt(a[order] ** 2 / np.sum(a ** 2)))
    K = _rand((7, d), 2)
    assert np.allclose(o.key_response_coords(K, U, w), K[:, order] * w)
    # power 1 reading keeps the same directions with lambda/sum weights
    _, w1, _ = o.eigen_weighted_basis(M_K, r, 1.0)
    assert np.allclose(w1, a[order] ** 2 / np.sum(a ** 2))


def _bf_assign(X, C):
    lab = []
    for x in X.tolist():
        best, bi = None, -1
        for g, c in enumerate(C.tolist()):
            dist = sum((xi - ci) ** 2 for xi, ci in zip(x, c))
            if best is None or dist < best:
                best, bi = dist, g
        lab.append(bi)
    return np.array(lab)


def test_kmeans_init_and_fixed_point_bruteforce():
    X = _rand((90, 3), 3)
    G = 5
    init = X[(2 * np.arange(G) + 1) * 90 // (2 * G)]
    lab1, C1 = o.kmeans(X, G, 1)
    assert np.array_equal(lab1, _bf_assign(X, init))
    for T in (2, 4):
        _, C_prev = o.kmeans(X, G, T - 1)
        lab, C = o.kmeans(X, G, T)
        assert np.array_equal(lab, _bf_assign(X, C_prev))
        for g in range(G):
            mem = [X[t] for t in range(90) if lab[t] == g]
            want = np.sum(mem, axis=0) / len(mem) if mem else C_prev[g]
            assert np.allclose(C[g], want, rtol=0, atol=1e-14)


def test_kmeans_empty_cluster_keeps_centre_and_ties_go_low():
    # duplicate points: centres 0 and 1 start identical, every tie goes to 0,
    # so centre 1 stays empty and keeps its starting value
    X = np.array([[0.0], [0.0], [0.0], [0.0], [10.0], [10.0]])
    lab, C = o.kmeans(X, 3, 3)      # init rows 1, 3, 5 -> 0, 0, 10
    assert lab.tolist() == [0, 0, 0, 0, 2, 2]
    assert C.tolist() == [[0.0], [0.0], [10.0]]


def test_kmeans_recovers_planted_clusters():
    rng = np.random.default_rng(4)
    centres = rng.standard_normal((4, 8)) * 20
    truth = np.repeat(np.arange(4), 50)
    X = centres[truth] + rng.standard_normal((200, 8))
    lab, _ = o.kmeans(X, 4, 8)
    # same partition up to relabelling
    for g in range(4):
        assert len(set(lab[truth == g])) == 1
    assert len(set(lab)) == 4


def test_query_coords_two_groups_closed_form():
    # G' = 2: y = s q.(mu0-mu1)/2 * [1,-1], so yhat = sign(q.(mu0-mu1)) [1,-1]
    mu = np.array([[1.0, 2.0, 0.0], [0.0, -1.0, 3.0]])
    Q = _rand((10, 3), 5)
    Y = o.query_response_coords(Q, mu, np.array([3, 4]), 0.7)
    sgn = np.sign(Q @ (mu[0] - mu[1]))
    assert np.allclose(Y, sgn[:, None] * np.array([1.0, -1.0]), atol=1e-15)


def test_query_coords_ignore_empty_groups_and_invariances():
    mu = _rand((6, 5), 6)
    sizes = np.array([3, 0, 2, 7, 0, 1])
    Q = _rand((20, 5), 7)
    Y = o.query_response_coords(Q, mu, sizes, 0.3)
    assert Y.shape == (20, 4)                          # only nonempty groups
    assert np.allclose(np.mean(Y ** 2, axis=1), 1.0)   # RMS normalised
    # centring: adding one vector to every centroid changes nothing
    Y2 = o.query_response_coords(Q, mu + np.array([1.0, -2.0, 0.5, 3.0, 0.0]), sizes, 0.3)
    assert np.allclose(Y, Y2, atol=1e-12)
    # RMS: scaling the query or the softmax scale changes nothing
    assert np.allclose(Y, o.query_response_coords(2.5 * Q, mu, sizes, 0.3), atol=1e-13)
    assert np.allclose(Y, o.query_response_coords(Q, mu, sizes, 1.7), atol=1e-13)
    # the *empty* rows' values must not matter
    mu3 = mu.copy()
    mu3[[1, 4]] = 99.0
    assert np.allclose(Y, o.query_response_coords(Q, mu3, sizes, 0.3))
    # sign: the coordinate of group g grows with q.mu_g
    e = np.zeros(5)
    e[0] = 1.0
    y = o.query_response_coords(e[None, :], mu, sizes, 1.0)[0]
    nz = mu[sizes > 0]
    assert np.array_equal(np.argsort(y), np.argsort(nz[:, 0]))


def test_stable_permutation_properties():
    lab = np.array([2, 0, 2, 1, 0, 2, 2, 1])
    perm, off = o.stable_group_permutation(lab, 4)
    assert perm.tolist() == [1, 4, 3, 7, 0, 2, 5, 6]
    assert off.tolist() == [0, 2, 4, 8, 8]


# ---------------------------------------------------------------- stage 2

def test_route_budget_hand_worked():
    g = _gold("route_budget.json")
    P = np.array(g["P"])
    qs, ks = np.array(g["q_sizes"]), np.array(g["kv_sizes"])
    for c in g["cases"]:
        sel = o.select_cells_budget(P, qs, ks, c["budget"])
        assert sorted(map(list, zip(*np.nonzero(sel)))) == c["selected"]
        assert int((qs[:, None] * ks[None, :])[sel].sum()) == c["routed"]


def test_route_topk_hand_worked():
    # fixed top-k (section 4 "Sparse Execution"): descending score, ties to the
    # smaller b, empty K/V groups never chosen, empty query groups route nowhere
    g = _gold("route_topk.json")
    P = np.array(g["P"])
    qs, ks = np.array(g["q_sizes"]), np.array(g["kv_sizes"])
    for c in g["cases"]:
        sel = o.select_cells_topk(P, qs, ks, c["k"])
        assert sorted(map(list, zip(*np.nonzero(sel)))) == c["selected"], f"k={c['k']}"
        assert int((qs[:, None] * ks[None, :])[sel].sum()) == c["routed"], f"k={c['k']}"


def test_cell_scores_closed_forms():
    qs = np.array([3, 0, 5])
    ks = np.array([2, 6, 0, 4])
    mu = _rand((4, 3), 8)
    # zero query centroid: P is proportional to K/V group size
    P = o.cell_scores(np.zeros((3, 3)), qs, mu, ks, 0.5)
    assert np.allclose(P[0], [2 / 12, 6 / 12, 0, 4 / 12]) and np.all(P[1] == 0)
    # ratio form: P_a0 / P_a1 = (n0/n1) exp(s qbar.(mu0 - mu1))
    qbar = _rand((3, 3), 9)
    P = o.cell_scores(qbar, qs, mu, ks, 0.5)
    want = (2 / 6) * math.exp(0.5 * qbar[2] @ (mu[0] - mu[1]))
    assert P[2, 0] / P[2, 1] == pytest.approx(want, rel=1e-12)
    assert np.allclose(P[[0, 2]].sum(axis=1), 1.0) and np.all(P[:, 2] == 0)


def test_route_topk_and_budget_properties():
    cfg = _small_cfg(top_k=0, density=0.3, M=16)
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    part = o.partition_head(Q, K, cfg)
    r = o.route_head(part, cfg, cfg.N)
    qs, ks = np.diff(part.q_off), np.diff(part.kv_off)
    budget = o.pair_budget(cfg.density, cfg.N, cfg.M)
    mand = 0
    for a in range(cfg.G_q):
        cols = r.col_idx[r.row_ptr[a]:r.row_ptr[a + 1]]
        assert np.all(np.diff(cols) > 0)
        if qs[a] == 0:
            assert len(cols) == 0
            continue
        assert len(cols) >= 1
        valid = np.flatnonzero(ks > 0)
        ranking = valid[np.argsort(-r.P[a, valid], kind="stable")]
        assert set(cols) == set(ranking[:len(cols)])        # a prefix of its own ranking
        mand += qs[a] * ks[ranking[0]]
    assert r.routed_pairs <= max(budget, mand)
    assert r.routed_pairs == sum(qs[a] * ks[b] for a in range(cfg.G_q)
                                 for b in r.col_idx[r.row_ptr[a]:r.row_ptr[a + 1]])
    top = o.select_cells_topk(r.P, qs, ks, 2)
    assert all(top[a].sum() == min(2, np.count_nonzero(ks)) for a in range(cfg.G_q) if qs[a] > 0)


def test_probe_density_matches_page_figure():
    # appendix A.2: 64 probe rows contribute M/N_q = 0.054% to 0.145%
    assert round(100 * o.executed_pair_density(0, 64, 118800), 3) == 0.054
    assert round(100 * o.executed_pair_density(0, 64, 44138), 3) == 0.145
    assert o.pair_budget(0.25, 100, 3) == 2500 - 300


# ---------------------------------------------------------------- stage 3

def test_dense_attention_two_key_closed_form():
    q = np.array([[0.3, -1.2, 0.5]])
    k = np.array([[1.0, 0.5, -0.2], [-0.4, 0.1, 0.9]])
    v = np.array([[2.0, -1.0], [0.5, 4.0]])
    s = 0.8
    O, lse = o.dense_attention(q, k, v, s)
    a1, a2 = s * q[0] @ k[0], s * q[0] @ k[1]
    p = 1.0 / (1.0 + math.exp(a2 - a1))
    assert np.allclose(O[0], p * v[0] + (1 - p) * v[1], atol=1e-15)
    assert lse[0] == pytest.approx(math.log(math.exp(a1) + math.exp(a2)), rel=1e-14)


def test_sparse_attention_matches_bruteforce_mask():
    # explicit N x N mask in pure Python floats vs the group-gather version
    cfg = _small_cfg(N=48, d=4, lat_h=6, lat_w=8, G_k=4, G_q=3, M_s=12, r_k=4, top_k=2, M=0)
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    part = o.partition_head(Q, K, cfg)
    r = o.route_head(part, cfg, cfg.N)
    routed = {a: set(r.col_idx[r.row_ptr[a]:r.row_ptr[a + 1]].tolist()) for a in range(cfg.G_q)}
    mask = [[int(part.kv_label[u]) in routed[int(part.q_label[t])] for u in range(48)] for t in range(48)]
    assert any(not all(row) for row in mask)            # something is dropped
    bf = np.array(o.masked_attention_bruteforce(Q.tolist(), K.tolist(), V.tolist(), mask, cfg.softmax_scale))
    O, _ = o.sparse_attention(Q, K, V, part, r, cfg.softmax_scale)
    assert np.allclose(O, bf, rtol=0, atol=1e-12)
    # rows subset gives the same rows
    rows = np.array([47, 3, 20])
    Or, _ = o.sparse_attention(Q, K, V, part, r, cfg.softmax_scale, rows)
    assert np.allclose(Or, O[rows], rtol=0, atol=1e-14)


def test_full_routing_equals_dense():
    # spec invariant: every cell routed, no probes -> dense attention
    cfg = _small_cfg(top_k=6, M=0)
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    res = o.sparsepr_head(Q, K, V, cfg)
    Od, lse = o.dense_attention(Q, K, V, cfg.softmax_scale)
    assert np.allclose(res.O_sparse, Od, rtol=0, atol=1e-12)
    assert np.allclose(res.lse, lse, rtol=0, atol=1e-12)
    assert np.array_equal(res.O, res.O_sparse)


def test_single_group_equals_dense():
    cfg = _small_cfg(G_k=1, G_q=1, top_k=0, density=0.01, M=0)
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    res = o.sparsepr_head(Q, K, V, cfg)
    assert res.route.routed_pairs == cfg.N * cfg.N     # mandatory cell exceeds the budget
    Od, _ = o.dense_attention(Q, K, V, cfg.softmax_scale)
    assert np.allclose(res.O_sparse, Od, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- stage 4

def test_probe_allocation_hand_worked():
    g = _gold("probe_allocation.json")
    for c in g["cases"]:
        assert o.probe_allocation(np.array(c["sizes"]), c["M"]).tolist() == c["m"]


def test_probe_selection_ranks_and_weights():
    g = _gold("probe_allocation.json")
    # build a partition by hand: one group per size, distances descending in t
    for c in g["cases"]:
        sizes = np.array(c["sizes"])
        N = int(sizes.sum())
        lab = np.repeat(np.arange(len(sizes)), sizes)
        dist = np.arange(N, 0, -1, dtype=np.float64)
        perm, off = o.stable_group_permutation(lab, len(sizes))
        part = o.HeadPartition(lab, lab, perm, perm, off, off, None, None, dist)
        idx, w = o.probe_select(part, c["M"])
        assert abs(w.sum() - 1.0) < 1e-15
        for a, m_a in enumerate(c["m"]):
            mine = [t for t in idx if lab[t] == a]
            assert len(mine) == m_a
            if m_a:
                members = np.flatnonzero(lab == a)[::-1]        # ascending distance
                ranks = [(2 * j + 1) * sizes[a] // (2 * m_a) for j in range(m_a)]
                assert sorted(mine) == sorted(members[ranks].tolist())
                assert np.allclose(w[np.isin(idx, mine)], c["weights_by_group"][a])
    for r in g["ranks"]:
        assert [(2 * j + 1) * r["n"] // (2 * r["m"]) for j in range(r["m"])] == r["ranks"]


def test_probe_selection_tie_break_on_index():
    lab = np.zeros(6, dtype=np.int64)
    dist = np.array([1.0, 0.5, 1.0, 0.5, 1.0, 0.5])
    perm, off = o.stable_group_permutation(lab, 1)
    part = o.HeadPartition(lab, lab, perm, perm, off, off, None, None, dist)
    idx, _ = o.probe_select(part, 3)
    # order by (dist, t): 1,3,5,0,2,4 -> ranks 1,3,5 -> t = 3,0,4
    assert idx.tolist() == [0, 3, 4]


# ---------------------------------------------------------------- stage 5

def test_ridge_matches_augmented_lstsq_and_large_lambda():
    rng = np.random.default_rng(10)
    Mp, d = 40, 6
    X = rng.standard_normal((Mp, d))
    R = rng.standard_normal((Mp, d)) * 0.1 + X @ rng.standard_normal((d, d)) * 0.05
    w = rng.uniform(0.5, 2.0, Mp)
    w /= w.sum()
    lam = 0.03
    fit = o.fit_residual(X, R, w, 3, lam)
    assert fit.rank_eff == 3
    xbar, rbar = w @ X, w @ R
    Xt = np.sqrt(w)[:, None] * (X - xbar)
    Rt = np.sqrt(w)[:, None] * (R - rbar)
    A = np.vstack([Xt, math.sqrt(lam) * np.eye(d)])
    b = np.vstack([Rt @ fit.V_r, np.zeros((d, 3))])
    B_ls = np.linalg.lstsq(A, b, rcond=None)[0]
    assert np.allclose(fit.B_r, B_ls, atol=1e-12)
    assert np.allclose(fit.x_bar, xbar) and np.allclose(fit.r_bar, rbar)
    # huge ridge: the feature term vanishes and the correction is the weighted mean residual
    big = o.fit_residual(X, R, w, 3, 1e12)
    Xn = rng.standard_normal((5, d))
    assert np.allclose(o.apply_correction(Xn, big) - Xn, rbar[None, :], atol=1e-9)


def test_planted_affine_residual_is_recovered():
    # R = b + x B0 with B0 = C P^T (rank 2 inside span(P)); lam = 0, rank >= 2
    rng = np.random.default_rng(11)
    Mp, d = 30, 5
    X = rng.standard_normal((Mp, d))
    Pbasis = np.linalg.qr(rng.standard_normal((d, 2)))[0]
    B0 = rng.standard_normal((d, 2)) @ Pbasis.T
    b = rng.standard_normal(d)
    R = b + X @ B0
    w = np.full(Mp, 1.0 / Mp)
    fit = o.fit_residual(X, R, w, 4, 0.0)
    assert fit.rank_eff == 2                               # numerical rank of the centred residual
    Xn = rng.standard_normal((7, d))
    assert np.allclose(o.apply_correction(Xn, fit) - Xn, b + Xn @ B0, atol=1e-10)
    # with rank 1 the feature term is confined to one direction of span(P)
    fit1 = o.fit_residual(X, R, w, 1, 0.0)
    corr = (Xn - fit1.x_bar) @ fit1.B_r @ fit1.V_r.T
    assert np.allclose(corr @ Pbasis @ Pbasis.T, corr, atol=1e-10)


def test_subspace_is_top_energy_and_orthonormal():
    rng = np.random.default_rng(12)
    Mp, d, r = 50, 8, 3
    X = rng.standard_normal((Mp, d))
    R = rng.standard_normal((Mp, d)) * np.array([5, 4, 3, 0.5, 0.4, 0.3, 0.2, 0.1])
    w = np.full(Mp, 1.0 / Mp)
    fit = o.fit_residual(X, R, w, r, 1e-3)
    assert np.allclose(fit.V_r.T @ fit.V_r, np.eye(r), atol=1e-12)
    Rt = np.sqrt(w)[:, None] * (R - w @ R)
    best = np.sum((Rt @ fit.V_r) ** 2)
    for s in range(20):                                  # Eckart-Young: no other r-frame captures more
        F = np.linalg.qr(rng.standard_normal((d, r)))[0]
        assert np.sum((Rt @ F) ** 2) <= best + 1e-12
    assert best == pytest.approx(np.sum(np.sort(np.linalg.eigvalsh(Rt.T @ Rt))[::-1][:r]), rel=1e-10)


def test_correction_formula_tiny_hand_case():
    fit = o.HeadFit(np.array([0.1, -0.2]), np.array([1.0, 2.0]), np.array([[2.0], [0.0]]),
                    np.array([[0.0], [1.0]]), 1)
    x = np.array([[3.0, 5.0]])
    # x + rbar + (x - xbar) B V^T = [3,5] + [.1,-.2] + ([2,3].[2,0]) [0,1] = [3.1, 8.8]
    assert np.allclose(o.apply_correction(x, fit), [[3.1, 8.8]])


# ---------------------------------------------------------------- whole call

def test_probe_rows_are_dense_rows_exactly():
    cfg = _small_cfg(top_k=2, M=24)
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    res = o.sparsepr_head(Q, K, V, cfg)
    Od, _ = o.dense_attention(Q, K, V, cfg.softmax_scale, res.probe_idx)
    assert len(res.probe_idx) == 24
    assert np.array_equal(res.O[res.probe_idx], Od)
    assert np.all(np.diff(res.probe_idx) > 0)


def test_nothing_dropped_means_no_correction():
    cfg = _small_cfg(top_k=6, M=24)
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    res = o.sparsepr_head(Q, K, V, cfg)
    Od, _ = o.dense_attention(Q, K, V, cfg.softmax_scale)
    assert np.abs(res.fit.r_bar).max() < 1e-14
    assert np.allclose(res.O, Od, rtol=0, atol=1e-12)


def test_no_probes_means_sparse_output():
    cfg = _small_cfg(top_k=2, M=0)
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    res = o.sparsepr_head(Q, K, V, cfg)
    assert np.array_equal(res.O, res.O_sparse)
    assert len(res.probe_idx) == 0


def test_partition_outputs_consistent():
    cfg = _small_cfg()
    Q, K, V = (as_f64(t)[0] for t in make_qkv(cfg))
    p = o.partition_head(Q, K, cfg)
    for lab, perm, off, G in ((p.kv_label, p.kv_perm, p.kv_off, cfg.G_k),
                              (p.q_label, p.q_perm, p.q_off, cfg.G_q)):
        assert sorted(perm.tolist()) == list(range(cfg.N))
        assert np.all(np.diff(lab[perm]) >= 0)
        for g in range(G):
            seg = perm[off[g]:off[g + 1]]
            assert np.all(lab[seg] == g) and np.all(np.diff(seg) > 0)
    # raw-space centroids are the member means
    for g in range(cfg.G_q):
        if p.q_off[g + 1] > p.q_off[g]:
            assert np.allclose(p.q_centroid[g], Q[p.q_label == g].mean(axis=0))
    # q_dist is the distance to the final query-coordinate centre
    lab, C = o.kmeans(p.query_coords, cfg.G_q, cfg.iters_q)
    assert np.allclose(p.q_dist, np.sum((p.query_coords - C[lab]) ** 2, axis=1))


def test_distance_rank_key_merges_rounding_noise_only():
    # values a few ulps apart rank as equal (the index decides); values that
    # differ in the 30th significant bit do not
    x = 7.123456789
    near = np.nextafter(np.nextafter(x, 10.0), 10.0)
    assert o.distance_rank_key(x) == o.distance_rank_key(near)
    assert o.distance_rank_key(x) < o.distance_rank_key(x * (1 + 2.0 ** -27))
    assert o.distance_rank_key(0.0) == 0.0
    # monotone on a sweep of magnitudes
    xs = np.sort(np.abs(np.random.default_rng(3).standard_normal(2000)) * 10.0 ** np.arange(-3, 3).repeat(334)[:2000])
    keys = np.array([o.distance_rank_key(v) for v in xs])
    assert np.all(np.diff(keys) >= 0)
    # within 2^-30 of the value
    assert np.all(np.abs(keys - xs) <= xs * 2.0 ** -30)


def test_distance_rank_key_at_a_rounding_boundary():
    # The key is a fixed function of the float64 value (30 significant bits,
    # half up).  At 1 + 2^-30, the midpoint between the keys 1 and 1 + 2^-29,
    # the value rounds up and its lower neighbour rounds down: two distances
    # one ulp apart get keys one step apart and rank by distance, not by
    # index.  So the probe order depends on the side of the boundary each
    # distance falls on; both sides compute the key from their own float64
    # distance, and parity needs those on the same side (for independent
    # rounding errors of a few ulps the chance of a straddle is about 2^-20
    # per tied pair).
    mid = 1.0 + 2.0 ** -30
    below = np.nextafter(mid, 0.0)
    assert o.distance_rank_key(mid) == 1.0 + 2.0 ** -29
    assert o.distance_rank_key(below) == 1.0
    assert o.distance_rank_key(np.nextafter(mid, 2.0)) == 1.0 + 2.0 ** -29

    def pick(dists):
        part = o.HeadPartition(kv_label=np.zeros(2, np.int64), q_label=np.zeros(2, np.int64),
                               kv_perm=np.arange(2), q_perm=np.arange(2), kv_off=np.array([0, 2]),
                               q_off=np.array([0, 2]), kv_centroid=np.zeros((1, 2)),
                               q_centroid=np.zeros((1, 2)), q_dist=np.array(dists))
        return o.probe_select(part, 1)[0].tolist()
    # one probe in a group of two takes rank 1, the later member in key order
    assert pick([below, mid]) == [1]       # keys 1 < 1 + 2^-29
    assert pick([mid, below]) == [0]       # the same two distances swapped
    assert pick([below, below]) == [1]     # equal keys: the index decides


def test_probe_selection_two_member_group_tie_is_ranked_by_index():
    # a group of two points: both lie at the same distance from their mean in
    # exact arithmetic; with one probe the rank is floor(2/2) = 1, the later
    # of the two in (distance, index) order, i.e. the higher index
    part = o.HeadPartition(kv_label=np.zeros(2, np.int64), q_label=np.zeros(2, np.int64),
                           kv_perm=np.arange(2), q_perm=np.arange(2), kv_off=np.array([0, 2]),
                           q_off=np.array([0, 2]), kv_centroid=np.zeros((1, 2)), q_centroid=np.zeros((1, 2)),
                           q_dist=np.array([0.3 + 2 ** -52, 0.3]))
    idx, w = o.probe_select(part, 1)
    assert idx.tolist() == [1] and np.allclose(w, [1.0])


def test_semantic_partition_clusters_raw_activations():
    # The semantic baseline clusters the raw rows: with four planted clusters
    # 30 units apart (unit noise), laid out cluster by cluster so that the
    # centred-stride initial rows fall one in each, every group is exactly one
    # planted cluster for both keys and queries, and q_dist is the squared
    # distance to the group mean in raw query space (scale ~ d, not G').
    rng = np.random.default_rng(7)
    d, n, G = 8, 400, 4
    planted = np.repeat(np.arange(G), n // G)
    centres = 30.0 * np.eye(G, d)
    Q = centres[planted] + rng.standard_normal((n, d))
    K = centres[planted] + rng.standard_normal((n, d))
    cfg = with_overrides(get_config(0), N=n, d=d, G_k=G, G_q=G, M=8, rank=2, partition="semantic")
    part = o.partition_head(Q, K, cfg)
    assert np.array_equal(part.kv_label, planted)
    assert np.array_equal(part.q_label, planted)
    means = np.stack([Q[planted == g].mean(axis=0) for g in range(G)])
    np.testing.assert_allclose(part.q_dist, ((Q - means[planted]) ** 2).sum(axis=1), rtol=1e-12)
    assert 4.0 < part.q_dist.mean() < 12.0
    # and the response-coupled partition of the same rows lives in other coordinates
    resp = o.partition_head(Q, K, with_overrides(cfg, partition="response", M_s=64, r_k=4))
    assert not np.allclose(resp.q_dist, part.q_dist)


def test_support_size_closed_forms():
    from oracle.diagnostics import support_size
    # uniform over 10 keys: mass 0.9 needs exactly 9 keys; one-hot needs 1
    assert len(support_size(np.full(10, 0.1), 0.9)) == 9
    assert list(support_size(np.eye(6)[4], 0.9)) == [4]
    # largest first: 0.5 + 0.3 + 0.15 reaches 0.9 with three keys
    assert sorted(support_size(np.array([0.05, 0.5, 0.15, 0.3]), 0.9).tolist()) == [1, 2, 3]


def test_pooled_support_of_identical_queries_is_their_support():
    from oracle.diagnostics import pooled_support
    rng = np.random.default_rng(3)
    N, d = 64, 8
    K = rng.standard_normal((N, d))
    Q = np.repeat(rng.standard_normal((1, d)), 16, axis=0)        # 16 copies of one query, one group
    part = o.HeadPartition(np.zeros(N, int), np.zeros(16, int), np.arange(N), np.arange(16), np.array([0, N]),
                           np.array([0, 16]), np.zeros((1, d)), np.zeros((1, d)), np.zeros(16))
    per, pooled = pooled_support(Q, K, part, 0.5, 0.9, 8)
    assert len(pooled) == 1 and np.allclose(per, per[0]) and pooled[0] == per[0]


def test_affine_split_exact_and_orthogonal_cases():
    from oracle.diagnostics import affine_residual_split
    rng = np.random.default_rng(5)
    X = rng.standard_normal((200, 6))
    R = 0.3 + X @ rng.standard_normal((6, 4))                   # exactly affine in X
    frac, orth, _ = affine_residual_split(X, R)
    assert frac > 1 - 1e-12 and orth < 1e-20 * 200
    A = np.hstack([np.ones((200, 1)), X])
    P = rng.standard_normal((200, 4))
    Rp = P - A @ np.linalg.lstsq(A, P, rcond=None)[0]            # orthogonal to [1, X]
    frac, orth, tot = affine_residual_split(X, Rp)
    assert abs(frac) < 1e-12 and np.isclose(orth, tot)


def test_warm_start_from_a_fixed_point_keeps_it():
    # Lloyd from the labels a cold run converged to: the centres are those
    # labels' means, so one more round reproduces the labels exactly.
    rng = np.random.default_rng(11)
    X = np.vstack([rng.normal(c, 0.5, size=(40, 3)) for c in (-6.0, 0.0, 6.0, 12.0)])
    lab, C = o.kmeans(X, 4, 50)
    lab_w, C_w = o.kmeans(X, 4, 1, init_labels=lab)
    assert np.array_equal(lab_w, lab)
    np.testing.assert_allclose(C_w, C, rtol=0, atol=1e-12)


def test_warm_start_empty_group_uses_stride_row_and_labels_are_clamped():
    # 1-D points; previous labels leave group 1 empty (and carry two out-of-range
    # values, clamped to 0 and G-1): initial centres are mean(0, 1, 2) = 1,
    # the stride row floor(3*6/6) = 3 -> x = 30, and mean(20, 21, 22) = 21.
    X = np.array([[0.0], [1.0], [2.0], [30.0], [20.0], [22.0]])
    init = np.array([0, 0, -4, 7, 2, 2])          # -4 -> 0, 7 -> 2: groups {0,1,2}, {}, {3,4,5}
    # group 2 = rows 3, 4, 5 -> mean(30, 20, 22) = 24; group 1 starts at row 3 -> 30
    lab, C = o.kmeans(X, 3, 1, init_labels=init)
    # brute force on the initial centres [1, 30, 24]
    c0 = np.array([1.0, 30.0, 24.0])
    want = np.argmin((X - c0[None, :]) ** 2, axis=1)
    assert np.array_equal(lab, want)
    assert list(want) == [0, 0, 0, 1, 2, 2]


# ---------------------------------------------------------------- near ties, eigen-gap

def test_assignment_near_ties_hand_worked():
    from oracle.diagnostics import assignment_near_ties
    C = np.array([[0.0, 0.0], [2.0, 0.0]])
    X = np.array([[1.0, 0.0],            # equidistant: a tie
                  [0.2, 0.0],            # clearly nearer centre 0
                  [1.0 + 1e-6, 0.0],     # gap 4e-6 of 1: not a tie at 1e-9
                  [1.0 + 1e-11, 0.0],    # gap 4e-11: a tie
                  [1.0, 5.0]])           # equidistant off the axis: a tie
    assert assignment_near_ties(X, C).tolist() == [0, 3, 4]
    assert assignment_near_ties(X, C[:1]).tolist() == []   # one centre: nothing to tie with


def test_kmeans_near_ties_follow_the_last_assignment():
    from oracle.diagnostics import kmeans_near_ties
    # 1-d points 0..3, G = 2: the start rows are 1 and 3, so point 2 is equidistant; the
    # first round gives it the lower centre (ties to the lowest index), the means move to
    # 1 and 3 again, and the second assignment ties on it once more
    X = np.arange(4.0)[:, None]
    assert kmeans_near_ties(X, 2, 1).tolist() == [2]
    assert kmeans_near_ties(X, 2, 2).tolist() == [2]
    labels, _ = o.kmeans(X, 2, 2)
    assert labels.tolist() == [0, 0, 0, 1]


def test_eigen_gap_hand_worked():
    from oracle.diagnostics import eigen_gap
    R = np.linalg.qr(_rand((4, 4), 12))[0]
    M = (R * np.array([5.0, 3.0, 3.0, 1.0])[None, :]) @ R.T
    assert eigen_gap(M, 1) == pytest.approx(0.4, abs=1e-14)        # (5 - 3) / 5
    assert abs(eigen_gap(M, 2)) < 1e-14                             # r_k splits the repeated pair
    assert eigen_gap(M, 3) == pytest.approx(0.4, abs=1e-14)        # (3 - 1) / 5
    assert eigen_gap(M, 4) == 1.0 and eigen_gap(np.zeros((3, 3)), 1) == 0.0


def test_route_near_ties_hand_worked():
    from oracle.diagnostics import route_near_ties
    P = np.array([[0.6, 0.2, 0.2], [0.7, 0.15, 0.15], [0.5, 0.25, 0.25], [0.4, 0.4, 0.2]])
    ones = np.ones(4, dtype=int)
    kv = np.ones(3, dtype=int)
    # the kept best cells (row 3 keeps (3,0): tie to the smaller b) use 4 pairs; the scan
    # order of the rest is (3,1) .4, (2,1) .25, (2,2) .25, (0,1) .2, ...; with budget 6,
    # (3,1) -> 5 and (2,1) -> 6 fit and (2,2) would make 7: the cut is at 0.25, tied with (2,1)
    r = route_near_ties(P, ones, kv, budget=6)
    assert r["mandatory"] == 1                      # row 3: 0.4 against 0.4
    assert r["budget_cut"] == 1
    assert route_near_ties(P, ones, kv, k=2)["topk"] == 3   # rows 0, 1, 2 tie at their 2nd/3rd cells
    sel = o.select_cells_budget(P, ones, kv, 6)
    assert sorted(map(list, zip(*np.nonzero(sel)))) == [[0, 0], [1, 0], [2, 0], [2, 1], [3, 0], [3, 1]]
