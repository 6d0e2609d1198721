"""The symmetric eigensolver of stages 1 and 4 on clustered spectra, through
the C ABI (sparsepr_sym_eigen), and a partition whose sampled-query metric
M_K has an exactly repeated leading eigenvalue inside the r_k directions
(paperlayer.ai appendix B.1: key coordinates from the leading
eigendirections of M_K; appendix A.3: the residual subspace from the
leading singular directions).

Checks against numpy's eigendecomposition: eigenvalues within 1e-12 ||A||,
eigenvectors orthonormal within 1e-10, residuals ||A v - lam v|| within
1e-10 ||A||, the sign convention, and the invariant subspace of every
cluster that lies wholly among the computed pairs (its projector), since
vectors inside a cluster are not unique."""
import numpy as np
import pytest
import torch

import free_block_sparse_group_amd as fb
from gpu_common import compare_head, log, run_gpu
from oracle import sparsepr_oracle as o
from synth import as_f64, get_config, make_qkv, with_overrides

pytestmark = pytest.mark.gpu


def hadamard(n):
    Hm = np.ones((1, 1))
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def random_orthogonal(d, seed):
    q, r = np.linalg.qr(np.random.default_rng(seed).standard_normal((d, d)))
    return q * np.sign(np.diag(r))[None, :]


def spectrum_cases(d):
    rng = np.random.default_rng([d, 5])
    tail = np.sort(rng.uniform(0.1, 2.0, d))[::-1]
    cases = {}
    # exactly repeated eigenvalues on a permuted diagonal (T splits exactly)
    lam = tail.copy()
    lam[:6] = [9.0, 9.0, 6.25, 4.0, 4.0, 4.0]
    cases["diag_repeats"] = (np.diag(lam[rng.permutation(d)]), 12)
    # exactly repeated eigenvalues in a Hadamard basis (entries exact in float64)
    Hn = hadamard(d)
    lam = np.round(tail * 64) / 64
    lam[:5] = [9.0, 9.0, 9.0, 6.25, 6.25]
    cases["hadamard_repeats"] = ((Hn * lam[None, :]) @ Hn / d, 10)
    # near-clusters at relative gaps 1e-13 .. 1e-6 in a random basis
    lam = tail.copy()
    lam[:8] = [10.0, 10.0 * (1 + 1e-13), 10.0 * (1 + 1e-9), 10.0 * (1 + 1e-6), 5.0, 5.0 * (1 + 1e-12), 3.0,
               3.0 * (1 + 1e-10)]
    R = random_orthogonal(d, [d, 6])
    A = (R * lam[None, :]) @ R.T
    cases["near_clusters"] = ((A + A.T) / 2, 16)
    # a rank-5 positive semi-definite matrix: 11 zero eigenvalues among the 16 asked for
    X = rng.standard_normal((5, d))
    cases["rank5_zero_cluster"] = (X.T @ X / 5, 16)
    # a generic symmetric matrix
    G = rng.standard_normal((d, d))
    cases["generic"] = ((G + G.T) / 2, 32)
    return cases


def check_eigen(A, nev, lam_g, vec_g, name):
    d = A.shape[0]
    nrm = np.abs(np.linalg.eigvalsh(A)).max()
    w, U = np.linalg.eigh(A)
    order = np.argsort(-w, kind="stable")
    w, U = w[order], U[:, order]
    V = vec_g.T                                        # [d, nev]
    lam_err = np.abs(lam_g - w[:nev]).max() / nrm
    orth = np.abs(V.T @ V - np.eye(nev)).max()
    res = np.abs(A @ V - V * lam_g[None, :]).max() / nrm
    log(f"  {name} d={d} nev={nev}: eigenvalue err {lam_err:.2e}, orthogonality {orth:.2e}, residual {res:.2e}")
    assert lam_err <= 1e-12, f"{name}: eigenvalues off by {lam_err:.3g} ||A||"
    assert orth <= 1e-10, f"{name}: eigenvectors not orthonormal ({orth:.3g})"
    assert res <= 1e-10, f"{name}: residual {res:.3g} ||A||"
    # sign convention: the largest-magnitude entry is positive (lowest index on ties)
    for e in range(nev):
        j = int(np.argmax(np.abs(V[:, e])))
        assert V[j, e] > 0, f"{name}: vector {e} breaks the sign convention"
    # invariant subspaces of clusters (gap <= 1e-5 ||A||) wholly inside the computed pairs
    e = 0
    while e < nev:
        f = e + 1
        while f < d and w[f - 1] - w[f] <= 1e-5 * nrm:
            f += 1
        if f <= nev and f - e > 1:
            Pg = V[:, e:f] @ V[:, e:f].T
            Pr = U[:, e:f] @ U[:, e:f].T
            dp = np.abs(Pg - Pr).max()
            log(f"    cluster {e}..{f - 1}: projector difference {dp:.2e}")
            assert dp <= 1e-9, f"{name}: cluster {e}..{f - 1} spans a different subspace ({dp:.3g})"
        e = f


@pytest.mark.parametrize("d", [64, 128])
def test_sym_eigen_clustered_spectra(d):
    cases = spectrum_cases(d)
    names = list(cases)
    A = np.stack([cases[n][0] for n in names])
    nev = max(cases[n][1] for n in names)
    log(f"[eigen] d={d}: {names}, nev={nev}")
    lam, vec = fb.sym_eigen(torch.from_numpy(A).cuda(), nev)
    torch.cuda.synchronize()
    lam, vec = lam.cpu().numpy(), vec.cpu().numpy()
    for i, n in enumerate(names):
        k = cases[n][1]
        check_eigen(A[i], k, lam[i, :k], vec[i, :k], n)


def test_partition_with_repeated_leading_eigenvalue():
    # the sampled queries are Hd diag(s) Hd / 8 (bf16-exact), so
    # M_K = (Hd/8) diag(s^2) (Hd/8) with eigenvalues 9, 9, 6.25, 4, 2.25, 1,
    # 0.25, 0, ...: the repeated leading pair lies inside r_k = 6 with equal
    # weights, so key coordinate distances do not depend on the basis the
    # solver picks inside it, and labels must match the oracle's bit for bit
    cfg = with_overrides(get_config(1), H=2, N=2048, frames=2, lat_h=32, lat_w=32, G_k=16, G_q=12, M=40, rank=8,
                         M_s=64, r_k=6)
    Q, K, V = make_qkv(cfg)
    d = cfg.d
    Hd = hadamard(d)
    s = np.zeros(d)
    s[:7] = [3.0, 3.0, 2.5, 2.0, 1.5, 1.0, 0.5]
    Qs = (Hd * s[None, :]) @ Hd / 8
    idx = o.sampled_query_indices(cfg.N, cfg.M_s)
    for h in range(cfg.H):
        Q[h, idx] = torch.from_numpy(Qs).to(torch.bfloat16)
    assert np.array_equal(as_f64(Q[0, idx]), Qs), "the sampled rows must be exact in bf16"
    log("[eigen] partition with M_K eigenvalues 9, 9, 6.25, ... (r_k = 6)")
    b, _ = run_gpu(cfg, Q, K, V)
    Q64, K64, V64 = as_f64(Q), as_f64(K), as_f64(V)
    for h in range(cfg.H):
        MK = o.key_response_metric(Q64[h], cfg.M_s)
        ev = np.sort(np.linalg.eigvalsh(MK))[::-1]
        assert abs(ev[0] - 9.0) < 1e-12 and abs(ev[1] - 9.0) < 1e-12 and ev[6] < ev[5]
        ref = o.sparsepr_head(Q64[h], K64[h], V64[h], cfg)
        diag = compare_head(cfg, b, h, ref, Q[h], K[h], V[h])
        log(f"  head {h}: {diag}")
