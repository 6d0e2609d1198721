"""Shared helpers of the GPU tests: run the HIP path through the C ABI and
compare it with the float64 oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import free_block_sparse_group_amd as fb
from oracle import diagnostics as od
from oracle import sparsepr_oracle as o
from synth import as_f64, make_qkv


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def out_tol(cfg):
    """Element-wise output tolerance: max-abs 1e-4 for float32 inputs, 2e-2 for bf16."""
    return 1e-4 if cfg.dtype == "fp32" else 2e-2


def relf_tol(cfg):
    """Relative Frobenius bound on the float32 intermediates (sparse output,
    exact probe rows): 1e-5 for float32 inputs, 1e-3 for bf16 inputs (scores
    on bf16 operands, fp16 weights in P.V)."""
    return 1e-5 if cfg.dtype == "fp32" else 1e-3


def half_ulp(cfg, ref):
    """Half a unit in the last place of the output dtype at each reference
    value: the final output is stored in the input dtype, so a bf16 output
    cannot be closer to the float64 value than this."""
    if cfg.dtype == "fp32":
        return np.zeros_like(ref)
    mag = np.maximum(np.abs(ref), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(mag)) - 8)


def run_gpu(cfg, Q, K, V):
    Qd, Kd, Vd = (t.cuda() for t in (Q, K, V))
    b = fb.SparsePRBuffers(cfg)
    fb.run_sparsepr(b, Qd, Kd, Vd)
    torch.cuda.synchronize()
    return b, (Qd, Kd, Vd)


def host(t):
    return t.detach().cpu().numpy()


def compare_head(cfg, b, h, ref: "o.HeadResult", Qh, Kh, Vh, check_outputs=True):
    """Compare head h of the GPU buffers with the oracle result; returns a dict
    of diagnostics and raises AssertionError on a parity failure."""
    N, d = cfg.N, cfg.d
    diag = {}
    part = ref.part
    # ---- partition: bit-exact integers
    kv_label = host(b.kv_label[h]).astype(np.int64)
    q_label = host(b.q_label[h]).astype(np.int64)
    diag["kv_label_mismatch"] = int(np.count_nonzero(kv_label != part.kv_label))
    diag["q_label_mismatch"] = int(np.count_nonzero(q_label != part.q_label))
    Q64, K64 = as_f64(Qh), as_f64(Kh)
    diag["eigen_gap_rk"] = od.eigen_gap(o.key_response_metric(Q64, cfg.M_s), cfg.r_k)
    if diag["kv_label_mismatch"] or diag["q_label_mismatch"]:
        # classify before failing: differing labels on float64 near ties are a
        # rounding-order question, anything else is a bug
        nt = od.partition_near_ties(Q64, K64, cfg)
        kv_bad = np.flatnonzero(kv_label != part.kv_label)
        q_bad = np.flatnonzero(q_label != part.q_label)
        msg = (f"head {h}: {len(kv_bad)} K/V labels differ ({np.isin(kv_bad, nt['kv_near_ties']).sum()} on near "
               f"ties), {len(q_bad)} query labels differ ({np.isin(q_bad, nt['q_near_ties']).sum()} on near ties); "
               f"eigen-gap at r_k {nt['eigen_gap']:.3g}")
        log("    " + msg)
        raise AssertionError(msg)
    assert np.array_equal(host(b.kv_perm[h]), part.kv_perm)
    assert np.array_equal(host(b.q_perm[h]), part.q_perm)
    assert np.array_equal(host(b.kv_off[h]), part.kv_off)
    assert np.array_equal(host(b.q_off[h]), part.q_off)
    # ---- group-major copies are bytewise gathers
    for name, src, perm in (("Qp", Qh, part.q_perm), ("Kp", Kh, part.kv_perm), ("Vp", Vh, part.kv_perm)):
        got = getattr(b, name)[h].cpu()
        assert torch.equal(got, src[torch.from_numpy(perm)]), f"{name} is not the gathered input"
    # ---- centroids and distances (float64, different summation order)
    np.testing.assert_allclose(host(b.kv_centroid[h]), part.kv_centroid, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(host(b.q_centroid[h]), part.q_centroid, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(host(b.q_dist[h]), part.q_dist, rtol=1e-8, atol=1e-10)
    # ---- route: bit-exact
    rp = host(b.row_ptr[h]).astype(np.int64)
    ci = host(b.col_idx[h])[: rp[-1]].astype(np.int64)
    if not (np.array_equal(rp, ref.route.row_ptr) and np.array_equal(ci, ref.route.col_idx)):
        qs, ks = np.diff(part.q_off), np.diff(part.kv_off)
        budget = o.pair_budget(cfg.density, N, cfg.M) if cfg.top_k == 0 else None
        nt = od.route_near_ties(ref.route.P, qs, ks, budget=budget, k=cfg.top_k)
        msg = f"head {h}: route differs; score near ties (1e-12) of the oracle's route: {nt}"
        log("    " + msg)
        raise AssertionError(msg)
    assert int(b.routed_pairs[h].item()) == ref.route.routed_pairs
    diag["density"] = o.executed_pair_density(ref.route.routed_pairs, cfg.M, N)
    if not check_outputs:
        return diag
    tol = out_tol(cfg)
    # ---- measure everything first, assert afterwards (the log shows all of it)
    # the oracle may have computed only some rows (ref.rows, original indices);
    # the GPU's sparse output is group-major, so look those rows up by slot
    rows = np.asarray(ref.rows, dtype=np.int64)
    slot = np.empty(N, dtype=np.int64)
    slot[part.q_perm] = np.arange(N)
    Op = host(b.Op[h])[slot[rows]]
    want = ref.O_sparse
    diag["rows_checked"] = int(len(rows))
    diag["Op_maxabs"] = float(np.abs(Op - want).max())
    diag["Op_relF"] = float(np.linalg.norm(Op - want) / np.linalg.norm(want))
    diag["lse_maxabs"] = float(np.abs(host(b.lse[h])[slot[rows]] - ref.lse).max())
    M = cfg.M
    probes_equal = True
    if M > 0:
        probes_equal = np.array_equal(host(b.probe_idx[h]).astype(np.int64), ref.probe_idx)
        Opr = host(b.O_probe[h])
        diag["O_probe_maxabs"] = float(np.abs(Opr - ref.O_probe).max())
        diag["O_probe_relF"] = float(np.linalg.norm(Opr - ref.O_probe) / np.linalg.norm(ref.O_probe))
        # the fit's regressor: the GPU's sparse output at the probe rows
        xg = host(b.Op[h])[slot[ref.probe_idx]]
        diag["x_probe_maxabs"] = float(np.abs(xg - ref.X_probe).max())
        diag["rank_eff"] = int(b.rank_eff[h].item())
        diag["rank_eff_ref"] = ref.fit.rank_eff
        sg = ref.fit.sing
        r = ref.fit.rank_eff
        if sg is not None and 0 < r < len(sg):
            diag["sv_gap_at_rank"] = float((sg[r - 1] - sg[r]) / sg[0])
        diag["rbar_maxabs"] = float(np.abs(host(b.r_bar[h]) - ref.fit.r_bar).max())
        diag["xbar_maxabs"] = float(np.abs(host(b.x_bar[h]) - ref.fit.x_bar).max())
        rg = diag["rank_eff"]
        Bg, Vg = host(b.B_r[h])[:, :rg], host(b.V_r[h])[:, :rg]
        Wg, Wr = Bg @ Vg.T, ref.fit.B_r @ ref.fit.V_r.T
        diag["BV_maxabs"] = float(np.abs(Wg - Wr).max())
        diag["BV_norm_ref"] = float(np.abs(Wr).max())
        # the fit stage on its own: the oracle's fit of the GPU's own float32
        # regressors and residuals (exact in float64) against the GPU's fit
        xg64 = xg.astype(np.float64)
        fit_g = o.fit_residual(xg64, Opr.astype(np.float64) - xg64, host(b.probe_w[h]), cfg.rank, cfg.lam)
        Wf = fit_g.B_r @ fit_g.V_r.T
        diag["fit_stage_rank"] = fit_g.rank_eff
        diag["fit_stage_BV_maxabs"] = float(np.abs(Wg - Wf).max()) if rg == fit_g.rank_eff else float("inf")
        diag["fit_stage_BV_norm"] = float(np.abs(Wf).max()) if Wf.size else 0.0
        diag["fit_stage_mean_maxabs"] = float(max(np.abs(host(b.r_bar[h]) - fit_g.r_bar).max(),
                                                  np.abs(host(b.x_bar[h]) - fit_g.x_bar).max()))
    O_all = b.O[h].float().cpu().numpy()
    O = O_all[rows]
    diag["O_maxabs"] = float(np.abs(O - ref.O).max())
    diag["O_relF"] = float(np.linalg.norm(O - ref.O) / np.linalg.norm(ref.O))
    # the final output is stored in the input dtype: where |O| >= 8 half a bf16
    # ulp (2^-5 there) alone exceeds 2e-2, so only there the allowance is tol
    # plus half an ulp of the dtype; everywhere else max-abs <= tol
    big = float(np.abs(ref.O).max()) >= 8.0
    excess = np.abs(O - ref.O) - (tol + (half_ulp(cfg, np.abs(ref.O) + tol) if big else 0.0))
    diag["O_excess_over_tol"] = float(excess.max())
    log(f"    head {h} diagnostics: {diag}")
    # sparse output: element-wise tolerance, and a relative Frobenius bound
    # that a kernel regression far below the element-wise tolerance still breaks
    assert diag["Op_maxabs"] <= tol, f"Op max-abs {diag['Op_maxabs']:.3g} > {tol}"
    assert diag["Op_relF"] <= relf_tol(cfg), f"Op relative Frobenius error {diag['Op_relF']:.3g}"
    assert diag["lse_maxabs"] <= tol, f"lse max-abs {diag['lse_maxabs']:.3g} > {tol}"
    if M > 0:
        assert probes_equal, "probe set differs"
        np.testing.assert_allclose(host(b.probe_w[h]), ref.probe_w, rtol=1e-15, atol=0)
        assert diag["O_probe_maxabs"] <= tol
        assert diag["O_probe_relF"] <= relf_tol(cfg), f"O_probe relF {diag['O_probe_relF']:.3g}"
        # fit: the same numerical rank; the weighted means are convex
        # combinations (weights >= 0 summing to 1, equal on both sides) of
        # per-probe quantities, so their error is at most the largest error of
        # those quantities (plus float64 rounding)
        assert diag["rank_eff"] == diag["rank_eff_ref"], "fit rank differs"
        slack = 1e-12 + 1e-9 * float(np.abs(ref.X_probe).max())
        assert diag["xbar_maxabs"] <= diag["x_probe_maxabs"] + slack, "x_bar error exceeds the regressor error"
        assert diag["rbar_maxabs"] <= diag["x_probe_maxabs"] + diag["O_probe_maxabs"] + slack, \
            "r_bar error exceeds the residual error"
        # given the same float32 inputs the float64 fit agrees to rounding (the
        # GPU takes V_r from the residual Gram matrix, the oracle from an SVD)
        assert diag["fit_stage_rank"] == diag["rank_eff"], "fit rank differs on the same inputs"
        assert diag["fit_stage_mean_maxabs"] <= 1e-12, "fit means differ on the same inputs"
        assert diag["fit_stage_BV_maxabs"] <= 1e-9 * diag["fit_stage_BV_norm"] + 1e-12, \
            f"B_r V_r^T differs on the same inputs: {diag['fit_stage_BV_maxabs']:.3g}"
        # end to end the fit also carries the float32 / bf16 errors of its
        # inputs, amplified by up to 1 / (2 sqrt(lambda)); a loose bound that
        # still catches a wrong term, sign or transpose
        assert diag["BV_maxabs"] <= 5e-2 * max(diag["BV_norm_ref"], 1e-6) + 1e-9, \
            f"B_r V_r^T differs: {diag['BV_maxabs']:.3g} vs max {diag['BV_norm_ref']:.3g}"
    assert diag["O_excess_over_tol"] <= 0, f"O max-abs {diag['O_maxabs']:.3g} exceeds {tol}" + \
        (" + half an output ulp" if big else "")
    if M > 0:
        # probe rows carry their exact dense rows
        pr = ref.probe_idx
        assert np.all(np.abs(O_all[pr] - ref.O_probe) <= tol + half_ulp(cfg, np.abs(ref.O_probe) + tol))
    return diag


def full_parity(cfg, heads=None, check_outputs=True):
    Q, K, V = make_qkv(cfg)
    b, _ = run_gpu(cfg, Q, K, V)
    heads = range(cfg.H) if heads is None else heads
    Q64, K64, V64 = as_f64(Q), as_f64(K), as_f64(V)
    out = []
    for h in heads:
        ref = o.sparsepr_head(Q64[h], K64[h], V64[h], cfg)
        diag = compare_head(cfg, b, h, ref, Q[h], K[h], V[h], check_outputs)
        log(f"  {cfg.name} head {h}: {diag}")
        out.append(diag)
    return b, out
