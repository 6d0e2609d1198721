"""GPU parity at the edges of the parameter ranges, against the float64
oracle: fits with more than 32 directions (chunked paths of the fit solve and
the correction), the largest group counts (1024 query and key groups, many
of them empty), the largest probe count, a ridge parameter of zero, and fixed
top-k routing on bf16 inputs."""
import pytest

from gpu_common import full_parity, log
from synth import get_config, with_overrides

pytestmark = pytest.mark.gpu

CASES = {
    # rank 48 > 32: two 32-direction chunks in the solve and the correction
    "rank48_d64": with_overrides(get_config(1), H=1, N=4096, frames=4, lat_h=32, lat_w=32, G_k=16, G_q=16, M=256,
                                 rank=48),
    # rank 100 at d = 128: four chunks, the last one partial
    "rank100_d128": with_overrides(get_config(2), H=1, N=3000, frames=3, lat_h=25, lat_w=40, G_k=16, G_q=16,
                                   M=400, rank=100, density=0.3),
    # 1024 groups on each side for 8192 tokens: many empty groups, a million route cells
    "groups1024": with_overrides(get_config(1), H=1, N=8192, G_k=1024, G_q=1024, M=1500, rank=8, density=0.2),
    # the largest probe count
    "probes4096": with_overrides(get_config(1), H=1, N=8192, G_k=32, G_q=32, M=4096, rank=16),
    # no ridge term, well-posed fit (M >> d)
    "lambda0": with_overrides(get_config(1), H=1, N=4096, frames=4, lat_h=32, lat_w=32, G_k=16, G_q=16, M=256,
                              rank=16, lam=0.0),
    # fixed top-k routing on bf16 inputs at d = 128
    "topk4_bf16_d128": with_overrides(get_config(2), H=2, N=2400, frames=3, lat_h=20, lat_w=40, G_k=20, G_q=24,
                                      M=40, rank=8, top_k=4),
}


@pytest.mark.parametrize("name", list(CASES))
def test_edge(name):
    cfg = CASES[name]
    log(f"[edge] {name}: H={cfg.H} N={cfg.N} d={cfg.d} G={cfg.G_k}/{cfg.G_q} M={cfg.M} rank={cfg.rank} "
        f"lam={cfg.lam} top_k={cfg.top_k}")
    full_parity(cfg)


def test_empty_groups_from_duplicate_rows():
    # keys and queries take only a few distinct values, so several k-means
    # centres start on identical points; ties go to the lowest centre, the
    # others stay empty (and keep their position), and routing, query
    # coordinates and probe allocation must skip the empty groups
    import numpy as np
    import torch
    from gpu_common import compare_head, run_gpu
    from oracle import sparsepr_oracle as o
    from synth import as_f64
    cfg = with_overrides(get_config(1), H=2, N=640, frames=1, lat_h=20, lat_w=32, G_k=12, G_q=10, M=24, rank=4,
                         M_s=64, density=0.4)
    rng = np.random.default_rng([99, 1])
    shape = (cfg.H, cfg.N, cfg.d)
    base_k = rng.standard_normal((cfg.H, 5, cfg.d))
    base_q = rng.standard_normal((cfg.H, 4, cfg.d))
    pick_k = rng.integers(0, 5, size=(cfg.H, cfg.N))
    pick_q = rng.integers(0, 4, size=(cfg.H, cfg.N))
    K = np.take_along_axis(base_k, pick_k[..., None], axis=1)
    Q = np.take_along_axis(base_q, pick_q[..., None], axis=1)
    V = rng.standard_normal(shape)
    Qt, Kt, Vt = (torch.from_numpy(x).to(torch.bfloat16) for x in (Q, K, V))
    log("[edge] duplicate rows: empty groups")
    b, _ = run_gpu(cfg, Qt, Kt, Vt)
    Q64, K64, V64 = as_f64(Qt), as_f64(Kt), as_f64(Vt)
    saw_empty = False
    for h in range(cfg.H):
        ref = o.sparsepr_head(Q64[h], K64[h], V64[h], cfg)
        saw_empty |= bool((np.diff(ref.part.kv_off) == 0).any() and (np.diff(ref.part.q_off) == 0).any())
        diag = compare_head(cfg, b, h, ref, Qt[h], Kt[h], Vt[h])
        log(f"  head {h}: {diag}")
    assert saw_empty, "the inputs were meant to leave some groups empty"
