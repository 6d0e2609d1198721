"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (every head in one call).  The float64 oracle recomputes one
or two heads (the last one always, to catch head-stride mistakes): their partition, routes and probe sets must match bit
for bit, and outputs are compared on sampled rows (plus every probe row, which
the oracle always computes) with the same tolerances as the small cases."""
import numpy as np
import pytest

from gpu_common import compare_head, log, run_gpu
from oracle import sparsepr_oracle as o
from synth import as_f64, get_config, make_qkv

pytestmark = pytest.mark.gpu

SAMPLED_ROWS = 384


def sampled_rows(N, seed):
    rng = np.random.default_rng([seed, 7])
    rows = rng.choice(N, size=min(N, SAMPLED_ROWS - 2), replace=False)
    return np.unique(np.concatenate([rows, [0, N - 1]]))


# (workload, heads the oracle recomputes); the long-video head takes the oracle
# about half a minute, so it checks one head
CASES = [(2, (0, 23)), (3, (23,)), (4, (0, 39))]


@pytest.mark.parametrize("cfg_id,heads", CASES)
def test_full_size_sampled(cfg_id, heads):
    cfg = get_config(cfg_id)
    log(f"[fullsize] {cfg.name}: H={cfg.H} N={cfg.N} d={cfg.d} G={cfg.G_k}/{cfg.G_q} M={cfg.M}")
    Q, K, V = make_qkv(cfg)
    b, _ = run_gpu(cfg, Q, K, V)
    for h in heads:
        q, k, v = as_f64(Q[h]), as_f64(K[h]), as_f64(V[h])
        ref = o.sparsepr_head(q, k, v, cfg, rows=sampled_rows(cfg.N, cfg_id * 1000 + h))
        diag = compare_head(cfg, b, h, ref, Q[h], K[h], V[h])
        log(f"  {cfg.name} head {h}: {diag}")
