"""Values far from unit scale: the fp16 copy of V takes a power-of-two scale per
head, so V multiplied by 2^22 (above the fp16 range at any fixed scale that
also serves unit values) or by 2^-20 (below its normal range) must give the
same attention as unit-scale V, multiplied back.  Scaling by a power of two is
exact in bf16, and the partition and routes do not depend on V, so the GPU's
sparse output and exact probe rows on the scaled V, divided by the factor,
are compared with the oracle's on the unscaled V at the usual tolerances; the
final output (whose ridge fit is not scale invariant) is compared with the
oracle run on the scaled V, relative to its size."""
import numpy as np
import pytest
import torch

from gpu_common import host, log, out_tol, relf_tol, run_gpu
from oracle import sparsepr_oracle as o
from synth import as_f64, get_config, make_qkv, with_overrides

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("log2_factor", [22, -20])
def test_v_far_from_unit_scale(log2_factor):
    cfg = with_overrides(get_config(2), H=2, N=2400, frames=3, lat_h=20, lat_w=40, G_k=20, G_q=24, M=40, rank=8,
                         density=0.3)
    Q, K, V = make_qkv(cfg)
    f = 2.0 ** log2_factor
    Vs = (V.float() * f).to(torch.bfloat16)
    assert torch.equal(Vs.float() / f, V.float()), "power-of-two scaling must be exact in bf16"
    log(f"[vrange] V x 2^{log2_factor}: max |V| {float(Vs.float().abs().max()):.3g}")
    b, _ = run_gpu(cfg, Q, K, Vs)
    Q64, K64, V64 = as_f64(Q), as_f64(K), as_f64(V)
    tol = out_tol(cfg)
    for h in range(cfg.H):
        ref = o.sparsepr_head(Q64[h], K64[h], V64[h], cfg)
        part = ref.part
        assert np.array_equal(host(b.q_label[h]), part.q_label) and np.array_equal(host(b.kv_label[h]), part.kv_label)
        slot = np.empty(cfg.N, dtype=np.int64)
        slot[part.q_perm] = np.arange(cfg.N)
        Op = host(b.Op[h])[slot] / f
        assert np.all(np.isfinite(Op))
        err = float(np.abs(Op - ref.O_sparse).max())
        relf = float(np.linalg.norm(Op - ref.O_sparse) / np.linalg.norm(ref.O_sparse))
        Opr = host(b.O_probe[h]) / f
        perr = float(np.abs(Opr - ref.O_probe).max())
        log(f"    head {h}: Op max-abs {err:.3g} relF {relf:.3g}, O_probe max-abs {perr:.3g}")
        assert err <= tol and relf <= relf_tol(cfg) and perr <= tol
        # the whole call on the scaled values, against the oracle on them
        refs = o.sparsepr_head(Q64[h], K64[h], as_f64(Vs)[h], cfg)
        O = b.O[h].float().cpu().numpy()
        assert np.all(np.isfinite(O))
        orel = float(np.linalg.norm(O - refs.O) / np.linalg.norm(refs.O))
        log(f"    head {h}: final O relF {orel:.3g} (scaled oracle)")
        assert orel <= 1e-2
