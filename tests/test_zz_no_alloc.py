"""sparsepr_route_noalloc (scratch in a static device array, for callers that
cannot allocate) against sparsepr_route (scratch in the caller's workspace),
through the C ABI: two calls in a row, the second on a smaller input, each
bit-exact against the workspace entry point on the same stage-1 outputs."""
import ctypes

import pytest
import torch

import free_block_sparse_group_amd as fb
from free_block_sparse_group_amd import binding as bd
from gpu_common import log
from synth import get_config, make_qkv, with_overrides

pytestmark = pytest.mark.gpu


def _route_both(cfg):
    Q, K, V = make_qkv(cfg)
    Qd, Kd, Vd = (t.cuda() for t in (Q, K, V))
    b = fb.SparsePRBuffers(cfg)
    fb.stage_partition(b, Qd, Kd, Vd)
    fb.stage_route(b)
    H, Gq, Gk = cfg.H, cfg.G_q, cfg.G_k
    rp = torch.full((H, Gq + 1), -7, dtype=torch.int32, device="cuda")
    ci = torch.full((H, Gq * Gk), -7, dtype=torch.int32, device="cuda")
    pairs = torch.full((H,), -7, dtype=torch.int64, device="cuda")
    p = bd._p
    fb.sparsepr_route_noalloc(b.shape, b.pp, b.rp, p(b.kv_off), p(b.q_off), p(b.kv_centroid), p(b.q_centroid),
                              p(rp), p(ci), p(pairs), bd.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(rp, b.row_ptr), "row_ptr differs"
    assert torch.equal(pairs, b.routed_pairs), "routed_pairs differs"
    for h in range(H):
        n = int(b.row_ptr[h, -1].item())
        assert torch.equal(ci[h, :n], b.col_idx[h, :n]), f"col_idx of head {h} differs"
    return int(b.routed_pairs.sum().item())


def test_route_noalloc_matches_workspace_route_twice():
    big = with_overrides(get_config(2), H=3, N=6000, frames=3, lat_h=40, lat_w=50, G_k=128, G_q=96, M=64, rank=8)
    small = with_overrides(get_config(1), H=2, N=2048, frames=2, lat_h=32, lat_w=32, G_k=16, G_q=12, M=40,
                           rank=8)
    log(f"[noalloc] first call: H={big.H} N={big.N} G={big.G_k}/{big.G_q}")
    p1 = _route_both(big)
    log(f"[noalloc] second, smaller call: H={small.H} N={small.N} G={small.G_k}/{small.G_q}")
    p2 = _route_both(small)
    log(f"[noalloc] routed pairs {p1}, {p2}: both bit-exact")


def test_route_noalloc_rejects_oversize_on_device():
    cfg = with_overrides(get_config(1), H=5, N=8192, G_k=1024, G_q=1024)
    shape, pp, rp, _ = bd.make_params(cfg)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the call fails on the host first
    with pytest.raises(bd.SparsePRError) as e:
        fb.sparsepr_route_noalloc(shape, pp, rp, *([fake] * 7), bd.current_stream())
    assert e.value.code == bd.SPARSEPR_EWORKSPACE
