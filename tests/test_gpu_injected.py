"""Block-sparse attention on injected groups: the planted Zipf clusters of
the world-model generator stand in for the partition (query and K/V groups
are the planted clusters), as in the kernel-only benchmark.  The HIP route
and attention are compared with the oracle's on the same layout: routes bit
for bit, the group-major sparse output within max-abs 2e-2 (bf16 inputs)."""
import numpy as np
import pytest
import torch

import free_block_sparse_group_amd as fb
from gpu_common import host, log, out_tol
from oracle import sparsepr_oracle as o
from synth import as_f64, get_config, make_qkv, planted_clusters, with_overrides

pytestmark = pytest.mark.gpu

# 256 planted clusters over 9000 tokens: groups of 4 to 1859 rows (ragged
# 128-row query tiles and 64-key tiles, many single-tile groups)
CFG = with_overrides(get_config(4), H=2, N=9000, frames=5, lat_h=30, lat_w=60, G_k=256, G_q=256, M=256,
                     rank=32, density=0.26)


def injected_partition(Q64, K64, labels, G):
    perm, off = o.stable_group_permutation(labels, G)
    kv_mu, _ = o.group_means(K64, labels, G)
    q_mu, _ = o.group_means(Q64, labels, G)
    return o.HeadPartition(labels, labels, perm, perm, off, off, kv_mu, q_mu, np.zeros(len(labels)))


def test_injected_planted_groups():
    cfg = CFG
    log(f"[injected] H={cfg.H} N={cfg.N} G={cfg.G_q} planted Zipf groups")
    Q, K, V = make_qkv(cfg)
    b = fb.SparsePRBuffers(cfg)
    parts = []
    for h in range(cfg.H):
        lab = planted_clusters(cfg, h)
        part = injected_partition(as_f64(Q[h]), as_f64(K[h]), lab, cfg.G_q)
        parts.append(part)
        perm = torch.from_numpy(part.q_perm)
        for t in (b.q_label, b.kv_label):
            t[h].copy_(torch.from_numpy(lab.astype(np.int32)))
        for t in (b.q_perm, b.kv_perm):
            t[h].copy_(perm.to(torch.int32))
        for t in (b.q_off, b.kv_off):
            t[h].copy_(torch.from_numpy(part.q_off.astype(np.int32)))
        b.Qp[h].copy_(Q[h][perm])
        b.Kp[h].copy_(K[h][perm])
        b.Vp[h].copy_(V[h][perm])
        b.kv_centroid[h].copy_(torch.from_numpy(part.kv_centroid))
        b.q_centroid[h].copy_(torch.from_numpy(part.q_centroid))
    fb.stage_route(b)
    fb.stage_attend(b)
    torch.cuda.synchronize()
    tol = out_tol(cfg)
    for h in range(cfg.H):
        part = parts[h]
        route = o.route_head(part, cfg, cfg.N)
        rp = host(b.row_ptr[h]).astype(np.int64)
        assert np.array_equal(rp, route.row_ptr), "row_ptr differs"
        assert np.array_equal(host(b.col_idx[h])[: rp[-1]].astype(np.int64), route.col_idx), "col_idx differs"
        assert int(b.routed_pairs[h].item()) == route.routed_pairs
        Q64, K64, V64 = as_f64(Q[h]), as_f64(K[h]), as_f64(V[h])
        O_ref, lse_ref = o.sparse_attention(Q64, K64, V64, part, route, cfg.softmax_scale)
        slot = np.empty(cfg.N, dtype=np.int64)
        slot[part.q_perm] = np.arange(cfg.N)
        Op = host(b.Op[h])[slot]
        err = float(np.abs(Op - O_ref).max())
        lerr = float(np.abs(host(b.lse[h])[slot] - lse_ref).max())
        sizes = np.diff(part.q_off)
        log(f"  head {h}: groups {sizes.min()}..{sizes.max()} rows, density "
            f"{route.routed_pairs / cfg.N ** 2:.4f}, Op max-abs {err:.3g}, lse max-abs {lerr:.3g}")
        assert err <= tol
        assert lerr <= 10 * tol
