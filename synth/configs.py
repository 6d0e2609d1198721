"""Workload configurations for the SparsePR attention call.

Five seeded synthetic workloads shaped like the activations of the video
diffusion transformers and world models that "Partition the Support,
Reconstruct the Residual" (arXiv:2608.18484) evaluates (paperlayer.ai
summary, section 5, "Models and benchmarks").  The models themselves are not
used; these tensors stand in for their attention inputs.

Hyperparameters that the pages leave open (their Table C.1 is named but not
enumerated, paperlayer.ai appendix C.2) are fixed here; each choice is listed
in the design notes with its reason.  This module holds no arithmetic of the
method: it is plain data shared by the oracle tests, the GPU tests and the
benchmark.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class SparsePRConfig:
    cfg_id: int            # 0..4, also the first word of every RNG seed
    name: str
    H: int                 # heads
    N: int                 # tokens (N_q = N_k, self-attention)
    d: int                 # head dim
    dtype: str             # "fp32" or "bf16"
    frames: int            # latent frames
    lat_h: int             # latent height (tokens)
    lat_w: int             # latent width (tokens)
    generator: str         # "clusters" | "smooth" | "ar1" | "ar1_zipf"
    G_k: int               # K/V groups
    G_q: int               # query groups
    M_s: int               # sampled queries for M_K
    r_k: int               # key-response coordinate rank
    iters_kv: int          # Lloyd iterations, K/V
    iters_q: int           # Lloyd iterations, queries
    eig_weight_power: float
    top_k: int             # >0: fixed top-k routing; 0: pair budget
    density: float         # executed-pair density target (incl. probes)
    M: int                 # probe rows
    rank: int              # probe-residual subspace rank r
    lam: float             # ridge lambda
    scale: float = 0.0     # 0 -> 1/sqrt(d)
    partition: str = "response"   # "response" (the method) or "semantic" (k-means on raw Q / K)
    warm: int = 0          # 1: k-means starts from the previous call's labels (kv_label / q_label on entry)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale > 0 else self.d ** -0.5


WORKLOADS = [
    SparsePRConfig(0, "tiny_fp32_planted8", 1, 1024, 64, "fp32", 1, 32, 32, "clusters",
                   G_k=8, G_q=8, M_s=64, r_k=16, iters_kv=8, iters_q=8, eig_weight_power=0.5,
                   top_k=2, density=1.0, M=32, rank=8, lam=1e-3),
    SparsePRConfig(1, "small_bf16_8x32x32", 4, 8192, 64, "bf16", 8, 32, 32, "smooth",
                   G_k=32, G_q=32, M_s=256, r_k=16, iters_kv=8, iters_q=8, eig_weight_power=0.5,
                   top_k=0, density=0.25, M=128, rank=16, lam=1e-3),
    SparsePRConfig(2, "videodit_bf16_13x45x56", 24, 32760, 128, "bf16", 13, 45, 56, "ar1",
                   G_k=128, G_q=128, M_s=256, r_k=16, iters_kv=8, iters_q=8, eig_weight_power=0.5,
                   top_k=0, density=0.25, M=256, rank=32, lam=1e-3),
    SparsePRConfig(3, "longvideo_bf16_33x45x80", 24, 118800, 128, "bf16", 33, 45, 80, "ar1",
                   G_k=256, G_q=256, M_s=256, r_k=16, iters_kv=8, iters_q=8, eig_weight_power=0.5,
                   top_k=0, density=0.22, M=512, rank=32, lam=1e-3),
    SparsePRConfig(4, "worldmodel_bf16_21x45x80_zipf", 40, 75600, 128, "bf16", 21, 45, 80, "ar1_zipf",
                   G_k=256, G_q=256, M_s=256, r_k=16, iters_kv=8, iters_q=8, eig_weight_power=0.5,
                   top_k=0, density=0.26, M=384, rank=32, lam=1e-3),
]


def get_config(i: int) -> SparsePRConfig:
    return WORKLOADS[i]


def with_overrides(cfg: SparsePRConfig, **kw) -> SparsePRConfig:
    """A copy of cfg with some fields replaced (shape overrides for small parity cases)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return SparsePRConfig(**d)
