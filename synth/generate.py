"""Seeded synthetic Q/K/V for the SparsePR attention call.

The tensors stand in for the attention inputs of video diffusion transformers
and video world models (arXiv:2608.18484, paperlayer.ai summary, section 5):
tokens are latent video positions ordered t = (f * lat_h + y) * lat_w + x,
with spatially smooth, temporally correlated activations.  Nothing here
computes any step of the method; the oracle and the GPU path both consume
exactly the tensors returned by `make_qkv`.

Seeds: every draw uses numpy's PCG64 via
``np.random.default_rng([cfg_id, head, stream])``; streams 0/1/2 are Q/K/V
noise, 3 the centres shared by Q and K, 4 the V centres, 5 the cluster
membership.
"""
import numpy as np
import torch

from .configs import SparsePRConfig

_Q, _K, _V, _QK_CENTRES, _V_CENTRES, _MEMBERS = range(6)


def _rng(cfg: SparsePRConfig, head: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cfg.cfg_id, head, stream])


def _smooth_fields(rng, frames, lat_h, lat_w, d, sigma=2.0):
    """White noise per (frame, channel), blurred by a periodic Gaussian of std
    `sigma` tokens (product of the 2-D FFT with the Gaussian's transfer
    function), then standardised per (frame, channel).  -> [frames, lat_h*lat_w, d]"""
    x = rng.standard_normal((frames, d, lat_h, lat_w), dtype=np.float32)
    fy = np.fft.fftfreq(lat_h)[:, None]
    fx = np.fft.rfftfreq(lat_w)[None, :]
    transfer = np.exp(-2.0 * np.pi ** 2 * sigma ** 2 * (fy ** 2 + fx ** 2)).astype(np.float32)
    xf = np.fft.rfft2(x, axes=(-2, -1)) * transfer
    x = np.fft.irfft2(xf, s=(lat_h, lat_w), axes=(-2, -1)).astype(np.float32)
    x -= x.mean(axis=(-2, -1), keepdims=True)
    x /= x.std(axis=(-2, -1), keepdims=True) + 1e-12
    return np.ascontiguousarray(x.reshape(frames, d, lat_h * lat_w).transpose(0, 2, 1))


def _zipf_sizes(N, n_clusters=256, s=1.1):
    """Largest-remainder integer sizes proportional to c^-s, c = 1..n_clusters, summing to N."""
    w = np.arange(1, n_clusters + 1, dtype=np.float64) ** (-s)
    share = N * w / w.sum()
    base = np.floor(share).astype(np.int64)
    left = N - int(base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:left]] += 1
    return base


def _one_tensor(cfg: SparsePRConfig, head: int, stream: int) -> np.ndarray:
    F, Hh, Ww, d, N = cfg.frames, cfg.lat_h, cfg.lat_w, cfg.d, cfg.N
    assert F * Hh * Ww == N, "frames*lat_h*lat_w must equal N"
    rng = _rng(cfg, head, stream)
    if cfg.generator == "clusters":
        # iid N(0,1) rows plus 8 planted Gaussian clusters; Q and K share centres
        members = _rng(cfg, head, _MEMBERS).integers(0, 8, size=N)
        centres = _rng(cfg, head, _V_CENTRES if stream == _V else _QK_CENTRES).standard_normal((8, d))
        x = centres[members] + rng.standard_normal((N, d))
        return x.astype(np.float64)
    if cfg.generator == "smooth":
        x = _smooth_fields(rng, F, Hh, Ww, d).reshape(N, d)
        x = x + 0.5 * rng.standard_normal((N, d), dtype=np.float32)
        return x
    if cfg.generator in ("ar1", "ar1_zipf"):
        e = _smooth_fields(rng, F, Hh, Ww, d)          # innovations, unit variance
        x = np.empty_like(e)
        x[0] = e[0]
        c = np.float32(np.sqrt(1.0 - 0.81))
        for f in range(1, F):
            x[f] = np.float32(0.9) * x[f - 1] + c * e[f]
        x = x.reshape(N, d)
        if cfg.generator == "ar1_zipf":
            sizes = _zipf_sizes(N)
            perm = _rng(cfg, head, _MEMBERS).permutation(N)
            cluster = np.empty(N, dtype=np.int64)
            cluster[perm] = np.repeat(np.arange(len(sizes)), sizes)
            offs = _rng(cfg, head, _V_CENTRES if stream == _V else _QK_CENTRES).standard_normal(
                (len(sizes), d)).astype(np.float32)
            x = (x + offs[cluster]) * np.float32(1.0 / np.sqrt(2.0))
            if stream == _K:
                x[: 3 * Hh * Ww] *= np.float32(2.0)      # conditioning prefix: frames 0-2
        return x
    raise ValueError(cfg.generator)


def planted_clusters(cfg: SparsePRConfig, head: int) -> np.ndarray:
    """Planted cluster id of every token of one head (generator "ar1_zipf"):
    the Zipf-sized clusters whose offsets Q and K share, in the order
    make_qkv draws them.  Used to inject exact groups in place of a
    partition."""
    if cfg.generator != "ar1_zipf":
        raise ValueError(f"{cfg.name}: no planted clusters (generator {cfg.generator})")
    sizes = _zipf_sizes(cfg.N)
    perm = _rng(cfg, head, _MEMBERS).permutation(cfg.N)
    cluster = np.empty(cfg.N, dtype=np.int64)
    cluster[perm] = np.repeat(np.arange(len(sizes)), sizes)
    return cluster


def make_qkv(cfg: SparsePRConfig, heads=None):
    """Return (Q, K, V) as CPU torch tensors [H, N, d] in the config's dtype
    (bf16 via round-to-nearest-even from the generated values)."""
    heads = range(cfg.H) if heads is None else heads
    tdt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    out = []
    for stream in (_Q, _K, _V):
        t = torch.empty((len(heads), cfg.N, cfg.d), dtype=tdt)
        for i, h in enumerate(heads):
            t[i] = torch.from_numpy(np.ascontiguousarray(_one_tensor(cfg, h, stream))).to(tdt)
        out.append(t)
    return tuple(out)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a generated tensor to a float64 numpy array."""
    return t.to(torch.float64).numpy()
