"""ctypes binding of libsparsepr.so (C ABI in include/sparsepr.h).

Argument marshalling only: every step of the SparsePR call runs in the HIP
library.  The functions below carry the C names and take device pointers as
Python ints (`tensor.data_ptr()`); `SparsePRBuffers` and `run_sparsepr` use
PyTorch only to allocate device memory and to pick the current stream.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparsepr.so")

SPARSEPR_OK, SPARSEPR_EINVAL, SPARSEPR_EWORKSPACE, SPARSEPR_EHIP, SPARSEPR_EUNSUPPORTED = 0, -1, -2, -3, -4
SPARSEPR_F32, SPARSEPR_BF16 = 0, 1

EXPORTED = ["sparsepr_workspace_size", "sparsepr_last_error", "sparsepr_version", "sparsepr_partition",
            "sparsepr_route", "sparsepr_attend", "sparsepr_probe_fit", "sparsepr_correct",
            "sparsepr_dense_attend", "sparsepr_dense_workspace_size", "sparsepr_attend_kernel_timing",
            "sparsepr_attend_kernel_time", "sparsepr_mfma_rate_probe", "sparsepr_tile_rate_probe",
            "sparsepr_sym_eigen_workspace_size",
            "sparsepr_sym_eigen", "sparsepr_route_noalloc"]


class Shape(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class PartitionParams(ctypes.Structure):
    _fields_ = [("G_k", ctypes.c_int32), ("G_q", ctypes.c_int32), ("M_s", ctypes.c_int32),
                ("r_k", ctypes.c_int32), ("iters_kv", ctypes.c_int32), ("iters_q", ctypes.c_int32),
                ("eig_weight_power", ctypes.c_double), ("semantic", ctypes.c_int32), ("warm", ctypes.c_int32)]


class RouteParams(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("density", ctypes.c_double), ("M", ctypes.c_int32)]


class FitParams(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int32), ("rank", ctypes.c_int32), ("lambda_", ctypes.c_double)]


class SparsePRError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (status {code})")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsparsepr.so; raises (never falls back) if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m free_block_sparse_group_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I32P = ctypes.c_void_p
    SP, PP, RP, FP = (ctypes.POINTER(Shape), ctypes.POINTER(PartitionParams), ctypes.POINTER(RouteParams),
                      ctypes.POINTER(FitParams))
    lib.sparsepr_workspace_size.restype = ctypes.c_size_t
    lib.sparsepr_workspace_size.argtypes = [SP, PP, RP, FP]
    lib.sparsepr_last_error.restype = ctypes.c_char_p
    lib.sparsepr_last_error.argtypes = []
    lib.sparsepr_version.restype = ctypes.c_char_p
    lib.sparsepr_version.argtypes = []
    lib.sparsepr_partition.restype = ctypes.c_int
    lib.sparsepr_partition.argtypes = [SP, PP, P, P, P] + [I32P] * 6 + [P, P, P] + [P, P, P] + \
        [P, ctypes.c_size_t, P]
    lib.sparsepr_route.restype = ctypes.c_int
    lib.sparsepr_route.argtypes = [SP, PP, RP, I32P, I32P, P, P, I32P, I32P, P, P, ctypes.c_size_t, P]
    lib.sparsepr_route_noalloc.restype = ctypes.c_int
    lib.sparsepr_route_noalloc.argtypes = [SP, PP, RP, I32P, I32P, P, P, I32P, I32P, P, P]
    lib.sparsepr_attend.restype = ctypes.c_int
    lib.sparsepr_attend.argtypes = [SP, PP, P, P, P, I32P, I32P, I32P, I32P, P, P, P, ctypes.c_size_t, P]
    lib.sparsepr_probe_fit.restype = ctypes.c_int
    lib.sparsepr_probe_fit.argtypes = [SP, PP, FP, P, P, P, I32P, I32P, I32P, P, P, I32P, P, P, P, P, P, P,
                                       I32P, P, ctypes.c_size_t, P]
    lib.sparsepr_correct.restype = ctypes.c_int
    lib.sparsepr_correct.argtypes = [SP, FP, P, I32P, I32P, P, P, P, P, P, I32P, P, P, ctypes.c_size_t, P]
    lib.sparsepr_dense_attend.restype = ctypes.c_int
    lib.sparsepr_dense_attend.argtypes = [SP, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.sparsepr_dense_workspace_size.restype = ctypes.c_size_t
    lib.sparsepr_dense_workspace_size.argtypes = [SP]
    lib.sparsepr_attend_kernel_timing.restype = ctypes.c_int
    lib.sparsepr_attend_kernel_timing.argtypes = [ctypes.c_int]
    lib.sparsepr_attend_kernel_time.restype = ctypes.c_int
    lib.sparsepr_attend_kernel_time.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    lib.sparsepr_mfma_rate_probe.restype = ctypes.c_int
    lib.sparsepr_mfma_rate_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P]
    lib.sparsepr_tile_rate_probe.restype = ctypes.c_int
    lib.sparsepr_tile_rate_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P]
    lib.sparsepr_sym_eigen_workspace_size.restype = ctypes.c_size_t
    lib.sparsepr_sym_eigen_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.sparsepr_sym_eigen.restype = ctypes.c_int
    lib.sparsepr_sym_eigen.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P, ctypes.c_size_t, P]
    _lib = lib
    return lib


def _check(rc):
    if rc != SPARSEPR_OK:
        raise SparsePRError(rc, load_library().sparsepr_last_error().decode())
    return rc


def last_error() -> str:
    return load_library().sparsepr_last_error().decode()


def version() -> str:
    return load_library().sparsepr_version().decode()


# ---- same-name wrappers (pointers as ints, structs by value object) --------

def sparsepr_workspace_size(shape, pp, rp, fp) -> int:
    n = load_library().sparsepr_workspace_size(ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(rp),
                                               ctypes.byref(fp))
    if n == 0:
        raise SparsePRError(SPARSEPR_EINVAL, last_error())
    return n


def sparsepr_partition(shape, pp, Q, K, V, kv_label, q_label, kv_perm, q_perm, kv_off, q_off, Qp, Kp, Vp,
                       kv_centroid, q_centroid, q_dist, ws, ws_bytes, stream):
    return _check(load_library().sparsepr_partition(
        ctypes.byref(shape), ctypes.byref(pp), Q, K, V, kv_label, q_label, kv_perm, q_perm, kv_off, q_off,
        Qp, Kp, Vp, kv_centroid, q_centroid, q_dist, ws, ws_bytes, stream))


def sparsepr_route(shape, pp, rp, kv_off, q_off, kv_centroid, q_centroid, row_ptr, col_idx, routed_pairs,
                   ws, ws_bytes, stream):
    return _check(load_library().sparsepr_route(
        ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(rp), kv_off, q_off, kv_centroid, q_centroid,
        row_ptr, col_idx, routed_pairs, ws, ws_bytes, stream))


def sparsepr_route_noalloc(shape, pp, rp, kv_off, q_off, kv_centroid, q_centroid, row_ptr, col_idx, routed_pairs,
                           stream):
    return _check(load_library().sparsepr_route_noalloc(
        ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(rp), kv_off, q_off, kv_centroid, q_centroid,
        row_ptr, col_idx, routed_pairs, stream))


def sparsepr_attend(shape, pp, Qp, Kp, Vp, q_off, kv_off, row_ptr, col_idx, Op, lse, ws, ws_bytes, stream):
    return _check(load_library().sparsepr_attend(
        ctypes.byref(shape), ctypes.byref(pp), Qp, Kp, Vp, q_off, kv_off, row_ptr, col_idx, Op, lse, ws,
        ws_bytes, stream))


def sparsepr_probe_fit(shape, pp, fp, Q, K, V, q_label, q_off, q_perm, q_dist, Op, probe_idx, probe_w, O_probe,
                       r_bar, x_bar, B_r, V_r, rank_eff, ws, ws_bytes, stream):
    return _check(load_library().sparsepr_probe_fit(
        ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(fp), Q, K, V, q_label, q_off, q_perm, q_dist, Op,
        probe_idx, probe_w, O_probe, r_bar, x_bar, B_r, V_r, rank_eff, ws, ws_bytes, stream))


def sparsepr_correct(shape, fp, Op, q_perm, probe_idx, O_probe, r_bar, x_bar, B_r, V_r, rank_eff, O, ws,
                     ws_bytes, stream):
    return _check(load_library().sparsepr_correct(
        ctypes.byref(shape), ctypes.byref(fp), Op, q_perm, probe_idx, O_probe, r_bar, x_bar, B_r, V_r, rank_eff,
        O, ws, ws_bytes, stream))


def sparsepr_dense_workspace_size(shape) -> int:
    n = load_library().sparsepr_dense_workspace_size(ctypes.byref(shape))
    if n == 0:
        raise SparsePRError(SPARSEPR_EINVAL, last_error())
    return n


def attend_kernel_timing(enable: bool):
    """Start (True) or stop (False) recording HIP events around the
    block-sparse attention kernel of every sparsepr_attend call."""
    return _check(load_library().sparsepr_attend_kernel_timing(1 if enable else 0))


def attend_kernel_time():
    """(summed kernel milliseconds, launches) of the recorded event pairs."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int(0)
    _check(load_library().sparsepr_attend_kernel_time(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def sparsepr_mfma_rate_probe(blocks, iters, sink, stream):
    """Launch the matrix-core rate probe (blocks x 256 threads, iters rounds
    of four bf16 32x32x16 MFMAs per wave); the caller times it."""
    return _check(load_library().sparsepr_mfma_rate_probe(blocks, iters, sink, stream))


def sparsepr_tile_rate_probe(blocks, iters, sink, stream):
    """Launch the tile-mix ceiling probe (blocks x 256 threads, iters tiles of
    the block-sparse kernel's d = 128 work per wave on register operands);
    the caller times it."""
    return _check(load_library().sparsepr_tile_rate_probe(blocks, iters, sink, stream))


def sparsepr_sym_eigen_workspace_size(H, d) -> int:
    n = load_library().sparsepr_sym_eigen_workspace_size(H, d)
    if n == 0:
        raise SparsePRError(SPARSEPR_EINVAL, last_error())
    return n


def sparsepr_sym_eigen(H, d, nev, A, eigval, eigvec, ws, ws_bytes, stream):
    return _check(load_library().sparsepr_sym_eigen(H, d, nev, A, eigval, eigvec, ws, ws_bytes, stream))


def sym_eigen(A, nev, stream=None):
    """Leading nev eigenpairs of the symmetric float64 device matrices A
    [H, d, d]: (eigval [H, nev], eigvec [H, nev, d]) as device tensors."""
    import torch
    H, d = A.shape[0], A.shape[1]
    lam = torch.empty(H, d, dtype=torch.float64, device=A.device)
    vec = torch.empty(H, d, d, dtype=torch.float64, device=A.device)
    n = sparsepr_sym_eigen_workspace_size(H, d)
    ws = torch.empty(n, dtype=torch.uint8, device=A.device)
    s = stream or current_stream()
    sparsepr_sym_eigen(H, d, nev, _p(A), _p(lam), _p(vec), _p(ws), n, s)
    return lam[:, :nev], vec[:, :nev]


def sparsepr_dense_attend(shape, Q, K, V, O, lse, ws, ws_bytes, stream):
    return _check(load_library().sparsepr_dense_attend(ctypes.byref(shape), Q, K, V, O, lse, ws, ws_bytes,
                                                       stream))


# ---- parameter structs from a workload description --------------------------

def make_params(cfg):
    """C structs for a workload (any object with the SparsePRConfig fields)."""
    shape = Shape(cfg.H, cfg.N, cfg.d, SPARSEPR_BF16 if cfg.dtype == "bf16" else SPARSEPR_F32, float(cfg.scale))
    semantic = 1 if getattr(cfg, "partition", "response") == "semantic" else 0
    pp = PartitionParams(cfg.G_k, cfg.G_q, cfg.M_s, cfg.r_k, cfg.iters_kv, cfg.iters_q, cfg.eig_weight_power,
                         semantic, int(getattr(cfg, "warm", 0)))
    rp = RouteParams(cfg.top_k, cfg.density, cfg.M)
    fp = FitParams(cfg.M, cfg.rank, cfg.lam)
    return shape, pp, rp, fp


class SparsePRBuffers:
    """Device buffers (PyTorch allocations) for one SparsePR call."""

    def __init__(self, cfg, device="cuda"):
        import torch
        self.cfg = cfg
        self.shape, self.pp, self.rp, self.fp = make_params(cfg)
        H, N, d, Gk, Gq, M = cfg.H, cfg.N, cfg.d, cfg.G_k, cfg.G_q, cfg.M
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        i32, f64, f32 = torch.int32, torch.float64, torch.float32
        e = dict(device=device)
        self.kv_label = torch.empty(H, N, dtype=i32, **e)
        self.q_label = torch.empty(H, N, dtype=i32, **e)
        self.kv_perm = torch.empty(H, N, dtype=i32, **e)
        self.q_perm = torch.empty(H, N, dtype=i32, **e)
        self.kv_off = torch.empty(H, Gk + 1, dtype=i32, **e)
        self.q_off = torch.empty(H, Gq + 1, dtype=i32, **e)
        self.Qp = torch.empty(H, N, d, dtype=dt, **e)
        self.Kp = torch.empty(H, N, d, dtype=dt, **e)
        self.Vp = torch.empty(H, N, d, dtype=dt, **e)
        self.kv_centroid = torch.empty(H, Gk, d, dtype=f64, **e)
        self.q_centroid = torch.empty(H, Gq, d, dtype=f64, **e)
        self.q_dist = torch.empty(H, N, dtype=f64, **e)
        self.row_ptr = torch.empty(H, Gq + 1, dtype=i32, **e)
        self.col_idx = torch.empty(H, Gq * Gk, dtype=i32, **e)
        self.routed_pairs = torch.empty(H, dtype=torch.int64, **e)
        self.Op = torch.empty(H, N, d, dtype=f32, **e)
        self.lse = torch.empty(H, N, dtype=f32, **e)
        Mb = max(M, 1)
        self.probe_idx = torch.empty(H, Mb, dtype=i32, **e)
        self.probe_w = torch.empty(H, Mb, dtype=f64, **e)
        self.O_probe = torch.empty(H, Mb, d, dtype=f32, **e)
        self.r_bar = torch.empty(H, d, dtype=f64, **e)
        self.x_bar = torch.empty(H, d, dtype=f64, **e)
        rb = max(cfg.rank, 1)
        self.B_r = torch.empty(H, d, rb, dtype=f64, **e)
        self.V_r = torch.empty(H, d, rb, dtype=f64, **e)
        self.rank_eff = torch.empty(H, dtype=i32, **e)
        self.O = torch.empty(H, N, d, dtype=dt, **e)
        self.ws_bytes = sparsepr_workspace_size(self.shape, self.pp, self.rp, self.fp)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, **e)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def current_stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def stage_partition(b: "SparsePRBuffers", Q, K, V, stream=None):
    s = stream or current_stream()
    return sparsepr_partition(b.shape, b.pp, _p(Q), _p(K), _p(V), _p(b.kv_label), _p(b.q_label), _p(b.kv_perm),
                              _p(b.q_perm), _p(b.kv_off), _p(b.q_off), _p(b.Qp), _p(b.Kp), _p(b.Vp),
                              _p(b.kv_centroid), _p(b.q_centroid), _p(b.q_dist), _p(b.ws), b.ws_bytes, s)


def stage_route(b, stream=None):
    s = stream or current_stream()
    return sparsepr_route(b.shape, b.pp, b.rp, _p(b.kv_off), _p(b.q_off), _p(b.kv_centroid), _p(b.q_centroid),
                          _p(b.row_ptr), _p(b.col_idx), _p(b.routed_pairs), _p(b.ws), b.ws_bytes, s)


def stage_attend(b, stream=None):
    s = stream or current_stream()
    return sparsepr_attend(b.shape, b.pp, _p(b.Qp), _p(b.Kp), _p(b.Vp), _p(b.q_off), _p(b.kv_off), _p(b.row_ptr),
                           _p(b.col_idx), _p(b.Op), _p(b.lse), _p(b.ws), b.ws_bytes, s)


def stage_probe_fit(b, Q, K, V, stream=None):
    s = stream or current_stream()
    return sparsepr_probe_fit(b.shape, b.pp, b.fp, _p(Q), _p(K), _p(V), _p(b.q_label), _p(b.q_off), _p(b.q_perm),
                              _p(b.q_dist), _p(b.Op), _p(b.probe_idx), _p(b.probe_w), _p(b.O_probe), _p(b.r_bar),
                              _p(b.x_bar), _p(b.B_r), _p(b.V_r), _p(b.rank_eff), _p(b.ws), b.ws_bytes, s)


def stage_correct(b, stream=None):
    s = stream or current_stream()
    return sparsepr_correct(b.shape, b.fp, _p(b.Op), _p(b.q_perm), _p(b.probe_idx), _p(b.O_probe), _p(b.r_bar),
                            _p(b.x_bar), _p(b.B_r), _p(b.V_r), _p(b.rank_eff), _p(b.O), _p(b.ws), b.ws_bytes, s)


def run_sparsepr(b: "SparsePRBuffers", Q, K, V, stream=None):
    """The five C-ABI calls in order on one stream (asynchronous)."""
    stage_partition(b, Q, K, V, stream)
    stage_route(b, stream)
    stage_attend(b, stream)
    stage_probe_fit(b, Q, K, V, stream)
    stage_correct(b, stream)
    return b.O


_dense_ws = {}


def dense_attention(cfg, Q, K, V, O, lse, stream=None, ws=None):
    """Dense attention from the same tile machinery; the scratch buffer is
    allocated once per (shape, device) unless one is passed."""
    import torch
    shape, _, _, _ = make_params(cfg)
    s = stream or current_stream()
    n = sparsepr_dense_workspace_size(shape)
    if ws is None:
        key = (cfg.H, cfg.N, cfg.d, cfg.dtype, str(Q.device))
        ws = _dense_ws.get(key)
        if ws is None or ws.numel() < n:
            ws = torch.empty(n, dtype=torch.uint8, device=Q.device)
            _dense_ws[key] = ws
    return sparsepr_dense_attend(shape, _p(Q), _p(K), _p(V), _p(O), _p(lse), _p(ws), n, s)
