"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/sparsepr.h declares, sizes workspaces, and rejects bad
arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

from free_block_sparse_group_amd import binding as b
from synth import WORKLOADS, with_overrides

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsepr.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.LIB_PATH):
        pytest.fail("libsparsepr.so is not built (python -m free_block_sparse_group_amd.build)")
    return b.load_library()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsepr_[a-z_]+)\s*\(", src)))


def test_header_declarations_are_exported(lib):
    names = _declared()
    assert len(names) == 17
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libsparsepr.so"
    assert sorted(b.EXPORTED) == names


def test_version_and_empty_error(lib):
    assert b.version().startswith("sparsepr-gfx950")
    assert isinstance(b.last_error(), str)


@pytest.mark.parametrize("cfg", WORKLOADS, ids=lambda c: c.name)
def test_workspace_size_positive_and_monotone(lib, cfg):
    shape, pp, rp, fp = b.make_params(cfg)
    n = b.sparsepr_workspace_size(shape, pp, rp, fp)
    assert n > 0
    big = with_overrides(cfg, H=cfg.H * 2)
    assert b.sparsepr_workspace_size(*b.make_params(big)) > n


def _params(**kw):
    cfg = with_overrides(WORKLOADS[1], **kw)
    return b.make_params(cfg)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), b.SPARSEPR_EUNSUPPORTED),
    (dict(N=0), b.SPARSEPR_EINVAL),
    (dict(G_k=0), b.SPARSEPR_EINVAL),
    (dict(G_q=9000), b.SPARSEPR_EINVAL),
    (dict(G_k=2000), b.SPARSEPR_EUNSUPPORTED),
    (dict(M_s=0), b.SPARSEPR_EINVAL),
    (dict(r_k=65), b.SPARSEPR_EINVAL),
    (dict(iters_q=0), b.SPARSEPR_EINVAL),
    (dict(top_k=0, density=0.0), b.SPARSEPR_EINVAL),
    (dict(top_k=0, density=1.5), b.SPARSEPR_EINVAL),
    (dict(M=-1), b.SPARSEPR_EINVAL),
    (dict(M=5000), b.SPARSEPR_EUNSUPPORTED),
    (dict(rank=65), b.SPARSEPR_EINVAL),
    (dict(lam=-1.0), b.SPARSEPR_EINVAL),
    # no ridge term with M <= d: the centred fit matrix is singular for any data
    (dict(lam=0.0, M=64), b.SPARSEPR_EINVAL),
    (dict(lam=0.0, M=10), b.SPARSEPR_EINVAL),
])
def test_workspace_size_rejects(lib, kw, code):
    shape, pp, rp, fp = _params(**kw)
    n = lib.sparsepr_workspace_size(ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(rp), ctypes.byref(fp))
    assert n == 0
    assert b.last_error() != ""


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def test_partition_rejects_null_and_small_workspace(lib):
    shape, pp, rp, fp = _params()
    args = [FAKE] * 3 + [FAKE] * 6 + [FAKE] * 3 + [FAKE] * 3
    rc = lib.sparsepr_partition(ctypes.byref(shape), ctypes.byref(pp), *([NULL] + args[1:]), FAKE, 1 << 40, NULL)
    assert rc == b.SPARSEPR_EINVAL and "'Q'" in b.last_error()
    rc = lib.sparsepr_partition(ctypes.byref(shape), ctypes.byref(pp), *args, FAKE, 16, NULL)
    assert rc == b.SPARSEPR_EWORKSPACE and "workspace too small" in b.last_error()
    bad = b.Shape(shape.H, shape.N, 80, shape.dtype, 0.0)
    rc = lib.sparsepr_partition(ctypes.byref(bad), ctypes.byref(pp), *args, FAKE, 1 << 40, NULL)
    assert rc == b.SPARSEPR_EUNSUPPORTED


def test_route_attend_fit_correct_dense_reject(lib):
    shape, pp, rp, fp = _params()
    S, P, R, F = (ctypes.byref(x) for x in (shape, pp, rp, fp))
    assert lib.sparsepr_route(S, P, R, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, NULL) == \
        b.SPARSEPR_EINVAL
    assert lib.sparsepr_route(S, P, R, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, NULL) == \
        b.SPARSEPR_EWORKSPACE
    assert lib.sparsepr_attend(S, P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 1 << 40,
                               NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_probe_fit(S, P, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_correct(S, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 1 << 40,
                                NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_dense_attend(S, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 1 << 40, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_dense_attend(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_dense_attend(S, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, NULL) == b.SPARSEPR_EWORKSPACE
    assert lib.sparsepr_dense_workspace_size(S) >= 2 * shape.H * shape.N * shape.d


def test_lambda_zero_accepted_when_well_posed(lib):
    # M > d, or no subspace (rank 0), or no probes: nothing to solve singularly
    for kw in (dict(lam=0.0, M=65), dict(lam=0.0, M=10, rank=0), dict(lam=0.0, M=0)):
        shape, pp, rp, fp = _params(**kw)
        assert lib.sparsepr_workspace_size(ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(rp),
                                           ctypes.byref(fp)) > 0, kw


def test_probe_fit_with_no_probes_is_a_noop(lib):
    shape, pp, rp, fp = _params(M=0)
    F = ctypes.byref(fp)
    # M = 0: returns OK without touching any pointer or the GPU
    assert lib.sparsepr_probe_fit(ctypes.byref(shape), ctypes.byref(pp), F, *([NULL] * 16), NULL, 0, NULL) == \
        b.SPARSEPR_OK


def test_kernel_timing_hook_host_side(lib):
    # enabling, disabling and reading an empty record never touch the device
    assert lib.sparsepr_attend_kernel_timing(1) == b.SPARSEPR_OK
    ms, n = ctypes.c_double(-1.0), ctypes.c_int(-1)
    assert lib.sparsepr_attend_kernel_time(ctypes.byref(ms), ctypes.byref(n)) == b.SPARSEPR_OK
    assert (ms.value, n.value) == (0.0, 0)
    assert lib.sparsepr_attend_kernel_time(None, ctypes.byref(n)) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_attend_kernel_timing(0) == b.SPARSEPR_OK


def test_partition_mode_must_be_zero_or_one(lib):
    shape, pp, rp, fp = _params()
    for v, ok in ((0, True), (1, True), (2, False), (-1, False)):
        pp.semantic = v
        n = lib.sparsepr_workspace_size(ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(rp), ctypes.byref(fp))
        assert (n > 0) == ok
        if not ok:
            assert b"semantic" in lib.sparsepr_last_error()


def test_route_noalloc_rejects_before_any_launch(lib):
    # null pointers, and more cells than its static scratch holds (2^22)
    shape, pp, rp, fp = _params()
    S, P, R = (ctypes.byref(x) for x in (shape, pp, rp))
    assert lib.sparsepr_route_noalloc(S, P, R, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == b.SPARSEPR_EINVAL
    shape, pp, rp, fp = _params(H=5, N=8192, G_k=1024, G_q=1024)
    rc = lib.sparsepr_route_noalloc(ctypes.byref(shape), ctypes.byref(pp), ctypes.byref(rp), *([FAKE] * 7), NULL)
    assert rc == b.SPARSEPR_EWORKSPACE and "static scratch" in b.last_error()


def test_sym_eigen_rejects_bad_arguments(lib):
    # validated on the host before any launch
    assert lib.sparsepr_sym_eigen_workspace_size(0, 64) == 0
    assert lib.sparsepr_sym_eigen_workspace_size(2, 96) == 0
    n = lib.sparsepr_sym_eigen_workspace_size(2, 128)
    assert n >= 2 * 128 * 128 * 8
    assert lib.sparsepr_sym_eigen(2, 128, 0, FAKE, FAKE, FAKE, FAKE, n, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_sym_eigen(2, 128, 129, FAKE, FAKE, FAKE, FAKE, n, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_sym_eigen(2, 96, 4, FAKE, FAKE, FAKE, FAKE, n, NULL) == b.SPARSEPR_EUNSUPPORTED
    assert lib.sparsepr_sym_eigen(2, 128, 4, NULL, FAKE, FAKE, FAKE, n, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_sym_eigen(2, 128, 4, FAKE, FAKE, FAKE, FAKE, n - 1, NULL) == b.SPARSEPR_EWORKSPACE


def test_mfma_rate_probe_rejects_bad_arguments(lib):
    # validated on the host before any launch
    assert lib.sparsepr_mfma_rate_probe(0, 10, FAKE, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_mfma_rate_probe(4, 0, FAKE, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_mfma_rate_probe(4, 10, NULL, NULL) == b.SPARSEPR_EINVAL
    assert "sink" in b.last_error()


def test_tile_rate_probe_rejects_bad_arguments(lib):
    assert lib.sparsepr_tile_rate_probe(0, 10, FAKE, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_tile_rate_probe(4, 0, FAKE, NULL) == b.SPARSEPR_EINVAL
    assert lib.sparsepr_tile_rate_probe(4, 10, NULL, NULL) == b.SPARSEPR_EINVAL
    assert "sink" in b.last_error()
