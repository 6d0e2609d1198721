"""SparsePR sparse attention for AMD Instinct MI355X (gfx950).

The compute path is libsparsepr.so (hand-written HIP kernels behind the C ABI
in include/sparsepr.h); this package is its ctypes binding.  Importing the
package does not load the library; the first call does, and raises if the
library has not been built.
"""
from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, SparsePRBuffers, SparsePRError, attend_kernel_time, attend_kernel_timing, dense_attention,
    load_library, make_params, run_sparsepr,
    sparsepr_attend, sparsepr_correct, sparsepr_dense_attend, sparsepr_dense_workspace_size, sparsepr_mfma_rate_probe,
    sparsepr_tile_rate_probe,
    sparsepr_partition, sparsepr_probe_fit,
    sparsepr_route, sparsepr_route_noalloc, sparsepr_sym_eigen, sparsepr_sym_eigen_workspace_size, sparsepr_workspace_size, stage_attend,
    stage_correct, stage_partition, stage_probe_fit, stage_route, sym_eigen, version,
)
