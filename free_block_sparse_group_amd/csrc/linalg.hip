// Small dense float64 linear algebra, one workgroup per matrix.
//
// Symmetric positive semi-definite eigensolver by one-sided (Hestenes)
// Jacobi on the matrix itself: columns of W = A are rotated pairwise until
// mutually orthogonal, so that W = A V with orthonormal V; then column p of W
// equals lambda_p v_p, which gives lambda_p = ||w_p|| and v_p = w_p / lambda_p
// without accumulating V.  This keeps only one d x d matrix (128 KiB at
// d = 128) in LDS.  Rounds use the circle-method pairing, so the d/2
// rotations of a round touch disjoint columns and run in parallel.
// Used for M_K (key-response coordinates, paperlayer.ai appendix B.1) and for
// the Gram matrix of the weighted, centred probe residuals (appendix A.3).
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

// TG threads share one rotation; each holds D/TG rows of both columns.
template <int D, int TG>
__global__ __launch_bounds__(TG * D / 2) void k_sym_eig(const double* __restrict__ A, double* __restrict__ eigval,
                                                        double* __restrict__ eigvec) {
  constexpr int NT = TG * D / 2;  // threads
  constexpr int LD = D + 2;       // padded column stride (doubles)
  constexpr int RPT = D / TG;     // rows per thread
  extern __shared__ double W[];   // W[p * LD + i]: column p, row i
  __shared__ double norms[D];
  __shared__ int order[D];
  __shared__ int rotated[2];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* Ah = A + (int64_t)h * D * D;
  for (int e = tid; e < D * D; e += NT) W[(e / D) * LD + (e % D)] = Ah[e];  // symmetric: row p = column p
  const int k = tid / TG, j = tid % TG, m = D - 1;
  // columns count as orthogonal once |w_p . w_q| <= D eps ||w_p|| ||w_q||: the
  // rounding error of the dot product itself, so sweeps stop instead of
  // chasing noise
  const double tol = (double)D * 2.220446049250313e-16;
  if (tid == 0) { rotated[0] = 1; rotated[1] = 0; }
  for (int sweep = 0; sweep < 60; ++sweep) {
    __syncthreads();
    if (!rotated[sweep & 1]) break;              // the previous sweep rotated nothing
    if (tid == 0) rotated[(sweep + 1) & 1] = 0;  // read again only after this sweep's barriers
    for (int r = 0; r < m; ++r) {
      int p, q;
      if (k == 0) { p = r; q = D - 1; }
      else { p = (r + k) % m; q = (r - k + m) % m; }
      double* wp = W + p * LD;
      double* wq = W + q * LD;
      double x[RPT], y[RPT];
      double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll
      for (int s = 0; s < RPT; ++s) {
        x[s] = wp[j + s * TG];
        y[s] = wq[j + s * TG];
        al = fma(x[s], x[s], al);
        be = fma(y[s], y[s], be);
        ga = fma(x[s], y[s], ga);
      }
      // butterfly: every lane of the group ends with bit-identical sums (each
      // lane adds the same pairs, only with the operands swapped)
#pragma unroll
      for (int o = TG / 2; o > 0; o >>= 1) {
        al += __shfl_xor(al, o, TG);
        be += __shfl_xor(be, o, TG);
        ga += __shfl_xor(ga, o, TG);
      }
      if (ga != 0.0 && fabs(ga) > tol * sqrt(al * be)) {
        const double zeta = (be - al) / (2.0 * ga);
        const double t = copysign(1.0, zeta) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / sqrt(1.0 + t * t), s = c * t;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
          wp[j + u * TG] = c * x[u] - s * y[u];
          wq[j + u * TG] = s * x[u] + c * y[u];
        }
        if (j == 0) rotated[(sweep + 1) & 1] = 1;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    for (int i = 0; i < D; ++i) s = fma(W[tid * LD + i], W[tid * LD + i], s);
    norms[tid] = sqrt(s);
  }
  __syncthreads();
  if (tid < D) {
    const double v = norms[tid];
    int rank = 0;
    for (int q = 0; q < D; ++q) rank += (norms[q] > v) || (norms[q] == v && q < tid);
    order[rank] = tid;
  }
  __syncthreads();
  if (tid < D) {
    const int p = order[tid];
    const double lam = norms[p];
    eigval[(int64_t)h * D + tid] = lam;
    // sign: largest-magnitude entry positive (lowest index on ties)
    int arg = 0;
    double best = -1.0;
    for (int i = 0; i < D; ++i) {
      const double a = fabs(W[p * LD + i]);
      if (a > best) { best = a; arg = i; }
    }
    const double sgn = W[p * LD + arg] < 0.0 ? -1.0 : 1.0;
    const double inv = lam > 0.0 ? sgn / lam : 0.0;
    double* out = eigvec + ((int64_t)h * D + tid) * D;
    for (int i = 0; i < D; ++i) out[i] = W[p * LD + i] * inv;
  }
}

void launch_sym_eig(const double* A, int H, int d, double* eigval, double* eigvec, hipStream_t st) {
  if (d == 128) {
    const size_t lds = sizeof(double) * 128 * (128 + 2);
    hipLaunchKernelGGL((k_sym_eig<128, 4>), dim3(H), dim3(4 * 64), lds, st, A, eigval, eigvec);
  } else {
    const size_t lds = sizeof(double) * 64 * (64 + 2);
    hipLaunchKernelGGL((k_sym_eig<64, 8>), dim3(H), dim3(8 * 32), lds, st, A, eigval, eigvec);
  }
}

void init_linalg_attributes() {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sym_eig<128, 4>), hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)(sizeof(double) * 128 * (128 + 2)));
}

}  // namespace spr
