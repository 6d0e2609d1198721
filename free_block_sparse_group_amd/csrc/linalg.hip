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

// Lane-group sum over TG lanes (TG <= 16, aligned) with DPP moves: each
// stage adds the value of a partner lane in the other half of the current
// span, so every lane of the group ends with the same bits (the same pairs
// are added, operands swapped).
template <int CTRL>
__device__ inline double dpp_move(double v) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(v), __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(v), __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

template <int TG>
__device__ inline void group_sum3(double& a, double& b, double& c) {
  static_assert(TG == 2 || TG == 4 || TG == 8 || TG == 16, "group of 2..16 lanes");
  if (TG >= 2) { a += dpp_move<0xB1>(a); b += dpp_move<0xB1>(b); c += dpp_move<0xB1>(c); }       // lanes ^1
  if (TG >= 4) { a += dpp_move<0x4E>(a); b += dpp_move<0x4E>(b); c += dpp_move<0x4E>(c); }       // lanes ^2
  if (TG >= 8) { a += dpp_move<0x141>(a); b += dpp_move<0x141>(b); c += dpp_move<0x141>(c); }    // mirror in 8
  if (TG >= 16) { a += dpp_move<0x140>(a); b += dpp_move<0x140>(b); c += dpp_move<0x140>(c); }   // mirror in 16
}

// TG threads share one rotation; each holds D/TG rows of both columns.
// Pairs are rotated when |w_p . w_q| > rot_tol ||w_p|| ||w_q||; the
// iteration ends after a sweep in which no pair had |w_p . w_q| > stop_tol
// ||w_p|| ||w_q||.  With stop_tol = rot_tol that is a sweep that rotated
// nothing; Jacobi converges quadratically, so stop_tol = sqrt(rot_tol) ends a
// sweep earlier with rotations of order rot_tol left undone.
template <int D, int TG>
__global__ __launch_bounds__(TG * D / 2) void k_sym_eig(const double* __restrict__ A, double* __restrict__ eigval,
                                                        double* __restrict__ eigvec, double rot_tol,
                                                        double stop_tol) {
  constexpr int NT = TG * D / 2;  // threads
  constexpr int LD = D + 2;       // padded column stride (doubles)
  constexpr int RPT = D / TG;     // rows per thread
  extern __shared__ double W[];   // W[p * LD + i]: column p, row i
  __shared__ double norms[D];
  __shared__ int order[D];
  __shared__ int big[2];   // a rotation larger than sqrt(rot_tol) in the sweep
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* Ah = A + (int64_t)h * D * D;
  for (int e = tid; e < D * D; e += NT) W[(e / D) * LD + (e % D)] = Ah[e];  // symmetric: row p = column p
  const int k = tid / TG, j = tid % TG, m = D - 1;
  // (tests squared, without a square root)
  const double tol2 = rot_tol * rot_tol, stop2 = stop_tol * stop_tol;
  if (tid == 0) { big[0] = 1; big[1] = 0; }
  for (int sweep = 0; sweep < 60; ++sweep) {
    __syncthreads();
    if (!big[sweep & 1]) break;             // the previous sweep made only small rotations
    if (tid == 0) big[(sweep + 1) & 1] = 0; // read again only after this sweep's barriers
    for (int r = 0; r < m; ++r) {
      int p, q;
      if (k == 0) { p = r; q = D - 1; }
      else { p = (r + k) % m; q = (r - k + m) % m; }
      double* wp = W + p * LD;
      double* wq = W + q * LD;
      double x[RPT], y[RPT];
#pragma unroll
      for (int s = 0; s < RPT; ++s) { x[s] = wp[j + s * TG]; y[s] = wq[j + s * TG]; }
      double al = 0.0, be = 0.0, ga = 0.0, al1 = 0.0, be1 = 0.0, ga1 = 0.0;
#pragma unroll
      for (int s = 0; s < RPT; s += 2) {
        al = fma(x[s], x[s], al);
        be = fma(y[s], y[s], be);
        ga = fma(x[s], y[s], ga);
        if (s + 1 < RPT) {
          al1 = fma(x[s + 1], x[s + 1], al1);
          be1 = fma(y[s + 1], y[s + 1], be1);
          ga1 = fma(x[s + 1], y[s + 1], ga1);
        }
      }
      al += al1;
      be += be1;
      ga += ga1;
      group_sum3<TG>(al, be, ga);
      if (ga * ga > tol2 * (al * be)) {
        // rotation that zeroes the pair's dot product: with g = 2 ga and
        // h = be - al, tan(theta) = sign(h) g / (|h| + sqrt(h^2 + g^2)); written
        // as c = u / sqrt(2 r u), s = sign(h) g / sqrt(2 r u) with
        // r = sqrt(h^2 + g^2), u = |h| + r (one square root, one reciprocal root)
        const double g = 2.0 * ga, hh = be - al;
        const double rr = sqrt(fma(hh, hh, g * g));
        const double u = fabs(hh) + rr;
        const double w = rsqrt(2.0 * rr * u);
        const double c = u * w, s = copysign(1.0, hh) * g * w;
#pragma unroll
        for (int t = 0; t < RPT; ++t) {
          wp[j + t * TG] = c * x[t] - s * y[t];
          wq[j + t * TG] = s * x[t] + c * y[t];
        }
        if (j == 0 && ga * ga > stop2 * (al * be)) big[(sweep + 1) & 1] = 1;
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

void launch_sym_eig(const double* A, int H, int d, double* eigval, double* eigvec, hipStream_t st, double rot_tol,
                    double stop_tol) {
  // default: the rounding level of a d-term dot product, run until a sweep rotates nothing
  if (rot_tol <= 0.0) rot_tol = (double)d * 2.220446049250313e-16;
  if (stop_tol <= 0.0) stop_tol = rot_tol;
  if (d == 128) {
    const size_t lds = sizeof(double) * 128 * (128 + 2);
    hipLaunchKernelGGL((k_sym_eig<128, 16>), dim3(H), dim3(16 * 64), lds, st, A, eigval, eigvec, rot_tol, stop_tol);
  } else {
    const size_t lds = sizeof(double) * 64 * (64 + 2);
    hipLaunchKernelGGL((k_sym_eig<64, 16>), dim3(H), dim3(16 * 32), lds, st, A, eigval, eigvec, rot_tol, stop_tol);
  }
}

void init_linalg_attributes() {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sym_eig<128, 16>), hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)(sizeof(double) * 128 * (128 + 2)));
}

}  // namespace spr
