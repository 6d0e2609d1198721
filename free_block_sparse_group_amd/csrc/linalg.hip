// Small dense float64 linear algebra, one workgroup per matrix: the leading
// eigenpairs of a symmetric matrix, for M_K (key-response coordinates,
// paperlayer.ai appendix B.1) and for the Gram matrix of the weighted,
// centred probe residuals (appendix A.3), whose eigenvectors are the right
// singular vectors of the residual matrix.
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

// A double moved between lanes by one DPP control (two 32-bit moves).  The
// sums below add, at each stage, the value of a partner lane in the other
// half of the current span, so every lane of a group ends with the same bits
// (the same pairs are added, operands swapped).
template <int CTRL>
__device__ inline double dpp_move(double v) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(v), __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(v), __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// ---------------------------------------------------------------- leading eigenpairs
// The leading nev eigenpairs of a symmetric D x D matrix (D = 64 or 128), one
// block of 256 threads per matrix, in four phases:
//  1. Householder tridiagonalisation Q^T A Q = T (A held whole in LDS; the
//     full symmetric trailing block is updated so that every matrix-vector
//     product reads LDS rows, conflict free); reflector k is kept in row k;
//  2. the nev largest eigenvalues of T by multisection on the Sturm count
//     (the number of negative pivots of the LDL^T factorisation of T - x I),
//     256 / nev threads per eigenvalue, to a relative width of a few eps;
//  3. each eigenvector of T from a twisted factorisation at its eigenvalue:
//     forward and backward pivots, the twist index with the smallest
//     |gamma_k|, then z_k = 1 and the two-sided recurrence (one thread per
//     eigenvector, 16 at a time, one LDS array each);
//  4. y = Q z by the reflectors in reverse order, 16 threads per vector in
//     registers (no barriers), then unit norm and the sign convention.
// Eigenvalues are accurate to about eps ||A||, eigenvectors to about
// eps ||A|| / gap.  The trace of A (the sum of all eigenvalues) is returned
// too.
constexpr int kEigChunk = 16;   // eigenvectors per phase-3/4 pass

// sum over a wave, the same bits in every lane (DPP within 16-lane rows, then
// lane swaps across rows and halves)
SPR_DEV double wave_sum_f64(double v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  {
    const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(v), __double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(v), __double2hiint(v), false, false);
    v = __hiloint2double(hi[0], lo[0]) + __hiloint2double(hi[1], lo[1]);
  }
  {
    const auto lo = __builtin_amdgcn_permlane32_swap(__double2loint(v), __double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(__double2hiint(v), __double2hiint(v), false, false);
    v = __hiloint2double(hi[0], lo[0]) + __hiloint2double(hi[1], lo[1]);
  }
  return v;
}

// sum over the 256 threads of the block in a fixed order; red[4] must not be
// in use by a pending reduction (callers alternate two buffers).  One barrier.
SPR_DEV double block_sum256(double v, double* red) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// number of eigenvalues of T (diagonal a, squared off-diagonal b2) below x
template <int D>
SPR_DEV int sturm_count(const double* a, const double* b2, double x, double pivmin) {
  double q = a[0] - x;
  if (fabs(q) < pivmin) q = -pivmin;
  int c = q < 0.0;
  for (int i = 1; i < D; ++i) {
    q = (a[i] - x) - b2[i - 1] / q;
    if (fabs(q) < pivmin) q = -pivmin;
    c += q < 0.0;
  }
  return c;
}

template <int D>
__global__ __launch_bounds__(256) void k_sym_eig_top(const double* __restrict__ A, int nev,
                                                     double* __restrict__ eigval, double* __restrict__ eigvec,
                                                     double* __restrict__ trace) {
  extern __shared__ double lds[];
  double* W = lds;                 // D x D, W[i * D + j]
  double* P = lds + D * D;         // kEigChunk x D phase-3 arrays
  __shared__ double ta[D], tb[D], tb2[D], tau[D], vk[D], wk[D], ev[D];
  __shared__ double red[2][4];
  __shared__ double sc[4];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* Ah = A + (int64_t)h * D * D;
  for (int e = tid; e < D * D; e += 256) W[e] = Ah[e];
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int i = 0; i < D; ++i) t += W[i * D + i];
    trace[h] = t;
  }
  // ---- 1. tridiagonalisation
  int rb = 0;
  for (int k = 0; k < D - 2; ++k) {
    const int m = D - k - 1;             // trailing size; x = W[k][k+1 .. D-1]
    const double* xr = W + k * D + k + 1;
    const double xj = tid < m ? xr[tid] : 0.0;
    const double x0 = xr[0];
    const double sig = block_sum256(tid >= 1 && tid < m ? xj * xj : 0.0, red[rb]);
    rb ^= 1;
    // reflector H = I - tau v v^T, v_0 = 1, H x = beta e_1
    double t = 0.0, beta = x0, scale = 0.0;
    if (sig > 0.0) {
      const double nrm = sqrt(fma(x0, x0, sig));
      beta = x0 >= 0.0 ? -nrm : nrm;
      t = (beta - x0) / beta;
      scale = 1.0 / (x0 - beta);
    }
    if (tid < m) vk[tid] = tid == 0 ? 1.0 : xj * scale;
    if (tid == 0) {
      ta[k] = W[k * D + k];
      tb[k] = beta;
      tau[k] = t;
    }
    __syncthreads();
    if (t == 0.0) {   // uniform: nothing to annihilate; the trailing block is unchanged
      if (tid >= 1 && tid < m) W[k * D + k + 1 + tid] = 0.0;
      continue;
    }
    // p = tau A_sub v (rows j of the symmetric block read as columns), and p.v
    double pi = 0.0;
    if (tid < m) {
      const double* col = W + (k + 1) * D + k + 1 + tid;
      double a0 = 0.0, a1 = 0.0;
      int j = 0;
      for (; j + 1 < m; j += 2) {
        a0 = fma(col[j * D], vk[j], a0);
        a1 = fma(col[(j + 1) * D], vk[j + 1], a1);
      }
      if (j < m) a0 = fma(col[j * D], vk[j], a0);
      pi = t * (a0 + a1);
    }
    const double pv = block_sum256(tid < m ? pi * vk[tid] : 0.0, red[rb]);
    rb ^= 1;
    if (tid < m) wk[tid] = fma(-0.5 * t * pv, vk[tid], pi);
    // v (without its leading 1) is kept in row k for the back-transformation
    if (tid >= 1 && tid < m) W[k * D + k + 1 + tid] = vk[tid];
    __syncthreads();
    // A_sub -= v w^T + w v^T
    {
      const int j = tid & 127, r0 = tid >> 7;
      if (j < m) {
        const double vj = vk[j], wj = wk[j];
        for (int i = r0; i < m; i += 2) {
          double* e = W + (k + 1 + i) * D + k + 1 + j;
          *e = fma(-vk[i], wj, fma(-wk[i], vj, *e));
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    ta[D - 2] = W[(D - 2) * D + D - 2];
    ta[D - 1] = W[(D - 1) * D + D - 1];
    tb[D - 2] = W[(D - 1) * D + D - 2];
    tb[D - 1] = 0.0;
  }
  __syncthreads();
  if (tid < D) tb2[tid] = tb[tid] * tb[tid];
  // Gershgorin interval and the pivot floor
  double glo = 0.0, ghi = 0.0, bmax = 0.0;
  if (tid < D) {
    const double r = fabs(tb[tid]) + (tid > 0 ? fabs(tb[tid - 1]) : 0.0);
    glo = ta[tid] - r;
    ghi = ta[tid] + r;
    bmax = tb[tid] * tb[tid];
  }
  // (block min / max through the sum helper's buffer layout)
  {
    double lo = glo, hi = ghi, bm = bmax;
    for (int o = 32; o > 0; o >>= 1) {
      lo = fmin(lo, __shfl_xor(lo, o));
      hi = fmax(hi, __shfl_xor(hi, o));
      bm = fmax(bm, __shfl_xor(bm, o));
    }
    if ((tid & 63) == 0 && tid < D) { red[0][tid >> 6] = lo; red[1][tid >> 6] = hi; sc[tid >> 6] = bm; }
  }
  __syncthreads();
  double gl = red[0][0], gu = red[1][0], b2max = sc[0];
  for (int w = 1; w < D / 64; ++w) { gl = fmin(gl, red[0][w]); gu = fmax(gu, red[1][w]); b2max = fmax(b2max, sc[w]); }
  const double span = fmax(gu - gl, fmax(fabs(gl), fabs(gu)) * 1e-15) + 1e-300;
  gl -= 2.0 * span * 2.220446049250313e-16 + 1e-300;
  gu += 2.0 * span * 2.220446049250313e-16 + 1e-300;
  const double pivmin = 2.2250738585072014e-308 * fmax(1.0, b2max);
  // absolute width: bisection resolves eigenvalues to about eps ||T|| anyway
  const double atol = 2.0 * 2.220446049250313e-16 * fmax(fabs(gl), fabs(gu)) + pivmin;
  // ---- 2. multisection for the nev largest eigenvalues
  {
    int tpe = 1;
    while (tpe * 2 * nev <= 256 && tpe < 64) tpe *= 2;   // threads per eigenvalue (power of two)
    const int e = tid / tpe, s = tid % tpe;
    const bool act = e < nev;
    const int target = D - 1 - e;       // lo: count <= target, hi: count > target
    double lo = gl, hi = gu;
    for (int it = 0; it < 80; ++it) {
      const double x = lo + (double)(s + 1) * ((hi - lo) / (double)(tpe + 1));
      const int c = act ? sturm_count<D>(ta, tb2, x, pivmin) : 0;
      double nlo = c <= target ? x : lo, nhi = c > target ? x : hi;
      for (int o = 1; o < tpe; o <<= 1) {
        nlo = fmax(nlo, __shfl_xor(nlo, o));
        nhi = fmin(nhi, __shfl_xor(nhi, o));
      }
      lo = nlo;
      hi = nhi;
      const bool done = !(hi - lo > 4.0 * 2.220446049250313e-16 * fmax(fabs(lo), fabs(hi)) + atol);
      if (__all(done || !act)) break;
    }
    if (act && s == 0) ev[e] = 0.5 * (lo + hi);
  }
  __syncthreads();
  // ---- 3 + 4. eigenvectors, kEigChunk at a time
  for (int c0 = 0; c0 < nev; c0 += kEigChunk) {
    const int nc = min(kEigChunk, nev - c0);
    if (tid < nc) {
      const double lam = ev[c0 + tid];
      double* z = P + tid * D;
      // forward pivots D+ (kept in z)
      double dp = ta[0] - lam;
      if (fabs(dp) < pivmin) dp = -pivmin;
      z[0] = dp;
      for (int i = 0; i + 1 < D; ++i) {
        dp = (ta[i + 1] - lam) - tb2[i] / dp;
        if (fabs(dp) < pivmin) dp = -pivmin;
        z[i + 1] = dp;
      }
      // backward pivots D- and the twist index with the smallest |gamma|
      double dm = ta[D - 1] - lam;
      if (fabs(dm) < pivmin) dm = -pivmin;
      int kt = D - 1;
      double gbest = fabs(z[D - 1] + dm - (ta[D - 1] - lam));
      for (int i = D - 2; i >= 0; --i) {
        dm = (ta[i] - lam) - tb2[i] / dm;
        if (fabs(dm) < pivmin) dm = -pivmin;
        const double g = fabs(z[i] + dm - (ta[i] - lam));
        if (g < gbest) { gbest = g; kt = i; }
      }
      // U-_i = b_i / D-_{i+1} for i >= kt, stored in z[i + 1]
      dm = ta[D - 1] - lam;
      if (fabs(dm) < pivmin) dm = -pivmin;
      for (int i = D - 2; i >= kt; --i) {
        z[i + 1] = tb[i] / dm;
        dm = (ta[i] - lam) - tb2[i] / dm;
        if (fabs(dm) < pivmin) dm = -pivmin;
      }
      // z_kt = 1, then outwards
      double zc = 1.0;
      for (int i = kt - 1; i >= 0; --i) {
        zc = -(tb[i] / z[i]) * zc;
        z[i] = zc;
      }
      z[kt] = 1.0;
      zc = 1.0;
      for (int i = kt; i + 1 < D; ++i) {
        zc = -z[i + 1] * zc;
        z[i + 1] = zc;
      }
    }
    __syncthreads();
    // back-transformation: 16 threads per vector, rows r = q + 16 u
    constexpr int RU = D / 16;
    const int cv = tid >> 4, q = tid & 15;
    if (cv < nc) {
      double zr[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) zr[u] = P[cv * D + q + 16 * u];
      for (int k = D - 3; k >= 0; --k) {
        const double t = tau[k];
        if (t == 0.0) continue;
        // v_i: 1 at i = k+1, W[k][i] for i > k+1, 0 for i <= k
        double part = 0.0, vr[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
          const int i = q + 16 * u;
          vr[u] = i == k + 1 ? 1.0 : (i > k + 1 ? W[k * D + i] : 0.0);
          part = fma(vr[u], zr[u], part);
        }
        part += dpp_move<0xB1>(part);
        part += dpp_move<0x4E>(part);
        part += dpp_move<0x141>(part);
        part += dpp_move<0x140>(part);
        const double f = t * part;
#pragma unroll
        for (int u = 0; u < RU; ++u) zr[u] = fma(-f, vr[u], zr[u]);
      }
      // unit norm, largest-magnitude entry positive (lowest index on ties)
      double n2 = 0.0, amax = -1.0;
      int imax = 0;
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        n2 = fma(zr[u], zr[u], n2);
        const double a = fabs(zr[u]);
        if (a > amax) { amax = a; imax = q + 16 * u; }
      }
      n2 += dpp_move<0xB1>(n2);
      n2 += dpp_move<0x4E>(n2);
      n2 += dpp_move<0x141>(n2);
      n2 += dpp_move<0x140>(n2);
      for (int o = 1; o < 16; o <<= 1) {
        const double a2 = __shfl_xor(amax, o, 16);
        const int i2 = __shfl_xor(imax, o, 16);
        if (a2 > amax || (a2 == amax && i2 < imax)) { amax = a2; imax = i2; }
      }
      // the sign of the winning entry, from the thread that holds it
      double sgn = 0.0;
#pragma unroll
      for (int u = 0; u < RU; ++u)
        if (q + 16 * u == imax) sgn = zr[u] < 0.0 ? -1.0 : 1.0;
      for (int o = 1; o < 16; o <<= 1) sgn += __shfl_xor(sgn, o, 16);
      const double inv = n2 > 0.0 ? sgn / sqrt(n2) : 0.0;
      double* out = eigvec + ((int64_t)h * D + c0 + cv) * D;
#pragma unroll
      for (int u = 0; u < RU; ++u) out[q + 16 * u] = zr[u] * inv;
    }
    __syncthreads();
  }
  if (tid < nev) eigval[(int64_t)h * D + tid] = ev[tid];
}

void launch_sym_eig_top(const double* A, int H, int d, int nev, double* eigval, double* eigvec, double* trace,
                        hipStream_t st) {
  if (nev <= 0) nev = 1;
  if (nev > d) nev = d;
  const size_t lds = sizeof(double) * ((size_t)d * d + (size_t)kEigChunk * d);
  if (d == 128)
    hipLaunchKernelGGL((k_sym_eig_top<128>), dim3(H), dim3(256), lds, st, A, nev, eigval, eigvec, trace);
  else
    hipLaunchKernelGGL((k_sym_eig_top<64>), dim3(H), dim3(256), lds, st, A, nev, eigval, eigvec, trace);
}

void init_linalg_attributes() {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sym_eig_top<128>), hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)(sizeof(double) * (128 * 128 + kEigChunk * 128)));
}

}  // namespace spr
