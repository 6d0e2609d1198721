// Small dense float64 linear algebra, one workgroup per matrix: the leading
// eigenpairs of a symmetric matrix, for M_K (key-response coordinates,
// paperlayer.ai appendix B.1) and for the Gram matrix of the weighted,
// centred probe residuals (appendix A.3), whose eigenvectors are the right
// singular vectors of the residual matrix.
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

// ---------------------------------------------------------------- leading eigenpairs
// The leading nev eigenpairs of a symmetric D x D matrix (D = 64 or 128), one
// block of 256 threads per matrix, in four phases:
//  1. Householder tridiagonalisation Q^T A Q = T with the matrix in LDS
//     (the full symmetric trailing block is updated, so every product reads
//     rows, conflict free); the matrix-vector product is split over
//     256 / D thread groups, the step's scalars and vectors are repeated
//     in every wave (wave sums; each wave's own LDS copy of v and w), so a
//     step needs two block barriers; reflector k is kept in row k for
//     phase 4;
//  2. the nev largest eigenvalues of T by multisection on the Sturm count
//     (the number of negative pivots of the LDL^T factorisation of T - x I),
//     256 / nev threads per eigenvalue, each evaluating two points, to a
//     width of a few eps (relative) plus 2 eps ||T||;
//  3. each eigenvector of T from a twisted factorisation at its eigenvalue:
//     forward and backward pivots, the twist index with the smallest
//     |gamma_k|, then z_k = 1 and the two-sided recurrence (one thread per
//     eigenvector, CH at a time, one LDS array each);
//  4. y = Q z by the reflectors in reverse order, 8, 16 or 32 threads per
//     vector (as many as the chunk of up to CH vectors allows; CH = 16 for
//     D = 128, 32 for D = 64) in registers with DPP sums (no barriers),
//     then unit norm and the sign convention.
// Eigenvalues are accurate to about eps ||A||, eigenvectors to about
// eps ||A|| / gap.  The trace of A (the sum of all eigenvalues) is returned
// too.  Reciprocals in the recurrences are v_rcp_f64 refined by two Newton
// steps (within an ulp or two of the quotient).
// eigenvectors per phase-3/4 pass (the LDS left beside the D x D matrix)
template <int D>
constexpr int eig_chunk() { return D == 128 ? 16 : 32; }

// sum over the 256 threads of the block in a fixed order; red[4] must not be
// in use by a pending reduction (callers alternate two buffers).  One barrier.
SPR_DEV double block_sum256(double v, double* red) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// sum over aligned groups of 8, 16 or 32 lanes (DPP and a row swap; same
// bits in each lane)
template <int TPV>
SPR_DEV double tpv_sum(double v) {
  static_assert(TPV == 8 || TPV == 16 || TPV == 32, "8, 16 or 32 lanes");
  v += dpp_move<0xB1>(v);                 // lanes ^1
  v += dpp_move<0x4E>(v);                 // lanes ^2
  v += dpp_move<0x141>(v);                // mirror within 8
  if (TPV >= 16) v += dpp_move<0x140>(v); // mirror within 16
  if (TPV == 32) {                        // the two 16-lane rows of each half
    const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(v), __double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(v), __double2hiint(v), false, false);
    v = __hiloint2double(hi[0], lo[0]) + __hiloint2double(hi[1], lo[1]);
  }
  return v;
}

// orders one wave's LDS writes before its later reads by other lanes of
// the same wave (a wave's LDS operations complete in issue order; this
// keeps the compiler from moving them)
SPR_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 1 / q to within an ulp or two: hardware estimate and two Newton steps
SPR_DEV double recip(double q) {
  double r = __builtin_amdgcn_rcp(q);
  double e = fma(-q, r, 1.0);
  r = fma(r, e, r);
  e = fma(-q, r, 1.0);
  return fma(r, e, r);
}

// number of eigenvalues of T (diagonal a, squared off-diagonal b2) below x0
// and below x1 (two independent recurrences for latency)
template <int D>
SPR_DEV void sturm_count2(const double* a, const double* b2, double x0, double x1, double pivmin, int& c0,
                          int& c1) {
  double q0 = a[0] - x0, q1 = a[0] - x1;
  if (fabs(q0) < pivmin) q0 = -pivmin;
  if (fabs(q1) < pivmin) q1 = -pivmin;
  int n0 = q0 < 0.0, n1 = q1 < 0.0;
#pragma unroll 8
  for (int i = 1; i < D; ++i) {
    const double ai = a[i], bi = b2[i - 1];
    q0 = fma(-bi, recip(q0), ai - x0);
    q1 = fma(-bi, recip(q1), ai - x1);
    if (fabs(q0) < pivmin) q0 = -pivmin;
    if (fabs(q1) < pivmin) q1 = -pivmin;
    n0 += q0 < 0.0;
    n1 += q1 < 0.0;
  }
  c0 = n0;
  c1 = n1;
}

// Phase 4 for vectors c0 .. c0 + nc - 1 (z in P, one row of D each): y = Q z
// by the reflectors in reverse order, TPV lanes per vector (rows q + TPV u)
// in registers with DPP sums, then unit norm and the sign convention.
template <int D, int TPV>
SPR_DEV void back_transform(const double* P, const double* W, const double* tau, int nc, int c0, int h,
                            double* __restrict__ eigvec) {
  constexpr int RV = D / TPV;
  const int tid = threadIdx.x, cv = tid / TPV, q = tid % TPV;
  if (cv >= nc) return;
  double zr[RV];
#pragma unroll
  for (int u = 0; u < RV; ++u) zr[u] = P[cv * D + q + TPV * u];
  for (int k = D - 3; k >= 0; --k) {
    const double t = tau[k];
    if (t == 0.0) continue;
    // v_i: 1 at i = k+1, row k of W for i > k+1, 0 for i <= k
    double part = 0.0, vr[RV];
#pragma unroll
    for (int u = 0; u < RV; ++u) {
      const int i = q + TPV * u;
      vr[u] = i == k + 1 ? 1.0 : (i > k + 1 ? W[k * D + i] : 0.0);
      part = fma(vr[u], zr[u], part);
    }
    part = tpv_sum<TPV>(part);
    const double f = t * part;
#pragma unroll
    for (int u = 0; u < RV; ++u) zr[u] = fma(-f, vr[u], zr[u]);
  }
  // unit norm, largest-magnitude entry positive (lowest index on ties)
  double n2 = 0.0, amax = -1.0;
  int imax = 0;
#pragma unroll
  for (int u = 0; u < RV; ++u) {
    n2 = fma(zr[u], zr[u], n2);
    const double av = fabs(zr[u]);
    if (av > amax) { amax = av; imax = q + TPV * u; }
  }
  n2 = tpv_sum<TPV>(n2);
  for (int o = 1; o < TPV; o <<= 1) {
    const double a2 = __shfl_xor(amax, o, TPV);
    const int i2 = __shfl_xor(imax, o, TPV);
    if (a2 > amax || (a2 == amax && i2 < imax)) { amax = a2; imax = i2; }
  }
  // the sign of the winning entry, from the thread that holds it
  double sgn = 0.0;
#pragma unroll
  for (int u = 0; u < RV; ++u)
    if (q + TPV * u == imax) sgn = zr[u] < 0.0 ? -1.0 : 1.0;
  for (int o = 1; o < TPV; o <<= 1) sgn += __shfl_xor(sgn, o, TPV);
  const double inv = n2 > 0.0 ? sgn / sqrt(n2) : 0.0;
  double* out = eigvec + ((int64_t)h * D + c0 + cv) * D;
#pragma unroll
  for (int u = 0; u < RV; ++u) out[q + TPV * u] = zr[u] * inv;
}

template <int D>
__global__ __launch_bounds__(256) void k_sym_eig_top(const double* __restrict__ A, int nev,
                                                     double* __restrict__ eigval, double* __restrict__ eigvec,
                                                     double* __restrict__ trace) {
  constexpr int CH = eig_chunk<D>();
  constexpr int NS = 256 / D;                 // thread groups splitting the product
  extern __shared__ double lds[];
  double* W = lds;                            // D x D, W[i * D + j]
  double* P = lds + D * D;                    // CH x D phase-3 arrays
  __shared__ double ta[D], tb[D], tb2[D], tau[D], ev[D];
  __shared__ double vbuf[4][D], wbuf[4][D];   // each wave's copy of v and w
  __shared__ double ps[NS][D];
  __shared__ double red[2][4];
  __shared__ double sc[4];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* Ah = A + (int64_t)h * D * D;
  for (int e = tid; e < D * D; e += 256) W[e] = Ah[e];
  __syncthreads();
  {
    const double tr = block_sum256(tid < D ? W[tid * D + tid] : 0.0, red[1]);
    if (tid == 0) trace[h] = tr;
  }
  // ---- 1. tridiagonalisation
  // Every wave computes the step's scalars and the vectors v, p, w in full
  // (lane l holds entries l + 64 c of the trailing block) from the same
  // values in the same lanes, so all waves hold identical copies, each in
  // its own LDS slot; only the matrix-vector partial sums and the updated
  // matrix cross waves, so a step needs two block barriers.
  constexpr int CPL = D / 64;
  const int ci = tid % D, cg = tid / D;       // product: output i = ci, j-range part cg
  const int wv = tid >> 6, ln = tid & 63;
  double* vw = vbuf[wv];
  double* ww = wbuf[wv];
  for (int k = 0; k < D - 2; ++k) {
    const int m = D - k - 1;                  // trailing size; x = W[k][k+1 .. D-1]
    const double* xr = W + k * D + k + 1;
    double x[CPL], s = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = ln + 64 * c;
      x[c] = j < m ? xr[j] : 0.0;
      if (j >= 1) s = fma(x[c], x[c], s);
    }
    const double sig = wave_sum_f64(s);
    const double x0 = __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(x[0])),
                                       __builtin_amdgcn_readfirstlane(__double2loint(x[0])));
    // reflector H = I - tau v v^T, v_0 = 1, H x = beta e_1
    double t = 0.0, beta = x0, scale = 0.0;
    if (sig > 0.0) {
      const double nrm = sqrt(fma(x0, x0, sig));
      beta = x0 >= 0.0 ? -nrm : nrm;
      t = (beta - x0) * recip(beta);
      scale = recip(x0 - beta);
    }
    if (t == 0.0) {   // uniform: nothing to annihilate; the trailing block is unchanged
      if (wv == 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int j = ln + 64 * c;
          if (j >= 1 && j < m) W[k * D + k + 1 + j] = 0.0;
        }
        if (ln == 0) { ta[k] = W[k * D + k]; tb[k] = beta; tau[k] = t; }
      }
      continue;
    }
    double v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = ln + 64 * c;
      v[c] = j == 0 ? 1.0 : x[c] * scale;     // 0 past the block
      if (j < m) vw[j] = v[c];
    }
    wave_lds_sync();
    // p partial sums: rows j of the symmetric block read as columns, the j
    // range split over NS groups, 8 products in flight
    {
      const int len = (m + NS - 1) / NS, j0 = cg * len, j1 = min(m, j0 + len);
      double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
      if (ci < m) {
        const double* colp = W + (k + 1) * D + k + 1 + ci;
        int j = j0;
        for (; j + 8 <= j1; j += 8) {
          double a8[8], v8[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) { a8[u] = colp[(j + u) * D]; v8[u] = vw[j + u]; }
          s0 = fma(a8[0], v8[0], s0); s1 = fma(a8[1], v8[1], s1);
          s2 = fma(a8[2], v8[2], s2); s3 = fma(a8[3], v8[3], s3);
          s0 = fma(a8[4], v8[4], s0); s1 = fma(a8[5], v8[5], s1);
          s2 = fma(a8[6], v8[6], s2); s3 = fma(a8[7], v8[7], s3);
        }
        for (; j < j1; ++j) s0 = fma(colp[j * D], vw[j], s0);
      }
      ps[cg][ci] = (s0 + s1) + (s2 + s3);
    }
    __syncthreads();
    // p = tau A_sub v and w = p - (tau / 2)(p . v) v, in every wave
    double p[CPL], pvs = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int i = ln + 64 * c;
      double a = 0.0;
      if (i < m) {
#pragma unroll
        for (int g = 0; g < NS; ++g) a += ps[g][i];
      }
      p[c] = a * t;
      pvs = fma(p[c], v[c], pvs);
    }
    const double pv = wave_sum_f64(pvs);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int i = ln + 64 * c;
      if (i < m) ww[i] = fma(-0.5 * t * pv, v[c], p[c]);
    }
    if (wv == 0) {
      // v (without its leading 1) is kept in row k for the back-transformation
      // (every wave has read row k before the barrier above)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int j = ln + 64 * c;
        if (j >= 1 && j < m) W[k * D + k + 1 + j] = v[c];
      }
      if (ln == 0) { ta[k] = W[k * D + k]; tb[k] = beta; tau[k] = t; }
    }
    wave_lds_sync();
    // A_sub -= v w^T + w v^T, column ci, rows cg + NS u, four at a time
    if (ci < m) {
      const double vj = vw[ci], wj = ww[ci];
      double* colp = W + (k + 1) * D + k + 1 + ci;
      int i = cg;
      for (; i + 3 * NS < m; i += 4 * NS) {
        double e4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e4[u] = colp[(i + u * NS) * D];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = i + u * NS;
          colp[r * D] = fma(-vw[r], wj, fma(-ww[r], vj, e4[u]));
        }
      }
      for (; i < m; i += NS) colp[i * D] = fma(-vw[i], wj, fma(-ww[i], vj, colp[i * D]));
    }
    __syncthreads();
  }
  __syncthreads();
  if (tid == 0) {
    ta[D - 2] = W[(D - 2) * D + D - 2];
    ta[D - 1] = W[(D - 1) * D + D - 1];
    tb[D - 2] = W[(D - 1) * D + D - 2];
    tb[D - 1] = 0.0;
  }
  __syncthreads();
  if (tid < D) tb2[tid] = tb[tid] * tb[tid];
  // Gershgorin interval and the pivot floor
  {
    double lo = 0.0, hi = 0.0, bm = 0.0;
    if (tid < D) {
      const double r = fabs(tb[tid]) + (tid > 0 ? fabs(tb[tid - 1]) : 0.0);
      lo = ta[tid] - r;
      hi = ta[tid] + r;
      bm = tb[tid] * tb[tid];
    }
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
    while (tpe * 2 * nev <= 256 && tpe < 64) tpe *= 2;   // threads per eigenvalue: the power of two with tpe nev <= 256
    const int e = tid / tpe, s = tid % tpe;
    const bool act = e < nev;
    const int target = D - 1 - e;       // lo: count <= target, hi: count > target
    const int np = 2 * tpe;             // points per iteration
    double lo = gl, hi = gu;
    for (int it = 0; it < 80; ++it) {
      const double step = (hi - lo) / (double)(np + 1);
      const double x0 = lo + (double)(2 * s + 1) * step, x1 = lo + (double)(2 * s + 2) * step;
      int c0 = 0, c1 = 0;
      if (act) sturm_count2<D>(ta, tb2, x0, x1, pivmin, c0, c1);
      double nlo = c1 <= target ? x1 : (c0 <= target ? x0 : lo);
      double nhi = c0 > target ? x0 : (c1 > target ? x1 : hi);
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
  // ---- 3 + 4. eigenvectors, CH at a time
  for (int c0 = 0; c0 < nev; c0 += CH) {
    const int nc = min(CH, nev - c0);
    if (tid < nc) {
      const double lam = ev[c0 + tid];
      double* z = P + tid * D;
      // forward pivots D+ (kept in z)
      double dp = ta[0] - lam;
      if (fabs(dp) < pivmin) dp = -pivmin;
      z[0] = dp;
#pragma unroll 8
      for (int i = 0; i + 1 < D; ++i) {
        dp = fma(-tb2[i], recip(dp), ta[i + 1] - lam);
        if (fabs(dp) < pivmin) dp = -pivmin;
        z[i + 1] = dp;
      }
      // backward pivots D- and the twist index with the smallest |gamma|
      double dm = ta[D - 1] - lam;
      if (fabs(dm) < pivmin) dm = -pivmin;
      int kt = D - 1;
      double gbest = fabs(z[D - 1] + dm - (ta[D - 1] - lam));
#pragma unroll 8
      for (int i = D - 2; i >= 0; --i) {
        dm = fma(-tb2[i], recip(dm), ta[i] - lam);
        if (fabs(dm) < pivmin) dm = -pivmin;
        const double g = fabs(z[i] + dm - (ta[i] - lam));
        if (g < gbest) { gbest = g; kt = i; }
      }
      // U-_i = b_i / D-_{i+1} for i >= kt, stored in z[i + 1]
      dm = ta[D - 1] - lam;
      if (fabs(dm) < pivmin) dm = -pivmin;
#pragma unroll 8
      for (int i = D - 2; i >= kt; --i) {
        const double rc = recip(dm);
        z[i + 1] = tb[i] * rc;
        dm = fma(-tb2[i], rc, ta[i] - lam);
        if (fabs(dm) < pivmin) dm = -pivmin;
      }
      // z_kt = 1, then outwards
      double zc = 1.0;
#pragma unroll 8
      for (int i = kt - 1; i >= 0; --i) {
        zc = -(tb[i] * recip(z[i])) * zc;
        z[i] = zc;
      }
      z[kt] = 1.0;
      zc = 1.0;
#pragma unroll 8
      for (int i = kt; i + 1 < D; ++i) {
        zc = -z[i + 1] * zc;
        z[i + 1] = zc;
      }
    }
    __syncthreads();
    // back-transformation: as many lanes per vector as the chunk allows
    if (nc * 32 <= 256) back_transform<D, 32>(P, W, tau, nc, c0, h, eigvec);
    else if (nc * 16 <= 256) back_transform<D, 16>(P, W, tau, nc, c0, h, eigvec);
    else back_transform<D, 8>(P, W, tau, nc, c0, h, eigvec);
    __syncthreads();
  }
  if (tid < nev) eigval[(int64_t)h * D + tid] = ev[tid];
}

template <int D>
static size_t eig_top_lds() {
  return sizeof(double) * ((size_t)D * D + (size_t)eig_chunk<D>() * D);
}

void launch_sym_eig_top(const double* A, int H, int d, int nev, double* eigval, double* eigvec, double* trace,
                        hipStream_t st) {
  if (nev <= 0) nev = 1;
  if (nev > d) nev = d;
  if (d == 128)
    hipLaunchKernelGGL((k_sym_eig_top<128>), dim3(H), dim3(256), eig_top_lds<128>(), st, A, nev, eigval, eigvec,
                       trace);
  else
    hipLaunchKernelGGL((k_sym_eig_top<64>), dim3(H), dim3(256), eig_top_lds<64>(), st, A, nev, eigval, eigvec,
                       trace);
}

void init_linalg_attributes() {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sym_eig_top<128>), hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)eig_top_lds<128>());
}

}  // namespace spr
