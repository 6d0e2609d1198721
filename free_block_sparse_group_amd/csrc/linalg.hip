// Small dense float64 linear algebra, one workgroup per matrix: the leading
// eigenpairs of a symmetric matrix, for M_K (key-response coordinates,
// paperlayer.ai appendix B.1) and for the Gram matrix of the weighted,
// centred probe residuals (appendix A.3), whose eigenvectors are the right
// singular vectors of the residual matrix.
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

// ---------------------------------------------------------------- leading eigenpairs
// The leading nev eigenpairs of a symmetric D x D matrix (D = 64 or 128) in
// two launches:
//  1. k_sym_tridiag, one block of 256 threads per matrix: Householder
//     tridiagonalisation Q^T A Q = T with the matrix in LDS (the full
//     symmetric trailing block is updated, so every product reads rows,
//     conflict free); the matrix-vector product is split over 256 / D
//     thread groups, the step's scalars and vectors are repeated in every
//     wave (wave sums; each wave's own LDS copy of v and w), so a step needs
//     two block barriers; T, the reflector factors and the reflectors
//     (reflector k in row k) go to a scratch area;
//  2. k_sym_eigpair, one block of 256 threads per eigenpair:
//     a. the eigenvalue by multisection on the Sturm count (the number of
//        negative pivots of the LDL^T factorisation of T - x I), two points
//        per thread (513 subintervals per round), to a width of a few eps
//        (relative) plus 2 eps ||T||;
//     b. the eigenvector of T from a twisted factorisation at it: forward
//        and backward pivots (two waves at once), the twist index with the
//        smallest |gamma_k|, then z_k = 1 and the two sides as running
//        products of per-index factors;
//     c. y = Q z by the reflectors in reverse order, 32 lanes in registers
//        with DPP sums (each lane's entries of the next two reflectors
//        loaded ahead from the scratch area), then unit norm and the sign
//        convention.
//  3. k_sym_cluster, one block per matrix: eigenpairs that have another
//     eigenvalue within kClusterTol ||T|| (flagged by step 2 from two Sturm
//     counts) have their vectors of T orthonormalised chain by chain
//     (two Gram-Schmidt passes against the chain's earlier vectors; a vector
//     that was almost inside their span is replaced by inverse iteration
//     from a fixed pseudo-random start, re-orthogonalised every step), then
//     back-transformed; without flags the block returns at once.
// T is split into unreduced blocks where an off-diagonal is below
// split_tol ||T|| (a perturbation of the size of the reduction's own
// rounding): an eigenvalue's vector is computed on its own block (ties
// between blocks are dealt out by per-block Sturm counts), so exactly
// repeated eigenvalues, which an unreduced block cannot have, get vectors
// with disjoint supports.
// Eigenvalues are accurate to about eps ||A||, eigenvectors to about
// eps ||A|| / gap, and the computed vectors are orthonormal to working
// accuracy also inside clusters.  The trace of A (the sum of all eigenvalues)
// is returned too.  Reciprocals in the recurrences are v_rcp_f64 refined by
// two Newton steps (within an ulp or two of the quotient).

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

// Scratch of one matrix: T (diagonal, off-diagonal), the reflector factors,
// the reflectors (row k: entries k+2 .. D-1 of reflector k), then the
// cluster pass's inputs: the bound on ||T||, and per eigenpair e its
// eigenvalue, cluster flag, block [p, q] and vector of T.
template <int D>
struct EigScr {
  static constexpr size_t kA = 0, kB = D, kTau = 2 * D;
  static constexpr size_t kW = 3 * D;
  static constexpr size_t kNrm = kW + (size_t)D * D;   // one value (8 slots)
  static constexpr size_t kLam = kNrm + 8;
  static constexpr size_t kFlag = kLam + D;
  static constexpr size_t kBlk = kFlag + D;             // p, q per eigenpair
  static constexpr size_t kZ = kBlk + 2 * D;            // D x D
  static constexpr size_t kSize = kZ + (size_t)D * D;
};
template <int D>
constexpr size_t tridiag_scratch() { return EigScr<D>::kSize; }

// off-diagonals of T at most split_tol ||T|| are set to zero
template <int D>
constexpr double split_tol() { return 4.0 * D * 2.220446049250313e-16; }
// eigenvalues closer than this times ||T|| are treated as one cluster: past
// it the one-step twisted factorisation leaves vectors orthogonal to about
// eps / kClusterTol = 2e-11
constexpr double kClusterTol = 1e-5;

template <int D>
__global__ __launch_bounds__(256) void k_sym_tridiag(const double* __restrict__ A, double* __restrict__ scr,
                                                     double* __restrict__ trace) {
  constexpr int NS = 256 / D;                 // thread groups splitting the product
  extern __shared__ double lds[];
  double* W = lds;                            // D x D, W[i * D + j]
  __shared__ double ta[D], tb[D], tau[D];
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
      for (; i + 7 * NS < m; i += 8 * NS) {
        double e8[8], v8[8], w8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = i + u * NS;
          e8[u] = colp[r * D];
          v8[u] = vw[r];
          w8[u] = ww[r];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) colp[(i + u * NS) * D] = fma(-v8[u], wj, fma(-w8[u], vj, e8[u]));
      }
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
  // Gershgorin bound on ||T||; negligible off-diagonals split T
  const double nrm = block_max_f64<256>(
      tid < D ? fabs(ta[tid]) + fabs(tb[tid]) + (tid > 0 ? fabs(tb[tid - 1]) : 0.0) : 0.0, red[0]);
  // T, the factors and the reflectors to the scratch area
  double* sh = scr + (int64_t)h * tridiag_scratch<D>();
  if (tid < D) {
    sh[EigScr<D>::kA + tid] = ta[tid];
    sh[EigScr<D>::kB + tid] = fabs(tb[tid]) <= split_tol<D>() * nrm ? 0.0 : tb[tid];
    sh[EigScr<D>::kTau + tid] = tau[tid];
  }
  if (tid == 0) sh[EigScr<D>::kNrm] = nrm;
  for (int e = tid; e < D * D; e += 256) sh[EigScr<D>::kW + e] = W[e];
}

// One eigenpair per block: eigenvalue nev - 1 - blockIdx.x from the top ...
// y = Q z for one vector (z in LDS): the reflectors (rows of Wg, in global
// memory, entries k+2 .. D-1 of row k) in reverse order, 32 lanes of wave 0
// holding D / 32 entries each, the next two reflectors' entries loaded ahead;
// then unit norm and the sign convention (largest-magnitude entry positive,
// lowest index on ties).
template <int D>
SPR_DEV void back_transform1(const double* z, const double* __restrict__ Wg, const double* tau, double* out,
                             int q /* lane 0 .. 31 of a wave */) {
  constexpr int RV = D / 32;
  double zr[RV], w0[RV], w1[RV];
#pragma unroll
  for (int u = 0; u < RV; ++u) zr[u] = z[q + 32 * u];
  auto load = [&](int k, double (&w)[RV]) {
#pragma unroll
    for (int u = 0; u < RV; ++u) {
      const int i = q + 32 * u;
      w[u] = (k >= 0 && i > k + 1) ? Wg[k * D + i] : 0.0;
    }
  };
  load(D - 3, w0);
  load(D - 4, w1);
  for (int k = D - 3; k >= 0; --k) {
    double vr[RV];
#pragma unroll
    for (int u = 0; u < RV; ++u) {
      const int i = q + 32 * u;
      vr[u] = i == k + 1 ? 1.0 : w0[u];
      w0[u] = w1[u];
    }
    load(k - 2, w1);
    const double t = tau[k];
    if (t == 0.0) continue;
    double part = 0.0;
#pragma unroll
    for (int u = 0; u < RV; ++u) part = fma(vr[u], zr[u], part);
    part = tpv_sum<32>(part);
    const double f = t * part;
#pragma unroll
    for (int u = 0; u < RV; ++u) zr[u] = fma(-f, vr[u], zr[u]);
  }
  double n2 = 0.0, amax = -1.0;
  int imax = 0;
#pragma unroll
  for (int u = 0; u < RV; ++u) {
    n2 = fma(zr[u], zr[u], n2);
    const double av = fabs(zr[u]);
    if (av > amax) { amax = av; imax = q + 32 * u; }
  }
  n2 = tpv_sum<32>(n2);
  for (int o = 1; o < 32; o <<= 1) {
    const double a2 = __shfl_xor(amax, o, 32);
    const int i2 = __shfl_xor(imax, o, 32);
    if (a2 > amax || (a2 == amax && i2 < imax)) { amax = a2; imax = i2; }
  }
  double sgn = 0.0;
#pragma unroll
  for (int u = 0; u < RV; ++u)
    if (q + 32 * u == imax) sgn = zr[u] < 0.0 ? -1.0 : 1.0;
  for (int o = 1; o < 32; o <<= 1) sgn += __shfl_xor(sgn, o, 32);
  const double inv = n2 > 0.0 ? sgn / sqrt(n2) : 0.0;
#pragma unroll
  for (int u = 0; u < RV; ++u) out[q + 32 * u] = zr[u] * inv;
}

// One eigenpair per block: eigenvalue number blockIdx.x from the largest of
// matrix blockIdx.y, from the tridiagonal form and reflectors in scratch.
template <int D>
__global__ __launch_bounds__(256) void k_sym_eigpair(double* __restrict__ scr, double* __restrict__ eigval,
                                                     double* __restrict__ eigvec) {
  __shared__ double ta[D], tb[D], tb2[D], tau[D], z[D], dpv[D], dmv[D];
  __shared__ double red[2][4];
  __shared__ double sc[4];
  __shared__ int kts[4];
  __shared__ int bst[D], bcl[D], bch[D];   // per unreduced block: first index, counts below lo and hi
  __shared__ int s_pq[2], s_flag;
  const int e = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  double* sh = scr + (int64_t)h * tridiag_scratch<D>();
  if (tid < D) {
    ta[tid] = sh[EigScr<D>::kA + tid];
    tb[tid] = sh[EigScr<D>::kB + tid];
    tau[tid] = sh[EigScr<D>::kTau + tid];
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
  // ---- a. multisection for eigenvalue e (counted from the largest)
  const int target = D - 1 - e;         // lo: count <= target, hi: count > target
  double lam, lo = gl, hi = gu;
  {
    __shared__ double blo[4], bhi[4];
    constexpr int np = 512;             // points per round
    for (int it = 0; it < 80; ++it) {
      const double step = (hi - lo) / (double)(np + 1);
      const double x0 = lo + (double)(2 * tid + 1) * step, x1 = lo + (double)(2 * tid + 2) * step;
      int c0 = 0, c1 = 0;
      sturm_count2<D>(ta, tb2, x0, x1, pivmin, c0, c1);
      double nlo = c1 <= target ? x1 : (c0 <= target ? x0 : lo);
      double nhi = c0 > target ? x0 : (c1 > target ? x1 : hi);
      for (int o = 1; o < 64; o <<= 1) {
        nlo = fmax(nlo, __shfl_xor(nlo, o));
        nhi = fmin(nhi, __shfl_xor(nhi, o));
      }
      if ((tid & 63) == 0) { blo[tid >> 6] = nlo; bhi[tid >> 6] = nhi; }
      __syncthreads();
      lo = fmax(fmax(blo[0], blo[1]), fmax(blo[2], blo[3]));
      hi = fmin(fmin(bhi[0], bhi[1]), fmin(bhi[2], bhi[3]));
      __syncthreads();
      // uniform: every thread holds the same lo and hi
      if (!(hi - lo > 4.0 * 2.220446049250313e-16 * fmax(fabs(lo), fabs(hi)) + atol)) break;
    }
    lam = 0.5 * (lo + hi);
  }
  // ---- the unreduced block [p, q] the eigenvalue is taken from, and whether
  // another eigenvalue lies within kClusterTol ||T|| of it
  if (tid == 0) {
    // per-block numbers of eigenvalues below lo and below hi (the Sturm
    // recurrence restarts where T is split: a zero off-diagonal)
    int nb = 0, start = 0, cl = 0, chn = 0, tot_lo = 0;
    double q0 = ta[0] - lo, q1 = ta[0] - hi;
    for (int i = 0;; ++i) {
      if (fabs(q0) < pivmin) q0 = -pivmin;
      if (fabs(q1) < pivmin) q1 = -pivmin;
      cl += q0 < 0.0;
      chn += q1 < 0.0;
      if (i + 1 == D || tb2[i] == 0.0) {
        bst[nb] = start; bcl[nb] = cl; bch[nb] = chn; ++nb;
        tot_lo += cl;
        if (i + 1 == D) break;
        start = i + 1; cl = 0; chn = 0;
        q0 = ta[i + 1] - lo;
        q1 = ta[i + 1] - hi;
      } else {
        q0 = fma(-tb2[i], recip(q0), ta[i + 1] - lo);
        q1 = fma(-tb2[i], recip(q1), ta[i + 1] - hi);
      }
    }
    // eigenvalues in [lo, hi) are ranked block by block: the one of rank
    // target - tot_lo belongs to the block where the running count passes it
    const int r = target - tot_lo;
    int p = 0, q = D - 1, cum = 0;
    for (int k = 0; k < nb; ++k) {
      const int c = bch[k] - bcl[k];
      if (r >= cum && r < cum + c) {
        p = bst[k];
        q = k + 1 < nb ? bst[k + 1] - 1 : D - 1;
        break;
      }
      cum += c;
    }
    s_pq[0] = p;
    s_pq[1] = q;
  } else if (tid == 64) {
    const double tc = kClusterTol * sh[EigScr<D>::kNrm];
    int c0 = 0, c1 = 0;
    sturm_count2<D>(ta, tb2, lam - tc, lam + tc, pivmin, c0, c1);
    s_flag = c1 - c0 >= 2;
  }
  __syncthreads();
  const int p = s_pq[0], q = s_pq[1];
  // ---- b. eigenvector of T by a twisted factorisation on [p, q]: the
  // forward (D+) and backward (D-) pivots run at once in two waves; the twist
  // index is the one with the smallest |gamma_k| = |D+_k + D-_k - (a_k - lambda)|
  // (the largest index on ties); z_kt = 1 and the two sides follow as running
  // products of per-index factors; z is zero outside the block.
  if (tid == 0) {
    double dp = ta[p] - lam;
    if (fabs(dp) < pivmin) dp = -pivmin;
    dpv[p] = dp;
#pragma unroll 8
    for (int i = p; i < q; ++i) {
      dp = fma(-tb2[i], recip(dp), ta[i + 1] - lam);
      if (fabs(dp) < pivmin) dp = -pivmin;
      dpv[i + 1] = dp;
    }
  } else if (tid == 64) {
    double dm = ta[q] - lam;
    if (fabs(dm) < pivmin) dm = -pivmin;
    dmv[q] = dm;
#pragma unroll 8
    for (int i = q - 1; i >= p; --i) {
      dm = fma(-tb2[i], recip(dm), ta[i] - lam);
      if (fabs(dm) < pivmin) dm = -pivmin;
      dmv[i] = dm;
    }
  } else if (tid >= 128 && tid - 128 < D && (tid - 128 < p || tid - 128 > q)) {
    z[tid - 128] = 0.0;
  }
  __syncthreads();
  int kt;
  {
    double g = __builtin_inf();
    int gi = -1;
    if (tid >= p && tid <= q) { g = fabs(dpv[tid] + dmv[tid] - (ta[tid] - lam)); gi = tid; }
    for (int o = 1; o < 64; o <<= 1) {
      const double g2 = __shfl_xor(g, o);
      const int i2 = __shfl_xor(gi, o);
      if (g2 < g || (g2 == g && i2 > gi)) { g = g2; gi = i2; }
    }
    if ((tid & 63) == 0) { red[0][tid >> 6] = g; kts[tid >> 6] = gi; }
    __syncthreads();
    double gb = red[0][0];
    kt = kts[0];
    for (int w = 1; w < D / 64; ++w)
      if (red[0][w] < gb || (red[0][w] == gb && kts[w] > kt)) { gb = red[0][w]; kt = kts[w]; }
  }
  // factors: z_i = -(b_i / D+_i) z_{i+1} below kt, z_{i+1} = -(b_i / D-_{i+1}) z_i above
  if (tid >= p && tid <= q) {
    const int i = tid;
    if (i < kt) z[i] = -(tb[i] * recip(dpv[i]));
    else if (i + 1 <= q) dpv[i] = tb[i] * recip(dmv[i + 1]);   // U-_i (D+_i is no longer needed there)
  }
  __syncthreads();
  if (tid == 0) {
    double zc = 1.0;
    for (int i = kt - 1; i >= p; --i) {
      zc = z[i] * zc;
      z[i] = zc;
    }
  } else if (tid == 64) {
    double zc = 1.0;
    z[kt] = 1.0;
    for (int i = kt; i + 1 <= q; ++i) {
      zc = -dpv[i] * zc;
      z[i + 1] = zc;
    }
  }
  __syncthreads();
  // ---- c. back-transformation, unit norm, sign; the eigenvalue.  A member
  // of a cluster leaves its vector of T to the cluster pass instead.
  if (s_flag) {
    if (tid < D) sh[EigScr<D>::kZ + (size_t)e * D + tid] = z[tid];
    if (tid == 0) {
      sh[EigScr<D>::kLam + e] = lam;
      sh[EigScr<D>::kFlag + e] = 1.0;
      sh[EigScr<D>::kBlk + 2 * e] = (double)p;
      sh[EigScr<D>::kBlk + 2 * e + 1] = (double)q;
    }
  } else {
    if (tid == 0) sh[EigScr<D>::kFlag + e] = 0.0;
    if (tid < 32) back_transform1<D>(z, sh + EigScr<D>::kW, tau, eigvec + ((int64_t)h * D + e) * D, tid);
  }
  if (tid == 0) eigval[(int64_t)h * D + e] = lam;
}

// a fixed pseudo-random number in [-0.5, 0.5) for entry i of start vector e
SPR_DEV double start_entry(int i, int e) {
  uint32_t x = (uint32_t)i * 0x9E3779B1u ^ ((uint32_t)e + 0x7F4A7C15u) * 0x85EBCA77u;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  x *= 0x297A2D39u;
  x ^= x >> 15;
  return (double)(x >> 8) * 0x1p-24 - 0.5;
}

// out = (T[p..q] - lam I)^-1 rhs by an LDL^T factorisation whose pivots are
// kept at least `guard` away from zero (one thread; zero outside [p, q])
template <int D>
SPR_DEV void tridiag_solve(const double* ta, const double* tb, int p, int q, double lam, double guard,
                           const double* rhs, double* out, double* dd, double* ll) {
  for (int i = 0; i < p; ++i) out[i] = 0.0;
  for (int i = q + 1; i < D; ++i) out[i] = 0.0;
  double d = ta[p] - lam;
  if (fabs(d) < guard) d = d < 0.0 ? -guard : guard;
  dd[p] = d;
  double y = rhs[p];
  out[p] = y;
  for (int i = p; i < q; ++i) {
    const double l = tb[i] * recip(d);
    ll[i] = l;
    d = fma(-l, tb[i], ta[i + 1] - lam);
    if (fabs(d) < guard) d = d < 0.0 ? -guard : guard;
    dd[i + 1] = d;
    y = fma(-l, y, rhs[i + 1]);
    out[i + 1] = y;
  }
  for (int i = p; i <= q; ++i) out[i] *= recip(dd[i]);
  for (int i = q - 1; i >= p; --i) out[i] = fma(-ll[i], out[i + 1], out[i]);
}

// Cluster pass, one block per matrix (see the overview at the top).
template <int D>
__global__ __launch_bounds__(256) void k_sym_cluster(double* __restrict__ scr, int nev,
                                                     double* __restrict__ eigvec) {
  __shared__ double ta[D], tb[D], tau[D], rv[D], xs[D], dd[D], ll[D];
  __shared__ double red[4];
  __shared__ int s_any;
  const int h = blockIdx.x, tid = threadIdx.x;
  double* sh = scr + (int64_t)h * tridiag_scratch<D>();
  if (tid == 0) s_any = 0;
  __syncthreads();
  if (tid < nev && sh[EigScr<D>::kFlag + tid] != 0.0) s_any = 1;
  __syncthreads();
  if (!s_any) return;   // uniform
  if (tid < D) {
    ta[tid] = sh[EigScr<D>::kA + tid];
    tb[tid] = sh[EigScr<D>::kB + tid];
    tau[tid] = sh[EigScr<D>::kTau + tid];
  }
  __syncthreads();
  const double nrm = sh[EigScr<D>::kNrm];
  const double tc = kClusterTol * nrm, guard = 2.220446049250313e-16 * nrm + 1e-300;
  // thread i owns entry i of every vector: it writes and later reads only its
  // own entries of the chain's vectors in scratch
  auto gram_schmidt = [&](double v, int c0, int c1) {
    for (int pass = 0; pass < 2; ++pass)
      for (int k = c0; k < c1; ++k) {
        const double zk = tid < D ? sh[EigScr<D>::kZ + (size_t)k * D + tid] : 0.0;
        const double dot = block_sum_f64_waves<256>(zk * v, red);
        v = fma(-dot, zk, v);
      }
    return v;
  };
  int cstart = -1;
  for (int e = 0; e < nev; ++e) {
    if (sh[EigScr<D>::kFlag + e] == 0.0) {   // uniform
      cstart = -1;
      continue;
    }
    const double lam = sh[EigScr<D>::kLam + e];
    if (cstart < 0 || !(sh[EigScr<D>::kLam + e - 1] - lam <= tc)) cstart = e;
    double* ze = sh + EigScr<D>::kZ + (size_t)e * D;
    double v = tid < D ? ze[tid] : 0.0;
    const double n2 = block_sum_f64_waves<256>(v * v, red);
    v *= n2 > 0.0 ? 1.0 / sqrt(n2) : 0.0;
    v = gram_schmidt(v, cstart, e);
    double r2 = block_sum_f64_waves<256>(v * v, red);
    if (r2 < 1e-6) {
      // the vector was (almost) inside the span of the chain's earlier ones:
      // inverse iteration on its block from a fixed start instead
      const int p = (int)sh[EigScr<D>::kBlk + 2 * e], q = (int)sh[EigScr<D>::kBlk + 2 * e + 1];
      v = (tid >= p && tid <= q) ? start_entry(tid, e) : 0.0;
      for (int it = 0; it < 3; ++it) {
        v = gram_schmidt(v, cstart, e);
        const double a = block_max_f64<256>(fabs(v), red);
        if (tid < D) rv[tid] = (a > 0.0 && a < 1e300) ? v / a : v;
        __syncthreads();
        if (tid == 0) tridiag_solve<D>(ta, tb, p, q, lam, guard, rv, xs, dd, ll);
        __syncthreads();
        v = tid < D ? xs[tid] : 0.0;
        const double b = block_max_f64<256>(fabs(v), red);
        if (b > 0.0 && b < 1e300) v /= b;
      }
      v = gram_schmidt(v, cstart, e);
      r2 = block_sum_f64_waves<256>(v * v, red);
    }
    v *= r2 > 0.0 ? 1.0 / sqrt(r2) : 0.0;
    if (tid < D) ze[tid] = v;
  }
  __syncthreads();
  // back-transform the flagged vectors: wave w takes e = w, w + 4, ...
  const int wv = tid >> 6, ln = tid & 63;
  for (int e = wv; e < nev; e += 4) {
    if (sh[EigScr<D>::kFlag + e] == 0.0) continue;   // uniform over the wave
    if (ln < 32)
      back_transform1<D>(sh + EigScr<D>::kZ + (size_t)e * D, sh + EigScr<D>::kW, tau,
                         eigvec + ((int64_t)h * D + e) * D, ln);
  }
}

void launch_sym_eig_top(const double* A, int H, int d, int nev, double* eigval, double* eigvec, double* trace,
                        double* scratch, hipStream_t st) {
  if (nev <= 0) nev = 1;
  if (nev > d) nev = d;
  if (d == 128) {
    hipLaunchKernelGGL((k_sym_tridiag<128>), dim3(H), dim3(256), sizeof(double) * 128 * 128, st, A, scratch, trace);
    hipLaunchKernelGGL((k_sym_eigpair<128>), dim3(nev, H), dim3(256), 0, st, scratch, eigval, eigvec);
    hipLaunchKernelGGL((k_sym_cluster<128>), dim3(H), dim3(256), 0, st, scratch, nev, eigvec);
  } else {
    hipLaunchKernelGGL((k_sym_tridiag<64>), dim3(H), dim3(256), sizeof(double) * 64 * 64, st, A, scratch, trace);
    hipLaunchKernelGGL((k_sym_eigpair<64>), dim3(nev, H), dim3(256), 0, st, scratch, eigval, eigvec);
    hipLaunchKernelGGL((k_sym_cluster<64>), dim3(H), dim3(256), 0, st, scratch, nev, eigvec);
  }
}

size_t sym_eig_scratch(int H, int d) {
  return (size_t)H * (d == 128 ? tridiag_scratch<128>() : tridiag_scratch<64>());
}

void init_linalg_attributes() {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sym_tridiag<128>), hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)(sizeof(double) * 128 * 128));
}

}  // namespace spr
