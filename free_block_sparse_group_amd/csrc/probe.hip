// Stages 4-5a kernels: query-group-stratified exact probe rows and the
// weighted ridge affine fit in the probe-residual subspace
// (arXiv:2608.18484, paperlayer.ai summary section 4 "Probe-Fitted Residual
// Reconstruction", appendices A.1-A.3; gist.science (nl) section 2B).
// Allocation and selection are integer work (bit-exact); the fit is float64.
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

hipError_t launch_probe_rows(const ProbeFitArgs& a, const int32_t* qidx);

// Probes per query group.  Fewer probes than nonempty groups: the M largest
// groups (ties to the smaller index) get one each.  Otherwise one each, and
// the other M - |A| are shared by largest remainder in proportion to group
// size (integer quotients; remainders ranked descending, ties to the smaller
// index), capped at the group size, the overflow shared again over the
// groups that still have room.  Then the (group, rank) list of probe slots.
__global__ __launch_bounds__(1024) void k_probe_alloc(const int32_t* __restrict__ q_off, int G, int M,
                                                      int32_t* __restrict__ alloc, int32_t* __restrict__ pgroup,
                                                      int32_t* __restrict__ prank) {
  __shared__ int n[kMaxGroups];
  __shared__ int m[kMaxGroups];
  __shared__ int act[kMaxGroups];
  __shared__ int64_t shr[kMaxGroups];
  __shared__ int64_t rem[kMaxGroups];
  __shared__ int64_t red[1024];
  __shared__ int base[kMaxGroups + 1];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int32_t* qo = q_off + (int64_t)h * (G + 1);
  for (int a = tid; a < G; a += 1024) { n[a] = qo[a + 1] - qo[a]; m[a] = 0; }
  __syncthreads();
  int64_t cnt = 0;
  for (int a = tid; a < G; a += 1024) cnt += n[a] > 0;
  const int nA = (int)block_sum_i64<1024>(cnt, red);
  if (M < nA) {
    for (int a = tid; a < G; a += 1024) {
      if (n[a] == 0) continue;
      int rank = 0;
      for (int b = 0; b < G; ++b) rank += n[b] > 0 && (n[b] > n[a] || (n[b] == n[a] && b < a));
      m[a] = rank < M ? 1 : 0;
    }
    __syncthreads();
  } else {
    for (int a = tid; a < G; a += 1024) { m[a] = n[a] > 0; act[a] = n[a] > 0; }
    __syncthreads();
    int64_t left = M - nA;
    // every round either finishes (nothing capped) or caps at least one more
    // group, so at most G + 1 rounds run; the bound is kept explicit
    for (int round = 0; left > 0 && round <= G + 1; ++round) {
      int64_t S = 0;
      for (int a = tid; a < G; a += 1024) S += act[a] ? n[a] : 0;
      S = block_sum_i64<1024>(S, red);
      int64_t given = 0;
      for (int a = tid; a < G; a += 1024) {
        shr[a] = act[a] ? (left * n[a]) / S : 0;
        rem[a] = act[a] ? (left * n[a]) % S : -1;
        given += shr[a];
      }
      given = block_sum_i64<1024>(given, red);   // also publishes shr/rem
      const int64_t spare = left - given;
      int64_t over = 0;
      for (int a = tid; a < G; a += 1024) {
        if (!act[a]) continue;
        int64_t rank = 0;
        for (int b = 0; b < G; ++b) rank += act[b] && (rem[b] > rem[a] || (rem[b] == rem[a] && b < a));
        const int64_t extra = shr[a] + (rank < spare ? 1 : 0);
        const int64_t room = n[a] - m[a];
        const int64_t take = extra < room ? extra : room;
        m[a] += (int)take;
        over += extra - take;
      }
      over = block_sum_i64<1024>(over, red);
      for (int a = tid; a < G; a += 1024) act[a] = act[a] && (m[a] < n[a]);
      __syncthreads();
      left = over;
    }
  }
  if (tid == 0) {
    int run = 0;
    for (int a = 0; a < G; ++a) { base[a] = run; run += m[a]; }
    base[G] = run;
  }
  __syncthreads();
  for (int a = tid; a < G; a += 1024) {
    alloc[(int64_t)h * G + a] = m[a];
    for (int j = 0; j < m[a]; ++j) {
      pgroup[(int64_t)h * M + base[a] + j] = a;
      prank[(int64_t)h * M + base[a] + j] = (int)(((int64_t)2 * j + 1) * n[a] / ((int64_t)2 * m[a]));
    }
  }
}

// order-preserving integer key of a double (total order, -0 < +0 aside)
SPR_DEV uint64_t dkey(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// For probe slot p: the member of its group with `rank` members before it in
// the (q_dist, token) order.  Radix descent over the distance keys, then the
// tie group in token order (q_perm lists a group's tokens ascending).
__global__ __launch_bounds__(256) void k_probe_select(const int32_t* __restrict__ q_off,
                                                      const int32_t* __restrict__ q_perm,
                                                      const double* __restrict__ q_dist, int N, int G, int M,
                                                      const int32_t* __restrict__ pgroup,
                                                      const int32_t* __restrict__ prank, int32_t* __restrict__ pt) {
  __shared__ int hist[256];
  __shared__ int cnts[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_below;
  __shared__ int s_found;
  const int h = blockIdx.y, slot = blockIdx.x, tid = threadIdx.x;
  const int a = pgroup[(int64_t)h * M + slot];
  const int r = prank[(int64_t)h * M + slot];
  const int b0 = q_off[(int64_t)h * (G + 1) + a], b1 = q_off[(int64_t)h * (G + 1) + a + 1];
  const int32_t* perm = q_perm + (int64_t)h * N;
  const double* dist = q_dist + (int64_t)h * N;
  if (tid == 0) { s_prefix = 0; s_below = 0; s_found = perm[b0]; }
  __syncthreads();
  for (int level = 7; level >= 0; --level) {
    hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    const int sh = 8 * level;
    for (int i = b0 + tid; i < b1; i += 256) {
      const uint64_t k = dkey(dist[perm[i]]);
      const uint64_t high = level == 7 ? 0 : (k >> (sh + 8));
      if (high == prefix) atomicAdd(&hist[(k >> sh) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int below = s_below, bin = 0;
      for (int v = 0; v < 256; ++v) {
        if (below + hist[v] > r) { bin = v; break; }
        below += hist[v];
      }
      s_below = below;
      s_prefix = (prefix << 8) | (uint64_t)bin;
    }
    __syncthreads();
  }
  const uint64_t target = s_prefix;
  const int want = r - s_below;   // index among the tied members, token order
  const int n = b1 - b0;
  const int per = (n + 255) / 256;
  const int c0 = b0 + tid * per, c1 = min(b1, c0 + per);
  int mine = 0;
  for (int i = c0; i < c1; ++i) mine += dkey(dist[perm[i]]) == target;
  cnts[tid] = mine;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) { const int x = cnts[t]; cnts[t] = run; run += x; }
  }
  __syncthreads();
  int k = cnts[tid];
  if (want >= k && want < k + mine) {
    for (int i = c0; i < c1; ++i) {
      if (dkey(dist[perm[i]]) == target) {
        if (k == want) { s_found = perm[i]; break; }
        ++k;
      }
    }
  }
  __syncthreads();
  if (tid == 0) pt[(int64_t)h * M + slot] = s_found;
}

// probe_idx ascending; weights (n_a/m_a) / (sum of probed n_a)
__global__ __launch_bounds__(1024) void k_probe_finalize(const int32_t* __restrict__ q_off, int G, int M,
                                                         const int32_t* __restrict__ alloc,
                                                         const int32_t* __restrict__ pgroup,
                                                         const int32_t* __restrict__ pt,
                                                         int32_t* __restrict__ probe_idx, double* __restrict__ probe_w) {
  __shared__ int64_t red[1024];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int32_t* qo = q_off + (int64_t)h * (G + 1);
  const int32_t* al = alloc + (int64_t)h * G;
  int64_t tot = 0;
  for (int a = tid; a < G; a += 1024) tot += al[a] > 0 ? qo[a + 1] - qo[a] : 0;
  tot = block_sum_i64<1024>(tot, red);
  const int32_t* t = pt + (int64_t)h * M;
  for (int p = tid; p < M; p += 1024) {
    const int tp = t[p];
    int rank = 0;
    for (int q = 0; q < M; ++q) rank += t[q] < tp || (t[q] == tp && q < p);
    const int a = pgroup[(int64_t)h * M + p];
    const double na = (double)(qo[a + 1] - qo[a]), ma = (double)al[a];
    probe_idx[(int64_t)h * M + rank] = tp;
    probe_w[(int64_t)h * M + rank] = (na / ma) / (double)tot;
  }
}

__global__ void k_inverse_perm(const int32_t* __restrict__ perm, int N, int32_t* __restrict__ inv) {
  const int h = blockIdx.y;
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s < N) inv[(int64_t)h * N + perm[(int64_t)h * N + s]] = (int32_t)s;
}

// x_bar = sum w x, r_bar = sum w (o_dense - x) over the probes (in probe order).
__global__ void k_fit_means(const float* __restrict__ Op, const int32_t* __restrict__ inv,
                            const int32_t* __restrict__ probe_idx, const double* __restrict__ w,
                            const float* __restrict__ O_probe, int N, int M, int d, double* __restrict__ x_bar,
                            double* __restrict__ r_bar) {
  const int h = blockIdx.x, c = threadIdx.x;
  if (c >= d) return;
  double xs = 0.0, rs = 0.0;
  for (int j = 0; j < M; ++j) {
    const int64_t slot = inv[(int64_t)h * N + probe_idx[(int64_t)h * M + j]];
    const double x = Op[((int64_t)h * N + slot) * d + c];
    const double o = O_probe[((int64_t)h * M + j) * d + c];
    const double wj = w[(int64_t)h * M + j];
    xs = fma(wj, x, xs);
    rs = fma(wj, o - x, rs);
  }
  x_bar[(int64_t)h * d + c] = xs;
  r_bar[(int64_t)h * d + c] = rs;
}

// Weighted centred Gram matrices gram[kind][h][i][j], row i per block, kind = blockIdx.z:
//  0: Rt^T Rt   1: Xt^T Xt + lambda I   2: Xt^T Rt
__global__ void k_fit_gram(const float* __restrict__ Op, const int32_t* __restrict__ inv,
                           const int32_t* __restrict__ probe_idx, const double* __restrict__ w,
                           const float* __restrict__ O_probe, const double* __restrict__ x_bar,
                           const double* __restrict__ r_bar, int N, int M, int d, double lambda,
                           double* __restrict__ gram) {
  const int h = blockIdx.y, i = blockIdx.x, kind = blockIdx.z, j = threadIdx.x;
  if (j >= d) return;
  const double xbi = x_bar[(int64_t)h * d + i], xbj = x_bar[(int64_t)h * d + j];
  const double rbi = r_bar[(int64_t)h * d + i], rbj = r_bar[(int64_t)h * d + j];
  double acc = 0.0;
  for (int m = 0; m < M; ++m) {
    const int64_t slot = inv[(int64_t)h * N + probe_idx[(int64_t)h * M + m]];
    const float* xr = Op + ((int64_t)h * N + slot) * d;
    const float* orow = O_probe + ((int64_t)h * M + m) * d;
    const double xi = xr[i], xj = xr[j];
    const double ri = (double)orow[i] - xi, rj = (double)orow[j] - xj;
    double ai, bj;
    if (kind == 0) { ai = ri - rbi; bj = rj - rbj; }
    else if (kind == 1) { ai = xi - xbi; bj = xj - xbj; }
    else { ai = xi - xbi; bj = rj - rbj; }
    acc = fma(w[(int64_t)h * M + m] * ai, bj, acc);
  }
  if (kind == 1 && i == j) acc += lambda;
  gram[(((int64_t)kind * gridDim.y + h) * d + i) * d + j] = acc;
}

// One block per head: numerical rank, Cholesky of the ridge matrix (packed
// lower triangle in LDS), B_r = (Xt^T Xt + lam I)^-1 (Xt^T Rt) V_r by forward
// and back substitution, 32 right-hand sides at a time.
constexpr double kRankTol = 1e-6;
__global__ __launch_bounds__(1024) void k_fit_solve(const double* __restrict__ gram, const double* __restrict__ feig,
                                                    const double* __restrict__ fvec, int d, int rank,
                                                    double* __restrict__ B_r, double* __restrict__ V_r,
                                                    int32_t* __restrict__ rank_eff) {
  extern __shared__ double sm[];
  double* Lp = sm;                                  // packed lower triangle, d(d+1)/2
  double* Y = sm + d * (d + 1) / 2;                 // [d][32]
  __shared__ int s_fail;
  const int h = blockIdx.x, tid = threadIdx.x;
  const int H = gridDim.x;
  const double* GX = gram + ((int64_t)1 * H + h) * d * d;   // Xt^T Xt + lambda I
  const double* GC = gram + ((int64_t)2 * H + h) * d * d;   // Xt^T Rt
  auto P = [&](int i, int j) -> double& { return Lp[i * (i + 1) / 2 + j]; };  // i >= j
  const double* ev = feig + (int64_t)h * d;
  int reff = 0;
  if (ev[0] > 0.0) {
    const double thr = kRankTol * kRankTol * ev[0];
    for (int i = 0; i < d; ++i) reff += ev[i] > thr;
  }
  reff = min(reff, rank);
  for (int e = tid; e < d * d; e += 1024) {
    const int i = e / d, j = e % d;
    if (j <= i) P(i, j) = GX[e];
  }
  if (tid == 0) s_fail = 0;
  __syncthreads();
  // right-looking Cholesky
  for (int k = 0; k < d; ++k) {
    if (tid == 0) {
      const double piv = P(k, k);
      if (!(piv > 0.0)) s_fail = 1;
      P(k, k) = piv > 0.0 ? sqrt(piv) : 1.0;
    }
    __syncthreads();
    const double lkk = P(k, k);
    for (int i = k + 1 + tid; i < d; i += 1024) P(i, k) /= lkk;
    __syncthreads();
    const int rem = d - k - 1;
    for (int e = tid; e < rem * rem; e += 1024) {
      const int i = k + 1 + e / rem, j = k + 1 + e % rem;
      if (j <= i) P(i, j) -= P(i, k) * P(j, k);
    }
    __syncthreads();
  }
  if (s_fail) reff = 0;
  for (int e = tid; e < d * rank; e += 1024) {
    B_r[(int64_t)h * d * rank + e] = 0.0;
    V_r[(int64_t)h * d * rank + e] = 0.0;
  }
  if (tid == 0) rank_eff[h] = reff;
  __syncthreads();
  const double* vecs = fvec + (int64_t)h * d * d;   // eigenvector k contiguous
  const int c = tid >> 5, part = tid & 31;          // 32 columns x 32 partial lanes
  for (int k0 = 0; k0 < reff; k0 += 32) {
    const int kc = min(32, reff - k0);
    // Y[:, c] = (Xt^T Rt) v_{k0+c}
    for (int e = tid; e < d * 32; e += 1024) {
      const int i = e / 32, cc = e % 32;
      double acc = 0.0;
      if (cc < kc)
        for (int j = 0; j < d; ++j) acc = fma(GC[(int64_t)i * d + j], vecs[(int64_t)(k0 + cc) * d + j], acc);
      Y[i * 32 + cc] = acc;
    }
    __syncthreads();
    // forward: L y = rhs
    for (int i = 0; i < d; ++i) {
      double s = 0.0;
      for (int j = part; j < i; j += 32) s = fma(P(i, j), Y[j * 32 + c], s);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 32);
      s = __shfl(s, 0, 32);
      __syncthreads();
      if (part == 0) Y[i * 32 + c] = (Y[i * 32 + c] - s) / P(i, i);
      __syncthreads();
    }
    // back: L^T b = y
    for (int i = d - 1; i >= 0; --i) {
      double s = 0.0;
      for (int j = i + 1 + part; j < d; j += 32) s = fma(P(j, i), Y[j * 32 + c], s);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 32);
      s = __shfl(s, 0, 32);
      __syncthreads();
      if (part == 0) Y[i * 32 + c] = (Y[i * 32 + c] - s) / P(i, i);
      __syncthreads();
    }
    for (int e = tid; e < d * 32; e += 1024) {
      const int i = e / 32, cc = e % 32;
      if (cc < kc) {
        B_r[((int64_t)h * d + i) * rank + k0 + cc] = Y[i * 32 + cc];
        V_r[((int64_t)h * d + i) * rank + k0 + cc] = vecs[(int64_t)(k0 + cc) * d + i];
      }
    }
    __syncthreads();
  }
}

static size_t fit_solve_lds(int d) { return sizeof(double) * ((size_t)d * (d + 1) / 2 + (size_t)d * 32); }

void init_probe_attributes() {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fit_solve), hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)fit_solve_lds(128));
}

hipError_t launch_probe_fit(const ProbeFitArgs& a) {
  const int H = a.H, N = a.N, d = a.d, G = a.G_q, M = a.M;
  hipStream_t st = a.stream;
  hipLaunchKernelGGL(k_probe_alloc, dim3(H), dim3(1024), 0, st, a.q_off, G, M, a.ws.alloc, a.ws.pgroup, a.ws.prank);
  hipLaunchKernelGGL(k_probe_select, dim3(M, H), dim3(256), 0, st, a.q_off, a.q_perm, a.q_dist, N, G, M,
                     a.ws.pgroup, a.ws.prank, a.ws.pt);
  hipLaunchKernelGGL(k_probe_finalize, dim3(H), dim3(1024), 0, st, a.q_off, G, M, a.ws.alloc, a.ws.pgroup, a.ws.pt,
                     a.probe_idx, a.probe_w);
  hipError_t e = launch_probe_rows(a, a.probe_idx);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_inverse_perm, dim3((N + 255) / 256, H), dim3(256), 0, st, a.q_perm, N, a.ws.inv_perm);
  hipLaunchKernelGGL(k_fit_means, dim3(H), dim3(128), 0, st, a.Op, a.ws.inv_perm, a.probe_idx, a.probe_w, a.O_probe,
                     N, M, d, a.x_bar, a.r_bar);
  hipLaunchKernelGGL(k_fit_gram, dim3(d, H, 3), dim3(128), 0, st, a.Op, a.ws.inv_perm, a.probe_idx, a.probe_w,
                     a.O_probe, a.x_bar, a.r_bar, N, M, d, a.lambda, a.ws.gram);
  // eigenvectors of Rt^T Rt (the kind-0 block, contiguous over heads)
  launch_sym_eig(a.ws.gram, H, d, a.ws.feig, a.ws.fvec, st);
  hipLaunchKernelGGL(k_fit_solve, dim3(H), dim3(1024), fit_solve_lds(d), st, a.ws.gram, a.ws.feig, a.ws.fvec, d,
                     a.rank, a.B_r, a.V_r, a.rank_eff);
  return hipGetLastError();
}

}  // namespace spr
