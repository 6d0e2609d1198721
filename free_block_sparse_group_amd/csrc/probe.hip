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

// Ranking key of a (nonnegative) distance: the float64 value rounded to 30
// significant bits (half up on the magnitude), so that distances equal in
// exact arithmetic but a few ulps apart after rounding compare equal and the
// token index decides; then an order-preserving integer image.
constexpr int kDistRankDrop = 64 - 12 - 29;   // low mantissa bits cleared
SPR_DEV uint64_t dkey(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t sign = b & 0x8000000000000000ull;
  b = (((b & 0x7fffffffffffffffull) + (1ull << (kDistRankDrop - 1))) & ~((1ull << kDistRankDrop) - 1)) | sign;
  return sign ? ~b : (b | 0x8000000000000000ull);
}

// Exclusive prefix sum over a 256-thread block (4 waves); returns the
// exclusive prefix of v and writes the block total to *total.
SPR_DEV int block_exclusive_scan256(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  int before = 0;
  for (int u = 0; u < wv; ++u) before += wsum[u];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + x - v;
}

// For probe slot p: the member of its group with `rank` members before it in
// the (q_dist, token) order.  Radix descent over the 64-bit distance keys, 8
// bits per level, with a parallel scan over the 256 bins; then the tie group
// in token order (q_perm lists a group's tokens ascending).  Groups of up to
// kSelCache members keep their keys in LDS for the eight passes.
constexpr int kSelCache = 4096;
__global__ __launch_bounds__(256) void k_probe_select(const int32_t* __restrict__ q_off,
                                                      const int32_t* __restrict__ q_perm,
                                                      const double* __restrict__ q_dist, int N, int G, int M,
                                                      const int32_t* __restrict__ pgroup,
                                                      const int32_t* __restrict__ prank, int32_t* __restrict__ pt,
                                                      int32_t* __restrict__ pslot) {
  __shared__ uint64_t keys[kSelCache];
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ uint64_t s_prefix;
  __shared__ int s_below;
  __shared__ int s_found, s_fslot;
  const int h = blockIdx.y, slot = blockIdx.x, tid = threadIdx.x;
  const int a = pgroup[(int64_t)h * M + slot];
  const int r = prank[(int64_t)h * M + slot];
  const int b0 = q_off[(int64_t)h * (G + 1) + a], b1 = q_off[(int64_t)h * (G + 1) + a + 1];
  const int n = b1 - b0;
  const int32_t* perm = q_perm + (int64_t)h * N + b0;
  const double* dist = q_dist + (int64_t)h * N;
  const bool cached = n <= kSelCache;
  if (cached)
    for (int i = tid; i < n; i += 256) keys[i] = dkey(dist[perm[i]]);
  if (tid == 0) { s_prefix = 0; s_below = 0; s_found = perm[0]; s_fslot = b0; }
  __syncthreads();
  for (int level = 7; level >= 0; --level) {
    hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    const int sh = 8 * level;
    for (int i = tid; i < n; i += 256) {
      const uint64_t k = cached ? keys[i] : dkey(dist[perm[i]]);
      const uint64_t high = level == 7 ? 0 : (k >> (sh + 8));
      if (high == prefix) atomicAdd(&hist[(k >> sh) & 255], 1);
    }
    __syncthreads();
    const int c = hist[tid];
    const int base = s_below;   // read before the scan's barriers; rewritten only after them
    int tot;
    const int below = base + block_exclusive_scan256(c, wsum, &tot);
    // exactly one bin holds the wanted rank (the rank is below the group size)
    if (below <= r && r < below + c) {
      s_below = below;
      s_prefix = (prefix << 8) | (uint64_t)tid;
    }
    __syncthreads();
  }
  const uint64_t target = s_prefix;
  const int want = r - s_below;   // index among the tied members, token order
  const int per = (n + 255) / 256;
  const int c0 = tid * per, c1 = min(n, c0 + per);
  int mine = 0;
  for (int i = c0; i < c1; ++i) mine += (cached ? keys[i] : dkey(dist[perm[i]])) == target;
  int tot;
  int k = block_exclusive_scan256(mine, wsum, &tot);
  if (want >= k && want < k + mine) {
    for (int i = c0; i < c1; ++i) {
      if ((cached ? keys[i] : dkey(dist[perm[i]])) == target) {
        if (k == want) { s_found = perm[i]; s_fslot = b0 + i; break; }
        ++k;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    pt[(int64_t)h * M + slot] = s_found;
    pslot[(int64_t)h * M + slot] = s_fslot;
  }
}

// probe_idx ascending; weights (n_a/m_a) / (sum of probed n_a); the
// group-major slot of each probe in the same order
__global__ __launch_bounds__(1024) void k_probe_finalize(const int32_t* __restrict__ q_off, int G, int M,
                                                         const int32_t* __restrict__ alloc,
                                                         const int32_t* __restrict__ pgroup,
                                                         const int32_t* __restrict__ pt,
                                                         const int32_t* __restrict__ pslot,
                                                         int32_t* __restrict__ probe_idx, double* __restrict__ probe_w,
                                                         int32_t* __restrict__ probe_slot) {
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
    probe_slot[(int64_t)h * M + rank] = pslot[(int64_t)h * M + p];
  }
}

// Probe rows gathered once: x = the sparse output row (group-major slot of
// the probe token), r = exact dense row - x, both float64 [H, M, d].
__global__ void k_fit_gather(const float* __restrict__ Op, const int32_t* __restrict__ probe_slot,
                             const float* __restrict__ O_probe, int N, int M, int d, double* __restrict__ fx,
                             double* __restrict__ fr) {
  const int m = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  if (c >= d) return;
  const int64_t slot = probe_slot[(int64_t)h * M + m];
  const double x = Op[((int64_t)h * N + slot) * d + c];
  const double o = O_probe[((int64_t)h * M + m) * d + c];
  fx[((int64_t)h * M + m) * d + c] = x;
  fr[((int64_t)h * M + m) * d + c] = o - x;
}

// x_bar = sum w x, r_bar = sum w r over the probes; four interleaved partial
// sums per channel, added in a fixed order.
__global__ __launch_bounds__(512) void k_fit_means(const double* __restrict__ fx, const double* __restrict__ fr,
                                                   const double* __restrict__ w, int M, int d,
                                                   double* __restrict__ x_bar, double* __restrict__ r_bar) {
  __shared__ double px[4][128], pr[4][128];
  const int h = blockIdx.x, c = threadIdx.x % 128, part = threadIdx.x / 128;
  double xs = 0.0, rs = 0.0;
  if (c < d)
#pragma unroll 8
    for (int m = part; m < M; m += 4) {
      const double wm = w[(int64_t)h * M + m];
      xs = fma(wm, fx[((int64_t)h * M + m) * d + c], xs);
      rs = fma(wm, fr[((int64_t)h * M + m) * d + c], rs);
    }
  px[part][c] = xs;
  pr[part][c] = rs;
  __syncthreads();
  if (part == 0 && c < d) {
    x_bar[(int64_t)h * d + c] = (px[0][c] + px[1][c]) + (px[2][c] + px[3][c]);
    r_bar[(int64_t)h * d + c] = (pr[0][c] + pr[1][c]) + (pr[2][c] + pr[3][c]);
  }
}

// Weighted centred Gram matrices gram[kind][h][i][j], kind = blockIdx.z:
//  0: Rt^T Rt   1: Xt^T Xt + lambda I   2: Xt^T Rt
// A block computes 16 rows i for every column j (one thread per j).  The
// probes pass through LDS 8192 / D at a time (64 KiB of right factors), every
// load of a chunk in flight together.
constexpr int kGramRows = 16;
template <int D>
__global__ __launch_bounds__(128) void k_fit_gram(const double* __restrict__ fx, const double* __restrict__ fr,
                                                  const double* __restrict__ w, const double* __restrict__ x_bar,
                                                  const double* __restrict__ r_bar, int M, double lambda,
                                                  double* __restrict__ gram) {
  constexpr int CH = 8192 / D;                  // probes per chunk
  constexpr int RSTEP = 128 / D;                // thread j stages column j % D of rows j / D + r RSTEP
  constexpr int NA = CH * kGramRows / 128;      // left entries per thread
  __shared__ double arow[CH][kGramRows];        // w_m (a_m,i - abar_i) for the block's rows
  __shared__ double bcol[CH][D];                // b_m,j - bbar_j
  const int d = D;
  const int h = blockIdx.y, i0 = blockIdx.x * kGramRows, kind = blockIdx.z, j = threadIdx.x;
  const double* A = (kind == 0 ? fr : fx) + (int64_t)h * M * d;   // left factor (rows i)
  const double* B = (kind == 1 ? fx : fr) + (int64_t)h * M * d;   // right factor (columns j)
  const double* abar = (kind == 0 ? r_bar : x_bar) + (int64_t)h * d;
  const double* bbar = (kind == 1 ? x_bar : r_bar) + (int64_t)h * d;
  const double bj_bar = j < d ? bbar[j] : 0.0;
  double acc[kGramRows];
#pragma unroll
  for (int u = 0; u < kGramRows; ++u) acc[u] = 0.0;
  for (int m0 = 0; m0 < M; m0 += CH) {
    __syncthreads();
    const int mc = min(CH, M - m0);
    {
      // (clamped, always-valid addresses; out-of-range entries are zeroed after the load)
      double av[NA], bv[CH / RSTEP];
#pragma unroll
      for (int r = 0; r < NA; ++r) {
        const int e = j + 128 * r, mm = e / kGramRows, u = e % kGramRows, m = m0 + mm, i = i0 + u;
        const int mcl = min(m, M - 1);
        const double val = w[(int64_t)h * M + mcl] * (A[(int64_t)mcl * d + i] - abar[i]);
        av[r] = m < M ? val : 0.0;
      }
      const int k = j % D, rs0 = j / D;
#pragma unroll
      for (int r = 0; r < CH / RSTEP; ++r) {
        const int mm = min(rs0 + r * RSTEP, mc - 1);
        bv[r] = B[(int64_t)(m0 + mm) * d + k];
      }
#pragma unroll
      for (int r = 0; r < NA; ++r) {
        const int e = j + 128 * r;
        arow[e / kGramRows][e % kGramRows] = av[r];
      }
#pragma unroll
      for (int r = 0; r < CH / RSTEP; ++r) {
        const int mm = rs0 + r * RSTEP;
        if (mm < mc) bcol[mm][k] = bv[r];
      }
    }
    __syncthreads();
    if (j < D)
#pragma unroll 2
      for (int mm = 0; mm < mc; ++mm) {
        const double bj = bcol[mm][j] - bj_bar;
#pragma unroll
        for (int u = 0; u < kGramRows; ++u) acc[u] = fma(arow[mm][u], bj, acc[u]);
      }
  }
  if (j >= d) return;
#pragma unroll
  for (int u = 0; u < kGramRows; ++u) {
    const int i = i0 + u;
    if (i >= d) break;
    double v = acc[u];
    if (kind == 1 && i == j) v += lambda;
    gram[(((int64_t)kind * gridDim.y + h) * d + i) * d + j] = v;
  }
}

// Right-hand sides of the fit, Y[h][i][k] = sum_j (Xt^T Rt)[i][j] v_k[j] for
// the leading eigenvectors v_k of Rt^T Rt (k < rank), one block per (i, h).
__global__ __launch_bounds__(128) void k_fit_rhs(const double* __restrict__ gram, const double* __restrict__ fvec,
                                                 int d, int rank, double* __restrict__ Y) {
  __shared__ double gi[128];
  const int i = blockIdx.x, h = blockIdx.y, k = threadIdx.x, H = gridDim.y;
  const double* GC = gram + (((int64_t)2 * H + h) * d + i) * d;   // row i of Xt^T Rt
  if (k < d) gi[k] = GC[k];
  __syncthreads();
  if (k >= rank) return;
  const double* v = fvec + ((int64_t)h * d + k) * d;
  double acc = 0.0;
  for (int j = 0; j < d; ++j) acc = fma(gi[j], v[j], acc);
  Y[((int64_t)h * d + i) * rank + k] = acc;
}

// One block per head: numerical rank, then B_r = (Xt^T Xt + lam I)^-1 Y by
// Gauss-Jordan elimination of the augmented matrix [Xt^T Xt + lam I | Y],
// Y = (Xt^T Rt) V_r, 32 right-hand sides at a time.  The matrix is symmetric
// positive definite, so no pivoting is needed and the step-k pivot is the
// Schur-complement diagonal (a nonpositive one marks the fit as failed).  The
// augmented matrix lives in registers: thread (ti, tj) of a 16 x 16 grid owns
// rows ti + 16u and columns tj + 16v.  Step k publishes the pivot row and
// column through double-buffered LDS, so each step needs one barrier.
constexpr double kRankTol = 1e-6;

template <int D>
__global__ __launch_bounds__(256) void k_fit_solve(const double* __restrict__ gram, const double* __restrict__ feig,
                                                   const double* __restrict__ fvec, const double* __restrict__ rhs,
                                                   int rank, double* __restrict__ B_r, double* __restrict__ V_r,
                                                   int32_t* __restrict__ rank_eff) {
  constexpr int W = D + 32;        // augmented width
  constexpr int RU = D / 16, CV = W / 16;
  __shared__ double prow[2][W];
  __shared__ double pcol[2][D];
  const int h = blockIdx.x, tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
  const int H = gridDim.x;
  const double* GX = gram + ((int64_t)1 * H + h) * D * D;   // Xt^T Xt + lambda I
  const double* ev = feig + (int64_t)h * D;
  // (only the leading `rank` eigenvalues are computed; they decide min(count, rank))
  int reff = 0;
  if (rank > 0 && ev[0] > 0.0) {
    const double thr = kRankTol * kRankTol * ev[0];   // eigenvalues are squared singular values
    for (int i = 0; i < rank; ++i) reff += ev[i] > thr;
  }
  for (int e = tid; e < D * rank; e += 256) {
    B_r[(int64_t)h * D * rank + e] = 0.0;
    V_r[(int64_t)h * D * rank + e] = 0.0;
  }
  const double* vecs = fvec + (int64_t)h * D * D;   // eigenvector k contiguous
  bool fail = false;
  for (int k0 = 0; k0 < reff && !fail; k0 += 32) {
    const int kc = min(32, reff - k0);
    double a[RU][CV];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
      for (int v = 0; v < CV; ++v) {
        const int i = ti + 16 * u, j = tj + 16 * v;
        if (j < D) a[u][v] = GX[(int64_t)i * D + j];
        else a[u][v] = (j - D) < kc ? rhs[((int64_t)h * D + i) * rank + k0 + (j - D)] : 0.0;
      }
    for (int k = 0; k < D; ++k) {
      const int buf = k & 1;
      // (register arrays indexed only by unrolled constants: compare-select, no scratch)
      if (ti == (k & 15)) {
#pragma unroll
        for (int u = 0; u < RU; ++u)
          if (u == (k >> 4)) {
#pragma unroll
            for (int v = 0; v < CV; ++v) prow[buf][tj + 16 * v] = a[u][v];
          }
      }
      if (tj == (k & 15)) {
#pragma unroll
        for (int v = 0; v < CV; ++v)
          if (v == (k >> 4)) {
#pragma unroll
            for (int u = 0; u < RU; ++u) pcol[buf][ti + 16 * u] = a[u][v];
          }
      }
      __syncthreads();
      double piv = prow[buf][k];
      if (!(piv > 0.0)) { fail = true; piv = 1.0; }   // same value in every thread
      const double inv = recip(piv);
      double pr[CV];
#pragma unroll
      for (int v = 0; v < CV; ++v) pr[v] = prow[buf][tj + 16 * v];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int i = ti + 16 * u;
        if (i == k) {
#pragma unroll
          for (int v = 0; v < CV; ++v) a[u][v] = pr[v] * inv;
        } else {
          const double f = pcol[buf][i] * inv;
#pragma unroll
          for (int v = 0; v < CV; ++v) a[u][v] = fma(-f, pr[v], a[u][v]);
        }
      }
    }
    if (fail) break;
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
      for (int v = 0; v < CV; ++v) {
        const int i = ti + 16 * u, c = tj + 16 * v - D;
        if (c >= 0 && c < kc) {
          B_r[((int64_t)h * D + i) * rank + k0 + c] = a[u][v];
          V_r[((int64_t)h * D + i) * rank + k0 + c] = vecs[(int64_t)(k0 + c) * D + i];
        }
      }
    __syncthreads();
  }
  if (fail) {
    // the ridge matrix is not positive definite (possible only with lambda = 0): no feature term
    __syncthreads();
    for (int e = tid; e < D * rank; e += 256) {
      B_r[(int64_t)h * D * rank + e] = 0.0;
      V_r[(int64_t)h * D * rank + e] = 0.0;
    }
    reff = 0;
  }
  if (tid == 0) rank_eff[h] = reff;
}

void init_probe_attributes() {}

hipError_t launch_probe_fit(const ProbeFitArgs& a) {
  const int H = a.H, N = a.N, d = a.d, G = a.G_q, M = a.M;
  hipStream_t st = a.stream;
  hipLaunchKernelGGL(k_probe_alloc, dim3(H), dim3(1024), 0, st, a.q_off, G, M, a.ws.alloc, a.ws.pgroup, a.ws.prank);
  hipLaunchKernelGGL(k_probe_select, dim3(M, H), dim3(256), 0, st, a.q_off, a.q_perm, a.q_dist, N, G, M,
                     a.ws.pgroup, a.ws.prank, a.ws.pt, a.ws.pslot);
  hipLaunchKernelGGL(k_probe_finalize, dim3(H), dim3(1024), 0, st, a.q_off, G, M, a.ws.alloc, a.ws.pgroup, a.ws.pt,
                     a.ws.pslot, a.probe_idx, a.probe_w, a.ws.probe_slot);
  hipError_t e = launch_probe_rows(a, a.probe_idx);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fit_gather, dim3(M, H), dim3(d), 0, st, a.Op, a.ws.probe_slot, a.O_probe, N, M, d, a.ws.fx,
                     a.ws.fr);
  hipLaunchKernelGGL(k_fit_means, dim3(H), dim3(512), 0, st, a.ws.fx, a.ws.fr, a.probe_w, M, d, a.x_bar, a.r_bar);
  if (d == 128)
    hipLaunchKernelGGL(k_fit_gram<128>, dim3(128 / kGramRows, H, 3), dim3(128), 0, st, a.ws.fx, a.ws.fr, a.probe_w,
                       a.x_bar, a.r_bar, M, a.lambda, a.ws.gram);
  else
    hipLaunchKernelGGL(k_fit_gram<64>, dim3(64 / kGramRows, H, 3), dim3(128), 0, st, a.ws.fx, a.ws.fr, a.probe_w,
                       a.x_bar, a.r_bar, M, a.lambda, a.ws.gram);
  // leading `rank` eigenpairs of Rt^T Rt (the kind-0 block, contiguous over
  // heads): squared singular values and right singular vectors of Rt
  if (a.rank > 0) {
    launch_sym_eig_top(a.ws.gram, H, d, a.rank, a.ws.feig, a.ws.fvec, a.ws.ftrace, a.ws.eigscr, st);
    hipLaunchKernelGGL(k_fit_rhs, dim3(d, H), dim3(128), 0, st, a.ws.gram, a.ws.fvec, d, a.rank, a.ws.frhs);
  }
  if (d == 128)
    hipLaunchKernelGGL(k_fit_solve<128>, dim3(H), dim3(256), 0, st, a.ws.gram, a.ws.feig, a.ws.fvec, a.ws.frhs,
                       a.rank, a.B_r, a.V_r, a.rank_eff);
  else
    hipLaunchKernelGGL(k_fit_solve<64>, dim3(H), dim3(256), 0, st, a.ws.gram, a.ws.feig, a.ws.fvec, a.ws.frhs,
                       a.rank, a.B_r, a.V_r, a.rank_eff);
  return hipGetLastError();
}

}  // namespace spr
