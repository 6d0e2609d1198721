// Stage 1 kernels: response-coupled partition and group-major permutation.
// Method: arXiv:2608.18484 ("Partition the Support, Reconstruct the
// Residual"), paperlayer.ai summary section 4 and appendices B.1-B.2, C.1;
// gist.science (nl) section 2A.  All partition arithmetic is float64 so that
// labels, permutations and offsets match a float64 reference exactly up to
// genuine near-ties; every reduction has a fixed order (no float atomics).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace spr {

// ---------------------------------------------------------------- M_K
// M_K[i][j] = (1/M_s) sum_s Q[idx_s][i] Q[idx_s][j], idx_s = floor((2s+1)N/(2M_s)).
// A block computes kGramRows rows i for every column j.  The sampled rows pass
// through LDS in the input type, 32 KiB at a time, copied with 16-byte
// loads that are all in flight together; each entry is then summed over s in
// order from LDS (row values broadcast, column values conflict free).
constexpr int kGramTileRows = 16;   // (query-response metric kernel below)
constexpr int kGramChunkRows = 32;
constexpr int kGramRows = 8;
constexpr int kGramBytes = 32768;
template <typename T, int D>
__global__ __launch_bounds__(256) void k_gram_mk(const T* __restrict__ Q, int N, int M_s, double* __restrict__ MK) {
  constexpr int VEC = 16 / sizeof(T);                   // elements per 16-byte copy
  constexpr int CH = (int)(kGramBytes / sizeof(T)) / D; // sampled rows per chunk
  constexpr int VPR = D / VEC;                          // copies per row
  constexpr int NG = 256 / D, RPT = kGramRows / NG;     // row groups; rows per thread (2 or 4)
  __shared__ __align__(16) T qs[kGramBytes / sizeof(T)];
  __shared__ int64_t rowoff[CH];
  const int h = blockIdx.y, i0 = blockIdx.x * kGramRows, tid = threadIdx.x;
  const T* q = Q + (int64_t)h * N * D;
  const int j = tid % D, rg = tid / D;
  double acc[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) acc[k] = 0.0;
  for (int s0 = 0; s0 < M_s; s0 += CH) {
    const int sc = min(CH, M_s - s0);
    __syncthreads();
    for (int s = tid; s < sc; s += 256) rowoff[s] = (((int64_t)2 * (s0 + s) + 1) * N / ((int64_t)2 * M_s)) * D;
    __syncthreads();
    const int nv = sc * VPR;
    for (int e0 = 0; e0 < nv; e0 += 8 * 256) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {   // clamped, always-valid sources; all 8 loads in flight
        const int e = min(e0 + u * 256 + tid, nv - 1);
        v[u] = *reinterpret_cast<const uint4*>(q + rowoff[e / VPR] + (e % VPR) * VEC);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * 256 + tid;
        if (e < nv) *reinterpret_cast<uint4*>(qs + (e / VPR) * D + (e % VPR) * VEC) = v[u];
      }
    }
    __syncthreads();
    // no branches in the loop, so the LDS reads of several samples overlap
#pragma unroll 4
    for (int s = 0; s < sc; ++s) {
      const double qj = (double)qs[s * D + j];
#pragma unroll
      for (int k = 0; k < RPT; ++k) acc[k] = fma((double)qs[s * D + i0 + rg + k * NG], qj, acc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < RPT; ++k) MK[((int64_t)h * D + i0 + rg + k * NG) * D + j] = acc[k] / (double)M_s;
}

// ---------------------------------------------------------------- key basis
// w_k = (lambda_k / sum lambda)^p, applied after the projection.  M_K is
// positive semi-definite, so the sum of its (clamped) eigenvalues is its
// trace; a rounding-level negative eigenvalue gets weight 0.
SPR_DEV double eig_weight(double lam, double tot, double p) {
  const double x = tot > 0.0 ? fmax(lam, 0.0) / tot : 0.0;
  const double y = (p == 0.5) ? sqrt(x) : (p == 1.0 ? x : pow(x, p));
  return tot > 0.0 ? y : 0.0;
}

__global__ void k_eig_weights(const double* __restrict__ eigval, const double* __restrict__ trace, int d, int r,
                              double p, double* __restrict__ w) {
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  if (t < r) w[(int64_t)h * r + t] = eig_weight(eigval[(int64_t)h * d + t], trace[h], p);
}

// ---------------------------------------------------------------- k-means
// Centres start at rows floor((2g+1)n/(2G)) (k_centre_start below).

// fp16 parts of one metric-applied centre for the certified assignment
// (assign.hip): thread i < D of the block holds v = Cp[i]; exponent e with
// max|v| 2^-e in [128, 256), the parts of v 2^-e padded to lp_dims(D),
// ||v 2^-e|| rounded up and cn as float; also the transposed float64 copy.
template <int BLOCK>
SPR_DEV void write_centre_lp(double v, double cnv, int D, int h, int g, int G, const LpAssign& lp, double* red) {
  const int tid = threadIdx.x;
  const int64_t hg = (int64_t)h * G + g;
  if (tid < D) lp.cpt[((int64_t)h * D + tid) * G + g] = v;
  const double mx = block_max_f64<BLOCK>(tid < D ? fabs(v) : 0.0, red);
  const int e = mx > 0.0 ? ilogb(mx) - 7 : 0;
  const double sv = tid < D ? ldexp(v, -e) : 0.0;
  const double ss = block_sum_f64_waves<BLOCK>(sv * sv, red);
  const int DP = lp_dims(D);
  if (tid < DP) {
    uint16_t hi, lo;
    split_f16(sv, hi, lo);
    lp.ch[hg * DP + tid] = hi;
    lp.cl[hg * DP + tid] = lo;
  }
  if (tid == 0) {
    lp.ce[hg] = e;
    lp.cn32[hg] = (float)cnv;
    lp.cnrm[hg] = (float)sqrt(ss) * 1.0000002f;
  }
}

// Entry i of the metric image A c is the sum, in order, of metric_parts(D)
// partial sums over consecutive ranges of j (each from zero, j in order).
// Column i of the symmetric A is read (the same entries as row i), so the
// lanes read consecutive addresses; a part's loads are all issued at once.
SPR_DEV int metric_parts(int D) { return D > 64 ? 2 : 4; }
SPR_DEV double metric_part(const double* __restrict__ Ah, const double* c, int D, int i, int q) {
  const int NQ = metric_parts(D), L = (D + NQ - 1) / NQ, j0 = q * L, j1 = min(D, j0 + L);
  double s = 0.0;
  int j = j0;
  for (; j + 8 <= j1; j += 8) {
    double a8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a8[u] = Ah[(int64_t)(j + u) * D + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s = fma(a8[u], c[j + u], s);
  }
  for (; j < j1; ++j) s = fma(Ah[(int64_t)j * D + i], c[j], s);
  return s;
}

// The starting centre g = row floor((2g+1)n/(2G)) of X, written to C; its
// metric image Cp = A c (A the metric, or identity when A == nullptr);
// cn = c . Cp; and the centre's fp16 parts.  One block of 128 per (group,
// head); D <= 128.
template <int RM>
__global__ __launch_bounds__(128) void k_centre_start(const Rows64 X, int n, double* __restrict__ C,
                                                      const double* __restrict__ A, int D, int G,
                                                      double* __restrict__ Cp, double* __restrict__ cn, LpAssign lp) {
  const int h = blockIdx.y, g = blockIdx.x, i = threadIdx.x;
  __shared__ double c[128];
  __shared__ double red[128];
  const int64_t t = ((int64_t)2 * g + 1) * n / ((int64_t)2 * G);
  if (i < D) {
    const double x = X.at<RM>(h, n, D, t, i);
    C[((int64_t)h * G + g) * D + i] = x;
    c[i] = x;
  }
  __syncthreads();
  double v = 0.0;
  if (i < D) {
    if (A) {
      const int NQ = metric_parts(D);
      v = metric_part(A + (int64_t)h * D * D, c, D, i, 0);
      for (int q = 1; q < NQ; ++q) v += metric_part(A + (int64_t)h * D * D, c, D, i, q);
    } else {
      v = c[i];
    }
    Cp[((int64_t)h * G + g) * D + i] = v;
  }
  double s = block_sum_f64_waves<128>(i < D ? c[i] * v : 0.0, red);
  if (i == 0) cn[(int64_t)h * G + g] = s;
  write_centre_lp<128>(v, s, D, h, g, G, lp, red);
}

// ---------------------------------------------------------------- stable counting sort
// counts[h][c][g] = occurrences of label g in chunk c (kSortChunk labels per
// chunk) come from the assignment kernels.
// base[h][c][g] = off[g] + sum_{c' < c} counts[h][c'][g]; off = exclusive scan of totals.
// Integer sums: the result does not depend on how the chunks are split.
// Up to kSortOneBlock chunks per head, one block per head (k_sort_scan);
// above, two launches of S x H blocks (S slices of consecutive chunks per
// head; in a block, P = 1024 / G threads per group each take a contiguous
// part of the slice): k_sort_part writes every part's sums
// spart[h][s][q][g], k_sort_base forms the group totals, their exclusive
// scan and each part's start from them, then writes base over its part.
constexpr int kSortOneBlock = 511;
static int sort_slices(int nchunks) { return std::max(1, std::min(kSortSlices, nchunks / 16)); }

// One block per head: P = 1024 / G threads per group each take a contiguous
// range of chunks.
__global__ __launch_bounds__(1024) void k_sort_scan(const int32_t* __restrict__ counts, int G, int nchunks,
                                                    int32_t* __restrict__ base, int32_t* __restrict__ off) {
  __shared__ int part[1024];
  __shared__ int scan[kMaxGroups + 1];
  __shared__ int wsum[16];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int P = 1024 / G;
  const int g = tid % G, q = tid / G;
  const bool act = q < P;
  const int c0 = act ? (int)((int64_t)nchunks * q / P) : 0, c1 = act ? (int)((int64_t)nchunks * (q + 1) / P) : 0;
  const int32_t* cnt = counts + (int64_t)h * nchunks * G + g;
  constexpr int KF = 8;   // loads in flight per thread (32 measured no faster)
  int sum = 0;
  int c = c0;
  for (; c + KF <= c1; c += KF) {
    int v[KF];
#pragma unroll
    for (int u = 0; u < KF; ++u) v[u] = cnt[(int64_t)(c + u) * G];
#pragma unroll
    for (int u = 0; u < KF; ++u) sum += v[u];
  }
  for (; c < c1; ++c) sum += cnt[(int64_t)c * G];
  if (act) part[q * G + g] = sum;
  __syncthreads();
  // group totals, then an exclusive scan over the groups
  int gt = 0;
  if (tid < G)
    for (int qq = 0; qq < P; ++qq) gt += part[qq * G + tid];
  int all;
  const int ex = block_exclusive_scan<1024>(gt, wsum, &all);
  if (tid < G) scan[tid] = ex;
  if (tid == 0) scan[G] = all;
  __syncthreads();
  for (int gg = tid; gg <= G; gg += 1024) off[(int64_t)h * (G + 1) + gg] = scan[gg];
  if (!act) return;
  int run = scan[g];
  for (int qq = 0; qq < q; ++qq) run += part[qq * G + g];
  int32_t* bs = base + (int64_t)h * nchunks * G + g;
  c = c0;
  for (; c + KF <= c1; c += KF) {
    int v[KF];
#pragma unroll
    for (int u = 0; u < KF; ++u) v[u] = cnt[(int64_t)(c + u) * G];
#pragma unroll
    for (int u = 0; u < KF; ++u) { bs[(int64_t)(c + u) * G] = run; run += v[u]; }
  }
  for (; c < c1; ++c) { bs[(int64_t)c * G] = run; run += cnt[(int64_t)c * G]; }
}


SPR_DEV void sort_part_range(int nchunks, int S, int s, int P, int q, int& c0, int& c1) {
  const int s0 = (int)((int64_t)nchunks * s / S), s1 = (int)((int64_t)nchunks * (s + 1) / S);
  c0 = s0 + (int)((int64_t)(s1 - s0) * q / P);
  c1 = s0 + (int)((int64_t)(s1 - s0) * (q + 1) / P);
}

__global__ __launch_bounds__(1024) void k_sort_part(const int32_t* __restrict__ counts, int G, int nchunks,
                                                    int32_t* __restrict__ spart) {
  const int s = blockIdx.x, S = gridDim.x, h = blockIdx.y, tid = threadIdx.x;
  const int P = 1024 / G, g = tid % G, q = tid / G;
  if (q >= P) return;
  int c0, c1;
  sort_part_range(nchunks, S, s, P, q, c0, c1);
  const int32_t* cnt = counts + (int64_t)h * nchunks * G + g;
  constexpr int KF = 8;   // loads in flight per thread
  int sum = 0, c = c0;
  for (; c + KF <= c1; c += KF) {
    int v[KF];
#pragma unroll
    for (int u = 0; u < KF; ++u) v[u] = cnt[(int64_t)(c + u) * G];
#pragma unroll
    for (int u = 0; u < KF; ++u) sum += v[u];
  }
  for (; c < c1; ++c) sum += cnt[(int64_t)c * G];
  spart[((int64_t)h * S + s) * 1024 + q * G + g] = sum;
}

__global__ __launch_bounds__(1024) void k_sort_base(const int32_t* __restrict__ counts, int G, int nchunks,
                                                    const int32_t* __restrict__ spart, int32_t* __restrict__ base,
                                                    int32_t* __restrict__ off) {
  __shared__ int colt[1024], colp[1024], own[1024];
  __shared__ int start[kMaxGroups];
  __shared__ int wsum[16];
  const int s = blockIdx.x, S = gridDim.x, h = blockIdx.y, tid = threadIdx.x;
  const int P = 1024 / G, g = tid % G, q = tid / G;
  const int32_t* sp = spart + (int64_t)h * S * 1024;
  // thread (g, q): part q's sums over all slices and over the slices before
  // this one, and this slice's own part q; then the group totals and this
  // slice's start within each group
  if (q < P) {
    int t = 0, pr = 0;
#pragma unroll
    for (int ss = 0; ss < kSortSlices; ++ss)
      if (ss < S) {
        const int v = sp[ss * 1024 + q * G + g];
        t += v;
        pr += ss < s ? v : 0;
      }
    colt[tid] = t;
    colp[tid] = pr;
    own[tid] = sp[s * 1024 + q * G + g];
  }
  __syncthreads();
  int gt = 0, pre = 0;
  if (tid < G)
    for (int qq = 0; qq < P; ++qq) {
      gt += colt[qq * G + tid];
      pre += colp[qq * G + tid];
    }
  int all;
  const int ex = block_exclusive_scan<1024>(gt, wsum, &all);
  if (tid < G) start[tid] = ex + pre;
  if (s == 0) {
    if (tid < G) off[(int64_t)h * (G + 1) + tid] = ex;
    if (tid == 0) off[(int64_t)h * (G + 1) + G] = all;
  }
  __syncthreads();
  if (q >= P) return;
  int run = start[g];
  for (int qq = 0; qq < q; ++qq) run += own[qq * G + g];
  int c0, c1;
  sort_part_range(nchunks, S, s, P, q, c0, c1);
  const int32_t* cnt = counts + (int64_t)h * nchunks * G + g;
  int32_t* bs = base + (int64_t)h * nchunks * G + g;
  constexpr int KF = 8;
  int c = c0;
  for (; c + KF <= c1; c += KF) {
    int v[KF];
#pragma unroll
    for (int u = 0; u < KF; ++u) v[u] = cnt[(int64_t)(c + u) * G];
#pragma unroll
    for (int u = 0; u < KF; ++u) { bs[(int64_t)(c + u) * G] = run; run += v[u]; }
  }
  for (; c < c1; ++c) { bs[(int64_t)c * G] = run; run += cnt[(int64_t)c * G]; }
}

static void launch_sort_scan(const int32_t* counts, int H, int G, int nchunks, int32_t* spart, int32_t* base,
                             int32_t* off, hipStream_t st) {
  if (nchunks <= kSortOneBlock) {
    hipLaunchKernelGGL(k_sort_scan, dim3(H), dim3(1024), 0, st, counts, G, nchunks, base, off);
    return;
  }
  const dim3 grid(sort_slices(nchunks), H);
  hipLaunchKernelGGL(k_sort_part, grid, dim3(1024), 0, st, counts, G, nchunks, spart);
  hipLaunchKernelGGL(k_sort_base, grid, dim3(1024), 0, st, counts, G, nchunks, spart, base, off);
}

// perm[base + rank within chunk among equal labels] = t (stable).  The rank
// comes from bit-sliced ballots: per label bit b, the wave's mask of lanes
// whose label has bit b set; the lanes with a label equal to this lane's
// are the AND over b of that mask or its complement (and the valid lanes),
// so rank = the number of such lanes below this one, plus those of the
// chunk's first wave for a lane of the second.
__global__ __launch_bounds__(kSortChunk) void k_sort_scatter(const int32_t* __restrict__ labels, int n, int G,
                                                             int nchunks, const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ perm) {
  static_assert(kSortChunk == 128, "two waves per chunk");
  constexpr int NBITS = 10;   // labels below kMaxGroups = 2^10
  static_assert((1 << NBITS) >= kMaxGroups, "label bits");
  __shared__ uint64_t w0mask[NBITS + 1];   // the first wave's masks: valid lanes, then one per bit
  const int h = blockIdx.y, c = blockIdx.x, i = threadIdx.x, w = i >> 6, lane = i & 63;
  const int64_t t = (int64_t)c * kSortChunk + i;
  const bool ok = t < n;
  const int mine = ok ? labels[(int64_t)h * n + t] : 0;
  uint64_t eq = __ballot(ok), eq0 = 0;
  if (w == 0 && lane == 0) w0mask[0] = eq;
  for (int b = 0; b < NBITS && ((G - 1) >> b) != 0; ++b) {
    const bool bit = (mine >> b) & 1;
    const uint64_t m = __ballot(bit);
    eq &= bit ? m : ~m;
    if (w == 0 && lane == 0) w0mask[1 + b] = m;
  }
  __syncthreads();
  if (!ok) return;
  int rank = __popcll(eq & ((1ull << lane) - 1ull));
  if (w == 1) {
    eq0 = w0mask[0];
    for (int b = 0; b < NBITS && ((G - 1) >> b) != 0; ++b) eq0 &= ((mine >> b) & 1) ? w0mask[1 + b] : ~w0mask[1 + b];
    rank += __popcll(eq0);
  }
  perm[(int64_t)h * n + base[((int64_t)h * nchunks + c) * G + mine] + rank] = (int32_t)t;
}

// Segmented mean over the sorted order: C[g] = mean of X rows perm[off[g]..off[g+1]);
// an empty group keeps C[g] (keep_empty) or gets zeros.  Fixed summation order.
// Vector path (D a multiple of the 16-byte slice, 256 / (D / slice) whole
// rows per pass): thread (r, c) sums slice c of members r, r + R, ... in
// order, 8 rows in flight each, then the R partial sums in order.  Otherwise
// member slots s, s+S, ... per thread and element, then slots in order.
// With Cp given, the block also writes the centre's metric image Cp = A c (A
// the metric, or the identity when A is null) and cn = c . Cp, summed in the
// same order as k_centre_start (an empty kept centre keeps both).
// With LAB (n <= kSmallKmeansN) the block takes its members from the labels
// instead: it lists the points with label g in increasing order (the order
// of the stable sort) in LDS, so a Lloyd round needs no sort.
template <int RM, bool LAB = false>
__global__ __launch_bounds__(256) void k_segment_mean(const Rows64 X, int n, int D,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ off, int G,
                                                      double* __restrict__ C, int keep_empty,
                                                      const double* __restrict__ A = nullptr,
                                                      double* __restrict__ Cp = nullptr,
                                                      double* __restrict__ cn = nullptr, LpAssign lp = {},
                                                      const int32_t* __restrict__ labels = nullptr) {
  __shared__ double part[256];
  __shared__ double cm[128];
  __shared__ int32_t mlist[LAB ? kSmallKmeansN : 1];
  constexpr int kIdxChunk = 1024;
  __shared__ int32_t sidx[LAB ? 1 : kIdxChunk];
  __shared__ int wtot[4];
  const int h = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  int b, e;
  const int32_t* ph;
  if (LAB) {
    // wave w scans labels [w S, (w + 1) S), S <= 2048, all loads in flight:
    // match masks by ballot (kept in scalar registers), then each match's
    // slot from the waves before it and the set bits before it
    static_assert(kSmallKmeansN <= 4 * 32 * 64, "one pass of 32 wave-widths per wave");
    const int32_t* lh = labels + (int64_t)h * n;
    const int wv = tid >> 6, ln = tid & 63;
    const int S = (n + 255) / 256 * 64, t0 = wv * S, t1 = min(n, t0 + S);
    int lv[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int i = t0 + 64 * u + ln;
      lv[u] = i < t1 ? lh[i] : -1;
    }
    uint64_t bm[32];
    int c = 0;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      bm[u] = __ballot(lv[u] == g);
      c += __popcll(bm[u]);
    }
    if (ln == 0) wtot[wv] = c;
    __syncthreads();
    int base = 0;
    for (int u = 0; u < wv; ++u) base += wtot[u];
    const uint64_t below = (1ull << ln) - 1ull;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      if ((bm[u] >> ln) & 1ull) mlist[base + __popcll(bm[u] & below)] = t0 + 64 * u + ln;
      base += __popcll(bm[u]);
    }
    b = 0;
    e = (wtot[0] + wtot[1]) + (wtot[2] + wtot[3]);
    ph = mlist;
    __syncthreads();
  } else {
    const int32_t* offh = off + (int64_t)h * (G + 1);
    b = offh[g];
    e = offh[g + 1];
    ph = perm + (int64_t)h * n;
  }
  double* cg = C + ((int64_t)h * G + g) * D;
  if (e == b) {
    if (!keep_empty)
      for (int k = tid; k < D; k += 256) cg[k] = 0.0;
    return;
  }
  constexpr int VEC = RowVec<RM>::VEC;
  const int TPR = D / VEC;
  if (D % VEC == 0 && D <= 128 && 256 % TPR == 0) {
    __shared__ double pv[256 * VEC];   // [R][D] partial sums, R = 256 / TPR
    const int R = 256 / TPR, r = tid / TPR, c = tid % TPR;
    double acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0;
    // eight member rows in flight; past the end a slot reloads the first
    // member and is not added.  The member indices of the sorted order are
    // first staged in LDS, kIdxChunk at a time (all loads at once), so that
    // a row load waits for no global index load; kIdxChunk is a multiple of
    // R, so each thread still adds its members b + r + k R in order.
    for (int m0 = b; m0 < e; m0 += kIdxChunk) {
      const int m1 = min(e, m0 + kIdxChunk);
      const int32_t* ix = ph + m0;
      if (!LAB) {
        for (int k = tid; k < m1 - m0; k += 256) sidx[k] = ph[m0 + k];
        __syncthreads();
        ix = sidx;
      }
      for (int m = m0 + r; m < m1; m += 8 * R) {
        int32_t idx[8];
        double v[8][VEC];
#pragma unroll
        for (int u = 0; u < 8; ++u) idx[u] = ix[(m + u * R < m1 ? m + u * R : m0) - m0];
#pragma unroll
        for (int u = 0; u < 8; ++u) RowVec<RM>::load(X, h, n, D, idx[u], c * VEC, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (m + u * R < m1)
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] += v[u][i];
      }
      if (!LAB) __syncthreads();   // this chunk's indices are read before the next one lands
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) pv[r * D + c * VEC + i] = acc[i];
    __syncthreads();
    if (tid < D) {
      double sum = 0.0;
      for (int rr = 0; rr < R; ++rr) sum += pv[rr * D + tid];
      const double mean = sum / (double)(e - b);
      cg[tid] = mean;
      cm[tid] = mean;
    }
  } else
  for (int d0 = 0; d0 < D; d0 += 128) {
    const int Dc = min(128, D - d0);
    const int S = 256 / Dc;
    const int s = tid / Dc, k = tid % Dc;
    double acc = 0.0;
    if (s < S) {
      // members b+s, b+s+S, ... in order; loads issued 8 at a time
      int m = b + s;
      for (; m + 7 * S < e; m += 8 * S) {
        int32_t idx[8];
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) idx[u] = ph[m + u * S];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = X.at<RM>(h, n, D, idx[u], d0 + k);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      for (; m < e; m += S) acc += X.at<RM>(h, n, D, ph[m], d0 + k);
    }
    __syncthreads();
    part[tid] = acc;
    __syncthreads();
    if (tid < Dc) {
      double sum = 0.0;
      for (int ss = 0; ss < S; ++ss) sum += part[ss * Dc + tid];
      const double mean = sum / (double)(e - b);
      cg[d0 + tid] = mean;
      if (d0 + tid < 128) cm[d0 + tid] = mean;
    }
  }
  if (Cp == nullptr) return;   // uniform over the block
  __syncthreads();
  double v = 0.0;
  if (A) {
    // the parts of Cp = A c on every thread: (i, q) = (tid % 128, tid / 128)
    // for D > 64, (tid % 64, tid / 64) otherwise
    const int NQ = metric_parts(D), span = 256 / NQ, i = tid % span, q = tid / span;
    part[tid] = i < D ? metric_part(A + (int64_t)h * D * D, cm, D, i, q) : 0.0;   // tid = q span + i
    __syncthreads();
    if (tid < D) {
      v = part[tid];
      for (int qq = 1; qq < NQ; ++qq) v += part[qq * span + tid];
    }
    __syncthreads();   // part[] is reused below
  } else if (tid < D) {
    v = cm[tid];
  }
  if (tid < D) Cp[((int64_t)h * G + g) * D + tid] = v;
  // the same sum as in k_centre_start (the waves past D add zeros)
  const double cnv = block_sum_f64_waves<256>(tid < D ? cm[tid] * v : 0.0, part);
  if (tid == 0) cn[(int64_t)h * G + g] = cnv;
  write_centre_lp<256>(v, cnv, D, h, g, G, lp, part);
}

// ---------------------------------------------------------------- query-response metric
// mu_bar = mean of nonempty K/V centroids (equal weights); A = sum_g (mu_g - mu_bar)(mu_g - mu_bar)^T;
// gprime = number of nonempty groups.  A block computes 16 rows i for every
// column j; centroids pass through LDS 32 at a time; sums run over g in order.
// Entries (i, j) and (j, i) take the same fmas in the same order, so A is
// exactly symmetric (its readers may take a column for a row).
template <int D>
__global__ __launch_bounds__(128) void k_metric(const double* __restrict__ mu, const int32_t* __restrict__ off,
                                                int G, double* __restrict__ A, int32_t* __restrict__ gprime) {
  __shared__ double ms[kGramChunkRows][128];   // the live centroids of a chunk, in order
  __shared__ int slot[kGramChunkRows];
  __shared__ int s_nl;
  __shared__ double mbar[128];
  const int h = blockIdx.y, i0 = blockIdx.x * kGramTileRows, j = threadIdx.x;
  const int32_t* offh = off + (int64_t)h * (G + 1);
  const double* muh = mu + (int64_t)h * G * D;
  constexpr int RSTEP = 128 / D;
  const int k = j % D, rs0 = j / D;   // thread j stages column k of rows rs0 + r RSTEP
  // stage the live rows of chunk [g0, g0 + gc) compacted in order; returns their number
  auto stage = [&](int g0, int gc) {
    __syncthreads();
    if (j < 64) {
      const bool lv = j < gc && offh[g0 + j + 1] > offh[g0 + j];
      const uint64_t m = __ballot(lv);
      if (j < gc) slot[j] = lv ? __popcll(m & ((1ull << j) - 1ull)) : -1;
      if (j == 0) s_nl = __popcll(m);
    }
    double v[kGramChunkRows / RSTEP];
#pragma unroll
    for (int r = 0; r < kGramChunkRows / RSTEP; ++r) {   // all loads in flight before the stores
      const int gg = min(rs0 + r * RSTEP, gc - 1);
      v[r] = muh[(int64_t)(g0 + gg) * D + k];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kGramChunkRows / RSTEP; ++r) {
      const int gg = rs0 + r * RSTEP;
      if (gg < gc && slot[gg] >= 0) ms[slot[gg]][k] = v[r];
    }
    __syncthreads();
    return s_nl;
  };
  int cnt = 0;
  double sum = 0.0;
  for (int g0 = 0; g0 < G; g0 += kGramChunkRows) {
    const int nl = stage(g0, min(kGramChunkRows, G - g0));
    cnt += nl;
    if (j < D)
      for (int gg = 0; gg < nl; ++gg) sum += ms[gg][j];
  }
  if (j < D) mbar[j] = sum / (double)cnt;
  __syncthreads();
  const double mj = j < D ? mbar[j] : 0.0;
  double mi[kGramTileRows], acc[kGramTileRows];
#pragma unroll
  for (int u = 0; u < kGramTileRows; ++u) { acc[u] = 0.0; mi[u] = mbar[i0 + u]; }
  for (int g0 = 0; g0 < G; g0 += kGramChunkRows) {
    const int nl = stage(g0, min(kGramChunkRows, G - g0));
    if (j < D)
#pragma unroll 2
      for (int gg = 0; gg < nl; ++gg) {
        const double bj = ms[gg][j] - mj;
#pragma unroll
        for (int u = 0; u < kGramTileRows; ++u) acc[u] = fma(ms[gg][i0 + u] - mi[u], bj, acc[u]);
      }
  }
  if (j >= D) return;
#pragma unroll
  for (int u = 0; u < kGramTileRows; ++u) A[((int64_t)h * D + i0 + u) * D + j] = acc[u];
  if (blockIdx.x == 0 && j == 0) gprime[h] = cnt;
}

// ---------------------------------------------------------------- row-tile float64 GEMM (MFMA)
// One kernel for the point-by-matrix products of the partition, each
// Y = X B^T with X = points x D and B = columns x D (columns <= 128), on
// the float64 matrix cores (v_mfma_f64_16x16x4_f64).  Block tile 64 points x
// 128 columns, four waves of 32 x 64 (2 x 4 MFMA blocks), D streamed through
// LDS 16 at a time.  MFMA f64 16x16x4 lane layout: A lane l = (row l%16,
// k l/16); B lane l = (column l%16, k l/16); D lane l register i = (row
// 4i + l/16, column l%16).
//  RG_QUAD1:  B = A, X = raw queries with row scales s, rows u - ubar_{label};
//             out = e^T A e, the squared distance of a query to its group
//             centre (the semantic baseline: A = I, s = 1).
//  RG_PROJ:   B = leading eigenvectors of M_K (one per row), X = raw keys;
//             Z[t][k] = (k_t . u_k) w_k, the eigen-weighted key coordinates
//             (r_k > 32; smaller ranks take k_proj_keys_mfma).
enum RowGemmMode { RG_QUAD1 = 0, RG_PROJ = 1 };
constexpr int RG_P = 64, RG_C = 128, RG_K = 16;
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int MODE, typename T>
SPR_DEV double rg_load_x(const T* Xh, int64_t t, int D, int k, const int32_t* lab, const double* cen, int G,
                         int h, const double* rs) {
  double v = load_f64(Xh, t * D + k);
  if (MODE == RG_QUAD1) v = v * rs[t] - cen[((int64_t)h * G + lab[t]) * D + k];
  return v;
}

template <int MODE, typename T>
__global__ __launch_bounds__(256) void k_rowgemm(const T* __restrict__ X, int n, int D,
                                                 const double* __restrict__ B, int ncols, int64_t bstride,
                                                 const double* __restrict__ cn,
                                                 const int32_t* __restrict__ lab_in,
                                                 const double* __restrict__ centres, int G,
                                                 double* __restrict__ out_vec, double* __restrict__ out_scalar,
                                                 const double* __restrict__ rowscale) {
  __shared__ double Xs[2][RG_K][RG_P + 1];
  __shared__ double Bs[2][RG_K][RG_C + 1];
  __shared__ double redv[2][RG_P];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;        // wave tile: rows 32 wr.., columns 64 wc..
  const int l16 = lane & 15, lq = lane >> 4;
  const int64_t p0 = (int64_t)blockIdx.x * RG_P;
  const T* Xh = X + (int64_t)h * n * D;
  const double* Bh = B + (int64_t)h * bstride;
  const int32_t* labh = MODE == RG_QUAD1 ? lab_in + (int64_t)h * n : nullptr;
  const double* rsh = MODE == RG_QUAD1 ? rowscale + (int64_t)h * n : nullptr;
  f64x4 acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f64x4{0.0, 0.0, 0.0, 0.0};
  // staging: thread owns 4 consecutive k of one point (xp = tid / 4) and 8 consecutive
  // k of one column (bc = tid / 2); registers hold the next chunk while this one runs
  const int xp = tid >> 2, xk = (tid & 3) * 4;
  const int bcol = tid >> 1, bk = (tid & 1) * 8;
  const int64_t xt = p0 + xp;
  double xr[4], br[8];
  const int nk = (D + RG_K - 1) / RG_K;
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + xk + j;
      xr[j] = (k < D && xt < n) ? rg_load_x<MODE>(Xh, xt, D, k, labh, centres, G, h, rsh) : 0.0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + bk + j;
      br[j] = (k < D && bcol < ncols) ? Bh[(int64_t)bcol * D + k] : 0.0;
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) Xs[buf][xk + j][xp] = xr[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) Bs[buf][bk + j][bcol] = br[j];
  };
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    const bool more = kc + 1 < nk;
    if (more) load_chunk((kc + 1) * RG_K);
#pragma unroll
    for (int ks = 0; ks < RG_K; ks += 4) {
      double af[2], bf[4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) af[rb] = Xs[buf][ks + lq][32 * wr + 16 * rb + l16];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) bf[cb] = Bs[buf][ks + lq][64 * wc + 16 * cb + l16];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[rb], bf[cb], acc[rb][cb], 0, 0, 0);
    }
    if (more) store_chunk(buf ^ 1);
    __syncthreads();
  }
  if (MODE == RG_PROJ) {
    // cn carries the eigen weights w_k; ncols = r_k output columns per point
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = 64 * wc + 16 * cb + l16;
      if (col >= ncols) continue;
      const double w = cn[(int64_t)h * ncols + col];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t t = p0 + 32 * wr + 16 * rb + 4 * i + lq;
          if (t < n) out_vec[((int64_t)h * n + t) * ncols + col] = acc[rb][cb][i] * w;
        }
    }
    return;
  }
  // quadratic form: sum over columns of x_col * (x^T A)_col; ncols = D <= 128
  double part[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[rb][i] = 0.0;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int col = 64 * wc + 16 * cb + l16;
    if (col >= ncols) continue;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = p0 + 32 * wr + 16 * rb + 4 * i + lq;
        const double x = t < n ? rg_load_x<MODE>(Xh, t, D, col, labh, centres, G, h, rsh) : 0.0;
        part[rb][i] = fma(x, acc[rb][cb][i], part[rb][i]);
      }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double v = part[rb][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 16);
      if (l16 == 0) redv[wc][32 * wr + 16 * rb + 4 * i + lq] = v;
    }
  __syncthreads();
  if (tid < RG_P) {
    // a squared distance: rounding can leave an exact zero slightly negative
    const int64_t t = p0 + tid;
    if (t < n) out_scalar[(int64_t)h * n + t] = fmax(redv[0][tid] + redv[1][tid], 0.0);
  }
}

template <int MODE, typename T>
static void launch_rowgemm(dim3 grid, hipStream_t st, const T* X, int n, int D, const double* B, int ncols,
                           int64_t bstride, const double* cn, const int32_t* lab_in, const double* centres, int G,
                           double* out_vec, double* out_scalar, const double* rowscale = nullptr) {
  hipLaunchKernelGGL((k_rowgemm<MODE, T>), grid, dim3(256), 0, st, X, n, D, B, ncols, bstride, cn, lab_in, centres,
                     G, out_vec, out_scalar, rowscale);
}

// ---------------------------------------------------------------- query row scales
// s_t = sqrt(G' / (q_t^T A q_t)) (0 when the form is 0) for every raw query,
// with q^T A q = 2 q^T U q, U the upper triangle of the symmetric A and its
// diagonal halved (A = U + U^T).  A workgroup stages U in LDS once and then
// streams 16-query tiles, one per wave at a time, on the float64 matrix cores
// as the transposed product (q U)^T = U^T q^T.  With the f64 16x16x4 layout
//   A (U^T): lane l = (column position p = l % 16, k slot l / 16),
//   B (q^T): lane l = (query l % 16, k slot l / 16),
//   D:       lane l, register i = (column position 4 i + l / 16, query l % 16),
// step (c, m) of column block j takes k = 16 c + 4 (l / 16) + m, and column
// position p of block j is column 16 j + 4 (p % 4) + p / 4.  Lane l of the
// result then holds (q U)[query][16 j + 4 (l / 16) + i], the same entries of
// q that it fed in steps (c = j, m = i), so the form needs 32 fmas per lane
// and two shuffles over the k slots, no data movement.  Block j has nonzero
// k-chunks c <= j only (36 of 64 at D = 128).  U sits in LDS in lane order,
// one 64-entry run per (j, c <= j, m), so each operand read is 512
// contiguous bytes.
template <int D>
constexpr int qscale_runs() { return 4 * (D / 16) * (D / 16 + 1) / 2; }
template <int D>
constexpr size_t qscale_lds() { return (size_t)qscale_runs<D>() * 64 * sizeof(double); }

// Entries 16 c + e0 .. + 3 of one query row for every chunk c, as loaded
// (bf16 words or floats; zeros past the last row), converted on use.
template <typename T, int NB>
struct QRaw {
  typedef typename std::conditional<sizeof(T) == 2, uint2, float4>::type W;
  W w[NB];
  SPR_DEV void load(const T* Q, int h, int n, int D, int64_t row, int e0) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if (row < n) w[c] = *reinterpret_cast<const W*>(Q + ((int64_t)h * n + row) * D + 16 * c + e0);
      else w[c] = {};
    }
  }
  SPR_DEV void get(int c, double (&v)[4]) const {
    if constexpr (sizeof(T) == 2) {
      v[0] = (double)__uint_as_float(w[c].x << 16); v[1] = (double)__uint_as_float(w[c].x & 0xffff0000u);
      v[2] = (double)__uint_as_float(w[c].y << 16); v[3] = (double)__uint_as_float(w[c].y & 0xffff0000u);
    } else {
      v[0] = w[c].x; v[1] = w[c].y; v[2] = w[c].z; v[3] = w[c].w;
    }
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_query_scale(const T* __restrict__ Q, const double* __restrict__ A,
                                                         const int32_t* __restrict__ gprime, int n,
                                                         double* __restrict__ qscale) {
  constexpr int NB = D / 16;
  extern __shared__ double su[];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, ks = lane >> 4;
  const double* Ah = A + (int64_t)h * D * D;
  // run r = 4 (j (j + 1) / 2 + c) + m, entry ll of the run = A-operand lane ll
  for (int e = tid; e < qscale_runs<D>() * 64; e += 256) {
    const int run = e >> 6, ll = e & 63, m = run & 3, jc = run >> 2;
    int j = 0;
    while ((j + 1) * (j + 2) / 2 <= jc) ++j;
    const int c = jc - j * (j + 1) / 2, pp = ll & 15;
    const int k = 16 * c + 4 * (ll >> 4) + m, col = 16 * j + 4 * (pp & 3) + (pp >> 2);
    const double a = Ah[(int64_t)k * D + col];
    su[e] = k < col ? a : (k == col ? 0.5 * a : 0.0);
  }
  __syncthreads();
  const double gp = (double)gprime[h];
  const int64_t ntiles = ((int64_t)n + 15) / 16, tstride = (int64_t)gridDim.x * 4;
  // the raw entries of the next tile are loaded while this one is multiplied
  QRaw<T, NB> nxt;
  int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  if (tile < ntiles) nxt.load(Q, h, n, D, tile * 16 + l16, 4 * ks);
  for (; tile < ntiles; tile += tstride) {
    const QRaw<T, NB> cur = nxt;
    if (tile + tstride < ntiles) nxt.load(Q, h, n, D, (tile + tstride) * 16 + l16, 4 * ks);
    const int64_t row = tile * 16 + l16;
    // chunk c feeds blocks j >= c; block c is complete after it, and its
    // entries of q are the four this lane has just fed
    f64x4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
    double form = 0.0;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      // keeps this chunk's operand reads in it (hoisted all at once they
      // would need 2 D^2 / 64 registers)
      asm volatile("" ::: "memory");
      double x[4];
      cur.get(c, x);
#pragma unroll
      for (int j = c; j < NB; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(su[(4 * (j * (j + 1) / 2 + c) + m) * 64 + lane], x[m],
                                                        acc[j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) form = fma(x[i], acc[c][i], form);
    }
    form += __shfl_xor(form, 16);
    form += __shfl_xor(form, 32);
    form *= 2.0;
    if (ks == 0 && row < n) qscale[(int64_t)h * n + row] = form > 0.0 ? sqrt(gp / form) : 0.0;
  }
}

// ---------------------------------------------------------------- permutation gather
// dst[h][slot] = src[h][perm[h][slot]], rows of d elements moved as 16-byte
// vectors; blockIdx.z picks the tensor (Q with the query permutation, K and
// V with the K/V permutation), so one launch moves all three.
template <typename T>
__global__ __launch_bounds__(256) void k_gather_rows(const T* __restrict__ Q, const T* __restrict__ K,
                                                     const T* __restrict__ V, const int32_t* __restrict__ q_perm,
                                                     const int32_t* __restrict__ kv_perm, int n, int d,
                                                     T* __restrict__ Qp, T* __restrict__ Kp, T* __restrict__ Vp) {
  const int h = blockIdx.y, z = blockIdx.z;
  const T* src = z == 0 ? Q : (z == 1 ? K : V);
  const int32_t* perm = z == 0 ? q_perm : kv_perm;
  T* dst = z == 0 ? Qp : (z == 1 ? Kp : Vp);
  const int vec_per_row = d * (int)sizeof(T) / 16;
  const int rows_per_block = 256 / vec_per_row;
  const int r = threadIdx.x / vec_per_row, v = threadIdx.x % vec_per_row;
  const int64_t slot = (int64_t)blockIdx.x * rows_per_block + r;
  if (slot >= n) return;
  const int64_t t = perm[(int64_t)h * n + slot];
  const uint4* sp = reinterpret_cast<const uint4*>(src + ((int64_t)h * n + t) * d);
  uint4* o = reinterpret_cast<uint4*>(dst + ((int64_t)h * n + slot) * d);
  o[v] = sp[v];
}

// ---------------------------------------------------------------- key projection
// Z[t][k] = (sum_i K[t][i] u_k[i]) w_k for the r leading eigenvectors.
template <typename T>
SPR_DEV void load8_f64(const T* p, double (&v)[8]) {   // 8 elements from a 16-byte aligned p
  if (sizeof(T) == 2) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = (double)__uint_as_float((i & 1) ? (wd[i >> 1] & 0xffff0000u) : (wd[i >> 1] << 16));
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// For r <= 16 NB (NB = 1, 2), D = 64 or 128, on the float64 matrix cores:
// a wave takes 16 keys at a time.  With the f64 16x16x4 layout, lane l
// feeds key l % 16 and, in step s, dim qS + s of its quarter q = l / 16
// (S = D / 4), and holds U[qS + s][16 b + l % 16] for every step s and
// column block b in registers (loaded once per wave), so each dot product
// runs as four interleaved partial sums of S dims: the same products, summed
// in another order.  Keys past n feed zeros and are not stored.
template <typename T, int D, int NB>
__global__ __launch_bounds__(256) void k_proj_keys_mfma(const T* __restrict__ K, const double* __restrict__ eigvec,
                                                        const double* __restrict__ eigval,
                                                        const double* __restrict__ trace, double p, int n, int r,
                                                        double* __restrict__ Z) {
  constexpr int S = D / 4;
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  const int h = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, q = lane >> 4;
  double u[NB][S], w[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int k = 16 * b + col;
    w[b] = k < r ? eig_weight(eigval[(int64_t)h * D + k], trace[h], p) : 0.0;
#pragma unroll
    for (int s = 0; s < S; ++s) u[b][s] = k < r ? eigvec[((int64_t)h * D + k) * D + q * S + s] : 0.0;
  }
  const int64_t groups = ((int64_t)n + 15) / 16;
  for (int64_t kg = (int64_t)blockIdx.x * 4 + wave; kg < groups; kg += (int64_t)gridDim.x * 4) {
    const int64_t key = kg * 16 + col;
    double x[S];
    if (key < n) {
      const T* row = K + ((int64_t)h * n + key) * D + q * S;
#pragma unroll
      for (int s8 = 0; s8 < S; s8 += 8) {
        double v8[8];
        load8_f64(row + s8, v8);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[s8 + i] = v8[i];
      }
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) x[s] = 0.0;
    }
    f64x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(x[s], u[b][s], acc[b], 0, 0, 0);
    // D lane l, register i: key 4 i + q of the group, column 16 b + l % 16
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t kr = kg * 16 + 4 * i + q;
        const int kc = 16 * b + col;
        if (kr < n && kc < r) Z[((int64_t)h * n + kr) * r + kc] = acc[b][i] * w[b];
      }
  }
}

// Squared distance of each query to its centre in query-response
// coordinates, d_t = (u - c)^T A (u - c) with u = s q, from the expanded
// form u^T A u - 2 u . Cp_c + cn_c: u^T A u = s^2 q^T A q = G' by the choice
// of s (0 for a zero form), Cp_c = A c and cn_c = c . Cp_c are the centre's
// metric image and norm from the last Lloyd update -- d multiply-adds per
// query instead of d^2.  Where the three terms cancel to below 2^-10 of
// their magnitudes (a query very close to its centre, e.g. duplicate rows),
// the expanded form could lose more than 2^-40 of the result, so the query
// is listed and k_qdist_direct computes (u - c)^T A (u - c) instead.
// d / 8 lanes per query, each with one 16-byte load of the query row (8 dims).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_qdist(const T* __restrict__ Q, const double* __restrict__ qscale,
                                               const int32_t* __restrict__ lab, const double* __restrict__ Cp,
                                               const double* __restrict__ cn, const int32_t* __restrict__ gprime,
                                               int n, int G, double* __restrict__ qdist,
                                               int32_t* __restrict__ list, int32_t* __restrict__ cnt) {
  constexpr int LPQ = D / 8, QPB = 256 / LPQ;   // lanes per query, queries per block
  const int h = blockIdx.y, j = threadIdx.x % LPQ;
  const int64_t t = (int64_t)blockIdx.x * QPB + threadIdx.x / LPQ;
  const bool ok = t < n;
  const int64_t row = (int64_t)h * n + (ok ? t : 0);
  const int c = lab[row];
  const double* cp = Cp + ((int64_t)h * G + c) * D + 8 * j;
  double qv[8];
  load8_f64(Q + row * D + 8 * j, qv);
  double dot = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) dot = fma(qv[i], cp[i], dot);
#pragma unroll
  for (int o = LPQ / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, LPQ);
  if (!ok || j != 0) return;
  const double s = qscale[row], cnc = cn[(int64_t)h * G + c];
  const double uau = s > 0.0 ? (double)gprime[h] : 0.0;
  const double x = -2.0 * s * dot;
  const double v = (uau + x) + cnc;
  const double mag = uau + fabs(x) + fabs(cnc);
  if (v > 0x1p-10 * mag) {
    qdist[row] = v;
  } else {
    const int w = atomicAdd(&cnt[h], 1);
    list[(int64_t)h * n + w] = (int32_t)t;
  }
}

// The direct form for the listed queries: one block per query, thread i
// computes (A e)_i over j in order, e = s q - c; then e . (A e) in a fixed
// tree.  (Every call on a block of 128 threads; d <= 128.)
template <typename T>
__global__ __launch_bounds__(128) void k_qdist_direct(const T* __restrict__ Q, const double* __restrict__ qscale,
                                                      const int32_t* __restrict__ lab, const double* __restrict__ C,
                                                      const double* __restrict__ A, int n, int d, int G,
                                                      const int32_t* __restrict__ list,
                                                      const int32_t* __restrict__ cnt, double* __restrict__ qdist) {
  __shared__ double e[128];
  __shared__ double red[128];
  const int h = blockIdx.y, i = threadIdx.x;
  const int total = cnt[h];
  const double* Ah = A + (int64_t)h * d * d;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int64_t row = (int64_t)h * n + list[(int64_t)h * n + w];
    const int c = lab[row];
    __syncthreads();
    if (i < d) e[i] = load_f64(Q + row * d, i) * qscale[row] - C[((int64_t)h * G + c) * d + i];
    __syncthreads();
    double ae = 0.0;
    if (i < d)
      for (int j = 0; j < d; ++j) ae = fma(Ah[(int64_t)i * d + j], e[j], ae);
    const double f = block_sum_f64<128>(i < d ? e[i] * ae : 0.0, red);
    if (i == 0) qdist[row] = fmax(f, 0.0);
  }
}

__global__ void k_zero_i32(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Warm start: the previous call's labels (clamped into [0, G), written back)
// counted per 128-point chunk in the layout the assignment kernels use, so
// the counting sort and the segment means turn them into starting centres.
__global__ __launch_bounds__(kSortChunk) void k_label_hist(int32_t* __restrict__ labels, int n, int G,
                                                          int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxGroups];
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  for (int g = tid; g < G; g += kSortChunk) hist[g] = 0;
  __syncthreads();
  const int64_t t = (int64_t)c * kSortChunk + tid;
  if (t < n) {
    int32_t* lp = labels + (int64_t)h * n + t;
    const int lab = min(max(*lp, 0), G - 1);
    *lp = lab;
    atomicAdd(&hist[lab], 1);
  }
  __syncthreads();
  int32_t* out = counts + ((int64_t)h * gridDim.x + c) * G;
  for (int g = tid; g < G; g += kSortChunk) out[g] = hist[g];
}

// identity metric and unit row scales for the semantic baseline's distances
__global__ void k_identity_unit(double* __restrict__ A, int d, double* __restrict__ s, int n) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)d * d) A[(int64_t)h * d * d + i] = (i / d == i % d) ? 1.0 : 0.0;
  if (i < n) s[(int64_t)h * n + i] = 1.0;
}

// ================================================================ launchers
template <typename T>
static hipError_t partition_impl(const PartitionArgs& a) {
  const int H = a.H, N = a.N, d = a.d, G_k = a.G_k, G_q = a.G_q, r = a.r_k;
  const T* Q = static_cast<const T*>(a.Q);
  const T* K = static_cast<const T*>(a.K);
  const T* V = static_cast<const T*>(a.V);
  hipStream_t st = a.stream;
  const int nchunks = (N + kSortChunk - 1) / kSortChunk;
  const dim3 tileGrid((N + 63) / 64, H);

  const int bf = std::is_same<T, bf16_t>::value ? 1 : 0;
  constexpr int RAW = std::is_same<T, bf16_t>::value ? ROWS_BF16 : ROWS_F32;
  // --- paired K/V k-means (B.1); V inherits the key's label
  auto kmeans = [&](const Rows64& X, int D, int G, int iters, const double* metric, int32_t* labels,
                    int32_t* perm, int32_t* off) {
    const LpAssign& lp = a.ws.lp;
    launch_lp_points(X, H, N, D, lp, st);
#define SPR_CALL(M)                                                                                      \
  hipLaunchKernelGGL((k_centre_start<M>), dim3(G, H), dim3(128), 0, st, X, N, a.ws.cent, metric, D, G, a.ws.centp, \
                     a.ws.cnorm, lp)
    SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
    if (a.warm) {
      // starting centres: the means of the previous labels' groups (an empty
      // group keeps its stride row)
      hipLaunchKernelGGL(k_label_hist, dim3(nchunks, H), dim3(kSortChunk), 0, st, labels, N, G, a.ws.counts);
      launch_sort_scan(a.ws.counts, H, G, nchunks, a.ws.sortpart, a.ws.base, off, st);
      hipLaunchKernelGGL(k_sort_scatter, dim3(nchunks, H), dim3(kSortChunk), 0, st, labels, N, G, nchunks,
                         a.ws.base, perm);
#define SPR_CALL(M) hipLaunchKernelGGL((k_segment_mean<M>), dim3(G, H), dim3(256), 0, st, X, N, D, perm, off, G, \
                                    a.ws.cent, 1, metric, a.ws.centp, a.ws.cnorm, lp)
      SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
    }
    // small n: the rounds take the means from the labels directly and the
    // stable sort runs once, on the last labels
    const bool from_labels = N <= kSmallKmeansN;
    for (int it = 0; it < iters; ++it) {
      launch_assign_lp(X, a.ws.centp, a.ws.cnorm, metric ? a.ws.gprime : nullptr, H, N, D, G, lp, labels, a.ws.counts,
                       st);
      if (from_labels) {
#define SPR_CALL(M) hipLaunchKernelGGL((k_segment_mean<M, true>), dim3(G, H), dim3(256), 0, st, X, N, D, nullptr, \
                                    nullptr, G, a.ws.cent, 1, metric, a.ws.centp, a.ws.cnorm, lp, labels)
        SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
        continue;
      }
      launch_sort_scan(a.ws.counts, H, G, nchunks, a.ws.sortpart, a.ws.base, off, st);
      hipLaunchKernelGGL(k_sort_scatter, dim3(nchunks, H), dim3(kSortChunk), 0, st, labels, N, G, nchunks,
                         a.ws.base, perm);
#define SPR_CALL(M) hipLaunchKernelGGL((k_segment_mean<M>), dim3(G, H), dim3(256), 0, st, X, N, D, perm, off, G, \
                                    a.ws.cent, 1, metric, a.ws.centp, a.ws.cnorm, lp)
      SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
    }
    if (from_labels) {
      launch_sort_scan(a.ws.counts, H, G, nchunks, a.ws.sortpart, a.ws.base, off, st);
      hipLaunchKernelGGL(k_sort_scatter, dim3(nchunks, H), dim3(kSortChunk), 0, st, labels, N, G, nchunks,
                         a.ws.base, perm);
    }
  };
  if (a.semantic) {
    // the pages' semantic baseline: k-means on the raw keys and the raw
    // queries (Euclidean: identity metric, unit row scales for the distances)
    kmeans(Rows64{nullptr, K, nullptr, bf}, d, G_k, a.iters_kv, nullptr, a.kv_label, a.kv_perm, a.kv_off);
    hipLaunchKernelGGL((k_segment_mean<RAW>), dim3(G_k, H), dim3(256), 0, st, Rows64{nullptr, K, nullptr, bf}, N, d,
                       a.kv_perm, a.kv_off, G_k, a.kv_centroid, 0, nullptr, nullptr, nullptr, LpAssign{});
    kmeans(Rows64{nullptr, Q, nullptr, bf}, d, G_q, a.iters_q, nullptr, a.q_label, a.q_perm, a.q_off);
    const int64_t span = std::max<int64_t>((int64_t)d * d, N);
    hipLaunchKernelGGL(k_identity_unit, dim3((unsigned)((span + 255) / 256), H), dim3(256), 0, st, a.ws.metric, d,
                       a.ws.qscale, N);
  } else {
  // --- key-response coordinates (B.1)
  if (d == 128)
    hipLaunchKernelGGL((k_gram_mk<T, 128>), dim3(128 / kGramRows, H), dim3(256), 0, st, Q, N, a.M_s, a.ws.mk);
  else
    hipLaunchKernelGGL((k_gram_mk<T, 64>), dim3(64 / kGramRows, H), dim3(256), 0, st, Q, N, a.M_s, a.ws.mk);
  launch_sym_eig_top(a.ws.mk, H, d, r, a.ws.eigval, a.ws.eigvec, a.ws.mtrace, a.ws.eigscr, st);
  // eigen weights: computed by the projection's blocks (r <= 32), or once for the row-GEMM projection
  if (r <= 32) {
    // 16 keys per wave and pass, four waves per block, up to 256 blocks per head
    const unsigned gx = (unsigned)std::min<int64_t>(256, ((int64_t)N + 63) / 64);
    const dim3 pg(gx, H);
#define SPR_PROJ(DD, NBB) \
  hipLaunchKernelGGL((k_proj_keys_mfma<T, DD, NBB>), pg, dim3(256), 0, st, K, a.ws.eigvec, a.ws.eigval, a.ws.mtrace, \
                     a.eig_power, N, r, a.ws.Z)
    if (d == 128) {
      if (r <= 16) SPR_PROJ(128, 1);
      else SPR_PROJ(128, 2);
    } else {
      if (r <= 16) SPR_PROJ(64, 1);
      else SPR_PROJ(64, 2);
    }
#undef SPR_PROJ
  } else {
    hipLaunchKernelGGL(k_eig_weights, dim3(H), dim3(128), 0, st, a.ws.eigval, a.ws.mtrace, d, r, a.eig_power,
                       a.ws.wk);
    launch_rowgemm<RG_PROJ, T>(tileGrid, st, K, N, d, a.ws.eigvec, r, (int64_t)d * d, a.ws.wk, nullptr, nullptr, 0,
                               a.ws.Z, nullptr);
  }
  // --- paired K/V k-means on Z (B.1); V inherits the key's label
  kmeans(Rows64{a.ws.Z, nullptr, nullptr, 0}, r, G_k, a.iters_kv, nullptr, a.kv_label, a.kv_perm, a.kv_off);
  hipLaunchKernelGGL((k_segment_mean<RAW>), dim3(G_k, H), dim3(256), 0, st, Rows64{nullptr, K, nullptr, bf}, N, d,
                     a.kv_perm, a.kv_off, G_k, a.kv_centroid, 0, nullptr, nullptr, nullptr, LpAssign{});
  // --- query-response coordinates (B.2, C.1) and query k-means
  if (d == 128)
    hipLaunchKernelGGL(k_metric<128>, dim3(128 / kGramTileRows, H), dim3(128), 0, st, a.kv_centroid, a.kv_off, G_k,
                       a.ws.metric, a.ws.gprime);
  else
    hipLaunchKernelGGL(k_metric<64>, dim3(64 / kGramTileRows, H), dim3(128), 0, st, a.kv_centroid, a.kv_off, G_k,
                       a.ws.metric, a.ws.gprime);
  {
    // about 2 workgroups per CU over all heads, at least ~8 tiles per wave
    const int64_t ntiles = ((int64_t)N + 15) / 16;
    const unsigned gq = (unsigned)std::max<int64_t>(1, std::min<int64_t>((ntiles + 31) / 32, std::max(1, 512 / H)));
    if (d == 128)
      hipLaunchKernelGGL((k_query_scale<T, 128>), dim3(gq, H), dim3(256), qscale_lds<128>(), st, Q, a.ws.metric,
                         a.ws.gprime, N, a.ws.qscale);
    else
      hipLaunchKernelGGL((k_query_scale<T, 64>), dim3(gq, H), dim3(256), qscale_lds<64>(), st, Q, a.ws.metric,
                         a.ws.gprime, N, a.ws.qscale);
  }
  kmeans(Rows64{nullptr, Q, a.ws.qscale, bf}, d, G_q, a.iters_q, a.ws.metric, a.q_label, a.q_perm, a.q_off);
  }
  // squared distance of each query to its centre
  if (a.semantic) {
    // (raw query space: the identity metric and unit scales, direct form)
    launch_rowgemm<RG_QUAD1, T>(tileGrid, st, Q, N, d, a.ws.metric, d, (int64_t)d * d, nullptr, a.q_label,
                                a.ws.cent, G_q, nullptr, a.q_dist, a.ws.qscale);
  } else {
    const LpAssign& lp = a.ws.lp;
    hipLaunchKernelGGL(k_zero_i32, dim3((H + 255) / 256), dim3(256), 0, st, lp.cnt, H);
    if (d == 128)
      hipLaunchKernelGGL((k_qdist<T, 128>), dim3((N + 15) / 16, H), dim3(256), 0, st, Q, a.ws.qscale, a.q_label,
                         a.ws.centp, a.ws.cnorm, a.ws.gprime, N, G_q, a.q_dist, lp.list, lp.cnt);
    else
      hipLaunchKernelGGL((k_qdist<T, 64>), dim3((N + 31) / 32, H), dim3(256), 0, st, Q, a.ws.qscale, a.q_label,
                         a.ws.centp, a.ws.cnorm, a.ws.gprime, N, G_q, a.q_dist, lp.list, lp.cnt);
    hipLaunchKernelGGL(k_qdist_direct<T>, dim3(64, H), dim3(128), 0, st, Q, a.ws.qscale, a.q_label, a.ws.cent,
                       a.ws.metric, N, d, G_q, lp.list, lp.cnt, a.q_dist);
  }
  hipLaunchKernelGGL((k_segment_mean<RAW>), dim3(G_q, H), dim3(256), 0, st, Rows64{nullptr, Q, nullptr, bf}, N, d,
                     a.q_perm, a.q_off, G_q, a.q_centroid, 0, nullptr, nullptr, nullptr, LpAssign{});
  // --- group-major layouts (s4 Sparse Execution)
  {
    const int rows_per_block = 256 / (d * (int)sizeof(T) / 16);
    const dim3 g((N + rows_per_block - 1) / rows_per_block, H, 3);
    hipLaunchKernelGGL(k_gather_rows<T>, g, dim3(256), 0, st, Q, K, V, a.q_perm, a.kv_perm, N, d,
                       static_cast<T*>(a.Qp), static_cast<T*>(a.Kp), static_cast<T*>(a.Vp));
  }
  return hipGetLastError();
}

void init_partition_attributes() {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_query_scale<bf16_t, 128>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)qscale_lds<128>());
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_query_scale<float, 128>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)qscale_lds<128>());
}

hipError_t launch_partition(const PartitionArgs& a) {
  return a.bf16 ? partition_impl<bf16_t>(a) : partition_impl<float>(a);
}

}  // namespace spr
