// Stage 1 kernels: response-coupled partition and group-major permutation.
// Method: arXiv:2608.18484 ("Partition the Support, Reconstruct the
// Residual"), paperlayer.ai summary section 4 and appendices B.1-B.2, C.1;
// gist.science (nl) section 2A.  All partition arithmetic is float64 so that
// labels, permutations and offsets match a float64 reference exactly up to
// genuine near-ties; every reduction has a fixed order (no float atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

// ---------------------------------------------------------------- M_K
// M_K[i][j] = (1/M_s) sum_s Q[idx_s][i] Q[idx_s][j], idx_s = floor((2s+1)N/(2M_s)).
template <typename T>
__global__ void k_gram_mk(const T* __restrict__ Q, int N, int d, int M_s, double* __restrict__ MK) {
  const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
  if (j >= d) return;
  const T* q = Q + (int64_t)h * N * d;
  double acc = 0.0;
  for (int s = 0; s < M_s; ++s) {
    const int64_t t = ((int64_t)2 * s + 1) * N / ((int64_t)2 * M_s);
    acc = fma(load_f64(q, t * d + i), load_f64(q, t * d + j), acc);
  }
  MK[((int64_t)h * d + i) * d + j] = acc / (double)M_s;
}

// ---------------------------------------------------------------- key basis
// w_k = (lambda_k / sum lambda)^p, applied after the projection.
__global__ void k_eig_weights(const double* __restrict__ eigval, int d, int r, double p,
                              double* __restrict__ w) {
  const int h = blockIdx.x;
  __shared__ double red[128];
  const int t = threadIdx.x;
  double v = t < d ? eigval[(int64_t)h * d + t] : 0.0;
  double tot = block_sum_f64<128>(v, red);
  if (t < r) {
    double x = tot > 0.0 ? eigval[(int64_t)h * d + t] / tot : 0.0;
    double y = (p == 0.5) ? sqrt(x) : (p == 1.0 ? x : pow(x, p));
    w[(int64_t)h * r + t] = tot > 0.0 ? y : 0.0;
  }
}

// Z[t][k] = (sum_j K[t][j] U[j][k]) * w_k, U = leading eigenvectors (E stores
// eigenvector k contiguously: E[k][j]).
template <typename T>
__global__ void k_project_keys(const T* __restrict__ K, const double* __restrict__ E,
                               const double* __restrict__ w, int N, int d, int r,
                               double* __restrict__ Z) {
  extern __shared__ double smem[];
  const int h = blockIdx.y;
  double* Us = smem;  // [r][d]
  for (int e = threadIdx.x; e < r * d; e += blockDim.x) Us[e] = E[((int64_t)h * d) * d + e];
  __syncthreads();
  const int rows_per = blockDim.x / r;
  const int tl = threadIdx.x / r, k = threadIdx.x % r;
  if (tl >= rows_per) return;
  const T* kh = K + (int64_t)h * N * d;
  const double wk = w[(int64_t)h * r + k];
  for (int64_t t = (int64_t)blockIdx.x * rows_per + tl; t < N; t += (int64_t)gridDim.x * rows_per) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc = fma(load_f64(kh, t * d + j), Us[k * d + j], acc);
    Z[((int64_t)h * N + t) * r + k] = acc * wk;
  }
}

// ---------------------------------------------------------------- k-means
// Centres start at rows floor((2g+1)n/(2G)).
__global__ void k_kmeans_init(const double* __restrict__ X, int n, int D, int G, double* __restrict__ C) {
  const int h = blockIdx.y, g = blockIdx.x;
  const int64_t t = ((int64_t)2 * g + 1) * n / ((int64_t)2 * G);
  for (int k = threadIdx.x; k < D; k += blockDim.x)
    C[((int64_t)h * G + g) * D + k] = X[((int64_t)h * n + t) * D + k];
}

// Cp = A c (A the metric, or identity when A == nullptr); cn = c . Cp.
// One block per (group, head); D <= 128.
__global__ void k_centre_metric(const double* __restrict__ C, const double* __restrict__ A, int D, int G,
                                double* __restrict__ Cp, double* __restrict__ cn) {
  const int h = blockIdx.y, g = blockIdx.x, i = threadIdx.x;
  __shared__ double c[128];
  __shared__ double red[128];
  const double* cg = C + ((int64_t)h * G + g) * D;
  if (i < D) c[i] = cg[i];
  __syncthreads();
  double v = 0.0;
  if (i < D) {
    if (A) {
      const double* Ai = A + ((int64_t)h * D + i) * D;
      for (int j = 0; j < D; ++j) v = fma(Ai[j], c[j], v);
    } else {
      v = c[i];
    }
    Cp[((int64_t)h * G + g) * D + i] = v;
  }
  double s = block_sum_f64<128>(i < D ? c[i] * v : 0.0, red);
  if (i == 0) cn[(int64_t)h * G + g] = s;
}

// ---------------------------------------------------------------- stable counting sort
// counts[h][c][g] = occurrences of label g in chunk c (256 labels per chunk).
__global__ __launch_bounds__(256) void k_sort_hist(const int32_t* __restrict__ labels, int n, int G,
                                                   int nchunks, int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxGroups];
  const int h = blockIdx.y, c = blockIdx.x;
  for (int g = threadIdx.x; g < G; g += 256) hist[g] = 0;
  __syncthreads();
  const int64_t t = (int64_t)c * 256 + threadIdx.x;
  if (t < n) atomicAdd(&hist[labels[(int64_t)h * n + t]], 1);
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += 256) counts[((int64_t)h * nchunks + c) * G + g] = hist[g];
}

// base[h][c][g] = off[g] + sum_{c' < c} counts[h][c'][g]; off = exclusive scan of totals.
__global__ __launch_bounds__(1024) void k_sort_scan(const int32_t* __restrict__ counts, int G, int nchunks,
                                                    int32_t* __restrict__ base, int32_t* __restrict__ off) {
  __shared__ int tot[kMaxGroups];
  __shared__ int scan[kMaxGroups + 1];
  const int h = blockIdx.x;
  for (int g = threadIdx.x; g < G; g += 1024) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int64_t e = ((int64_t)h * nchunks + c) * G + g;
      base[e] = run;
      run += counts[e];
    }
    tot[g] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int g = 0; g < G; ++g) { scan[g] = run; run += tot[g]; }
    scan[G] = run;
  }
  __syncthreads();
  for (int g = threadIdx.x; g <= G; g += 1024) off[(int64_t)h * (G + 1) + g] = scan[g];
  for (int g = threadIdx.x; g < G; g += 1024)
    for (int c = 0; c < nchunks; ++c) base[((int64_t)h * nchunks + c) * G + g] += scan[g];
}

// perm[base + rank within chunk among equal labels] = t (stable).
__global__ __launch_bounds__(256) void k_sort_scatter(const int32_t* __restrict__ labels, int n, int G,
                                                      int nchunks, const int32_t* __restrict__ base,
                                                      int32_t* __restrict__ perm) {
  __shared__ int lab[256];
  const int h = blockIdx.y, c = blockIdx.x, i = threadIdx.x;
  const int64_t t = (int64_t)c * 256 + i;
  lab[i] = t < n ? labels[(int64_t)h * n + t] : -1;
  __syncthreads();
  if (t >= n) return;
  const int mine = lab[i];
  int rank = 0;
  for (int j = 0; j < i; ++j) rank += (lab[j] == mine);
  perm[(int64_t)h * n + base[((int64_t)h * nchunks + c) * G + mine] + rank] = (int32_t)t;
}

// Segmented mean over the sorted order: C[g] = mean of X rows perm[off[g]..off[g+1]);
// an empty group keeps C[g] (keep_empty) or gets zeros.  Fixed summation order:
// member slots s, s+S, ... per thread, then slots in order.
template <typename T>
__global__ __launch_bounds__(256) void k_segment_mean(const T* __restrict__ X, int n, int D,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ off, int G,
                                                      double* __restrict__ C, int keep_empty) {
  __shared__ double part[256];
  const int h = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const int32_t* offh = off + (int64_t)h * (G + 1);
  const int b = offh[g], e = offh[g + 1];
  double* cg = C + ((int64_t)h * G + g) * D;
  if (e == b) {
    if (!keep_empty)
      for (int k = tid; k < D; k += 256) cg[k] = 0.0;
    return;
  }
  const int32_t* ph = perm + (int64_t)h * n;
  const T* Xh = X + (int64_t)h * n * D;
  for (int d0 = 0; d0 < D; d0 += 128) {
    const int Dc = min(128, D - d0);
    const int S = 256 / Dc;
    const int s = tid / Dc, k = tid % Dc;
    double acc = 0.0;
    if (s < S)
      for (int m = b + s; m < e; m += S) acc += load_f64(Xh, (int64_t)ph[m] * D + d0 + k);
    __syncthreads();
    part[tid] = acc;
    __syncthreads();
    if (tid < Dc) {
      double sum = 0.0;
      for (int ss = 0; ss < S; ++ss) sum += part[ss * Dc + tid];
      cg[d0 + tid] = sum / (double)(e - b);
    }
  }
}

// ---------------------------------------------------------------- query-response metric
// mu_bar = mean of nonempty K/V centroids (equal weights); A = sum_g (mu_g - mu_bar)(mu_g - mu_bar)^T;
// gprime = number of nonempty groups.  Row i of A per block.
__global__ void k_metric(const double* __restrict__ mu, const int32_t* __restrict__ off, int G, int d,
                         double* __restrict__ A, int32_t* __restrict__ gprime) {
  __shared__ double mbar[128];
  const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
  const int32_t* offh = off + (int64_t)h * (G + 1);
  const double* muh = mu + (int64_t)h * G * d;
  int cnt = 0;
  double s = 0.0;
  for (int g = 0; g < G; ++g)
    if (offh[g + 1] > offh[g]) { ++cnt; if (j < d) s += muh[(int64_t)g * d + j]; }
  if (j < d) mbar[j] = s / (double)cnt;
  __syncthreads();
  if (j >= d) return;
  const double mi = mbar[i], mj = mbar[j];
  double acc = 0.0;
  for (int g = 0; g < G; ++g)
    if (offh[g + 1] > offh[g]) acc = fma(muh[(int64_t)g * d + i] - mi, muh[(int64_t)g * d + j] - mj, acc);
  A[((int64_t)h * d + i) * d + j] = acc;
  if (i == 0 && j == 0) gprime[h] = cnt;
}

// ---------------------------------------------------------------- row-tile float64 GEMM
// One kernel for the three point-by-matrix products of the partition, each
// Y = X B^T with X = 64 points x D and B = columns x D, register-tiled: a
// thread owns 4 points x CPT columns, D streamed through LDS 16 at a time.
//  RG_ASSIGN: B = metric-applied centres; label = argmin_g (cn_g - 2 x . Cp_g),
//             ties to the lowest g (||x||^2 is common to every g and left out).
//  RG_QUAD0:  B = A (symmetric metric), X = raw queries; u = q sqrt(G'/(q^T A q))
//             (0 when the form is 0).  The RMS-normalised logit profiles then
//             satisfy ||yhat_t - yhat_s||^2 = (u_t - u_s)^T A (u_t - u_s).
//  RG_QUAD1:  B = A, X = u - ubar_{label}; out = e^T A e, the squared distance
//             of a query to its group centre in query-response coordinates.
enum RowGemmMode { RG_ASSIGN = 0, RG_QUAD0 = 1, RG_QUAD1 = 2 };
constexpr int RG_P = 64, RG_K = 16;

template <int MODE, typename T>
SPR_DEV double rg_load_x(const T* Xh, int64_t t, int D, int k, const int32_t* lab, const double* cen, int G,
                         int h) {
  double v = load_f64(Xh, t * D + k);
  if (MODE == RG_QUAD1) v -= cen[((int64_t)h * G + lab[t]) * D + k];
  return v;
}

template <int MODE, typename T, int BC>
__global__ __launch_bounds__(256) void k_rowgemm(const T* __restrict__ X, int n, int D,
                                                 const double* __restrict__ B, int ncols,
                                                 const double* __restrict__ cn,
                                                 const int32_t* __restrict__ lab_in,
                                                 const double* __restrict__ centres, int G,
                                                 const int32_t* __restrict__ gprime,
                                                 int32_t* __restrict__ lab_out, double* __restrict__ out_vec,
                                                 double* __restrict__ out_scalar) {
  constexpr int CPT = BC / 16;
  __shared__ __align__(16) double Xs[RG_K][RG_P];
  __shared__ __align__(16) double Bs[RG_K][BC];
  __shared__ double redv[16][RG_P];
  __shared__ int redi[16][RG_P];
  const int h = blockIdx.y, tid = threadIdx.x, tp = tid & 15, tc = tid >> 4;
  const int64_t p0 = (int64_t)blockIdx.x * RG_P;
  const T* Xh = X + (int64_t)h * n * D;
  const double* Bh = B + (int64_t)h * ncols * D;
  const int32_t* labh = MODE == RG_QUAD1 ? lab_in + (int64_t)h * n : nullptr;
  double bv[4];
  int bi[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) { bv[a] = __builtin_inf(); bi[a] = 0x7fffffff; }
  double acc[4][CPT];
  for (int c0 = 0; c0 < ncols; c0 += BC) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[a][c] = 0.0;
    for (int k0 = 0; k0 < D; k0 += RG_K) {
      const int kc = min(RG_K, D - k0);
      __syncthreads();
      for (int e = tid; e < RG_K * RG_P; e += 256) {
        const int pp = e / RG_K, kk = e % RG_K;
        const int64_t t = p0 + pp;
        Xs[kk][pp] = (kk < kc && t < n) ? rg_load_x<MODE>(Xh, t, D, k0 + kk, labh, centres, G, h) : 0.0;
      }
      for (int e = tid; e < RG_K * BC; e += 256) {
        const int cc = e / RG_K, kk = e % RG_K;
        const int col = c0 + cc;
        Bs[kk][cc] = (kk < kc && col < ncols) ? Bh[(int64_t)col * D + k0 + kk] : 0.0;
      }
      __syncthreads();
#pragma unroll 4
      for (int kk = 0; kk < kc; ++kk) {
        double xv[4], bw[CPT];
#pragma unroll
        for (int a = 0; a < 4; a += 2) {
          const double2 v = *reinterpret_cast<const double2*>(&Xs[kk][tp * 4 + a]);
          xv[a] = v.x; xv[a + 1] = v.y;
        }
#pragma unroll
        for (int c = 0; c < CPT; c += 2) {
          const double2 v = *reinterpret_cast<const double2*>(&Bs[kk][tc * CPT + c]);
          bw[c] = v.x; bw[c + 1] = v.y;
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < CPT; ++c) acc[a][c] = fma(xv[a], bw[c], acc[a][c]);
      }
    }
    if (MODE == RG_ASSIGN) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int g = c0 + tc * CPT + c;
        if (g < ncols) {
          const double c2 = cn[(int64_t)h * ncols + g];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const double dist = c2 - 2.0 * acc[a][c];
            if (dist < bv[a]) { bv[a] = dist; bi[a] = g; }
          }
        }
      }
    }
  }
  if (MODE == RG_ASSIGN) {
#pragma unroll
    for (int a = 0; a < 4; ++a) { redv[tc][tp * 4 + a] = bv[a]; redi[tc][tp * 4 + a] = bi[a]; }
    __syncthreads();
    if (tid < RG_P && p0 + tid < n) {
      double v = redv[0][tid];
      int gi = redi[0][tid];
      for (int s = 1; s < 16; ++s) {
        const double v2 = redv[s][tid];
        const int g2 = redi[s][tid];
        if (v2 < v || (v2 == v && g2 < gi)) { v = v2; gi = g2; }
      }
      lab_out[(int64_t)h * n + p0 + tid] = gi;
    }
    return;
  }
  // quadratic form: sum over columns of x_col * (x^T A)_col
  double xr[4][CPT];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t t = p0 + tp * 4 + a;
    double part = 0.0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = tc * CPT + c;
      xr[a][c] = (t < n && col < ncols) ? rg_load_x<MODE>(Xh, t, D, col, labh, centres, G, h) : 0.0;
      part = fma(xr[a][c], acc[a][c], part);
    }
    redv[tc][tp * 4 + a] = part;
  }
  __syncthreads();
  if (tid < RG_P) {
    double form = 0.0;
    for (int s = 0; s < 16; ++s) form += redv[s][tid];
    const int64_t t = p0 + tid;
    if (MODE == RG_QUAD1) {
      if (t < n) out_scalar[(int64_t)h * n + t] = form;
    } else {
      redv[0][tid] = form > 0.0 ? sqrt((double)gprime[h] / form) : 0.0;
    }
  }
  if (MODE == RG_QUAD0) {
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t t = p0 + tp * 4 + a;
      const double sc = redv[0][tp * 4 + a];
      if (t < n)
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int col = tc * CPT + c;
          if (col < ncols) out_vec[((int64_t)h * n + t) * D + col] = xr[a][c] * sc;
        }
    }
  }
}

template <int MODE, typename T>
static void launch_rowgemm(dim3 grid, hipStream_t st, const T* X, int n, int D, const double* B, int ncols,
                           const double* cn, const int32_t* lab_in, const double* centres, int G,
                           const int32_t* gprime, int32_t* lab_out, double* out_vec, double* out_scalar) {
  if (ncols > 64)
    hipLaunchKernelGGL((k_rowgemm<MODE, T, 128>), grid, dim3(256), 0, st, X, n, D, B, ncols, cn, lab_in, centres,
                       G, gprime, lab_out, out_vec, out_scalar);
  else
    hipLaunchKernelGGL((k_rowgemm<MODE, T, 64>), grid, dim3(256), 0, st, X, n, D, B, ncols, cn, lab_in, centres,
                       G, gprime, lab_out, out_vec, out_scalar);
}

// ---------------------------------------------------------------- permutation gather
// dst[h][slot] = src[h][perm[h][slot]], rows of d elements moved as 16-byte vectors.
template <typename T>
__global__ __launch_bounds__(256) void k_gather_rows(const T* __restrict__ src, const int32_t* __restrict__ perm,
                                                     int n, int d, T* __restrict__ dst) {
  const int h = blockIdx.y;
  const int vec_per_row = d * (int)sizeof(T) / 16;
  const int rows_per_block = 256 / vec_per_row;
  const int r = threadIdx.x / vec_per_row, v = threadIdx.x % vec_per_row;
  const int64_t slot = (int64_t)blockIdx.x * rows_per_block + r;
  if (slot >= n) return;
  const int64_t t = perm[(int64_t)h * n + slot];
  const uint4* s = reinterpret_cast<const uint4*>(src + ((int64_t)h * n + t) * d);
  uint4* o = reinterpret_cast<uint4*>(dst + ((int64_t)h * n + slot) * d);
  o[v] = s[v];
}

// ================================================================ launchers
template <typename T>
static hipError_t partition_impl(const PartitionArgs& a) {
  const int H = a.H, N = a.N, d = a.d, G_k = a.G_k, G_q = a.G_q, r = a.r_k;
  const T* Q = static_cast<const T*>(a.Q);
  const T* K = static_cast<const T*>(a.K);
  const T* V = static_cast<const T*>(a.V);
  hipStream_t st = a.stream;
  const int nchunks = (N + 255) / 256;
  const dim3 tileGrid((N + 63) / 64, H);

  // --- key-response coordinates (B.1)
  hipLaunchKernelGGL(k_gram_mk<T>, dim3(d, H), dim3(128), 0, st, Q, N, d, a.M_s, a.ws.mk);
  launch_sym_eig(a.ws.mk, H, d, a.ws.eigval, a.ws.eigvec, st);
  hipLaunchKernelGGL(k_eig_weights, dim3(H), dim3(128), 0, st, a.ws.eigval, d, r, a.eig_power, a.ws.wk);
  {
    const int rows_per = 256 / r;
    const int blocks = std::min<int64_t>((N + rows_per - 1) / rows_per, 4096);
    hipLaunchKernelGGL(k_project_keys<T>, dim3(blocks, H), dim3(256), sizeof(double) * r * d, st, K,
                       a.ws.eigvec, a.ws.wk, N, d, r, a.ws.Z);
  }
  // --- paired K/V k-means on Z (B.1); V inherits the key's label
  auto kmeans = [&](const double* X, int D, int G, int iters, const double* metric, int32_t* labels,
                    int32_t* perm, int32_t* off) {
    hipLaunchKernelGGL(k_kmeans_init, dim3(G, H), dim3(128), 0, st, X, N, D, G, a.ws.cent);
    hipLaunchKernelGGL(k_centre_metric, dim3(G, H), dim3(128), 0, st, a.ws.cent, metric, D, G, a.ws.centp,
                       a.ws.cnorm);
    for (int it = 0; it < iters; ++it) {
      launch_rowgemm<RG_ASSIGN, double>(tileGrid, st, X, N, D, a.ws.centp, G, a.ws.cnorm, nullptr, nullptr, 0,
                                        nullptr, labels, nullptr, nullptr);
      hipLaunchKernelGGL(k_sort_hist, dim3(nchunks, H), dim3(256), 0, st, labels, N, G, nchunks, a.ws.counts);
      hipLaunchKernelGGL(k_sort_scan, dim3(H), dim3(1024), 0, st, a.ws.counts, G, nchunks, a.ws.base, off);
      hipLaunchKernelGGL(k_sort_scatter, dim3(nchunks, H), dim3(256), 0, st, labels, N, G, nchunks, a.ws.base,
                         perm);
      hipLaunchKernelGGL(k_segment_mean<double>, dim3(G, H), dim3(256), 0, st, X, N, D, perm, off, G, a.ws.cent,
                         1);
      hipLaunchKernelGGL(k_centre_metric, dim3(G, H), dim3(128), 0, st, a.ws.cent, metric, D, G, a.ws.centp,
                         a.ws.cnorm);
    }
  };
  kmeans(a.ws.Z, r, G_k, a.iters_kv, nullptr, a.kv_label, a.kv_perm, a.kv_off);
  hipLaunchKernelGGL(k_segment_mean<T>, dim3(G_k, H), dim3(256), 0, st, K, N, d, a.kv_perm, a.kv_off, G_k,
                     a.kv_centroid, 0);
  // --- query-response coordinates (B.2, C.1) and query k-means
  hipLaunchKernelGGL(k_metric, dim3(d, H), dim3(128), 0, st, a.kv_centroid, a.kv_off, G_k, d, a.ws.metric,
                     a.ws.gprime);
  launch_rowgemm<RG_QUAD0, T>(tileGrid, st, Q, N, d, a.ws.metric, d, nullptr, nullptr, nullptr, 0, a.ws.gprime,
                              nullptr, a.ws.U, nullptr);
  kmeans(a.ws.U, d, G_q, a.iters_q, a.ws.metric, a.q_label, a.q_perm, a.q_off);
  launch_rowgemm<RG_QUAD1, double>(tileGrid, st, a.ws.U, N, d, a.ws.metric, d, nullptr, a.q_label, a.ws.cent,
                                   G_q, nullptr, nullptr, nullptr, a.q_dist);
  hipLaunchKernelGGL(k_segment_mean<T>, dim3(G_q, H), dim3(256), 0, st, Q, N, d, a.q_perm, a.q_off, G_q,
                     a.q_centroid, 0);
  // --- group-major layouts (s4 Sparse Execution)
  {
    const int rows_per_block = 256 / (d * (int)sizeof(T) / 16);
    const dim3 g((N + rows_per_block - 1) / rows_per_block, H);
    hipLaunchKernelGGL(k_gather_rows<T>, g, dim3(256), 0, st, Q, a.q_perm, N, d, static_cast<T*>(a.Qp));
    hipLaunchKernelGGL(k_gather_rows<T>, g, dim3(256), 0, st, K, a.kv_perm, N, d, static_cast<T*>(a.Kp));
    hipLaunchKernelGGL(k_gather_rows<T>, g, dim3(256), 0, st, V, a.kv_perm, N, d, static_cast<T*>(a.Vp));
  }
  return hipGetLastError();
}

void init_partition_attributes() {
  const int mx = (int)(sizeof(double) * 128 * 128);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_project_keys<float>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, mx);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_project_keys<bf16_t>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, mx);
}

hipError_t launch_partition(const PartitionArgs& a) {
  return a.bf16 ? partition_impl<bf16_t>(a) : partition_impl<float>(a);
}

}  // namespace spr
