// Stage 2 kernels: shared routing under a query-key pair budget
// (arXiv:2608.18484: abstract -- K/V-group centroids induce the coordinates
// used for shared routing; paperlayer.ai summary section 4 "Sparse
// Execution" -- cells are selected under a pair budget with true cell costs).
// Scores are float64; selection is integer arithmetic on exact cell costs.
#include "common.hpp"
#include "kernels.hpp"

#include <mutex>

namespace spr {

// P[a][b] = softmax over nonempty b of (s qbar_a . mu_b + ln n_b); zero rows
// for empty query groups and zero columns for empty K/V groups.
__global__ __launch_bounds__(256) void k_route_scores(const double* __restrict__ qbar, const double* __restrict__ mu,
                                                      const int32_t* __restrict__ q_off,
                                                      const int32_t* __restrict__ kv_off, int G_q, int G_k, int d,
                                                      double scale, double* __restrict__ P) {
  __shared__ double red[256];
  __shared__ double qa[128];
  const int h = blockIdx.y, a = blockIdx.x, tid = threadIdx.x;
  const int32_t* qo = q_off + (int64_t)h * (G_q + 1);
  const int32_t* ko = kv_off + (int64_t)h * (G_k + 1);
  double* Pa = P + ((int64_t)h * G_q + a) * G_k;
  if (qo[a + 1] == qo[a]) {
    for (int b = tid; b < G_k; b += 256) Pa[b] = 0.0;
    return;
  }
  if (tid < d) qa[tid] = qbar[((int64_t)h * G_q + a) * d + tid];
  __syncthreads();
  constexpr int PER = kMaxGroups / 256;
  double L[PER];
  double mx = -__builtin_inf();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = tid + 256 * i;
    L[i] = -__builtin_inf();
    if (b < G_k) {
      const int nb = ko[b + 1] - ko[b];
      if (nb > 0) {
        const double* mb = mu + ((int64_t)h * G_k + b) * d;
        double dot = 0.0;
#pragma unroll 16
        for (int k = 0; k < d; ++k) dot = fma(qa[k], mb[k], dot);
        L[i] = scale * dot + log((double)nb);
        mx = fmax(mx, L[i]);
      }
    }
  }
  mx = block_max_f64<256>(mx, red);
  double e[PER];
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    e[i] = (L[i] == -__builtin_inf()) ? 0.0 : exp(L[i] - mx);
    s += e[i];
  }
  s = block_sum_f64<256>(s, red);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = tid + 256 * i;
    if (b < G_k) Pa[b] = e[i] / s;
  }
}

// One block per head: mandatory best cell per nonempty query group, then
// either top-k per group or the global greedy budget scan, then CSR.
// The budget scan order is (P desc, a asc, b asc); the first cell that does
// not fit ends it.  The cut is found by an 8-level radix descent over the
// bit patterns of P (nonnegative doubles order like their bits) with exact
// int64 cost histograms, so no sort is needed; it stops early once the bin
// holding the first cell that does not fit has no other cell (that cell's
// bits are then the cut).  Row work goes one wave per
// query group (lanes over K/V groups); scans over bins, tie counts and rows
// are block-parallel.
// Up to RS_LDS_CELLS cells (SMALL) the scores and the selection flags live
// in LDS for the whole kernel; otherwise they are read from and kept in
// global memory.
constexpr int RS_THREADS = 1024;
constexpr int RS_WAVES = RS_THREADS / 64;
constexpr int RS_TIES = 2048;
constexpr int RS_LDS_CELLS = 4096;
template <bool SMALL>
__global__ __launch_bounds__(RS_THREADS) void k_route_select(const double* __restrict__ P,
                                                             const int32_t* __restrict__ q_off,
                                                             const int32_t* __restrict__ kv_off, int G_q, int G_k,
                                                             int top_k, int64_t budget, uint8_t* __restrict__ sel,
                                                             int32_t* __restrict__ row_ptr,
                                                             int32_t* __restrict__ col_idx,
                                                             int64_t* __restrict__ routed_pairs) {
  __shared__ int qn[kMaxGroups];
  __shared__ int kn[kMaxGroups];
  __shared__ unsigned long long hist[256];
  __shared__ unsigned int hcnt[256];
  __shared__ int64_t red[RS_THREADS];
  __shared__ int64_t wsum64[RS_WAVES];
  __shared__ int wsum32[RS_WAVES];
  __shared__ int tie_cells[RS_TIES];
  __shared__ int rowbase[kMaxGroups];
  __shared__ uint64_t s_prefix, s_vo;
  __shared__ int64_t s_above;
  __shared__ int s_done;
  __shared__ double Ps[SMALL ? RS_LDS_CELLS : 1];
  __shared__ uint8_t Ss[SMALL ? RS_LDS_CELLS : 1];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* qo = q_off + (int64_t)h * (G_q + 1);
  const int32_t* ko = kv_off + (int64_t)h * (G_k + 1);
  const int ncell = G_q * G_k;
  const double* Pg = P + (int64_t)h * ncell;
  const double* Ph = SMALL ? Ps : Pg;
  uint8_t* S = SMALL ? Ss : sel + (int64_t)h * ncell;
  for (int a = tid; a < G_q; a += RS_THREADS) qn[a] = qo[a + 1] - qo[a];
  for (int b = tid; b < G_k; b += RS_THREADS) kn[b] = ko[b + 1] - ko[b];
  for (int c = tid; c < ncell; c += RS_THREADS) {
    S[c] = 0;
    if (SMALL) Ps[c] = Pg[c];
  }
  __syncthreads();
  // mandatory best cell (largest P, ties to the smaller b), one wave per row
  int64_t mand = 0;
  for (int a = wv; a < G_q; a += RS_WAVES) {
    if (qn[a] == 0) continue;
    double bv = -1.0;
    int best = 0x7fffffff;
    for (int b = lane; b < G_k; b += 64) {
      if (kn[b] == 0) continue;
      const double v = Ph[(int64_t)a * G_k + b];
      if (v > bv) { bv = v; best = b; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o);
      const int ob = __shfl_xor(best, o);
      if (ov > bv || (ov == bv && ob < best)) { bv = ov; best = ob; }
    }
    if (lane == 0) {
      S[(int64_t)a * G_k + best] = 1;
      mand += (int64_t)qn[a] * kn[best];
    }
  }
  mand = block_sum_i64<RS_THREADS>(mand, red);   // barrier inside also publishes S
  if (top_k > 0) {
    for (int a = tid; a < G_q; a += RS_THREADS) {
      if (qn[a] == 0) continue;
      for (int r = 1; r < top_k; ++r) {
        int best = -1;
        double bv = -1.0;
        for (int b = 0; b < G_k; ++b) {
          const int64_t c = (int64_t)a * G_k + b;
          if (kn[b] > 0 && !S[c] && Ph[c] > bv) { bv = Ph[c]; best = b; }
        }
        if (best < 0) break;
        S[(int64_t)a * G_k + best] = 1;
      }
    }
    __syncthreads();
  } else {
    const int64_t room = budget - mand;
    // total cost of the optional cells
    int64_t tot = 0;
    for (int a = wv; a < G_q; a += RS_WAVES) {
      if (qn[a] == 0) continue;
      for (int b = lane; b < G_k; b += 64)
        if (kn[b] > 0 && !S[(int64_t)a * G_k + b]) tot += (int64_t)qn[a] * kn[b];
    }
    tot = block_sum_i64<RS_THREADS>(tot, red);
    if (room >= 0 && tot <= room) {
      for (int a = wv; a < G_q; a += RS_WAVES)
        for (int b = lane; b < G_k; b += 64)
          if (qn[a] > 0 && kn[b] > 0) S[(int64_t)a * G_k + b] = 1;
      __syncthreads();
    } else if (room >= 0) {
      // radix descent for v_o = bits of the overflow cell's score
      if (tid == 0) { s_prefix = 0; s_above = 0; s_done = 0; }
      __syncthreads();
      for (int level = 7; level >= 0; --level) {
        if (tid < 256) { hist[tid] = 0; hcnt[tid] = 0; }
        __syncthreads();
        const uint64_t prefix = s_prefix;
        const int64_t above0 = s_above;
        const int sh = 8 * level;
        // a wave whose contributing lanes all fall in one bin (scores that
        // share their leading bytes, the usual case at the first levels)
        // adds its cost sum with one atomic instead of one per lane
        for (int a = wv; a < G_q; a += RS_WAVES) {
          if (qn[a] == 0) continue;
          for (int b0 = 0; b0 < G_k; b0 += 64) {
            const int b = b0 + lane;
            bool take = false;
            int bin = 0;
            int64_t cost = 0;
            if (b < G_k && kn[b] > 0) {
              const int64_t c = (int64_t)a * G_k + b;
              if (!S[c]) {
                const uint64_t bits = (uint64_t)__double_as_longlong(Ph[c]);
                const uint64_t high = (level == 7) ? 0 : (bits >> (sh + 8));
                if (high == prefix) {
                  take = true;
                  bin = (int)((bits >> sh) & 255);
                  cost = (int64_t)qn[a] * kn[b];
                }
              }
            }
            const unsigned long long m = __ballot(take);
            if (m == 0) continue;
            const int first = __builtin_ctzll(m);
            const int bin0 = __shfl(bin, first);
            if (__ballot(take && bin != bin0) == 0) {
              int64_t cs = cost;
#pragma unroll
              for (int o = 32; o > 0; o >>= 1) cs += __shfl_xor(cs, o);
              if (lane == first) {
                atomicAdd(&hist[bin0], (unsigned long long)cs);
                atomicAdd(&hcnt[bin0], (unsigned int)__popcll(m));
              }
            } else if (take) {
              atomicAdd(&hist[bin], (unsigned long long)cost);
              atomicAdd(&hcnt[bin], 1u);
            }
          }
        }
        __syncthreads();
        // thread t < 256 holds bin 255 - t, so the exclusive prefix is the cost strictly above
        const int64_t hv = tid < 256 ? (int64_t)hist[255 - tid] : 0;
        int64_t all;
        const int64_t above = above0 + block_exclusive_scan<RS_THREADS>(hv, wsum64, &all);
        if (tid < 256 && above <= room && room < above + hv) {
          s_above = above;
          s_prefix = (prefix << 8) | (uint64_t)(255 - tid);
          if (level > 0 && hcnt[255 - tid] == 1) s_done = 1;   // the overflow cell is alone in its bin
        }
        __syncthreads();
        if (s_done) {   // uniform: that cell's score is v_o; no need to descend further
          const uint64_t pf = s_prefix;
          for (int a = wv; a < G_q; a += RS_WAVES) {
            if (qn[a] == 0) continue;
            for (int b = lane; b < G_k; b += 64) {
              const int64_t c = (int64_t)a * G_k + b;
              if (kn[b] == 0 || S[c]) continue;
              const uint64_t bits = (uint64_t)__double_as_longlong(Ph[c]);
              if ((bits >> sh) == pf) s_vo = bits;   // exactly one cell
            }
          }
          __syncthreads();
          break;
        }
      }
      const uint64_t vo = s_done ? s_vo : s_prefix;
      // cells strictly above v_o are in; the tie group at v_o is taken in index order
      const int per = (ncell + RS_THREADS - 1) / RS_THREADS;
      const int c0 = min(ncell, tid * per), c1 = min(ncell, c0 + per);
      int mine = 0;
      {
        int a = c0 / G_k, b = c0 % G_k;
        for (int c = c0; c < c1; ++c) {
          if (qn[a] > 0 && kn[b] > 0 && !S[c]) {
            const uint64_t bits = (uint64_t)__double_as_longlong(Ph[c]);
            if (bits > vo) S[c] = 2;
            else if (bits == vo) ++mine;
          }
          if (++b == G_k) { b = 0; ++a; }
        }
      }
      int nties;
      int w = block_exclusive_scan<RS_THREADS>(mine, wsum32, &nties);
      if (nties <= RS_TIES && mine > 0) {
        int a = c0 / G_k, b = c0 % G_k;
        for (int c = c0; c < c1; ++c) {
          if (qn[a] > 0 && kn[b] > 0 && S[c] == 0 && (uint64_t)__double_as_longlong(Ph[c]) == vo) tie_cells[w++] = c;
          if (++b == G_k) { b = 0; ++a; }
        }
      }
      __syncthreads();
      if (tid == 0) {
        int64_t used = mand + s_above;
        if (nties <= RS_TIES) {
          for (int i = 0; i < nties; ++i) {
            const int c = tie_cells[i];
            const int64_t cost = (int64_t)qn[c / G_k] * kn[c % G_k];
            if (used + cost > budget) break;
            used += cost;
            S[c] = 2;
          }
        } else {
          for (int c = 0; c < ncell; ++c) {
            const int a = c / G_k, b = c % G_k;
            if (qn[a] == 0 || kn[b] == 0 || S[c]) continue;
            if ((uint64_t)__double_as_longlong(Ph[c]) != vo) continue;
            const int64_t cost = (int64_t)qn[a] * kn[b];
            if (used + cost > budget) break;
            used += cost;
            S[c] = 2;
          }
        }
      }
      __syncthreads();
    }
  }
  // CSR: rows in a order, columns ascending; row counts and compaction by wave ballots
  for (int a = wv; a < G_q; a += RS_WAVES) {
    int n = 0;
    for (int b0 = 0; b0 < G_k; b0 += 64) {
      const int b = b0 + lane;
      n += __popcll(__ballot(b < G_k && S[(int64_t)a * G_k + b] != 0));
    }
    if (lane == 0) rowbase[a] = n;
  }
  __syncthreads();
  const int cnt = tid < G_q ? rowbase[tid] : 0;
  int nnz;
  const int start = block_exclusive_scan<RS_THREADS>(cnt, wsum32, &nnz);
  int32_t* rp = row_ptr + (int64_t)h * (G_q + 1);
  if (tid < G_q) { rowbase[tid] = start; rp[tid] = start; }
  if (tid == 0) rp[G_q] = nnz;
  __syncthreads();
  int32_t* ci = col_idx + (int64_t)h * G_q * G_k;
  int64_t pairs = 0;
  for (int a = wv; a < G_q; a += RS_WAVES) {
    int w = rowbase[a];
    for (int b0 = 0; b0 < G_k; b0 += 64) {
      const int b = b0 + lane;
      const bool f = b < G_k && S[(int64_t)a * G_k + b] != 0;
      const unsigned long long m = __ballot(f);
      if (f) {
        ci[w + __popcll(m & ((1ull << lane) - 1ull))] = b;
        pairs += (int64_t)qn[a] * kn[b];
      }
      w += __popcll(m);
    }
  }
  pairs = block_sum_i64<RS_THREADS>(pairs, red);
  if (tid == 0) routed_pairs[h] = pairs;
}

// ---- scratch for callers that cannot allocate
// A file-scope device array holds the cell scores and selection flags of
// sparsepr_route_noalloc (every GPU the library runs on keeps its own copy
// until the process ends).  In host code `scratch` names a host-side stand-in,
// never the device memory: the device address is looked up once per device
// with hipGetSymbolAddress and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[kRouteScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

hipError_t route_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t route_scratch_need(int H, int G_q, int G_k) {
  const size_t cells = (size_t)H * G_q * G_k;
  const size_t p_bytes = (cells * sizeof(double) + 255) & ~size_t(255);
  return p_bytes + cells;
}

void route_scratch_carve(void* base, int H, int G_q, int G_k, Workspace* w) {
  const size_t cells = (size_t)H * G_q * G_k;
  const size_t p_bytes = (cells * sizeof(double) + 255) & ~size_t(255);
  w->P = static_cast<double*>(base);
  w->sel = static_cast<uint8_t*>(base) + p_bytes;
}

hipError_t launch_route(const RouteArgs& a) {
  hipLaunchKernelGGL(k_route_scores, dim3(a.G_q, a.H), dim3(256), 0, a.stream, a.q_centroid, a.kv_centroid,
                     a.q_off, a.kv_off, a.G_q, a.G_k, a.d, a.scale, a.ws.P);
  const int64_t budget = (int64_t)floor(a.density * ((double)a.N * (double)a.N)) - (int64_t)a.M * a.N;
  if ((int64_t)a.G_q * a.G_k <= RS_LDS_CELLS)
    hipLaunchKernelGGL(k_route_select<true>, dim3(a.H), dim3(RS_THREADS), 0, a.stream, a.ws.P, a.q_off, a.kv_off,
                       a.G_q, a.G_k, a.top_k, budget, a.ws.sel, a.row_ptr, a.col_idx, a.routed_pairs);
  else
    hipLaunchKernelGGL(k_route_select<false>, dim3(a.H), dim3(RS_THREADS), 0, a.stream, a.ws.P, a.q_off, a.kv_off,
                       a.G_q, a.G_k, a.top_k, budget, a.ws.sel, a.row_ptr, a.col_idx, a.routed_pairs);
  return hipGetLastError();
}

}  // namespace spr
