// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>

namespace spr {

constexpr int kSortSlices = 16;   // chunk slices per head of the counting sort's scan
constexpr int kMaxGroups = 1024;  // G_k, G_q upper bound (LDS histograms)
constexpr int kSortChunk = 128;   // points per chunk of the stable counting sort
constexpr int kMaxProbes = 4096;   // M upper bound
constexpr int kAttnBM = 128;       // query rows per work item of the 4-wave attention kernels (the smallest)
constexpr int kProbeSplits = 16;   // key splits of the dense probe-row pass
constexpr int kSmallKmeansN = 8192; // up to this many points a Lloyd round skips the sort

// Scratch regions carved out of the caller's workspace (see workspace.cpp).
// Certified low-precision k-means assignment (assign.hip): fp16 hi/lo parts
// of the points (fixed for one k-means) and of the metric-applied centres
// (rewritten after every update), with power-of-two scales and norms.
struct LpAssign {
  uint16_t *xh, *xl;   // [H,n,DP]
  int32_t* xe;         // [H,n]   point exponents
  float* xn;           // [H,n]   ||x 2^-e|| (rounded up)
  uint16_t *ch, *cl;   // [H,G,DP]
  int32_t* ce;         // [H,G]   centre exponents
  float* cn32;         // [H,G]   cn_g as float
  float* cnrm;         // [H,G]   ||Cp_g 2^-e|| (rounded up)
  double* cpt;         // [H,D,G] metric-applied centres, transposed (float64 pass)
  int32_t* list;       // [H,n]   queries whose distances take the direct form
  int32_t* cnt;        // [H]     their number
};
// Rows of the k-means points in float64: stored rows X [H,n,D], or input
// rows Q [H,n,D] (bf16 or float) times a per-row scale s [H,n] (1 when s is
// null), read on the fly -- the query coordinates u = s q are never stored.
// Kernels take the access mode as a template argument (no per-element
// branches); mode() gives it for a launch.
enum RowsMode { ROWS_F64 = 0, ROWS_BF16_SCALED = 1, ROWS_F32_SCALED = 2, ROWS_BF16 = 3, ROWS_F32 = 4 };
struct Rows64 {
  const double* X;
  const void* Q;
  const double* s;
  int bf16;
  int mode() const {
    if (X) return ROWS_F64;
    if (s) return bf16 ? ROWS_BF16_SCALED : ROWS_F32_SCALED;
    return bf16 ? ROWS_BF16 : ROWS_F32;
  }
  template <int M>
  __device__ __forceinline__ double at(int h, int n, int D, int64_t t, int k) const {
    const int64_t e = ((int64_t)h * n + t) * D + k;
    if (M == ROWS_F64) return X[e];
    const double q = (M == ROWS_BF16_SCALED || M == ROWS_BF16) ? (double)(float)static_cast<const __bf16*>(Q)[e]
                                                                : (double)static_cast<const float*>(Q)[e];
    return (M == ROWS_BF16_SCALED || M == ROWS_F32_SCALED) ? q * s[(int64_t)h * n + t] : q;
  }
};
#define SPR_ROWS_SWITCH(MODEV, CALL)              \
  switch (MODEV) {                                \
    case ROWS_F64: CALL(ROWS_F64); break;         \
    case ROWS_BF16_SCALED: CALL(ROWS_BF16_SCALED); break; \
    case ROWS_F32_SCALED: CALL(ROWS_F32_SCALED); break;   \
    case ROWS_BF16: CALL(ROWS_BF16); break;       \
    default: CALL(ROWS_F32); break;               \
  }

// 16-byte row slices of the k-means points as float64: VEC elements of row
// t from column k0 (k0 a multiple of VEC), times the row scale in the
// scaled modes (the same products as Rows64::at).
template <int RM>
struct RowVec {
  static constexpr int ES = RM == ROWS_F64 ? 8 : ((RM == ROWS_BF16_SCALED || RM == ROWS_BF16) ? 2 : 4);
  static constexpr int VEC = 16 / ES;
  static __device__ __forceinline__ void load(const Rows64& X, int h, int n, int D, int64_t t, int k0,
                                              double (&v)[VEC]) {
    const int64_t e = ((int64_t)h * n + t) * D + k0;
    if (RM == ROWS_F64) {
      const double2 w = *reinterpret_cast<const double2*>(X.X + e);
      v[0] = w.x;
      v[1 % VEC] = w.y;
      return;
    }
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const char*>(X.Q) + e * ES);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const double sc = (RM == ROWS_BF16_SCALED || RM == ROWS_F32_SCALED) ? X.s[(int64_t)h * n + t] : 1.0;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      double q;
      if (ES == 2) q = (double)__builtin_bit_cast(float, (i & 1) ? (wd[i >> 1] & 0xffff0000u) : (wd[i >> 1] << 16));
      else q = (double)__builtin_bit_cast(float, wd[i]);
      v[i] = (RM == ROWS_BF16_SCALED || RM == ROWS_F32_SCALED) ? q * sc : q;
    }
  }
};

// padded dims of the fp16 parts: a power of two from 16 to 128
__host__ __device__ inline int lp_dims(int D) { return D <= 16 ? 16 : (D <= 32 ? 32 : (D <= 64 ? 64 : 128)); }

struct Workspace {
  // partition
  double* mk;        // [H,d,d]   M_K
  double* eigval;    // [H,d]     leading r_k eigenvalues, descending
  double* eigvec;    // [H,d,d]   leading r_k eigenvectors, vector k contiguous
  double* mtrace;    // [H]       trace of M_K (the sum of its eigenvalues)
  double* eigscr;    // eigensolver scratch: T and the reflectors per head
  double* wk;        // [H,d]     eigen weights
  double* Z;         // [H,N,r_k] key-response coordinates
  double* qscale;    // [H,N]     row scales of the query coordinates, u = qscale q
  double* metric;    // [H,d,d]   A = C C^T of the centred K/V centroids
  int32_t* gprime;   // [H]
  double* cent;      // [H,Gmax,Dmax] k-means centres
  double* centp;     // [H,Gmax,Dmax] metric-applied centres
  double* cnorm;     // [H,Gmax]
  int32_t* counts;   // [H,nchunks,Gmax]
  int32_t* base;     // [H,nchunks,Gmax]
  int32_t* sortpart; // [H,kSortSlices,1024] per-slice part sums of the counting sort's scan
  LpAssign lp;       // certified assignment buffers
  // route
  double* P;         // [H,G_q,G_k] cell scores
  uint8_t* sel;      // [H,G_q,G_k] selected cells
  // attention
  int32_t* tiles;    // [H,G_q+1] prefix of 128-row tiles per query group
  int4* tdesc;       // [H,maxT]  per row tile: first row, end row, row_ptr of its group, segment count
  int2* segs;        // [H,G_q*G_k] per routed cell (CSR order): first key row, key count
  uint16_t* vh;      // [H,N,d]   fp16 copy of V (x 2^-e per head) for the bf16 attention kernels
  float* vpart;      // [H,64]    max |V| per slice of a head
  float* vinv;       // [H]       2^-e, the scale of the head's fp16 V
  float* vscale;     // [H]       2^e, undone in the attention epilogues
  float* spart;      // [S,H,N,d] key-split partial outputs of the sparse pass (S > 1 only)
  float* smpart;     // [S,H,N]
  float* slpart;     // [S,H,N]
  // probes / fit
  int32_t* alloc;    // [H,G_q]   probes per group
  int32_t* pgroup;   // [H,M]     group of each probe slot
  int32_t* prank;    // [H,M]     rank inside the group
  int32_t* pt;       // [H,M]     chosen token (selection order)
  int32_t* pslot;    // [H,M]     its group-major slot (selection order)
  int32_t* probe_slot; // [H,M]   group-major slot of each probe, probe_idx order
  float* opart;      // [S,H,M,d] split-K partial outputs
  float* mpart;      // [S,H,M]   split-K partial max (log2 units)
  float* lpart;      // [S,H,M]   split-K partial sums
  double* fx;        // [H,M,d]   sparse output at the probes
  double* fr;        // [H,M,d]   exact - sparse at the probes
  double* gram;      // [3,H,d,d] Rt^T Rt, Xt^T Xt + lam I, Xt^T Rt
  double* fitvec;    // [H,2,d]   x_bar, r_bar (scratch copy)
  double* feig;      // [H,d]     leading rank eigenvalues of Rt^T Rt
  double* fvec;      // [H,d,d]   their eigenvectors
  double* ftrace;    // [H]       trace of Rt^T Rt
  double* frhs;      // [H,d,rank] (Xt^T Rt) V_r
  // correction
  int32_t* probe_pos;// [H,N]     probe number of each token, -1 if none
  float* corr_b;     // [H,ceil(rank/32),d/2,64] B_r chunks in matrix-core fragment order (float32)
  float* corr_c;     // [H,ceil(rank/32),32]     -xbar B_r per chunk (float32)
  uint16_t* corr_h;  // [H,ceil(rank/32),2,32d]  fp16 fragments of B_r (scaled) and V_r per chunk (bf16 outputs)
  int32_t* corr_e;   // [H,ceil(rank/32)]        power-of-two scale exponent of each B_r chunk
};

void launch_lp_points(const Rows64& X, int H, int n, int D, const LpAssign& lp, hipStream_t st);
// also writes the label counts of every kSortChunk-point chunk: counts[H][chunk][G];
// gprime [H] (the query metric form: ||y||^2 = G') or null (identity metric)
void launch_assign_lp(const Rows64& X, const double* Cp, const double* cn, const int32_t* gprime, int H, int n, int D,
                      int G, const LpAssign& lp, int32_t* labels, int32_t* counts, hipStream_t st);

struct PartitionArgs {
  int H, N, d, G_k, G_q, M_s, r_k, iters_kv, iters_q;
  double eig_power;
  bool bf16;
  bool semantic;   // k-means on the raw keys / queries (the pages' baseline)
  bool warm;       // k-means starts from the labels found in kv_label / q_label
  const void *Q, *K, *V;
  int32_t *kv_label, *q_label, *kv_perm, *q_perm, *kv_off, *q_off;
  void *Qp, *Kp, *Vp;
  double *kv_centroid, *q_centroid, *q_dist;
  Workspace ws;
  hipStream_t stream;
};

struct RouteArgs {
  int H, N, d, G_k, G_q, top_k, M;
  double density, scale;
  const int32_t *kv_off, *q_off;
  const double *kv_centroid, *q_centroid;
  int32_t *row_ptr, *col_idx;
  int64_t* routed_pairs;
  Workspace ws;
  hipStream_t stream;
};

struct AttendArgs {
  int H, N, d, G_k, G_q;
  float scale;
  bool bf16;
  const void *Qp, *Kp, *Vp;
  const int32_t *q_off, *kv_off, *row_ptr, *col_idx;
  float *Op, *lse;
  Workspace ws;
  hipStream_t stream;
};

struct ProbeFitArgs {
  int H, N, d, G_q, M, rank;
  float scale;
  double lambda;
  bool bf16;
  const void *Q, *K, *V;
  const int32_t *q_label, *q_off, *q_perm;
  const double* q_dist;
  const float* Op;
  int32_t* probe_idx;
  double* probe_w;
  float* O_probe;
  double *r_bar, *x_bar, *B_r, *V_r;
  int32_t* rank_eff;
  Workspace ws;
  hipStream_t stream;
};

struct CorrectArgs {
  int H, N, d, M, rank;
  bool bf16;
  const float* Op;
  const int32_t* q_perm;
  const int32_t* probe_idx;
  const float* O_probe;
  const double *r_bar, *x_bar, *B_r, *V_r;
  const int32_t* rank_eff;
  void* O;
  Workspace ws;
  hipStream_t stream;
};

struct DenseArgs {
  int H, N, d;
  float scale;
  bool bf16;
  const void *Q, *K, *V;
  void* O;
  float* lse;
  uint16_t* vh;      // [H,N,d] scratch (bf16 inputs)
  float *vpart, *vinv, *vscale;   // [H,64], [H], [H] scratch: the per-head scale of vh
  hipStream_t stream;
};

// Static scratch of sparsepr_route_noalloc: H * G_q * G_k cells of float64
// scores and uint8 flags, at most kRouteScratchBytes (2^22 cells).
constexpr size_t kRouteScratchBytes = ((size_t)1 << 22) * 9;
// device address of that scratch on the current device (looked up once per device)
hipError_t route_scratch(void** out);
size_t route_scratch_need(int H, int G_q, int G_k);
void route_scratch_carve(void* base, int H, int G_q, int G_k, Workspace* w);

hipError_t launch_partition(const PartitionArgs& a);
hipError_t launch_route(const RouteArgs& a);
hipError_t launch_attend(const AttendArgs& a);
hipError_t launch_probe_fit(const ProbeFitArgs& a);
hipError_t launch_correct(const CorrectArgs& a);
hipError_t launch_dense(const DenseArgs& a);
// Measurement hook: records a HIP event on st (begin or end of the
// block-sparse attention kernel) while kernel timing is enabled.
void kernel_timer_mark(hipStream_t st);
// key splits the sparse pass uses for this shape (workspace sizing and launch agree)
int attend_splits(int H, int N, int G_q, bool bf16);

// matrix-core rate probe: blocks x 256 threads, iters rounds of 4 bf16 MFMAs per wave
hipError_t launch_mfma_rate(int blocks, int iters, float* sink, hipStream_t st);
hipError_t launch_tile_rate(int blocks, int iters, float* sink, hipStream_t st);

// leading nev (1..d) eigenpairs of symmetric A [H,d,d] (d = 64 or 128), one
// block per matrix: eigval [H,d] entries 0..nev-1 (descending), eigvec [H,d,d]
// rows 0..nev-1 (unit, largest-magnitude entry positive), trace [H] = tr A.
// A is not modified; the other entries are not written.
// leading nev eigenpairs of H symmetric d x d matrices; scratch holds
// sym_eig_scratch(H, d) doubles
void launch_sym_eig_top(const double* A, int H, int d, int nev, double* eigval, double* eigvec, double* trace,
                        double* scratch, hipStream_t st);
size_t sym_eig_scratch(int H, int d);

}  // namespace spr
