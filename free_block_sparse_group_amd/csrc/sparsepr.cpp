// C-ABI entry points: argument validation, workspace carving and launch
// sequencing for the SparsePR attention call.  Every check runs on the host
// before anything is enqueued; kernels are in the *.hip files.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sparsepr.h"
#include "kernels.hpp"

namespace spr {
void init_linalg_attributes();
void init_attention_attributes();
void init_probe_attributes();
void init_partition_attributes();
}  // namespace spr

namespace {
// events recorded around the block-sparse attention kernel while timing is on
std::mutex g_timer_mu;
std::atomic<bool> g_timer_on{false};
std::vector<hipEvent_t> g_timer_events;   // begin, end, begin, end, ...

void clear_timer_events() {
  for (hipEvent_t e : g_timer_events) hipEventDestroy(e);
  g_timer_events.clear();
}
}  // namespace

void spr::kernel_timer_mark(hipStream_t st) {
  if (!g_timer_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return;
  hipEventRecord(e, st);
  g_timer_events.push_back(e);
}

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SPARSEPR_OK;
}

void init_once() {
  static std::once_flag flag;
  std::call_once(flag, [] {
    spr::init_linalg_attributes();
    spr::init_attention_attributes();
    spr::init_probe_attributes();
    spr::init_partition_attributes();
  });
}

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPARSEPR_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- validation -----------------------------------------------------------

int check_shape(const sparsepr_shape* s) {
  if (!s) return fail(SPARSEPR_EINVAL, "shape is null");
  if (s->H < 1 || s->N < 1) return fail(SPARSEPR_EINVAL, "H and N must be >= 1 (got H=%d N=%d)", s->H, s->N);
  if (s->N >= (1 << 30)) return fail(SPARSEPR_EUNSUPPORTED, "N must be < 2^30 (got %d)", s->N);
  if (s->d != 64 && s->d != 128) return fail(SPARSEPR_EUNSUPPORTED, "d must be 64 or 128 (got %d)", s->d);
  if (s->dtype != SPARSEPR_F32 && s->dtype != SPARSEPR_BF16)
    return fail(SPARSEPR_EUNSUPPORTED, "dtype must be SPARSEPR_F32 or SPARSEPR_BF16 (got %d)", s->dtype);
  if (!(s->scale >= 0.0f) || std::isinf(s->scale)) return fail(SPARSEPR_EINVAL, "scale must be finite and >= 0");
  return SPARSEPR_OK;
}

int check_groups(const sparsepr_shape* s, const sparsepr_partition_params* p) {
  if (!p) return fail(SPARSEPR_EINVAL, "partition params are null");
  if (p->G_k < 1 || p->G_k > s->N || p->G_q < 1 || p->G_q > s->N)
    return fail(SPARSEPR_EINVAL, "need 1 <= G_k, G_q <= N (got G_k=%d G_q=%d N=%d)", p->G_k, p->G_q, s->N);
  if (p->G_k > spr::kMaxGroups || p->G_q > spr::kMaxGroups)
    return fail(SPARSEPR_EUNSUPPORTED, "G_k and G_q must be <= %d", spr::kMaxGroups);
  return SPARSEPR_OK;
}

int check_partition(const sparsepr_shape* s, const sparsepr_partition_params* p) {
  int rc = check_groups(s, p);
  if (rc) return rc;
  if (p->M_s < 1 || p->M_s > s->N) return fail(SPARSEPR_EINVAL, "need 1 <= M_s <= N (got %d)", p->M_s);
  if (p->r_k < 1 || p->r_k > s->d) return fail(SPARSEPR_EINVAL, "need 1 <= r_k <= d (got %d)", p->r_k);
  if (p->iters_kv < 1 || p->iters_q < 1) return fail(SPARSEPR_EINVAL, "k-means iterations must be >= 1");
  if (!(p->eig_weight_power >= 0.0) || std::isinf(p->eig_weight_power))
    return fail(SPARSEPR_EINVAL, "eig_weight_power must be finite and >= 0");
  if (p->semantic != 0 && p->semantic != 1) return fail(SPARSEPR_EINVAL, "semantic must be 0 or 1");
  if (p->warm != 0 && p->warm != 1) return fail(SPARSEPR_EINVAL, "warm must be 0 or 1");
  return SPARSEPR_OK;
}

int check_route(const sparsepr_shape* s, const sparsepr_route_params* r) {
  if (!r) return fail(SPARSEPR_EINVAL, "route params are null");
  if (r->top_k < 0) return fail(SPARSEPR_EINVAL, "top_k must be >= 0");
  if (r->top_k == 0 && !(r->density > 0.0 && r->density <= 1.0))
    return fail(SPARSEPR_EINVAL, "density must be in (0, 1] when top_k == 0");
  if (r->M < 0 || r->M > s->N) return fail(SPARSEPR_EINVAL, "need 0 <= M <= N (got %d)", r->M);
  return SPARSEPR_OK;
}

int check_fit(const sparsepr_shape* s, const sparsepr_fit_params* f) {
  if (!f) return fail(SPARSEPR_EINVAL, "fit params are null");
  if (f->M < 0 || f->M > s->N) return fail(SPARSEPR_EINVAL, "need 0 <= M <= N (got %d)", f->M);
  if (f->M > spr::kMaxProbes) return fail(SPARSEPR_EUNSUPPORTED, "M must be <= %d", spr::kMaxProbes);
  if (f->rank < 0 || f->rank > s->d) return fail(SPARSEPR_EINVAL, "need 0 <= rank <= d (got %d)", f->rank);
  if (!(f->lambda >= 0.0) || std::isinf(f->lambda)) return fail(SPARSEPR_EINVAL, "lambda must be finite and >= 0");
  // weighted centring leaves the M probe regressors a rank of at most M - 1,
  // so without the ridge term the d x d fit matrix is singular whenever M <= d
  // and the fit would hinge on how rounding lands on a zero pivot
  if (f->lambda == 0.0 && f->rank > 0 && f->M > 0 && f->M <= s->d)
    return fail(SPARSEPR_EINVAL, "lambda = 0 needs more probes than head dims (M=%d, d=%d): the fit matrix is singular",
                f->M, s->d);
  return SPARSEPR_OK;
}

#define REQUIRE_PTR(p)                                                           \
  do {                                                                           \
    if (!(p)) return fail(SPARSEPR_EINVAL, "pointer argument '%s' is null", #p); \
  } while (0)

// ---- workspace ------------------------------------------------------------

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

double softmax_scale(const sparsepr_shape* s) { return s->scale > 0.0f ? (double)s->scale : std::pow((double)s->d, -0.5); }

size_t carve_partition(const sparsepr_shape* s, const sparsepr_partition_params* p, char* base, spr::Workspace* w) {
  const size_t H = s->H, N = s->N, d = s->d;
  const size_t Gmax = std::max(p->G_k, p->G_q), Dmax = d, nch = (N + spr::kSortChunk - 1) / spr::kSortChunk;
  Carver c{base};
  spr::Workspace t{};
  t.mk = c.take<double>(H * d * d);
  t.eigval = c.take<double>(H * d);
  t.eigvec = c.take<double>(H * d * d);
  t.mtrace = c.take<double>(H);
  t.eigscr = c.take<double>(spr::sym_eig_scratch((int)H, (int)d));
  t.wk = c.take<double>(H * d);
  t.Z = c.take<double>(H * N * p->r_k);
  t.qscale = c.take<double>(H * N);
  t.metric = c.take<double>(H * d * d);
  t.gprime = c.take<int32_t>(H);
  t.cent = c.take<double>(H * Gmax * Dmax);
  t.centp = c.take<double>(H * Gmax * Dmax);
  t.cnorm = c.take<double>(H * Gmax);
  t.counts = c.take<int32_t>(H * nch * Gmax);
  t.base = c.take<int32_t>(H * nch * Gmax);
  t.sortpart = c.take<int32_t>(H * spr::kSortSlices * 1024);
  const size_t DP = (size_t)spr::lp_dims((int)d);   // r_k <= d, so this covers both k-means
  t.lp.xh = c.take<uint16_t>(H * N * DP);
  t.lp.xl = c.take<uint16_t>(H * N * DP);
  t.lp.xe = c.take<int32_t>(H * N);
  t.lp.xn = c.take<float>(H * N);
  t.lp.ch = c.take<uint16_t>(H * Gmax * DP);
  t.lp.cl = c.take<uint16_t>(H * Gmax * DP);
  t.lp.ce = c.take<int32_t>(H * Gmax);
  t.lp.cn32 = c.take<float>(H * Gmax);
  t.lp.cnrm = c.take<float>(H * Gmax);
  t.lp.cpt = c.take<double>(H * Gmax * Dmax);
  t.lp.list = c.take<int32_t>(H * N);
  t.lp.cnt = c.take<int32_t>(H);
  if (w) *w = t;
  return c.off;
}

size_t carve_route(const sparsepr_shape* s, const sparsepr_partition_params* p, char* base, spr::Workspace* w) {
  Carver c{base};
  spr::Workspace t{};
  t.P = c.take<double>((size_t)s->H * p->G_q * p->G_k);
  t.sel = c.take<uint8_t>((size_t)s->H * p->G_q * p->G_k);
  if (w) *w = t;
  return c.off;
}

size_t carve_attend(const sparsepr_shape* s, const sparsepr_partition_params* p, char* base, spr::Workspace* w) {
  Carver c{base};
  spr::Workspace t{};
  t.tiles = c.take<int32_t>((size_t)s->H * (p->G_q + 1));
  t.tdesc = c.take<int4>((size_t)s->H * ((s->N + spr::kAttnBM - 1) / spr::kAttnBM + p->G_q));
  t.segs = c.take<int2>((size_t)s->H * p->G_q * p->G_k);
  t.vh = s->dtype == SPARSEPR_BF16 ? c.take<uint16_t>((size_t)s->H * s->N * s->d) : nullptr;
  t.vpart = c.take<float>((size_t)s->H * 64);
  t.vinv = c.take<float>((size_t)s->H);
  t.vscale = c.take<float>((size_t)s->H);
  const size_t S = (size_t)spr::attend_splits(s->H, s->N, p->G_q, s->dtype == SPARSEPR_BF16);
  if (S > 1) {
    t.spart = c.take<float>(S * s->H * s->N * s->d);
    t.smpart = c.take<float>(S * s->H * s->N);
    t.slpart = c.take<float>(S * s->H * s->N);
  }
  if (w) *w = t;
  return c.off;
}

size_t carve_probe_fit(const sparsepr_shape* s, const sparsepr_partition_params* p, const sparsepr_fit_params* f,
                       char* base, spr::Workspace* w) {
  const size_t H = s->H, N = s->N, d = s->d, M = std::max(f->M, 1), S = spr::kProbeSplits;
  Carver c{base};
  spr::Workspace t{};
  t.alloc = c.take<int32_t>(H * p->G_q);
  t.pgroup = c.take<int32_t>(H * M);
  t.prank = c.take<int32_t>(H * M);
  t.pt = c.take<int32_t>(H * M);
  t.pslot = c.take<int32_t>(H * M);
  t.probe_slot = c.take<int32_t>(H * M);
  t.opart = c.take<float>(S * H * M * d);
  t.mpart = c.take<float>(S * H * M);
  t.lpart = c.take<float>(S * H * M);
  t.fx = c.take<double>(H * M * d);
  t.fr = c.take<double>(H * M * d);
  t.gram = c.take<double>(3 * H * d * d);
  t.feig = c.take<double>(H * d);
  t.fvec = c.take<double>(H * d * d);
  t.ftrace = c.take<double>(H);
  t.eigscr = c.take<double>(spr::sym_eig_scratch((int)H, (int)d));
  t.frhs = c.take<double>(H * d * std::max(f->rank, 1));
  t.vh = s->dtype == SPARSEPR_BF16 ? c.take<uint16_t>(H * N * d) : nullptr;
  t.vpart = c.take<float>(H * 64);
  t.vinv = c.take<float>(H);
  t.vscale = c.take<float>(H);
  if (w) *w = t;
  return c.off;
}

size_t carve_correct(const sparsepr_shape* s, const sparsepr_fit_params* f, char* base, spr::Workspace* w) {
  const size_t H = s->H, d = s->d, nch = std::max<size_t>(1, ((size_t)f->rank + 31) / 32);
  Carver c{base};
  spr::Workspace t{};
  t.probe_pos = c.take<int32_t>(H * s->N);
  t.corr_b = c.take<float>(H * nch * (d / 2) * 64);
  t.corr_c = c.take<float>(H * nch * 32);
  t.corr_h = c.take<uint16_t>(H * nch * 2 * 32 * d);
  t.corr_e = c.take<int32_t>(H * nch);
  if (w) *w = t;
  return c.off;
}

size_t carve_dense(const sparsepr_shape* s, char* base, spr::DenseArgs* a) {
  Carver c{base};
  const bool bf = s->dtype == SPARSEPR_BF16;
  uint16_t* t = bf ? c.take<uint16_t>((size_t)s->H * s->N * s->d) : nullptr;
  float* vpart = bf ? c.take<float>((size_t)s->H * 64) : nullptr;
  float* vinv = bf ? c.take<float>((size_t)s->H) : nullptr;
  float* vscale = bf ? c.take<float>((size_t)s->H) : nullptr;
  if (a) { a->vh = t; a->vpart = vpart; a->vinv = vinv; a->vscale = vscale; }
  return c.off;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need > 0 && !ws) return fail(SPARSEPR_EINVAL, "workspace pointer is null");
  if (have < need) return fail(SPARSEPR_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", have, need);
  return SPARSEPR_OK;
}

}  // namespace

extern "C" {

const char* sparsepr_last_error(void) { return g_err.c_str(); }

const char* sparsepr_version(void) { return "sparsepr-gfx950 0.1.0"; }

int sparsepr_attend_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  clear_timer_events();
  g_timer_on.store(enable != 0);
  return SPARSEPR_OK;
}

int sparsepr_attend_kernel_time(double* total_ms, int* launches) {
  if (!total_ms || !launches) return fail(SPARSEPR_EINVAL, "null output pointer");
  std::lock_guard<std::mutex> lk(g_timer_mu);
  double sum = 0.0;
  const size_t n = g_timer_events.size() / 2;
  for (size_t i = 0; i < n; ++i) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(g_timer_events[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timer_events[2 * i], g_timer_events[2 * i + 1]);
    if (e != hipSuccess) return fail(SPARSEPR_EHIP, "kernel timing events: %s", hipGetErrorString(e));
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int)n;
  return SPARSEPR_OK;
}

size_t sparsepr_workspace_size(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                               const sparsepr_route_params* rp, const sparsepr_fit_params* fp) {
  if (check_shape(shape) || check_partition(shape, pp) || check_route(shape, rp) || check_fit(shape, fp)) return 0;
  size_t need = carve_partition(shape, pp, nullptr, nullptr);
  need = std::max(need, carve_route(shape, pp, nullptr, nullptr));
  need = std::max(need, carve_attend(shape, pp, nullptr, nullptr));
  need = std::max(need, carve_probe_fit(shape, pp, fp, nullptr, nullptr));
  need = std::max(need, carve_correct(shape, fp, nullptr, nullptr));
  g_err.clear();
  return need;
}

int sparsepr_partition(const sparsepr_shape* shape, const sparsepr_partition_params* pp, const void* Q, const void* K,
                       const void* V, int32_t* kv_label, int32_t* q_label, int32_t* kv_perm, int32_t* q_perm,
                       int32_t* kv_off, int32_t* q_off, void* Qp, void* Kp, void* Vp, double* kv_centroid,
                       double* q_centroid, double* q_dist, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_partition(shape, pp))) return rc;
  REQUIRE_PTR(Q); REQUIRE_PTR(K); REQUIRE_PTR(V);
  REQUIRE_PTR(kv_label); REQUIRE_PTR(q_label); REQUIRE_PTR(kv_perm); REQUIRE_PTR(q_perm);
  REQUIRE_PTR(kv_off); REQUIRE_PTR(q_off); REQUIRE_PTR(Qp); REQUIRE_PTR(Kp); REQUIRE_PTR(Vp);
  REQUIRE_PTR(kv_centroid); REQUIRE_PTR(q_centroid); REQUIRE_PTR(q_dist);
  if ((rc = check_ws(ws, ws_bytes, carve_partition(shape, pp, nullptr, nullptr)))) return rc;
  init_once();
  spr::PartitionArgs a{};
  a.H = shape->H; a.N = shape->N; a.d = shape->d;
  a.G_k = pp->G_k; a.G_q = pp->G_q; a.M_s = pp->M_s; a.r_k = pp->r_k;
  a.iters_kv = pp->iters_kv; a.iters_q = pp->iters_q; a.eig_power = pp->eig_weight_power;
  a.semantic = pp->semantic != 0;
  a.warm = pp->warm != 0;
  a.bf16 = shape->dtype == SPARSEPR_BF16;
  a.Q = Q; a.K = K; a.V = V;
  a.kv_label = kv_label; a.q_label = q_label; a.kv_perm = kv_perm; a.q_perm = q_perm;
  a.kv_off = kv_off; a.q_off = q_off; a.Qp = Qp; a.Kp = Kp; a.Vp = Vp;
  a.kv_centroid = kv_centroid; a.q_centroid = q_centroid; a.q_dist = q_dist;
  carve_partition(shape, pp, static_cast<char*>(ws), &a.ws);
  a.stream = static_cast<hipStream_t>(stream);
  return check_hip(spr::launch_partition(a), "sparsepr_partition launch");
}

int sparsepr_route(const sparsepr_shape* shape, const sparsepr_partition_params* pp, const sparsepr_route_params* rp,
                   const int32_t* kv_off, const int32_t* q_off, const double* kv_centroid, const double* q_centroid,
                   int32_t* row_ptr, int32_t* col_idx, int64_t* routed_pairs, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_groups(shape, pp))) return rc;
  if ((rc = check_route(shape, rp))) return rc;
  REQUIRE_PTR(kv_off); REQUIRE_PTR(q_off); REQUIRE_PTR(kv_centroid); REQUIRE_PTR(q_centroid);
  REQUIRE_PTR(row_ptr); REQUIRE_PTR(col_idx); REQUIRE_PTR(routed_pairs);
  if ((rc = check_ws(ws, ws_bytes, carve_route(shape, pp, nullptr, nullptr)))) return rc;
  init_once();
  spr::RouteArgs a{};
  a.H = shape->H; a.N = shape->N; a.d = shape->d; a.G_k = pp->G_k; a.G_q = pp->G_q;
  a.top_k = rp->top_k; a.M = rp->M; a.density = rp->density; a.scale = softmax_scale(shape);
  a.kv_off = kv_off; a.q_off = q_off; a.kv_centroid = kv_centroid; a.q_centroid = q_centroid;
  a.row_ptr = row_ptr; a.col_idx = col_idx; a.routed_pairs = routed_pairs;
  carve_route(shape, pp, static_cast<char*>(ws), &a.ws);
  a.stream = static_cast<hipStream_t>(stream);
  return check_hip(spr::launch_route(a), "sparsepr_route launch");
}

int sparsepr_route_noalloc(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                           const sparsepr_route_params* rp, const int32_t* kv_off, const int32_t* q_off,
                           const double* kv_centroid, const double* q_centroid, int32_t* row_ptr, int32_t* col_idx,
                           int64_t* routed_pairs, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_groups(shape, pp))) return rc;
  if ((rc = check_route(shape, rp))) return rc;
  REQUIRE_PTR(kv_off); REQUIRE_PTR(q_off); REQUIRE_PTR(kv_centroid); REQUIRE_PTR(q_centroid);
  REQUIRE_PTR(row_ptr); REQUIRE_PTR(col_idx); REQUIRE_PTR(routed_pairs);
  const size_t need = spr::route_scratch_need(shape->H, pp->G_q, pp->G_k);
  if (need > spr::kRouteScratchBytes)
    return fail(SPARSEPR_EWORKSPACE,
                "sparsepr_route_noalloc: H*G_q*G_k = %lld cells need %zu bytes of scratch; its static scratch holds "
                "%zu (2^22 cells)",
                (long long)shape->H * pp->G_q * pp->G_k, need, spr::kRouteScratchBytes);
  init_once();
  void* scr = nullptr;
  if ((rc = check_hip(spr::route_scratch(&scr), "sparsepr_route_noalloc scratch address"))) return rc;
  spr::RouteArgs a{};
  a.H = shape->H; a.N = shape->N; a.d = shape->d; a.G_k = pp->G_k; a.G_q = pp->G_q;
  a.top_k = rp->top_k; a.M = rp->M; a.density = rp->density; a.scale = softmax_scale(shape);
  a.kv_off = kv_off; a.q_off = q_off; a.kv_centroid = kv_centroid; a.q_centroid = q_centroid;
  a.row_ptr = row_ptr; a.col_idx = col_idx; a.routed_pairs = routed_pairs;
  spr::route_scratch_carve(scr, shape->H, pp->G_q, pp->G_k, &a.ws);
  a.stream = static_cast<hipStream_t>(stream);
  return check_hip(spr::launch_route(a), "sparsepr_route_noalloc launch");
}

int sparsepr_attend(const sparsepr_shape* shape, const sparsepr_partition_params* pp, const void* Qp, const void* Kp,
                    const void* Vp, const int32_t* q_off, const int32_t* kv_off, const int32_t* row_ptr,
                    const int32_t* col_idx, float* Op, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_groups(shape, pp))) return rc;
  REQUIRE_PTR(Qp); REQUIRE_PTR(Kp); REQUIRE_PTR(Vp); REQUIRE_PTR(q_off); REQUIRE_PTR(kv_off);
  REQUIRE_PTR(row_ptr); REQUIRE_PTR(col_idx); REQUIRE_PTR(Op); REQUIRE_PTR(lse);
  if ((rc = check_ws(ws, ws_bytes, carve_attend(shape, pp, nullptr, nullptr)))) return rc;
  init_once();
  spr::AttendArgs a{};
  a.H = shape->H; a.N = shape->N; a.d = shape->d; a.G_k = pp->G_k; a.G_q = pp->G_q;
  a.scale = (float)softmax_scale(shape);
  a.bf16 = shape->dtype == SPARSEPR_BF16;
  a.Qp = Qp; a.Kp = Kp; a.Vp = Vp; a.q_off = q_off; a.kv_off = kv_off; a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.Op = Op; a.lse = lse;
  carve_attend(shape, pp, static_cast<char*>(ws), &a.ws);
  a.stream = static_cast<hipStream_t>(stream);
  return check_hip(spr::launch_attend(a), "sparsepr_attend launch");
}

int sparsepr_probe_fit(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                       const sparsepr_fit_params* fp, const void* Q, const void* K, const void* V,
                       const int32_t* q_label, const int32_t* q_off, const int32_t* q_perm, const double* q_dist,
                       const float* Op, int32_t* probe_idx, double* probe_w, float* O_probe, double* r_bar,
                       double* x_bar, double* B_r, double* V_r, int32_t* rank_eff, void* ws, size_t ws_bytes,
                       void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_groups(shape, pp))) return rc;
  if ((rc = check_fit(shape, fp))) return rc;
  if (fp->M == 0) return ok();
  REQUIRE_PTR(Q); REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(q_label); REQUIRE_PTR(q_off);
  REQUIRE_PTR(q_perm); REQUIRE_PTR(q_dist); REQUIRE_PTR(Op); REQUIRE_PTR(probe_idx); REQUIRE_PTR(probe_w);
  REQUIRE_PTR(O_probe); REQUIRE_PTR(r_bar); REQUIRE_PTR(x_bar); REQUIRE_PTR(rank_eff);
  if (fp->rank > 0) { REQUIRE_PTR(B_r); REQUIRE_PTR(V_r); }
  if ((rc = check_ws(ws, ws_bytes, carve_probe_fit(shape, pp, fp, nullptr, nullptr)))) return rc;
  init_once();
  spr::ProbeFitArgs a{};
  a.H = shape->H; a.N = shape->N; a.d = shape->d; a.G_q = pp->G_q; a.M = fp->M; a.rank = fp->rank;
  a.scale = (float)softmax_scale(shape); a.lambda = fp->lambda;
  a.bf16 = shape->dtype == SPARSEPR_BF16;
  a.Q = Q; a.K = K; a.V = V; a.q_label = q_label; a.q_off = q_off; a.q_perm = q_perm; a.q_dist = q_dist;
  a.Op = Op; a.probe_idx = probe_idx; a.probe_w = probe_w; a.O_probe = O_probe;
  a.r_bar = r_bar; a.x_bar = x_bar; a.B_r = B_r; a.V_r = V_r; a.rank_eff = rank_eff;
  carve_probe_fit(shape, pp, fp, static_cast<char*>(ws), &a.ws);
  a.stream = static_cast<hipStream_t>(stream);
  return check_hip(spr::launch_probe_fit(a), "sparsepr_probe_fit launch");
}

int sparsepr_correct(const sparsepr_shape* shape, const sparsepr_fit_params* fp, const float* Op,
                     const int32_t* q_perm, const int32_t* probe_idx, const float* O_probe, const double* r_bar,
                     const double* x_bar, const double* B_r, const double* V_r, const int32_t* rank_eff, void* O,
                     void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_fit(shape, fp))) return rc;
  REQUIRE_PTR(Op); REQUIRE_PTR(q_perm); REQUIRE_PTR(O);
  if (fp->M > 0) {
    REQUIRE_PTR(probe_idx); REQUIRE_PTR(O_probe); REQUIRE_PTR(r_bar); REQUIRE_PTR(x_bar); REQUIRE_PTR(rank_eff);
    if (fp->rank > 0) { REQUIRE_PTR(B_r); REQUIRE_PTR(V_r); }
  }
  if ((rc = check_ws(ws, ws_bytes, fp->M > 0 ? carve_correct(shape, fp, nullptr, nullptr) : 0))) return rc;
  init_once();
  spr::CorrectArgs a{};
  a.H = shape->H; a.N = shape->N; a.d = shape->d; a.M = fp->M; a.rank = fp->rank;
  a.bf16 = shape->dtype == SPARSEPR_BF16;
  a.Op = Op; a.q_perm = q_perm; a.probe_idx = probe_idx; a.O_probe = O_probe;
  a.r_bar = r_bar; a.x_bar = x_bar; a.B_r = B_r; a.V_r = V_r; a.rank_eff = rank_eff; a.O = O;
  if (fp->M > 0) carve_correct(shape, fp, static_cast<char*>(ws), &a.ws);
  a.stream = static_cast<hipStream_t>(stream);
  return check_hip(spr::launch_correct(a), "sparsepr_correct launch");
}

size_t sparsepr_dense_workspace_size(const sparsepr_shape* shape) {
  if (check_shape(shape)) return 0;
  g_err.clear();
  return std::max<size_t>(carve_dense(shape, nullptr, nullptr), 1);
}

int sparsepr_dense_attend(const sparsepr_shape* shape, const void* Q, const void* K, const void* V, void* O,
                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE_PTR(Q); REQUIRE_PTR(K); REQUIRE_PTR(V); REQUIRE_PTR(O); REQUIRE_PTR(lse);
  if ((rc = check_ws(ws, ws_bytes, carve_dense(shape, nullptr, nullptr)))) return rc;
  init_once();
  spr::DenseArgs a{};
  a.H = shape->H; a.N = shape->N; a.d = shape->d;
  a.scale = (float)softmax_scale(shape);
  a.bf16 = shape->dtype == SPARSEPR_BF16;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.lse = lse;
  carve_dense(shape, static_cast<char*>(ws), &a);
  a.stream = static_cast<hipStream_t>(stream);
  return check_hip(spr::launch_dense(a), "sparsepr_dense_attend launch");
}

size_t sparsepr_sym_eigen_workspace_size(int32_t H, int32_t d) {
  if (H < 1) return fail(SPARSEPR_EINVAL, "H must be >= 1 (got %d)", H), 0;
  if (d != 64 && d != 128) return fail(SPARSEPR_EUNSUPPORTED, "d must be 64 or 128 (got %d)", d), 0;
  g_err.clear();
  return (spr::sym_eig_scratch(H, d) + (size_t)H) * sizeof(double);
}

int sparsepr_sym_eigen(int32_t H, int32_t d, int32_t nev, const double* A, double* eigval, double* eigvec, void* ws,
                       size_t ws_bytes, void* stream) {
  const size_t need = sparsepr_sym_eigen_workspace_size(H, d);
  if (need == 0) return H < 1 ? SPARSEPR_EINVAL : SPARSEPR_EUNSUPPORTED;
  if (nev < 1 || nev > d) return fail(SPARSEPR_EINVAL, "need 1 <= nev <= d (got nev=%d, d=%d)", nev, d);
  REQUIRE_PTR(A); REQUIRE_PTR(eigval); REQUIRE_PTR(eigvec);
  int rc = check_ws(ws, ws_bytes, need);
  if (rc) return rc;
  init_once();
  double* scr = static_cast<double*>(ws);
  double* trace = scr + spr::sym_eig_scratch(H, d);
  spr::launch_sym_eig_top(A, H, d, nev, eigval, eigvec, trace, scr, static_cast<hipStream_t>(stream));
  return check_hip(hipGetLastError(), "sparsepr_sym_eigen launch");
}

int sparsepr_mfma_rate_probe(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks < 1 || iters < 1) return fail(SPARSEPR_EINVAL, "sparsepr_mfma_rate_probe: blocks and iters must be >= 1");
  REQUIRE_PTR(sink);
  return check_hip(spr::launch_mfma_rate(blocks, iters, sink, static_cast<hipStream_t>(stream)),
                   "sparsepr_mfma_rate_probe launch");
}

int sparsepr_tile_rate_probe(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks < 1 || iters < 1) return fail(SPARSEPR_EINVAL, "sparsepr_tile_rate_probe: blocks and iters must be >= 1");
  REQUIRE_PTR(sink);
  return check_hip(spr::launch_tile_rate(blocks, iters, sink, static_cast<hipStream_t>(stream)),
                   "sparsepr_tile_rate_probe launch");
}

}  // extern "C"
