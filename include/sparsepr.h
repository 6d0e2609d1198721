/*
 * sparsepr.h -- C ABI of the SparsePR attention call on AMD Instinct MI355X (gfx950).
 *
 * Method: "Partition the Support, Reconstruct the Residual: Training-Free
 * Sparse Attention for Video Generation and World Models" (Taghavi, Langari,
 * Pandey, arXiv:2608.18484).  Citations name the page and its section:
 * "paperlayer.ai s4" = the paperlayer.ai summary, section 4 (Method); "A.2",
 * "B.1", "C.1" ... = its appendices; "gist-nl s2" = the gist.science Dutch
 * technical summary, section 2.
 *
 * One call = five stages, each an entry point, run in this order on one HIP
 * stream for a batch of H independent heads (self-attention, N queries = N
 * keys, head dim d, non-causal):
 *   sparsepr_partition -> sparsepr_route -> sparsepr_attend
 *     -> sparsepr_probe_fit -> sparsepr_correct
 *
 * Conventions (all entry points)
 *  - Pointers marked [device] are device memory owned by the caller; the
 *    library never allocates, frees or keeps them, and holds no state between
 *    calls.  Scratch memory comes from the caller's workspace `ws`
 *    (ws_bytes >= sparsepr_workspace_size(...); contents on entry are ignored).
 *  - Every tensor is contiguous row-major.  [H,N,d] means head-major, then
 *    token, then channel.  Index tensors are int32 unless stated.
 *    perm[h][slot] = original token index placed at that slot.
 *  - `stream` is a hipStream_t passed as void*.  Work is enqueued
 *    asynchronously; no entry point synchronises the host, and sizes that
 *    depend on data (routed cells, probe sets) stay on the device.
 *  - Arguments are checked on the host before anything is enqueued; on any
 *    error nothing is launched and a negative sparsepr_status is returned;
 *    sparsepr_last_error() then describes it (thread-local, valid until the
 *    next call on that thread).
 *  - Results are deterministic: the same inputs give bitwise-identical
 *    outputs (no floating-point atomics; fixed reduction orders).
 *  - Supported: d in {64, 128}; dtype bf16 or fp32 for Q/K/V and the final
 *    output; 1 <= G_k, G_q <= 1024; 0 <= M <= 4096, M <= N; N < 2^30.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARSEPR_OK = 0,
  SPARSEPR_EINVAL = -1,        /* bad shape, parameter or null pointer            */
  SPARSEPR_EWORKSPACE = -2,    /* ws_bytes below sparsepr_workspace_size()        */
  SPARSEPR_EHIP = -3,          /* a HIP runtime call or kernel launch failed      */
  SPARSEPR_EUNSUPPORTED = -4   /* valid but outside what this build implements    */
} sparsepr_status;

typedef enum { SPARSEPR_F32 = 0, SPARSEPR_BF16 = 1 } sparsepr_dtype;

typedef struct {
  int32_t H, N, d;   /* heads, tokens, head dim                                  */
  int32_t dtype;     /* sparsepr_dtype of Q, K, V, Qp/Kp/Vp and the output O      */
  float scale;       /* softmax scale; 0 selects 1/sqrt(d)                         */
} sparsepr_shape;

/* Response-coupled partition (gist-nl s2A; paperlayer.ai s4, B.1, B.2). */
typedef struct {
  int32_t G_k;               /* K/V groups                                        */
  int32_t G_q;               /* query groups                                      */
  int32_t M_s;               /* sampled queries for M_K = Q_s^T Q_s / M_s         */
  int32_t r_k;               /* key-response coordinate rank, 1 <= r_k <= d        */
  int32_t iters_kv, iters_q; /* Lloyd iterations (>= 1) for keys and queries       */
  double eig_weight_power;   /* eigen weights (lambda/sum)^p; 0.5 by default       */
  int32_t semantic;          /* 0: response-coupled (the method); 1: the semantic
                                baseline of the pages' ablations (s3.1 O3, appendix
                                D): k-means on the raw keys and on the raw queries,
                                same counts, rules and iterations; M_s, r_k and
                                eig_weight_power are then unused                  */
  int32_t warm;              /* 0: k-means starts at the centred-stride rows; 1:
                                warm start across successive calls (C.1): kv_label
                                and q_label hold the previous call's labels on
                                entry (values clamped into [0, G)), each group with
                                members starts at its members' mean in this call's
                                coordinates, an empty one at its stride row        */
} sparsepr_partition_params;

/* Routing under a query-key pair budget (paperlayer.ai s4 "Sparse Execution"). */
typedef struct {
  int32_t top_k;   /* > 0: each query group keeps its top_k cells; 0: pair budget  */
  double density;  /* executed-pair target in (0,1], probe rows included (s5, C.3) */
  int32_t M;       /* probe rows (their M*N pairs come out of the budget)           */
} sparsepr_route_params;

/* Probe-fitted residual reconstruction (gist-nl s2B; paperlayer.ai s4, A.2, A.3). */
typedef struct {
  int32_t M;       /* exact probe rows, 0 <= M <= min(N, 4096)                     */
  int32_t rank;    /* subspace rank r, 0 <= r <= d                                 */
  double lambda;   /* ridge regularisation, >= 0 (weights sum to 1); 0 only with M > d or rank 0 */
} sparsepr_fit_params;

/* Bytes of device workspace needed by every entry point for these arguments;
 * 0 if the arguments are invalid (sparsepr_last_error() says why).           */
size_t sparsepr_workspace_size(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                               const sparsepr_route_params* rp, const sparsepr_fit_params* fp);

/* Message for the last failing call on this thread ("" if none). */
const char* sparsepr_last_error(void);

/* Library version string. */
const char* sparsepr_version(void);

/*
 * Stage 1 -- response-coupled partition and group-major permutation
 * (gist-nl s2A; paperlayer.ai s4 "Response-Coupled Partitioning",
 * B.1 "Key-response coordinates", B.2 "Query-response coordinates", C.1;
 * layout: s4 "Sparse Execution").
 * Per head: deterministic sampled queries -> M_K -> eigen-weighted key
 * coordinates -> k-means -> paired K/V groups (V inherits the key's label);
 * nonempty K/V-group key centroids, centred with equal weights -> RMS-normalised
 * query logit profiles -> k-means -> query groups.  One asymmetric pass.
 * In  [device]: Q, K, V [H,N,d] dtype, original token order.
 * Out [device]: kv_label, q_label [H,N]; kv_perm, q_perm [H,N] (stable:
 *   ascending original index inside a group); kv_off [H,G_k+1], q_off [H,G_q+1]
 *   (exclusive prefix sums of group sizes); Qp = Q[q_perm], Kp = K[kv_perm],
 *   Vp = V[kv_perm] [H,N,d] dtype; kv_centroid [H,G_k,d] and q_centroid
 *   [H,G_q,d] float64 means of the raw keys / queries of each group (0 for an
 *   empty group); q_dist [H,N] float64 squared distance of each query to its
 *   group centre in query-response coordinates (raw query space when
 *   pp->semantic is 1).
 *   With pp->warm = 1, kv_label and q_label are also inputs (read before
 *   they are overwritten).
 * Errors (host, nothing enqueued): SPARSEPR_EINVAL for semantic or warm not
 *   0 or 1, besides the shape, group-count and parameter checks.
 */
int sparsepr_partition(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                       const void* Q, const void* K, const void* V,
                       int32_t* kv_label, int32_t* q_label, int32_t* kv_perm, int32_t* q_perm,
                       int32_t* kv_off, int32_t* q_off, void* Qp, void* Kp, void* Vp,
                       double* kv_centroid, double* q_centroid, double* q_dist,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 2 -- shared routing (abstract: centroids induce query-response
 * coordinates for shared routing; paperlayer.ai s4 "Sparse Execution": cells
 * selected under a query-key pair budget with true cell costs).
 * Cell score P_ab = softmax over nonempty b of (s qbar_a . mu_b + ln n_b).
 * top_k > 0: the top_k cells of each nonempty query group.  top_k == 0: every
 * nonempty query group keeps its best cell, then cells in order (P desc, a asc,
 * b asc) are added while sum n_a n_b <= floor(density N^2) - M N, stopping at
 * the first that does not fit.  If the kept best cells alone exceed the budget
 * the call still succeeds and routed_pairs reports the larger count.
 * In  [device]: kv_off, q_off, kv_centroid, q_centroid from stage 1.
 * Out [device]: CSR route per head: row_ptr [H,G_q+1] (offsets into that head's
 *   col_idx row block), col_idx [H, G_q*G_k] (per query group, routed K/V groups
 *   in ascending order; entries past row_ptr[G_q] are unspecified);
 *   routed_pairs [H] int64 = sum over routed cells of n_a n_b.
 */
int sparsepr_route(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                   const sparsepr_route_params* rp,
                   const int32_t* kv_off, const int32_t* q_off,
                   const double* kv_centroid, const double* q_centroid,
                   int32_t* row_ptr, int32_t* col_idx, int64_t* routed_pairs,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 2 for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same routing, arguments and results as sparsepr_route, with
 * its scratch (float64 cell scores and uint8 selection flags, 9 bytes per
 * cell) in a static device array of the library instead of `ws`.  That array
 * holds at most 2^22 cells (H * G_q * G_k <= 4194304, 36 MiB), reserved on
 * every GPU the library runs on until the process ends; larger calls return
 * SPARSEPR_EWORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller.  Its kernels write
 * every cell they read within the call, so nothing carries over from the
 * previous call.  Calls no allocating routine.
 */
int sparsepr_route_noalloc(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                           const sparsepr_route_params* rp, const int32_t* kv_off, const int32_t* q_off,
                           const double* kv_centroid, const double* q_centroid, int32_t* row_ptr, int32_t* col_idx,
                           int64_t* routed_pairs, void* stream);

/*
 * Stage 3 -- variable-block sparse attention with renormalised hard drop
 * (paperlayer.ai s4 "Sparse Execution", A.1): a query of group a attends, with
 * one softmax, to exactly the keys of its routed K/V groups; skipped
 * interactions are dropped and the retained weights renormalised.
 * In  [device]: Qp, Kp, Vp [H,N,d] dtype (group-major), q_off, kv_off, row_ptr,
 *   col_idx from stages 1-2.
 * Out [device]: Op [H,N,d] float32, group-major (slot order of Qp);
 *   lse [H,N] float32 natural-log sum of exp(s q.k) over the routed keys.
 * bf16 inputs: P.V runs on fp16 matrix cores over a copy of V scaled per head
 * by a power of two chosen on the device from max |V| (largest entry in
 * [2^14, 2^15)), so any finite V is in range; entries below 2^-28 of the
 * head's largest contribute as zero.  The exact probe rows of stage 4 and
 * the dense baseline use the same scheme.
 */
int sparsepr_attend(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                    const void* Qp, const void* Kp, const void* Vp,
                    const int32_t* q_off, const int32_t* kv_off,
                    const int32_t* row_ptr, const int32_t* col_idx,
                    float* Op, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Stages 4-5a -- query-group-stratified exact probes and the affine fit
 * (paperlayer.ai s4 "Probe-Fitted Residual Reconstruction", A.2, A.3;
 * gist-nl s2B).  Probes: one per nonempty query group, the rest by largest
 * remainder in proportion to group size (capped at the size); inside a group
 * the members at ranks floor((2j+1) n_a / (2 m_a)) of the (q_dist, index)
 * order; weight (n_a/m_a) / sum of probed n_a.  Each probe row is evaluated
 * against all N keys; residual R = O_dense - O_sparse.  Fit: x = sparse output;
 * weighted centring; V_r = leading right singular vectors of the weighted
 * centred residual (r_eff = min(rank, #sigma > 1e-6 sigma_1));
 * B_r = (Xt^T Xt + lambda I)^-1 Xt^T Rt V_r.
 * In  [device]: Q, K, V [H,N,d] dtype (original order); q_label, q_off,
 *   q_perm, q_dist from stage 1; Op [H,N,d] float32 from stage 3.
 * Out [device]: probe_idx [H,M] original indices, ascending; probe_w [H,M]
 *   float64; O_probe [H,M,d] float32 exact dense rows; r_bar, x_bar [H,d]
 *   float64; B_r, V_r [H,d,rank] float64 (columns >= rank_eff are zero);
 *   rank_eff [H].  With M = 0 nothing is written and the call is a no-op.
 */
int sparsepr_probe_fit(const sparsepr_shape* shape, const sparsepr_partition_params* pp,
                       const sparsepr_fit_params* fp,
                       const void* Q, const void* K, const void* V,
                       const int32_t* q_label, const int32_t* q_off, const int32_t* q_perm,
                       const double* q_dist, const float* Op,
                       int32_t* probe_idx, double* probe_w, float* O_probe,
                       double* r_bar, double* x_bar, double* B_r, double* V_r, int32_t* rank_eff,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 5b -- correction and restoration (gist-nl s2B; paperlayer.ai s4
 * "Sparse Execution": output restored to the original query order).
 * Unprobed rows: O_t = x_t + r_bar + (x_t - x_bar) B_r V_r^T (fit in float64;
 * the sum in float32; the product on float32 matrix cores for float32 inputs,
 * on fp16 matrix cores with power-of-two scales per row and per 32-direction
 * chunk and float32 accumulation for bf16 inputs, whose output rounding is
 * far coarser); probe rows: their exact dense rows; M = 0: O_t = x_t.
 * Written in original token order, cast once to dtype (round to nearest even).
 * In  [device]: Op, q_perm, and (if M > 0) probe_idx, O_probe, r_bar, x_bar,
 *   B_r, V_r, rank_eff from stages 3-5a.
 * Out [device]: O [H,N,d] dtype.
 */
int sparsepr_correct(const sparsepr_shape* shape, const sparsepr_fit_params* fp,
                     const float* Op, const int32_t* q_perm, const int32_t* probe_idx,
                     const float* O_probe, const double* r_bar, const double* x_bar,
                     const double* B_r, const double* V_r, const int32_t* rank_eff,
                     void* O, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace sparsepr_dense_attend needs (0 if the shape is invalid). */
size_t sparsepr_dense_workspace_size(const sparsepr_shape* shape);

/*
 * Dense attention built from the same tile machinery as sparsepr_attend
 * (the matched dense baseline of paperlayer.ai s5 / C.3): softmax(s Q K^T) V
 * over all N keys.  In [device]: Q, K, V [H,N,d] dtype.  Out [device]:
 * O [H,N,d] dtype, lse [H,N] float32.  ws: sparsepr_dense_workspace_size()
 * bytes of scratch (an fp16 copy of V for bf16 inputs).
 */
int sparsepr_dense_attend(const sparsepr_shape* shape, const void* Q, const void* K, const void* V,
                          void* O, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Measurement hook for the benchmark (not part of the method).  While
 * enabled, every sparsepr_attend call records two HIP events on its stream,
 * just before and just after the block-sparse attention kernel (the prep
 * kernel -- work-item descriptors and the fp16 copy of V -- and the
 * key-split combine are outside the pair).  sparsepr_attend_kernel_timing(1) discards earlier
 * events and enables recording, (0) discards them and disables it; neither
 * touches the device.  Enable it only around eager (not graph-captured)
 * launches, from one host thread.  sparsepr_attend_kernel_time waits for the
 * recorded events and returns the summed kernel time in milliseconds and the
 * number of launches measured.  Both return SPARSEPR_OK, or SPARSEPR_EINVAL
 * (null output pointer) / SPARSEPR_EHIP (an event query failed).
 */
int sparsepr_attend_kernel_timing(int enable);
int sparsepr_attend_kernel_time(double* total_ms, int* launches);

/*
 * Matrix-core rate probe for the benchmark (not part of the method): the
 * measured counterpart of the bf16 dense MFMA peak.  Launches `blocks`
 * workgroups of 256 threads on `stream`; each wave runs `iters` rounds of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands, so one
 * launch performs blocks * 4 * iters * 4 * 32768 flop with no memory traffic
 * in the loop; the caller times it.  Each thread writes one float to
 * sink [device, blocks * 256 floats].  Returns SPARSEPR_OK, SPARSEPR_EINVAL
 * (blocks or iters < 1, null sink) or SPARSEPR_EHIP.
 */
int sparsepr_mfma_rate_probe(int32_t blocks, int32_t iters, float* sink, void* stream);

/*
 * Tile-mix ceiling probe for the benchmark (not part of the method): the
 * rate at which a wave can issue the block-sparse kernel's per-tile work for
 * d = 128 -- per 64-key tile of its 32 query rows, 16 v_mfma_f32_32x32x16_bf16
 * score products, the online softmax (maximum, lazy rescale, exponentials,
 * fp16 weights, row sums) and 16 v_mfma_f32_32x32x16_f16 P.V products -- on
 * register operands, with no memory traffic and no barriers, at that
 * kernel's occupancy (two workgroups of 256 threads per CU).  Launches
 * `blocks` workgroups on `stream`; each of their 4 waves runs `iters` tiles,
 * so one launch performs blocks * 4 * iters * 32 * 64 * 4 * 128 flop; the
 * caller times it.  Each thread writes one float to sink [device,
 * blocks * 256 floats].  Returns SPARSEPR_OK, SPARSEPR_EINVAL (blocks or
 * iters < 1, null sink) or SPARSEPR_EHIP.
 */
int sparsepr_tile_rate_probe(int32_t blocks, int32_t iters, float* sink, void* stream);

/*
 * The symmetric eigensolver that stages 1 and 4 run inside their calls,
 * exported so that it can be checked on its own: the leading `nev`
 * eigenpairs of H symmetric d x d float64 matrices.  Stage 1 takes the
 * leading eigendirections of the sampled-query metric M_K for the key
 * coordinates (paperlayer.ai appendix B.1); stage 4 takes the leading right
 * singular vectors of the weighted, centred probe residuals as the
 * eigenvectors of their Gram matrix (appendix A.3).
 *   A       [H,d,d] float64, device, row-major, symmetric (only read)
 *   eigval  [H,d]   float64, device: entries 0 .. nev-1 of each row are the
 *           leading eigenvalues in descending order; the rest is not written
 *   eigvec  [H,d,d] float64, device: row e (e < nev) of each matrix is the
 *           unit eigenvector of eigval[e], its largest-magnitude entry
 *           positive (lowest index on ties); other rows are not written.
 *           Vectors of repeated or clustered eigenvalues are orthonormal.
 *   ws      device workspace of sparsepr_sym_eigen_workspace_size(H, d) bytes
 * d must be 64 or 128 and 1 <= nev <= d, H >= 1.  Asynchronous on `stream`;
 * returns SPARSEPR_OK, SPARSEPR_EINVAL (bad sizes, null pointer),
 * SPARSEPR_EUNSUPPORTED (other d), SPARSEPR_EWORKSPACE or SPARSEPR_EHIP.
 */
size_t sparsepr_sym_eigen_workspace_size(int32_t H, int32_t d);
int sparsepr_sym_eigen(int32_t H, int32_t d, int32_t nev, const double* A, double* eigval, double* eigvec,
                       void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEPR_H */
