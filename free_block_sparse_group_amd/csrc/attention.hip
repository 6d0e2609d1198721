// Stage 3 kernels: variable-block sparse attention with renormalised hard
// drop (arXiv:2608.18484, paperlayer.ai summary section 4 "Sparse
// Execution", appendix A.1), the dense probe rows (appendix A.2) and the dense
// baseline, all from one tile machinery.
//
// bf16 path (gfx950 MFMA, wave64):
//  - a work item is up to 128 query rows of one query group (4 waves x 32;
//    the dense kernel at d = 128 takes 256 rows with 8 waves, so that one
//    K/V tile in LDS serves twice the rows);
//  - its key set is the virtual concatenation of the routed K/V groups'
//    contiguous ranges in the group-major layout, walked in 64-key tiles, so
//    only the last tile of a work item is partial;
//  - K tiles (bf16) and V tiles (fp16, scaled per head) go from global
//    memory straight into LDS (global_load_lds_dwordx4, no register
//    staging), row-major with their 16-byte chunks XOR-swizzled per row so
//    that the MFMA operand reads are bank-conflict free; the V^T operand is
//    read with the transposing ds_read_b64_tr_b16; double-buffered with one
//    barrier per tile;
//  - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q stays in registers as the B
//    operand): each lane then holds 16 scores of one query, and the P^T B
//    operand of O^T = V^T P^T is a register-only repack of those scores once
//    the contraction index is permuted consistently on the V side;
//  - PV runs in fp16 (v_mfma_f32_32x32x16_f16): the weights are at most 2^8,
//    so fp16 holds them with 4x the precision of bf16 at the same rate; V is
//    converted with a power-of-two scale per head that puts its largest
//    magnitude in [2^14, 2^15) (no overflow, no subnormals but for entries
//    below 2^-28 of the largest), undone in the epilogue;
//  - online softmax in the log2 domain with a lazy rescale: the running
//    maximum is only moved when a tile raises it by more than 8 (2^8 bound
//    on the unnormalised weights), which changes no result; only the last,
//    partial tile of a work item is masked;
//  - fp32 accumulation; output normalised at the end (or written as
//    unnormalised partials for the split-key probe pass).
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace spr {

constexpr int BN = 64;          // keys per tile
constexpr float kRescaleThreshold = 8.0f;
constexpr int kVMaxParts = 64;           // slices per head of the max |V| pass

typedef __fp16 fp16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
typedef __attribute__((address_space(3))) void lds_void;

enum AttnMode { MODE_SPARSE = 0, MODE_DENSE = 1, MODE_PROBE = 2 };

struct AttnParams {
  const void* Q;          // [H,N,D]: Qp (sparse), Q (dense), Q original (probe, gathered)
  const void* K;          // [H,N,D]
  const void* V;          // [H,N,D]: fp16 x 2^-e per head for the bf16 kernel, fp32 for the fp32 kernel
  int N;
  float scale_log2;       // softmax scale * log2(e)
  // sparse mapping
  const int32_t* tiles;   // [H,G_q+1]
  const int4* tdesc;      // [H,maxT] row tile: first row, end row, row_ptr of its group, segment count
  const int2* segs;       // [H,G_q*G_k] routed cell (CSR order): first key row, key count
  int G_q, G_k, maxT;
  // probe mapping
  const int32_t* qidx;    // [H,M] token index of each probe row
  int M, splits;          // splits: key splits (probe rows; sparse rows when > 1)
  // outputs
  float* O32;             // sparse: Op [H,N,D] (partial O [S,H,N,D] when split); probe: partial O [S,H,M,D]
  void* Oout;             // dense: O [H,N,D] in the input dtype
  float* lse;             // [H,N] (sparse, dense)
  float* mpart;           // [S,H,M] (probe) or [S,H,N] (split sparse)
  float* lpart;           // [S,H,M] (probe) or [S,H,N] (split sparse)
  const float* vscale;    // [H] 2^e undoing the per-head scale of the fp16 V (bf16 kernel)
};

// The key sequence of a work item is the virtual concatenation of nseg
// contiguous row ranges ("segments"): segment s covers virtual positions
// [sv[s], sv[s+1]) and starts at global row sg[s].  The table sits in LDS,
// so walking it never waits on global memory (the K/V copies in flight stay
// in flight).  A cursor holds the segment containing the last position
// asked for; positions must not decrease between calls.
struct SegCursor {
  const int* sv;         // [nseg + 1] virtual starts, sv[nseg] = L (LDS)
  const int* sg;         // [nseg]     global start rows (LDS)
  int nseg, si;
  int vstart, vend;      // virtual range of the current segment
  int gstart;            // global start row of the current segment
  SPR_DEV void init(const int* v, const int* g, int n) {
    sv = v; sg = g; nseg = n; si = 0;
    vstart = 0;
    vend = n > 0 ? __builtin_amdgcn_readfirstlane(v[1]) : 0;
    gstart = n > 0 ? __builtin_amdgcn_readfirstlane(g[0]) : 0;
  }
  // move to the segment holding virtual position v (stays on the last
  // segment past the end); with a block-uniform v the cursor stays uniform
  SPR_DEV void seek(int v) {
    while (v >= vend && si + 1 < nseg) {
      ++si;
      vstart = vend;
      vend = sv[si + 1];
      gstart = sg[si];
    }
  }
  // seek for a block-uniform v on the block-uniform cursor: the entries it
  // reads are then the same in every lane, so they are kept in scalar
  // registers (scalar cursor tests and row base).  Not for lane-private
  // copies walking lane-dependent positions.
  SPR_DEV void seek_uniform(int v) {
    while (v >= vend && si + 1 < nseg) {
      ++si;
      vstart = vend;
      vend = __builtin_amdgcn_readfirstlane(sv[si + 1]);
      gstart = __builtin_amdgcn_readfirstlane(sg[si]);
    }
  }
  // global row of virtual position v; -1 past the end
  SPR_DEV int locate(int v) {
    seek(v);
    return v < vend ? gstart + (v - vstart) : -1;
  }
};

// LDS segment table of one block.
struct SegSmem {
  int sv[kMaxGroups + 1];
  int sg[kMaxGroups];
  int wsum[4];
};

// Work item of block (blockIdx.x, head h): query rows [r0, r1), key sequence
// (cursor over the block's segment table) of length L, of which key tiles
// [t0, t1) are this block's, and the key split it is (0 unless the keys are
// split).  Returns false (uniformly over the block) if the block has no work.
// Every thread of the block must call it; it contains barriers.
//
// Sparse rows: work item w = (tile T, split s), w = T * splits + s, tiles in
// the work order of k_attend_prep (heaviest query groups first).  Blocks
// are dealt to the eight XCDs round-robin by linear id (gridDim.x is a
// multiple of 8), so block x of head h runs on XCD x % 8 and takes
// w = ((x + h) % 8) * per + x / 8: each XCD runs a contiguous run of work
// items, heaviest first, and the row tiles of one query group -- which read
// the same routed keys -- share that XCD's L2 (dealing consecutive items to
// different XCDs instead measured 5 % slower).  The run an XCD gets rotates
// with the head, so the heavy first runs do not all land on one XCD.
template <int MODE, int BM>
SPR_DEV bool work_item(const AttnParams& p, int h, SegSmem& sm, int& r0, int& r1, SegCursor& cur, int& L, int& t0,
                       int& t1, int& split) {
  const int tid = threadIdx.x;
  split = 0;
  int nseg = 1;
  if (MODE == MODE_SPARSE) {
    const int32_t* tl = p.tiles + (int64_t)h * (p.G_q + 1);
    const int S = p.splits;
    const int nwork = tl[p.G_q] * S;
    const int per = (nwork + 7) >> 3;
    const int x = blockIdx.x;
    if ((x >> 3) >= per) return false;
    const int w = ((x + h) & 7) * per + (x >> 3);
    if (w >= nwork) return false;
    const int T = w / S;
    split = w - T * S;
    // the tile's rows and its group's routed segments, prepared per call
    const int4 td = p.tdesc[(int64_t)h * p.maxT + T];
    r0 = td.x;
    r1 = td.y;
    nseg = td.w;
    const int2* sgh = p.segs + (int64_t)h * p.G_q * p.G_k + td.z;
    // segment table: each of the first 256 threads takes 4 consecutive segments
    int len[4], local = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sidx = 4 * tid + u;
      len[u] = 0;
      if (tid < 256 && sidx < nseg) {
        const int2 sgv = sgh[sidx];
        sm.sg[sidx] = sgv.x;
        len[u] = sgv.y;
      }
      local += len[u];
    }
    // exclusive scan of the per-thread sums over the first 256 threads
    const int lane = tid & 63, wv = tid >> 6;
    int xs = tid < 256 ? local : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(xs, o);
      if (lane >= o) xs += y;
    }
    if (lane == 63 && wv < 4) sm.wsum[wv] = xs;
    __syncthreads();
    int before = 0;
    for (int u = 0; u < wv && u < 4; ++u) before += sm.wsum[u];
    L = sm.wsum[0] + sm.wsum[1] + sm.wsum[2] + sm.wsum[3];
    int run = before + xs - (tid < 256 ? local : 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sidx = 4 * tid + u;
      if (tid < 256 && sidx < nseg) sm.sv[sidx] = run;
      run += len[u];
    }
    if (tid == 0) sm.sv[nseg] = L;
    const int nt = (L + BN - 1) / BN;
    t0 = (int)((int64_t)nt * split / S);
    t1 = (int)((int64_t)nt * (split + 1) / S);
  } else if (MODE == MODE_DENSE) {
    r0 = blockIdx.x * BM;
    r1 = min(r0 + BM, p.N);
    L = p.N;
    if (tid == 0) { sm.sv[0] = 0; sm.sv[1] = L; sm.sg[0] = 0; }
    t0 = 0;
    t1 = (L + BN - 1) / BN;
  } else {
    r0 = blockIdx.x * BM;
    r1 = min(r0 + BM, p.M);
    split = blockIdx.z;
    const int k0 = (int)((int64_t)p.N * split / p.splits), k1 = (int)((int64_t)p.N * (split + 1) / p.splits);
    L = k1 - k0;
    if (tid == 0) { sm.sv[0] = 0; sm.sv[1] = L; sm.sg[0] = k0; }
    t0 = 0;
    t1 = (L + BN - 1) / BN;
  }
  __syncthreads();
  cur.init(sm.sv, sm.sg, nseg);
  return true;
}

// LDS tiles.  K and V tiles are both stored row-major (one key per row,
// D / 8 16-byte chunks) and filled by direct global->LDS copies
// (global_load_lds_dwordx4: no register staging).  Chunks are XOR-swizzled
// per row so that every operand read is free of bank conflicts on the
// 64-bank LDS (16 lanes of a 16-byte read, or 32 lanes of an 8-byte read,
// are served per cycle):
//  - K, read as the A operand of S^T = K Q^T: 16 lanes read chunk c of 16
//    consecutive rows, so the rows' swizzles must be distinct over 16 bank
//    groups: row & 15 for D = 128 (256-byte rows), (row / 2) & 7 for D = 64
//    (two 128-byte rows per bank line);
//  - V, read transposed with ds_read_b64_tr_b16 as the A operand of
//    O^T = V^T P^T: 32 lanes read 4 consecutive rows x 4 chunks, so the 4
//    rows' swizzles must move the chunk set {4j..4j+3} to disjoint sets:
//    4 (row % 4) for D = 128, 4 ((row / 2) % 2) for D = 64.
template <int D>
SPR_DEV int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
SPR_DEV int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// Global rows of NR increasing virtual positions of the tile the cursor was
// sought to; -1 past the end.  `fast` (uniform) = the tile lies in the
// cursor's segment; otherwise a lane-private copy walks the table.
template <int NR>
SPR_DEV void tile_rows(const SegCursor& cur, bool fast, const int (&v)[NR], int L, int (&g)[NR]) {
  if (fast) {
#pragma unroll
    for (int i = 0; i < NR; ++i) g[i] = v[i] < L ? cur.gstart + (v[i] - cur.vstart) : -1;
  } else {
    SegCursor t = cur;
#pragma unroll
    for (int i = 0; i < NR; ++i) g[i] = v[i] < L ? t.locate(v[i]) : -1;
  }
}

// Direct global->LDS copies of one 64-key tile of K (bf16) and V (fp16 x
// 2^-e).  Each wave instruction copies RPI rows: lane -> (row rl, physical
// chunk pc), loading logical chunk pc ^ swizzle(row).  Fast path (the whole
// tile lies in the cursor's segment): rows are contiguous from a uniform
// base, so the address is a scalar base plus a loop-invariant lane offset.
// Otherwise each lane walks the table; rows past the end of the key
// sequence copy row 0 (finite data; their weights are exactly zero).
template <int D, int WPB>
constexpr int kCopyInstr = BN * (D / 8) / (64 * WPB);   // copy instructions per wave, tile and tensor

// Byte offsets, within a tile, of this lane's copies (loop-invariant).
template <int D, int WPB>
SPR_DEV void copy_offsets(int wave, int lane, uint32_t (&ko)[kCopyInstr<D, WPB>], uint32_t (&vo)[kCopyInstr<D, WPB>]) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, NI = kCopyInstr<D, WPB>;
  const int pc = lane % CPR, rl = lane / CPR;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = (wave * NI + i) * RPI + rl;
    ko[i] = (uint32_t)(r * D + ((pc ^ k_swz<D>(r)) << 3)) * 2u;
    vo[i] = (uint32_t)(r * D + ((pc ^ v_swz<D>(r)) << 3)) * 2u;
  }
}

template <int D, int WPB>
SPR_DEV void issue_tile(const uint16_t* __restrict__ Kh, const uint16_t* __restrict__ Vh, const SegCursor& cur,
                        bool fast, int pos, int L, int wave, int lane, uint16_t* sK, uint16_t* sV,
                        uint32_t (&ko)[kCopyInstr<D, WPB>], uint32_t (&vo)[kCopyInstr<D, WPB>]) {
  constexpr int CPR = D / 8;                 // chunks per row
  constexpr int RPI = 64 / CPR;              // rows per wave instruction
  constexpr int NI = kCopyInstr<D, WPB>;     // instructions per wave and tensor
  const int pc = lane % CPR, rl = lane / CPR;
  int g[NI];
  // The empty asm makes the offsets loop-carried values, so the compiler
  // does not hoist their 64-bit extensions out of the tile loop (which costs
  // a 64-bit add per copy and twice the registers) and selects the
  // scalar-base form of the copy below instead.
#pragma unroll
  for (int i = 0; i < NI; ++i) asm volatile("" : "+v"(ko[i]), "+v"(vo[i]));
  if (fast) {
    // uniform row base (scalar registers) + unsigned 32-bit lane offsets
    const int gb = __builtin_amdgcn_readfirstlane(cur.gstart + (pos - cur.vstart));
    const char* kb = reinterpret_cast<const char*>(Kh + (int64_t)gb * D);
    const char* vb = reinterpret_cast<const char*>(Vh + (int64_t)gb * D);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + ko[i]), (lds_void*)(sK + (wave * NI + i) * 512),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vb + vo[i]), (lds_void*)(sV + (wave * NI + i) * 512),
                                       16, 0, 0);
    }
    return;
  }
  int v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) v[i] = pos + (wave * NI + i) * RPI + rl;
  tile_rows<NI>(cur, false, v, L, g);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = (wave * NI + i) * RPI + rl;
    const int64_t gr = g[i] < 0 ? 0 : g[i];
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(Kh + gr * D + ((pc ^ k_swz<D>(r)) << 3)),
                                     (lds_void*)(sK + (wave * NI + i) * 512), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(Vh + gr * D + ((pc ^ v_swz<D>(r)) << 3)),
                                     (lds_void*)(sV + (wave * NI + i) * 512), 16, 0, 0);
  }
}

SPR_DEV void wait_tile() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's direct LDS copies have landed
}

template <int D>
struct AttnState {
  bf16x8 qf[D / 16];
  f32x16 oacc[D / 32];
  float m_used;
  float lsum;
  // loop-invariant byte offsets of this lane's operand reads in a tile
  int koff[D / 16];   // K chunk (2s + hf) of row l32, step s
  int voff[D / 32];   // V^T transposed read, channel block jb (keys of the first read)
};

// Lane offsets of the operand reads.  K: row l32 (+32 rows for the second
// key block, an immediate), logical chunk 2s + hf.  V^T fragment (channels
// jb*32 + 16*bq + 0..15 of lane block bq = (lane / 16) % 2, keys 4hf + 0..3
// and 8 + 4hf + 0..3 of each 16): in ds_read_b64_tr_b16 lane m of a 16-lane
// block supplies the address of 4 channels (4 (m % 4) onwards) of key m / 4,
// and receives channel (m) of the block's 4 keys.
template <int D>
SPR_DEV void init_offsets(AttnState<D>& st, int lane) {
  const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) st.koff[s] = (l32 * D + (((2 * s + hf) ^ k_swz<D>(l32)) << 3)) * 2;
  const int m = lane & 15, bq = (lane >> 4) & 1;
  const int key = 4 * hf + (m >> 2);
#pragma unroll
  for (int jb = 0; jb < D / 32; ++jb) {
    const int ch = jb * 32 + 16 * bq + 4 * (m & 3);
    const int lc = ch >> 3;
    st.voff[jb] = (key * D + ((lc ^ v_swz<D>(key)) << 3) + (ch & 4)) * 2;
  }
}

// S^T of one 64-key tile for one wave (32 queries): rows = keys (2 blocks of
// 32), columns = the wave's queries.
template <int D>
SPR_DEV void qk_tile(f32x16 (&sacc)[2], const AttnState<D>& st, const uint16_t* sK) {
  constexpr int KS = D / 16;
  const char* kb = reinterpret_cast<const char*>(sK);
  sacc[0] = f32x16{};
  sacc[1] = f32x16{};
  // The two key blocks advance together (two independent accumulation
  // chains), and the operand reads run two steps ahead of the products, so
  // a wait for LDS covers several products instead of one.
  bf16x8 a0[KS], a1[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    a0[s] = *reinterpret_cast<const bf16x8*>(kb + st.koff[s]);
    a1[s] = *reinterpret_cast<const bf16x8*>(kb + st.koff[s] + 32 * D * 2);
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[s], st.qf[s], sacc[0], 0, 0, 0);
    sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[s], st.qf[s], sacc[1], 0, 0, 0);
  }
  // schedule: reads of steps 0 and 1, then per step the reads of step s + 2
  // (masks: 0x100 LDS reads, 0x008 matrix products)
  constexpr int AHEAD = 2;
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s + AHEAD < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

// Value of the partner lane l ^ 32 combined with op, in every lane (one VALU
// lane swap between the two halves of the wave instead of an LDS permute).
SPR_DEV float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SPR_DEV float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online softmax of one tile's scores for one wave: masks the keys past
// nvalid, moves the running maximum when the tile raises it past the
// threshold (rescaling the output and the row sum), and returns the fp16
// weights in the B-operand layout of the P.V products.
template <int D>
SPR_DEV void tile_weights(AttnState<D>& st, f32x16 (&sc)[2], int nvalid, float c, int hf, f16x8 (&pf)[2][2]) {
  constexpr int JB = D / 32;
  if (nvalid < BN) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = nb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (key >= nvalid) sc[nb][i] = -__builtin_inff();
      }
  }
  // ---- online softmax (log2 domain, lazy rescale)
  float mraw = -__builtin_inff();
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, sc[nb][i]);
  mraw = halves_max(mraw);
  const float mloc = mraw * c;
  if (mloc > st.m_used + kRescaleThreshold) {
    const float alpha = __builtin_amdgcn_exp2f(st.m_used - mloc);
    st.m_used = mloc;
    st.lsum *= alpha;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.oacc[jb][i] *= alpha;
  }
  const float negm = -st.m_used;
  // the row sum adds the fp16 values that enter P.V (two per v_dot2_f32_f16),
  // so the normalisation matches the weights actually applied
  float ls0 = 0.0f, ls1 = 0.0f;
  const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[nb][sp * 8 + e], c, negm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[nb][sp * 8 + e + 1], c, negm));
        const f16x2 pk = {(_Float16)p0, (_Float16)p1};
        pf[nb][sp][e] = pk[0];
        pf[nb][sp][e + 1] = pk[1];
        if (sp == 0) ls0 = __builtin_amdgcn_fdot2(pk, one2, ls0, false);
        else ls1 = __builtin_amdgcn_fdot2(pk, one2, ls1, false);
      }
  st.lsum += ls0 + ls1;
}

// Online softmax of one tile's scores and O^T += V^T P^T for one wave.
template <int D>
SPR_DEV void softmax_pv(AttnState<D>& st, f32x16 (&sc)[2], const uint16_t* Vt, int nvalid, float c, int lane) {
  constexpr int JB = D / 32;
  const int hf = lane >> 5;
  f16x8 pf[2][2];
  tile_weights<D>(st, sc, nvalid, c, hf, pf);
  // ---- O^T += V^T P^T
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const char* vb = reinterpret_cast<const char*>(Vt);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        // keys nb*32 + sp*16 + {4hf..4hf+3} then + 8: the contraction order of P^T
        const char* p0 = vb + st.voff[jb] + (nb * 32 + sp * 16) * D * 2;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * D * 2));
        const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        st.oacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[nb][sp], st.oacc[jb], 0, 0, 0);
      }
}

// One 64-key tile for one wave (32 queries): S^T, then softmax and PV.
template <int D>
SPR_DEV void compute_tile(AttnState<D>& st, const uint16_t* sK, const uint16_t* Vt, int nvalid, float c, int lane) {
  f32x16 sacc[2];
  qk_tile<D>(sacc, st, sK);
  softmax_pv<D>(st, sacc, Vt, nvalid, c, lane);
}

template <int D, int MODE, int WPB>
__global__ __launch_bounds__(64 * WPB, WPB == 8 ? 1 : (D == 64 ? 3 : 2)) void k_attn_bf16(AttnParams p) {
  constexpr int KS = D / 16, JB = D / 32;
  __shared__ __align__(16) uint16_t sK0[BN * D];
  __shared__ __align__(16) uint16_t sV0[BN * D];
  __shared__ __align__(16) uint16_t sK1[BN * D];
  __shared__ __align__(16) uint16_t sV1[BN * D];
  __shared__ SegSmem segs;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y;
  const bf16_t* Qh = static_cast<const bf16_t*>(p.Q) + (int64_t)h * p.N * D;
  const uint16_t* Kh = static_cast<const uint16_t*>(p.K) + (int64_t)h * p.N * D;
  const uint16_t* Vh = static_cast<const uint16_t*>(p.V) + (int64_t)h * p.N * D;

  int r0, r1, L, t0, t1, split;
  SegCursor cur;
  if (!work_item<MODE, 32 * WPB>(p, h, segs, r0, r1, cur, L, t0, t1, split)) return;
  const int wrow0 = r0 + wave * 32;
  const bool wave_active = wrow0 < r1;
  const int myrow = wrow0 + l32;
  const bool row_ok = myrow < r1;

  AttnState<D> st;
  {
    int64_t qrow = -1;
    if (row_ok) qrow = (MODE == MODE_PROBE) ? (int64_t)p.qidx[(int64_t)h * p.M + myrow] : (int64_t)myrow;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (qrow >= 0) st.qf[s] = *reinterpret_cast<const bf16x8*>(Qh + qrow * D + s * 16 + hf * 8);
      else st.qf[s] = bf16x8{};
    }
  }
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) st.oacc[jb] = f32x16{};
  st.m_used = -__builtin_inff();
  st.lsum = 0.0f;
  const float c = p.scale_log2;

  init_offsets<D>(st, lane);
  uint32_t cko[kCopyInstr<D, WPB>], cvo[kCopyInstr<D, WPB>];
  copy_offsets<D, WPB>(wave, lane, cko, cvo);
  // issue the copies of the key tile at virtual position pos (positions
  // increase, so the uniform cursor only moves forward)
  auto fetch = [&](int pos, uint16_t* sK, uint16_t* sV) {
    // one key range (dense, probe rows): every tile is in the single segment
    if (MODE == MODE_SPARSE) cur.seek_uniform(pos);
    const bool fast = pos + BN <= cur.vend;
    issue_tile<D, WPB>(Kh, Vh, cur, fast, pos, L, wave, lane, sK, sV, cko, cvo);
  };
  if (t1 > t0) fetch(t0 * BN, sK0, sV0);
  wait_tile();
  __syncthreads();
  for (int t = t0; t < t1; t += 2) {
    // even tile from stage 0, prefetch into stage 1
    const bool more1 = t + 1 < t1;
    if (more1) fetch((t + 1) * BN, sK1, sV1);
    if (wave_active) compute_tile<D>(st, sK0, sV0, min(BN, L - t * BN), c, lane);
    wait_tile();
    __syncthreads();
    if (!more1) break;
    // odd tile from stage 1, prefetch into stage 0
    const bool more2 = t + 2 < t1;
    if (more2) fetch((t + 2) * BN, sK0, sV0);
    if (wave_active) compute_tile<D>(st, sK1, sV1, min(BN, L - (t + 1) * BN), c, lane);
    wait_tile();
    __syncthreads();
  }

  if (!row_ok) return;
  const float ltot = halves_sum(st.lsum);
  const float kVUnscale = p.vscale[h];
  if (MODE == MODE_PROBE || (MODE == MODE_SPARSE && p.splits > 1)) {
    // partial (unnormalised) output of one key split, combined afterwards
    const int R = MODE == MODE_PROBE ? p.M : p.N;
    const int64_t prow = ((int64_t)split * gridDim.y + h) * R + myrow;
    float* out = p.O32 + prow * D;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = jb * 32 + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(out + j0) =
            make_float4(st.oacc[jb][4 * g] * kVUnscale, st.oacc[jb][4 * g + 1] * kVUnscale,
                        st.oacc[jb][4 * g + 2] * kVUnscale, st.oacc[jb][4 * g + 3] * kVUnscale);
      }
    if (hf == 0) {
      p.mpart[prow] = (t1 > t0) ? st.m_used : -__builtin_inff();
      p.lpart[prow] = ltot;
    }
    return;
  }
  const float inv = kVUnscale / ltot;
  const int64_t orow = (int64_t)h * p.N + myrow;
  if (MODE == MODE_SPARSE) {
    float* out = p.O32 + orow * D;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = jb * 32 + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(out + j0) =
            make_float4(st.oacc[jb][4 * g] * inv, st.oacc[jb][4 * g + 1] * inv, st.oacc[jb][4 * g + 2] * inv,
                        st.oacc[jb][4 * g + 3] * inv);
      }
  } else {
    bf16_t* out = static_cast<bf16_t*>(p.Oout) + orow * D;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = jb * 32 + 8 * g + 4 * hf;
        bf16x4 v;
        v[0] = (bf16_t)(st.oacc[jb][4 * g] * inv);
        v[1] = (bf16_t)(st.oacc[jb][4 * g + 1] * inv);
        v[2] = (bf16_t)(st.oacc[jb][4 * g + 2] * inv);
        v[3] = (bf16_t)(st.oacc[jb][4 * g + 3] * inv);
        *reinterpret_cast<bf16x4*>(out + j0) = v;
      }
  }
  if (hf == 0) p.lse[orow] = (st.m_used + log2f(ltot)) * 0.69314718055994530942f;
}

// Per-head scale of the fp16 copy of V.  k_vmax: the largest |v| of each of
// kVMaxParts slices of every head (bf16: the magnitude bits order like the
// values); k_vexp: per head e = ilogb(max |v|) - 14, clamped to [-110, 110]
// (0 for an all-zero head), vinv = 2^-e for the conversion and vscale = 2^e
// for the epilogues.
__global__ __launch_bounds__(256) void k_vmax(const uint4* __restrict__ V, int64_t n8h, float* __restrict__ part) {
  __shared__ uint32_t red[4];
  const int h = blockIdx.y, slice = blockIdx.x, tid = threadIdx.x;
  const int64_t b = n8h * slice / kVMaxParts, e = n8h * (slice + 1) / kVMaxParts;
  const uint4* Vh = V + (int64_t)h * n8h;
  uint32_t m = 0;
  for (int64_t i = b + tid; i < e; i += 256) {
    const uint4 w = Vh[i];
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(in[k] & 0x7fffu, (in[k] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) part[(int64_t)h * kVMaxParts + slice] = __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3])) << 16);
}

__global__ void k_vexp(const float* __restrict__ part, int H, float* __restrict__ vinv, float* __restrict__ vscale) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float m = 0.0f;
  for (int s = 0; s < kVMaxParts; ++s) m = fmaxf(m, part[(int64_t)h * kVMaxParts + s]);
  const int e = m > 0.0f ? min(110, max(-110, ilogbf(m) - 14)) : 0;
  vinv[h] = ldexpf(1.0f, -e);
  vscale[h] = ldexpf(1.0f, e);
}

// V (bf16) -> fp16 times the head's 2^-e, 8 elements per thread.
SPR_DEV void v_to_f16_at(const uint4* __restrict__ V, uint4* __restrict__ Vh, int64_t i, float sc) {
  const uint4 w = V[i];
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = __uint_as_float(in[k] << 16) * sc;
    const float hi = __uint_as_float(in[k] & 0xffff0000u) * sc;
    out[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
  }
  Vh[i] = make_uint4(out[0], out[1], out[2], out[3]);
}

__global__ void k_v_to_f16(const uint4* __restrict__ V, uint4* __restrict__ Vh, int64_t n8, int64_t n8h,
                           const float* __restrict__ vinv) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n8) v_to_f16_at(V, Vh, i, vinv[i / n8h]);
}

// ---------------------------------------------------------------- fp32 path
// float32 inputs on the fp32 matrix cores (v_mfma_f32_32x32x2_f32), with the
// work mapping and outputs of the bf16 kernel: a work item is up to 128 query
// rows (4 waves x 32); its keys pass through LDS in 32-key tiles, double
// buffered and loaded through registers.
//  - S^T = K Q^T: Q, pre-multiplied by the softmax scale in log2 units, stays
//    in registers as the B operand.  Step 4j + b of the 2-deep products takes
//    dim 8j + 4hf + b in lane half hf, so a lane reads four consecutive dims
//    of its key with one 16-byte LDS read; K rows have their 16-byte chunks
//    XOR-swizzled by the key index (conflict free).
//  - O^T += V^T P^T: step 4m + c takes key 8m + 4hf + c in lane half hf,
//    which is the lane's own score register 4m + c, so P needs no repacking;
//    V rows are padded to D + 8 floats, which puts the two halves' rows
//    (4 keys apart) 32 banks apart.
//  - online softmax in log2 units with the lazy rescale of the bf16 kernel
//    (threshold 8); weights, sums and accumulators in float32.
constexpr int KB32 = 32;   // keys per fp32 tile

template <int D>
SPR_DEV int kf32_swz(int key) { return key & (D / 4 - 1); }

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void k_attn_f32m(AttnParams p) {
  constexpr int CH = D / 4;                  // 16-byte chunks per row
  constexpr int VS = D + 8;                  // V row stride (floats)
  constexpr int JB = D / 32;
  constexpr int NL = KB32 * CH / 256;        // chunks per thread and tensor
  __shared__ __align__(16) float sK[2][KB32 * D];
  __shared__ __align__(16) float sV[2][KB32 * VS];
  __shared__ SegSmem segs;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y;
  const float* Qh = static_cast<const float*>(p.Q) + (int64_t)h * p.N * D;
  const float* Kh = static_cast<const float*>(p.K) + (int64_t)h * p.N * D;
  const float* Vh = static_cast<const float*>(p.V) + (int64_t)h * p.N * D;
  int r0, r1, L, t0, t1, split;
  SegCursor cur;
  if (!work_item<MODE, kAttnBM>(p, h, segs, r0, r1, cur, L, t0, t1, split)) return;
  const int kbeg = t0 * BN, kend = min(t1 * BN, L);
  const int wrow0 = r0 + wave * 32;
  const bool wave_active = wrow0 < r1;
  const int myrow = wrow0 + l32;
  const bool row_ok = myrow < r1;

  // Q: lane holds dims 8j + 4hf .. +3 of its query for every j
  float qf[D / 2];
  {
    int64_t qrow = -1;
    if (row_ok) qrow = (MODE == MODE_PROBE) ? (int64_t)p.qidx[(int64_t)h * p.M + myrow] : (int64_t)myrow;
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (qrow >= 0) v = *reinterpret_cast<const float4*>(Qh + qrow * D + 8 * j + 4 * hf);
      qf[4 * j] = v.x * p.scale_log2;
      qf[4 * j + 1] = v.y * p.scale_log2;
      qf[4 * j + 2] = v.z * p.scale_log2;
      qf[4 * j + 3] = v.w * p.scale_log2;
    }
  }
  f32x16 oacc[JB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) oacc[jb] = f32x16{};
  float m_used = -__builtin_inff(), lsum = 0.0f;

  // tile staging: chunk e = tid + 256 u is row e / CH, chunk e % CH of both tensors
  float4 kr[NL], vr[NL];
  auto load_regs = [&](int pos) {
    if (MODE == MODE_SPARSE) cur.seek_uniform(pos);
    const bool fast = pos + KB32 <= cur.vend;
    int v[NL], g[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) v[u] = pos + (tid + 256 * u) / CH;
    tile_rows<NL>(cur, fast, v, kend, g);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int c = (tid + 256 * u) % CH;
      kr[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      vr[u] = kr[u];
      if (g[u] >= 0) {
        kr[u] = *reinterpret_cast<const float4*>(Kh + (int64_t)g[u] * D + 4 * c);
        vr[u] = *reinterpret_cast<const float4*>(Vh + (int64_t)g[u] * D + 4 * c);
      }
    }
  };
  auto store_regs = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int e = tid + 256 * u, r = e / CH, c = e % CH;
      *reinterpret_cast<float4*>(&sK[buf][r * D + 4 * (c ^ kf32_swz<D>(r))]) = kr[u];
      *reinterpret_cast<float4*>(&sV[buf][r * VS + 4 * c]) = vr[u];
    }
  };
  auto compute = [&](int buf, int nvalid) {
    // ---- S^T (32 keys x 32 queries)
    f32x16 sacc = {};
    const float* kb = sK[buf] + l32 * D;
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      const float4 kc = *reinterpret_cast<const float4*>(kb + 4 * ((2 * j + hf) ^ kf32_swz<D>(l32)));
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kc.x, qf[4 * j], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kc.y, qf[4 * j + 1], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kc.z, qf[4 * j + 2], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kc.w, qf[4 * j + 3], sacc, 0, 0, 0);
    }
    // ---- online softmax; register i holds key 8 (i / 4) + 4 hf + i % 4
    if (nvalid < KB32) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * hf + (i & 3) >= nvalid) sacc[i] = -__builtin_inff();
    }
    float mraw = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, sacc[i]);
    mraw = halves_max(mraw);
    if (mraw > m_used + kRescaleThreshold) {
      const float alpha = __builtin_amdgcn_exp2f(m_used - mraw);
      m_used = mraw;
      lsum *= alpha;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[jb][i] *= alpha;
    }
    float ls = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sacc[i] = __builtin_amdgcn_exp2f(sacc[i] - m_used);
      ls += sacc[i];
    }
    lsum += ls;
    // ---- O^T += V^T P^T
    const float* vb = sV[buf] + 4 * hf * VS + l32;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = vb[(8 * (i >> 2) + (i & 3)) * VS + 32 * jb];
        oacc[jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[i], oacc[jb], 0, 0, 0);
      }
  };
  if (kbeg < kend) {
    load_regs(kbeg);
    store_regs(0);
  }
  __syncthreads();
  int buf = 0;
  for (int pos = kbeg; pos < kend; pos += KB32) {
    const bool more = pos + KB32 < kend;
    if (more) load_regs(pos + KB32);
    if (wave_active) compute(buf, min(KB32, kend - pos));
    if (more) store_regs(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  if (!row_ok) return;
  const float ltot = halves_sum(lsum);
  if (MODE == MODE_PROBE || (MODE == MODE_SPARSE && p.splits > 1)) {
    const int R = MODE == MODE_PROBE ? p.M : p.N;
    const int64_t prow = ((int64_t)split * gridDim.y + h) * R + myrow;
    float* out = p.O32 + prow * D;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(out + jb * 32 + 8 * g + 4 * hf) =
            make_float4(oacc[jb][4 * g], oacc[jb][4 * g + 1], oacc[jb][4 * g + 2], oacc[jb][4 * g + 3]);
    if (hf == 0) {
      p.mpart[prow] = kbeg < kend ? m_used : -__builtin_inff();
      p.lpart[prow] = ltot;
    }
    return;
  }
  const float inv = 1.0f / ltot;
  const int64_t orow = (int64_t)h * p.N + myrow;
  float* out = (MODE == MODE_SPARSE ? p.O32 : static_cast<float*>(p.Oout)) + orow * D;
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(out + jb * 32 + 8 * g + 4 * hf) =
          make_float4(oacc[jb][4 * g] * inv, oacc[jb][4 * g + 1] * inv, oacc[jb][4 * g + 2] * inv,
                      oacc[jb][4 * g + 3] * inv);
  if (hf == 0) p.lse[orow] = (m_used + log2f(ltot)) * 0.69314718055994530942f;
}

// Per-call preparation of the sparse pass.  Blocks 0 .. H-1, one per head:
// the work order of the row tiles, per row tile its rows, its group's CSR
// row start and segment count, and per routed cell (CSR order) the key
// segment's first row and length, so a work item finds all of it with two
// dependent reads.  Work order: query groups by routed key count, largest
// first (ties to the smaller group index), a group's ceil(n_a / bm) tiles
// of bm rows together; tiles[h][a] = the first tile of group a in that order,
// tiles[h][G_q] = the number of tiles.  Heaviest first keeps a long work
// item from starting last.  The blocks after them write the fp16 copy of V
// (1024 x 8 elements each; none for float inputs).
__global__ __launch_bounds__(1024) void k_attend_prep(const int32_t* __restrict__ q_off,
                                                      const int32_t* __restrict__ row_ptr,
                                                      const int32_t* __restrict__ col_idx,
                                                      const int32_t* __restrict__ kv_off, int H, int G_q, int G_k,
                                                      int bm, int maxT, int32_t* __restrict__ tiles,
                                                      int4* __restrict__ tdesc, int2* __restrict__ segs,
                                                      const uint4* __restrict__ V, uint4* __restrict__ Vh,
                                                      int64_t n8, int64_t n8h, const float* __restrict__ vinv) {
  __shared__ int wsum[16];
  __shared__ int skeys[kMaxGroups];    // routed keys per group (-1: no tiles)
  __shared__ int sorder[kMaxGroups];   // group at each position of the work order
  const int h = blockIdx.x, tid = threadIdx.x;
  if (h >= H) {   // uniform over the block
    const int64_t i = (int64_t)(h - H) * 1024 + tid;
    if (i < n8) v_to_f16_at(V, Vh, i, vinv[i / n8h]);
    return;
  }
  const int32_t* qo = q_off + (int64_t)h * (G_q + 1);
  const int32_t* rp = row_ptr + (int64_t)h * (G_q + 1);
  const int32_t* ko = kv_off + (int64_t)h * (G_k + 1);
  const int32_t* ch = col_idx + (int64_t)h * G_q * G_k;
  int32_t* tl = tiles + (int64_t)h * (G_q + 1);
  // G_q <= kMaxGroups = 1024: one group per thread
  const int na = tid < G_q ? (qo[tid + 1] - qo[tid] + bm - 1) / bm : 0;
  int keys = -1;
  if (na > 0) {
    keys = 0;
    for (int e = rp[tid]; e < rp[tid + 1]; ++e) keys += ko[ch[e] + 1] - ko[ch[e]];
  }
  skeys[tid] = keys;
  __syncthreads();
  if (tid < G_q) {
    int rank = 0;
    for (int a = 0; a < G_q; ++a) {
      const int ka = skeys[a];
      rank += (ka > keys || (ka == keys && a < tid)) ? 1 : 0;
    }
    sorder[rank] = tid;
  }
  __syncthreads();
  const int g = tid < G_q ? sorder[tid] : 0;
  const int ng = tid < G_q ? (qo[g + 1] - qo[g] + bm - 1) / bm : 0;
  int total;
  const int t0 = block_exclusive_scan<1024>(ng, wsum, &total);
  if (tid < G_q) tl[g] = t0;
  if (tid == 0) tl[G_q] = total;
  if (tid < G_q) {
    const int rs = rp[g], ns = rp[g + 1] - rs, q1 = qo[g + 1];
    for (int t = 0; t < ng; ++t) {
      const int r0 = qo[g] + t * bm;
      tdesc[(int64_t)h * maxT + t0 + t] = make_int4(r0, min(r0 + bm, q1), rs, ns);
    }
  }
  const int nnz = rp[G_q];
  int2* sh = segs + (int64_t)h * G_q * G_k;
  for (int e = tid; e < nnz; e += 1024) {
    const int b = ch[e];
    sh[e] = make_int2(ko[b], ko[b + 1] - ko[b]);
  }
}

// Split-key combine: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the
// S partials of each row (m in log2 units); lse (natural log) when asked.
// A block of 256 threads takes 1024 / d rows, four channels per thread
// (16-byte partial loads and output stores; a row's weights are computed once
// per thread).
__global__ __launch_bounds__(256) void k_split_combine(const float* __restrict__ opart,
                                                       const float* __restrict__ mpart,
                                                       const float* __restrict__ lpart, int H, int R, int d,
                                                       int splits, float* __restrict__ out,
                                                       float* __restrict__ lse) {
  const int h = blockIdx.y, tpr = d / 4, rows = 256 / tpr;
  const int j = blockIdx.x * rows + threadIdx.x / tpr, c = (threadIdx.x % tpr) * 4;
  if (j >= R) return;
  float mx = -__builtin_inff();
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, mpart[((int64_t)s * H + h) * R + j]);
  float l = 0.0f, o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const int64_t r = ((int64_t)s * H + h) * R + j;
    const float ms = mpart[r];
    const float wgt = ms == -__builtin_inff() ? 0.0f : exp2f(ms - mx);
    l = fmaf(lpart[r], wgt, l);
    const float4 ov = *reinterpret_cast<const float4*>(opart + r * d + c);
    o0 = fmaf(ov.x, wgt, o0);
    o1 = fmaf(ov.y, wgt, o1);
    o2 = fmaf(ov.z, wgt, o2);
    o3 = fmaf(ov.w, wgt, o3);
  }
  *reinterpret_cast<float4*>(out + ((int64_t)h * R + j) * d + c) = make_float4(o0 / l, o1 / l, o2 / l, o3 / l);
  if (lse != nullptr && c == 0) lse[(int64_t)h * R + j] = (mx + log2f(l)) * 0.69314718055994530942f;
}

static dim3 combine_grid(int R, int d, int H) {
  const int rows = 1024 / d;
  return dim3((unsigned)((R + rows - 1) / rows), (unsigned)H);
}

// ================================================================ launchers
// Waves (of 32 query rows) per block.  The block-sparse and probe-row
// passes run 4: two blocks share a CU and their phases drift apart, so one
// block's softmax runs beside the other's matrix products.  The dense
// kernel at d = 128 (bf16) runs 8: one K/V tile in LDS then serves 256 rows,
// halving the copy instructions per row, which is worth more there (4 %)
// than the phase drift; for the block-sparse pass the 256-row tiles also
// leave more rows of small query groups idle (4 % slower on Zipf groups).
template <int MODE>
constexpr int attn_waves(int d, bool bf16) { return MODE == MODE_DENSE && bf16 && d == 128 ? 8 : 4; }
template <int MODE>
constexpr int attn_rows(int d, bool bf16) { return 32 * attn_waves<MODE>(d, bf16); }

template <int MODE>
static void launch_attn(const AttnParams& p, int d, bool bf16, dim3 grid, hipStream_t st) {
  constexpr int W128 = attn_waves<MODE>(128, true);
  if (bf16) {
    if (d == 128) hipLaunchKernelGGL((k_attn_bf16<128, MODE, W128>), grid, dim3(64 * W128), 0, st, p);
    else hipLaunchKernelGGL((k_attn_bf16<64, MODE, 4>), grid, dim3(256), 0, st, p);
  } else {
    if (d == 128) hipLaunchKernelGGL((k_attn_f32m<128, MODE>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_attn_f32m<64, MODE>), grid, dim3(256), 0, st, p);
  }
}

void init_attention_attributes() {}

// per-head scale of the fp16 V copy: slice maxima, then 2^-e and 2^e per head
static void v_scales(const void* V, int H, int N, int d, float* vpart, float* vinv, float* vscale, hipStream_t st) {
  const int64_t n8h = (int64_t)N * d / 8;
  hipLaunchKernelGGL(k_vmax, dim3(kVMaxParts, H), dim3(256), 0, st, static_cast<const uint4*>(V), n8h, vpart);
  hipLaunchKernelGGL(k_vexp, dim3((H + 255) / 256), dim3(256), 0, st, vpart, H, vinv, vscale);
}

// fp16 copy of V for the bf16 kernels (scratch `vh`, H*N*d halves, scaled per head)
static const void* prepare_v(const void* V, bool bf16, int H, int N, int d, uint16_t* vh, float* vpart, float* vinv,
                             float* vscale, hipStream_t st) {
  if (!bf16) return V;
  v_scales(V, H, N, d, vpart, vinv, vscale, st);
  const int64_t n8 = (int64_t)H * N * d / 8, n8h = (int64_t)N * d / 8;
  hipLaunchKernelGGL(k_v_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint4*>(V), reinterpret_cast<uint4*>(vh), n8, n8h, vinv);
  return vh;
}

// Key splits of the sparse pass: enough work items to fill the chip about
// two blocks deep when the row tiles alone would not (bf16 and fp32 kernels).
int attend_splits(int H, int N, int G_q, bool bf16) {
  (void)bf16;   // both kernels take key splits
  static_assert(attn_rows<MODE_SPARSE>(128, true) == kAttnBM && attn_rows<MODE_SPARSE>(64, true) == kAttnBM,
                "the sparse pass works in tiles of kAttnBM rows");
  const int64_t tiles = (int64_t)H * ((N + kAttnBM - 1) / kAttnBM + G_q);
  const int64_t want = 256 * 2;
  if (tiles >= want) return 1;
  return (int)std::min<int64_t>(8, (want + tiles - 1) / tiles);
}

hipError_t launch_attend(const AttendArgs& a) {
  // upper bound on row tiles per head: sum ceil(n_a/bm) <= N/bm + G_q
  const int bm = kAttnBM;
  const int maxT = (a.N + bm - 1) / bm + a.G_q;
  const int64_t n8 = a.bf16 ? (int64_t)a.H * a.N * a.d / 8 : 0;
  if (a.bf16) v_scales(a.Vp, a.H, a.N, a.d, a.ws.vpart, a.ws.vinv, a.ws.vscale, a.stream);
  hipLaunchKernelGGL(k_attend_prep, dim3((unsigned)(a.H + (n8 + 1023) / 1024)), dim3(1024), 0, a.stream, a.q_off,
                     a.row_ptr, a.col_idx, a.kv_off, a.H, a.G_q, a.G_k, bm, maxT, a.ws.tiles, a.ws.tdesc, a.ws.segs,
                     static_cast<const uint4*>(a.Vp), reinterpret_cast<uint4*>(a.ws.vh), n8,
                     (int64_t)a.N * a.d / 8, a.ws.vinv);
  AttnParams p{};
  p.vscale = a.ws.vscale;
  p.Q = a.Qp; p.K = a.Kp;
  p.V = a.bf16 ? static_cast<const void*>(a.ws.vh) : a.Vp;
  p.N = a.N;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.tiles = a.ws.tiles; p.tdesc = a.ws.tdesc; p.segs = a.ws.segs;
  p.G_q = a.G_q; p.G_k = a.G_k; p.maxT = maxT;
  const int S = attend_splits(a.H, a.N, a.G_q, a.bf16);
  p.splits = S;
  if (S > 1) {
    p.O32 = a.ws.spart; p.mpart = a.ws.smpart; p.lpart = a.ws.slpart;
  } else {
    p.O32 = a.Op; p.lse = a.lse;
  }
  const int gx = (int)((((int64_t)maxT * S + 7) / 8) * 8);
  kernel_timer_mark(a.stream);
  launch_attn<MODE_SPARSE>(p, a.d, a.bf16, dim3(gx, a.H), a.stream);
  kernel_timer_mark(a.stream);
  if (S > 1)
    hipLaunchKernelGGL(k_split_combine, combine_grid(a.N, a.d, a.H), dim3(256), 0, a.stream,
                       a.ws.spart, a.ws.smpart, a.ws.slpart, a.H, a.N, a.d, S, a.Op, a.lse);
  return hipGetLastError();
}

hipError_t launch_dense(const DenseArgs& a) {
  AttnParams p{};
  p.Q = a.Q; p.K = a.K;
  p.V = prepare_v(a.V, a.bf16, a.H, a.N, a.d, a.vh, a.vpart, a.vinv, a.vscale, a.stream);
  p.vscale = a.vscale;
  p.N = a.N;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.Oout = a.O; p.lse = a.lse;
  const int bm = a.bf16 && a.d == 128 ? attn_rows<MODE_DENSE>(128, true) : kAttnBM;
  launch_attn<MODE_DENSE>(p, a.d, a.bf16, dim3((a.N + bm - 1) / bm, a.H), a.stream);
  return hipGetLastError();
}

// dense rows for the M probes: split-key pass + combine
hipError_t launch_probe_rows(const ProbeFitArgs& a, const int32_t* qidx) {
  AttnParams p{};
  p.Q = a.Q; p.K = a.K;
  p.V = prepare_v(a.V, a.bf16, a.H, a.N, a.d, a.ws.vh, a.ws.vpart, a.ws.vinv, a.ws.vscale, a.stream);
  p.vscale = a.ws.vscale;
  p.N = a.N;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.qidx = qidx; p.M = a.M; p.splits = kProbeSplits;
  p.O32 = a.ws.opart; p.mpart = a.ws.mpart; p.lpart = a.ws.lpart;
  const int bm = kAttnBM;
  launch_attn<MODE_PROBE>(p, a.d, a.bf16, dim3((a.M + bm - 1) / bm, a.H, kProbeSplits), a.stream);
  hipLaunchKernelGGL(k_split_combine, combine_grid(a.M, a.d, a.H), dim3(256), 0, a.stream,
                     a.ws.opart, a.ws.mpart, a.ws.lpart, a.H, a.M, a.d, kProbeSplits, a.O_probe, nullptr);
  return hipGetLastError();
}

// Ceiling of the tile's instruction mix (a measurement, not part of the
// method).  Each wave repeats the per-tile work of the block-sparse
// k_attn_bf16<128, MODE_SPARSE, 4> for its 32 query rows: the 16 score
// products, the online softmax of tile_weights and the 16 P.V products, on
// register operands -- no LDS or global traffic, no barriers -- at that
// kernel's occupancy (the launch reserves the same LDS, so two blocks of
// 256 threads share a CU).
// The key and value operands pass through an empty asm every tile so that
// the compiler keeps the score products inside the loop.
__global__ __launch_bounds__(256, 2) void k_tile_rate(int iters, float c, float* __restrict__ sink) {
  constexpr int D = 128, KS = D / 16, JB = D / 32;
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  AttnState<D> st;
  bf16x8 ka[4];
  f16x8 va[4];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) st.qf[s][i] = (bf16_t)(0.0625f * (float)(((lane + 3 * s + i) & 7) - 4));
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ka[u][i] = (bf16_t)(0.0625f * (float)(((5 * lane + u + i) & 7) - 3));
      va[u][i] = (_Float16)(0.015625f * (float)(((lane + 7 * u + i) & 15) - 8));
    }
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) st.oacc[jb] = f32x16{};
  st.m_used = -__builtin_inff();
  st.lsum = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(ka[u]), "+v"(va[u]));
    f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s & 3], st.qf[s], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[(s + 1) & 3], st.qf[s], sc[1], 0, 0, 0);
    }
    f16x8 pf[2][2];
    tile_weights<D>(st, sc, BN, c, hf, pf);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
          st.oacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[(2 * nb + sp + jb) & 3], pf[nb][sp], st.oacc[jb],
                                                                0, 0, 0);
  }
  float s = st.lsum;
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += st.oacc[jb][i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The launch reserves (unused) dynamic LDS of the attention block's size, so
// that no more blocks share a CU than in the attention kernel.
hipError_t launch_tile_rate(int blocks, int iters, float* sink, hipStream_t st) {
  constexpr int kLds = 2 * 2 * BN * 128 * 2 + (int)sizeof(SegSmem);
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_tile_rate),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (e != hipSuccess) return e;
  const float c = 1.4426950408889634f / sqrtf(128.0f);
  hipLaunchKernelGGL(k_tile_rate, dim3(blocks), dim3(256), kLds, st, iters, c, sink);
  return hipGetLastError();
}

}  // namespace spr
