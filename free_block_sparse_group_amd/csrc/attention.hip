// Stage 3 kernels: variable-block sparse attention with renormalised hard
// drop (arXiv:2608.18484, paperlayer.ai summary section 4 "Sparse
// Execution", appendix A.1), the dense probe rows (appendix A.2) and the dense
// baseline, all from one tile machinery.
//
// bf16 path (gfx950 MFMA, wave64):
//  - a work item is up to 128 query rows of one query group (4 waves x 32);
//  - its key set is the virtual concatenation of the routed K/V groups'
//    contiguous ranges in the group-major layout, walked in 64-key tiles, so
//    only the last tile of a work item is partial;
//  - K tiles are staged row-major in LDS, V tiles transposed (channel-major),
//    both double-buffered with one barrier per tile;
//  - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q stays in registers as the B
//    operand): each lane then holds 16 scores of one query, and the P^T B
//    operand of O^T = V^T P^T is a register-only repack of those scores once
//    the contraction index is permuted consistently on the V^T side;
//  - the PV product runs in fp16 (v_mfma_f32_32x32x16_f16): the weights are
//    at most 2^8 (see below), so fp16 holds them with 4x the precision of
//    bf16 at the same MFMA rate; V is staged as fp16 after an exact 2^-6
//    scale (bf16 values convert exactly; |v| up to 4e6 stays in range) and the
//    scale is undone in the epilogue;
//  - online softmax in the log2 domain with a lazy rescale: the running
//    maximum is only moved when a tile raises it by more than 8 (2^8 bound
//    on the unnormalised weights), which changes no result;
//  - fp32 accumulation; output normalised at the end (or written as
//    unnormalised partials for the split-key probe pass).
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

constexpr int BN = 64;          // keys per tile
constexpr int KPAD = 8;         // bf16 padding per K row
constexpr int VPAD = 8;         // bf16 padding per V^T row
constexpr float kRescaleThreshold = 8.0f;
constexpr float kVScale = 0.015625f;     // 2^-6 applied to V before the fp16 conversion
constexpr float kVUnscale = 64.0f;

enum AttnMode { MODE_SPARSE = 0, MODE_DENSE = 1, MODE_PROBE = 2 };

struct AttnParams {
  const void* Q;          // [H,N,D]: Qp (sparse), Q (dense), Q original (probe, gathered)
  const void* K;          // [H,N,D]
  const void* V;          // [H,N,D]
  int N;
  float scale_log2;       // softmax scale * log2(e)
  // sparse mapping
  const int32_t* q_off;   // [H,G_q+1]
  const int32_t* tiles;   // [H,G_q+1]
  const int32_t* row_ptr; // [H,G_q+1]
  const int32_t* col_idx; // [H,G_q*G_k]
  const int32_t* kv_off;  // [H,G_k+1]
  int G_q, G_k;
  // probe mapping
  const int32_t* qidx;    // [H,M] token index of each probe row
  int M, splits;
  // outputs
  float* O32;             // sparse: Op [H,N,D]; probe: partial O [S,H,M,D]
  void* Oout;             // dense: O [H,N,D] in the input dtype
  float* lse;             // [H,N] (sparse, dense)
  float* mpart;           // [S,H,M] (probe)
  float* lpart;           // [S,H,M] (probe)
};

// Walks the virtual concatenation of key ranges.
struct SegCursor {
  const int32_t* cols;   // routed K/V groups (sparse) or nullptr (single range)
  const int32_t* kv_off;
  int nseg, si;
  int vstart, vend;      // virtual range of the current segment
  int gstart;            // global start row of the current segment
  SPR_DEV void init_single(int k0, int k1) {
    cols = nullptr; nseg = 1; si = 0; vstart = 0; vend = k1 - k0; gstart = k0;
  }
  SPR_DEV void init_segments(const int32_t* c, const int32_t* off, int n) {
    cols = c; kv_off = off; nseg = n; si = 0; vstart = 0;
    if (n > 0) { const int b = c[0]; gstart = off[b]; vend = off[b + 1] - off[b]; }
    else { gstart = 0; vend = 0; }
  }
  // global row of virtual position v (v must not decrease between calls); -1 past the end
  SPR_DEV int locate(int v) {
    while (v >= vend) {
      if (si + 1 >= nseg) return -1;
      ++si;
      const int b = cols[si];
      vstart = vend;
      gstart = kv_off[b];
      vend = vstart + (kv_off[b + 1] - kv_off[b]);
    }
    return gstart + (v - vstart);
  }
};

template <int D>
struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

// Thread (rq, cc) moves rows 4rq..4rq+3, channels 8cc..8cc+7 of a 64-key tile.
template <int D>
SPR_DEV void load_tile(const bf16_t* __restrict__ Kh, const bf16_t* __restrict__ Vh, SegCursor& cur, int pos,
                       int tid, TileRegs<D>& r) {
  constexpr int CC = D / 8;
  const int rq = tid / CC, cc = tid % CC;
  if (rq >= BN / 4) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = cur.locate(pos + 4 * rq + i);
    if (g >= 0) {
      r.k[i] = *reinterpret_cast<const uint4*>(Kh + (int64_t)g * D + cc * 8);
      r.v[i] = *reinterpret_cast<const uint4*>(Vh + (int64_t)g * D + cc * 8);
    } else {
      r.k[i] = make_uint4(0, 0, 0, 0);
      r.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

SPR_DEV uint32_t lo16(uint32_t w) { return w & 0xffffu; }
SPR_DEV uint32_t hi16(uint32_t w) { return w >> 16; }

// bf16 bit pattern -> float -> scaled fp16 bit pattern (exact for |v| * 2^-6 >= 2^-14)
SPR_DEV uint32_t bf16_to_f16_scaled(uint32_t bits16) {
  const float f = __uint_as_float(bits16 << 16) * kVScale;
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int D>
SPR_DEV void store_tile(bf16_t* Ks, uint16_t* Vt, int tid, const TileRegs<D>& r) {
  constexpr int CC = D / 8;
  constexpr int KLD = D + KPAD, VLD = BN + VPAD;
  const int rq = tid / CC, cc = tid % CC;
  if (rq >= BN / 4) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(Ks + (4 * rq + i) * KLD + cc * 8) = r.k[i];
  // V^T (fp16): key quad 4rq..4rq+3 goes to position 16*(rq/4) + 4*swap(rq%4) where
  // the middle two quads of every 16 are swapped (the order the PV operand reads).
  const int qd = rq & 3;
  const int sq = (qd == 1) ? 2 : (qd == 2 ? 1 : qd);
  const int col = 16 * (rq >> 2) + 4 * sq;
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r.v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r.v[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r.v[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r.v[3]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int wi = c >> 1;
    const bool hi = c & 1;
    const uint32_t e0 = bf16_to_f16_scaled(hi ? hi16(w0[wi]) : lo16(w0[wi]));
    const uint32_t e1 = bf16_to_f16_scaled(hi ? hi16(w1[wi]) : lo16(w1[wi]));
    const uint32_t e2 = bf16_to_f16_scaled(hi ? hi16(w2[wi]) : lo16(w2[wi]));
    const uint32_t e3 = bf16_to_f16_scaled(hi ? hi16(w3[wi]) : lo16(w3[wi]));
    uint2 pk;
    pk.x = e0 | (e1 << 16);
    pk.y = e2 | (e3 << 16);
    *reinterpret_cast<uint2*>(Vt + (cc * 8 + c) * VLD + col) = pk;
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnParams p) {
  constexpr int KLD = D + KPAD, VLD = BN + VPAD;
  constexpr int KS = D / 16;     // k-steps of the QK^T contraction
  constexpr int JB = D / 32;     // 32-channel blocks of the output
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* Ks[2];
  uint16_t* Vt[2];
  Ks[0] = reinterpret_cast<bf16_t*>(smem_raw);
  Vt[0] = reinterpret_cast<uint16_t*>(Ks[0] + BN * KLD);
  Ks[1] = reinterpret_cast<bf16_t*>(Vt[0] + D * VLD);
  Vt[1] = reinterpret_cast<uint16_t*>(Ks[1] + BN * KLD);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y;
  const bf16_t* Qh = static_cast<const bf16_t*>(p.Q) + (int64_t)h * p.N * D;
  const bf16_t* Kh = static_cast<const bf16_t*>(p.K) + (int64_t)h * p.N * D;
  const bf16_t* Vh = static_cast<const bf16_t*>(p.V) + (int64_t)h * p.N * D;

  // ---- work item: query rows [r0, r1) and the key sequence
  int r0, r1;
  SegCursor cur;
  int L;
  if (MODE == MODE_SPARSE) {
    const int32_t* tl = p.tiles + (int64_t)h * (p.G_q + 1);
    const int T = blockIdx.x;
    if (T >= tl[p.G_q]) return;
    int lo = 0, hi = p.G_q;   // largest a with tl[a] <= T
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tl[mid] <= T) lo = mid; else hi = mid;
    }
    const int a = lo;
    const int32_t* qo = p.q_off + (int64_t)h * (p.G_q + 1);
    r0 = qo[a] + (T - tl[a]) * kAttnBM;
    r1 = min(r0 + kAttnBM, qo[a + 1]);
    const int32_t* rp = p.row_ptr + (int64_t)h * (p.G_q + 1);
    const int32_t* cols = p.col_idx + (int64_t)h * p.G_q * p.G_k + rp[a];
    const int nseg = rp[a + 1] - rp[a];
    const int32_t* ko = p.kv_off + (int64_t)h * (p.G_k + 1);
    L = 0;
    for (int s = 0; s < nseg; ++s) L += ko[cols[s] + 1] - ko[cols[s]];
    cur.init_segments(cols, ko, nseg);
  } else if (MODE == MODE_DENSE) {
    r0 = blockIdx.x * kAttnBM;
    r1 = min(r0 + kAttnBM, p.N);
    L = p.N;
    cur.init_single(0, p.N);
  } else {
    r0 = blockIdx.x * kAttnBM;
    r1 = min(r0 + kAttnBM, p.M);
    const int s = blockIdx.z;
    const int k0 = (int)((int64_t)p.N * s / p.splits), k1 = (int)((int64_t)p.N * (s + 1) / p.splits);
    L = k1 - k0;
    cur.init_single(k0, k1);
  }
  const int wrow0 = r0 + wave * 32;
  const bool wave_active = wrow0 < r1;
  const int myrow = wrow0 + l32;
  const bool row_ok = myrow < r1;

  // ---- Q fragment (B operand: column = query l32, k = 8*hf + 0..7 within each 16-step)
  bf16x8 qf[KS];
  {
    int64_t qrow = -1;
    if (row_ok) qrow = (MODE == MODE_PROBE) ? (int64_t)p.qidx[(int64_t)h * p.M + myrow] : (int64_t)myrow;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (qrow >= 0) qf[s] = *reinterpret_cast<const bf16x8*>(Qh + qrow * D + s * 16 + hf * 8);
      else qf[s] = bf16x8{};
    }
  }

  f32x16 oacc[JB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) oacc[jb] = f32x16{};
  float m_used = -__builtin_inff();
  float lsum = 0.0f;

  const int ntiles = (L + BN - 1) / BN;
  TileRegs<D> regs;
  if (ntiles > 0) {
    load_tile<D>(Kh, Vh, cur, 0, tid, regs);
    store_tile<D>(Ks[0], Vt[0], tid, regs);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile<D>(Kh, Vh, cur, (t + 1) * BN, tid, regs);
    if (wave_active) {
      const bf16_t* K_s = Ks[buf];
      const uint16_t* V_s = Vt[buf];
      // S^T tile: rows = keys (2 blocks of 32), columns = the wave's 32 queries
      f32x16 sacc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        sacc[nb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(K_s + (nb * 32 + l32) * KLD + s * 16 + hf * 8);
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[nb], 0, 0, 0);
        }
      }
      const int nvalid = min(BN, L - t * BN);
      float mloc = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = nb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
          float x = sacc[nb][i] * p.scale_log2;
          if (key >= nvalid) x = -__builtin_inff();
          sacc[nb][i] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      if (mloc > m_used + kRescaleThreshold) {
        const float alpha = exp2f(m_used - mloc);
        m_used = mloc;
        lsum *= alpha;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[jb][i] *= alpha;
      }
      f16x8 pf[2][2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = exp2f(sacc[nb][sp * 8 + e] - m_used);
            lsum += pv;
            pf[nb][sp][e] = (_Float16)pv;
          }
      // O^T += V^T P^T
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            const f16x8 a =
                *reinterpret_cast<const f16x8*>(V_s + (jb * 32 + l32) * VLD + nb * 32 + sp * 16 + hf * 8);
            oacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[nb][sp], oacc[jb], 0, 0, 0);
          }
    }
    if (more) store_tile<D>(Ks[buf ^ 1], Vt[buf ^ 1], tid, regs);
    __syncthreads();
  }

  if (!row_ok) return;
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (MODE == MODE_PROBE) {
    const int s = blockIdx.z;
    const int64_t prow = ((int64_t)s * gridDim.y + h) * p.M + myrow;
    float* out = p.O32 + prow * D;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = jb * 32 + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(out + j0) =
            make_float4(oacc[jb][4 * g] * kVUnscale, oacc[jb][4 * g + 1] * kVUnscale,
                        oacc[jb][4 * g + 2] * kVUnscale, oacc[jb][4 * g + 3] * kVUnscale);
      }
    if (hf == 0) {
      p.mpart[prow] = (L > 0) ? m_used : -__builtin_inff();
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
        *reinterpret_cast<float4*>(out + j0) = make_float4(oacc[jb][4 * g] * inv, oacc[jb][4 * g + 1] * inv,
                                                           oacc[jb][4 * g + 2] * inv, oacc[jb][4 * g + 3] * inv);
      }
  } else {
    bf16_t* out = static_cast<bf16_t*>(p.Oout) + orow * D;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = jb * 32 + 8 * g + 4 * hf;
        bf16x4 v;
        v[0] = (bf16_t)(oacc[jb][4 * g] * inv);
        v[1] = (bf16_t)(oacc[jb][4 * g + 1] * inv);
        v[2] = (bf16_t)(oacc[jb][4 * g + 2] * inv);
        v[3] = (bf16_t)(oacc[jb][4 * g + 3] * inv);
        *reinterpret_cast<bf16x4*>(out + j0) = v;
      }
  }
  if (hf == 0) p.lse[orow] = (m_used + log2f(ltot)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for float32 inputs: TPQ = D/32 threads per query row each
// own 32 channels; keys staged 32 at a time in LDS; exact per-key online
// softmax.  Same work mapping and outputs as the bf16 kernel.
template <int D, int MODE>
__global__ __launch_bounds__(128 * (D / 32)) void k_attn_f32(AttnParams p) {
  constexpr int TPQ = D / 32, KT = 32;
  __shared__ float Ksm[KT][D];
  __shared__ float Vsm[KT][D];
  const int tid = threadIdx.x, h = blockIdx.y;
  const int qr = tid / TPQ, part = tid % TPQ;
  const float* Qh = static_cast<const float*>(p.Q) + (int64_t)h * p.N * D;
  const float* Kh = static_cast<const float*>(p.K) + (int64_t)h * p.N * D;
  const float* Vh = static_cast<const float*>(p.V) + (int64_t)h * p.N * D;
  int r0, r1, L;
  SegCursor cur;
  if (MODE == MODE_SPARSE) {
    const int32_t* tl = p.tiles + (int64_t)h * (p.G_q + 1);
    const int T = blockIdx.x;
    if (T >= tl[p.G_q]) return;
    int lo = 0, hi = p.G_q;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tl[mid] <= T) lo = mid; else hi = mid;
    }
    const int a = lo;
    const int32_t* qo = p.q_off + (int64_t)h * (p.G_q + 1);
    r0 = qo[a] + (T - tl[a]) * kAttnBM;
    r1 = min(r0 + kAttnBM, qo[a + 1]);
    const int32_t* rp = p.row_ptr + (int64_t)h * (p.G_q + 1);
    const int32_t* cols = p.col_idx + (int64_t)h * p.G_q * p.G_k + rp[a];
    const int nseg = rp[a + 1] - rp[a];
    const int32_t* ko = p.kv_off + (int64_t)h * (p.G_k + 1);
    L = 0;
    for (int s = 0; s < nseg; ++s) L += ko[cols[s] + 1] - ko[cols[s]];
    cur.init_segments(cols, ko, nseg);
  } else if (MODE == MODE_DENSE) {
    r0 = blockIdx.x * kAttnBM;
    r1 = min(r0 + kAttnBM, p.N);
    L = p.N;
    cur.init_single(0, p.N);
  } else {
    r0 = blockIdx.x * kAttnBM;
    r1 = min(r0 + kAttnBM, p.M);
    const int s = blockIdx.z;
    const int k0 = (int)((int64_t)p.N * s / p.splits), k1 = (int)((int64_t)p.N * (s + 1) / p.splits);
    L = k1 - k0;
    cur.init_single(k0, k1);
  }
  const int myrow = r0 + qr;
  const bool row_ok = myrow < r1;
  float q[32], o[32];
  int64_t qrow = -1;
  if (row_ok) qrow = (MODE == MODE_PROBE) ? (int64_t)p.qidx[(int64_t)h * p.M + myrow] : (int64_t)myrow;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    q[c] = qrow >= 0 ? Qh[qrow * D + part * 32 + c] * p.scale_log2 : 0.0f;
    o[c] = 0.0f;
  }
  float m = -__builtin_inff(), l = 0.0f;
  for (int pos = 0; pos < L; pos += KT) {
    __syncthreads();
    for (int e = tid; e < KT * D; e += blockDim.x) {
      const int kr = e / D, c = e % D;
      const int g = (pos + kr < L) ? cur.locate(pos + kr) : -1;
      Ksm[kr][c] = g >= 0 ? Kh[(int64_t)g * D + c] : 0.0f;
      Vsm[kr][c] = g >= 0 ? Vh[(int64_t)g * D + c] : 0.0f;
    }
    __syncthreads();
    const int nk = min(KT, L - pos);
    for (int kk = 0; kk < nk; ++kk) {
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < 32; ++c) s = fmaf(q[c], Ksm[kk][part * 32 + c], s);
#pragma unroll
      for (int off = TPQ / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, TPQ);
      s = __shfl(s, 0, TPQ);
      const float mn = fmaxf(m, s);
      const float corr = exp2f(m - mn);
      const float pw = exp2f(s - mn);
      l = l * corr + pw;
#pragma unroll
      for (int c = 0; c < 32; ++c) o[c] = fmaf(o[c], corr, pw * Vsm[kk][part * 32 + c]);
      m = mn;
    }
  }
  if (!row_ok) return;
  if (MODE == MODE_PROBE) {
    const int s = blockIdx.z;
    const int64_t prow = ((int64_t)s * gridDim.y + h) * p.M + myrow;
#pragma unroll
    for (int c = 0; c < 32; ++c) p.O32[prow * D + part * 32 + c] = o[c];
    if (part == 0) { p.mpart[prow] = m; p.lpart[prow] = l; }
    return;
  }
  const float inv = 1.0f / l;
  const int64_t orow = (int64_t)h * p.N + myrow;
  if (MODE == MODE_SPARSE) {
#pragma unroll
    for (int c = 0; c < 32; ++c) p.O32[orow * D + part * 32 + c] = o[c] * inv;
  } else {
    float* out = static_cast<float*>(p.Oout);
#pragma unroll
    for (int c = 0; c < 32; ++c) out[orow * D + part * 32 + c] = o[c] * inv;
  }
  if (part == 0) p.lse[orow] = (m + log2f(l)) * 0.69314718055994530942f;
}

// tiles[h][a] = sum_{a' < a} ceil(n_a' / 128): work-item prefix per head.
__global__ void k_tile_prefix(const int32_t* __restrict__ q_off, int G_q, int32_t* __restrict__ tiles) {
  const int h = blockIdx.x;
  if (threadIdx.x != 0) return;
  const int32_t* qo = q_off + (int64_t)h * (G_q + 1);
  int32_t* tl = tiles + (int64_t)h * (G_q + 1);
  int run = 0;
  for (int a = 0; a < G_q; ++a) {
    tl[a] = run;
    run += (qo[a + 1] - qo[a] + kAttnBM - 1) / kAttnBM;
  }
  tl[G_q] = run;
}

// Split-key combine for the probe rows: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
__global__ void k_probe_combine(const float* __restrict__ opart, const float* __restrict__ mpart,
                                const float* __restrict__ lpart, int H, int M, int d, int splits,
                                float* __restrict__ O_probe) {
  const int h = blockIdx.y, j = blockIdx.x, c = threadIdx.x;
  if (c >= d) return;
  float mx = -__builtin_inff();
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, mpart[((int64_t)s * H + h) * M + j]);
  float l = 0.0f, o = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const int64_t r = ((int64_t)s * H + h) * M + j;
    const float ms = mpart[r];
    const float wgt = ms == -__builtin_inff() ? 0.0f : exp2f(ms - mx);
    l = fmaf(lpart[r], wgt, l);
    o = fmaf(opart[r * d + c], wgt, o);
  }
  O_probe[((int64_t)h * M + j) * d + c] = o / l;
}

// ================================================================ launchers
static size_t attn_lds_bytes(int d) {
  return 2 * (sizeof(bf16_t) * (size_t)BN * (d + KPAD) + sizeof(uint16_t) * (size_t)d * (BN + VPAD));
}

template <int MODE>
static void launch_attn(const AttnParams& p, int d, bool bf16, dim3 grid, hipStream_t st) {
  if (bf16) {
    if (d == 128) hipLaunchKernelGGL((k_attn_bf16<128, MODE>), grid, dim3(256), attn_lds_bytes(128), st, p);
    else hipLaunchKernelGGL((k_attn_bf16<64, MODE>), grid, dim3(256), attn_lds_bytes(64), st, p);
  } else {
    if (d == 128) hipLaunchKernelGGL((k_attn_f32<128, MODE>), grid, dim3(512), 0, st, p);
    else hipLaunchKernelGGL((k_attn_f32<64, MODE>), grid, dim3(256), 0, st, p);
  }
}

void init_attention_attributes() {
  const int b128 = (int)attn_lds_bytes(128), b64 = (int)attn_lds_bytes(64);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<128, MODE_SPARSE>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, b128);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<128, MODE_DENSE>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, b128);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<128, MODE_PROBE>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, b128);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<64, MODE_SPARSE>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, b64);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<64, MODE_DENSE>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, b64);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<64, MODE_PROBE>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, b64);
}

hipError_t launch_attend(const AttendArgs& a) {
  hipLaunchKernelGGL(k_tile_prefix, dim3(a.H), dim3(64), 0, a.stream, a.q_off, a.G_q, a.ws.tiles);
  AttnParams p{};
  p.Q = a.Qp; p.K = a.Kp; p.V = a.Vp;
  p.N = a.N;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.q_off = a.q_off; p.tiles = a.ws.tiles; p.row_ptr = a.row_ptr; p.col_idx = a.col_idx; p.kv_off = a.kv_off;
  p.G_q = a.G_q; p.G_k = a.G_k;
  p.O32 = a.Op; p.lse = a.lse;
  // upper bound on work items per head: sum ceil(n_a/128) <= N/128 + G_q
  const int maxT = (a.N + kAttnBM - 1) / kAttnBM + a.G_q;
  launch_attn<MODE_SPARSE>(p, a.d, a.bf16, dim3(maxT, a.H), a.stream);
  return hipGetLastError();
}

hipError_t launch_dense(const DenseArgs& a) {
  AttnParams p{};
  p.Q = a.Q; p.K = a.K; p.V = a.V;
  p.N = a.N;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.Oout = a.O; p.lse = a.lse;
  launch_attn<MODE_DENSE>(p, a.d, a.bf16, dim3((a.N + kAttnBM - 1) / kAttnBM, a.H), a.stream);
  return hipGetLastError();
}

// dense rows for the M probes: split-key pass + combine
hipError_t launch_probe_rows(const ProbeFitArgs& a, const int32_t* qidx) {
  AttnParams p{};
  p.Q = a.Q; p.K = a.K; p.V = a.V;
  p.N = a.N;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.qidx = qidx; p.M = a.M; p.splits = kProbeSplits;
  p.O32 = a.ws.opart; p.mpart = a.ws.mpart; p.lpart = a.ws.lpart;
  launch_attn<MODE_PROBE>(p, a.d, a.bf16, dim3((a.M + kAttnBM - 1) / kAttnBM, a.H, kProbeSplits), a.stream);
  hipLaunchKernelGGL(k_probe_combine, dim3(a.M, a.H), dim3(128), 0, a.stream, a.ws.opart, a.ws.mpart, a.ws.lpart,
                     a.H, a.M, a.d, kProbeSplits, a.O_probe);
  return hipGetLastError();
}

}  // namespace spr
