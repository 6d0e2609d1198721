// Certified k-means assignment on the fp16 matrix cores (the Lloyd rounds
// of the partition: paperlayer.ai summary appendix B.1-B.2 and C.1, where the
// GPU k-means of the pages also computes distances in reduced precision).
//
// The assignment is label = argmin_g (cn_g - 2 x . Cp_g) with ties to the
// lowest g, in float64.  Here the dot products run on
// v_mfma_f32_32x32x16_f16 with every operand split into two fp16 parts
// (hi = fp16(v), lo = fp16(v - hi); x and each centre carry their own
// power-of-two scale so the parts stay in fp16 range): x.c ~ xh.ch + xh.cl +
// xl.ch, accurate to about 2^-17 of |x| |c| after fp32 accumulation.  With a
// rigorous bound E on every score's error (from the largest ||Cp_g|| and
// |cn_g|), a point whose two best computed scores are more than 2E apart has
// the same argmin in exact arithmetic, hence in float64; the few others are
// recomputed in float64 at the end of the same block, so the labels are
// those of the float64 assignment.
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Per point: exponent e with max_d |x_d| 2^-e in [128, 256) (0 for a zero
// point), the fp16 parts of x 2^-e padded to DP dims, and ||x 2^-e||.
// G8 = DP / 8 threads per point, 8 dims each.
template <int DP, int RM>
__global__ __launch_bounds__(256) void k_lp_points(const Rows64 X, int n, int D,
                                                   uint16_t* __restrict__ xh, uint16_t* __restrict__ xl,
                                                   int32_t* __restrict__ xe, float* __restrict__ xn) {
  constexpr int G8 = DP / 8, PPB = 256 / G8;
  const int h = blockIdx.y, tid = threadIdx.x, part = tid % G8;
  const int64_t t = (int64_t)blockIdx.x * PPB + tid / G8;
  const bool ok = t < n;
  double v[8];
  double mx = 0.0;
  constexpr int VEC = RowVec<RM>::VEC;
  if (ok && part * 8 + 8 <= D && D % VEC == 0) {   // 16-byte loads
#pragma unroll
    for (int q = 0; q < 8 / VEC; ++q) {
      double w[VEC];
      RowVec<RM>::load(X, h, n, D, t, part * 8 + q * VEC, w);
#pragma unroll
      for (int i = 0; i < VEC; ++i) v[q * VEC + i] = w[i];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = part * 8 + u;
      v[u] = (ok && k < D) ? X.at<RM>(h, n, D, t, k) : 0.0;
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) mx = fmax(mx, fabs(v[u]));
#pragma unroll
  for (int o = G8 / 2; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, G8));
  const int e = mx > 0.0 ? ilogb(mx) - 7 : 0;
  double ss = 0.0;
  uint16_t hv[8], lv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const double s = ldexp(v[u], -e);
    ss = fma(s, s, ss);
    split_f16(s, hv[u], lv[u]);
  }
#pragma unroll
  for (int o = G8 / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, G8);
  if (!ok) return;
  const int64_t base = ((int64_t)h * n + t) * DP + part * 8;
  uint4 ph, pl;
  ph.x = hv[0] | ((uint32_t)hv[1] << 16); ph.y = hv[2] | ((uint32_t)hv[3] << 16);
  ph.z = hv[4] | ((uint32_t)hv[5] << 16); ph.w = hv[6] | ((uint32_t)hv[7] << 16);
  pl.x = lv[0] | ((uint32_t)lv[1] << 16); pl.y = lv[2] | ((uint32_t)lv[3] << 16);
  pl.z = lv[4] | ((uint32_t)lv[5] << 16); pl.w = lv[6] | ((uint32_t)lv[7] << 16);
  *reinterpret_cast<uint4*>(xh + base) = ph;
  *reinterpret_cast<uint4*>(xl + base) = pl;
  if (part == 0) {
    xe[(int64_t)h * n + t] = e;
    xn[(int64_t)h * n + t] = (float)sqrt(ss) * 1.0000002f;   // rounded up
  }
}

// Block of 4 waves = 128 points; centres pass through LDS 32 at a time.
// Centre rows as the A operand (lane l: centre l % 32, dims 8(l/32)..+7 of a
// 16-dim step), points as B: the accumulator gives lane l the scores of point
// l % 32 against centres 8(i/4) + 4(l/32) + i % 4 of the tile.
// Points left uncertain are assigned in float64 by the block itself at the
// end: one wave per point, the point in LDS, lanes over centres reading the
// transposed metric-applied centres (coalesced), score_g = cn_g - 2 x . Cp_g
// summed over dims in order, ties to the lowest g.
template <int DP, int RM>
__global__ __launch_bounds__(256) void k_assign_lp(const uint16_t* __restrict__ xh, const uint16_t* __restrict__ xl,
                                                   const int32_t* __restrict__ xe, const float* __restrict__ xn,
                                                   const uint16_t* __restrict__ ch, const uint16_t* __restrict__ cl,
                                                   const int32_t* __restrict__ ce, const float* __restrict__ cn32,
                                                   const float* __restrict__ cnrm, int n, int G,
                                                   const Rows64 X, int D, const double* __restrict__ cpt,
                                                   const double* __restrict__ cn,
                                                   int32_t* __restrict__ labels, int32_t* __restrict__ counts) {
  constexpr int KS = DP / 16, LDC = DP + 8;
  // Error of one computed score against the exact one: |E_g| <= KX ||x|| ||Cp_g||
  // + 2^-21 |cn_g| <= KX ||x|| max_g ||Cp_g|| + 2^-21 max_g |cn_g| = E.
  // Per product term: split error 3 * 2^-22; fp32 accumulation (worst case,
  // every addition rounded): the chain of 16 KS hi.hi terms, the two adds of
  // the combination, and the cross chain of 32 KS terms scaled by 2^-10; the
  // score doubles all of it and its own rounding adds 2^-24 (|cn| + 2 ||x||
  // ||c||).  KX takes 10 % on top.
  constexpr float KX = 1.1f * (2.0f * ((16.0f * KS + 2.0f) * 0x1p-24f + (32.0f * KS + 1.0f) * 0x1p-34f +
                                       3.0f * 0x1p-22f) +
                               2.0f * 0x1p-24f);
  __shared__ int hist[kMaxGroups];
  __shared__ __align__(16) uint16_t sh[32 * LDC];
  __shared__ __align__(16) uint16_t sl[32 * LDC];
  __shared__ float sf[32], scn[32];
  __shared__ float s_bn4[4], s_bc4[4];
  __shared__ int s_nl;                 // uncertain points of the block
  __shared__ int32_t s_list[128];
  __shared__ double xs[4][128];        // their rows, one per wave
  const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, l = tid & 63, l32 = l & 31, hf = l >> 5;
  const int64_t pt = (int64_t)blockIdx.x * 128 + wave * 32 + l32;
  const bool ok = pt < n;
  const int64_t pr = (int64_t)h * n + (ok ? pt : n - 1);
  f16x8_t bh[KS], bl[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    bh[s] = *reinterpret_cast<const f16x8_t*>(xh + pr * DP + 16 * s + 8 * hf);
    bl[s] = *reinterpret_cast<const f16x8_t*>(xl + pr * DP + 16 * s + 8 * hf);
  }
  const int ex = xe[pr];
  const float xnv = ldexpf(xn[pr], ex);
  const float fx = -ldexpf(1.0f, ex);   // score = cn + (-2^ex)(2^(ce+1)) acc
  // the bound's two factors, maximised over all centres
  float bnmax, bcmax;
  {
    float bn = 0.0f, bc = 0.0f;
    for (int g = tid; g < G; g += 256) {
      const int64_t hg = (int64_t)h * G + g;
      bn = fmaxf(bn, KX * ldexpf(cnrm[hg], ce[hg]));
      bc = fmaxf(bc, ldexpf(fabsf(cn32[hg]), -21));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      bn = fmaxf(bn, __shfl_xor(bn, o));
      bc = fmaxf(bc, __shfl_xor(bc, o));
    }
    if (l == 0) { s_bn4[wave] = bn; s_bc4[wave] = bc; }
    __syncthreads();
    bnmax = fmaxf(fmaxf(s_bn4[0], s_bn4[1]), fmaxf(s_bn4[2], s_bn4[3]));
    bcmax = fmaxf(fmaxf(s_bc4[0], s_bc4[1]), fmaxf(s_bc4[2], s_bc4[3]));
  }
  // best and second-best computed scores (b1 at centre i1, b2)
  float b1 = __builtin_inff(), b2 = __builtin_inff();
  int i1 = 0x7fffffff;
  const uint16_t* chh = ch + (int64_t)h * G * DP;
  const uint16_t* clh = cl + (int64_t)h * G * DP;
  // the next tile of 32 centre rows (hi, lo; DP / 8 chunks of 16 bytes per
  // row each) and its per-centre 2^(e+1) and cn (+inf past the last centre,
  // so it never wins) travel in registers while the current tile is used
  constexpr int CPT = 32 * (DP / 8), NPT = (CPT + 255) / 256;
  uint4 nh[NPT], nl[NPT];
  float nsf = 0.0f, nscn = 0.0f;
  auto load_next = [&](int c0) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int e = tid + 256 * u, r = e / (DP / 8), q = e % (DP / 8), g = c0 + r;
      nh[u] = make_uint4(0, 0, 0, 0);
      nl[u] = make_uint4(0, 0, 0, 0);
      if (e < CPT && g < G) {
        nh[u] = *reinterpret_cast<const uint4*>(chh + (int64_t)g * DP + q * 8);
        nl[u] = *reinterpret_cast<const uint4*>(clh + (int64_t)g * DP + q * 8);
      }
    }
    if (tid < 32) {
      const int g = c0 + tid;
      nsf = ldexpf(1.0f, (g < G ? ce[(int64_t)h * G + g] : 0) + 1);
      nscn = g < G ? cn32[(int64_t)h * G + g] : __builtin_inff();
    }
  };
  load_next(0);
  for (int c0 = 0; c0 < G; c0 += 32) {
    __syncthreads();   // the previous tile's LDS reads are done
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int e = tid + 256 * u, r = e / (DP / 8), q = e % (DP / 8);
      if (e < CPT) {
        *reinterpret_cast<uint4*>(sh + r * LDC + q * 8) = nh[u];
        *reinterpret_cast<uint4*>(sl + r * LDC + q * 8) = nl[u];
      }
    }
    if (tid < 32) { sf[tid] = nsf; scn[tid] = nscn; }
    __syncthreads();
    if (c0 + 32 < G) load_next(c0 + 32);
    // hi.hi products in one accumulator, the 2^-11-smaller cross terms in
    // another (their roundings stay at the cross terms' scale)
    f32x16 ahh = {}, axx = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const f16x8_t ah = *reinterpret_cast<const f16x8_t*>(sh + l32 * LDC + 16 * s + 8 * hf);
      const f16x8_t al = *reinterpret_cast<const f16x8_t*>(sl + l32 * LDC + 16 * s + 8 * hf);
      ahh = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh[s], ahh, 0, 0, 0);
      axx = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl[s], axx, 0, 0, 0);
      axx = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh[s], axx, 0, 0, 0);
    }
    const f32x16 acc = ahh + axx;
    const int cb = c0 + 4 * hf;   // centre of score i: cb + 8 (i / 4) + i % 4
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * hf + (i & 3);
      const float sc = fmaf(acc[i], fx * sf[r], scn[r]);
      i1 = sc < b1 ? cb + (8 * (i >> 2) + (i & 3)) : i1;
      b2 = __builtin_amdgcn_fmed3f(b1, b2, sc);   // the second smallest of b1 <= b2 and sc
      b1 = fminf(b1, sc);
    }
  }
  // merge the two half-waves' candidates of the same point
  {
    const float ob1 = __shfl_xor(b1, 32), ob2 = __shfl_xor(b2, 32);
    const int oi1 = __shfl_xor(i1, 32);
    if (ob1 < b1 || (ob1 == b1 && oi1 < i1)) {
      b2 = fminf(b1, ob2);
      b1 = ob1;
      i1 = oi1;
    } else {
      b2 = fminf(b2, ob1);
    }
  }
  for (int g = tid; g < G; g += 256) hist[g] = 0;
  if (tid == 0) s_nl = 0;
  __syncthreads();
  if (ok && hf == 0) {
    // certain when the two best computed scores are further apart than twice
    // the bound: then s_g - s_best >= (b2 - E) - (b1 + E) > 0 for every other g
    const float E = fmaf(xnv, bnmax, bcmax);
    if (b2 - b1 > 2.0f * E && i1 < G) {
      labels[(int64_t)h * n + pt] = i1;
      atomicAdd(&hist[i1], 1);
    } else {
      s_list[atomicAdd(&s_nl, 1)] = (int32_t)pt;
    }
  }
  __syncthreads();
  // the float64 pass over the uncertain points (each result is independent
  // of the list order)
  const int nunc = s_nl;
  const double* ct = cpt + (int64_t)h * D * G;
  for (int w = wave; w < nunc; w += 4) {
    const int64_t t = s_list[w];
    for (int k = l; k < D; k += 64) xs[wave][k] = X.at<RM>(h, n, D, t, k);
    __builtin_amdgcn_wave_barrier();   // the wave's LDS writes precede its reads
    double best = __builtin_inf();
    int bi = 0x7fffffff;
    for (int g = l; g < G; g += 64) {
      double dot = 0.0;
#pragma unroll 8
      for (int k = 0; k < D; ++k) dot = fma(xs[wave][k], ct[(int64_t)k * G + g], dot);
      const double sc = cn[(int64_t)h * G + g] - 2.0 * dot;
      if (sc < best) { best = sc; bi = g; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    if (l == 0) {
      labels[(int64_t)h * n + t] = bi;
      atomicAdd(&hist[bi], 1);
    }
    __builtin_amdgcn_wave_barrier();   // reads done before the next point is staged
  }
  __syncthreads();
  // label counts of this 128-point chunk
  int32_t* ch_counts = counts + ((int64_t)h * gridDim.x + blockIdx.x) * G;
  for (int g = tid; g < G; g += 256) ch_counts[g] = hist[g];
}

template <int DP>
static void launch_lp_points_t(const Rows64& X, int H, int n, int D, const LpAssign& lp, hipStream_t st) {
  constexpr int PPB = 256 / (DP / 8);
  const dim3 grid((n + PPB - 1) / PPB, H);
#define SPR_CALL(M) hipLaunchKernelGGL((k_lp_points<DP, M>), grid, dim3(256), 0, st, X, n, D, lp.xh, lp.xl, lp.xe, lp.xn)
  SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
}

template <int DP>
static void launch_assign_t(const Rows64& X, const double* Cp, const double* cn, int H, int n, int D, int G,
                            const LpAssign& lp, int32_t* labels, int32_t* counts, hipStream_t st) {
  static_assert(kSortChunk == 128, "one assignment block per counting-sort chunk");
#define SPR_CALL(M)                                                                                              \
  hipLaunchKernelGGL((k_assign_lp<DP, M>), dim3((n + 127) / 128, H), dim3(256), 0, st, lp.xh, lp.xl, lp.xe, lp.xn, \
                     lp.ch, lp.cl, lp.ce, lp.cn32, lp.cnrm, n, G, X, D, lp.cpt, cn, labels, counts)
  SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
}

#define SPR_DP_SWITCH(DPV, CALL) \
  switch (DPV) {                 \
    case 16: CALL(16); break;    \
    case 32: CALL(32); break;    \
    case 48: CALL(48); break;    \
    case 64: CALL(64); break;    \
    case 80: CALL(80); break;    \
    case 96: CALL(96); break;    \
    case 112: CALL(112); break;  \
    default: CALL(128); break;   \
  }

void launch_lp_points(const Rows64& X, int H, int n, int D, const LpAssign& lp, hipStream_t st) {
  const int dp = lp_dims(D);
#define SPR_CALL(V) launch_lp_points_t<V>(X, H, n, D, lp, st)
  SPR_DP_SWITCH(dp, SPR_CALL)
#undef SPR_CALL
}

void launch_assign_lp(const Rows64& X, const double* Cp, const double* cn, int H, int n, int D, int G,
                      const LpAssign& lp, int32_t* labels, int32_t* counts, hipStream_t st) {
  const int dp = lp_dims(D);
#define SPR_CALL(V) launch_assign_t<V>(X, Cp, cn, H, n, D, G, lp, labels, counts, st)
  SPR_DP_SWITCH(dp, SPR_CALL)
#undef SPR_CALL
}

}  // namespace spr
