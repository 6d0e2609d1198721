// Certified k-means assignment on the fp16 matrix cores (the Lloyd rounds
// of the partition: paperlayer.ai summary appendix B.1-B.2 and C.1, where the
// GPU k-means of the pages also computes distances in reduced precision).
//
// The assignment is label = argmin_g (cn_g - 2 x . Cp_g) with ties to the
// lowest g, in float64.  Here the dot products run on
// v_mfma_f32_32x32x16_f16 with every operand split into two fp16 parts
// (hi = fp16(v), lo = fp16(v - hi); each centre, and each 128-point chunk
// of points, carries a power-of-two scale so the parts stay in fp16 range):
// x.c ~ xh.ch + xh.cl + xl.ch, accurate to about 2^-17 of |x| |c| after fp32
// accumulation.  With a rigorous bound E on every score's error (from the
// largest ||Cp_g|| and |cn_g|, plus the subnormal parts of points much
// smaller than their chunk's largest and the index bits packed into the
// scores), a point whose two best computed scores are more than 2E apart has
// the same argmin in exact arithmetic, hence in float64; the few others are
// recomputed in float64 at the end of the same block, so the labels are
// those of the float64 assignment.  The margin also covers the rounding of a
// float64 evaluation of the expanded distance ||y||^2 - 2 y.c + ||c||^2 in the
// coordinates the method defines (y the point, c a centre; y = C^T u in the
// query metric form, where ||y||^2 = u^T A u = G'): with at most 1024 terms
// per dot product that error is below 2^-40 (||y|| + ||c||)^2, so a point
// certified here has the same argmin under any such float64 evaluation, not
// only in exact arithmetic.
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// Threads per point of k_lp_points: DP / 8 (8 dims each; DP is a power of
// two, so this is a segment width a lane shuffle reduces correctly).
template <int DP>
constexpr int lp_point_lanes() {
  return DP / 8;
}

// Per 128-point chunk (the points of one assignment block): exponent e with
// max |x_d| 2^-e over the chunk's points in [128, 256) (0 for an all-zero
// chunk); per point the fp16 parts of x 2^-e padded to DP dims, ||x 2^-e||
// and e.  One exponent per chunk makes the point scale uniform in the
// assignment block.  G8 = DP / 8 threads per point, 8 dims each (dims past
// D are zeros); the block takes the chunk in 128 / (256 / G8) passes, once
// for the maximum and once for the parts.
template <int DP, int RM>
__global__ __launch_bounds__(256) void k_lp_points(const Rows64 X, int n, int D,
                                                   uint16_t* __restrict__ xh, uint16_t* __restrict__ xl,
                                                   int32_t* __restrict__ xe, float* __restrict__ xn) {
  constexpr int G8 = lp_point_lanes<DP>(), PPB = 256 / G8, NP = 128 / PPB;
  static_assert(NP >= 1 && NP * PPB == 128, "a block covers one 128-point chunk");
  constexpr int VEC = RowVec<RM>::VEC;
  __shared__ double s_mx[4];
  const int h = blockIdx.y, tid = threadIdx.x, part = tid % G8;
  auto load = [&](int64_t t, double (&v)[8]) {
    const bool ok = t < n;
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
  };
  double mx = 0.0;
  for (int p = 0; p < NP; ++p) {
    double v[8];
    load((int64_t)blockIdx.x * 128 + p * PPB + tid / G8, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = fmax(mx, fabs(v[u]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) s_mx[tid >> 6] = mx;
  __syncthreads();
  mx = fmax(fmax(s_mx[0], s_mx[1]), fmax(s_mx[2], s_mx[3]));
  const int e = mx > 0.0 ? ilogb(mx) - 7 : 0;
  for (int p = 0; p < NP; ++p) {
    const int64_t t = (int64_t)blockIdx.x * 128 + p * PPB + tid / G8;
    double v[8];
    load(t, v);
    double ss = 0.0;
    uint16_t hv[8], lv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double sv = ldexp(v[u], -e);
      ss = fma(sv, sv, ss);
      split_f16(sv, hv[u], lv[u]);
    }
#pragma unroll
    for (int o = G8 / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, G8);
    if (t >= n) continue;
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
__global__ __launch_bounds__(256, 3) void k_assign_lp(const uint16_t* __restrict__ xh, const uint16_t* __restrict__ xl,
                                                   const int32_t* __restrict__ xe, const float* __restrict__ xn,
                                                   const uint16_t* __restrict__ ch, const uint16_t* __restrict__ cl,
                                                   const int32_t* __restrict__ ce, const float* __restrict__ cn32,
                                                   const float* __restrict__ cnrm, int n, int G,
                                                   const Rows64 X, int D, const double* __restrict__ cpt,
                                                   const double* __restrict__ cn,
                                                   const int32_t* __restrict__ gprime,
                                                   int32_t* __restrict__ labels, int32_t* __restrict__ counts) {
  // LDS centre rows: DP / 8 16-byte chunks and one chunk of padding, an odd
  // stride, so 16 consecutive rows read at one chunk hit 16 distinct bank
  // groups and every operand read is a row base plus a constant
  constexpr int KS = DP / 16, CPR = DP / 8, RS = CPR + 1, TILE = 32 * RS * 8;
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
  // two buffers of one 32-centre tile: hi parts, then lo parts; separate
  // objects, so the compiler sees that the copies into one do not touch the
  // reads of the other
  __shared__ __align__(16) uint16_t stile0[2 * TILE];
  __shared__ __align__(16) uint16_t stile1[2 * TILE];
  __shared__ float s_sf0[32], s_scn0[32], s_sf1[32], s_scn1[32];
  __shared__ float s_bn4[4], s_bc4[4];
  __shared__ int s_nl;                 // uncertain points of the block
  __shared__ int32_t s_list[128];
  __shared__ double xs[4][128];        // their rows, one per wave
  __shared__ double s_bb[12];          // per-wave minima of the block-wide pass (three points)
  __shared__ int s_bi[12];
  const int h = blockIdx.y, tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, l32 = l & 31, hf = l >> 5;
  const int64_t pt = (int64_t)blockIdx.x * 128 + wave * 32 + l32;
  const bool ok = pt < n;
  const int64_t pr = (int64_t)h * n + (ok ? pt : n - 1);
  f16x8_t bh[KS], bl[KS];   // the points' fp16 parts (B operand), loaded below
  int ex;                    // the block's point exponent
  // best and second-best packed scores: the low 4 bits of a score's float
  // carry its place i in the lane's 16 scores of the tile (perturbing it by
  // at most 15 units in the last place, which the certificate covers); i1 is
  // the first centre of the tile that holds the best so far
  float b1 = __builtin_inff(), b2 = __builtin_inff();
  int i1 = 0x7fffffff;
  const uint16_t* chh = ch + (int64_t)h * G * DP;
  const uint16_t* clh = cl + (int64_t)h * G * DP;
  // Centre tiles go from global memory straight into LDS (one 16-byte chunk
  // per lane and copy, no register staging), double-buffered with one
  // barrier per tile.  A copy fills RI whole padded rows (lanes on a padding
  // slot or past the last row stay idle); the 2 NIP copies of a tile (hi and
  // lo parts) are dealt round-robin to the waves.  Rows past the last centre
  // copy row G - 1 (their cn is a huge sentinel, so they never win).  Each
  // wave waits for its own copies before the barrier that publishes the tile.
  constexpr int RI = 64 / RS, NIP = (32 + RI - 1) / RI;
  auto copy_tile = [&](int c0, uint16_t* dst) {
#pragma unroll
    for (int j = wave; j < 2 * NIP; j += 4) {
      const int part = j / NIP, k = j % NIP;
      const int r = k * RI + l / RS, p = l % RS;
      if (l < RI * RS && r < 32 && p < CPR) {
        // uniform tile base plus a 32-bit lane offset (row G - 1 at most)
        const char* tb = reinterpret_cast<const char*>((part ? clh : chh) + (int64_t)c0 * DP);
        const uint32_t off = (uint32_t)((min(c0 + r, G - 1) - c0) * DP * 2 + p * 16);
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(tb + off),
                                         (lds_void*)(dst + part * TILE + k * RI * RS * 8), 16, 0, 0);
      }
    }
  };
  // per-centre exponent and cn of the tile after next (2^126 past the last
  // centre: finite, so packing stays a number, and never the best) travel in
  // registers of the first 32 threads, raw: they are only used (the factor
  // -2^(ex + e + 1) formed) when stored a tile later, so no wait on them
  // holds up the tile copies issued next to them
  int nce = 0;
  float nscn = 0.0f;
  auto load_small = [&](int c0) {
    if (tid < 32) {
      const int g = c0 + tid;
      nce = g < G ? ce[(int64_t)h * G + g] : 0;
      nscn = g < G ? cn32[(int64_t)h * G + g] : 0x1p126f;
    }
  };
  // One tile: publish it, start the next one's copies into the other
  // buffer, score the 32 centres, wait for this wave's copies.
  auto tile_step = [&](int c0, const uint16_t* th, const float* sf, const float* scn, uint16_t* nxt, float* nsfb,
                       float* nscnb) {
    __syncthreads();   // tile c0 is in LDS; the other buffer's readers are done
    if (c0 + 32 < G) {
      copy_tile(c0 + 32, nxt);
      if (tid < 32) { nsfb[tid] = -ldexpf(1.0f, ex + nce + 1); nscnb[tid] = nscn; }
      load_small(c0 + 64);
    }
    const uint16_t* tl = th + TILE;
    // operand of 16-dim step s: row l32, chunk 2 s + hf
    auto frag = [&](const uint16_t* t, int s) {
      return *reinterpret_cast<const f16x8_t*>(t + (l32 * RS + 2 * s + hf) * 8);
    };
    // One accumulator: the 2^-11-smaller cross terms first, so that their
    // roundings stay at their own scale (32 KS of them, each within 2^-24 of
    // a running sum below 2^-10 sum |x_d c_d|), then the hi.hi products on
    // top (16 KS roundings, each within 2^-24 of (1 + 2^-10) sum |x_d c_d|):
    // inside the bound's 16 KS + 2 and 32 KS + 1 roundings.  The hi parts
    // are read twice rather than held.
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const f16x8_t ah = frag(th, s), al = frag(tl, s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl[s], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(frag(th, s), bh[s], acc, 0, 0, 0);
    // the per-centre factors are read here, not while the products run (that
    // would hold 32 more registers through the tile and cost a wave per SIMD)
    __builtin_amdgcn_sched_barrier(0);
    // centre of score i: c0 + 4 hf + 8 (i / 4) + i % 4
    const float b1_in = b1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * hf + (i & 3);
      const float sc = fmaf(acc[i], sf[r], scn[r]);
      const float pk = __uint_as_float((__float_as_uint(sc) & ~15u) | (uint32_t)i);
      b2 = __builtin_amdgcn_fmed3f(b1, b2, pk);   // the second smallest of b1 <= b2 and pk
      b1 = __builtin_amdgcn_fmed3f(b1, pk, -0x1.fffffep127f);   // min(b1, pk) of finite scores, no canonicalising
    }
    i1 = b1 < b1_in ? c0 : i1;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of the next tile have landed
  };
  // the first tile's copies go out before the points' loads, so that their
  // latencies overlap
  copy_tile(0, stile0);
  load_small(0);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    bh[s] = *reinterpret_cast<const f16x8_t*>(xh + pr * DP + 16 * s + 8 * hf);
    bl[s] = *reinterpret_cast<const f16x8_t*>(xl + pr * DP + 16 * s + 8 * hf);
  }
  // the points of a block share one exponent (one 128-point chunk of
  // k_lp_points): score = cn + (-2^(ex + ce + 1)) acc, one factor per centre
  ex = xe[pr];
  const float xnv = ldexpf(xn[pr], ex);
  // the bound's two factors, maximised over all centres: per wave here, over
  // the waves after the tile loop (whose barriers publish them)
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
  }
  if (tid < 32) { s_sf0[tid] = -ldexpf(1.0f, ex + nce + 1); s_scn0[tid] = nscn; }
  load_small(32);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of tile 0 have landed
  for (int c0 = 0; c0 < G; c0 += 64) {
    tile_step(c0, stile0, s_sf0, s_scn0, stile1, s_sf1, s_scn1);
    if (c0 + 32 < G) tile_step(c0 + 32, stile1, s_sf1, s_scn1, stile0, s_sf0, s_scn0);
  }
  const float bnmax = fmaxf(fmaxf(s_bn4[0], s_bn4[1]), fmaxf(s_bn4[2], s_bn4[3]));
  const float bcmax = fmaxf(fmaxf(s_bc4[0], s_bc4[1]), fmaxf(s_bc4[2], s_bc4[3]));
  if (i1 != 0x7fffffff) {
    const int i = (int)(__float_as_uint(b1) & 15u);
    i1 += 8 * (i >> 2) + (i & 3) + 4 * hf;
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
    // certain when the two best packed scores are further apart than twice
    // the bound: then s_g - s_best >= (b2 - E) - (b1 + E) > 0 for every other g.
    // E adds the float64 expanded-distance error 2^-40 (||y|| + max_g ||c_g||)^2,
    // ||c_g||^2 = cn_g (= 2^21 bcmax at most), ||y||^2 = G' in the metric form;
    // the split residual of x that the relative term does not cover (a point
    // much smaller than the largest of its chunk has subnormal fp16 parts: at
    // most 2^-25 per dim in units of 2^ex, so 2^(ex-24) sqrt(DP) max||Cp_g||
    // on a score); and the packing, 15 units in the last place of a score,
    // below 2^-19 (max|cn_g| + 2 ||x|| max||Cp_g||).
    const float cnmax = ldexpf(bcmax, 21);
    const float cmax = sqrtf(cnmax);
    const float cpmax = bnmax * (1.0f / KX) * 1.001f;
    const float ynorm = gprime != nullptr ? sqrtf((float)gprime[h]) * 1.0001f : xnv;
    const float E = fmaf(xnv, bnmax, bcmax) + 0x1p-40f * (ynorm + cmax) * (ynorm + cmax) +
                    ldexpf(1.1f * sqrtf((float)DP) * cpmax, ex - 24) +
                    0x1p-19f * 1.01f * (cnmax + 2.0f * xnv * cpmax);
    if (b2 - b1 > 2.0f * E && i1 < G) {
      labels[(int64_t)h * n + pt] = i1;
      atomicAdd(&hist[i1], 1);
    } else {
      s_list[atomicAdd(&s_nl, 1)] = (int32_t)pt;
    }
  }
  __syncthreads();
  // the float64 pass over the uncertain points (each result is independent
  // of the list order).  Up to three points: the whole block on all of them
  // at once, one centre per thread; more: one wave per point.  Either way each score
  // sums its dims in order, and the minimum takes the lowest index on ties.
  const int nunc = s_nl;
  const double* ct = cpt + (int64_t)h * D * G;
  auto score = [&](const double* x, int g) {
    double dot = 0.0;
#pragma unroll 8
    for (int k = 0; k < D; ++k) dot = fma(x[k], ct[(int64_t)k * G + g], dot);
    return cn[(int64_t)h * G + g] - 2.0 * dot;
  };
  auto wave_argmin = [&](double& best, int& bi) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
  };
  if (nunc > 0 && nunc <= 3) {
    // all (up to three) points in one pass: each centre entry is loaded once
    // for every point (rows of absent points are zeros, their results
    // unused); each point's score is the same in-order sum as score()
    for (int u = 0; u < 3; ++u) {
      const int64_t t = u < nunc ? s_list[u] : 0;
      for (int k = tid; k < D; k += 256) xs[u][k] = u < nunc ? X.at<RM>(h, n, D, t, k) : 0.0;
    }
    __syncthreads();
    double best[3] = {__builtin_inf(), __builtin_inf(), __builtin_inf()};
    int bi[3] = {0x7fffffff, 0x7fffffff, 0x7fffffff};
    for (int g = tid; g < G; g += 256) {
      double dot[3] = {0.0, 0.0, 0.0};
      const double* cg = ct + g;
#pragma unroll 8
      for (int k = 0; k < D; ++k) {
        const double c = cg[(int64_t)k * G];
#pragma unroll
        for (int u = 0; u < 3; ++u) dot[u] = fma(xs[u][k], c, dot[u]);
      }
      const double cng = cn[(int64_t)h * G + g];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const double sc = cng - 2.0 * dot[u];
        if (sc < best[u]) { best[u] = sc; bi[u] = g; }
      }
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      wave_argmin(best[u], bi[u]);
      if (l == 0) { s_bb[4 * u + wave] = best[u]; s_bi[4 * u + wave] = bi[u]; }
    }
    __syncthreads();
    if (tid < nunc) {
      double b = s_bb[4 * tid];
      int bix = s_bi[4 * tid];
      for (int w = 1; w < 4; ++w)
        if (s_bb[4 * tid + w] < b || (s_bb[4 * tid + w] == b && s_bi[4 * tid + w] < bix)) {
          b = s_bb[4 * tid + w];
          bix = s_bi[4 * tid + w];
        }
      labels[(int64_t)h * n + s_list[tid]] = bix;
      atomicAdd(&hist[bix], 1);
    }
  } else {
    for (int w = wave; w < nunc; w += 4) {
      const int64_t t = s_list[w];
      for (int k = l; k < D; k += 64) xs[wave][k] = X.at<RM>(h, n, D, t, k);
      __builtin_amdgcn_wave_barrier();   // the wave's LDS writes precede its reads
      double best = __builtin_inf();
      int bi = 0x7fffffff;
      for (int g = l; g < G; g += 64) {
        const double sc = score(xs[wave], g);
        if (sc < best) { best = sc; bi = g; }
      }
      wave_argmin(best, bi);
      if (l == 0) {
        labels[(int64_t)h * n + t] = bi;
        atomicAdd(&hist[bi], 1);
      }
      __builtin_amdgcn_wave_barrier();   // reads done before the next point is staged
    }
  }
  __syncthreads();
  // label counts of this 128-point chunk
  int32_t* ch_counts = counts + ((int64_t)h * gridDim.x + blockIdx.x) * G;
  for (int g = tid; g < G; g += 256) ch_counts[g] = hist[g];
}

template <int DP>
static void launch_lp_points_t(const Rows64& X, int H, int n, int D, const LpAssign& lp, hipStream_t st) {
  const dim3 grid((n + 127) / 128, H);
#define SPR_CALL(M) hipLaunchKernelGGL((k_lp_points<DP, M>), grid, dim3(256), 0, st, X, n, D, lp.xh, lp.xl, lp.xe, lp.xn)
  SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
}

template <int DP>
static void launch_assign_t(const Rows64& X, const double* Cp, const double* cn, const int32_t* gprime, int H, int n,
                            int D, int G, const LpAssign& lp, int32_t* labels, int32_t* counts, hipStream_t st) {
  static_assert(kSortChunk == 128, "one assignment block per counting-sort chunk");
#define SPR_CALL(M)                                                                                              \
  hipLaunchKernelGGL((k_assign_lp<DP, M>), dim3((n + 127) / 128, H), dim3(256), 0, st, lp.xh, lp.xl, lp.xe, lp.xn, \
                     lp.ch, lp.cl, lp.ce, lp.cn32, lp.cnrm, n, G, X, D, lp.cpt, cn, gprime, labels, counts)
  SPR_ROWS_SWITCH(X.mode(), SPR_CALL)
#undef SPR_CALL
}

#define SPR_DP_SWITCH(DPV, CALL) \
  switch (DPV) {                 \
    case 16: CALL(16); break;    \
    case 32: CALL(32); break;    \
    case 64: CALL(64); break;    \
    default: CALL(128); break;   \
  }

void launch_lp_points(const Rows64& X, int H, int n, int D, const LpAssign& lp, hipStream_t st) {
  const int dp = lp_dims(D);
#define SPR_CALL(V) launch_lp_points_t<V>(X, H, n, D, lp, st)
  SPR_DP_SWITCH(dp, SPR_CALL)
#undef SPR_CALL
}

void launch_assign_lp(const Rows64& X, const double* Cp, const double* cn, const int32_t* gprime, int H, int n, int D,
                      int G, const LpAssign& lp, int32_t* labels, int32_t* counts, hipStream_t st) {
  const int dp = lp_dims(D);
#define SPR_CALL(V) launch_assign_t<V>(X, Cp, cn, gprime, H, n, D, G, lp, labels, counts, st)
  SPR_DP_SWITCH(dp, SPR_CALL)
#undef SPR_CALL
}

}  // namespace spr
