// Stage 5b kernels: apply the fitted affine residual map to the unprobed rows,
// put the exact dense rows at the probes, and restore original token order
// (arXiv:2608.18484, gist.science (nl) section 2B; paperlayer.ai summary
// section 4 "Sparse Execution").  HBM-bound: one read of Op (float32), one
// write of O (dtype), plus an r-rank float32 update per row.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace spr {

__global__ void k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_probe_pos(const int32_t* __restrict__ probe_idx, int N, int M, int32_t* __restrict__ pos) {
  const int h = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < M) pos[(int64_t)h * N + probe_idx[(int64_t)h * M + j]] = j;
}

// Per head and 32-rank chunk of the fit: B_r in the fragment order the
// correction kernel's first product reads (lane l, step t: row
// (d/2)(l/32) + t, rank l%32), and -xbar B_r for its initial accumulator.
// Ranks at or past rank_eff are zero.
template <int D>
__global__ __launch_bounds__(256) void k_correct_prep(const double* __restrict__ x_bar, const double* __restrict__ B_r,
                                                      const int32_t* __restrict__ rank_eff, int rank,
                                                      float* __restrict__ corr_b, float* __restrict__ corr_c) {
  constexpr int KH = D / 2;
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, nch = gridDim.x;
  const int k0 = 32 * chunk, reff = rank_eff[h];
  const double* Bh = B_r + (int64_t)h * D * rank;
  float* ob = corr_b + ((int64_t)h * nch + chunk) * KH * 64;
  for (int e = tid; e < KH * 64; e += 256) {
    const int t = e >> 6, l = e & 63, kk = k0 + (l & 31);
    ob[e] = kk < reff ? (float)Bh[(int64_t)(KH * (l >> 5) + t) * rank + kk] : 0.0f;
  }
  if (tid < 32) {
    const int kk = k0 + tid;
    double c = 0.0;
    if (kk < reff)
      for (int i = 0; i < D; ++i) c = fma(x_bar[(int64_t)h * D + i], Bh[(int64_t)i * rank + kk], c);
    corr_c[((int64_t)h * nch + chunk) * 32 + tid] = (float)(-c);
  }
}

// One wave corrects 32 consecutive group-major slots at a time with fp32
// matrix cores, in two chained products:
//   Z^T   = B_r^T (x - xbar)^T     [32 ranks x 32 rows], contraction over d
//   out^T = V_r Z^T                [d x 32 rows],        contraction over ranks
// both on v_mfma_f32_32x32x2f32.  The accumulator layout of the first product
// (lane l, register i: rank 8(i/4) + 4(l/32) + i%4, row l%32) is the B-operand
// layout of the second when its contraction steps take the ranks in that
// order, so Z never leaves registers.  xbar enters as the initial accumulator
// -xbar B_r, and out starts from x + rbar.  B_r fragments stay in registers
// and V_r (float32) in LDS across the block's tiles; fits with more than 32
// directions run in 32-rank chunks that reload both.  The finished rows go
// back through the wave's LDS tile so each row is stored to its original
// position with full 16-byte lanes; probe rows take their exact dense rows.
constexpr int kCorrWaves = 8;

template <int D, typename T>
__global__ __launch_bounds__(kCorrWaves * 64) void k_correct(
    const float* __restrict__ Op, const int32_t* __restrict__ q_perm, const int32_t* __restrict__ probe_pos,
    const float* __restrict__ O_probe, const double* __restrict__ r_bar, const float* __restrict__ corr_b,
    const float* __restrict__ corr_c, const double* __restrict__ V_r, const int32_t* __restrict__ rank_eff, int N,
    int M, int rank, int has_fit, int steps, T* __restrict__ O) {
  constexpr int LDX = D + 4;      // padded row (floats), rows 16-byte aligned
  constexpr int LDV = 36;         // V_r chunk row: 32 ranks + pad
  constexpr int NB = D / 32;      // 32-channel output tiles
  constexpr int KH = D / 2;       // contraction steps of the first product
  constexpr int EPL = 16 / (int)sizeof(T);   // output elements per 16-byte lane store
  constexpr int LPR = D / EPL;               // lanes per output row
  constexpr int RPP = 64 / LPR;              // rows per store pass
  constexpr int NT = kCorrWaves * 64;
  __shared__ float Xs[kCorrWaves][32 * LDX];
  __shared__ float Vs[D * LDV];
  __shared__ float rb[D];
  const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int lr = l & 31, hf = l >> 5;
  float* X = Xs[wave];
  const int reff = has_fit ? rank_eff[h] : 0;
  if (tid < D) rb[tid] = has_fit ? (float)r_bar[(int64_t)h * D + tid] : 0.0f;
  const int nch = (reff + 31) / 32;
  const double* Vh = V_r + (int64_t)h * D * rank;
  const int nch_alloc = (rank + 31) / 32;
  float bfr[KH];
  f32x16 zinit;
  // chunk k0..k0+31 of the fit: V_r into LDS (block-wide), B_r fragments and
  // -xbar B_r into registers
  auto load_chunk = [&](int chunk) {
    const int k0 = 32 * chunk;
    for (int e = tid; e < D * 32; e += NT) {
      const int i = e >> 5, kk = e & 31;
      Vs[i * LDV + kk] = k0 + kk < reff ? (float)Vh[(int64_t)i * rank + k0 + kk] : 0.0f;
    }
    const float* fb = corr_b + ((int64_t)h * nch_alloc + chunk) * KH * 64;
#pragma unroll
    for (int t = 0; t < KH; ++t) bfr[t] = fb[t * 64 + l];
    const float* fc = corr_c + ((int64_t)h * nch_alloc + chunk) * 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) zinit[i] = fc[8 * (i >> 2) + 4 * hf + (i & 3)];
  };
  if (nch == 1) load_chunk(0);
  __syncthreads();
  for (int it = 0; it < steps; ++it) {
    // the block takes kCorrWaves consecutive tiles per step, one per wave
    const int64_t blk0 = ((int64_t)blockIdx.x * steps + it) * kCorrWaves * 32;
    if (blk0 >= N) break;   // uniform over the block
    const int64_t s0 = blk0 + wave * 32;
    const bool active = s0 < N;
    const int rows = active ? (int)min<int64_t>(32, N - s0) : 0;
    // destinations of the rows this lane stores (and their probe numbers),
    // fetched before the products so their latency overlaps them (at most 8
    // store passes; more are fetched in the store loop)
    constexpr int NP = 32 / RPP, NPF = NP <= 8 ? NP : 1;
    int32_t tdst[NPF];
    int jprobe[NPF];
    if constexpr (NP <= 8) {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int r = pp * RPP + l / LPR;
        tdst[pp] = r < rows ? q_perm[(int64_t)h * N + s0 + r] : 0;
      }
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int r = pp * RPP + l / LPR;
        jprobe[pp] = (has_fit && r < rows) ? probe_pos[(int64_t)h * N + tdst[pp]] : -1;
      }
    }
    f32x16 acc[NB];
    if (active) {
      const float* src = Op + ((int64_t)h * N + s0) * D;
#pragma unroll 4
      for (int e = l; e < 32 * D / 4; e += 64) {
        const int r = e / (D / 4), c4 = e % (D / 4);
        f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (r < rows) v = *reinterpret_cast<const f32x4*>(src + (int64_t)r * D + 4 * c4);
        *reinterpret_cast<f32x4*>(X + r * LDX + 4 * c4) = v;
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = 32 * cb + 8 * q + 4 * hf;
          const f32x4 xv = *reinterpret_cast<const f32x4*>(X + lr * LDX + ch);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[cb][4 * q + u] = xv[u] + rb[ch + u];
        }
    }
    for (int chunk = 0; chunk < nch; ++chunk) {
      if (nch > 1) {
        __syncthreads();
        load_chunk(chunk);
        __syncthreads();
      }
      if (!active) continue;
      f32x16 z = zinit;
#pragma unroll
      for (int t = 0; t < KH; t += 4) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(X + lr * LDX + KH * hf + t);
        z = __builtin_amdgcn_mfma_f32_32x32x2f32(bfr[t + 0], xv[0], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x2f32(bfr[t + 1], xv[1], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x2f32(bfr[t + 2], xv[2], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x2f32(bfr[t + 3], xv[3], z, 0, 0, 0);
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(Vs + (32 * cb + lr) * LDV + 8 * q + 4 * hf);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[0], z[4 * q + 0], acc[cb], 0, 0, 0);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[1], z[4 * q + 1], acc[cb], 0, 0, 0);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[2], z[4 * q + 2], acc[cb], 0, 0, 0);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[3], z[4 * q + 3], acc[cb], 0, 0, 0);
        }
    }
    if (!active) continue;
    // finished rows back into the tile (each element has one owner lane)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[cb][4 * q], acc[cb][4 * q + 1], acc[cb][4 * q + 2], acc[cb][4 * q + 3]};
        *reinterpret_cast<f32x4*>(X + lr * LDX + 32 * cb + 8 * q + 4 * hf) = v;
      }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + l / LPR, c = (l % LPR) * EPL;
      if (r < rows) {
        int64_t t;
        int j;
        if constexpr (NP <= 8) {
          t = tdst[pp];
          j = jprobe[pp];
        } else {
          t = q_perm[(int64_t)h * N + s0 + r];
          j = has_fit ? probe_pos[(int64_t)h * N + t] : -1;
        }
        float v[EPL];
        if (j >= 0) {
          const float* pr = O_probe + ((int64_t)h * M + j) * D + c;
#pragma unroll
          for (int u = 0; u < EPL; u += 4) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(pr + u);
            v[u] = w[0]; v[u + 1] = w[1]; v[u + 2] = w[2]; v[u + 3] = w[3];
          }
        } else {
#pragma unroll
          for (int u = 0; u < EPL; u += 4) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(X + r * LDX + c + u);
            v[u] = w[0]; v[u + 1] = w[1]; v[u + 2] = w[2]; v[u + 3] = w[3];
          }
        }
        T* dst = O + ((int64_t)h * N + t) * D + c;
        if constexpr (sizeof(T) == 2) {
          bf16x8 o;
#pragma unroll
          for (int u = 0; u < 8; ++u) o[u] = (bf16_t)v[u];
          *reinterpret_cast<bf16x8*>(dst) = o;
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
}

// ---------------------------------------------------------------- bf16 outputs
// The same correction on the fp16 matrix cores (v_mfma_f32_32x32x16_f16) for
// outputs stored in bf16:
//   Z^T   = B_r^T (x - xbar)^T   (x - xbar formed in float32, then rounded to
//           fp16 after a per-row power-of-two scale; each B_r chunk scaled by
//           a power of two to fit fp16)
//   out^T = V_r Z^T              (Z rounded to fp16 after a per-row power-of-two
//           scale; each lane's accumulator values belong to one row)
// The added term carries a relative error of about 2^-10 of the norm of Z,
// below half an ulp of the bf16 output unless the correction exceeds the
// output itself several times over.  The exact dense rows at the probes are
// written over the corrected ones by a second kernel.
//
// Per head and 32-rank chunk: fp16 fragments of the first product's A
// operand (B_r^T: lane l, d-step s: entries d = 16s + 8(l/32) + j, rank l%32)
// and of the second's A operand (V_r: lane l, 32-channel block cb, rank-step
// t: channel 32cb + l%32, ranks 16t + 4(l/32) + (j%4) + 8(j/4) -- the order in
// which the first product's accumulator hands its ranks to the second product
// as its B operand), zero past rank_eff.
template <int D>
__global__ __launch_bounds__(256) void k_correct_prep16(const double* __restrict__ B_r,
                                                        const double* __restrict__ V_r,
                                                        const int32_t* __restrict__ rank_eff, int rank,
                                                        uint16_t* __restrict__ frag, int32_t* __restrict__ bexp) {
  constexpr int NS = D / 16, NB = D / 32;
  __shared__ double red[4];
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, nch = gridDim.x;
  const int k0 = 32 * chunk, reff = rank_eff[h];
  const double* Bh = B_r + (int64_t)h * D * rank;
  const double* Vh = V_r + (int64_t)h * D * rank;
  double mx = 0.0;
  for (int e = tid; e < D * 32; e += 256) {
    const int i = e >> 5, kk = k0 + (e & 31);
    if (kk < reff) mx = fmax(mx, fabs(Bh[(int64_t)i * rank + kk]));
  }
  mx = block_max_f64<256>(mx, red);
  const int eb = mx > 0.0 ? ilogb(mx) - 14 : 0;   // max |B 2^-eb| < 2^15
  if (tid == 0) bexp[(int64_t)h * nch + chunk] = eb;
  uint16_t* fb = frag + ((int64_t)h * nch + chunk) * 2 * 32 * D;
  uint16_t* fv = fb + 32 * D;
  for (int e = tid; e < NS * 512; e += 256) {
    const int s = e >> 9, l = (e >> 3) & 63, j = e & 7;
    const int kk = k0 + (l & 31), i = 16 * s + 8 * (l >> 5) + j;
    const double v = kk < reff ? ldexp(Bh[(int64_t)i * rank + kk], -eb) : 0.0;
    fb[e] = __builtin_bit_cast(uint16_t, f16_via_f32(v));
  }
  for (int e = tid; e < NB * 2 * 512; e += 256) {
    const int cb = e >> 10, t = (e >> 9) & 1, l = (e >> 3) & 63, j = e & 7;
    const int kk = k0 + 16 * t + 4 * (l >> 5) + (j & 3) + 8 * (j >> 2), ch = 32 * cb + (l & 31);
    const double v = kk < reff ? Vh[(int64_t)ch * rank + kk] : 0.0;
    fv[e] = __builtin_bit_cast(uint16_t, f16_via_f32(v));
  }
}

// max of v and the partner lane's (l ^ 32) value, in every lane
SPR_DEV float halves_max_f32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// orders one wave's LDS writes before its later reads by other lanes of the
// same wave (and the reverse)
SPR_DEV void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Eight waves per block, one block per CU; every wave walks its own 32-slot
// tiles of the head (stride: all waves of the head's blocks) through its own
// LDS tile, with the next tile's Op rows in flight in registers while the
// current one is corrected; no block barrier after the start.  Op is read
// and O written once: non-temporal loads and stores.
constexpr int kCorr16Waves = 8;

template <int D>
__global__ __launch_bounds__(kCorr16Waves * 64, 1) void k_correct16(
    const float* __restrict__ Op, const int32_t* __restrict__ q_perm, const double* __restrict__ x_bar,
    const double* __restrict__ r_bar, const uint16_t* __restrict__ frag, const int32_t* __restrict__ bexp,
    const int32_t* __restrict__ rank_eff, int N, int rank, int has_fit, bf16_t* __restrict__ O) {
  constexpr int LDX = D + 4;
  constexpr int NB = D / 32, NS = D / 16;
  constexpr int PF = 32 * D / 4 / 64;         // 16-byte row pieces per lane and tile
  constexpr int LPR = D / 8, RPP = 64 / LPR, NP = 32 / RPP;   // output stores: 8 bf16 per lane
  __shared__ float Xs[kCorr16Waves][32 * LDX];
  __shared__ float xb[D], rb[D];
  __shared__ __align__(16) uint16_t fr1[2 * 32 * D];   // the fragments of a one-chunk fit
  const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int lr = l & 31, hf = l >> 5;
  float* X = Xs[wave];
  const int reff = has_fit ? rank_eff[h] : 0;
  const int nch = (reff + 31) / 32, nch_alloc = (rank + 31) / 32;
  if (tid < D) {
    xb[tid] = has_fit ? (float)x_bar[(int64_t)h * D + tid] : 0.0f;
    rb[tid] = has_fit ? (float)r_bar[(int64_t)h * D + tid] : 0.0f;
  }
  if (nch == 1) {
    const uint4* g = reinterpret_cast<const uint4*>(frag + (int64_t)h * nch_alloc * 2 * 32 * D);
    for (int e = tid; e < 2 * 32 * D / 8; e += kCorr16Waves * 64) reinterpret_cast<uint4*>(fr1)[e] = g[e];
  }
  __syncthreads();
  const int ntile = (N + 31) / 32;
  const int stride = gridDim.x * kCorr16Waves;
  int tile = blockIdx.x * kCorr16Waves + wave;
  const float* src = Op + (int64_t)h * N * D;
  f32x4 pre[PF];
  auto fetch = [&](int tl) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int e = l + 64 * u, r = e / (D / 4), c4 = e % (D / 4);
      const int64_t row = (int64_t)tl * 32 + r;
      pre[u] = row < N ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + row * D + 4 * c4))
                       : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  if (tile < ntile) fetch(tile);
  for (; tile < ntile; tile += stride) {
    const int64_t s0 = (int64_t)tile * 32;
    const int rows = (int)min<int64_t>(32, N - s0);
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int e = l + 64 * u, r = e / (D / 4), c4 = e % (D / 4);
      *reinterpret_cast<f32x4*>(X + r * LDX + 4 * c4) = pre[u];
    }
    wave_sync_lds();
    // destinations of the lane's store rows, issued before the next tile's
    // rows so that the stores wait for them only
    int32_t tdst[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + l / LPR;
      tdst[pp] = r < rows ? q_perm[(int64_t)h * N + s0 + r] : 0;
    }
    if (tile + stride < ntile) fetch(tile + stride);
    f32x16 acc[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = 32 * cb + 8 * q + 4 * hf;
        const f32x4 xv = *reinterpret_cast<const f32x4*>(X + lr * LDX + ch);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[cb][4 * q + u] = xv[u] + rb[ch + u];
      }
    // the row's largest |x - xbar| (the two half-waves read its two halves)
    // sets the power-of-two scale of its fp16 operand
    float xm = 0.0f;
    if (nch > 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int d0 = 16 * s + 8 * hf;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(X + lr * LDX + d0);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(X + lr * LDX + d0 + 4);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          xm = __builtin_fmaxf(xm, __builtin_fmaxf(__builtin_fabsf(x0[u] - xb[d0 + u]),
                                                   __builtin_fabsf(x1[u] - xb[d0 + 4 + u])));
      }
      xm = halves_max_f32(xm);
    }
    const int ex = xm > 0.0f ? min(110, max(-110, ilogbf(xm) - 14)) : 0;
    const float xsc = ldexpf(1.0f, -ex);
    for (int chunk = 0; chunk < nch; ++chunk) {
      const uint16_t* fb = nch == 1 ? fr1 : frag + ((int64_t)h * nch_alloc + chunk) * 2 * 32 * D;
      const uint16_t* fv = fb + 32 * D;
      f32x16 z = {};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int d0 = 16 * s + 8 * hf;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(X + lr * LDX + d0);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(X + lr * LDX + d0 + 4);
        f16x8 b;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          b[u] = (_Float16)((x0[u] - xb[d0 + u]) * xsc);
          b[4 + u] = (_Float16)((x1[u] - xb[d0 + 4 + u]) * xsc);
        }
        const f16x8 a = *reinterpret_cast<const f16x8*>(fb + (s * 64 + l) * 8);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, z, 0, 0, 0);
      }
      // per-row power-of-two scale of Z for fp16 (both half-waves hold the row)
      float zm = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) zm = __builtin_fmaxf(zm, __builtin_fabsf(z[i]));
      zm = halves_max_f32(zm);
      const int ez = zm > 0.0f ? ilogbf(zm) - 14 : 0;
      const float zsc = ldexpf(1.0f, -ez), osc = ldexpf(1.0f, ez + ex + bexp[(int64_t)h * nch_alloc + chunk]);
      f16x8 p0, p1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p0[j] = (_Float16)(z[j] * zsc);
        p1[j] = (_Float16)(z[8 + j] * zsc);
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const f16x8 v0 = *reinterpret_cast<const f16x8*>(fv + ((cb * 2 + 0) * 64 + l) * 8);
        const f16x8 v1 = *reinterpret_cast<const f16x8*>(fv + ((cb * 2 + 1) * 64 + l) * 8);
        f32x16 pr = {};
        pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(v0, p0, pr, 0, 0, 0);
        pr = __builtin_amdgcn_mfma_f32_32x32x16_f16(v1, p1, pr, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[cb][i] = fmaf(pr[i], osc, acc[cb][i]);
      }
    }
    // finished rows back into the tile (each element has one owner lane),
    // then stored to their original positions with 16-byte lanes
    wave_sync_lds();
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[cb][4 * q], acc[cb][4 * q + 1], acc[cb][4 * q + 2], acc[cb][4 * q + 3]};
        *reinterpret_cast<f32x4*>(X + lr * LDX + 32 * cb + 8 * q + 4 * hf) = v;
      }
    wave_sync_lds();
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + l / LPR, c = (l % LPR) * 8;
      if (r < rows) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(X + r * LDX + c);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(X + r * LDX + c + 4);
        bf16x8 o;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          o[u] = (bf16_t)w0[u];
          o[4 + u] = (bf16_t)w1[u];
        }
        __builtin_nontemporal_store(o, reinterpret_cast<bf16x8*>(O + ((int64_t)h * N + tdst[pp]) * D + c));
      }
    }
    wave_sync_lds();   // the tile's reads precede the next tile's writes
  }
}

// the exact dense rows at the probes, over the corrected rows (bf16 outputs)
template <int D>
__global__ __launch_bounds__(256) void k_probe_rows16(const int32_t* __restrict__ probe_idx,
                                                       const float* __restrict__ O_probe, int N, int M,
                                                       bf16_t* __restrict__ O) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int h = blockIdx.y, j = blockIdx.x * RPB + threadIdx.x / LPR, c = (threadIdx.x % LPR) * 8;
  if (j >= M) return;
  const float* sp = O_probe + ((int64_t)h * M + j) * D + c;
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(sp);
  const f32x4 w1 = *reinterpret_cast<const f32x4*>(sp + 4);
  bf16x8 o;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    o[u] = (bf16_t)w0[u];
    o[4 + u] = (bf16_t)w1[u];
  }
  *reinterpret_cast<bf16x8*>(O + ((int64_t)h * N + probe_idx[(int64_t)h * M + j]) * D + c) = o;
}

template <int D>
static void launch_correct16_t(const CorrectArgs& a, int has_fit) {
  if (has_fit && a.rank > 0)
    hipLaunchKernelGGL((k_correct_prep16<D>), dim3((a.rank + 31) / 32, a.H), dim3(256), 0, a.stream, a.B_r, a.V_r,
                       a.rank_eff, a.rank, a.ws.corr_h, a.ws.corr_e);
  // one block per CU over all heads: at most 256 blocks in all (one CU each),
  // so no block waits for a second round behind the others
  const int ntile = (a.N + 31) / 32;
  const int per_head = std::max(1, std::min(256 / a.H, (ntile + kCorr16Waves - 1) / kCorr16Waves));
  hipLaunchKernelGGL((k_correct16<D>), dim3(per_head, a.H), dim3(kCorr16Waves * 64), 0, a.stream, a.Op, a.q_perm,
                     a.x_bar, a.r_bar, a.ws.corr_h, a.ws.corr_e, a.rank_eff, a.N, a.rank, has_fit,
                     static_cast<bf16_t*>(a.O));
  if (has_fit) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((k_probe_rows16<D>), dim3((a.M + RPB - 1) / RPB, a.H), dim3(256), 0, a.stream, a.probe_idx,
                       a.O_probe, a.N, a.M, static_cast<bf16_t*>(a.O));
  }
}

template <int D, typename T>
static void launch_correct_t(const CorrectArgs& a, int has_fit) {
  // about two waves per SIMD over the chip; a block walks runs of
  // kCorrWaves consecutive 32-slot tiles
  const int64_t tiles = (a.N + 31) / 32;
  const int64_t block_steps = (tiles + kCorrWaves - 1) / kCorrWaves;   // per head
  const int64_t blocks_wanted = 256;
  const int steps = (int)std::max<int64_t>(1, (block_steps * a.H + blocks_wanted - 1) / blocks_wanted);
  const int blocks = (int)((block_steps + steps - 1) / steps);
  if (has_fit)
    hipLaunchKernelGGL((k_correct_prep<D>), dim3(std::max(1, (a.rank + 31) / 32), a.H), dim3(256), 0, a.stream,
                       a.x_bar, a.B_r, a.rank_eff, a.rank, a.ws.corr_b, a.ws.corr_c);
  hipLaunchKernelGGL((k_correct<D, T>), dim3(blocks, a.H), dim3(kCorrWaves * 64), 0, a.stream, a.Op, a.q_perm,
                     a.ws.probe_pos, a.O_probe, a.r_bar, a.ws.corr_b, a.ws.corr_c, a.V_r, a.rank_eff, a.N, a.M,
                     a.rank, has_fit, steps, static_cast<T*>(a.O));
}

hipError_t launch_correct(const CorrectArgs& a) {
  const int has_fit = a.M > 0;
  if (a.bf16) {
    if (a.d == 128) launch_correct16_t<128>(a, has_fit);
    else launch_correct16_t<64>(a, has_fit);
    return hipGetLastError();
  }
  if (has_fit) {
    const int64_t n = (int64_t)a.H * a.N;
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, a.stream, a.ws.probe_pos, n, -1);
    hipLaunchKernelGGL(k_probe_pos, dim3((a.M + 255) / 256, a.H), dim3(256), 0, a.stream, a.probe_idx, a.N, a.M,
                       a.ws.probe_pos);
  }
  if (a.d == 128) launch_correct_t<128, float>(a, has_fit);
  else launch_correct_t<64, float>(a, has_fit);
  return hipGetLastError();
}

}  // namespace spr
