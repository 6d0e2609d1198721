// Shared device helpers for the SparsePR HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPR_DEV __device__ __forceinline__

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace spr {

// 1 / q to within an ulp or two: hardware estimate and two Newton steps
SPR_DEV double recip(double q) {
  double r = __builtin_amdgcn_rcp(q);
  double e = fma(-q, r, 1.0);
  r = fma(r, e, r);
  e = fma(-q, r, 1.0);
  return fma(r, e, r);
}

constexpr int kWave = 64;

// Element loads that upcast either storage type.
SPR_DEV double load_f64(const double* p, int64_t i) { return p[i]; }
SPR_DEV double load_f64(const float* p, int64_t i) { return (double)p[i]; }
SPR_DEV double load_f64(const bf16_t* p, int64_t i) { return (double)(float)p[i]; }
SPR_DEV float load_f32(const float* p, int64_t i) { return p[i]; }
SPR_DEV float load_f32(const bf16_t* p, int64_t i) { return (float)p[i]; }

SPR_DEV void store_cast(float* p, int64_t i, float v) { p[i] = v; }
SPR_DEV void store_cast(bf16_t* p, int64_t i, float v) { p[i] = (bf16_t)v; }

// v rounded to float, then to fp16 (round to nearest even both times).
// gfx950 converts float64 to float and float to fp16 but has no direct
// float64 -> fp16 conversion; without the empty asm the compiler fuses the
// two casts into one exactly rounded conversion done in integer code, about
// ten times the work.  The two roundings stay within (2^-11 + 2^-24) |v|.
SPR_DEV _Float16 f16_via_f32(double v) {
  float f = (float)v;
  asm volatile("" : "+v"(f));
  return (_Float16)f;
}

// hi/lo fp16 parts of v (|v| < 2^9): hi is v rounded to float and then to
// fp16, lo the same rounding of the exact residual v - hi, so that
// |v - hi - lo| <= (2^-11 + 2^-24)^2 |v| (plus the fp16 subnormal spacing)
SPR_DEV void split_f16(double v, uint16_t& hi, uint16_t& lo) {
  const _Float16 h = f16_via_f32(v);
  const _Float16 l = f16_via_f32(v - (double)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

// A double moved between lanes by one DPP control (two 32-bit moves).
template <int CTRL>
SPR_DEV double dpp_move(double v) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(v), __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(v), __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// The partner values of v across the halves of each 32-lane and of the
// 64-lane span (v_permlane16_swap / v_permlane32_swap), summed by op.
template <typename Op>
SPR_DEV double cross_rows(double v, Op op) {
  {
    const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(v), __double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(v), __double2hiint(v), false, false);
    v = op(__hiloint2double(hi[0], lo[0]), __hiloint2double(hi[1], lo[1]));
  }
  {
    const auto lo = __builtin_amdgcn_permlane32_swap(__double2loint(v), __double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(__double2hiint(v), __double2hiint(v), false, false);
    v = op(__hiloint2double(hi[0], lo[0]), __hiloint2double(hi[1], lo[1]));
  }
  return v;
}

// Reduction over a wave (all 64 lanes active), the same bits in every lane:
// at each stage a lane combines its value with a partner's in the other half
// of the current span (DPP within 16-lane rows, then lane swaps across rows
// and halves), so partners form the same pairs with the operands swapped.
template <typename Op>
SPR_DEV double wave_reduce_f64(double v, Op op) {
  v = op(v, dpp_move<0xB1>(v));    // lanes ^1
  v = op(v, dpp_move<0x4E>(v));    // lanes ^2
  v = op(v, dpp_move<0x141>(v));   // mirror within 8
  v = op(v, dpp_move<0x140>(v));   // mirror within 16
  return cross_rows(v, op);
}
SPR_DEV double wave_sum_f64(double v) {
  return wave_reduce_f64(v, [](double a, double b) { return a + b; });
}
SPR_DEV double wave_max_f64(double v) {
  return wave_reduce_f64(v, [](double a, double b) { return fmax(a, b); });
}

// Block reductions (BLOCK a multiple of 64, every thread calling): a wave
// reduction, then the BLOCK / 64 wave results in wave order.  red holds
// BLOCK / 64 entries; two barriers (red may be reused right after).
template <int BLOCK>
SPR_DEV double block_sum_f64_waves(double v, double* red) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < BLOCK / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

template <int BLOCK>
SPR_DEV double block_max_f64(double v, double* red) {
  v = wave_max_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < BLOCK / 64; ++w) r = fmax(r, red[w]);
  __syncthreads();
  return r;
}

// integer sums are exact in any order
template <int BLOCK>
SPR_DEV int64_t block_sum_i64(int64_t v, int64_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t r = 0;
#pragma unroll
  for (int w = 0; w < BLOCK / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

// Deterministic block-wide sum of doubles: fixed tree over an LDS array of
// blockDim.x entries (blockDim.x a power of two).  All threads get the result.
template <int BLOCK>
SPR_DEV double block_sum_f64(double v, double* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
#pragma unroll
  for (int s = BLOCK / 2; s > 0; s >>= 1) {
    if (t < s) red[t] = red[t] + red[t + s];
    __syncthreads();
  }
  double r = red[0];
  __syncthreads();
  return r;
}

// Exclusive prefix sum over a block of BLOCK threads (a multiple of 64):
// wave-level shuffle scan, then the totals of the preceding waves.  Every
// thread returns its exclusive prefix; *total receives the block total.
// wsum holds BLOCK/64 entries.  Contains two barriers.
template <int BLOCK, typename T>
SPR_DEV T block_exclusive_scan(T v, T* wsum, T* total) {
  constexpr int NW = BLOCK / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  T before = 0, tot = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    const T t = wsum[u];
    before += u < wv ? t : T(0);
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return before + x - v;
}

}  // namespace spr
