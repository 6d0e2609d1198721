// Stage 5b kernels: apply the fitted affine residual map to the unprobed rows,
// put the exact dense rows at the probes, and restore original token order
// (arXiv:2608.18484, gist.science (nl) section 2B; paperlayer.ai summary
// section 4 "Sparse Execution").  HBM-bound: one read of Op (float32), one
// write of O (dtype), plus an r-rank float32 update per row.
#include "common.hpp"
#include "kernels.hpp"

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

// 64 slots per block.  Thread (tr, tc): rows 4tr..4tr+3 of the tile,
// channels tc + 16c.  The rank-r update runs in chunks of 32 directions:
// z = (x - xbar) B_r[:, chunk], out += z V_r[:, chunk]^T.
template <int D, typename T>
__global__ __launch_bounds__(256) void k_correct(const float* __restrict__ Op, const int32_t* __restrict__ q_perm,
                                                 const int32_t* __restrict__ probe_pos,
                                                 const float* __restrict__ O_probe, const double* __restrict__ r_bar,
                                                 const double* __restrict__ x_bar, const double* __restrict__ B_r,
                                                 const double* __restrict__ V_r, const int32_t* __restrict__ rank_eff,
                                                 int N, int M, int rank, int has_fit, T* __restrict__ O) {
  constexpr int CPT = D / 16;    // channels per thread
  __shared__ float Xs[64][D + 1];   // x - xbar
  __shared__ float Bs[D][33];
  __shared__ float Vs[D][33];
  __shared__ float Zs[64][33];
  __shared__ float rb[D], xb[D];
  const int h = blockIdx.y, tid = threadIdx.x;
  const int64_t s0 = (int64_t)blockIdx.x * 64;
  const int tr = tid >> 4, tc = tid & 15;
  const int reff = has_fit ? rank_eff[h] : 0;
  if (tid < D) {
    rb[tid] = has_fit ? (float)r_bar[(int64_t)h * D + tid] : 0.0f;
    xb[tid] = has_fit ? (float)x_bar[(int64_t)h * D + tid] : 0.0f;
  }
  __syncthreads();
  float out[4][CPT];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t slot = s0 + tr * 4 + a;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tc + 16 * c;
      const float x = slot < N ? Op[((int64_t)h * N + slot) * D + ch] : 0.0f;
      out[a][c] = x + rb[ch];
      Xs[tr * 4 + a][ch] = x - xb[ch];
    }
  }
  for (int k0 = 0; k0 < reff; k0 += 32) {
    const int kc = min(32, reff - k0);
    __syncthreads();
    for (int e = tid; e < D * 32; e += 256) {
      const int i = e / 32, k = e % 32;
      Bs[i][k] = k < kc ? (float)B_r[((int64_t)h * D + i) * rank + k0 + k] : 0.0f;
      Vs[i][k] = k < kc ? (float)V_r[((int64_t)h * D + i) * rank + k0 + k] : 0.0f;
    }
    __syncthreads();
    {
      const int row = tid >> 2, kq = (tid & 3) * 8;
      float z[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) z[k] = 0.0f;
      for (int i = 0; i < D; ++i) {
        const float xv = Xs[row][i];
#pragma unroll
        for (int k = 0; k < 8; ++k) z[k] = fmaf(xv, Bs[i][kq + k], z[k]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) Zs[row][kq + k] = z[k];
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ch = tc + 16 * c;
        float acc = out[a][c];
        for (int k = 0; k < 32; ++k) acc = fmaf(Zs[tr * 4 + a][k], Vs[ch][k], acc);
        out[a][c] = acc;
      }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t slot = s0 + tr * 4 + a;
    if (slot >= N) continue;
    const int64_t t = q_perm[(int64_t)h * N + slot];
    const int j = has_fit ? probe_pos[(int64_t)h * N + t] : -1;
    T* dst = O + ((int64_t)h * N + t) * D;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tc + 16 * c;
      const float v = j >= 0 ? O_probe[((int64_t)h * M + j) * D + ch] : out[a][c];
      store_cast(dst, ch, v);
    }
  }
}

template <int D, typename T>
static void launch_correct_t(const CorrectArgs& a, int has_fit) {
  hipLaunchKernelGGL((k_correct<D, T>), dim3((a.N + 63) / 64, a.H), dim3(256), 0, a.stream, a.Op, a.q_perm,
                     a.ws.probe_pos, a.O_probe, a.r_bar, a.x_bar, a.B_r, a.V_r, a.rank_eff, a.N, a.M, a.rank,
                     has_fit, static_cast<T*>(a.O));
}

hipError_t launch_correct(const CorrectArgs& a) {
  const int has_fit = a.M > 0;
  if (has_fit) {
    const int64_t n = (int64_t)a.H * a.N;
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, a.stream, a.ws.probe_pos, n, -1);
    hipLaunchKernelGGL(k_probe_pos, dim3((a.M + 255) / 256, a.H), dim3(256), 0, a.stream, a.probe_idx, a.N, a.M,
                       a.ws.probe_pos);
  }
  if (a.d == 128) {
    if (a.bf16) launch_correct_t<128, bf16_t>(a, has_fit); else launch_correct_t<128, float>(a, has_fit);
  } else {
    if (a.bf16) launch_correct_t<64, bf16_t>(a, has_fit); else launch_correct_t<64, float>(a, has_fit);
  }
  return hipGetLastError();
}

}  // namespace spr
