// jssa_calib_moments: second moments of the calibration group-mean queries and
// of the keys, per KV head (paper summary page, §3.2 Joint Query-Key Subspace;
// README page §2 Calibration).  These sums are the only pass over calibration
// data; the basis then needs a single symmetric eigenproblem per KV head,
// solved on the host by jssa_basis.
//
// Two launches: stage_kernel writes fp32 rows x_t (qbar_t, k_t; MLA: their
// 512 latent dims) to the workspace; gram_kernel accumulates the d x d sums
// sum_t x_t x_t^T tile by tile (64 x 64 per block, tokens in fixed order, no
// atomics, so the result is deterministic) and adds them to gq / gk.
#include "common.h"
#include "kernels.h"

namespace jssa {

__global__ __launch_bounds__(256) void stage_kernel(CalibArgs a) {
  const int t = blockIdx.x, h = blockIdx.y;
  const int din = a.mla ? kMlaLatent + kMlaRope : a.d;
  for (int i = threadIdx.x; i < a.dm; i += 256) {
    const uint16_t* qp = a.q + ((int64_t)t * a.Hq + (int64_t)h * a.G) * din + i;
    float s = 0.0f;
    for (int g = 0; g < a.G; ++g) s += bf16_to_f32(qp[(int64_t)g * din]);
    a.xq[((int64_t)h * a.T + t) * a.dm + i] = s / (float)a.G;
    const uint16_t* kp = a.mla ? a.k + (int64_t)t * din + i : a.k + ((int64_t)t * a.Hkv + h) * a.d + i;
    a.xk[((int64_t)h * a.T + t) * a.dm + i] = bf16_to_f32(*kp);
  }
}

// grid: (tiles_i * tiles_j, Hkv, 2 sources); 64 x 64 output tile, 4 x 4 per thread
__global__ __launch_bounds__(256) void gram_kernel(CalibArgs a) {
  constexpr int TT = 32;
  __shared__ float xi[TT][64];
  __shared__ float xj[TT][64];
  const int tiles = a.dm / 64;
  const int ti = blockIdx.x / tiles, tj = blockIdx.x % tiles, h = blockIdx.y, src = blockIdx.z;
  const float* x = (src == 0 ? a.xq : a.xk) + (int64_t)h * a.T * a.dm;
  float* g = (src == 0 ? a.gq : a.gk) + (int64_t)h * a.dm * a.dm;
  const int tid = (int)threadIdx.x, r0 = (tid / 16) * 4, c0 = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int t0 = 0; t0 < a.T; t0 += TT) {
    for (int k = tid; k < TT * 64; k += 256) {
      const int tt = k / 64, e = k % 64;
      const bool in = t0 + tt < a.T;
      xi[tt][e] = in ? x[(int64_t)(t0 + tt) * a.dm + ti * 64 + e] : 0.0f;
      xj[tt][e] = in ? x[(int64_t)(t0 + tt) * a.dm + tj * 64 + e] : 0.0f;
    }
    __syncthreads();
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = __builtin_fmaf(xi[tt][r0 + p], xj[tt][c0 + q], acc[p][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) g[(int64_t)(ti * 64 + r0 + p) * a.dm + tj * 64 + c0 + q] += acc[p][q];
}

hipError_t launch_calib(const CalibArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(stage_kernel, dim3(a.T, a.Hkv), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles = a.dm / 64;
  hipLaunchKernelGGL(gram_kernel, dim3(tiles * tiles, a.Hkv, 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
