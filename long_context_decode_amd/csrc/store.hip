// jssa_store: project new keys with the calibrated basis and append them,
// FP8-quantised with one fp32 scale per (token, KV head), to the projected
// scoring cache (paper summary page, §3.4 Projected Scoring Cache:
// K_proj = K M^T kept in FP8; MLA scores on 64 latent + 64 RoPE dims).
//
// One wavefront per (new token, KV head).  Lane o computes output o (and
// o + 64 for the 128-dim MLA representation) with one fp32 FMA chain over the
// input dims; the per-token absmax is a wave max; codes are written into the
// piece-major (page, head) block: byte (i/16)*page*16 + slot*16 + i%16.
#include "common.h"
#include "kernels.h"

namespace jssa {

__global__ __launch_bounds__(256) void store_kernel(StoreArgs a) {
  const int wave = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = lane_id();
  const int t = wave / a.Hkv, h = wave % a.Hkv;
  if (t >= a.T) return;
  const int sl = a.slot[t];
  if (sl < 0) return;
  const int page = sl / a.P, sip = sl % a.P;

  // input row (bf16) and the rows of M this lane needs
  const uint16_t* row = a.mla ? a.k_new + (int64_t)t * (kMlaLatent + kMlaRope)
                              : a.k_new + ((int64_t)t * a.Hkv + h) * a.d;
  const int din = a.mla ? kMlaLatent : a.d;
  float y[2] = {0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = lane + 64 * k;
    if (o < a.r) {
      y[k] = project_row(a.M + ((int64_t)(a.mla ? 0 : h) * a.r + o) * din, row, din);
    } else if (a.mla && o < a.S) {
      y[k] = bf16_to_f32(row[kMlaLatent + (o - a.r)]);   // RoPE dims pass through
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (lane + 64 * k < a.S) amax = fmaxf(amax, fabsf(y[k]));
  amax = wave_max(amax);
  const float scale = amax / 448.0f;

#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = lane + 64 * k;
    if (o < a.S) {
      const uint32_t code = (scale > 0.0f) ? f32_to_fp8(y[k] / scale) : 0u;
      a.kp[kp_offset(page, h, sip, o, a.Hkv, a.S, a.P)] = (uint8_t)code;
    }
  }
  if (lane == 0) a.kp_scale[((int64_t)page * a.Hkv + h) * a.P + sip] = scale;
}

hipError_t launch_store(const StoreArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.T * a.Hkv;
  if (waves == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL(store_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
