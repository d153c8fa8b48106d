// jssa_store: project new keys with the calibrated basis and append them,
// FP8-quantised with one fp32 scale per (token, KV head), to the projected
// scoring cache (paper summary page, §3.4 Projected Scoring Cache:
// K_proj = K M^T kept in FP8; MLA scores on 64 latent + 64 RoPE dims).
//
// The scale format (fp32, one-byte power of two, none) follows the shape; the
// BF16-key format stores y itself rounded to bf16 (two bytes per element, no
// scale).
//
// One wavefront per (new token, KV head).  The projected outputs are done
// eight at a time: lane l takes part l & 7 of output 8 pass + (l >> 3)
// (project_part / proj_combine); the MLA RoPE dims pass through, one per
// lane.  The per-token absmax is a wave max; codes are written into the
// piece-major (page, head) block: byte (i/16)*page*16 + slot*16 + i%16.
#include "common.h"
#include "kernels.h"

namespace jssa {

namespace {
constexpr int kMaxPasses = 16;   // r <= 128
}

__global__ __launch_bounds__(256) void store_kernel(StoreArgs a) {
  const int wave = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = lane_id();
  const int t = wave / a.Hkv, h = wave % a.Hkv;
  if (t >= a.T) return;                               // uniform per wavefront
  const int sl = a.slot[t];
  if (sl < 0) return;
  const int page = sl / a.P, sip = sl % a.P;
  const int oi = lane >> 3, part = lane & 7;

  const uint16_t* row = a.mla ? a.k_new + (int64_t)t * (kMlaLatent + kMlaRope)
                              : a.k_new + ((int64_t)t * a.Hkv + h) * a.d;
  const int din = a.mla ? kMlaLatent : a.d;
  const float* Mh = a.M + (int64_t)(a.mla ? 0 : h) * a.r * din;
  const int passes = a.r >> 3;
  float y[kMaxPasses];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < kMaxPasses; ++p) {
    if (p < passes) {
      y[p] = proj_combine(project_part(Mh + (int64_t)(p * 8 + oi) * din, row, din, part));
      amax = fmaxf(amax, fabsf(y[p]));
    }
  }
  float yr = 0.0f;
  if (a.mla) {                                        // RoPE dims: lane l -> output r + l
    yr = bf16_to_f32(row[kMlaLatent + lane]);
    amax = fmaxf(amax, fabsf(yr));
  }
  if (a.sfmt == 3) {                                  // BF16 keys: y rounded, no scale
#pragma unroll
    for (int p = 0; p < kMaxPasses; ++p) {
      if (p < passes && part == 0)
        *reinterpret_cast<uint16_t*>(a.kp + kp_offset(page, h, sip, 2 * (p * 8 + oi), a.Hkv, 2 * a.S, a.P)) =
            f32_to_bf16(y[p]);
    }
    if (a.mla)
      *reinterpret_cast<uint16_t*>(a.kp + kp_offset(page, h, sip, 2 * (a.r + lane), a.Hkv, 2 * a.S, a.P)) =
          f32_to_bf16(yr);
    return;
  }
  amax = wave_max(amax);
  uint32_t stored;
  const float div = quant_divisor(amax, a.sfmt, &stored);

#pragma unroll
  for (int p = 0; p < kMaxPasses; ++p) {
    if (p < passes && part == 0) {
      const uint32_t code = (div > 0.0f) ? f32_to_fp8(y[p] / div) : 0u;
      a.kp[kp_offset(page, h, sip, p * 8 + oi, a.Hkv, a.S, a.P)] = (uint8_t)code;
    }
  }
  if (a.mla) {
    const uint32_t code = (div > 0.0f) ? f32_to_fp8(yr / div) : 0u;
    a.kp[kp_offset(page, h, sip, a.r + lane, a.Hkv, a.S, a.P)] = (uint8_t)code;
  }
  if (lane == 0) store_scale(a.kp_scale, ((int64_t)page * a.Hkv + h) * a.P + sip, a.sfmt, stored);
}

hipError_t launch_store(const StoreArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.T * a.Hkv;
  if (waves == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL(store_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
