// Per-wavefront pieces of the GQA flash-decode shared by attend_kernel and the
// fused select + attend kernel (paper summary page, §3.3 Gather-Free Indexed
// Attention: each K/V row is read in place through the block table and serves
// every query head of its KV head).
//
// A wavefront takes 64 positions at a time ("batch"); lane i holds the slot
// (physical page * P + offset) of position i of the batch, or -1.  Row r of 16
// lanes handles positions 16r .. 16r + 15, one per iteration; a lane holds D/16
// elements of a row, 8 contiguous ones of each 128-dim block (one 16-byte load
// per block, so that a load instruction covers 256 contiguous bytes of a row).
// Per batch:
//   A. the K rows are requested 16 (d = 128) or 8 (d = 256) at a time, q.k is
//      formed with v_dot2_f32_bf16 on bf16 pairs and summed over the row with
//      DPP; each position's logit (base 2, scaled by sm * log2 e) lands in the
//      lane that owns the position;
//   B. one softmax update per batch: the wave max of the 64 logits, a single
//      rescale of the running state, p = 2^(x - m) per lane;
//   C. the V rows are requested 8 (d = 128) or 4 (d = 256) at a time and
//      o += p v, p broadcast along the row with DPP (row_newbcast).
// The running max is uniform over the wavefront, so the rows' partial sums add
// directly (wave_state_sum).
#pragma once

#include "common.h"

namespace jssa {

template <int D>
struct AttendShape {
  static constexpr int EPL = D / 16;    // elements per lane
  static constexpr int NV = EPL / 8;    // 16-byte loads per lane per row
  static constexpr int NP = EPL / 2;    // bf16 pairs per lane per row
  static constexpr int GRP = 8 / NV;    // V rows whose loads are in flight together (32 VGPRs)
  static constexpr int GRPK = 16 / NV;  // K rows whose loads are in flight together (64 VGPRs)
};

// 16 bytes of a K or V row; a full-cache scan reads every row once, so its
// loads are streaming (non-temporal) ones
template <bool STREAM>
__device__ __forceinline__ uint4 load_row_piece(const uint16_t* p) {
  return STREAM ? load_stream_u4(p) : *reinterpret_cast<const uint4*>(p);
}

// The G query heads of a KV head as bf16 pairs, this lane's dims (unscaled;
// the scale is applied to the row sums).  q points at the group's first head.
template <int D, int G>
__device__ __forceinline__ void load_query_pairs(const uint16_t* q, int c16, uint32_t (&qp)[G][AttendShape<D>::NP]) {
  constexpr int NV = AttendShape<D>::NV;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint4 u = *reinterpret_cast<const uint4*>(q + (int64_t)g * D + c16 * 8 + v * 128);
      qp[g][4 * v] = u.x;
      qp[g][4 * v + 1] = u.y;
      qp[g][4 * v + 2] = u.z;
      qp[g][4 * v + 3] = u.w;
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void attend_state_init(float (&m)[G], float (&l)[G], float (&o)[G][AttendShape<D>::EPL]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < AttendShape<D>::EPL; ++e) o[g][e] = 0.0f;
  }
}

// One batch of 64 positions (lane i: slot ri of position i, -1 = none).
// kbase / vbase point at this lane's first element of slot 0's row of the KV
// head; row_stride = elements between consecutive slots.
template <int D, int G, bool STREAM>
__device__ __forceinline__ void attend_batch(const uint16_t* kbase, const uint16_t* vbase, int64_t row_stride, int ri,
                                             const uint32_t (&qp)[G][AttendShape<D>::NP], float sm_log2, int c16,
                                             float (&m)[G], float (&l)[G], float (&o)[G][AttendShape<D>::EPL]) {
  constexpr int EPL = AttendShape<D>::EPL, NV = AttendShape<D>::NV;
  constexpr int GRP = AttendShape<D>::GRP, GRPK = AttendShape<D>::GRPK;
  // ---- A: logits of the 64 positions (row r, iteration u -> position 16r + u)
  float xs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) xs[g] = -INFINITY;
#pragma unroll
  for (int u0 = 0; u0 < 16; u0 += GRPK) {
    uint4 kr[GRPK][NV];
#pragma unroll
    for (int u = 0; u < GRPK; ++u) {
      const int rr = row_bcast(ri, u0 + u);
      const int64_t ro = (int64_t)(rr < 0 ? 0 : rr) * row_stride;
#pragma unroll
      for (int v = 0; v < NV; ++v) kr[u][v] = load_row_piece<STREAM>(kbase + ro + v * 128);
    }
#pragma unroll
    for (int u = 0; u < GRPK; ++u) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc = dot2_bf16(kr[u][v].x, qp[g][4 * v], acc);
          acc = dot2_bf16(kr[u][v].y, qp[g][4 * v + 1], acc);
          acc = dot2_bf16(kr[u][v].z, qp[g][4 * v + 2], acc);
          acc = dot2_bf16(kr[u][v].w, qp[g][4 * v + 3], acc);
        }
        const float x = row16_sum(acc) * sm_log2;
        if (c16 == u0 + u) xs[g] = x;
      }
    }
  }
  if (ri < 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) xs[g] = -INFINITY;
  }
  // ---- B: one softmax update for the batch
  float p[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mn = fmaxf(m[g], wave_max(xs[g]));
    if (mn > m[g]) {                     // uniform over the wavefront
      const float al = __builtin_amdgcn_exp2f(m[g] - mn);
      l[g] *= al;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] *= al;
      m[g] = mn;
    }
    p[g] = (m[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(xs[g] - m[g]);
    l[g] += p[g];
  }
  // ---- C: o += p v over the 64 rows
#pragma unroll
  for (int u0 = 0; u0 < 16; u0 += GRP) {
    uint4 vr[GRP][NV];
#pragma unroll
    for (int u = 0; u < GRP; ++u) {
      const int rr = row_bcast(ri, u0 + u);
      const int64_t ro = (int64_t)(rr < 0 ? 0 : rr) * row_stride;
#pragma unroll
      for (int v = 0; v < NV; ++v) vr[u][v] = load_row_piece<STREAM>(vbase + ro + v * 128);
    }
#pragma unroll
    for (int u = 0; u < GRP; ++u) {
      float pp[G];
#pragma unroll
      for (int g = 0; g < G; ++g) pp[g] = row_bcast_f(p[g], u0 + u);
      // a missing position's row is read from slot 0: its weight is 0, and
      // its values are zeroed so that whatever slot 0 holds adds nothing
      const bool ok = row_bcast(ri, u0 + u) >= 0;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint4 vv = vr[u][v];
        const uint32_t ww[4] = {ok ? vv.x : 0u, ok ? vv.y : 0u, ok ? vv.z : 0u, ok ? vv.w : 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = bf16_lo(ww[e]), v1 = bf16_hi(ww[e]);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            o[g][v * 8 + 2 * e] = __builtin_fmaf(pp[g], v0, o[g][v * 8 + 2 * e]);
            o[g][v * 8 + 2 * e + 1] = __builtin_fmaf(pp[g], v1, o[g][v * 8 + 2 * e + 1]);
          }
        }
      }
    }
  }
}

// The wavefront's state summed over its four lane rows and its lanes' l: every
// lane of row 0 then holds the wavefront's o for its dims, every lane its l.
template <int D, int G>
__device__ __forceinline__ void wave_state_sum(float (&l)[G], float (&o)[G][AttendShape<D>::EPL]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = wave_sum(l[g]);
#pragma unroll
    for (int e = 0; e < AttendShape<D>::EPL; ++e) {
      o[g][e] += __shfl_xor(o[g][e], 16);
      o[g][e] += __shfl_xor(o[g][e], 32);
    }
  }
}

}  // namespace jssa
