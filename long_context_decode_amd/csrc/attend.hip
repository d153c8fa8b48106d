// jssa_attend / jssa_full_decode: split-K flash-decode over a per-KV-head
// position list (paper summary page, §3.3 Gather-Free Indexed Attention:
// attention reads the selected tokens directly from the original paged KV
// cache, one launch per layer resolves each KV head's own index set, and every
// query head uses the set of its KV head) or over a dense / sliding-window
// range (README page §3: the Full-KV baseline; §4 notes: sliding-window layers
// keep dense attention).
//
// Block = (split, KV head, sequence), 4 wavefronts.  A wavefront takes 64
// positions at a time: each lane resolves one position to its K/V row offset
// through the block table, then rows of 16 lanes walk the 64 rows, four at a
// time; a lane holds D/16 contiguous elements of K and V (one 16-byte load for
// d = 128).  Each loaded row is used by all G query heads of the KV head.  The
// online softmax runs in base 2 (logits pre-scaled by sm * log2 e); partials
// (unnormalised o, running max, running sum) are merged across the rows of a
// wave with lane shuffles, across waves in LDS, and across splits by
// merge_kernel.
#include "common.h"
#include "kernels.h"

namespace jssa {

namespace {

constexpr int kAttendThreads = 256;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ void online_update(float x, float& m, float& l, float* o, const float* v, int n) {
  const float mn = fmaxf(m, x);
  const float ms = (mn == -INFINITY) ? 0.0f : mn;
  const float alpha = __builtin_amdgcn_exp2f(m - ms);
  const float p = __builtin_amdgcn_exp2f(x - ms);
  l = l * alpha + p;
  for (int e = 0; e < n; ++e) o[e] = o[e] * alpha + p * v[e];
  m = mn;
}

__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float mo, float lo, const float* oo,
                                            int n) {
  const float mn = fmaxf(m, mo);
  const float ms = (mn == -INFINITY) ? 0.0f : mn;
  const float a = __builtin_amdgcn_exp2f(m - ms), b = __builtin_amdgcn_exp2f(mo - ms);
  l = l * a + lo * b;
  for (int e = 0; e < n; ++e) o[e] = o[e] * a + oo[e] * b;
  m = mn;
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(kAttendThreads) void attend_kernel(AttendArgs a) {
  constexpr int EPL = D / 16;  // elements per lane
  constexpr int NV = EPL / 8;  // 16-byte loads per lane per row
  __shared__ float red_o[4][G][D];
  __shared__ float red_ml[4][G][2];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = (int)threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int row = lane >> 4, c16 = lane & 15;

  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  int lo = 0, n_tok;
  if (a.indices) {
    n_tok = N < a.B ? N : a.B;
  } else {
    lo = (a.window > 0 && N > a.window) ? N - a.window : 0;
    n_tok = N - lo;
  }
  const int i0 = s * a.split_len;
  if (i0 >= n_tok) return;
  const int i1 = min(i0 + a.split_len, n_tok);

  float qf[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + (int64_t)h * G + g) * D + c16 * EPL;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint4 u = *reinterpret_cast<const uint4*>(qp + v * 8);
      const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[g][v * 8 + 2 * e] = bf16_lo(ws[e]) * a.sm_log2;
        qf[g][v * 8 + 2 * e + 1] = bf16_hi(ws[e]) * a.sm_log2;
      }
    }
  }
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.0f;
  }

  const int64_t row_stride = (int64_t)a.Hkv * D;   // elements between consecutive slots
  const int32_t* idx = a.indices ? a.indices + ((int64_t)b * a.Hkv + h) * a.B : nullptr;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  for (int base = i0 + w * 64; base < i1; base += 256) {
    // lane -> one position of this batch of 64, resolved to its row offset
    const int ii = base + lane;
    int64_t off = -1;
    if (ii < i1) {
      const int t = idx ? idx[ii] : lo + ii;
      if (t >= 0) off = ((int64_t)bt[t / a.P] * a.P + (t % a.P)) * row_stride + (int64_t)h * D;
    }
    const int cnt = min(64, i1 - base);
    for (int it = 0; it < 16; it += 4) {
      if (it * 4 >= cnt) break;
      uint4 kr[4][NV], vr[4][NV];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int src = (it + u) * 4 + row;
        const int lo32 = __shfl((int)(off & 0xffffffff), src);
        const int hi32 = __shfl((int)(off >> 32), src);
        int64_t ro = ((int64_t)hi32 << 32) | (uint32_t)lo32;
        ok[u] = src < cnt && ro >= 0;
        if (!ok[u]) ro = 0;
        const uint16_t* kp = a.k_cache + ro + c16 * EPL;
        const uint16_t* vp = a.v_cache + ro + c16 * EPL;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          kr[u][v] = *reinterpret_cast<const uint4*>(kp + v * 8);
          vr[u][v] = *reinterpret_cast<const uint4*>(vp + v * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float kf[EPL], vf[EPL];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const uint32_t kw[4] = {kr[u][v].x, kr[u][v].y, kr[u][v].z, kr[u][v].w};
          const uint32_t vw[4] = {vr[u][v].x, vr[u][v].y, vr[u][v].z, vr[u][v].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[v * 8 + 2 * e] = bf16_lo(kw[e]);
            kf[v * 8 + 2 * e + 1] = bf16_hi(kw[e]);
            vf[v * 8 + 2 * e] = bf16_lo(vw[e]);
            vf[v * 8 + 2 * e + 1] = bf16_hi(vw[e]);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float part = 0.0f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) part = __builtin_fmaf(qf[g][e], kf[e], part);
          float x = row16_sum(part);
          if (!ok[u]) x = -INFINITY;
          online_update(x, m[g], l[g], o[g], vf, EPL);
        }
      }
    }
  }

  // merge the four rows of the wavefront (lanes c16, c16+16, c16+32, c16+48)
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      float oo[EPL];
      const float mo = __shfl_xor(m[g], sh), lo2 = __shfl_xor(l[g], sh);
#pragma unroll
      for (int e = 0; e < EPL; ++e) oo[e] = __shfl_xor(o[g][e], sh);
      merge_state(m[g], l[g], o[g], mo, lo2, oo, EPL);
    }
    if (row == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[w][g][c16 * EPL + e] = o[g][e];
      if (c16 == 0) {
        red_ml[w][g][0] = m[g];
        red_ml[w][g][1] = l[g];
      }
    }
  }
  __syncthreads();
  // merge the four wavefronts and write this split's partial
  for (int k = tid; k < G * D; k += kAttendThreads) {
    const int g = k / D, dim = k % D;
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) mm = fmaxf(mm, red_ml[ww][g][0]);
    const float ms = (mm == -INFINITY) ? 0.0f : mm;
    float acc = 0.0f, ll = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = __builtin_amdgcn_exp2f(red_ml[ww][g][0] - ms);
      acc += red_o[ww][g][dim] * f;
      ll += red_ml[ww][g][1] * f;
    }
    const int64_t pj = ((int64_t)b * a.Hq + (int64_t)h * G + g) * a.splits + s;
    a.part_o[pj * D + dim] = acc;
    if (dim == 0) {
      a.part_ml[pj * 2] = mm;
      a.part_ml[pj * 2 + 1] = ll;
    }
  }
}

// Combine the splits of every (sequence, query head): o = sum_s 2^(m_s - m*) o_s /
// sum_s 2^(m_s - m*) l_s, lse = ln 2 * (m* + log2 sum_s 2^(m_s - m*) l_s).
__global__ __launch_bounds__(256) void merge_kernel(AttendArgs a, int D) {
  const int j = blockIdx.x, b = blockIdx.y, tid = (int)threadIdx.x;
  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  int n_tok;
  if (a.indices) n_tok = N < a.B ? N : a.B;
  else n_tok = (a.window > 0 && N > a.window) ? a.window : N;
  const int ns = min(a.splits, (n_tok + a.split_len - 1) / a.split_len);
  const int64_t pj0 = ((int64_t)b * a.Hq + j) * a.splits;
  float mm = -INFINITY;
  for (int s = 0; s < ns; ++s)
    if (a.part_ml[(pj0 + s) * 2 + 1] > 0.0f) mm = fmaxf(mm, a.part_ml[(pj0 + s) * 2]);
  const float ms = (mm == -INFINITY) ? 0.0f : mm;
  float L = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float ls = a.part_ml[(pj0 + s) * 2 + 1];
    if (ls > 0.0f) L += ls * __builtin_amdgcn_exp2f(a.part_ml[(pj0 + s) * 2] - ms);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  for (int dim = tid; dim < D; dim += 256) {
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s) {
      const float ls = a.part_ml[(pj0 + s) * 2 + 1];
      if (ls > 0.0f) acc += a.part_o[(pj0 + s) * D + dim] * __builtin_amdgcn_exp2f(a.part_ml[(pj0 + s) * 2] - ms);
    }
    a.out[((int64_t)b * a.Hq + j) * D + dim] = f32_to_bf16(acc * inv);
  }
  if (tid == 0 && a.lse_out)
    a.lse_out[(int64_t)b * a.Hq + j] = L > 0.0f ? (mm + __log2f(L)) * kLn2 : -INFINITY;
}

namespace {

template <int D, int G>
hipError_t launch_dg(const AttendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attend_kernel<D, G>), dim3(a.splits, a.Hkv, a.batch), dim3(kAttendThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.Hq, a.batch), dim3(256), 0, s, a, D);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttendArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return launch_dg<D, 1>(a, s);
    case 2: return launch_dg<D, 2>(a, s);
    case 4: return launch_dg<D, 4>(a, s);
    case 8: return launch_dg<D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, int head_dim, hipStream_t s) {
  switch (head_dim) {
    case 128: return launch_d<128>(a, s);
    case 256: return launch_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jssa
