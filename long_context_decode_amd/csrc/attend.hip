// jssa_attend / jssa_full_decode: split-K flash-decode over a per-KV-head
// position list (paper summary page, §3.3 Gather-Free Indexed Attention:
// attention reads the selected tokens directly from the original paged KV
// cache, one launch per layer resolves each KV head's own index set, and every
// query head uses the set of its KV head) or over a dense / sliding-window
// range (README page §3: the Full-KV baseline; §4 notes: sliding-window layers
// keep dense attention).
//
// Block = (split, KV head, sequence), 4 wavefronts; a wavefront takes 64
// positions at a time, lane i resolving position i to its K/V row through the
// block table, and runs the batch of attend_core.h (K rows, one softmax update,
// V rows; each loaded row serves all G query heads of the KV head).  Each
// wavefront writes its own partial (o, m, l), and merge_kernel combines them.
// DENSE instantiates the full-KV / sliding-window baseline (positions [lo, N)
// instead of an index list).
#include <mutex>

#include "attend_core.h"
#include "common.h"
#include "kernels.h"

namespace jssa {

// Split-K partials of jssa_attend_noalloc (for callers that cannot allocate):
// each GPU the library runs on holds its own copy until the process ends.  In
// host code this name is only a stand-in for the symbol; the device address
// comes from hipGetSymbolAddress (attend_scratch).
static __device__ __align__(256) unsigned char scratch[kAttendScratchBytes];

hipError_t attend_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device dev current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

constexpr int kAttendThreads = 256;
constexpr float kLn2 = 0.69314718055994530942f;

}  // namespace

// Combine the splits of every (sequence, query head): o = sum_s 2^(m_s - m*) o_s /
// sum_s 2^(m_s - m*) l_s, lse = ln 2 * (m* + log2 sum_s 2^(m_s - m*) l_s).
// One block per (query head, sequence).  Every load goes out first: thread s
// reads split s's (m_s, l_s), and each thread requests its share of the
// partial outputs (for D < 256 the block splits into 256 / D groups that take
// interleaved splits of every dim; for D >= 256 a thread takes D / 256 dims
// of every split), up to 16 splits at once, clamped to the last split that
// exists.  The block max and the weights 2^(m_s - m*) are formed while those
// loads are in flight (two barriers), then the products are summed (groups
// added through LDS with a third barrier).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(AttendArgs a) {
  constexpr int SG = D >= 256 ? 1 : 256 / D;   // thread groups over the splits
  constexpr int DPT = D >= 256 ? D / 256 : 1;  // dims per thread
  constexpr int MB = 16;                       // splits per thread per batch of loads
  __shared__ float wsplit[256];
  __shared__ float wred[2][4];
  __shared__ float gpart[SG > 1 ? (SG - 1) * D : 1];
  const int j = blockIdx.x, b = blockIdx.y, tid = (int)threadIdx.x, lane = lane_id(), w = tid >> 6;
  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  int n_tok;
  if (a.indices) n_tok = N < a.B ? N : a.B;
  else n_tok = (a.window > 0 && N > a.window) ? a.window : N;
  // partials of the splits that hold positions (a.parts per split: one per
  // wavefront for the GQA kernel, one per block for the MLA kernels)
  const int ns = min(a.splits, (n_tok + a.split_len - 1) / a.split_len) * a.parts;
  const int64_t pj0 = ((int64_t)b * a.Hq + j) * ((int64_t)a.splits * a.parts);
  uint16_t* orow = a.out + ((int64_t)b * a.Hq + j) * D;
  if (ns <= 0) {                               // no positions: zeros
    for (int d = tid; d < D; d += 256) orow[d] = 0;
    if (tid == 0 && a.lse_out) a.lse_out[(int64_t)b * a.Hq + j] = -INFINITY;
    return;
  }
  const int g = SG > 1 ? tid / D : 0;
  const int d0 = SG > 1 ? tid % D : tid;
  const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (pj0 + (tid < ns ? tid : ns - 1)) * 2);
  float pv[MB][DPT];
  auto fetch = [&](int b0) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int sp = g + (b0 + i) * SG;
      const float* src = a.part_o + (pj0 + (sp < ns ? sp : ns - 1)) * D + d0;
#pragma unroll
      for (int k = 0; k < DPT; ++k) pv[i][k] = src[k * 256];
    }
  };
  fetch(0);

  const float ms = (tid < ns && ml.y > 0.0f) ? ml.x : -INFINITY;
  const float ls = tid < ns ? ml.y : 0.0f;
  const float wm = wave_max(ms);
  if (lane == 0) wred[0][w] = wm;
  __syncthreads();
  const float mm = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
  const float msafe = (mm == -INFINITY) ? 0.0f : mm;
  const float f = (tid < ns && ls > 0.0f) ? __builtin_amdgcn_exp2f(ms - msafe) : 0.0f;
  wsplit[tid] = f;
  const float lw = wave_sum(ls * f);
  if (lane == 0) wred[1][w] = lw;
  __syncthreads();
  const float L = (wred[1][0] + wred[1][1]) + (wred[1][2] + wred[1][3]);
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;

  float acc[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) acc[k] = 0.0f;
  const int mine = (ns - g + SG - 1) / SG;     // splits g, g + SG, ... below ns
  for (int b0 = 0; b0 < mine; b0 += MB) {
    if (b0 > 0) fetch(b0);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int sp = g + (b0 + i) * SG;
      const float wt = sp < ns ? wsplit[sp] : 0.0f;
#pragma unroll
      for (int k = 0; k < DPT; ++k) acc[k] = __builtin_fmaf(pv[i][k], wt, acc[k]);
    }
  }
  if (SG > 1) {
    if (g > 0) gpart[(g - 1) * D + d0] = acc[0];
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int q = 1; q < SG; ++q) acc[0] += gpart[(q - 1) * D + d0];
      orow[d0] = f32_to_bf16(acc[0] * inv);
    }
  } else {
#pragma unroll
    for (int k = 0; k < DPT; ++k) orow[d0 + k * 256] = f32_to_bf16(acc[k] * inv);
  }
  if (tid == 0 && a.lse_out) a.lse_out[(int64_t)b * a.Hq + j] = L > 0.0f ? (mm + log2f(L)) * kLn2 : -INFINITY;
}

// Lane (row, c16) of a wavefront holds dims 128 v + 8 c16 ... 128 v + 8 c16 + 7
// (v < D / 128) of the query, the K and V rows and the output, so that each
// 16-byte load instruction covers 256 contiguous bytes of a row.
template <int D, int G, bool DENSE>
__global__ __launch_bounds__(kAttendThreads) void attend_kernel(AttendArgs a) {
  constexpr int EPL = AttendShape<D>::EPL, NP = AttendShape<D>::NP;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = (int)threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int row = lane >> 4, c16 = lane & 15;

  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  int lo = 0, n_tok;
  if (!DENSE) {
    n_tok = N < a.B ? N : a.B;
  } else {
    lo = (a.window > 0 && N > a.window) ? N - a.window : 0;
    n_tok = N - lo;
  }
  const int i0 = s * a.split_len;
  if (i0 >= n_tok) return;
  const int i1 = min(i0 + a.split_len, n_tok);

  uint32_t qp[G][NP];
  load_query_pairs<D, G>(a.q + ((int64_t)b * a.Hq + (int64_t)h * G) * D, c16, qp);
  float m[G], l[G], o[G][EPL];
  attend_state_init<D, G>(m, l, o);

  const int64_t row_stride = (int64_t)a.Hkv * D;  // elements between consecutive token slots
  const uint16_t* kbase = a.k_cache + (int64_t)h * D + c16 * 8;
  const uint16_t* vbase = a.v_cache + (int64_t)h * D + c16 * 8;
  const int32_t* idx = DENSE ? nullptr : a.indices + ((int64_t)b * a.Hkv + h) * a.B;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  // lane -> slot index (physical page * P + slot) of position ii, or -1 (a
  // listed position outside [0, N) counts as missing)
  auto slot_of = [&](int ii) -> int {
    if (ii >= i1) return -1;
    const int t = DENSE ? lo + ii : idx[ii];
    return (t >= 0 && t < N) ? bt[t / a.P] * a.P + (t % a.P) : -1;
  };
  int ri = slot_of(i0 + w * 64 + lane);
  for (int base = i0 + w * 64; base < i1; base += 256) {
    // the next batch's slots are resolved while this batch is in flight
    const int ri_next = slot_of(base + 256 + lane);
    attend_batch<D, G, DENSE>(kbase, vbase, row_stride, ri, qp, a.sm_log2, c16, m, l, o);
    ri = ri_next;
  }

  // this wavefront's partial (o, m, l) goes out as partial 4 s + w
  wave_state_sum<D, G>(l, o);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t pj = ((int64_t)b * a.Hq + (int64_t)h * G + g) * ((int64_t)a.splits * 4) + s * 4 + w;
    if (row == 0) {
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(&a.part_o[pj * D + (e >> 3) * 128 + c16 * 8 + (e & 7)]) =
            make_float4(o[g][e], o[g][e + 1], o[g][e + 2], o[g][e + 3]);
      if (c16 == 0) {
        a.part_ml[pj * 2] = m[g];
        a.part_ml[pj * 2 + 1] = l[g];
      }
    }
  }
}

namespace {

template <int D, int G>
hipError_t launch_dg(const AttendArgs& a, hipStream_t s) {
  if (a.indices)
    hipLaunchKernelGGL((attend_kernel<D, G, false>), dim3(a.splits, a.Hkv, a.batch), dim3(kAttendThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attend_kernel<D, G, true>), dim3(a.splits, a.Hkv, a.batch), dim3(kAttendThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a, D, s);
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

hipError_t launch_merge(const AttendArgs& a, int dv, hipStream_t s) {
  switch (dv) {
    case 128: hipLaunchKernelGGL(merge_kernel<128>, dim3(a.Hq, a.batch), dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(merge_kernel<256>, dim3(a.Hq, a.batch), dim3(256), 0, s, a); break;
    case 512: hipLaunchKernelGGL(merge_kernel<512>, dim3(a.Hq, a.batch), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, int head_dim, hipStream_t s) {
  switch (head_dim) {
    case 128: return launch_d<128>(a, s);
    case 256: return launch_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jssa
