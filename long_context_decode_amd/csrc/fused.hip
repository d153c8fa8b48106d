// jssa_decode in a single launch per layer, for short sequences (paper summary
// page, §3.3 Gather-Free Indexed Attention: one launch per layer resolves every
// KV head's own index set; README page, "Paper-to-code map": scoring and top-k
// are one fused op).  One 1024-thread block per (sequence, KV head):
//   1. qbar (fp64, the G heads in order, / G) and qhat = M qbar (fp64, eight
//      threads per output over interleaved float4 groups, xor-tree sum,
//      rounded once to fp32): the arithmetic of the select prologue, so the
//      scores are bit-identical to the split path's; the new token is projected
//      and stored as jssa_store stores it;
//   2. the sequence's block table goes to LDS, then every position t < N is
//      scored once with the shared scoring function into an LDS key array;
//   3. top-B: the block radix select over the LDS keys and the ordered
//      compaction of the finish kernel (ties at the B-th key: lowest
//      positions), written ascending and -1 padded;
//   4. the G query heads attend over the selected rows read in place through
//      the LDS block table (gather-free).  Lane (row, c) of a wavefront takes
//      position 4c + row of the wavefront's run and, as in attend_kernel, 8 dims
//      of each 128-dim block of a row; runs are sized so that all 16 wavefronts
//      share the B positions.  The wavefronts' (o, m, l) are merged in LDS into
//      the bf16 output and the natural-log lse.
// It applies to GQA caches whose capacity (max_pages x P) fits the key array,
// r <= 64 and G x d <= 512; longer sequences take the split path (prologue,
// stream, finish, attend, merge), where one block per (sequence, KV head)
// would leave most CUs idle.
#include "common.h"
#include "kernels.h"
#include "radix.h"

namespace jssa {

namespace {

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr float kLn2f = 0.69314718055994530942f;

template <int R, int D, int G>
__global__ __launch_bounds__(kFusedThreads) void decode_fused_kernel(FusedArgs a) {
  constexpr int S = R * 16;
  constexpr int EPL = D / 16;    // elements per lane of a row
  constexpr int NV = EPL / 8;    // 16-byte loads per lane per row
  constexpr int NP = EPL / 2;    // bf16 pairs per lane per row
  constexpr int NF = D / 32;     // float4 groups of a row of M per thread
  constexpr int TPT = 4 / R;     // tokens per thread with loads in flight together (<= 8 pieces)
  constexpr int GRP = 4;         // rows whose loads are in flight together
  constexpr bool VE = NV == 1;   // d = 128: the first group's V rows go out with its K rows
  const int h = blockIdx.x, b = blockIdx.y, tid = (int)threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int row = lane >> 4, c16 = lane & 15;
  const bool bf = a.sfmt == 3;
  const int rp = bf ? 2 * R : R;                 // 16-byte pieces per token

  __shared__ __align__(16) uint32_t pool[kCandCap];   // keys; then the wavefronts' partial outputs
  __shared__ int32_t sel[kFusedMaxB];
  __shared__ int32_t lbt[kCandCap / 16];
  __shared__ __align__(16) uint32_t hist[2 * kHistWords];
  __shared__ uint32_t tmp[64];
  __shared__ double qbar[D];
  __shared__ float qh[S];
  __shared__ float ynew[S];
  __shared__ float wml[kFusedWaves][G][2];

  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  const int K = N < a.B ? N : a.B;
  const int n_pages = (N + a.P - 1) / a.P;
  const int lp = 31 - __builtin_clz(a.P);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  for (int p = tid; p < n_pages; p += kFusedThreads) lbt[p] = bt[p];

  // ---- 1. qbar, qhat, the new token
  const int64_t qrow0 = (int64_t)b * a.Hq + (int64_t)h * G;
  for (int i = tid; i < D; i += kFusedThreads) {
    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) acc += (double)bf16_to_f32(a.q[(qrow0 + g) * D + i]);
    qbar[i] = acc / (double)G;
  }
  const float* Mh = a.M + (int64_t)h * a.r * D;
  const int mo = tid >> 3, mpart = tid & 7;
  const int new_slot = a.k_new ? a.slot_new[b] : -1;
  if (new_slot >= 0) {
    const uint16_t* krow = a.k_new + ((int64_t)b * a.Hkv + h) * D;
    float pv = 0.0f;
    if (mo < a.r) pv = project_part(Mh + (int64_t)mo * D, krow, D, mpart);
    pv = proj_combine(pv);
    if (mo < a.r && mpart == 0) ynew[mo] = pv;
  }
  __syncthreads();
  {
    double v = 0.0;
    if (mo < a.r) {
      const float* m = Mh + (int64_t)mo * D + mpart * 4;
      const double* qb = qbar + mpart * 4;
#pragma unroll
      for (int k = 0; k < NF; ++k) {
        const float4 mv = *reinterpret_cast<const float4*>(m + k * 32);
        const double* qq = qb + k * 32;
        v = __builtin_fma((double)mv.x, qq[0], v);
        v = __builtin_fma((double)mv.y, qq[1], v);
        v = __builtin_fma((double)mv.z, qq[2], v);
        v = __builtin_fma((double)mv.w, qq[3], v);
      }
    }
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if (mo < S && mpart == 0) qh[mo] = (float)v;
  }
  if (new_slot >= 0) {
    const int page = new_slot / a.P, sip = new_slot % a.P;
    if (bf) {                                  // BF16 keys: y rounded, no scale
      if (tid < S)
        *reinterpret_cast<uint16_t*>(a.kp + kp_offset(page, h, sip, 2 * tid, a.Hkv, 2 * S, a.P)) =
            f32_to_bf16(ynew[tid]);
    } else if (tid < 64) {
      float am = 0.0f;
      for (int o = tid; o < S; o += 64) am = fmaxf(am, fabsf(ynew[o]));
      am = wave_max(am);
      uint32_t stored;
      const float div = quant_divisor(am, a.sfmt, &stored);
      for (int o = tid; o < S; o += 64) {
        const uint32_t code = (div > 0.0f) ? f32_to_fp8(ynew[o] / div) : 0u;
        a.kp[kp_offset(page, h, sip, o, a.Hkv, S, a.P)] = (uint8_t)code;
      }
      if (tid == 0) store_scale(a.kp_scale, ((int64_t)page * a.Hkv + h) * a.P + sip, a.sfmt, stored);
    }
  }
  __syncthreads();                             // qh, lbt and the stored token are visible to the block

  // ---- 2. every position's key
  for (int t0 = 0; t0 < N; t0 += TPT * kFusedThreads) {
    asm volatile("" ::: "memory");             // qh is re-read from LDS each round
    uint4 pc[TPT][2 * R];
    float sc[TPT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int t = t0 + j * kFusedThreads + tid;
      const int tc = t < N ? t : 0;            // clamped, unconditional loads
      const int64_t phys = lbt[tc >> lp];
      const int slot = tc & (a.P - 1);
      const uint8_t* base = a.kp + (phys * a.Hkv + h) * ((int64_t)rp * 16 * a.P) + slot * 16;
#pragma unroll
      for (int k = 0; k < 2 * R; ++k)
        if (k < rp) pc[j][k] = *reinterpret_cast<const uint4*>(base + (int64_t)k * a.P * 16);
      sc[j] = load_scale(a.kp_scale, (phys * a.Hkv + h) * a.P + slot, a.sfmt);
    }
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int t = t0 + j * kFusedThreads + tid;
      if (t < N) {
        const float s = bf ? score_pieces_bf16<2 * R>(pc[j], qh)
                           : score_pieces<R>(reinterpret_cast<const uint4(&)[R]>(pc[j]), qh);
        pool[t] = score_key(s * sc[j]);
      }
    }
  }
  __syncthreads();

  // ---- 3. top-B, ascending, -1 padded
  int32_t* out_idx = a.indices + ((int64_t)b * a.Hkv + h) * a.B;
  for (int i = K + tid; i < a.B; i += kFusedThreads) out_idx[i] = -1;
  if (N <= a.B) {
    for (int i = tid; i < N; i += kFusedThreads) {
      sel[i] = i;
      out_idx[i] = i;
    }
  } else {
    uint32_t kth, need;
    block_radix_select<kFusedThreads>(pool, N, (uint32_t)K, hist, tmp, &kth, &need);
    // ordered compaction: thread owns a contiguous run of positions
    const int per = (N + kFusedThreads - 1) / kFusedThreads;
    const int i0 = tid * per, i1 = min(i0 + per, N);
    uint32_t gt = 0, eq = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = pool[i];
      gt += key > kth;
      eq += key == kth;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kFusedThreads>(gt | (eq << 16), tmp, &tot);
    uint32_t gb = ex & 0xffffu, eb = ex >> 16;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = pool[i];
      int dst = -1;
      if (key > kth) {
        dst = (int)(gb + (eb < need ? eb : need));
        ++gb;
      } else if (key == kth) {
        if (eb < need) dst = (int)(gb + eb);
        ++eb;
      }
      if (dst >= 0) {
        sel[dst] = i;
        out_idx[dst] = i;
      }
    }
  }
  __syncthreads();                             // sel complete; the keys are no longer read

  // ---- 4. attention of the G heads over sel[0..K)
  uint32_t qp[G][NP];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint16_t* q = a.q + (qrow0 + g) * D + c16 * 8;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint4 u = *reinterpret_cast<const uint4*>(q + v * 128);
      qp[g][4 * v] = u.x;
      qp[g][4 * v + 1] = u.y;
      qp[g][4 * v + 2] = u.z;
      qp[g][4 * v + 3] = u.w;
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
  const int64_t row_stride = (int64_t)a.Hkv * D;
  const uint16_t* kbase = a.k_cache + (int64_t)h * D + c16 * 8;
  const uint16_t* vbase = a.v_cache + (int64_t)h * D + c16 * 8;
  // run length: the K positions spread over the 16 wavefronts, a multiple of 4
  // (one position per lane row and iteration), at most 64
  int run = (K + kFusedWaves - 1) / kFusedWaves;
  run = (run + 3) & ~3;
  if (run > 64) run = 64;
  const int iters = run >> 2;
  for (int base = w * run; base < K; base += kFusedWaves * run) {
    const int pi = 4 * c16 + row;              // this lane's position within the run
    const int ii = base + pi;
    int ri = -1;
    if (pi < run && ii < K) {
      const int t = sel[ii];
      ri = lbt[t >> lp] * a.P + (t & (a.P - 1));
    }
    // logits: iteration u, lane row r -> position 4u + r, held by lane 16r + u
    float xs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) xs[g] = -INFINITY;
    uint4 v0r[GRP][NV];                        // the first group's V rows (d = 128: requested with its K rows)
#pragma unroll
    for (int u0 = 0; u0 < 16; u0 += GRP) {   // compile-time lane indices for the row broadcasts
      if (u0 >= iters) break;                  // uniform
      uint4 kr[GRP][NV];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int rr = row_bcast(ri, u0 + u);
        const int64_t ro = (int64_t)(rr < 0 ? 0 : rr) * row_stride;
#pragma unroll
        for (int v = 0; v < NV; ++v) kr[u][v] = *reinterpret_cast<const uint4*>(kbase + ro + v * 128);
      }
      if (VE && u0 == 0) {
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
          const int rr = row_bcast(ri, u);
          const int64_t ro = (int64_t)(rr < 0 ? 0 : rr) * row_stride;
#pragma unroll
          for (int v = 0; v < NV; ++v) v0r[u][v] = *reinterpret_cast<const uint4*>(vbase + ro + v * 128);
        }
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
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
          const float x = row16_sum(acc) * a.sm_log2;
          if (c16 == u0 + u) xs[g] = x;
        }
      }
    }
    if (ri < 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) xs[g] = -INFINITY;
    }
    float p[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(m[g], wave_max(xs[g]));
      if (mn > m[g]) {                         // uniform over the wavefront
        const float al = __builtin_amdgcn_exp2f(m[g] - mn);
        l[g] *= al;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] *= al;
        m[g] = mn;
      }
      p[g] = (m[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(xs[g] - m[g]);
      l[g] += p[g];
    }
#pragma unroll
    for (int u0 = 0; u0 < 16; u0 += GRP) {
      if (u0 >= iters) break;
      uint4 vr[GRP][NV];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int rr = row_bcast(ri, u0 + u);
        const int64_t ro = (int64_t)(rr < 0 ? 0 : rr) * row_stride;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          vr[u][v] = (VE && u0 == 0) ? v0r[u][v] : *reinterpret_cast<const uint4*>(vbase + ro + v * 128);
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        float pp[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pp[g] = row_bcast_f(p[g], u0 + u);
        // a missing position's row is read from slot 0 with weight 0, its
        // values zeroed so that whatever slot 0 holds adds nothing
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

  // the wavefront's state: rows summed, then (o, m, l) to LDS (the key array
  // is free: every thread passed the barrier after the compaction)
  float* wo = reinterpret_cast<float*>(pool);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = wave_sum(l[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      o[g][e] += __shfl_xor(o[g][e], 16);
      o[g][e] += __shfl_xor(o[g][e], 32);
    }
    if (row == 0) {
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(&wo[(w * G + g) * D + (e >> 3) * 128 + c16 * 8 + (e & 7)]) =
            make_float4(o[g][e], o[g][e + 1], o[g][e + 2], o[g][e + 3]);
    }
    if (lane == 0) {
      wml[w][g][0] = m[g];
      wml[w][g][1] = l[g];
    }
  }
  __syncthreads();
  // merge: thread (g, dim) over the 16 wavefronts
  if (tid < G * D) {
    const int g = tid / D, dim = tid % D;
    float mm = -INFINITY;
#pragma unroll
    for (int v = 0; v < kFusedWaves; ++v)
      if (wml[v][g][1] > 0.0f) mm = fmaxf(mm, wml[v][g][0]);
    const float ms = (mm == -INFINITY) ? 0.0f : mm;
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int v = 0; v < kFusedWaves; ++v) {
      const float lw = wml[v][g][1];
      if (lw > 0.0f) {
        const float f = __builtin_amdgcn_exp2f(wml[v][g][0] - ms);
        L = __builtin_fmaf(lw, f, L);
        acc = __builtin_fmaf(wo[(v * G + g) * D + dim], f, acc);
      }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    a.out[(qrow0 + g) * D + dim] = f32_to_bf16(acc * inv);
    if (dim == 0 && a.lse_out) a.lse_out[qrow0 + g] = L > 0.0f ? (mm + log2f(L)) * kLn2f : -INFINITY;
  }
}

template <int R, int D>
hipError_t launch_fused_rd(const FusedArgs& a, hipStream_t s) {
  const dim3 grid(a.Hkv, a.batch);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((decode_fused_kernel<R, D, 1>), grid, dim3(kFusedThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_fused_kernel<R, D, 2>), grid, dim3(kFusedThreads), 0, s, a); break;
    case 4:
      if constexpr (D == 128) {
        hipLaunchKernelGGL((decode_fused_kernel<R, D, 4>), grid, dim3(kFusedThreads), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int R>
hipError_t launch_fused_r(const FusedArgs& a, hipStream_t s) {
  return a.d == 128 ? launch_fused_rd<R, 128>(a, s) : a.d == 256 ? launch_fused_rd<R, 256>(a, s) : hipErrorInvalidValue;
}

}  // namespace

bool fused_applies(int mla, int d, int G, int r, int64_t capacity, int B) {
  if (mla || r > 64 || (d != 128 && d != 256) || capacity > kCandCap || B > kFusedMaxB) return false;
  return d == 128 ? (G == 1 || G == 2 || G == 4) : (G == 1 || G == 2);
}

hipError_t launch_fused(const FusedArgs& a, hipStream_t s) {
  switch (a.S / 16) {
    case 1: return launch_fused_r<1>(a, s);
    case 2: return launch_fused_r<2>(a, s);
    case 3: return launch_fused_r<3>(a, s);
    case 4: return launch_fused_r<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jssa
