// jssa_select: group-mean projected query, FP8 projected-score stream and
// exact per-KV-head top-B (paper summary page, §3.1 Overview steps 1-2 and
// Theoretical Foundation Eq. 1; README page §4: budget B per decode step and
// KV head).
//
// Three launches on one stream:
//  1. prologue  (one block per (sequence, KV head)): qbar = mean of the G query
//     heads, qhat = M qbar (fp64, rounded once to fp32); scores a strided sample of the sequence's
//     pages and picks a threshold key tau that about 4B tokens should clear
//     (tau = "all" when the whole sequence fits the candidate buffer).
//  2. stream    (blocks over (chunk of pages, group of KV heads, sequence)):
//     every lane owns one (KV head, slot) of a page and reads that token's
//     16-byte FP8 pieces (a wavefront reads one contiguous run per piece),
//     computes its score and key into LDS; at the end of the chunk one wave
//     per head compacts the keys >= tau, in position order, into the
//     candidate buffer and records (base, count) for the chunk.
//  3. finish    (one 1024-thread block per (sequence, KV head)): copies the
//     candidates into LDS in chunk order (so they are in position order),
//     radix-selects the B-th largest key, and writes the winners ascending
//     with an ordered prefix-sum compaction (ties at the B-th key: lowest
//     positions).  If the candidates cannot contain the exact top-B (fewer
//     than B cleared tau, or the buffer overflowed) or the caller asked for
//     it, the block instead runs an exact radix select that re-scores every
//     token of the sequence itself (same scoring function, same bits).
#include "common.h"
#include "kernels.h"

namespace jssa {

namespace {

constexpr int kPrologueThreads = 256;
constexpr int kFinishThreads = 1024;
constexpr int kStreamThreads = 256;
constexpr int kMaxCp = 64;             // pages per stream chunk, at most

// ------------------------------------------------------------------ radix select

// Pick the digit d of the current pass so that fewer than k matching keys have
// a larger digit and at least k have a digit >= d.  Run by wave 0 only.
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t k, uint32_t* bcast) {
  const int l = lane_id();
  const uint32_t c0 = hist[4 * l], c1 = hist[4 * l + 1], c2 = hist[4 * l + 2], c3 = hist[4 * l + 3];
  const uint32_t s = c0 + c1 + c2 + c3;
  uint32_t suf = s;  // inclusive suffix sum over lanes >= l
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t v = (uint32_t)__shfl_down((int)suf, o);
    if (l + o < 64) suf += v;
  }
  uint32_t above = suf - s;
  const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    if (above < k && k <= above + cs[j]) {
      bcast[0] = (uint32_t)(4 * l + j);
      bcast[1] = k - above;
    }
    above += cs[j];
  }
}

// k-th largest key (1-based) of keys[0..n) held in LDS, and how many keys equal
// to it belong to the top k.  Skips the leading bits that all keys share.
template <int NT>
__device__ void radix_select_lds(const uint32_t* keys, int n, uint32_t k, uint32_t* hist, uint32_t* tmp,
                                 uint32_t* kth, uint32_t* need) {
  const int tid = (int)threadIdx.x;
  const uint32_t ref = keys[0];
  uint32_t orv = 0;
  for (int i = tid; i < n; i += NT) orv |= keys[i] ^ ref;
  orv = block_or<NT>(orv, tmp);
  if (orv == 0u) {
    *kth = ref;
    *need = k;
    return;
  }
  int hb = 31 - __builtin_clz(orv);
  uint32_t hi_mask = (hb == 31) ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = ref & hi_mask;
  while (true) {
    const int shift = hb >= 7 ? hb - 7 : 0;
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = keys[i];
      if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (tid < 64) find_digit(hist, k, tmp + 32);
    __syncthreads();
    const uint32_t d = tmp[32];
    k = tmp[33];
    hi_mask = ~((1u << shift) - 1u);
    prefix = (prefix & ~(0xffu << shift)) | (d << shift);
    prefix &= hi_mask;
    __syncthreads();
    if (shift == 0) break;
    hb = shift - 1;
  }
  *kth = prefix;
  *need = k;
}

// ------------------------------------------------------------------ token access

template <int R>
__device__ __forceinline__ void load_token(const SelectArgs& a, int64_t phys, int head, int slot, uint4 (&pc)[R],
                                           float& sc) {
  const uint8_t* base = a.kp + (phys * a.Hkv + head) * ((int64_t)R * 16 * a.P) + slot * 16;
#pragma unroll
  for (int j = 0; j < R; ++j) pc[j] = *reinterpret_cast<const uint4*>(base + (int64_t)j * a.P * 16);
  sc = a.kp_scale[(phys * a.Hkv + head) * a.P + slot];
}

template <int R>
__device__ __forceinline__ uint32_t token_key(const SelectArgs& a, int b, int head, int t, const float* qh) {
  const int64_t phys = a.block_table[(int64_t)b * a.max_pages + t / a.P];
  uint4 pc[R];
  float sc;
  load_token<R>(a, phys, head, t % a.P, pc, sc);
  return score_key(score_pieces<R>(pc, qh) * sc);
}

__device__ __forceinline__ int seq_len_of(const SelectArgs& a, int b) {
  const int n = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

}  // namespace

// ================================================================== 1. prologue

template <int R>
__global__ __launch_bounds__(kPrologueThreads) void select_prologue(SelectArgs a) {
  constexpr int S = R * 16;
  const int h = blockIdx.x, b = blockIdx.y, tid = (int)threadIdx.x;
  __shared__ double qbar[kMlaLatent + kMlaRope];
  __shared__ float qh[S];
  __shared__ uint32_t skeys[kSampleMax];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[64];
  const int N = seq_len_of(a, b);
  const int din = a.mla ? kMlaLatent + kMlaRope : a.d;

  // qbar: mean of the G query heads of KV head h.  The projection runs in fp64
  // and is rounded to fp32 once, so qhat carries one rounding.
  for (int i = tid; i < din; i += kPrologueThreads) {
    double s = 0.0;
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + (int64_t)h * a.G) * din + i;
    for (int g = 0; g < a.G; ++g) s += (double)bf16_to_f32(qp[(int64_t)g * din]);
    qbar[i] = s / (double)a.G;
  }
  __syncthreads();
  // qhat = M qbar (MLA: [M qbar[:512] ; qbar[512:]])
  for (int o = tid; o < S; o += kPrologueThreads) {
    double v;
    if (o < a.r) {
      const int dm = a.mla ? kMlaLatent : a.d;
      const float* m = a.M + ((int64_t)(a.mla ? 0 : h) * a.r + o) * dm;
      double acc = 0.0;
      for (int i = 0; i < dm; ++i) acc = __builtin_fma((double)m[i], qbar[i], acc);
      v = acc;
    } else {
      v = qbar[kMlaLatent + (o - a.r)];
    }
    qh[o] = (float)v;
    a.qhat[((int64_t)b * a.Hkv + h) * S + o] = (float)v;
  }
  __syncthreads();

  uint32_t tau;
  if (a.force_exact) {
    tau = 0xffffffffu;                   // stream keeps nothing; finish runs the exact path
  } else if (N <= kCandCap) {
    tau = 0u;                            // every token is a candidate
  } else {
    // strided page sample; tau = the ks-th largest sampled key with
    // ks / sample = target / N, target = min(4B, cap/2) candidates
    const int n_pages = (N + a.P - 1) / a.P;
    int64_t want = (int64_t)32 * N / a.B;
    if (want < 2048) want = 2048;
    if (want > kSampleMax) want = kSampleMax;
    int sp = (int)((want + a.P - 1) / a.P);
    if (sp > kSampleMax / a.P) sp = kSampleMax / a.P;
    if (sp > n_pages) sp = n_pages;
    const int ns = sp * a.P;
    uint32_t valid = 0;
    for (int u = tid; u < ns; u += kPrologueThreads) {
      const int i = u / a.P, slot = u % a.P;
      const int pl = (int)(((int64_t)i * n_pages) / sp);
      const int t = pl * a.P + slot;
      uint32_t key = 0u;
      if (t < N) {
        key = token_key<R>(a, b, h, t, qh);
        ++valid;
      }
      skeys[u] = key;
    }
    uint32_t nvalid;
    (void)block_excl_scan<kPrologueThreads>(valid, tmp, &nvalid);
    const int64_t target = (int64_t)(4 * a.B < kCandCap / 2 ? 4 * a.B : kCandCap / 2);
    int64_t ks = (nvalid * target + N - 1) / N;
    if (ks < 1) ks = 1;
    if (ks > (int64_t)nvalid) ks = nvalid;
    uint32_t kth, need;
    radix_select_lds<kPrologueThreads>(skeys, ns, (uint32_t)ks, hist, tmp, &kth, &need);
    tau = kth;
  }
  if (tid == 0) {
    a.tau[(int64_t)b * a.Hkv + h] = tau;
    a.counter[(int64_t)b * a.Hkv + h] = 0u;
  }
}

// ================================================================== 2. stream

template <int R, int P>
__global__ __launch_bounds__(kStreamThreads) void select_stream(SelectArgs a) {
  constexpr int S = R * 16;
  constexpr int HPW = 64 / P;  // KV heads covered by one wavefront
  __shared__ uint32_t keys[HPW][kMaxCp * P];
  const int c = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int N = seq_len_of(a, b);
  const int n_pages = (N + P - 1) / P;
  const int page0 = c * a.cp;
  if (page0 >= n_pages) return;
  const int pages_here = min(a.cp, n_pages - page0);
  const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
  const int hl = lane / P, slot = lane % P;
  const int head = hg * HPW + hl;
  const bool active = head < a.Hkv;
  const int headc = active ? head : 0;

  float qh[S];
  {
    const float* src = a.qhat + ((int64_t)b * a.Hkv + headc) * S;
#pragma unroll
    for (int i = 0; i < S; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + i);
      qh[i] = v.x;
      qh[i + 1] = v.y;
      qh[i + 2] = v.z;
      qh[i + 3] = v.w;
    }
  }

  // this wave's pages: a contiguous run of the chunk, in order
  const int per = a.cp / 4;
  const int pb = w * per;
  const int pe = min(pb + per, pages_here);
  int phys_l = 0;
  if (lane < per && pb + lane < pages_here)
    phys_l = a.block_table[(int64_t)b * a.max_pages + page0 + pb + lane];
  const int64_t maxN = (int64_t)a.max_pages * P;
  float* sout = a.scores_out ? a.scores_out + ((int64_t)b * a.Hkv + headc) * maxN : nullptr;

  if (pb < pe) {
    uint4 cur[R];
    float csc = 0.0f;
    {
      const int64_t phys = __builtin_amdgcn_readlane(phys_l, 0);
      if (active) load_token<R>(a, phys, head, slot, cur, csc);
    }
    for (int pi = pb; pi < pe; ++pi) {
      uint4 nxt[R];
      float nsc = 0.0f;
      if (pi + 1 < pe) {
        const int64_t phys = __builtin_amdgcn_readlane(phys_l, pi + 1 - pb);
        if (active) load_token<R>(a, phys, head, slot, nxt, nsc);
      }
      const int t = (page0 + pi) * P + slot;
      uint32_t key = 0u;
      if (active && t < N) {
        const float s = score_pieces<R>(cur, qh) * csc;
        key = score_key(s);
        if (sout) sout[t] = s;
      }
      keys[hl][pi * P + slot] = key;
#pragma unroll
      for (int j = 0; j < R; ++j) cur[j] = nxt[j];
      csc = nsc;
    }
  }
  __syncthreads();

  // ordered compaction of keys >= tau, one wavefront per KV head
  const int n = pages_here * P;
  for (int h2 = w; h2 < HPW; h2 += 4) {
    const int head2 = hg * HPW + h2;
    if (head2 >= a.Hkv) break;
    const int64_t bh = (int64_t)b * a.Hkv + head2;
    uint32_t tau = a.tau[bh];
    if (tau == 0u) tau = 1u;                         // key 0 marks "no token"
    uint32_t cnt = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const bool f = i < n && keys[h2][i] >= tau;
      cnt += (uint32_t)__popcll(ballot(f));
    }
    uint32_t base = 0;
    if (lane == 0) {
      base = cnt ? atomicAdd(&a.counter[bh], cnt) : 0u;
      int32_t* tab = a.chunk_tab + (bh * a.max_chunks + c) * 2;
      tab[0] = (int32_t)base;
      tab[1] = (int32_t)cnt;
    }
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
    if (cnt == 0) continue;
    uint32_t run = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const uint32_t key = i < n ? keys[h2][i] : 0u;
      const bool f = i < n && key >= tau;
      const uint64_t m = ballot(f);
      const uint32_t pos = base + run + lanes_below(m);
      if (f && pos < (uint32_t)kCandCap) {
        a.cand_key[bh * kCandCap + pos] = key;
        a.cand_idx[bh * kCandCap + pos] = page0 * P + i;
      }
      run += (uint32_t)__popcll(m);
    }
  }
}

// ================================================================== 3. finish

namespace {

// Exact top-K of one (sequence, KV head) by re-scoring every token: four
// 8-bit radix passes over the keys, then an ordered compaction pass.
template <int R>
__device__ void exact_stream_select(const SelectArgs& a, int b, int h, int N, int K, const float* qh,
                                    uint32_t* hist, uint32_t* tmp, int32_t* out) {
  const int tid = (int)threadIdx.x;
  uint32_t prefix = 0u, hi_mask = 0u, k = (uint32_t)K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kFinishThreads) hist[i] = 0u;
    __syncthreads();
    for (int t0 = 0; t0 < N; t0 += kFinishThreads) {
      const int t = t0 + tid;
      if (t < N) {
        const uint32_t key = token_key<R>(a, b, h, t, qh);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) find_digit(hist, k, tmp + 32);
    __syncthreads();
    prefix |= tmp[32] << shift;
    k = tmp[33];
    hi_mask |= 0xffu << shift;
    __syncthreads();
  }
  const uint32_t kth = prefix, need = k;
  uint32_t gt_run = 0, eq_run = 0;
  for (int t0 = 0; t0 < N; t0 += kFinishThreads) {
    const int t = t0 + tid;
    const uint32_t key = t < N ? token_key<R>(a, b, h, t, qh) : 0u;
    const uint32_t gt = key > kth ? 1u : 0u, eq = (t < N && key == kth) ? 1u : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kFinishThreads>(gt | (eq << 16), tmp, &tot);
    const uint32_t gb = gt_run + (ex & 0xffffu), eb = eq_run + (ex >> 16);
    if (gt) out[gb + (eb < need ? eb : need)] = t;
    else if (eq && eb < need) out[gb + eb] = t;
    gt_run += tot & 0xffffu;
    eq_run += tot >> 16;
  }
}

}  // namespace

template <int R>
__global__ __launch_bounds__(kFinishThreads) void select_finish(SelectArgs a) {
  constexpr int S = R * 16;
  constexpr int E = kCandCap / kFinishThreads;
  const int h = blockIdx.x, b = blockIdx.y, tid = (int)threadIdx.x;
  __shared__ uint32_t lkey[kCandCap];
  __shared__ int32_t lidx[kCandCap];
  __shared__ uint32_t coff[kMaxChunks];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[64];
  __shared__ float qh[S];
  const int64_t bh = (int64_t)b * a.Hkv + h;
  int32_t* out = a.indices + bh * a.B;
  const int N = seq_len_of(a, b);
  const int K = N < a.B ? N : a.B;
  for (int i = K + tid; i < a.B; i += kFinishThreads) out[i] = -1;
  if (K == 0) return;

  const uint32_t total = a.counter[bh];
  const uint32_t tau = a.tau[bh];
  const int n_pages = (N + a.P - 1) / a.P;
  const int n_chunks = (n_pages + a.cp - 1) / a.cp;
  const bool ok = !a.force_exact && total <= (uint32_t)kCandCap && total >= (uint32_t)K &&
                  n_chunks <= kMaxChunks && (tau != 0u || total == (uint32_t)N);
  if (!ok) {
    for (int i = tid; i < S; i += kFinishThreads) qh[i] = a.qhat[bh * S + i];
    __syncthreads();
    exact_stream_select<R>(a, b, h, N, K, qh, hist, tmp, out);
    return;
  }

  // chunk offsets in chunk (= position) order
  const int32_t* tab = a.chunk_tab + bh * a.max_chunks * 2;
  uint32_t carry = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += kFinishThreads) {
    const int c = c0 + tid;
    const uint32_t cnt = c < n_chunks ? (uint32_t)tab[2 * c + 1] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kFinishThreads>(cnt, tmp, &tot);
    if (c < n_chunks) coff[c] = carry + ex;
    carry += tot;
  }
  __syncthreads();
  // copy candidates: one wavefront per chunk
  const int lane = lane_id(), w = tid >> 6;
  for (int c = w; c < n_chunks; c += kFinishThreads / 64) {
    const int base = tab[2 * c], cnt = tab[2 * c + 1];
    const uint32_t dst = coff[c];
    for (int i = lane; i < cnt; i += 64) {
      lkey[dst + i] = a.cand_key[bh * kCandCap + base + i];
      lidx[dst + i] = a.cand_idx[bh * kCandCap + base + i];
    }
  }
  __syncthreads();
  const int n = (int)total;
  if (n <= K) {                                // everything that is there is selected
    for (int i = tid; i < n; i += kFinishThreads) out[i] = lidx[i];
    return;
  }
  uint32_t kth, need;
  radix_select_lds<kFinishThreads>(lkey, n, (uint32_t)K, hist, tmp, &kth, &need);
  // ordered compaction: thread owns a contiguous run of E' positions
  const int per = (n + kFinishThreads - 1) / kFinishThreads;
  const int i0 = tid * per, i1 = min(i0 + per, n);
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = lkey[i];
    gt += key > kth;
    eq += key == kth;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<kFinishThreads>(gt | (eq << 16), tmp, &tot);
  uint32_t gb = ex & 0xffffu, eb = ex >> 16;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = lkey[i];
    if (key > kth) {
      out[gb + (eb < need ? eb : need)] = lidx[i];
      ++gb;
    } else if (key == kth) {
      if (eb < need) out[gb + eb] = lidx[i];
      ++eb;
    }
  }
  (void)E;
}

// ================================================================== launch

namespace {

template <int R, int P>
hipError_t launch_select_rp(const SelectArgs& a, int stages, hipStream_t s) {
  constexpr int HPW = 64 / P;
  hipError_t e = hipSuccess;
  if (stages & 1) {
    hipLaunchKernelGGL(select_prologue<R>, dim3(a.Hkv, a.batch), dim3(kPrologueThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 2) {
    const int hg = (a.Hkv + HPW - 1) / HPW;
    hipLaunchKernelGGL((select_stream<R, P>), dim3(a.max_chunks, hg, a.batch), dim3(kStreamThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 4) {
    hipLaunchKernelGGL(select_finish<R>, dim3(a.Hkv, a.batch), dim3(kFinishThreads), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

template <int R>
hipError_t launch_select_r(const SelectArgs& a, int stages, hipStream_t s) {
  switch (a.P) {
    case 16: return launch_select_rp<R, 16>(a, stages, s);
    case 32: return launch_select_rp<R, 32>(a, stages, s);
    case 64: return launch_select_rp<R, 64>(a, stages, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, int stages, hipStream_t s) {
  switch (a.S / 16) {
    case 1: return launch_select_r<1>(a, stages, s);
    case 2: return launch_select_r<2>(a, stages, s);
    case 3: return launch_select_r<3>(a, stages, s);
    case 4: return launch_select_r<4>(a, stages, s);
    case 5: return launch_select_r<5>(a, stages, s);
    case 6: return launch_select_r<6>(a, stages, s);
    case 7: return launch_select_r<7>(a, stages, s);
    case 8: return launch_select_r<8>(a, stages, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jssa
