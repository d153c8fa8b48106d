// jssa_select: group-mean projected query, FP8 projected-score stream and
// exact per-KV-head top-B (paper summary page, §3.1 Overview steps 1-2 and
// Theoretical Foundation Eq. 1; README page §4: budget B per decode step and
// KV head).
//
// Three launches on one stream:
//  1. prologue  (one block per (sequence, KV head)): qbar = mean of the G query
//     heads, qhat = M qbar (fp64, rounded once to fp32); scores a strided
//     sample of the sequence's pages and picks a threshold key tau that about
//     2B tokens should clear (tau = "all" when the whole sequence fits the
//     candidate buffer).  In jssa_decode it also stores the new token.
//  2. stream    (a wavefront scores one chunk of consecutive pages for one
//     KV head; the four wavefronts of a block take four KV heads of the same
//     pages, or, with fewer KV heads, consecutive chunks): lane = (page of the
//     round, slot), and every lane reads its token's 16-byte pieces (FP8
//     codes, or BF16 keys: twice the pieces) for all rounds at once with
//     streaming (non-temporal) loads, since each byte is read once per step;
//     the head's projected query sits in scalar registers.  The keys >= tau
//     are compacted in position order from the ballot masks into the
//     wavefront's LDS area, and its (chunk, KV head) region of the candidate
//     buffer goes out as whole 128-byte lines: a header entry holding the
//     count, then the candidates.  No block barrier.
//  3. finish    (one 1024-thread block per (sequence, KV head)): gathers the
//     candidates into LDS in chunk order (so they are in position order),
//     radix-selects the B-th largest key, and writes the winners ascending
//     with an ordered prefix-sum compaction (ties at the B-th key: lowest
//     positions).  If the candidates cannot contain the exact top-B (fewer
//     than B cleared tau, or the buffer overflowed) or the caller asked for
//     it, the block instead runs an exact radix select that re-scores every
//     token of the sequence itself (same scoring function, same bits).
#include "common.h"
#include "kernels.h"
#include "radix.h"

namespace jssa {

namespace {

constexpr int kPrologueThreads = 1024;
constexpr int kFinishThreads = 1024;
constexpr int kStreamThreads = 64 * kStreamWaves;

// ------------------------------------------------------------------ token access

// the token's R 16-byte pieces (R = TokenPieces) and its scale (1 without one)
template <int R>
__device__ __forceinline__ void load_token(const SelectArgs& a, int64_t phys, int head, int slot, uint4 (&pc)[R],
                                           float& sc) {
  const uint8_t* base = a.kp + (phys * a.Hkv + head) * ((int64_t)R * 16 * a.P) + slot * 16;
#pragma unroll
  for (int j = 0; j < R; ++j) pc[j] = *reinterpret_cast<const uint4*>(base + (int64_t)j * a.P * 16);
  sc = load_scale(a.kp_scale, (phys * a.Hkv + head) * a.P + slot, a.sfmt);
}

// load_token for the stream kernel: the scale format fixed at compile time,
// and streaming loads (each byte of the scoring cache is read once per step)
template <int R, int SF>
__device__ __forceinline__ void load_token_sf(const SelectArgs& a, int64_t phys, int head, int slot, uint4 (&pc)[R],
                                              float& sc) {
  const uint8_t* base = a.kp + (phys * a.Hkv + head) * ((int64_t)R * 16 * a.P) + slot * 16;
#pragma unroll
  for (int j = 0; j < R; ++j) pc[j] = load_stream_u4(base + (int64_t)j * a.P * 16);
  sc = load_scale_stream(a.kp_scale, (phys * a.Hkv + head) * a.P + slot, SF);
}

template <int R, bool BF>
__device__ __forceinline__ uint32_t token_key(const SelectArgs& a, int b, int head, int t, const float* qh) {
  constexpr int RP = TokenPieces<R, BF>::value;
  const int64_t phys = a.block_table[(int64_t)b * a.max_pages + t / a.P];
  uint4 pc[RP];
  float sc;
  load_token<RP>(a, phys, head, t % a.P, pc, sc);
  return score_key(score_token<R, BF>(pc, qh) * sc);
}

__device__ __forceinline__ int seq_len_of(const SelectArgs& a, int b) {
  const int n = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

}  // namespace

// ================================================================== 1. prologue

template <int R, bool BF>
__global__ __launch_bounds__(kPrologueThreads) void select_prologue(SelectArgs a) {
  constexpr int S = R * 16;
  constexpr int RP = TokenPieces<R, BF>::value;
  constexpr int TPT = RP >= 8 ? 1 : 8 / RP;    // sampled tokens per thread with loads in flight together
  const int h = blockIdx.x, b = blockIdx.y, tid = (int)threadIdx.x;
  __shared__ double qbar[kMlaLatent + kMlaRope];
  __shared__ double qpart[8 * (kMlaLatent + kMlaRope)];   // head-group partials of qbar (G <= 128)
  __shared__ float qh[S];
  __shared__ float ynew[S];
  __shared__ uint32_t skeys[kSampleMax];
  __shared__ int32_t sph[kSampleMax];                      // physical page of each sampled token, -1: none
  __shared__ __align__(16) uint32_t hist[2 * kHistWords];
  __shared__ uint32_t tmp[64];
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const int N = seq_len_of(a, b);
  const int din = a.mla ? kMlaLatent + kMlaRope : a.d;
  const int dm = a.mla ? kMlaLatent : a.d;
  const float* Mh = a.M + (int64_t)(a.mla ? 0 : h) * a.r * dm;

  // qbar loads go out first, beside the sequence-length load: heads in groups
  // of up to 16, a thread takes one group's heads over 8 dims (groups x
  // chunks <= 8 x 72 units, so one unit per thread)
  const int hg = a.G < 16 ? a.G : 16;
  const int groups = a.G / hg;
  const int chunks = din >> 3;
  const bool qact = tid < groups * chunks;
  const int qgrp = tid / chunks, qc = tid % chunks;
  uint4 qv[16];
  if (qact) {
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + (int64_t)h * a.G + qgrp * hg) * din + qc * 8;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < hg) qv[j] = *reinterpret_cast<const uint4*>(qp + (int64_t)j * din);
  }

  // this thread's rows of M for qhat (8 threads per output, float4 groups
  // part, part + 8, ...): loaded now, beside the query, when they are at most
  // 4 groups (d = 128), so that qhat does not wait for them later
  const int mo = tid >> 3, mpart = tid & 7;
  const int nf = dm / 32;                      // float4 groups per thread: 4, 8 or 16
  const bool mpre = nf <= 4 && mo < a.r;
  float4 mpv[4];
  {
    // unconditional loads from a clamped row (dims < 128 <= dm), so that no
    // branch join waits for them
    const float* m = Mh + (int64_t)(mo < a.r ? mo : 0) * dm + mpart * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) mpv[k] = *reinterpret_cast<const float4*>(m + k * 32);
  }

  // sample plan: a strided set of whole pages; tau will be the ks-th largest
  // sampled key with ks / sample = target / N, target = min(2B, cap/2)
  const bool sampled = !a.force_exact && N > kCandCap;
  int sp = 0, n_pages = 0;
  if (sampled) {
    n_pages = (N + a.P - 1) / a.P;
    // about 32 samples per expected selection (so that ks, the sampled keys
    // above tau, is about 64: the candidate count then varies by about 1/8),
    // at least 1024 (where that floor applies, ks = 2B 1024 / N >= 64), and
    // no more than 128 KB of scoring cache (one CU reads the whole sample, in
    // one round of loads up to 128-byte tokens)
    constexpr int kByteCap = (128 * 1024) / (RP * 16);
    int64_t want = (int64_t)32 * N / a.B;
    if (want > kByteCap) want = kByteCap;
    if (want < 1024) want = 1024;
    if (want > kSampleMax) want = kSampleMax;
    sp = (int)((want + a.P - 1) / a.P);
    if (sp > kSampleMax / a.P) sp = kSampleMax / a.P;
    if (sp > n_pages) sp = n_pages;
  }
  const int ns = sp * a.P;
  // sample loads go out in two steps around the query work: the block-table
  // entries of every round first (with the query loads), then each round's
  // scoring-cache rows (round 0 as soon as the query is summed).  Round r covers the
  // sample indices u = (r TPT + j) threads + tid, j < TPT.  P (16, 32 or 64)
  // divides the thread count, so every index of this thread has slot tid mod P.
  const int lp = 31 - __builtin_clz(a.P);
  const int sslot = tid & (a.P - 1);
  uint4 pc[TPT][RP];
  float sc[TPT];
  constexpr int KS = kSampleMax / kPrologueThreads;
  int ph[KS];
  if (sampled) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int u = k * kPrologueThreads + tid;
      // sample page i -> logical page floor(i n_pages / sp); exact in fp64
      // (i n_pages < 2^53, and a quotient that is not an integer lies at
      // least 1/sp below the next one)
      const int pl = (int)(((double)(u >> lp) * (double)n_pages) / (double)sp);
      const bool ok = u < ns && pl * a.P + sslot < N;
      // unconditional (clamped) loads: no branch join waits for them
      const int e = a.block_table[(int64_t)b * a.max_pages + (ok ? pl : 0)];
      ph[k] = ok ? e : -1;
    }
  }
  auto issue_rows = [&](int r) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int u = (r * TPT + j) * kPrologueThreads + tid;
      const int pg = u < ns ? sph[u] : -1;
      load_token<RP>(a, pg >= 0 ? pg : 0, h, sslot, pc[j], sc[j]);
    }
  };

  // qbar: mean of the G query heads of KV head h (fp64): per dim the group's
  // heads in order, then the group partials in group order
  if (qact) {
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < hg) {
        acc[0] += (double)bf16_lo(qv[j].x);
        acc[1] += (double)bf16_hi(qv[j].x);
        acc[2] += (double)bf16_lo(qv[j].y);
        acc[3] += (double)bf16_hi(qv[j].y);
        acc[4] += (double)bf16_lo(qv[j].z);
        acc[5] += (double)bf16_hi(qv[j].z);
        acc[6] += (double)bf16_lo(qv[j].w);
        acc[7] += (double)bf16_hi(qv[j].w);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) qpart[qgrp * din + qc * 8 + k] = acc[k];
  }
  // the query registers are free now: the sample pages go to LDS and round
  // 0's rows go out (each thread reads back only its own sph entries)
  if (sampled) {
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (k * kPrologueThreads + tid < ns) sph[k * kPrologueThreads + tid] = ph[k];
    issue_rows(0);
  }
  __syncthreads();
  for (int i = tid; i < din; i += kPrologueThreads) {
    double acc = 0.0;
    for (int g = 0; g < groups; ++g) acc += qpart[g * din + i];
    qbar[i] = acc / (double)a.G;
  }
  // the new token of this sequence (jssa_decode): projected exactly as
  // jssa_store does (eight threads per output, project_part / proj_combine)
  const int new_slot = a.k_new ? a.slot_new[b] : -1;
  if (new_slot >= 0) {
    const uint16_t* row = a.mla ? a.k_new + (int64_t)b * din : a.k_new + ((int64_t)b * a.Hkv + h) * a.d;
    const int o = tid >> 3, part = tid & 7;
    float v = 0.0f;
    if (o < a.r) v = project_part(Mh + (int64_t)o * dm, row, dm, part);
    v = proj_combine(v);
    if (o < a.r && part == 0) ynew[o] = v;
    if (a.mla && tid < kMlaRope) ynew[a.r + tid] = bf16_to_f32(row[kMlaLatent + tid]);
  }
  __syncthreads();
  // qhat = M qbar (MLA: [M qbar[:512] ; qbar[512:]]) in fp64, rounded once to
  // fp32: 8 threads per output, thread p taking the float4 groups p, p + 8,
  // ... (the 8 threads of an output read 128 contiguous bytes per step), partial
  // sums added in a fixed xor order
  {
    const int o = mo, part = mpart;
    double v = 0.0;
    if (mpre) {
      const double* qb = qbar + part * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < nf) {
          const double* qq = qb + k * 32;
          v = __builtin_fma((double)mpv[k].x, qq[0], v);
          v = __builtin_fma((double)mpv[k].y, qq[1], v);
          v = __builtin_fma((double)mpv[k].z, qq[2], v);
          v = __builtin_fma((double)mpv[k].w, qq[3], v);
        }
      }
    } else if (o < a.r) {
      const float* m = Mh + (int64_t)o * dm + part * 4;
      const double* qb = qbar + part * 4;
      // all 16 loads (d = 512) in flight together, 8 when the sample rows in
      // flight beside them are BF16 keys of more than 128 bytes
      constexpr int MB = RP > 8 ? 8 : 16;
      for (int k0 = 0; k0 < nf; k0 += MB) {
        float4 mv[MB];
#pragma unroll
        for (int k = 0; k < MB; ++k)
          if (k0 + k < nf) mv[k] = *reinterpret_cast<const float4*>(m + (k0 + k) * 32);
#pragma unroll
        for (int k = 0; k < MB; ++k) {
          if (k0 + k < nf) {
            const double* qq = qb + (k0 + k) * 32;
            v = __builtin_fma((double)mv[k].x, qq[0], v);
            v = __builtin_fma((double)mv[k].y, qq[1], v);
            v = __builtin_fma((double)mv[k].z, qq[2], v);
            v = __builtin_fma((double)mv[k].w, qq[3], v);
          }
        }
      }
    }
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if (o < S && part == 0) {
      if (o >= a.r) v = qbar[kMlaLatent + (o - a.r)];
      qh[o] = (float)v;
      a.qhat[bh * S + o] = (float)v;
    }
  }
  if (BF && new_slot >= 0 && tid < S) {        // BF16 keys: y rounded, no scale
    const int page = new_slot / a.P, sip = new_slot % a.P;
    *reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a.kp) + kp_offset(page, h, sip, 2 * tid, a.Hkv, 2 * S, a.P)) =
        f32_to_bf16(ynew[tid]);
  }
  if (!BF && new_slot >= 0 && tid < 64) {
    float am = 0.0f;
    for (int o = tid; o < S; o += 64) am = fmaxf(am, fabsf(ynew[o]));
    am = wave_max(am);
    uint32_t stored;
    const float div = quant_divisor(am, a.sfmt, &stored);
    const int page = new_slot / a.P, sip = new_slot % a.P;
    for (int o = tid; o < S; o += 64) {
      const uint32_t code = (div > 0.0f) ? f32_to_fp8(ynew[o] / div) : 0u;
      const_cast<uint8_t*>(a.kp)[kp_offset(page, h, sip, o, a.Hkv, S, a.P)] = (uint8_t)code;
    }
    if (tid == 0) store_scale(const_cast<void*>(a.kp_scale), ((int64_t)page * a.Hkv + h) * a.P + sip, a.sfmt, stored);
  }
  __syncthreads();

  uint32_t tau;
  if (a.force_exact) {
    tau = 0xffffffffu;                   // stream keeps nothing; finish runs the exact path
  } else if (!sampled) {
    tau = 0u;                            // every token is a candidate
  } else {
    for (int r = 0; r * TPT * kPrologueThreads < ns; ++r) {
      asm volatile("" ::: "memory");     // qh is re-read from LDS each round, not held in registers
      if (r > 0) issue_rows(r);
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        const int u = (r * TPT + j) * kPrologueThreads + tid;
        if (u < ns) skeys[u] = sph[u] >= 0 ? score_key(score_token<R, BF>(pc[j], qh) * sc[j]) : 0u;
      }
    }
    // sampled pages are full pages except when every page is sampled (then
    // the last one holds N - (n_pages - 1) P tokens)
    const uint32_t nvalid = sp == n_pages ? (uint32_t)N : (uint32_t)ns;
    const int64_t target = (int64_t)(2 * a.B < kCandCap / 2 ? 2 * a.B : kCandCap / 2);
    int64_t ks = (nvalid * target + N - 1) / N;
    if (ks < 1) ks = 1;
    if (ks > (int64_t)nvalid) ks = nvalid;
    uint32_t kth, need;
    __syncthreads();                     // every sampled key is in LDS
    // two 11-bit digits suffice for an estimate: tau = the lower edge of the
    // 22-bit bin holding the ks-th sampled key
    block_radix_select<kPrologueThreads>(skeys, ns, (uint32_t)ks, hist, tmp, &kth, &need, kDigitBits - 1);
    tau = kth;
  }
  if (tid == 0) a.tau[bh] = tau;
}

// ================================================================== 2. stream

template <int R, int P, int SF>
__global__ __launch_bounds__(kStreamThreads) void select_stream(SelectArgs a) {
  constexpr int S = R * 16;
  constexpr bool BF = SF == 3;                 // BF16 keys
  constexpr int RP = TokenPieces<R, BF>::value;
  constexpr int PR = 64 / P;                   // pages of one round: lane = (page of the round, slot)
  constexpr int NR = RP >= 16 ? 1 : 16 / RP;   // rounds (tokens per lane), all loads in flight together
  // passes of NR rounds per wavefront: two for tokens of 8 or more pieces
  // (MLA), so that a chunk covers 4 pages and the finish has half the regions
  constexpr int NP = RP >= 8 ? 2 : 1;
  constexpr int WP = NP * NR * PR;             // pages of a wavefront = one chunk
  constexpr int RL = WP * P + kRegionPad;      // entries of one (chunk, KV head) region
  __shared__ __align__(16) uint2 stage[kStreamWaves][WP * P];
  const int lane = lane_id();
  // wavefront -> (KV head of the block's head group, chunk of the block's
  // chunk group); the index is made wave-uniform explicitly so that the head's
  // projected query can live in scalar registers
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int hl = w % a.heads_pb, cw = w / a.heads_pb;
  const int head = blockIdx.x * a.heads_pb + hl;
  const int c = blockIdx.y * a.chunks_pb + cw;
  const int b = blockIdx.z;
  const int N = seq_len_of(a, b);
  const int n_pages = (N + P - 1) / P;
  if (cw >= a.chunks_pb || head >= a.Hkv || c * WP >= n_pages) return;   // uniform over the wavefront
  const int64_t bh = (int64_t)b * a.Hkv + head;
  const int pr = lane / P, slot = lane % P;
  const int page0 = c * WP;

  // this chunk's physical pages: lane i < WP holds page page0 + i
  int phys_l = 0;
  if (lane < WP && page0 + lane < n_pages) phys_l = a.block_table[(int64_t)b * a.max_pages + page0 + lane];
  uint4 pc[NR][RP];
  float sc[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int pg = k * PR + pr;                // page of the chunk this lane reads in round k
    const int64_t phys = __shfl(phys_l, pg);
    if (page0 + pg < n_pages) load_token_sf<RP, SF>(a, phys, head, slot, pc[k], sc[k]);
  }
  // the head's projected query, uniform over the wavefront
  float qh[S];
  {
    const float* src = a.qhat + bh * S;
#pragma unroll
    for (int i = 0; i < S; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + i);
      qh[i] = uniform_f(v.x);
      qh[i + 1] = uniform_f(v.y);
      qh[i + 2] = uniform_f(v.z);
      qh[i + 3] = uniform_f(v.w);
    }
  }
  uint32_t tau = a.tau[bh];
  if (tau == 0u) tau = 1u;                     // key 0 marks "no token"
  const int64_t maxN = (int64_t)a.max_pages * P;
  float* sout = a.scores_out ? a.scores_out + bh * maxN : nullptr;

  // each round's keys >= tau go, in position order (round-major, then lane),
  // to this wavefront's LDS staging area
  uint2* st = stage[threadIdx.x >> 6];
  uint32_t cnt = 0;
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    if constexpr (NP > 1) {
      if (pass > 0) {                          // the next pass's rows (pass 0's were loaded above)
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const int pg = (pass * NR + k) * PR + pr;
          const int64_t phys = __shfl(phys_l, pg);
          if (page0 + pg < n_pages) load_token_sf<RP, SF>(a, phys, head, slot, pc[k], sc[k]);
        }
      }
    }
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int t = (page0 + (pass * NR + k) * PR + pr) * P + slot;
    uint32_t key = 0u;
    if (t < N) {
      const float s = score_token<R, BF>(pc[k], qh) * sc[k];
      key = score_key(s);
      if (sout) sout[t] = s;
    }
    const uint64_t m = ballot(key >= tau);
    if (m & (1ull << lane)) st[cnt + lanes_below(m)] = make_uint2(key, (uint32_t)t);
    cnt += (uint32_t)__popcll(m);
  }
  }
  // the staged entries were written by this wavefront's own LDS instructions,
  // which complete in order; wait for them before reading them back
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // the region goes out as whole 128-byte lines: a header entry (x = the
  // count), then the candidates, the last line padded (scattered partial-line
  // stores of the candidates had measured 6.8 us slower at 128K)
  const int len = (int)((cnt + 16) & ~15u);
  uint2* dst = a.cand + (bh * a.max_chunks + c) * (int64_t)RL;
  for (int e = lane; e < len; e += 64) {
    const uint32_t k = (uint32_t)e - 1u;
    uint2 v = make_uint2(cnt, 0u);
    if (e > 0) v = k < cnt ? st[k] : make_uint2(0u, 0u);
    dst[e] = v;
  }
}

// ================================================================== 3. finish

namespace {

// Exact top-K of one (sequence, KV head) by re-scoring every token: four
// 8-bit radix passes over the keys, then an ordered compaction pass.
template <int R, bool BF>
__device__ void exact_stream_select(const SelectArgs& a, int b, int h, int N, int K, const float* qh,
                                    uint32_t* hist, uint32_t* tmp, int32_t* out) {
  const int tid = (int)threadIdx.x;
  uint32_t prefix = 0u, hi_mask = 0u, k = (uint32_t)K;
  for (int shift = 32 - kDigitBits; ; shift = shift > kDigitBits ? shift - kDigitBits : 0) {
    for (int i = tid; i < kHistWords; i += kFinishThreads) hist[i] = 0u;
    __syncthreads();
    for (int t0 = 0; t0 < N; t0 += kFinishThreads) {
      asm volatile("" ::: "memory");   // qh is re-read from LDS, not held in registers
      const int t = t0 + tid;
      if (t < N) {
        const uint32_t key = token_key<R, BF>(a, b, h, t, qh);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[bin_slot((key >> shift) & (kBins - 1u))], 1u);
      }
    }
    __syncthreads();
    find_digit<kFinishThreads>(hist, k, tmp, tmp + 48);
    __syncthreads();
    prefix = (prefix & ~((kBins - 1u) << shift)) | (tmp[48] << shift);
    k = tmp[49];
    hi_mask = ~((1u << shift) - 1u);
    prefix &= hi_mask;
    __syncthreads();
    if (shift == 0) break;
  }
  const uint32_t kth = prefix, need = k;
  uint32_t gt_run = 0, eq_run = 0;
  for (int t0 = 0; t0 < N; t0 += kFinishThreads) {
    asm volatile("" ::: "memory");
    const int t = t0 + tid;
    const uint32_t key = t < N ? token_key<R, BF>(a, b, h, t, qh) : 0u;
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

template <int R, bool BF>
__global__ __launch_bounds__(kFinishThreads) void select_finish(SelectArgs a) {
  constexpr int S = R * 16;
  const int h = blockIdx.x, b = blockIdx.y, tid = (int)threadIdx.x;
  __shared__ uint32_t lkey[kCandCap];
  __shared__ int32_t lidx[kCandCap];
  __shared__ uint32_t coff[kMaxChunks + 1];
  __shared__ __align__(16) uint32_t hist[2 * kHistWords];
  __shared__ uint32_t tmp[64];
  __shared__ float qh[S];
  const int64_t bh = (int64_t)b * a.Hkv + h;
  int32_t* out = a.indices + bh * a.B;
  const int N = seq_len_of(a, b);
  const int K = N < a.B ? N : a.B;
  for (int i = K + tid; i < a.B; i += kFinishThreads) out[i] = -1;
  if (K == 0) return;

  const uint32_t tau = a.tau[bh];
  const int n_pages = (N + a.P - 1) / a.P;
  const int n_chunks = (n_pages + a.cp - 1) / a.cp;
  // chunk offsets in chunk (= position) order.  A region is a header entry
  // (x = the chunk's count) followed by its candidates; the first line of
  // region tid (header + 15 candidates) is requested before the count scan
  const int rl = a.reg_len;
  const uint2* regions = a.cand + bh * a.max_chunks * (int64_t)rl;
  const bool pact = !a.force_exact && tid < n_chunks;
  uint4 pre[8];
  if (pact) {
    const uint4* src = reinterpret_cast<const uint4*>(regions + (int64_t)tid * rl);
#pragma unroll
    for (int j = 0; j < 8; ++j) pre[j] = src[j];
  }
  // (a count is at most the chunk's tokens; the clamp keeps every read inside
  // the region whatever the header holds)
  const uint32_t cap_chunk = (uint32_t)(a.cp * a.P);
  const uint32_t cnt0 = pact ? min(pre[0].x, cap_chunk) : 0u;
  uint32_t carry = 0;
  for (int c0 = 0; c0 < n_chunks && !a.force_exact; c0 += kFinishThreads) {
    const int c = c0 + tid;
    const uint32_t cnt = c0 == 0 ? cnt0 : (c < n_chunks ? min(regions[(int64_t)c * rl].x, cap_chunk) : 0u);
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kFinishThreads>(cnt, tmp, &tot);
    if (c < n_chunks) coff[c] = carry + ex;
    carry += tot;
  }
  const uint32_t total = carry;
  const bool ok = !a.force_exact && total <= (uint32_t)kCandCap && total >= (uint32_t)K &&
                  (tau != 0u || total == (uint32_t)N);
  if (!ok) {
    for (int i = tid; i < S; i += kFinishThreads) qh[i] = a.qhat[bh * S + i];
    __syncthreads();
    exact_stream_select<R, BF>(a, b, h, N, K, qh, hist, tmp, out);
    return;
  }
  if (tid == 0) coff[n_chunks] = carry;
  __syncthreads();
  // gather the candidates in position order: thread c copies the first 15
  // candidates of chunk c (entries 1..15 of its region) to its offset (read
  // unconditionally, prefetched for c = tid)
  {
    for (int c = tid; c < n_chunks; c += kFinishThreads) {
      const int cnt = (int)(coff[c + 1] - coff[c]);
      const uint2* src = regions + (int64_t)c * rl;
      const uint32_t dst = coff[c];
      uint4 v[8];
      if (c == tid) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = pre[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = reinterpret_cast<const uint4*>(src)[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // entries 2j and 2j + 1 are candidates 2j - 1 and 2j
        if (j > 0 && 2 * j - 1 < cnt) {
          lkey[dst + 2 * j - 1] = v[j].x;
          lidx[dst + 2 * j - 1] = (int32_t)v[j].y;
        }
        if (2 * j < cnt) {
          lkey[dst + 2 * j] = v[j].z;
          lidx[dst + 2 * j] = (int32_t)v[j].w;
        }
      }
    }
    // the rest: lpc lanes per chunk (more when the chunks are few), each lane
    // with four clamped loads in flight, so that a tail of up to 4 lpc
    // entries costs one round trip
    const int w = tid >> 6, lane = tid & 63;
    const int lpc = n_chunks >= 256 ? 4 : (n_chunks >= 64 ? 16 : 64);
    const int cpw = 64 / lpc, sub = lane % lpc;
    for (int c = w * cpw + lane / lpc; c < n_chunks; c += (kFinishThreads / 64) * cpw) {
      const int cnt = (int)(coff[c + 1] - coff[c]);
      const uint2* src = regions + (int64_t)c * rl + 1;    // candidate i at entry 1 + i
      const uint32_t dst = coff[c];
      for (int i0 = 15 + sub; i0 < cnt; i0 += 4 * lpc) {
        uint2 e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e[k] = src[i0 + k * lpc < cnt ? i0 + k * lpc : i0];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (i0 + k * lpc < cnt) {
            lkey[dst + i0 + k * lpc] = e[k].x;
            lidx[dst + i0 + k * lpc] = (int32_t)e[k].y;
          }
        }
      }
    }
  }
  __syncthreads();
  const int n = (int)total;
  if (n <= K) {                                // everything that is there is selected
    for (int i = tid; i < n; i += kFinishThreads) out[i] = lidx[i];
    return;
  }
  uint32_t kth, need;
  block_radix_select<kFinishThreads>(lkey, n, (uint32_t)K, hist, tmp, &kth, &need);
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
}

// ================================================================== launch

namespace {

template <int R, int P, bool BF>
hipError_t launch_select_rpb(const SelectArgs& a, int stages, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (stages & 1) {
    hipLaunchKernelGGL((select_prologue<R, BF>), dim3(a.Hkv, a.batch), dim3(kPrologueThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 2) {
    const int hgroups = (a.Hkv + a.heads_pb - 1) / a.heads_pb;
    const int cgroups = (a.max_chunks + a.chunks_pb - 1) / a.chunks_pb;
    const dim3 grid(hgroups, cgroups, a.batch);
    if (BF)
      hipLaunchKernelGGL((select_stream<R, P, 3>), grid, dim3(kStreamThreads), 0, s, a);
    else if (a.sfmt == 1)
      hipLaunchKernelGGL((select_stream<R, P, 1>), grid, dim3(kStreamThreads), 0, s, a);
    else if (a.sfmt == 2)
      hipLaunchKernelGGL((select_stream<R, P, 2>), grid, dim3(kStreamThreads), 0, s, a);
    else
      hipLaunchKernelGGL((select_stream<R, P, 0>), grid, dim3(kStreamThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 4) {
    hipLaunchKernelGGL((select_finish<R, BF>), dim3(a.Hkv, a.batch), dim3(kFinishThreads), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

template <int R, int P>
hipError_t launch_select_rp(const SelectArgs& a, int stages, hipStream_t s) {
  return a.sfmt == 3 ? launch_select_rpb<R, P, true>(a, stages, s) : launch_select_rpb<R, P, false>(a, stages, s);
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
