// Block-wide radix select over 32-bit keys in LDS (the select kernels and the
// single-launch decode kernel).
#pragma once

#include "common.h"

namespace jssa {

constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

// Histogram bins are stored transposed with one word of padding per row: bin d
// at word (d % 32) * 65 + d / 32.  Lane l of a wavefront then reads "its" 32
// consecutive bins [32l, 32l + 32) with reads that are consecutive across
// lanes, and neighbouring bins (where keys cluster) sit in different banks.
constexpr int kHistWords = 32 * 65;
__device__ __forceinline__ uint32_t bin_slot(uint32_t d) { return (d & 31u) * 65u + (d >> 5); }

// Pick the digit d of the current pass so that fewer than k matching keys have
// a larger digit and at least k have a digit >= d: thread t owns kBins/NT
// consecutive bins; the count above its bins comes from a block prefix sum.
// (Used by the exact re-scoring path, where the whole block streams tokens.)
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t k, uint32_t* tmp, uint32_t* bcast) {
  constexpr int BPT = kBins / NT;
  const int tid = (int)threadIdx.x;
  uint32_t c[BPT], s = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    c[j] = hist[bin_slot((uint32_t)(tid * BPT + j))];
    s += c[j];
  }
  uint32_t total;
  const uint32_t ex = block_excl_scan<NT>(s, tmp, &total);
  uint32_t above = total - ex - s;  // keys in the bins of higher threads
#pragma unroll
  for (int j = BPT - 1; j >= 0; --j) {
    if (above < k && k <= above + c[j]) {
      bcast[0] = (uint32_t)(tid * BPT + j);
      bcast[1] = k - above;
    }
    above += c[j];
  }
}


// Wave 0 only: find the digit d with count(digit > d) < k <= count(digit >= d)
// and publish d and k - count(digit > d) in bcast[0..1].
__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, uint32_t k, uint32_t* bcast) {
  const int l = lane_id();
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) sum += hist[j * 65 + l];
  const uint32_t pre = wave_incl_scan(sum);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63);
  const uint32_t suf = total - pre + sum;  // inclusive suffix sum over lanes >= l
  const uint32_t above = suf - sum;
  // the lane whose 32 bins hold the k-th key, then the bin among those 32,
  // with lanes 0..31 taking one bin each (uniform control flow)
  const int ls = (int)__builtin_ctzll(ballot(above < k && k <= suf));
  const uint32_t above_ls = (uint32_t)__builtin_amdgcn_readlane((int)above, ls);
  const uint32_t tot_ls = (uint32_t)__builtin_amdgcn_readlane((int)sum, ls);
  const uint32_t cj = l < 32 ? hist[l * 65 + ls] : 0u;
  const uint32_t pj = wave_incl_scan(cj);
  const uint32_t incl = above_ls + (tot_ls - pj + cj), excl = incl - cj;
  const bool hit = l < 32 && excl < k && k <= incl;
  const int js = (int)__builtin_ctzll(ballot(hit));
  if (l == js) {
    bcast[0] = (uint32_t)(ls * 32 + js);
    bcast[1] = k - excl;
    bcast[2] = cj;                       // keys in the digit's bin
  }
}

// k-th largest key (1-based) of keys[0..n) in LDS and how many keys equal to it
// belong to the top k.  Skips the leading bits all keys share, then resolves
// kDigitBits bits per pass: every thread adds its keys to an LDS histogram,
// wave 0 finds the digit; two block barriers per pass (the histogram of the
// next pass is cleared during the current one).  hist2 holds 2 * kHistWords words.
//
// With stop_shift > 0 the digits below bit stop_shift are not resolved: *kth
// is then the lower edge (low bits zero) of the bin holding the k-th key, a
// bound <= the k-th key, and *need is not meaningful.  With stop_shift == 0,
// once the k-th key's bin holds exactly the keys still needed (all of them
// belong to the top k), the passes end: *kth is then one below the bin's
// lower edge and *need is 0, which selects the same set (key > *kth).
template <int NT>
__device__ void block_radix_select(const uint32_t* keys, int n, uint32_t k, uint32_t* hist2, uint32_t* tmp,
                                   uint32_t* kth, uint32_t* need, int stop_shift = 0) {
  const int tid = (int)threadIdx.x;
  for (int i = tid; i < kHistWords; i += NT) hist2[i] = 0u;
  const uint32_t ref = keys[0];
  uint32_t orv = 0;
  for (int i = tid; i < n; i += NT) orv |= keys[i] ^ ref;
  orv = block_or<NT>(orv, tmp);       // barriers also publish the cleared histogram
  if (orv == 0u) {
    *kth = ref;
    *need = k;
    return;
  }
  int hb = 31 - __builtin_clz(orv);
  uint32_t hi_mask = (hb == 31) ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = ref & hi_mask;
  for (int pass = 0;; ++pass) {
    uint32_t* cur = hist2 + (pass & 1) * kHistWords;
    uint32_t* nxt = hist2 + ((pass + 1) & 1) * kHistWords;
    const int shift = hb >= kDigitBits - 1 ? hb - (kDigitBits - 1) : 0;
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = keys[i];
      if ((key & hi_mask) == prefix) atomicAdd(&cur[bin_slot((key >> shift) & (kBins - 1u))], 1u);
    }
    for (int i = tid; i < kHistWords; i += NT) nxt[i] = 0u;
    __syncthreads();
    if (tid < 64) wave_find_digit(cur, k, tmp + 48);
    __syncthreads();
    prefix = (prefix & ~((kBins - 1u) << shift)) | (tmp[48] << shift);
    k = tmp[49];
    hi_mask = ~((1u << shift) - 1u);
    prefix &= hi_mask;
    if (shift <= stop_shift) break;
    if (stop_shift == 0 && tmp[50] == k && prefix > 0u) {
      *kth = prefix - 1u;
      *need = 0u;
      __syncthreads();                 // tmp is reused by the caller
      return;
    }
    hb = shift - 1;
  }
  *kth = prefix;
  *need = k;
  __syncthreads();                     // tmp is reused by the caller
}

}  // namespace jssa
