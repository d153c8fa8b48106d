// Device helpers shared by the JSSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jssa {

constexpr int kWave = 64;

typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- streaming loads

// Loads of data that one step reads exactly once (the scoring cache in the
// score stream): marked non-temporal, so that they do not displace what the
// caches hold for later reads.
__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_stream_u32(const void* p) {
  return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi over bf16 pairs, fp32 accumulate (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- FP8 (OCP E4M3FN on gfx950)

// Four codes packed little-endian in a dword -> four floats (exact).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// fp32 -> E4M3FN code, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t f32_to_fp8(float x) {
  x = fminf(fmaxf(x, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xffu;
}

// ---------------------------------------------------------------- projection of a key row

// Projection of one bf16 row by one fp32 row of M, split over eight lanes:
// project_part gives part p (0..7) of y = sum_i m[i] x[i], one fp32 FMA chain
// over the 8-element chunks c = p, p + 8, p + 16, ... in order (din % 64 == 0;
// at each step the eight parts read eight consecutive chunks, 256 contiguous
// bytes of m), and proj_combine adds the parts of eight consecutive lanes
// (p = lane & 7) as ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)), leaving
// the same value in all eight (fp32 addition commutes).  jssa_store and the
// store fused into jssa_decode both use this order, so a key gets the same
// codes either way.
__device__ __forceinline__ float project_part(const float* __restrict__ m, const uint16_t* __restrict__ x, int din,
                                              int part) {
  float acc = 0.0f;
#pragma unroll 4
  for (int i = part * 8; i < din; i += 64) {
    const uint4 kv = *reinterpret_cast<const uint4*>(x + i);
    const float4 m0 = *reinterpret_cast<const float4*>(m + i);
    const float4 m1 = *reinterpret_cast<const float4*>(m + i + 4);
    acc = __builtin_fmaf(m0.x, bf16_lo(kv.x), acc);
    acc = __builtin_fmaf(m0.y, bf16_hi(kv.x), acc);
    acc = __builtin_fmaf(m0.z, bf16_lo(kv.y), acc);
    acc = __builtin_fmaf(m0.w, bf16_hi(kv.y), acc);
    acc = __builtin_fmaf(m1.x, bf16_lo(kv.z), acc);
    acc = __builtin_fmaf(m1.y, bf16_hi(kv.z), acc);
    acc = __builtin_fmaf(m1.z, bf16_lo(kv.w), acc);
    acc = __builtin_fmaf(m1.w, bf16_hi(kv.w), acc);
  }
  return acc;
}

// Every lane of the wavefront must execute this.
__device__ __forceinline__ float proj_combine(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  return v;
}

// Scale of one projected key (scoring-cache format sfmt: 0 fp32, 1 E8M0, 2
// none; 3, BF16 keys, has no scale and does not quantise).  Returns the divisor of y (0 for an all-zero row of a scaled format)
// and the stored representation: fp32 bits, the E8M0 byte e + 127 with
// e = ceil(log2(amax / 448)) clamped to [-127, 127], or nothing.
__device__ __forceinline__ float quant_divisor(float amax, int sfmt, uint32_t* stored) {
  if (sfmt == 2) {
    *stored = 0u;
    return 1.0f;
  }
  const float s = amax / 448.0f;
  if (sfmt == 0) {
    *stored = __float_as_uint(s);
    return s;
  }
  if (!(s > 0.0f)) {
    *stored = 0u;
    return 0.0f;
  }
  int e;
  const float m = frexpf(s, &e);          // s = m 2^e, m in [0.5, 1)
  if (m == 0.5f) e -= 1;                   // s is itself 2^(e-1)
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  *stored = (uint32_t)(e + 127);
  return ldexpf(1.0f, e);                  // exact (2^-127 is an fp32 subnormal)
}

__device__ __forceinline__ void store_scale(void* base, int64_t i, int sfmt, uint32_t stored) {
  if (sfmt == 0) static_cast<float*>(base)[i] = __uint_as_float(stored);
  else if (sfmt == 1) static_cast<uint8_t*>(base)[i] = (uint8_t)stored;
}

// The factor a score is multiplied by: the fp32 scale, 2^(E - 127), or 1 (no
// scale, BF16 keys).
// (E8M0 scale arrays start 4-byte aligned; the word of element i lies inside
// the array because the page size is a multiple of 4.)
// E8M0 byte E -> 2^(E - 127) (E = 0: 2^-127, a subnormal fp32)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float(e ? (e << 23) : 0x00400000u); }

__device__ __forceinline__ float load_scale(const void* base, int64_t i, int sfmt) {
  if (sfmt == 0) return static_cast<const float*>(base)[i];
  if (sfmt == 1) {       // the aligned word holding the byte (four lanes share one load)
    const uint32_t w = static_cast<const uint32_t*>(base)[i >> 2];
    return e8m0_to_f32((w >> ((i & 3) * 8)) & 0xffu);
  }
  return 1.0f;
}

// load_scale with streaming (non-temporal) loads
__device__ __forceinline__ float load_scale_stream(const void* base, int64_t i, int sfmt) {
  if (sfmt == 0) return __uint_as_float(load_stream_u32(static_cast<const uint32_t*>(base) + i));
  if (sfmt == 1) {
    const uint32_t w = load_stream_u32(static_cast<const uint32_t*>(base) + (i >> 2));
    return e8m0_to_f32((w >> ((i & 3) * 8)) & 0xffu);
  }
  return 1.0f;
}

// Byte offset of element o of the projected key at (page, head, slot) in the
// piece-major scoring cache [pages][Hkv][S/16][P][16] (BF16 keys: the bytes
// 2o, 2o + 1 of a cache of 2S bytes per token).
__device__ __forceinline__ int64_t kp_offset(int64_t page, int head, int slot, int o, int Hkv, int S, int P) {
  return (page * Hkv + head) * ((int64_t)S * P) + (o >> 4) * (P * 16) + slot * 16 + (o & 15);
}

// ---------------------------------------------------------------- scores and keys

// Projected score of one token before the scale: sum_i qhat_i * dec(code_i) in
// fp32, as four FMA chains (chain e takes the elements i with i % 16 in
// [4e, 4e+4)), summed (c0 + c1) + (c2 + c3).  Every kernel that scores a token
// uses this function, so they all get the same bits.  R = scoring dims / 16;
// `pc` holds the token's R 16-byte pieces.
template <int R>
__device__ __forceinline__ float score_pieces(const uint4 (&pc)[R], const float* qh) {
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint32_t w[4] = {pc[j].x, pc[j].y, pc[j].z, pc[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float f[4];
      fp8x4_to_f32(w[e], f);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[e] = __builtin_fmaf(f[i], qh[j * 16 + e * 4 + i], acc[e]);
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// The same score over BF16 projected keys (the scoring-cache format without
// FP8, two bytes per element): RP = 2 x scoring dims / 16 pieces of 8 values;
// chain e takes the elements i with i % 8 in {2e, 2e + 1}.
template <int RP>
__device__ __forceinline__ float score_pieces_bf16(const uint4 (&pc)[RP], const float* qh) {
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const uint32_t w[4] = {pc[j].x, pc[j].y, pc[j].z, pc[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = __builtin_fmaf(bf16_lo(w[e]), qh[j * 8 + e * 2], acc[e]);
      acc[e] = __builtin_fmaf(bf16_hi(w[e]), qh[j * 8 + e * 2 + 1], acc[e]);
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// 16-byte pieces per token and KV head: S/16 FP8 codes, or 2S/16 for BF16 keys.
template <int R, bool BF>
struct TokenPieces {
  static constexpr int value = BF ? 2 * R : R;
};

template <int R, bool BF>
__device__ __forceinline__ float score_token(const uint4 (&pc)[TokenPieces<R, BF>::value], const float* qh) {
  if constexpr (BF) return score_pieces_bf16<2 * R>(pc, qh);
  else return score_pieces<R>(pc, qh);
}

// Order-preserving float -> uint32 map; -0 and +0 share one key.  Finite
// scores map to keys >= 0x00800000, so key 0 is free to mean "no token".
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- lane utilities

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// A value the caller knows to be the same in every lane, moved to a scalar
// register (the bits of lane 0; readfirstlane works on 32-bit integers).
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Lane u (0..15) of every row of 16 lanes, broadcast to the whole row (DPP
// row_newbcast).  u must be a constant once the caller's loop is unrolled.
template <int U>
__device__ __forceinline__ int row_bcast_c(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x150 + U, 0xf, 0xf, false);
}
__device__ __forceinline__ int row_bcast(int x, int u) {
  switch (u) {
    case 0: return row_bcast_c<0>(x);
    case 1: return row_bcast_c<1>(x);
    case 2: return row_bcast_c<2>(x);
    case 3: return row_bcast_c<3>(x);
    case 4: return row_bcast_c<4>(x);
    case 5: return row_bcast_c<5>(x);
    case 6: return row_bcast_c<6>(x);
    case 7: return row_bcast_c<7>(x);
    case 8: return row_bcast_c<8>(x);
    case 9: return row_bcast_c<9>(x);
    case 10: return row_bcast_c<10>(x);
    case 11: return row_bcast_c<11>(x);
    case 12: return row_bcast_c<12>(x);
    case 13: return row_bcast_c<13>(x);
    case 14: return row_bcast_c<14>(x);
    default: return row_bcast_c<15>(x);
  }
}
__device__ __forceinline__ float row_bcast_f(float x, int u) { return __int_as_float(row_bcast(__float_as_int(x), u)); }

// Sum over each row of 16 lanes (DPP row rotations); every lane of the row
// receives the row total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0x128>(x);  // row_ror:8
  x += dpp_f<0x124>(x);  // row_ror:4
  x += dpp_f<0x122>(x);  // row_ror:2
  x += dpp_f<0x121>(x);  // row_ror:1
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o);
  return x;
}

// x from the lane `CTRL` selects (DPP), 0 where the control has no source lane
// or the row is masked off.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the wave with DPP: row shifts 1, 2, 4, 8 within
// each row of 16 lanes, then row_bcast:15 and row_bcast:31 carry the row
// totals across rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u<0x111, 0xf>(x);  // row_shr:1
  x += dpp_u<0x112, 0xf>(x);  // row_shr:2
  x += dpp_u<0x114, 0xf>(x);  // row_shr:4
  x += dpp_u<0x118, 0xf>(x);  // row_shr:8
  x += dpp_u<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_u<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Block-wide exclusive prefix sum of one uint32 per thread; `tmp` is LDS with
// at least NT/64 + 1 words.  Returns the exclusive prefix; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tmp, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int l = lane_id(), w = (int)(threadIdx.x >> 6);
  uint32_t inc = wave_incl_scan(x);
  if (l == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    uint32_t v = (l < NW) ? tmp[l] : 0u;
    uint32_t vi = wave_incl_scan(v);
    if (l < NW) tmp[l] = vi - v;
    if (l == NW - 1) tmp[NW] = vi;
  }
  __syncthreads();
  uint32_t res = tmp[w] + inc - x;
  *total = tmp[NW];
  __syncthreads();
  return res;
}

template <int NT>
__device__ __forceinline__ uint32_t block_or(uint32_t x, uint32_t* tmp) {
  constexpr int NW = NT / 64;
  const int l = lane_id(), w = (int)(threadIdx.x >> 6);
  x = wave_or(x);
  if (l == 0) tmp[w] = x;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) r |= tmp[i];
  __syncthreads();
  return r;
}

}  // namespace jssa
