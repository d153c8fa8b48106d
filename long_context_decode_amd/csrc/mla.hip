// MLA attention over latent rows (README page, paper-to-code map: JSSA on MLA
// uses FlashMLA sparse attention over the selected positions; summary page
// §3.4: 64 latent + 64 RoPE scoring dims).  Every query head of sequence b
// attends to the same rows [c (512) ; k_pe (64)]: logits sm * q . row over all
// 576 dims, values = the first 512 dims of the row.
//
// This is a dense contraction per sequence (Q 128x576 times 576xn, then
// P 128xn times nx512), so it runs on the matrix cores: v_mfma_f32_16x16x32_bf16
// (lane l holds A[l%16][8(l/16)..+8], B[8(l/16)..+8][l%16] and returns
// D[4(l/16)+j][l%16]).  Two kernels share that product and differ in what
// limits them:
//
// mla_sparse_kernel: the B selected rows (a few thousand per sequence).  The
// work per sequence is small, so it is split over many blocks and the fp32
// partials of the splits dominate the traffic; blocks of 32 heads keep the
// partials at 2 KB per (head, split) while filling two blocks per CU.
// Block = (split of the selected rows, block of 32 query heads, sequence),
// 4 wavefronts.  Per tile of 32 rows:
//   * the rows are gathered once into LDS (row stride 584 elements); the next
//     tile's loads are in flight in registers while the current one computes;
//   * S = Q K^T: wavefront w takes heads [16 (w & 1), +16) over the dims
//     [288 (w >> 1), +288) (9 K-steps) for all 32 rows, so its part of Q
//     stays in registers (9 MFMA operands) for the whole block and K comes
//     from LDS; the two dim halves are summed through LDS, wavefront w
//     finishing rows [16 (w >> 1), +16);
//   * online softmax per head (base 2): the two wavefronts holding a head's
//     rows exchange tile maxima and sums through LDS; every wavefront keeps
//     the running state of all 32 heads and rescales its part of the output;
//   * O += P V: wavefront w owns output dims [128w, 128w+128) (2 x 8 tiles of
//     16x16), P (bf16) comes from LDS, V is read column-wise from the same LDS
//     tile with the transposing LDS read (4 rows of one dim per instruction).
//
// mla_dense_kernel: all positions [lo, N) (lo = N - window for a window, else
// 0), the full-KV baseline.  Long row streams per block, so the tile loop is
// what counts.  Block = (split of the rows, block of 64 query heads,
// sequence), 4 wavefronts of 16 heads each, two blocks per CU.  Each
// wavefront runs its own online softmax over every row of the split; the only
// synchronisation is the hand-over of the row tiles:
//   * tiles of 32 rows are copied from the cache straight into LDS
//     (global_load_lds_dwordx4, no registers), double buffered: tile k+1 is
//     in flight while tile k is used.  A row of 72 16-byte pieces is stored
//     with its pieces permuted within aligned groups of 8 (XOR with a function
//     of the row), which keeps both LDS read patterns below free of bank
//     conflicts;
//   * the products are taken transposed, rows in the M dimension and heads in
//     N: S^T = K Q^T (A = K rows from LDS, B = the wavefront's Q, held in
//     registers for the whole block), so that a lane ends up with 8 logits of
//     one head (rows 4(l/16)+j and 16+4(l/16)+j, head l%16).  The softmax of
//     a head is then lane-local apart from two cross-lane max steps, and the
//     8 probabilities, packed to bf16, are directly the B operand of
//     O^T += V^T P^T over those 8 rows (the K order of the product is the
//     permutation the layout gives);
//   * V^T comes from the same LDS tile through the transposing read
//     ds_read_b64_tr_b16 (4 rows of one dim per lane, two reads per operand);
//   * the running max may lag the true one by up to 2^8 (probabilities up to
//     256 before normalisation), so the 32 output tiles are rescaled only
//     when a head's max rises further.
//
// Both write each split's partial (unnormalised o, running max, running sum)
// to the workspace, and merge_kernel<512> combines the splits.  Block order:
// the head blocks of one (split, sequence) read the same rows.  Workgroups
// are dealt to the 8 XCDs round robin (workgroup L runs on XCD L mod 8), so
// the linear block id is laid out to put those head blocks on one XCD, one
// after another, where the later ones find the rows in its L2.
#include "common.h"
#include "kernels.h"

namespace jssa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = kMlaLatent + kMlaRope;  // 576
constexpr int kV = kMlaLatent;             // 512
constexpr int kThreads = 256;
constexpr int kTile = 32;                  // rows per tile
constexpr int kChunkRows = 1024;           // rows resolved at a time (32 tiles)
constexpr int kTilesPerChunk = kChunkRows / kTile;
constexpr int kKSteps = kD / 32;           // 18

// sparse kernel
constexpr int kSpHeads = 32;               // query heads per block
constexpr int kRow = kD + 8;               // LDS row stride of K rows (elements)
constexpr int kPRow = kTile + 8;           // LDS row stride of P (elements)
constexpr int kKHalf = kKSteps / 2;        // 9 K-steps per wavefront
constexpr int kPieces = kTile * (kD / 8) / kThreads;   // 16-byte pieces per thread per tile: 9

// dense kernel
constexpr int kHW = 16;                    // query heads per wavefront
constexpr int kDnHeads = 64;               // query heads per block
constexpr int kRowBytes = kD * 2;          // 1152: 72 pieces of 16 bytes
constexpr int kTileBytes = kTile * kRowBytes;
constexpr int kCopies = kTileBytes / (kThreads * 16);   // 16-byte copies per thread per tile: 9
constexpr int kDimTiles = kV / 16;         // 32
constexpr float kSlack = 8.0f;             // log2 units the running max may lag
constexpr int kPB = 2;                     // dim tiles whose V operands are read together

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane 4k + a supplies the address of 4 consecutive bf16 and lane 4a' + b'
// receives element b' of the chunks of lanes a', 4 + a', 8 + a', 12 + a' (k = 0..3).
__device__ __forceinline__ bf16x4 ds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(const_cast<void*>(p)));
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x122>(x));
  x = fmaxf(x, dpp_f<0x121>(x));
  return x;
}

// piece permutation of tile row t in the dense kernel: piece p is stored at
// p ^ swz(t).  Rows t..t+7 (aligned) get 8 distinct values (the 16-byte K
// reads of 8 lanes on 8 rows cover all banks) and rows t..t+3 distinct values
// of swz >> 1 (the 8-byte transposing reads of 4 rows x 16 dims cover all banks).
__device__ __forceinline__ int swz(int t) { return (((t & 3) << 1) | ((t >> 2) & 1)) ^ (((t >> 3) & 1) << 1); }

__device__ __forceinline__ float lanes16_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float lanes16_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

}  // namespace

// ---------------------------------------------------------------- sparse

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void mla_sparse_kernel(AttendArgs a) {
  __shared__ __align__(16) uint16_t Kt[kTile * kRow];
  __shared__ __align__(16) uint16_t Ps[kSpHeads * kPRow];
  __shared__ __align__(16) float red_m[2][kSpHeads];     // [row half][head] tile maxima
  __shared__ __align__(16) float red_l[2][kSpHeads];     // [row half][head] tile sums
  __shared__ int rows[kChunkRows];                  // physical rows of the current chunk of tiles
  __shared__ f32x4 Sx[4][64];                       // [heads half][row half][lane] S halves in exchange

  const int HB = a.Hq / kSpHeads;
  const int L = (int)blockIdx.x;
  const int rest = L >> 3, hb = rest % HB;
  const int u = (rest / HB) * 8 + (L & 7);      // unit = (split, sequence)
  if (u >= a.splits * a.batch) return;
  const int s = u % a.splits, b = u / a.splits;
  const int tid = (int)threadIdx.x, l = lane_id(), w = tid >> 6;
  const int g = l >> 4, c = l & 15;
  const int mt = w & 1, rt = w >> 1;             // S: heads 16 mt .., rows 16 rt .. of the tile
  const int kh = rt;                             // and dims [288 kh, +288) of the product
  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  const int n_tok = N < a.B ? N : a.B;
  const int i0 = s * a.split_len;
  if (i0 >= n_tok) return;
  const int i1 = min(i0 + a.split_len, n_tok);
  const int n_tiles = (i1 - i0 + kTile - 1) / kTile;
  const int32_t* idx = a.indices + (int64_t)b * a.B;    // Hkv = 1
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  // physical rows (-1: none) of the chunk of tiles ch into rows[]: every
  // thread resolves 4 positions, index and block-table loads batched and
  // unconditional (clamped to the split's last position and to page 0), so
  // that no load sits behind a branch
  auto fill_chunk = [&](int ch) {
    const int base = i0 + ch * kChunkRows;
    int tv[kChunkRows / kThreads], pv[kChunkRows / kThreads];
#pragma unroll
    for (int j = 0; j < kChunkRows / kThreads; ++j) {
      const int ii = base + tid + j * kThreads;
      tv[j] = idx[ii < i1 ? ii : i1 - 1];
      if (ii >= i1 || tv[j] >= N) tv[j] = -1;     // a listed position outside [0, N) counts as missing
    }
#pragma unroll
    for (int j = 0; j < kChunkRows / kThreads; ++j) pv[j] = bt[(tv[j] < 0 ? 0 : tv[j]) / a.P];
#pragma unroll
    for (int j = 0; j < kChunkRows / kThreads; ++j)
      rows[tid + j * kThreads] = tv[j] >= 0 ? pv[j] * a.P + tv[j] % a.P : -1;
  };
  // the tile's 32 x 72 16-byte pieces, 9 per thread, all loads in flight
  // together.  A missing row (past the split's end) is loaded from the tile's
  // first row, which exists unless the index list holds a position outside
  // [0, N) there (then row 0 of the cache, which exists whenever any row
  // does): its logits are masked to -inf, so its weight is 0 and its
  // (finite) values add nothing.  `vld` records whether this lane's S row
  // 16 rt + c of the tile exists.
  auto fetch = [&](int kt, u32x4 (&reg)[kPieces], bool& vld) {
    const int* rw = rows + (kt % kTilesPerChunk) * kTile;
    const int r0 = max(rw[0], 0);
    int rr[kPieces];
#pragma unroll
    for (int k = 0; k < kPieces; ++k) rr[k] = rw[(tid + k * kThreads) / (kD / 8)];
    vld = rw[rt * 16 + c] >= 0;
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int cc = (tid + k * kThreads) % (kD / 8);
      reg[k] = *reinterpret_cast<const u32x4*>(a.k_cache + (int64_t)(rr[k] < 0 ? r0 : rr[k]) * kD + cc * 8);
    }
  };
  auto put = [&](const u32x4 (&reg)[kPieces]) {
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int q = tid + k * kThreads, tt = q / (kD / 8), cc = q % (kD / 8);
      *reinterpret_cast<u32x4*>(&Kt[tt * kRow + cc * 8]) = reg[k];
    }
  };

  // this wavefront's 16 heads of Q over its half of the 576 dims as MFMA A
  // operands (lane: head 16 mt + c, dims (9 kh + ks) * 32 + 8 g .. + 8),
  // loaded while the first chunk's rows resolve
  bf16x8 qa[kKHalf];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + hb * kSpHeads + mt * 16 + c) * kD + kh * kKHalf * 32 + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKHalf; ++ks) qa[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32);
  }
  fill_chunk(0);
  __syncthreads();
  u32x4 reg[kPieces];
  bool vnext;
  fetch(0, reg, vnext);

  // running state of heads mt' * 16 + 4 g + j (mt' = 0, 1; j = 0..3): the
  // rows of this lane's output accumulators
  float m_run[2][4], l_run[2][4];
  f32x4 O[2][8];
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m_run[m2][j] = -INFINITY;
      l_run[m2][j] = 0.0f;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) O[m2][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  for (int k = 0; k < n_tiles; ++k) {
    __syncthreads();                                   // previous tile consumed
    put(reg);
    const bool valid = vnext;
    if (k + 1 < n_tiles && (k + 1) % kTilesPerChunk == 0) fill_chunk((k + 1) / kTilesPerChunk);
    __syncthreads();
    // next tile's loads overlap this tile's math (the last tile fetches itself
    // again, so that the loads are unconditional and need no register copies)
    fetch(k + 1 < n_tiles ? k + 1 : k, reg, vnext);

    // ---- S = Q K^T over this wavefront's half of the dims for both row
    // halves of the tile (heads 16 mt + 4 g + j, rows 16 t + c); the half of
    // the other wavefront's row half goes to it through LDS
    f32x4 S0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, S1 = S0;
#pragma unroll
    for (int k0 = 0; k0 < kKHalf; k0 += 3) {         // K operands of 3 K-steps read together
      bf16x8 b0[3], b1[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int col = (kh * kKHalf + k0 + i) * 32 + g * 8;
        b0[i] = *reinterpret_cast<const bf16x8*>(&Kt[c * kRow + col]);
        b1[i] = *reinterpret_cast<const bf16x8*>(&Kt[(16 + c) * kRow + col]);
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        S0 = mfma16(qa[k0 + i], b0[i], S0);
        S1 = mfma16(qa[k0 + i], b1[i], S1);
      }
    }
    f32x4 S, So;                                       // own and other row half (element selects)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S[i] = rt == 0 ? S0[i] : S1[i];
      So[i] = rt == 0 ? S1[i] : S0[i];
    }
    Sx[mt * 2 + (rt ^ 1)][l] = So;
    __syncthreads();
    S += Sx[mt * 2 + rt][l];
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = valid ? S[j] * a.sm_log2 : -INFINITY;
      const float tm = row16_max(x[j]);
      if (c == 0) red_m[rt][mt * 16 + g * 4 + j] = tm;
    }
    __syncthreads();
    // ---- new running max of every head this lane accumulates (both halves of
    // the tile); the state and this lane's output rows are rescaled at once
    float m_own[4];                                    // new maxima of heads 16 mt + 4 g + j
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hh = m2 * 16 + g * 4 + j;
        const float mn = fmaxf(m_run[m2][j], fmaxf(red_m[0][hh], red_m[1][hh]));
        const float ms = (mn == -INFINITY) ? 0.0f : mn;
        const float al = __builtin_amdgcn_exp2f(m_run[m2][j] - ms);
        m_run[m2][j] = mn;
        l_run[m2][j] *= al;
        if (m2 == 0) m_own[j] = ms;
        else m_own[j] = mt == 0 ? m_own[j] : ms;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) O[m2][nt][j] *= al;
      }
    // ---- P of this wavefront's (16 heads x 16 rows), its row sums
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = mt * 16 + g * 4 + j;
      const float ms = m_own[j];
      const float p = __builtin_amdgcn_exp2f(x[j] - ms);
      const float ps = row16_sum(p);
      if (c == 0) red_l[rt][hh] = ps;
      Ps[hh * kPRow + rt * 16 + c] = __builtin_bit_cast(uint16_t, (__bf16)p);
    }
    __syncthreads();
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hh = m2 * 16 + g * 4 + j;
        l_run[m2][j] += red_l[0][hh] + red_l[1][hh];
      }

    // ---- O += P V for output dims [128w, 128w + 128): one K-step of 32 rows
    bf16x8 ap[2];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) ap[m2] = *reinterpret_cast<const bf16x8*>(&Ps[(m2 * 16 + c) * kPRow + g * 8]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      // B operand: rows 8g .. 8g+7 of dim w*128 + nt*16 + c, two transposing
      // reads of 4 rows each (lane 4k + a of the group points at row +k, dims +4a ..)
      const int dim0 = w * 128 + nt * 16 + (c & 3) * 4;
      const int row0 = g * 8 + (c >> 2);
      const bf16x4 v0 = ds_read_tr(&Kt[row0 * kRow + dim0]);
      const bf16x4 v1 = ds_read_tr(&Kt[(row0 + 4) * kRow + dim0]);
      const bf16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) O[m2][nt] = mfma16(ap[m2], bv, O[m2][nt]);
    }
  }

  // ---- this split's partial
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int head = hb * kSpHeads + m2 * 16 + g * 4 + j;
      const int64_t pj = ((int64_t)b * a.Hq + head) * a.splits + s;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) a.part_o[pj * kV + w * 128 + nt * 16 + c] = O[m2][nt][j];
      if (w == 0 && c == 0) {
        a.part_ml[pj * 2] = m_run[m2][j];
        a.part_ml[pj * 2 + 1] = l_run[m2][j];
      }
    }
}

// ---------------------------------------------------------------- dense

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void mla_dense_kernel(AttendArgs a) {
  __shared__ __align__(16) unsigned char tile0[kTileBytes];
  __shared__ __align__(16) unsigned char tile1[kTileBytes];
  __shared__ int rows[kChunkRows];                  // physical rows of the current chunk of tiles

  const int HB = (a.Hq + kDnHeads - 1) / kDnHeads;
  const int L = (int)blockIdx.x;
  const int rest = L >> 3, hb = rest % HB;
  const int u = (rest / HB) * 8 + (L & 7);      // unit = (split, sequence)
  if (u >= a.splits * a.batch) return;
  const int s = u % a.splits, b = u / a.splits;
  const int tid = (int)threadIdx.x, l = lane_id(), w = tid >> 6;
  const int g = l >> 4, c = l & 15;
  const int head0 = hb * kDnHeads + w * kHW;          // this wavefront's heads head0 .. head0 + 15
  const bool wact = head0 < a.Hq;                // Hq is a multiple of 16
  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  const int n_tok = (a.window > 0 && N > a.window) ? a.window : N;
  const int lo = N - n_tok;
  const int i0 = s * a.split_len;
  if (i0 >= n_tok) return;
  const int i1 = min(i0 + a.split_len, n_tok);
  const int n_tiles = (i1 - i0 + kTile - 1) / kTile;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  // physical rows (-1: none) of the chunk of tiles ch into rows[]: every
  // thread resolves 4 positions, block-table loads batched and unconditional
  // (clamped to page 0)
  auto fill_chunk = [&](int ch) {
    const int base = i0 + ch * kChunkRows;
    int tv[kChunkRows / kThreads], pv[kChunkRows / kThreads];
#pragma unroll
    for (int j = 0; j < kChunkRows / kThreads; ++j) {
      const int ii = base + tid + j * kThreads;
      tv[j] = ii < i1 ? lo + ii : -1;
    }
#pragma unroll
    for (int j = 0; j < kChunkRows / kThreads; ++j) pv[j] = bt[(tv[j] < 0 ? 0 : tv[j]) / a.P];
#pragma unroll
    for (int j = 0; j < kChunkRows / kThreads; ++j)
      rows[tid + j * kThreads] = tv[j] >= 0 ? pv[j] * a.P + tv[j] % a.P : -1;
  };
  // copies of tile kt into dst: wavefront w writes the 1 KB stretches
  // 9w .. 9w+8 of the tile, lane l the 16-byte slot 64 (9w + k) + l, which
  // is piece (slot mod 72) ^ swz(row) of row slot / 72.  A missing row (past
  // the split's end) is copied from the tile's first row,
  // which always exists: its logits are masked to -inf, so its weight is 0
  // and its (finite) values add nothing.  Returns the tile's row-valid mask.
  auto issue = [&](int kt, unsigned char* dst) -> uint32_t {
    const int* rw = rows + (kt % kTilesPerChunk) * kTile;
    const int r0 = rw[0];
    const uint32_t vm = (uint32_t)ballot(l < kTile && rw[l & (kTile - 1)] >= 0);
    // the slot arithmetic is redone per tile (an opaque copy of the lane id
    // keeps it from being hoisted into 9 registers live across the loop)
    int lv = l;
    asm volatile("" : "+v"(lv));
    // all row numbers first (the copies count as LDS writes, so reads placed
    // after one would wait for it)
    int rr[kCopies], po[kCopies];
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const int q = (w * kCopies + k) * 64 + lv;
      const int t = q / (kRowBytes / 16), pc = q % (kRowBytes / 16);
      rr[k] = rw[t];
      po[k] = (pc ^ swz(t)) * 8;
    }
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const uint16_t* src = a.k_cache + (int64_t)(rr[k] < 0 ? r0 : rr[k]) * kD + po[k];
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(dst + (w * kCopies + k) * 1024),
                                       16, 0, 0);
    }
    return vm;
  };

  // the wavefront's Q^T as MFMA B operands (lane: head head0 + c, dims
  // 32 ks + 8 g .. + 8), loaded while the first chunk's rows resolve
  bf16x8 qb[kKSteps];
  {
    const int hq = min(head0 + c, a.Hq - 1);
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + hq) * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32);
  }
  fill_chunk(0);
  __syncthreads();
  uint32_t vm = issue(0, tile0);

  // per-lane LDS byte offsets.  S^T A operand: rows c and 16 + c, piece
  // 4 ks + g -> (ks ^ f2) * 64 + ((g ^ swz) & 3) * 16.
  const int fS = swz(c);
  const int f2 = (fS >> 2) & 1;
  const int sb = c * kRowBytes + (((g ^ fS) & 3) << 4);
  const int s_even = sb + (f2 << 6), s_odd = sb - (f2 << 6);   // (ks ^ f2) * 64 = ks * 64 +- f2 * 64
  // V^T A operand: lane (g, 4 kk + aa) points at row 4 g + kk (and 16 more),
  // dims 16 dt + 4 aa .. + 4 = half (aa & 1) of piece 2 dt + (aa >> 1).
  const int kk = c >> 2, aa = c & 3;
  const int tvr = 4 * g + kk;
  const int fV = swz(tvr);
  const int fv = (fV >> 1) & 3;
  const int vb = tvr * kRowBytes + ((((aa >> 1) ^ fV) & 1) << 4) + ((aa & 1) << 3);

  // running state of head head0 + c (the same in the 4 lane groups); l_run
  // sums this lane's rows only
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 O[kDimTiles];                            // O^T: dims 16 dt + 4 g + j, head c
#pragma unroll
  for (int dt = 0; dt < kDimTiles; ++dt) O[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto body = [&](int k, const unsigned char* cur, unsigned char* nxt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this lane's copies of tile k have landed
    __syncthreads();                                    // everyone's have; tile k-1 is consumed
    uint32_t vm_next = 0u;
    if (k + 1 < n_tiles) {
      if ((k + 1) % kTilesPerChunk == 0) {
        fill_chunk((k + 1) / kTilesPerChunk);
        __syncthreads();
      }
      vm_next = issue(k + 1, nxt);                      // in flight while tile k is used
    }
    if (wact) {
      // ---- S^T = K Q^T: rows 4 g + j (S0) and 16 + 4 g + j (S1), head c
      f32x4 S0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, S1 = S0;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const int off = ((ks & 1) ? s_odd : s_even) + (ks << 6);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(cur + off);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(cur + off + 16 * kRowBytes);
        S0 = mfma16(a0, qb[ks], S0);
        S1 = mfma16(a1, qb[ks], S1);
      }
      // ---- online softmax of head c over the tile's 32 rows (base 2)
      float x0[4], x1[4], mx = -INFINITY;
      const uint32_t vg = vm >> (4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x0[j] = ((vg >> j) & 1u) ? S0[j] * a.sm_log2 : -INFINITY;
        x1[j] = ((vg >> (16 + j)) & 1u) ? S1[j] * a.sm_log2 : -INFINITY;
        mx = fmaxf(mx, fmaxf(x0[j], x1[j]));
      }
      mx = lanes16_max(mx);
      if (ballot(mx > m_run + kSlack) != 0ull) {        // some head's max rose by more than the slack
        const float mn = fmaxf(m_run, mx);
        const float al = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - mn);
        m_run = mn;
        l_run *= al;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) O[dt] *= al;
      }
      const float ms = (m_run == -INFINITY) ? 0.0f : m_run;
      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(x0[j] - ms);
        const float p1 = __builtin_amdgcn_exp2f(x1[j] - ms);
        l_run += p0 + p1;
        pb[j] = (__bf16)p0;
        pb[4 + j] = (__bf16)p1;
      }
      // ---- O^T += V^T P^T over the tile (K order: rows 4 g .. 4 g + 3, then 16 + 4 g ..)
#pragma unroll
      for (int d0 = 0; d0 < kDimTiles; d0 += kPB) {   // operands of kPB dim tiles in flight together
        bf16x8 av[kPB];
#pragma unroll
        for (int i = 0; i < kPB; ++i) {
          const int dt = d0 + i;
          const int off = vb + (((dt & ~3) | ((dt & 3) ^ fv)) << 5);
          const bf16x4 v0 = ds_read_tr(cur + off);
          const bf16x4 v1 = ds_read_tr(cur + off + 16 * kRowBytes);
          av[i] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < kPB; ++i) O[d0 + i] = mfma16(av[i], pb, O[d0 + i]);
      }
    }
    vm = vm_next;
  };
  // two tiles per trip, so that every LDS access names its buffer
  for (int k = 0; k < n_tiles; k += 2) {
    body(k, tile0, tile1);
    if (k + 1 < n_tiles) body(k + 1, tile1, tile0);
  }

  // ---- this split's partial
  l_run = lanes16_sum(l_run);
  if (wact) {
    const int64_t pj = ((int64_t)b * a.Hq + head0 + c) * a.splits + s;
    float* po = a.part_o + pj * kV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16) = make_float4(O[dt][0], O[dt][1], O[dt][2], O[dt][3]);
    if (g == 0) {
      a.part_ml[pj * 2] = m_run;
      a.part_ml[pj * 2 + 1] = l_run;
    }
  }
}

hipError_t launch_mla_attend(const AttendArgs& a, hipStream_t s) {
  const int units = a.splits * a.batch;
  const int padded = ((units + 7) / 8) * 8;
  if (a.indices)
    hipLaunchKernelGGL(mla_sparse_kernel, dim3((unsigned)(padded * (a.Hq / kSpHeads))), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(mla_dense_kernel, dim3((unsigned)(padded * ((a.Hq + kDnHeads - 1) / kDnHeads))),
                       dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a, kV, s);
}

}  // namespace jssa
