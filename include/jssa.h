/*
 * jssa.h — C ABI of the Joint Subspace Sparse Attention (JSSA) decode hot path
 * on AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Method (paper summary page "Summary (Overview)" of arXiv 2610.19026,
 * §3.1 Overview): for every layer and KV head keep an FP8 cache of keys
 * projected onto an r-dim orthonormal basis M (K_proj = K M^T, §3.4); at each
 * decode step average the G query heads of the KV head, project the mean with
 * M, score every cached token against K_proj (Eq. 1), keep the top-B
 * positions of that KV head, and attend the full-dimensional queries of the
 * group to those positions in place in the paged bf16 KV cache (§3.3,
 * "gather-free indexed attention").  M comes from calibration (Eq. 5).
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller unless a
 *     function says "host".  Row-major, densely packed.  bf16 is passed as
 *     uint16_t bit patterns.  FP8 is OCP E4M3FN.
 *   - Work is enqueued asynchronously on `stream`; no function synchronises,
 *     allocates device memory or keeps state between calls (the library caches
 *     nothing but device properties).  Calls are thread-safe; two calls that
 *     share a workspace must be ordered by the caller.
 *   - Arguments are validated on the host before anything is launched; on
 *     error nothing is enqueued and a negative jssa_status is returned.
 *     A failed launch returns JSSA_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Alignment: q, k_cache, v_cache, k_new, M, kp, workspace and the
 *     calibration inputs q_cal, k_cal are 16-byte aligned (the kernels read
 *     them with 16-byte vector loads); every other device pointer is 4-byte
 *     aligned.  Allocations from hipMalloc or torch are.  A misaligned
 *     pointer returns JSSA_ERR_ALIGN before anything is launched.
 *   - Caller obligations that are NOT checked on the device: every
 *     block_table entry used (positions < seq_lens[b]) names a valid page;
 *     seq_lens[b] <= max_pages_per_seq * page_size (larger values are clamped);
 *     indices hold positions < seq_lens[b] or -1.
 *   - Positions are logical token positions within a sequence; a position t
 *     lives in page block_table[b][t / page_size], slot t % page_size.
 *
 * Shapes (GQA): q [batch, Hq, d]; k_cache, v_cache [num_pages, page, Hkv, d]
 * (one token's slice is contiguous over d, the standard paged GQA layout);
 * block_table int32 [batch, max_pages_per_seq]; seq_lens int32 [batch]
 * (N, including the token being decoded); M fp32 [Hkv, r, d].
 * Shapes (MLA, kind = JSSA_KIND_MLA): Hkv = 1, d = 576 = 512 latent + 64 RoPE;
 * q [batch, Hq, 576]; k_cache = latent cache [num_pages, page, 576];
 * M fp32 [r, 512] acting on the latent part; outputs have 512 dims.
 *
 * Projected scoring cache (written by jssa_store, read by jssa_select):
 *   kp       uint8 [num_pages, Hkv, S/16, page, 16]   (S = scoring dims:
 *            r for GQA, r + 64 for MLA; 16-byte pieces, piece-major inside
 *            one (page, KV head) block so a wavefront reads it contiguously)
 *   kp_scale [num_pages, Hkv, page], by jssa_shape.scale_format:
 *            JSSA_SCALE_FP32  fp32 scale (the default);
 *            JSSA_SCALE_E8M0  uint8 E with value 2^(E - 127) (one byte);
 *            JSSA_SCALE_NONE  no scale array (NULL), codes of y itself
 *   The element i of the projected key of (page p, slot s, head h) is
 *   kp[p][h][i/16][s][i%16] * scale(kp_scale[p][h][s]).  The one-byte and
 *   scale-free forms move the footprint toward the README page's r bytes per
 *   token and KV head ("Notes").
 *   JSSA_KEYS_BF16 (the README page's jssa_fp8_projk off: BF16 projected keys)
 *   stores y itself rounded to bf16, two bytes per element and no scale array
 *   (NULL): kp uint8 [num_pages, Hkv, 2S/16, page, 16], element i in the
 *   little-endian bytes 2i, 2i + 1 of the token's 2S bytes (the layout above
 *   with 2S one-byte elements).
 */
#ifndef JSSA_H_
#define JSSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JSSA_OK = 0,
  JSSA_ERR_NULL = -1,         /* a required pointer is NULL */
  JSSA_ERR_SHAPE = -2,        /* inconsistent sizes (e.g. Hq % Hkv != 0, budget <= 0) */
  JSSA_ERR_UNSUPPORTED = -3,  /* valid but not built (e.g. d not in {128, 256}) */
  JSSA_ERR_WORKSPACE = -4,    /* workspace smaller than jssa_workspace_bytes() */
  JSSA_ERR_HIP = -5,          /* a HIP launch or runtime call failed */
  JSSA_ERR_ALIGN = -6         /* a device pointer is not aligned as the conventions require */
} jssa_status;

enum { JSSA_KIND_GQA = 0, JSSA_KIND_MLA = 1 };

/* jssa_shape.select_mode: the selection strategy, and the path jssa_decode
 * takes.  Every mode returns the same index set and the same scores.
 *   AUTO          jssa_select: sampled threshold + candidate compaction in one
 *                 pass over the scoring cache, exact top-B of the candidates in
 *                 LDS; falls back to EXACT_STREAM per (sequence, KV head)
 *                 whenever the candidate set could miss a member of the top-B.
 *                 jssa_decode: the single-launch path (FUSED) when the shape
 *                 allows it, else SPLIT.
 *   EXACT_STREAM  per (sequence, KV head) radix select over recomputed scores
 *                 (several passes over the scoring cache; slow, data
 *                 independent); jssa_decode takes the split path.
 *   SPLIT         as AUTO, but jssa_decode always takes the split path: select
 *                 prologue, score stream and finish, then split-K attention and
 *                 merge (five launches per layer).
 *   FUSED         jssa_decode in one launch per layer (summary page §3.3: one
 *                 launch per layer): one block per (sequence, KV head) forms
 *                 qhat, stores the new token, scores every position exactly
 *                 into on-chip memory, selects the top-B and attends.  Only for
 *                 GQA with max_pages_per_seq * page_size <= 12288, rank <= 64
 *                 and G * head_dim <= 512; jssa_decode returns
 *                 JSSA_ERR_UNSUPPORTED for other shapes.  jssa_select treats
 *                 SPLIT and FUSED as AUTO. */
enum { JSSA_SELECT_AUTO = 0, JSSA_SELECT_EXACT_STREAM = 1, JSSA_SELECT_SPLIT = 2, JSSA_SELECT_FUSED = 3 };

/* jssa_shape.scale_format: the scoring cache's format, FP8 codes with a
 * per-(token, KV head) scale of one of three kinds, or BF16 keys. */
enum { JSSA_SCALE_FP32 = 0, JSSA_SCALE_E8M0 = 1, JSSA_SCALE_NONE = 2, JSSA_KEYS_BF16 = 3 };

typedef struct jssa_shape {
  int32_t kind;               /* JSSA_KIND_GQA or JSSA_KIND_MLA */
  int32_t batch;              /* sequences in the step, >= 1 */
  int32_t num_q_heads;        /* Hq; GQA: Hq % Hkv == 0, G = Hq/Hkv in {1,2,4,8}; MLA: multiple of 32, <= 128 */
  int32_t num_kv_heads;       /* Hkv; MLA: 1 */
  int32_t head_dim;           /* d: GQA 128 or 256; MLA 576 */
  int32_t page_size;          /* tokens per page: 16, 32 or 64 */
  int32_t max_pages_per_seq;  /* row stride of block_table */
  int32_t rank;               /* r: GQA r % 16 == 0, r <= min(d, 128); MLA latent rank, 64 */
  int32_t budget;             /* B: 1..4096 */
  int32_t select_mode;        /* JSSA_SELECT_AUTO, _EXACT_STREAM, _SPLIT or _FUSED */
  int32_t scale_format;       /* JSSA_SCALE_FP32 (0), JSSA_SCALE_E8M0, JSSA_SCALE_NONE or JSSA_KEYS_BF16 */
} jssa_shape;

/* Human-readable name of a jssa_status value (static string, never NULL). */
const char* jssa_status_string(int32_t status);

/* Bytes of device workspace that jssa_select / jssa_attend / jssa_decode /
 * jssa_full_decode need for this shape (all positions < max_pages_per_seq *
 * page_size).  Writes *bytes; returns a jssa_status. */
int32_t jssa_workspace_bytes(const jssa_shape* shape, size_t* bytes);

/* Whether jssa_decode with this shape runs as one launch per layer (*single = 1:
 * JSSA_SELECT_FUSED, or JSSA_SELECT_AUTO on a shape the single launch covers)
 * or through the split path (*single = 0).  Returns JSSA_ERR_UNSUPPORTED for
 * JSSA_SELECT_FUSED on a shape the single launch does not cover, as
 * jssa_decode would. */
int32_t jssa_decode_path(const jssa_shape* shape, int32_t* single);

/* Split-K plan of one attention call of this shape (the summary page's §3.3
 * Gather-Free Indexed Attention splits a head's positions over several
 * workgroups whose partial results are merged by log-sum-exp): *splits is the
 * number of position ranges jssa_attend (sparse != 0) or jssa_full_decode
 * with this window (sparse == 0; window 0 = every position) uses per
 * (sequence, KV head), and *capacity the number the workspace of
 * jssa_workspace_bytes holds; *splits <= *capacity for every window.
 * Returns JSSA_ERR_NULL for a NULL output, JSSA_ERR_SHAPE for window < 0 and
 * the shape's own validation status otherwise.  Launches nothing. */
int32_t jssa_attend_splits(const jssa_shape* shape, int32_t sparse, int32_t window, int32_t* splits,
                           int32_t* capacity);

/* Bytes of the projected scoring cache per page (kp) and scale elements per
 * page (kp_scale: fp32 for JSSA_SCALE_FP32, bytes for JSSA_SCALE_E8M0, 0 for
 * JSSA_SCALE_NONE and JSSA_KEYS_BF16), so callers can size both buffers. */
int32_t jssa_kp_page_bytes(const jssa_shape* shape, int64_t* kp_bytes_per_page,
                           int64_t* scale_elems_per_page);

/* jssa_store — project new keys with M and append them, FP8-quantised, to the
 * scoring cache (summary page §3.4: K_proj = K M^T, kept in FP8).
 *   GQA: y = M_h k (fp32 accumulate); MLA: y = [M c ; k_pe] (128 dims).
 *   scale = max_i |y_i| / 448 (fp32), codes = E4M3FN(y / scale), round to
 *   nearest even, saturating; an all-zero y stores scale 0 and zero codes.
 *   JSSA_SCALE_E8M0: the scale is rounded up to a power of two 2^e (e = ceil
 *   log2 of the fp32 scale, clamped to [-127, 127]; stored byte e + 127, 0 for
 *   a zero row) and codes = E4M3FN(y / 2^e); JSSA_SCALE_NONE: codes = E4M3FN(y);
 *   JSSA_KEYS_BF16: y rounded to bf16 (nearest, ties to even), no scale.
 * k_new : GQA bf16 [T, Hkv, d]; MLA bf16 [T, 576]
 * slot  : int32 [T], physical page * page_size + slot in page; < 0 skips the row
 * T = 0 returns JSSA_OK at once (no pointer is read, nothing is launched); T < 0 is JSSA_ERR_SHAPE.
 * M     : GQA fp32 [Hkv, r, d]; MLA fp32 [r, 512]
 * kp, kp_scale : the scoring cache (layout above), written at the slots only
 *                (kp_scale may be NULL with JSSA_SCALE_NONE or JSSA_KEYS_BF16). */
int32_t jssa_store(const jssa_shape* shape, const uint16_t* k_new, const int32_t* slot, int32_t T,
                   const float* M, uint8_t* kp, void* kp_scale, hipStream_t stream);

/* jssa_select — per (sequence b, KV head h): qbar = mean of the G query heads
 * of h (heads h*G .. h*G+G-1), qhat = M_h qbar (fp32; MLA: [M qbar[:512];
 * qbar[512:]]), score s_t = scale_t * sum_i qhat_i * kp_t,i (fp32) for
 * every position t < seq_lens[b], then the min(B, N) positions with the
 * largest score (summary page §3.1 steps 1-2, Eq. 1).  Ties at the B-th
 * score go to the lowest position; -0 counts as +0.
 * indices   : out int32 [batch, Hkv, B], ascending positions, -1 padded
 * scores_out: optional out fp32 [batch, Hkv, max_pages_per_seq*page] (NULL: not
 *             written); positions >= seq_lens[b] are left untouched. */
int32_t jssa_select(const jssa_shape* shape, const uint16_t* q, const float* M, const uint8_t* kp,
                    const void* kp_scale, const int32_t* block_table, const int32_t* seq_lens,
                    int32_t* indices, float* scores_out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* jssa_select_stages — the three phases of jssa_select, for callers that time
 * or interleave them: JSSA_STAGE_PROLOGUE (qhat and the sampled threshold),
 * JSSA_STAGE_STREAM (FP8 score stream over every cached token + candidate
 * compaction), JSSA_STAGE_FINISH (exact top-B from the candidates, or the
 * exact re-scoring fallback).  `stages` is a bit mask; phases run in that
 * order, and a phase reads what the previous phase left in `workspace`, so
 * one jssa_select equals PROLOGUE, STREAM, FINISH issued in order on one
 * stream with the same arguments.  Other arguments as jssa_select. */
enum { JSSA_STAGE_PROLOGUE = 1, JSSA_STAGE_STREAM = 2, JSSA_STAGE_FINISH = 4, JSSA_STAGE_ALL = 7 };
int32_t jssa_select_stages(const jssa_shape* shape, int32_t stages, const uint16_t* q, const float* M,
                           const uint8_t* kp, const void* kp_scale, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t* indices, float* scores_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* jssa_attend — gather-free indexed attention (summary page §3.3): query head
 * j attends, with exact softmax, over the positions that its KV head h = j/G
 * selected, reading K/V rows in place through the block table.  Logits are
 * sm_scale * q_j . k_t; out = sum softmax * v_t.  GQA out bf16 [batch, Hq, d];
 * MLA keys are the 576-dim latent rows, values their first 512 dims, out bf16
 * [batch, Hq, 512] (v_cache ignored, may be NULL).  lse_out (optional, fp32
 * [batch, Hq], natural log) receives log sum exp of the logits.  An empty set
 * gives out = 0 and lse = -inf.
 * indices : int32 [batch, Hkv, B] as written by jssa_select; an entry outside
 *           [0, seq_lens[b]) (such as the -1 padding) is skipped, so a bad
 *           index drops a position instead of reading outside the caches. */
int32_t jssa_attend(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                    const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* indices, float sm_scale, uint16_t* out, float* lse_out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* jssa_attend_noalloc — jssa_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results, with no workspace.  The
 * split-K partials go to a device array inside the library, 64 MiB per GPU,
 * which each GPU the library runs on holds until the process ends; the call
 * itself allocates nothing.
 * Returns JSSA_ERR_WORKSPACE when the shape's partials exceed that array
 * (batch * Hq * splits * partials per split * (d_v + 2) floats; about 4 MiB at
 * batch 8, 32 query heads, d = 128, 128K context), JSSA_ERR_HIP when the array
 * cannot be located on the current device.  Every call on one GPU uses the
 * same array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. */
int32_t jssa_attend_noalloc(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* indices, float sm_scale, uint16_t* out, float* lse_out,
                            hipStream_t stream);

/* jssa_decode — one decode step: [jssa_store of k_new at slot_new, skipped when
 * k_new is NULL] -> jssa_select -> jssa_attend, all on `stream`.  k_new holds
 * one new key per sequence (T = batch), i.e. the token at position
 * seq_lens[b]-1, so the token being decoded is itself eligible for selection.
 * The results equal those of the three calls; shape->select_mode picks the
 * split path (five launches) or the single-launch one (see JSSA_SELECT_FUSED). */
int32_t jssa_decode(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_new,
                    const int32_t* slot_new, const float* M, uint8_t* kp, void* kp_scale,
                    const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* block_table,
                    const int32_t* seq_lens, int32_t* indices, float sm_scale, uint16_t* out,
                    float* lse_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* jssa_full_decode — the dense baseline (README page §3, "Full-KV" decode):
 * the same attention over every position t < N (window == 0) or over the
 * last `window` positions [N - window, N) (window > 0: sliding-window layers,
 * which keep dense attention).  MLA: keys are the 576-dim latent rows, values
 * their first 512 dims (as in jssa_attend); out bf16 [batch, Hq, 512],
 * v_cache ignored. */
int32_t jssa_full_decode(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                         int32_t window, float sm_scale, uint16_t* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* jssa_gather_attend — the gather-then-attend baseline that gather-free indexed
 * attention replaces (summary page §3.3 and "Ablation Studies", Figure 6;
 * README page "4. vLLM configuration reference": indexed attention off).  Same
 * arguments and result as jssa_attend: the selected K/V rows of every (sequence,
 * KV head) are first copied into a staging cache inside the workspace (slot i of
 * head h holds that head's i-th selected position, with an identity block
 * table), then the dense attention of jssa_full_decode runs over the first
 * min(N, B) staged slots.  indices must be as jssa_select writes them (the -1
 * entries only as trailing padding); a -1 inside the first min(N, B) entries is
 * staged as a zero row and takes part in the softmax.  The workspace from
 * jssa_workspace_bytes includes the staging cache (batch * ceil(B/page) * page
 * rows of K and V per KV head). */
int32_t jssa_gather_attend(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                           const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* indices, float sm_scale, uint16_t* out, float* lse_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* jssa_calib_moments — calibration second moments (summary page §3.2; README
 * page §2): ADDS sum_t qbar_t qbar_t^T to gq and sum_t k_t k_t^T to gk (fp32,
 * [Hkv, dm, dm]; dm = d, MLA dm = 512 over the latent dims), so a long
 * calibration set can be streamed in chunks; the caller zero-initialises gq, gk.
 * The 1/T of the second moment is left out: the basis normalises each moment
 * to unit trace, which cancels it.
 * q_cal : bf16 [T, Hq, d] (MLA [T, Hq, 576]); k_cal : bf16 [T, Hkv, d] (MLA [T, 576]).
 * workspace: at least jssa_calib_workspace_bytes(shape, T) bytes (fp32 staging). */
int32_t jssa_calib_workspace_bytes(const jssa_shape* shape, int32_t T, size_t* bytes);
int32_t jssa_calib_moments(const jssa_shape* shape, const uint16_t* q_cal, const uint16_t* k_cal,
                           int32_t T, float* gq, float* gk, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* jssa_basis — HOST function: M* = TopEig_r(G~_Qbar + G~_K)^T (summary page
 * Eq. 5), each moment normalised to unit trace, per KV head, eigenvectors as
 * rows in descending eigenvalue order, each row's largest-magnitude entry made
 * positive.  gq, gk: HOST fp32 [Hkv, dm, dm] (dm = d, MLA 512), as summed by
 * jssa_calib_moments; M_out: HOST fp32 [Hkv, r, dm].  Symmetric eigensolver in
 * double precision (Householder tridiagonalisation + implicit QL). */
int32_t jssa_basis(const jssa_shape* shape, const float* gq, const float* gk, float* M_out);

#ifdef __cplusplus
}
#endif

#endif /* JSSA_H_ */
