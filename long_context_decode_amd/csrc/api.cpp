// C ABI of the JSSA decode path: host-side validation, launch planning and
// workspace layout.  Every check runs before anything is enqueued; kernels are
// launched asynchronously on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "jssa.h"
#include "kernels.h"

namespace jssa {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int kind, batch, Hq, Hkv, d, P, max_pages, r, S, B, G, mla, dv, sfmt;
  int64_t maxN;
  int cp, max_chunks, heads_pb, chunks_pb;
  int sp_splits, sp_len;     // sparse attention split plan
  int dn_splits, dn_len;     // dense (window 0) split plan
  int ml_splits, ml_len;     // MLA sparse attention split plan
  int md_splits, md_len;     // MLA dense (window 0) split plan
  int stage_pages;            // gather-then-attend staging cache: pages per sequence
  int split_cap;              // splits the workspace's partials hold per (sequence, query head)
  size_t off_qhat, off_tau, off_cand, off_part_o, off_part_ml;
  size_t off_stage_k, off_stage_v, off_stage_table, off_stage_lens, total;
};

// Split plan of the attention kernels: about 512 blocks of four wavefronts,
// each wavefront taking whole batches of 64 positions.
void split_plan(int64_t n_tok_max, int pairs, int* splits, int* len) {
  if (n_tok_max <= 0) {
    *splits = 1;
    *len = 256;
    return;
  }
  int64_t s = cdiv(512, std::max(pairs, 1));
  s = std::min<int64_t>(s, cdiv(n_tok_max, 256));
  s = std::max<int64_t>(1, std::min<int64_t>(s, 64));    // 4 partials per split, at most 256 per head
  const int64_t l = cdiv(cdiv(n_tok_max, s), 256) * 256;
  *len = (int)l;
  *splits = (int)cdiv(n_tok_max, l);
}

// MLA dense split plan: about 512 blocks of (split, 64 heads, sequence) (two
// per CU), at least 128 rows per split, at most 256 splits (the merge holds
// one split per thread), 64-row multiples.
void mla_dense_plan(int64_t n, int batch, int Hq, int* splits, int* len) {
  if (n <= 0) {
    *splits = 1;
    *len = 64;
    return;
  }
  int64_t sp = cdiv(512, (int64_t)batch * cdiv(Hq, 64));
  sp = std::max<int64_t>(1, std::min<int64_t>({sp, cdiv(n, 128), 256}));
  *len = (int)(cdiv(cdiv(n, sp), 64) * 64);
  *splits = (int)cdiv(n, *len);
}

// Most splits a plan of this shape can take, whatever the row count: the
// GQA plan takes at most min(cdiv(512, pairs), 64) splits, the MLA dense plan
// at most min(cdiv(512, batch * head blocks of 64), 256) and the MLA sparse
// plan at most min(cdiv(512, batch * head blocks of 32), 64).
int split_capacity(const Plan& p) {
  if (!p.mla) return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(512, (int64_t)p.batch * p.Hkv), 64));
  const int64_t dense = std::min<int64_t>(cdiv(512, (int64_t)p.batch * cdiv(p.Hq, 64)), 256);
  const int64_t sparse = std::min<int64_t>(cdiv(512, (int64_t)p.batch * std::max(1, p.Hq / 32)), 64);
  return (int)std::max<int64_t>(1, std::max(dense, sparse));
}

constexpr float kLog2e = 1.44269504088896340736f;

// formats without a scale array
bool scale_free(int sfmt) { return sfmt == JSSA_SCALE_NONE || sfmt == JSSA_KEYS_BF16; }

int32_t validate_shape(const jssa_shape* sh) {
  if (!sh) return JSSA_ERR_NULL;
  if (sh->kind != JSSA_KIND_GQA && sh->kind != JSSA_KIND_MLA) return JSSA_ERR_UNSUPPORTED;
  if (sh->batch < 1 || sh->num_q_heads < 1 || sh->num_kv_heads < 1 || sh->max_pages_per_seq < 1)
    return JSSA_ERR_SHAPE;
  if (sh->num_q_heads % sh->num_kv_heads != 0) return JSSA_ERR_SHAPE;
  if (sh->budget < 1 || sh->budget > 4096) return JSSA_ERR_SHAPE;
  if (sh->page_size != 16 && sh->page_size != 32 && sh->page_size != 64) return JSSA_ERR_UNSUPPORTED;
  if (sh->select_mode < JSSA_SELECT_AUTO || sh->select_mode > JSSA_SELECT_FUSED) return JSSA_ERR_SHAPE;
  if (sh->scale_format != JSSA_SCALE_FP32 && sh->scale_format != JSSA_SCALE_E8M0 &&
      sh->scale_format != JSSA_SCALE_NONE && sh->scale_format != JSSA_KEYS_BF16)
    return JSSA_ERR_UNSUPPORTED;
  if (sh->rank < 16 || sh->rank % 16 != 0) return JSSA_ERR_UNSUPPORTED;
  if (sh->kind == JSSA_KIND_GQA) {
    if (sh->head_dim != 128 && sh->head_dim != 256) return JSSA_ERR_UNSUPPORTED;
    const int g = sh->num_q_heads / sh->num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return JSSA_ERR_UNSUPPORTED;
    if (sh->rank > std::min(sh->head_dim, 128)) return JSSA_ERR_UNSUPPORTED;
  } else {
    if (sh->num_kv_heads != 1 || sh->head_dim != kMlaLatent + kMlaRope) return JSSA_ERR_UNSUPPORTED;
    if (sh->num_q_heads % 32 != 0 || sh->num_q_heads > 128) return JSSA_ERR_UNSUPPORTED;
    if (sh->rank > 64) return JSSA_ERR_UNSUPPORTED;
  }
  return JSSA_OK;
}

int32_t make_plan(const jssa_shape* sh, Plan* p) {
  const int32_t st = validate_shape(sh);
  if (st != JSSA_OK) return st;
  p->kind = sh->kind;
  p->mla = sh->kind == JSSA_KIND_MLA;
  p->sfmt = sh->scale_format;
  p->batch = sh->batch;
  p->Hq = sh->num_q_heads;
  p->Hkv = sh->num_kv_heads;
  p->d = sh->head_dim;
  p->P = sh->page_size;
  p->max_pages = sh->max_pages_per_seq;
  p->r = sh->rank;
  p->S = p->mla ? sh->rank + kMlaRope : sh->rank;
  p->B = sh->budget;
  p->G = p->Hq / p->Hkv;
  p->dv = p->mla ? kMlaLatent : p->d;
  p->maxN = (int64_t)p->max_pages * p->P;
  // stream chunk: the pages one wavefront scores for one KV head, 64 / P pages
  // per round and 16 / (16-byte pieces per token) rounds, in two passes for
  // tokens of 8 or more pieces
  const int pieces = (p->sfmt == JSSA_KEYS_BF16 ? 2 : 1) * (p->S / 16);
  p->cp = (64 / p->P) * std::max(1, 16 / pieces) * (pieces >= 8 ? 2 : 1);
  p->heads_pb = std::min(p->Hkv, kStreamWaves);
  p->chunks_pb = kStreamWaves / p->heads_pb;
  p->max_chunks = (int)cdiv(p->max_pages, p->cp);
  if (p->max_chunks > kMaxChunks) return JSSA_ERR_UNSUPPORTED;
  split_plan(std::min<int64_t>(p->B, p->maxN), p->batch * p->Hkv, &p->sp_splits, &p->sp_len);
  split_plan(p->maxN, p->batch * p->Hkv, &p->dn_splits, &p->dn_len);
  {
    // MLA: blocks of (split, 32 heads, sequence), about 512 in all (two per
    // CU), 32-row tiles
    const int64_t n = std::min<int64_t>(p->B, p->maxN);
    int64_t sp = cdiv(512, (int64_t)p->batch * std::max(1, p->Hq / 32));
    sp = std::max<int64_t>(1, std::min<int64_t>({sp, cdiv(n, 32), 64}));
    p->ml_len = (int)(cdiv(cdiv(n, sp), 32) * 32);
    p->ml_splits = (int)cdiv(n, p->ml_len);
    mla_dense_plan(p->maxN, p->batch, p->Hq, &p->md_splits, &p->md_len);
  }
  p->stage_pages = (int)cdiv(p->B, p->P);
  int st_splits, st_len;                    // dense attention over the staging cache
  if (p->mla) mla_dense_plan((int64_t)p->stage_pages * p->P, p->batch, p->Hq, &st_splits, &st_len);
  else split_plan((int64_t)p->stage_pages * p->P, p->batch * p->Hkv, &st_splits, &st_len);
  const size_t bh = (size_t)p->batch * p->Hkv;
  const size_t cand = bh * p->max_chunks * (size_t)(p->cp * p->P + kRegionPad);   // one region per stream chunk
  size_t off = 0;
  p->off_qhat = off;    off = align_up(off + bh * p->S * sizeof(float));
  p->off_tau = off;     off = align_up(off + bh * sizeof(uint32_t));
  p->off_cand = off;    off = align_up(off + cand * 2 * sizeof(uint32_t));
  // split-K partials: one per block for MLA, one per wavefront (4 per split)
  // for GQA.  Sized for the most splits any plan of this shape can take: a
  // window shorter than the capacity rounds its split length to fewer rows
  // than the full plan does and may therefore take more splits than it.
  p->split_cap = split_capacity(*p);
  const size_t parts = p->mla ? (size_t)p->split_cap : (size_t)p->split_cap * 4;
  const int most = p->mla ? std::max({p->ml_splits, p->md_splits, st_splits})
                          : std::max({p->sp_splits, p->dn_splits, st_splits});
  if (most > p->split_cap) return JSSA_ERR_UNSUPPORTED;   // cannot happen: split_capacity bounds every plan
  const size_t pj = (size_t)p->batch * p->Hq * parts;
  p->off_part_o = off;  off = align_up(off + pj * p->dv * sizeof(float));
  p->off_part_ml = off; off = align_up(off + pj * 2 * sizeof(float));
  const size_t stage_rows = (size_t)p->batch * p->stage_pages * p->P * p->Hkv;
  p->off_stage_k = off; off = align_up(off + stage_rows * p->d * sizeof(uint16_t));
  p->off_stage_v = off; off = align_up(off + (p->mla ? 0 : stage_rows * p->d * sizeof(uint16_t)));
  p->off_stage_table = off; off = align_up(off + (size_t)p->batch * p->stage_pages * sizeof(int32_t));
  p->off_stage_lens = off; off = align_up(off + (size_t)p->batch * sizeof(int32_t));
  p->total = off;
  return JSSA_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? JSSA_OK : JSSA_ERR_HIP; }

// The alignment conventions of the ABI (a NULL pointer passes): vector-read
// tensors on 16 bytes, every other device pointer on 4.
bool al(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
template <typename... T>
bool al16(const T*... p) { return (al(p, 16) && ...); }
template <typename... T>
bool al4(const T*... p) { return (al(p, 4) && ...); }

int32_t do_store(const Plan& p, const uint16_t* k_new, const int32_t* slot, int32_t T, const float* M,
                 uint8_t* kp, void* kp_scale, hipStream_t stream) {
  if (T < 0) return JSSA_ERR_SHAPE;
  if (T == 0) return JSSA_OK;
  if (!k_new || !slot || !M || !kp || (!kp_scale && !scale_free(p.sfmt))) return JSSA_ERR_NULL;
  if (!al16(k_new, M, kp) || !al4(slot, kp_scale)) return JSSA_ERR_ALIGN;
  StoreArgs a{};
  a.k_new = k_new;
  a.slot = slot;
  a.M = M;
  a.kp = kp;
  a.kp_scale = kp_scale;
  a.T = T;
  a.Hkv = p.Hkv;
  a.P = p.P;
  a.d = p.d;
  a.r = p.r;
  a.S = p.S;
  a.mla = p.mla;
  a.sfmt = p.sfmt;
  return hip_status(launch_store(a, stream));
}

int32_t do_select(const Plan& p, int select_mode, int stages, const uint16_t* q, const float* M, const uint8_t* kp,
                  const void* kp_scale, const int32_t* block_table, const int32_t* seq_lens, int32_t* indices,
                  float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream, const uint16_t* k_new = nullptr,
                  const int32_t* slot_new = nullptr) {
  if (!q || !M || !kp || (!kp_scale && !scale_free(p.sfmt)) || !block_table || !seq_lens || !indices || !ws)
    return JSSA_ERR_NULL;
  if (!al16(q, M, kp, ws, k_new) || !al4(kp_scale, block_table, seq_lens, indices, scores_out, slot_new))
    return JSSA_ERR_ALIGN;
  if (ws_bytes < p.total) return JSSA_ERR_WORKSPACE;
  SelectArgs a{};
  a.q = q;
  a.M = M;
  a.kp = kp;
  a.kp_scale = kp_scale;
  a.sfmt = p.sfmt;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.indices = indices;
  a.scores_out = scores_out;
  a.qhat = at<float>(ws, p.off_qhat);
  a.tau = at<uint32_t>(ws, p.off_tau);
  a.k_new = k_new;
  a.slot_new = slot_new;
  a.cand = at<uint2>(ws, p.off_cand);
  a.batch = p.batch;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.d = p.d;
  a.P = p.P;
  a.max_pages = p.max_pages;
  a.r = p.r;
  a.S = p.S;
  a.B = p.B;
  a.G = p.G;
  a.mla = p.mla;
  a.cp = p.cp;
  a.max_chunks = p.max_chunks;
  a.heads_pb = p.heads_pb;
  a.chunks_pb = p.chunks_pb;
  a.reg_len = p.cp * p.P + kRegionPad;
  a.force_exact = select_mode == JSSA_SELECT_EXACT_STREAM;
  return hip_status(launch_select(a, stages, stream));
}

// Split plan of one attention call: over the selected positions (sparse), all
// positions (window 0) or the last `window` positions.
void attend_plan(const Plan& p, bool sparse, int window, int* splits, int* len) {
  if (p.mla) {
    if (sparse) {
      *splits = p.ml_splits;
      *len = p.ml_len;
    } else if (window > 0) {
      mla_dense_plan(std::min<int64_t>(window, p.maxN), p.batch, p.Hq, splits, len);
    } else {
      *splits = p.md_splits;
      *len = p.md_len;
    }
    return;
  }
  if (sparse) {
    *splits = p.sp_splits;
    *len = p.sp_len;
  } else if (window > 0) {
    split_plan(std::min<int64_t>(window, p.maxN), p.batch * p.Hkv, splits, len);
  } else {
    *splits = p.dn_splits;
    *len = p.dn_len;
  }
}

// The attention launches with the split-K partials at part_o / part_ml
// (pointer checks done by the caller).
int32_t run_attend(const Plan& p, const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens, const int32_t* indices, int window,
                   float sm_scale, uint16_t* out, float* lse_out, float* part_o, float* part_ml,
                   hipStream_t stream) {
  AttendArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.indices = indices;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.out = out;
  a.lse_out = lse_out;
  a.sm_log2 = sm_scale * kLog2e;
  a.batch = p.batch;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.P = p.P;
  a.max_pages = p.max_pages;
  a.B = p.B;
  a.G = p.G;
  a.window = indices ? 0 : window;
  a.parts = p.mla ? 1 : 4;
  attend_plan(p, indices != nullptr, a.window, &a.splits, &a.split_len);
  if (a.splits > p.split_cap) return JSSA_ERR_UNSUPPORTED;    // cannot happen (split_capacity)
  if (p.mla) return hip_status(launch_mla_attend(a, stream));
  return hip_status(launch_attend(a, p.d, stream));
}

int32_t do_attend(const Plan& p, const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                  const int32_t* block_table, const int32_t* seq_lens, const int32_t* indices, int window,
                  float sm_scale, uint16_t* out, float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k_cache || (!v_cache && !p.mla) || !block_table || !seq_lens || !out || !ws) return JSSA_ERR_NULL;
  if (!al16(q, k_cache, v_cache, ws) || !al4(block_table, seq_lens, indices, out, lse_out)) return JSSA_ERR_ALIGN;
  if (ws_bytes < p.total) return JSSA_ERR_WORKSPACE;
  if (window < 0) return JSSA_ERR_SHAPE;
  return run_attend(p, q, k_cache, v_cache, block_table, seq_lens, indices, window, sm_scale, out, lse_out,
                    at<float>(ws, p.off_part_o), at<float>(ws, p.off_part_ml), stream);
}

}  // namespace
}  // namespace jssa

using namespace jssa;

extern "C" {

const char* jssa_status_string(int32_t status) {
  switch (status) {
    case JSSA_OK: return "ok";
    case JSSA_ERR_NULL: return "null pointer argument";
    case JSSA_ERR_SHAPE: return "inconsistent shape";
    case JSSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case JSSA_ERR_WORKSPACE: return "workspace too small";
    case JSSA_ERR_ALIGN: return "misaligned device pointer";
    case JSSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t jssa_workspace_bytes(const jssa_shape* shape, size_t* bytes) {
  if (!bytes) return JSSA_ERR_NULL;
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  *bytes = p.total;
  return JSSA_OK;
}

int32_t jssa_decode_path(const jssa_shape* shape, int32_t* single) {
  if (!single) return JSSA_ERR_NULL;
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  const bool fits = fused_applies(p.mla, p.d, p.G, p.r, p.maxN, p.B);
  if (shape->select_mode == JSSA_SELECT_FUSED && !fits) return JSSA_ERR_UNSUPPORTED;
  *single = (shape->select_mode == JSSA_SELECT_FUSED || (shape->select_mode == JSSA_SELECT_AUTO && fits)) ? 1 : 0;
  return JSSA_OK;
}

int32_t jssa_attend_splits(const jssa_shape* shape, int32_t sparse, int32_t window, int32_t* splits,
                           int32_t* capacity) {
  if (!splits || !capacity) return JSSA_ERR_NULL;
  if (window < 0) return JSSA_ERR_SHAPE;
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  int len = 0;
  attend_plan(p, sparse != 0, sparse ? 0 : window, splits, &len);
  *capacity = p.split_cap;
  return JSSA_OK;
}

int32_t jssa_kp_page_bytes(const jssa_shape* shape, int64_t* kp_bytes_per_page, int64_t* scale_elems_per_page) {
  if (!kp_bytes_per_page || !scale_elems_per_page) return JSSA_ERR_NULL;
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  *kp_bytes_per_page = (int64_t)p.Hkv * p.P * p.S * (p.sfmt == JSSA_KEYS_BF16 ? 2 : 1);
  *scale_elems_per_page = scale_free(p.sfmt) ? 0 : (int64_t)p.Hkv * p.P;
  return JSSA_OK;
}

int32_t jssa_store(const jssa_shape* shape, const uint16_t* k_new, const int32_t* slot, int32_t T, const float* M,
                   uint8_t* kp, void* kp_scale, hipStream_t stream) {
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  return do_store(p, k_new, slot, T, M, kp, kp_scale, stream);
}

int32_t jssa_select(const jssa_shape* shape, const uint16_t* q, const float* M, const uint8_t* kp,
                    const void* kp_scale, const int32_t* block_table, const int32_t* seq_lens, int32_t* indices,
                    float* scores_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  return do_select(p, shape->select_mode, JSSA_STAGE_ALL, q, M, kp, kp_scale, block_table, seq_lens, indices,
                   scores_out, workspace, workspace_bytes, stream);
}

int32_t jssa_select_stages(const jssa_shape* shape, int32_t stages, const uint16_t* q, const float* M,
                           const uint8_t* kp, const void* kp_scale, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t* indices, float* scores_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  if (stages < 0 || stages > JSSA_STAGE_ALL) return JSSA_ERR_SHAPE;
  return do_select(p, shape->select_mode, stages, q, M, kp, kp_scale, block_table, seq_lens, indices, scores_out,
                   workspace, workspace_bytes, stream);
}

int32_t jssa_attend(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* block_table, const int32_t* seq_lens, const int32_t* indices, float sm_scale,
                    uint16_t* out, float* lse_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  if (!indices) return JSSA_ERR_NULL;
  return do_attend(p, q, k_cache, v_cache, block_table, seq_lens, indices, 0, sm_scale, out, lse_out, workspace,
                   workspace_bytes, stream);
}

int32_t jssa_attend_noalloc(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* indices, float sm_scale, uint16_t* out, float* lse_out,
                            hipStream_t stream) {
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  if (!q || !k_cache || (!v_cache && !p.mla) || !block_table || !seq_lens || !indices || !out) return JSSA_ERR_NULL;
  if (!al16(q, k_cache, v_cache) || !al4(block_table, seq_lens, indices, out, lse_out)) return JSSA_ERR_ALIGN;
  // the partials of this call's split plan, laid out from the start of the
  // library's scratch array: o [batch, Hq, splits * parts, dv], then (m, l)
  int splits = 0, len = 0;
  attend_plan(p, true, 0, &splits, &len);
  const size_t parts = (size_t)p.batch * p.Hq * splits * (p.mla ? 1 : 4);
  const size_t o_bytes = align_up(parts * p.dv * sizeof(float));
  if (o_bytes + align_up(parts * 2 * sizeof(float)) > kAttendScratchBytes) return JSSA_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (attend_scratch(&scratch) != hipSuccess) return JSSA_ERR_HIP;
  return run_attend(p, q, k_cache, v_cache, block_table, seq_lens, indices, 0, sm_scale, out, lse_out,
                    static_cast<float*>(scratch), at<float>(scratch, o_bytes), stream);
}

int32_t jssa_decode(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_new, const int32_t* slot_new,
                    const float* M, uint8_t* kp, void* kp_scale, const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* block_table, const int32_t* seq_lens, int32_t* indices, float sm_scale,
                    uint16_t* out, float* lse_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  // validate everything before the first launch
  if (!q || !M || !kp || (!kp_scale && !scale_free(p.sfmt)) || !k_cache || !block_table || !seq_lens ||
      !indices || !out || !workspace)
    return JSSA_ERR_NULL;
  if (!p.mla && !v_cache) return JSSA_ERR_NULL;
  if (k_new && !slot_new) return JSSA_ERR_NULL;
  if (!al16(q, k_new, M, kp, k_cache, v_cache, workspace) ||
      !al4(slot_new, kp_scale, block_table, seq_lens, indices, out, lse_out))
    return JSSA_ERR_ALIGN;
  if (workspace_bytes < p.total) return JSSA_ERR_WORKSPACE;
  int32_t single = 0;
  st = jssa_decode_path(shape, &single);
  if (st != JSSA_OK) return st;
  if (single) {
    FusedArgs f{};
    f.q = q;
    f.k_new = k_new;
    f.slot_new = k_new ? slot_new : nullptr;
    f.M = M;
    f.kp = kp;
    f.kp_scale = kp_scale;
    f.k_cache = k_cache;
    f.v_cache = v_cache;
    f.block_table = block_table;
    f.seq_lens = seq_lens;
    f.indices = indices;
    f.out = out;
    f.lse_out = lse_out;
    f.sm_log2 = sm_scale * kLog2e;
    f.batch = p.batch;
    f.Hq = p.Hq;
    f.Hkv = p.Hkv;
    f.d = p.d;
    f.P = p.P;
    f.max_pages = p.max_pages;
    f.r = p.r;
    f.S = p.S;
    f.B = p.B;
    f.G = p.G;
    f.sfmt = p.sfmt;
    return hip_status(launch_fused(f, stream));
  }
  // the prologue of select stores the new token
  st = do_select(p, shape->select_mode, JSSA_STAGE_ALL, q, M, kp, kp_scale, block_table, seq_lens, indices, nullptr,
                 workspace, workspace_bytes, stream, k_new, k_new ? slot_new : nullptr);
  if (st != JSSA_OK) return st;
  return do_attend(p, q, k_cache, v_cache, block_table, seq_lens, indices, 0, sm_scale, out, lse_out, workspace,
                   workspace_bytes, stream);
}

int32_t jssa_full_decode(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens, int32_t window,
                         float sm_scale, uint16_t* out, float* lse_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  return do_attend(p, q, k_cache, v_cache, block_table, seq_lens, nullptr, window, sm_scale, out, lse_out, workspace,
                   workspace_bytes, stream);
}

int32_t jssa_gather_attend(const jssa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                           const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* indices, float sm_scale, uint16_t* out, float* lse_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  const int32_t st = make_plan(shape, &p);
  if (st != JSSA_OK) return st;
  if (!q || !k_cache || (!v_cache && !p.mla) || !block_table || !seq_lens || !indices || !out || !workspace)
    return JSSA_ERR_NULL;
  if (!al16(q, k_cache, v_cache, workspace) || !al4(block_table, seq_lens, indices, out, lse_out))
    return JSSA_ERR_ALIGN;
  if (workspace_bytes < p.total) return JSSA_ERR_WORKSPACE;
  GatherArgs g{};
  g.k_cache = k_cache;
  g.v_cache = p.mla ? nullptr : v_cache;
  g.block_table = block_table;
  g.seq_lens = seq_lens;
  g.indices = indices;
  g.stage_k = at<uint16_t>(workspace, p.off_stage_k);
  g.stage_v = p.mla ? nullptr : at<uint16_t>(workspace, p.off_stage_v);
  g.stage_table = at<int32_t>(workspace, p.off_stage_table);
  g.stage_lens = at<int32_t>(workspace, p.off_stage_lens);
  g.batch = p.batch;
  g.Hkv = p.Hkv;
  g.P = p.P;
  g.max_pages = p.max_pages;
  g.B = p.B;
  g.row_elems = p.d;
  g.stage_pages = p.stage_pages;
  hipError_t e = launch_gather(g, stream);
  if (e != hipSuccess) return JSSA_ERR_HIP;
  // dense attention over the staging cache: its own page count and split plans
  Plan ps = p;
  ps.max_pages = p.stage_pages;
  ps.maxN = (int64_t)p.stage_pages * p.P;
  split_plan(ps.maxN, p.batch * p.Hkv, &ps.dn_splits, &ps.dn_len);
  mla_dense_plan(ps.maxN, p.batch, p.Hq, &ps.md_splits, &ps.md_len);
  return do_attend(ps, q, g.stage_k, g.stage_v, g.stage_table, g.stage_lens, nullptr, 0, sm_scale, out, lse_out,
                   workspace, workspace_bytes, stream);
}

int32_t jssa_calib_workspace_bytes(const jssa_shape* shape, int32_t T, size_t* bytes) {
  if (!bytes) return JSSA_ERR_NULL;
  const int32_t st = validate_shape(shape);
  if (st != JSSA_OK) return st;
  if (T < 0) return JSSA_ERR_SHAPE;
  const int dm = shape->kind == JSSA_KIND_MLA ? kMlaLatent : shape->head_dim;
  *bytes = align_up((size_t)T * shape->num_kv_heads * dm * sizeof(float)) * 2;
  return JSSA_OK;
}

int32_t jssa_calib_moments(const jssa_shape* shape, const uint16_t* q_cal, const uint16_t* k_cal, int32_t T,
                           float* gq, float* gk, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  const int32_t st = jssa_calib_workspace_bytes(shape, T, &need);
  if (st != JSSA_OK) return st;
  if (T == 0) return JSSA_OK;
  if (!q_cal || !k_cal || !gq || !gk || !workspace) return JSSA_ERR_NULL;
  if (!al16(q_cal, k_cal, workspace) || !al4(gq, gk)) return JSSA_ERR_ALIGN;
  if (workspace_bytes < need) return JSSA_ERR_WORKSPACE;
  CalibArgs a{};
  a.q = q_cal;
  a.k = k_cal;
  a.gq = gq;
  a.gk = gk;
  a.T = T;
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.d = shape->head_dim;
  a.mla = shape->kind == JSSA_KIND_MLA;
  a.dm = a.mla ? kMlaLatent : a.d;
  a.G = a.Hq / a.Hkv;
  a.xq = static_cast<float*>(workspace);
  a.xk = at<float>(workspace, need / 2);
  return hip_status(launch_calib(a, stream));
}

int32_t jssa_basis(const jssa_shape* shape, const float* gq, const float* gk, float* M_out) {
  const int32_t st = validate_shape(shape);
  if (st != JSSA_OK) return st;
  if (!gq || !gk || !M_out) return JSSA_ERR_NULL;
  const int dm = shape->kind == JSSA_KIND_MLA ? kMlaLatent : shape->head_dim;
  if (shape->rank > dm) return JSSA_ERR_SHAPE;
  try {
    return basis_impl(shape->num_kv_heads, dm, shape->rank, gq, gk, M_out);
  } catch (...) {                        // allocation failure inside the solver
    return JSSA_ERR_UNSUPPORTED;
  }
}

}  // extern "C"
