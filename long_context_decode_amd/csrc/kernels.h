// Internal interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jssa {

constexpr int kCandCap = 12288;       // candidates the finish kernel holds in LDS per (sequence, KV head)
constexpr int kSampleMax = 8192;      // sampled tokens per (sequence, KV head)
constexpr int kMaxChunks = 8192;      // stream chunks per sequence the finish kernel can order
constexpr int kRegionPad = 16;        // a candidate region holds one chunk's tokens plus one 128-byte line
constexpr int kStreamWaves = 4;       // wavefronts of a score-stream block
constexpr int kMlaLatent = 512;
constexpr int kMlaRope = 64;

struct StoreArgs {
  const uint16_t* k_new;
  const int32_t* slot;
  const float* M;
  uint8_t* kp;
  void* kp_scale;          // fp32 / E8M0 bytes / unused, by sfmt
  int T, Hkv, P, d, r, S, mla;
  int sfmt;                // 0 fp32 scale, 1 E8M0 byte, 2 none
};

struct SelectArgs {
  const uint16_t* q;
  const float* M;
  const uint8_t* kp;
  const void* kp_scale;    // fp32 / E8M0 bytes / unused, by sfmt
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t* indices;
  float* scores_out;
  // workspace
  float* qhat;          // [batch, Hkv, S]
  uint32_t* tau;        // [batch, Hkv]
  uint2* cand;          // [batch, Hkv, max_chunks, reg_len]: per chunk a header entry (x = count), then
                        // the chunk's (key, position) candidates in position order
  int reg_len;          // entries per region: cp * P + kRegionPad
  // new-token store fused into the prologue (k_new == NULL: none)
  const uint16_t* k_new;
  const int32_t* slot_new;
  int batch, Hq, Hkv, d, P, max_pages, r, S, B, G, mla;
  int cp;               // pages per stream chunk: the pages one wavefront scores (16 / pieces rounds of 64 / P)
  int max_chunks;
  int heads_pb, chunks_pb;  // stream block: wavefront w scores KV head w % heads_pb of the block's head
                            // group over chunk w / heads_pb of its chunk group (heads_pb * chunks_pb <= 4)
  int force_exact;
  int sfmt;             // 0 fp32 scale, 1 E8M0 byte, 2 none
};

struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* indices;  // NULL: dense positions [lo, N)
  float* part_o;           // [batch, Hq, splits * parts, dv]
  float* part_ml;          // [batch, Hq, splits * parts, 2]  (running max in log2 units, sum)
  uint16_t* out;           // [batch, Hq, dv]
  float* lse_out;          // [batch, Hq] or NULL
  float sm_log2;           // sm_scale * log2(e)
  int batch, Hq, Hkv, P, max_pages, B, G, window;
  int splits, split_len;
  int parts;               // partials per split: 4 (one per wavefront, GQA) or 1 (MLA)
};

// jssa_decode in one launch (fused.hip): one block per (sequence, KV head)
constexpr int kFusedMaxB = 4096;      // selected positions the block holds in LDS

struct FusedArgs {
  const uint16_t* q;
  const uint16_t* k_new;   // NULL: no new token
  const int32_t* slot_new;
  const float* M;
  uint8_t* kp;
  void* kp_scale;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t* indices;
  uint16_t* out;
  float* lse_out;
  float sm_log2;
  int batch, Hq, Hkv, d, P, max_pages, r, S, B, G;
  int sfmt;
};

struct GatherArgs {
  const uint16_t* k_cache;
  const uint16_t* v_cache;   // NULL for MLA (one latent row)
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* indices;    // [batch, Hkv, B]
  uint16_t* stage_k;         // staging cache [batch * stage_pages, P, Hkv, row_elems]
  uint16_t* stage_v;
  int32_t* stage_table;      // [batch, stage_pages] identity block table
  int32_t* stage_lens;       // [batch] min(N, B)
  int batch, Hkv, P, max_pages, B, row_elems, stage_pages;
};

struct CalibArgs {
  const uint16_t* q;
  const uint16_t* k;
  float* gq;
  float* gk;
  float* xq;               // workspace: fp32 qbar rows [Hkv, T, dm]
  float* xk;               // workspace: fp32 key rows  [Hkv, T, dm]
  int T, Hq, Hkv, d, dm, G, mla;
};

hipError_t launch_store(const StoreArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int stages, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, int head_dim, hipStream_t s);
hipError_t launch_mla_attend(const AttendArgs& a, hipStream_t s);
hipError_t launch_merge(const AttendArgs& a, int dv, hipStream_t s);
// the partials scratch of jssa_attend_noalloc: a file-scope device array of
// kAttendScratchBytes, one per GPU; *ptr = its address on the current device
constexpr size_t kAttendScratchBytes = (size_t)64 << 20;
hipError_t attend_scratch(void** ptr);
hipError_t launch_calib(const CalibArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_fused(const FusedArgs& a, hipStream_t s);
// whether the single-launch decode handles this shape (capacity = max_pages * P)
bool fused_applies(int mla, int d, int G, int r, int64_t capacity, int B);

// host: per-head top-r eigenvectors of the unit-trace-normalised moment sum
int32_t basis_impl(int hkv, int n, int r, const float* gq, const float* gk, float* m_out);

}  // namespace jssa
