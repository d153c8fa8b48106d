// Gather-then-attend, the baseline that gather-free indexed attention avoids
// (paper summary page, §3.3 Gather-Free Indexed Attention and "Ablation
// Studies", Figure 6: selected rows are first copied into a contiguous staging
// buffer, then a dense attention kernel runs over it; README page "4. vLLM
// configuration reference": the indexed attention switched off).
//
// gather_kernel copies, for every (sequence b, KV head h), the K and V rows of
// the positions indices[b, h, i] into staging slot (b * pages_per_seq + i / P) * P
// + i % P, head h, of a staging cache laid out like the paged cache
// ([pages, P, Hkv, d]; MLA: latent rows [pages, P, 576]).  Each head keeps its
// own selection at the same slot index i, so a dense attention over slots
// [0, n_sel) with the identity block table (also written here, with the staged
// lengths n_sel = min(N, B)) attends exactly to each head's own set.
//
// Block = (chunk of 64 selected positions, KV head, sequence), 256 threads:
// the chunk's source slots are resolved into LDS, then the rows are copied in
// 16-byte pieces, consecutive threads on consecutive pieces of a row.
#include "common.h"
#include "kernels.h"

namespace jssa {

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  __shared__ int src[64];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = (int)threadIdx.x;
  int N = a.seq_lens[b];
  const int cap = a.max_pages * a.P;
  N = N < 0 ? 0 : (N > cap ? cap : N);
  const int n_sel = N < a.B ? N : a.B;
  if (chunk == 0 && h == 0 && tid == 0) a.stage_lens[b] = n_sel;
  if (h == 0 && tid < 64)                                // identity block table of the staging cache
    for (int p = chunk * 64 + tid; p < a.stage_pages; p += 64 * (int)gridDim.x)
      a.stage_table[(int64_t)b * a.stage_pages + p] = b * a.stage_pages + p;
  const int i0 = chunk * 64;
  if (i0 >= n_sel) return;
  const int n = min(64, n_sel - i0);
  if (tid < 64) {
    int s = -1;
    if (tid < n) {
      const int t = a.indices[((int64_t)b * a.Hkv + h) * a.B + i0 + tid];
      if (t >= 0 && t < N) s = a.block_table[(int64_t)b * a.max_pages + t / a.P] * a.P + t % a.P;
    }
    src[tid] = s;
  }
  __syncthreads();
  const int E = a.row_elems / 8;                         // 16-byte pieces per row
  const int64_t row_stride = (int64_t)a.Hkv * a.row_elems;
  for (int p = tid; p < n * E; p += 256) {
    const int i = p / E, e = p % E;
    const int s = src[i];
    const int dst_slot = (b * a.stage_pages + (i0 + i) / a.P) * a.P + (i0 + i) % a.P;
    const int64_t so = (int64_t)(s < 0 ? 0 : s) * row_stride + (int64_t)h * a.row_elems + e * 8;
    const int64_t dof = (int64_t)dst_slot * row_stride + (int64_t)h * a.row_elems + e * 8;
    uint4 kv = *reinterpret_cast<const uint4*>(a.k_cache + so);
    if (s < 0) kv = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(a.stage_k + dof) = kv;
    if (a.v_cache) {
      uint4 vv = *reinterpret_cast<const uint4*>(a.v_cache + so);
      if (s < 0) vv = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(a.stage_v + dof) = vv;
    }
  }
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int chunks = (a.B + 63) / 64;
  hipLaunchKernelGGL(gather_kernel, dim3(chunks, a.Hkv, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jssa
