// Attention and its merge in one call: the self-planning split-K attention
// over the page lists and the log-sum-exp merge of its per-segment partials
// ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
// Hierarchy", MOIRA abstract, sentence on self-planning attention).  The
// partials pass through a caller workspace; the same kernels as
// sparse_decode_attn followed by sparse_merge_splits.

#include "common.h"

extern "C" sparse_status sparse_decode_attn_merge(
    const sparse_dims* dims, const uint16_t* q, const uint16_t* kv, int64_t stride_page,
    int64_t stride_head, int64_t pool_pages, const int32_t* ctx_lens, const int32_t* sel_counts,
    const int32_t* sel_pages, const int32_t* sel_phys, float scale, int32_t workers,
    float* part_o, float* part_lse, int64_t max_parts, float* out, float* out_lse,
    void* stream) {
  int wmax = 0;
  sparse_status st = sp::check_attn(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens,
                                    sel_counts, sel_pages, sel_phys, scale, workers, wmax);
  if (st != SPARSE_OK) return st;
  if (!part_o || !part_lse || !sp::aligned(part_o, 16)) return SPARSE_ERR_INVALID;
  if (max_parts != (int64_t)dims->batch * dims->num_kv_heads + wmax) return SPARSE_ERR_INVALID;
  if (!out || !out_lse || !sp::aligned(out, 16)) return SPARSE_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  sp::enqueue_attn(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens, sel_counts,
                   sel_pages, sel_phys, scale, wmax, part_o, part_lse, s);
  sp::enqueue_merge(dims, part_o, part_lse, sel_counts, wmax, out, out_lse, s);
  return sp::launch_status();
}
