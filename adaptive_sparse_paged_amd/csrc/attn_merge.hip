// Attention and its merge in one call: the self-planning split-K attention
// over the page lists and the log-sum-exp merge of its per-segment partials
// ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
// Hierarchy", MOIRA abstract, sentence on self-planning attention).  The
// partials pass through a caller workspace; the same kernels as
// sparse_decode_attn followed by sparse_merge_splits.

#include "common.h"

#include <mutex>

namespace sp {

// The partials of sparse_decode_attn_merge_noalloc: one array per device,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: every host use goes through the device
// address that scratch_ptr() resolves with hipGetSymbolAddress.
constexpr size_t kNoAllocBytes = SPARSE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device: resolved on the first
// call made with that device current, then kept (one address per device).
// Returns nullptr when the device or the symbol cannot be queried.
static void* scratch_ptr() {
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace sp

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

extern "C" sparse_status sparse_decode_attn_merge_noalloc(
    const sparse_dims* dims, const uint16_t* q, const uint16_t* kv, int64_t stride_page,
    int64_t stride_head, int64_t pool_pages, const int32_t* ctx_lens, const int32_t* sel_counts,
    const int32_t* sel_pages, const int32_t* sel_phys, float scale, int32_t workers, float* out,
    float* out_lse, void* stream) {
  int wmax = 0;
  sparse_status st = sp::check_attn(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens,
                                    sel_counts, sel_pages, sel_phys, scale, workers, wmax);
  if (st != SPARSE_OK) return st;
  if (!out || !out_lse || !sp::aligned(out, 16)) return SPARSE_ERR_INVALID;
  const int group = dims->num_q_heads / dims->num_kv_heads;
  const int64_t parts = (int64_t)dims->batch * dims->num_kv_heads + wmax;
  if ((uint64_t)parts * group * (sp::kD + 1) * sizeof(float) > sp::kNoAllocBytes)
    return SPARSE_ERR_WORKSPACE;
  float* part_o = static_cast<float*>(sp::scratch_ptr());
  if (!part_o) return SPARSE_ERR_HIP;
  float* part_lse = part_o + parts * group * sp::kD;
  hipStream_t s = (hipStream_t)stream;
  sp::enqueue_attn(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens, sel_counts,
                   sel_pages, sel_phys, scale, wmax, part_o, part_lse, s);
  sp::enqueue_merge(dims, part_o, part_lse, sel_counts, wmax, out, out_lse, s);
  return sp::launch_status();
}
