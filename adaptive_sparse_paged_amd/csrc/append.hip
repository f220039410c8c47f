// Decode-time append: the step's new token enters its page and that page's
// per-channel key summary is refreshed, so the next scoring sees it.  The
// pages fix the step as "per request, layer, KV head and step" ("Adaptive
// DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", MOIRA
// abstract, coverage-rule sentence); writing the current token before the
// step is the usual decode order.
//
// One 256-thread workgroup per request; wave w handles KV heads w, w+4, ...
// Lane l owns channels 2l and 2l+1: one 4-byte store of the K row, two 2-byte
// stores into the channel-major V tile, and an order-key min/max update of
// the summary (the same total order, -0 below +0, as the summary builder).

#include "common.h"

namespace sp {

__device__ __forceinline__ uint32_t okey(uint32_t b) {
  return (b & 0x8000u) ? (0xFFFFu - b) : (b | 0x8000u);
}
__device__ __forceinline__ uint32_t okey_bits(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7FFFu) : (0xFFFFu - k);
}

__global__ __launch_bounds__(256) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ kv, int64_t stride_page, int64_t stride_head, int64_t pool_pages,
    const int32_t* __restrict__ page_table, int32_t* __restrict__ ctx_lens,
    uint16_t* __restrict__ summ, int hkv, int max_pages) {
  __shared__ int s_ok;
  const int b = blockIdx.x;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int L = ctx_lens[b];
  const int p = L / kP, t = L - (L / kP) * kP;
  int x = -1;
  if (L >= 0 && p < max_pages) x = page_table[(int64_t)b * max_pages + p];
  const bool ok = (x >= 0) && (x < pool_pages);
  if (ok) {
    for (int h = wv; h < hkv; h += 4) {
      const int64_t src = ((int64_t)b * hkv + h) * kD;
      const uint32_t kw = reinterpret_cast<const uint32_t*>(k_new + src)[lane];
      const uint32_t vw = reinterpret_cast<const uint32_t*>(v_new + src)[lane];
      uint16_t* kt = kv + (int64_t)x * stride_page + (int64_t)h * stride_head;
      uint16_t* vt = kt + kTile;
      reinterpret_cast<uint32_t*>(kt + t * kD)[lane] = kw;       // K row t
      vt[(2 * lane) * kP + t] = (uint16_t)(vw & 0xFFFFu);        // V column t
      vt[(2 * lane + 1) * kP + t] = (uint16_t)(vw >> 16);
      uint32_t* sm = reinterpret_cast<uint32_t*>(summ + ((int64_t)x * hkv + h) * (2 * kD));
      uint32_t lo = kw, hi = kw;
      if (t > 0) {
        const uint32_t olo = sm[lane], ohi = sm[kD / 2 + lane];
        const uint32_t k0 = okey(kw & 0xFFFFu), k1 = okey(kw >> 16);
        lo = okey_bits(min(okey(olo & 0xFFFFu), k0)) | (okey_bits(min(okey(olo >> 16), k1)) << 16);
        hi = okey_bits(max(okey(ohi & 0xFFFFu), k0)) | (okey_bits(max(okey(ohi >> 16), k1)) << 16);
      }
      sm[lane] = lo;
      sm[kD / 2 + lane] = hi;
    }
  }
  if (threadIdx.x == 0) s_ok = ok ? 1 : 0;
  __syncthreads();   // every wave has read ctx_lens[b] before it advances
  if (threadIdx.x == 0 && s_ok) ctx_lens[b] = L + 1;
}

}  // namespace sp

extern "C" sparse_status sparse_append_tokens(const sparse_dims* dims, const uint16_t* k_new,
                                              const uint16_t* v_new, uint16_t* kv,
                                              int64_t stride_page, int64_t stride_head,
                                              int64_t pool_pages, const int32_t* page_table,
                                              int32_t* ctx_lens, uint16_t* summ, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if ((st = sp::check_pool(kv, stride_page, stride_head, pool_pages)) != SPARSE_OK) return st;
  if (!k_new || !v_new || !page_table || !ctx_lens || !summ) return SPARSE_ERR_INVALID;
  if (!sp::aligned(k_new, 4) || !sp::aligned(v_new, 4) || !sp::aligned(summ, 16))
    return SPARSE_ERR_INVALID;
  hipLaunchKernelGGL(sp::append_kernel, dim3(dims->batch), dim3(256), 0, (hipStream_t)stream,
                     k_new, v_new, kv, stride_page, stride_head, pool_pages, page_table,
                     ctx_lens, summ, dims->num_kv_heads, dims->max_pages);
  return sp::launch_status();
}
