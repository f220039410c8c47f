// Per-page per-channel key summaries (kmin, kmax) -- prefill/append time.
//
// The Quest-style summary: for each channel, the min and the max of the key
// over the page's valid tokens ("HiSparse: Scaling Sparse Attention Decoding
// with Hierarchical KV Cache", abstract: Quest is one of the evaluated
// sparse-attention families).  Bit-exact: comparisons run on an integer key
// that orders bf16 patterns numerically with -0 below +0.

#include "common.h"

namespace sp {

__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  return (b & 0x8000u) ? (0xFFFFu - b) : (b | 0x8000u);
}
__device__ __forceinline__ uint32_t key_bits(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7FFFu) : (0xFFFFu - k);
}

// One wave per (listed page, KV head); lane l owns channels 2l and 2l+1, so
// each token row of the tile is one coalesced 256-byte wave load, and the
// loads of all valid rows are issued before the first comparison.
__global__ __launch_bounds__(256) void summaries_kernel(
    const uint16_t* __restrict__ kv, int64_t stride_page, int64_t stride_head, int64_t pool_pages,
    const int32_t* __restrict__ pages, const int32_t* __restrict__ valid, int n, int hkv,
    uint16_t* __restrict__ summ) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (item >= n * hkv) return;
  const int i = item / hkv, h = item - (item / hkv) * hkv;
  // both ids in one round trip: the empty asm keeps the compiler from
  // issuing the second load only after the first one's test
  int x = pages[i], nv = valid[i];
  asm volatile("" : "+v"(x), "+v"(nv));
  nv = min(max(nv, 0), kP);
  if (x < 0 || x >= pool_pages || nv == 0) return;
  const uint32_t* tile =
      reinterpret_cast<const uint32_t*>(kv + (int64_t)x * stride_page + (int64_t)h * stride_head);
  uint32_t w[kP];
#pragma unroll
  for (int t = 0; t < kP; ++t)
    w[t] = (t < nv) ? __builtin_nontemporal_load(tile + t * (kD / 2) + lane) : 0u;
  uint32_t lo0 = 0xFFFFu, lo1 = 0xFFFFu, hi0 = 0u, hi1 = 0u;
#pragma unroll
  for (int t = 0; t < kP; ++t) {
    if (t >= nv) break;
    const uint32_t k0 = order_key(w[t] & 0xFFFFu), k1 = order_key(w[t] >> 16);
    lo0 = min(lo0, k0);
    hi0 = max(hi0, k0);
    lo1 = min(lo1, k1);
    hi1 = max(hi1, k1);
  }
  uint32_t* out = reinterpret_cast<uint32_t*>(summ + ((int64_t)x * hkv + h) * (2 * kD));
  out[lane] = key_bits(lo0) | (key_bits(lo1) << 16);
  out[kD / 2 + lane] = key_bits(hi0) | (key_bits(hi1) << 16);
}

}  // namespace sp

extern "C" sparse_status sparse_build_page_summaries(const sparse_dims* dims, const uint16_t* kv,
                                                     int64_t stride_page, int64_t stride_head,
                                                     int64_t pool_pages, const int32_t* pages,
                                                     const int32_t* valid, int32_t n,
                                                     uint16_t* summ, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if ((st = sp::check_pool(kv, stride_page, stride_head, pool_pages)) != SPARSE_OK) return st;
  if (n < 0) return SPARSE_ERR_INVALID;
  if (n == 0) return SPARSE_OK;
  if (!pages || !valid || !summ || !sp::aligned(summ, 16)) return SPARSE_ERR_INVALID;
  const int64_t items = (int64_t)n * dims->num_kv_heads;
  if (items > (int64_t)INT32_MAX - 4) return SPARSE_ERR_INVALID;
  const int blocks = (int)((items + 3) / 4);
  hipLaunchKernelGGL(sp::summaries_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, kv,
                     stride_page, stride_head, pool_pages, pages, valid, n, dims->num_kv_heads,
                     summ);
  return sp::launch_status();
}
