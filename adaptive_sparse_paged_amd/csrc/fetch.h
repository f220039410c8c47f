// Copies of host-tier cache units from pinned host memory into their HBM
// slots (the fetch kernels and the one-launch resolve), and the launch that
// fetches and attends a step's misses beside the attention over its hits.
#pragma once

#include "common.h"

namespace sp {

constexpr int kUnitElems = 2 * kTile;   // one cache unit: K tile + V tile (8 KiB)

// A placed miss: its unit id (per request h * max_pages + p; pooled
// (b * Hkv + h) * max_pages + p) and its slot (per request, or in the pool).
struct MissRec {
  int32_t unit;
  int32_t slot;
};

// One wave copies one unit: 8 KiB read from pinned host memory
// (device-initiated, non-temporal) and written into the slot.
__device__ __forceinline__ void copy_unit(const uint16_t* __restrict__ src,
                                          uint16_t* __restrict__ dst) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const int lane = lane_id();
  u32x4 t[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) t[k] = __builtin_nontemporal_load(s + k * 64 + lane);
#pragma unroll
  for (int k = 0; k < 8; ++k) d[k * 64 + lane] = t[k];
}

// Host and slot addresses of a per-request miss of request b (C slots each)
// and of a pooled miss.
__device__ __forceinline__ void copy_request_miss(const uint16_t* __restrict__ host_kv,
                                                  uint16_t* __restrict__ cache_kv, int hkv,
                                                  int max_pages, int C, int b, MissRec m) {
  const int h = m.unit / max_pages, p = m.unit - (m.unit / max_pages) * max_pages;
  copy_unit(host_kv + (((int64_t)b * max_pages + p) * hkv + h) * kUnitElems,
            cache_kv + ((int64_t)b * C + m.slot) * kUnitElems);
}

__device__ __forceinline__ void copy_pooled_miss(const uint16_t* __restrict__ host_kv,
                                                 uint16_t* __restrict__ cache_kv, int hkv,
                                                 int max_pages, MissRec m) {
  const int per_req = hkv * max_pages;       // pooled ids fit in 31 bits
  const int b = m.unit / per_req, rest = m.unit - b * per_req;
  const int64_t h = rest / max_pages, p = rest - h * max_pages;
  copy_unit(host_kv + (((int64_t)b * max_pages + p) * hkv + h) * kUnitElems,
            cache_kv + (int64_t)m.slot * kUnitElems);
}

// The fetch of the per-unit miss lists with the attention over them, and
// sparse_decode_attn over (sel_counts, sel_pages, hit_phys) on cache_kv, in
// one launch (attn.hip).
void enqueue_fetch_attn(const sparse_dims* dims, const uint16_t* host_kv, uint16_t* cache_kv,
                        int64_t pool_slots, int32_t* step_counter, const uint16_t* q,
                        const int32_t* ctx_lens, const int32_t* sel_counts,
                        const int32_t* sel_pages, const int32_t* hit_phys,
                        const int32_t* miss_counts, const int32_t* miss_pages,
                        const int32_t* miss_phys, float scale, int wmax, float* part_o,
                        float* part_lse, float* miss_part_o, float* miss_part_lse,
                        hipStream_t stream);

}  // namespace sp
