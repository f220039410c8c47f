// Copies of host-tier cache units from pinned host memory into their HBM
// slots, shared by the fetch kernels and the kernel that runs the fetch beside
// the attention over the hits.
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

// Where the resolve left its placed misses.  Per request: misses [B][C] and
// counts [B].  Pooled: misses [P] and counts [1] = P (B = 1 here).
struct MissTable {
  const MissRec* misses;
  const int32_t* counts;
  int B;
  int C;
  bool pooled;
};

// Wave fw of FW copies the misses whose position in the concatenation of
// the requests' miss lists is fw, fw + FW, ...  The per-request counts are
// read 64 at a time in one vector load (lane i: request b0 + i), so with
// nothing to copy a wave leaves after one round trip.
__device__ __forceinline__ void fetch_misses(int fw, int FW, const uint16_t* __restrict__ host_kv,
                                             uint16_t* __restrict__ cache_kv, int hkv,
                                             int max_pages, const MissTable& t) {
  if (t.pooled) {
    const int P = t.counts[0];
    for (int i = fw; i < P; i += FW) copy_pooled_miss(host_kv, cache_kv, hkv, max_pages,
                                                      t.misses[i]);
    return;
  }
  const int lane = lane_id();
  int base = 0;                              // misses of the requests before b0, mod FW
  for (int b0 = 0; b0 < t.B; b0 += 64) {
    const int cnt = (b0 + lane < t.B) ? max(t.counts[b0 + lane], 0) : 0;
    const int incl = wave_incl_scan(cnt);
    unsigned long long busy = __ballot(cnt > 0);
    while (busy) {                           // the requests of this block with misses
      const int j = __ffsll((long long)busy) - 1;
      busy &= busy - 1;
      const int cb = __builtin_amdgcn_readlane(cnt, j);
      const int pre = __builtin_amdgcn_readlane(incl, j) - cb;     // before b0 + j in block
      const int bb = (int)(((int64_t)base + pre) % FW);
      const int b = b0 + j;
      for (int i = ((fw - bb) % FW + FW) % FW; i < cb; i += FW)
        copy_request_miss(host_kv, cache_kv, hkv, max_pages, t.C, b,
                          t.misses[(int64_t)b * t.C + i]);
    }
    base = (int)(((int64_t)base + __builtin_amdgcn_readlane(incl, 63)) % FW);
  }
}

// The fetch of `t` and sparse_decode_attn over (sel_counts, sel_pages,
// hit_phys) on cache_kv, in one launch (attn.hip).
void enqueue_fetch_attn(const sparse_dims* dims, const uint16_t* host_kv, uint16_t* cache_kv,
                        int64_t pool_slots, const MissTable& t, int32_t* step_counter,
                        const uint16_t* q, const int32_t* ctx_lens, const int32_t* sel_counts,
                        const int32_t* sel_pages, const int32_t* hit_phys, float scale, int wmax,
                        float* part_o, float* part_lse, hipStream_t stream);

}  // namespace sp
