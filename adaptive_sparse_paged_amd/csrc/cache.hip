// Host-resident KV tier with a fixed-size HBM page cache, resolved inside the
// decode graph ("HiSparse: Scaling Sparse Attention Decoding with
// Hierarchical KV Cache", abstract: full KV history in host memory, a small
// fixed-size GPU cache per request, and one in-graph resolver doing hit
// detection, LRU replacement and host-to-device fetch; only placement changes,
// so outputs are unchanged).
//
// Cache unit = one (logical page p, KV head h) of a request: its K tile and
// channel-major V tile (8 KiB), unit id v = h * max_pages + p.  Rules:
//   * requested set R of a request = union of its KV heads' page lists;
//     resident units of R are hits and get the step as their stamp;
//   * misses, in ascending unit id, take slots in ascending slot index from
//     the available set: the lowest free slots if they suffice, otherwise all
//     free slots plus the r least recently used resident units outside R,
//     ordered by (stamp, unit id), r = misses - free;
//   * misses that find no slot (more distinct units than slots) get slot -1
//     and set the overflow flag.
// resolve_kernel: one 1024-thread workgroup per request (radix select of the
// victims on LDS histograms; block prefix sums for ranks).  fetch_kernel: one
// wave per missed unit copies its 8 KiB from pinned host memory into the slot
// (device-initiated reads over PCIe; no host involvement).

#include "common.h"

namespace sp {

constexpr int kResThreads = 1024;
constexpr int kMaxSlots = 8192;
constexpr int kUnitElems = 2 * kTile;   // K tile + V tile
constexpr int kMaxKvHeads = 64;

struct MissRec {
  int32_t unit;
  int32_t slot;
};

__global__ __launch_bounds__(kResThreads) void resolve_kernel(
    const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages, int hkv,
    int max_pages, int C, const int32_t* __restrict__ step_counter, int32_t* __restrict__ slot_tag,
    int32_t* __restrict__ slot_stamp, int32_t* __restrict__ unit_slot,
    int32_t* __restrict__ sel_phys, int32_t* __restrict__ stats, MissRec* __restrict__ misses,
    int32_t* __restrict__ miss_count) {
  __shared__ uint8_t req[kMaxSlots];       // slot holds a unit requested this step
  __shared__ int32_t avail[kMaxSlots];     // available slots, ascending
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan32[kResThreads / 64];
  __shared__ unsigned long long scan64[kResThreads / 64];
  __shared__ int32_t head_off[kMaxKvHeads + 1];
  __shared__ int s_bin;
  __shared__ uint32_t s_below;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int step = *step_counter;
  int32_t* tags = slot_tag + (int64_t)b * C;
  int32_t* stamps = slot_stamp + (int64_t)b * C;
  int32_t* umap = unit_slot + (int64_t)b * hkv * max_pages;

  for (int s = tid; s < C; s += kResThreads) req[s] = 0;
  if (tid == 0) {
    int acc = 0;
    for (int h = 0; h < hkv; ++h) {
      head_off[h] = acc;
      acc += min(max(sel_counts[b * hkv + h], 0), max_pages);
    }
    head_off[hkv] = acc;
  }
  __syncthreads();
  const int E = head_off[hkv];

  // ---- pass 1: hits (stamp, mark, slot id) and the number of misses ------
  // Elements e = tid + 1024 k, up to 8 per thread per batch, loads issued
  // together; only the totals are needed here (ranks come in pass 2).
  uint32_t M = 0u, H = 0u;
  {
    constexpr int kBatch = 8;
    uint32_t m_local = 0u, h_local = 0u;
    for (int base = 0; base < E; base += kBatch * kResThreads) {
      int64_t li[kBatch];
      int v[kBatch], s[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int e = base + k * kResThreads + tid;
        li[k] = -1;
        v[k] = -1;
        if (e < E) {
          int h = 0;
          while (e >= head_off[h + 1]) ++h;
          li[k] = (int64_t)(b * hkv + h) * max_pages + (e - head_off[h]);
          const int p = sel_pages[li[k]];
          if (p >= 0 && p < max_pages) v[k] = h * max_pages + p;
        }
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) s[k] = (v[k] >= 0) ? umap[v[k]] : -2;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (li[k] < 0) continue;
        int sk = s[k];
        if (sk >= C) sk = -2;                // corrupt state: never index past the cache
        if (sk >= 0) {
          ++h_local;
          req[sk] = 1;
          stamps[sk] = step;
          sel_phys[li[k]] = b * C + sk;
        } else if (sk == -1) {
          ++m_local;
        } else {
          sel_phys[li[k]] = -1;              // page id out of range: an empty page
        }
      }
    }
    unsigned long long tot;
    block_excl_scan<unsigned long long, kResThreads>(
        ((unsigned long long)h_local << 32) | m_local, scan64, tot);
    M = (uint32_t)tot;
    H = (uint32_t)(tot >> 32);
  }
  // (block_excl_scan ends with a barrier: every req mark is visible here)
  if (M == 0u) {                 // every requested unit is resident: nothing to place
    if (tid == 0) {
      stats[b * 4 + 0] = (int32_t)H;
      stats[b * 4 + 1] = 0;
      stats[b * 4 + 2] = 0;
      stats[b * 4 + 3] = 0;
      miss_count[b] = 0;
    }
    return;
  }

  // ---- free slots and victim candidates ----------------------------------
  constexpr int kSPT = kMaxSlots / kResThreads;   // slots per thread, strided
  uint32_t nfree = 0u, ncand = 0u;
  for (int k = 0; k < kSPT; ++k) {
    const int s = k * kResThreads + tid;
    if (s < C) {
      const int tg = tags[s];
      nfree += (tg < 0) ? 1u : 0u;
      ncand += (tg >= 0 && !req[s]) ? 1u : 0u;
    }
  }
  uint32_t F, NC;
  block_excl_scan<uint32_t, kResThreads>(nfree, scan32, F);
  block_excl_scan<uint32_t, kResThreads>(ncand, scan32, NC);
  const uint32_t r = (M > F) ? min(M - F, NC) : 0u;   // victims to take

  // ---- r least recently used candidates: radix select on (stamp, unit) --
  // key = stamp * 2^32 + unit; keys are distinct, so exactly r keys are <= kappa
  unsigned long long kappa = 0ull;
  bool take_all = (r == NC);
  if (r > 0u && !take_all) {
    unsigned long long kmin = ~0ull, kmax = 0ull;
    for (int k = 0; k < kSPT; ++k) {
      const int s = k * kResThreads + tid;
      if (s < C && tags[s] >= 0 && !req[s]) {
        const unsigned long long key =
            ((unsigned long long)(uint32_t)stamps[s] << 32) | (uint32_t)tags[s];
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
    // block min / max through the 64-bit lane shuffles and LDS
    __shared__ unsigned long long red_lo[kResThreads / 64], red_hi[kResThreads / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, (unsigned long long)__shfl_xor((long long)kmin, o, 64));
      kmax = max(kmax, (unsigned long long)__shfl_xor((long long)kmax, o, 64));
    }
    if (lane_id() == 0) {
      red_lo[tid >> 6] = kmin;
      red_hi[tid >> 6] = kmax;
    }
    __syncthreads();
    kmin = ~0ull;
    kmax = 0ull;
    for (int w = 0; w < kResThreads / 64; ++w) {
      kmin = min(kmin, red_lo[w]);
      kmax = max(kmax, red_hi[w]);
    }
    const int top = 63 - __clzll(kmin ^ kmax);   // kmin != kmax since r < NC
    unsigned long long hi_mask = (top == 63) ? 0ull : ~((2ull << top) - 1ull);
    unsigned long long prefix = kmin & hi_mask;
    uint32_t need = r;                            // keys still to take, ascending
    int lo = top + 1;
    while (lo > 0) {
      const int width = min(11, lo);
      const int sh = lo - width, nb = 1 << width;
      for (int k = tid; k < nb; k += kResThreads) hist[k] = 0u;
      __syncthreads();
      for (int k = 0; k < kSPT; ++k) {
        const int s = k * kResThreads + tid;
        if (s < C && tags[s] >= 0 && !req[s]) {
          const unsigned long long key =
              ((unsigned long long)(uint32_t)stamps[s] << 32) | (uint32_t)tags[s];
          if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
        }
      }
      __syncthreads();
      // the bin where the count from the bottom reaches `need`
      const int b0 = 2 * tid, b1 = 2 * tid + 1;
      const uint32_t c0 = (b0 < nb) ? hist[b0] : 0u, c1 = (b1 < nb) ? hist[b1] : 0u;
      uint32_t tot;
      const uint32_t below0 = block_excl_scan<uint32_t, kResThreads>(c0 + c1, scan32, tot);
      const uint32_t below1 = below0 + c0;
      if (b0 < nb && below0 < need && need <= below0 + c0) {
        s_bin = b0;
        s_below = below0;
      }
      if (b1 < nb && below1 < need && need <= below1 + c1) {
        s_bin = b1;
        s_below = below1;
      }
      __syncthreads();
      need -= s_below;
      prefix |= (unsigned long long)s_bin << sh;
      hi_mask |= (unsigned long long)(nb - 1) << sh;
      lo = sh;
      __syncthreads();
    }
    kappa = prefix;   // the r-th smallest key
  }

  // ---- available slots in ascending order: free, plus victims -------------
  uint32_t navail = 0u;
  // slots are ranked in ascending order, so each thread takes a blocked run
  const int run = (C + kResThreads - 1) / kResThreads;
  const int s0 = tid * run;
  for (int k = 0; k < run; ++k) {
    const int s = s0 + k;
    if (s >= C) break;
    const int tg = tags[s];
    bool av = tg < 0;
    if (!av && r > 0u && !req[s]) {
      const unsigned long long key =
          ((unsigned long long)(uint32_t)stamps[s] << 32) | (uint32_t)tg;
      av = take_all || key <= kappa;
    }
    navail += av ? 1u : 0u;
  }
  uint32_t A;
  uint32_t rank = block_excl_scan<uint32_t, kResThreads>(navail, scan32, A);
  for (int k = 0; k < run; ++k) {
    const int s = s0 + k;
    if (s >= C) break;
    const int tg = tags[s];
    bool av = tg < 0;
    if (!av && r > 0u && !req[s]) {
      const unsigned long long key =
          ((unsigned long long)(uint32_t)stamps[s] << 32) | (uint32_t)tg;
      av = take_all || key <= kappa;
    }
    if (av) avail[rank++] = s;
  }
  const uint32_t placed = min(M, A);
  __syncthreads();

  // ---- pass 2: misses in ascending unit id take avail[0..placed) ----------
  uint32_t ev_local = 0u, mbase = 0u;
  for (int base = 0; base < E; base += kResThreads) {
    const int e = base + tid;
    uint32_t miss = 0u;
    int v = -1;
    int64_t li = 0;
    if (e < E) {
      int h = 0;
      while (e >= head_off[h + 1]) ++h;
      const int i = e - head_off[h];
      li = (int64_t)(b * hkv + h) * max_pages + i;
      const int p = sel_pages[li];
      if (p >= 0 && p < max_pages) {
        v = h * max_pages + p;
        miss = (umap[v] == -1) ? 1u : 0u;
      }
    }
    uint32_t tot;
    const uint32_t mr = mbase + block_excl_scan<uint32_t, kResThreads>(miss, scan32, tot);
    if (miss) {
      if (mr < placed) {
        const int s = avail[mr];
        const int old = tags[s];
        if (old >= 0) {
          if (old < hkv * max_pages) umap[old] = -1;
          ++ev_local;
        }
        tags[s] = v;
        stamps[s] = step;
        umap[v] = s;
        sel_phys[li] = b * C + s;
        misses[(int64_t)b * C + mr] = MissRec{v, s};
      } else {
        sel_phys[li] = -1;
      }
    }
    mbase += tot;
  }
  uint32_t evictions;
  block_excl_scan<uint32_t, kResThreads>(ev_local, scan32, evictions);
  if (tid == 0) {
    stats[b * 4 + 0] = (int32_t)H;
    stats[b * 4 + 1] = (int32_t)M;
    stats[b * 4 + 2] = (int32_t)evictions;
    stats[b * 4 + 3] = (M > placed) ? 1 : 0;
    miss_count[b] = (int32_t)placed;
  }
}

// One wave per missed unit: 8 KiB from pinned host memory into the slot.
__global__ __launch_bounds__(256) void fetch_kernel(const uint16_t* __restrict__ host_kv,
                                                    uint16_t* __restrict__ cache_kv, int hkv,
                                                    int max_pages, int C,
                                                    const MissRec* __restrict__ misses,
                                                    const int32_t* __restrict__ miss_count,
                                                    int waves_per_req,
                                                    int32_t* __restrict__ step_counter) {
  const int b = blockIdx.y;
  // every resolve workgroup has read the step (the resolve kernel ran first on
  // this stream): advance it for the next call
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *step_counter += 1;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  const int cnt = miss_count[b];
  for (int i = w; i < cnt; i += waves_per_req) {
    const MissRec m = misses[(int64_t)b * C + i];
    const int h = m.unit / max_pages, p = m.unit - (m.unit / max_pages) * max_pages;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        host_kv + (((int64_t)b * max_pages + p) * hkv + h) * kUnitElems);
    u32x4* dst = reinterpret_cast<u32x4*>(cache_kv + ((int64_t)b * C + m.slot) * kUnitElems);
    u32x4 t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = __builtin_nontemporal_load(src + k * 64 + lane);
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k * 64 + lane] = t[k];
  }
}

}  // namespace sp

extern "C" size_t sparse_cache_workspace_bytes(const sparse_dims* dims, int32_t capacity) {
  if (sp::check_dims(dims) != SPARSE_OK || capacity < 1) return 0;
  return (size_t)dims->batch * ((size_t)capacity * sizeof(sp::MissRec) + sizeof(int32_t)) + 256;
}

extern "C" sparse_status sparse_hbm_cache_resolve(
    const sparse_dims* dims, const int32_t* sel_counts, const int32_t* sel_pages,
    const uint16_t* host_kv, uint16_t* cache_kv, int32_t capacity, int32_t* slot_tag,
    int32_t* slot_stamp, int32_t* unit_slot, int32_t* step_counter, int32_t* sel_phys,
    int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!sel_counts || !sel_pages || !host_kv || !cache_kv || !slot_tag || !slot_stamp ||
      !unit_slot || !step_counter || !sel_phys || !stats)
    return SPARSE_ERR_INVALID;
  if (capacity < 1) return SPARSE_ERR_INVALID;
  if (capacity > sp::kMaxSlots || dims->num_kv_heads > sp::kMaxKvHeads) return SPARSE_ERR_UNSUPPORTED;
  if (!sp::aligned(host_kv, 16) || !sp::aligned(cache_kv, 16)) return SPARSE_ERR_INVALID;
  if (!ws || ws_bytes < sparse_cache_workspace_bytes(dims, capacity) || !sp::aligned(ws, 8))
    return SPARSE_ERR_WORKSPACE;
  const int B = dims->batch, hkv = dims->num_kv_heads;
  sp::MissRec* misses = static_cast<sp::MissRec*>(ws);
  int32_t* miss_count = reinterpret_cast<int32_t*>(misses + (size_t)B * capacity);
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(sp::resolve_kernel, dim3(B), dim3(sp::kResThreads), 0, s, sel_counts,
                     sel_pages, hkv, dims->max_pages, capacity, step_counter, slot_tag, slot_stamp,
                     unit_slot, sel_phys, stats, misses, miss_count);
  if (hipGetLastError() != hipSuccess) return SPARSE_ERR_HIP;
  const int waves_per_req = 256;   // 64 workgroups of 4 waves per request
  hipLaunchKernelGGL(sp::fetch_kernel, dim3(waves_per_req / 4, B), dim3(256), 0, s, host_kv,
                     cache_kv, hkv, dims->max_pages, capacity, misses, miss_count,
                     waves_per_req, step_counter);
  return sp::launch_status();
}
