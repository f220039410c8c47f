// Host-resident KV tier with a fixed-size HBM page cache, resolved inside the
// decode graph ("HiSparse: Scaling Sparse Attention Decoding with
// Hierarchical KV Cache", abstract: full KV history in host memory, a small
// fixed-size GPU cache per request, and one resolver inside the graph that
// finds hits, replaces least recently used entries and fetches misses from the
// host; outputs stay the same because only where KV lives changes).
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

#include <algorithm>

#include "common.h"
#include "fetch.h"
#include "lru_select.h"

namespace sp {

constexpr int kResThreads = 1024;
constexpr int kMaxSlots = 8192;
constexpr int kMaxKvHeads = 64;

// Per-request ticket word of the resolve: bits [0, 22) misses, [22, 44) hits
// counted by the hit-pass workgroups, [44, 64) workgroups done.  A request
// has at most 64 * 32768 = 2^21 list entries, so the counts never carry.
constexpr int kTkHitShift = 22;
constexpr int kTkDoneShift = 44;
constexpr unsigned long long kTkCountMask = (1ull << kTkHitShift) - 1ull;

// Misses of request b, placed by its last workgroup (the kernel below):
// requested-slot marks, victims, available slots, then the misses in
// ascending unit id take them.  M (>= 1) and H are the request's miss and hit
// totals from the ticket.  With miss lists, each unit's placed misses are also
// written in list order (a unit's misses are a contiguous run of the
// request's misses, which go head by head).  The slots' tags and stamps are
// read once into LDS: the victim search reads them several times.  (A
// requested slot's stamp may have been rewritten by another workgroup
// meanwhile; requested slots are never candidates, and only the stamps of
// candidates are used.)
// head_off[h] = the first entry of head h when a request's lists are laid
// end to end in head order, head_off[hkv] = the request's entry count.
// Wave 0 reads the hkv counts at once and scans them; then a barrier.
__device__ __forceinline__ void request_heads(const int32_t* __restrict__ sel_counts, int b,
                                              int hkv, int max_pages, int32_t* head_off) {
  const int t = threadIdx.x;
  if (t < 64) {                              // hkv <= kMaxKvHeads = 64
    int c = sel_counts[b * hkv + min(t, hkv - 1)];
    c = (t < hkv) ? min(max(c, 0), max_pages) : 0;
    const int incl = wave_incl_scan(c);
    if (t < hkv) head_off[t] = incl - c;
    if (t == hkv - 1) head_off[hkv] = incl;
  }
  __syncthreads();
}

// The head of each entry ee[k] (0 <= ee[k] < head_off[hkv]): how many heads
// after the first start at or before it.  Broadcast reads of the offsets,
// instead of a chain of dependent reads per entry.
template <int K>
__device__ __forceinline__ void entry_heads(const int (&ee)[K], int (&hh)[K],
                                            const int32_t* head_off, int hkv) {
#pragma unroll
  for (int k = 0; k < K; ++k) hh[k] = 0;
  for (int h2 = 1; h2 < hkv; ++h2) {
    const int o = head_off[h2];
#pragma unroll
    for (int k = 0; k < K; ++k) hh[k] += (ee[k] >= o) ? 1 : 0;
  }
}

constexpr int kPlaceEpt = 4;                 // list entries per thread per ranking round

__device__ __forceinline__ uint32_t resolve_place(
    int b, const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages,
    int hkv, int max_pages, int C, int recency_shift, int step, int32_t* __restrict__ tags,
    int32_t* __restrict__ stamps, int32_t* __restrict__ umap, int32_t* __restrict__ sel_phys,
    int32_t* __restrict__ stats, MissRec* __restrict__ misses, int32_t* __restrict__ miss_count,
    uint32_t M, uint32_t H, int32_t* __restrict__ miss_counts, int32_t* __restrict__ miss_pages,
    int32_t* __restrict__ miss_phys) {
  __shared__ uint8_t req[kMaxSlots];       // slot holds a unit requested this step
  __shared__ int32_t avail[kMaxSlots];     // available slots, ascending
  __shared__ int32_t s_tag[kMaxSlots];     // the slots' tags and stamps before this step
  __shared__ int32_t s_stamp[kMaxSlots];
  __shared__ SelectScratch sel;
  __shared__ uint32_t scan32[kResThreads / 64];
  __shared__ int32_t head_off[kMaxKvHeads + 1];
  __shared__ uint32_t head_miss[kMaxKvHeads];     // misses per head, then their prefix
  const int tid = threadIdx.x;
  constexpr int kSPT = kMaxSlots / kResThreads;   // slots per thread, strided

  // Every global read below is issued in batches: a thread's loads of one
  // batch go out together (indices clamped in range, values pinned by empty
  // asm statements so that no load moves under a test), and only then are
  // any of them used.  A load under a per-lane condition, or one behind a
  // data-dependent loop, becomes its own round trip.
  {
    int tg[kSPT], st[kSPT];
#pragma unroll
    for (int k = 0; k < kSPT; ++k) {
      const int sl = min(k * kResThreads + tid, C - 1);
      tg[k] = tags[sl];
      st[k] = stamps[sl];
    }
#pragma unroll
    for (int k = 0; k < kSPT; ++k) asm volatile("" : "+v"(tg[k]), "+v"(st[k]));
#pragma unroll
    for (int k = 0; k < kSPT; ++k) {
      const int sl = k * kResThreads + tid;
      if (sl < C) {
        req[sl] = 0;
        s_tag[sl] = tg[k];
        s_stamp[sl] = st[k];
      }
    }
  }
  if (tid < hkv) head_miss[tid] = 0u;
  request_heads(sel_counts, b, hkv, max_pages, head_off);
  const int E = head_off[hkv];

  // ---- the requested slots (units resident before this step) and each
  // head's miss count; the other workgroups only stamped them, and never
  // change the unit map, so it still holds the state before this step
  {
    constexpr int kBatch = 8;
    for (int base = 0; base < E; base += kBatch * kResThreads) {
      int hh[kBatch], pg[kBatch], v[kBatch], sm[kBatch];
      int64_t li[kBatch];
      int ee[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) ee[k] = min(base + k * kResThreads + tid, E - 1);
      entry_heads(ee, hh, head_off, hkv);
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        li[k] = (int64_t)(b * hkv + hh[k]) * max_pages + (ee[k] - head_off[hh[k]]);
#pragma unroll
      for (int k = 0; k < kBatch; ++k) pg[k] = sel_pages[li[k]];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) asm volatile("" : "+v"(pg[k]));
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const bool in = base + k * kResThreads + tid < E;
        v[k] = (in && pg[k] >= 0 && pg[k] < max_pages) ? hh[k] * max_pages + pg[k] : -1;
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) sm[k] = umap[max(v[k], 0)];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) asm volatile("" : "+v"(sm[k]));
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (v[k] < 0) continue;
        if (sm[k] >= 0 && sm[k] < C) req[sm[k]] = 1;
        if (sm[k] == -1) atomicAdd(&head_miss[hh[k]], 1u);
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0u;
    for (int h = 0; h < hkv; ++h) {
      const uint32_t m = head_miss[h];
      head_miss[h] = acc;            // misses of the heads before h
      acc += m;
    }
  }

  // ---- free slots and victim candidates ----------------------------------
  uint32_t nfree = 0u, ncand = 0u;
  for (int k = 0; k < kSPT; ++k) {
    const int s = k * kResThreads + tid;
    if (s < C) {
      const int tg = s_tag[s];
      nfree += (tg < 0) ? 1u : 0u;
      ncand += (tg >= 0 && !req[s]) ? 1u : 0u;
    }
  }
  uint32_t F, NC;
  block_excl_scan<uint32_t, kResThreads>(nfree, scan32, F);
  block_excl_scan<uint32_t, kResThreads>(ncand, scan32, NC);
  const uint32_t r = (M > F) ? min(M - F, NC) : 0u;   // victims to take

  // ---- r least recently used candidates: radix select on the keys -------
  // key = (stamp >> shift) * 2^tag_bits + unit; keys are distinct, so
  // exactly r keys are <= kappa
  const int tag_bits = unit_tag_bits((long long)hkv * max_pages);
  unsigned long long kappa = 0ull;
  const bool take_all = (r == NC);
  if (r > 0u && !take_all) {
    kappa = select_rth_key<kResThreads>(
        C, r,
        [&](int s, unsigned long long& key) {
          const int tg = s_tag[s];
          key = lru_key(s_stamp[s], tg, recency_shift, tag_bits);
          return tg >= 0 && !req[s];
        },
        sel);
  }

  // ---- available slots in ascending order: free, plus victims -------------
  uint32_t navail = 0u;
  // slots are ranked in ascending order, so each thread takes a blocked run
  const int run = (C + kResThreads - 1) / kResThreads;
  const int s0 = tid * run;
  for (int k = 0; k < run; ++k) {
    const int s = s0 + k;
    if (s >= C) break;
    const int tg = s_tag[s];
    bool av = tg < 0;
    if (!av && r > 0u && !req[s])
      av = take_all || lru_key(s_stamp[s], tg, recency_shift, tag_bits) <= kappa;
    navail += av ? 1u : 0u;
  }
  uint32_t A;
  uint32_t rank = block_excl_scan<uint32_t, kResThreads>(navail, scan32, A);
  for (int k = 0; k < run; ++k) {
    const int s = s0 + k;
    if (s >= C) break;
    const int tg = s_tag[s];
    bool av = tg < 0;
    if (!av && r > 0u && !req[s])
      av = take_all || lru_key(s_stamp[s], tg, recency_shift, tag_bits) <= kappa;
    if (av) avail[rank++] = s;
  }
  const uint32_t placed = min(M, A);
  __syncthreads();

  // ---- misses in ascending unit id take avail[0..placed) ------------------
  // Rounds of kPlaceEpt * 1024 list entries; thread t ranks the blocked run
  // of kPlaceEpt entries starting at kPlaceEpt t, its loads issued together.
  uint32_t ev_local = 0u, mbase = 0u;
  for (int base = 0; base < E; base += kPlaceEpt * kResThreads) {
    int hh[kPlaceEpt], pp[kPlaceEpt], vv[kPlaceEpt];
    int64_t li[kPlaceEpt];
    int ee[kPlaceEpt];
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) ee[k] = min(base + kPlaceEpt * tid + k, E - 1);
    entry_heads(ee, hh, head_off, hkv);
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k)
      li[k] = (int64_t)(b * hkv + hh[k]) * max_pages + (ee[k] - head_off[hh[k]]);
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) pp[k] = sel_pages[li[k]];
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) asm volatile("" : "+v"(pp[k]));
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) {
      const bool in = base + kPlaceEpt * tid + k < E;
      vv[k] = (in && pp[k] >= 0 && pp[k] < max_pages) ? hh[k] * max_pages + pp[k] : -1;
    }
    int sm[kPlaceEpt];
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) sm[k] = umap[max(vv[k], 0)];
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) asm volatile("" : "+v"(sm[k]));
    uint32_t mine = 0u;
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) {
      const bool miss = vv[k] >= 0 && sm[k] == -1;
      if (!miss) vv[k] = -1;
      mine += miss ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t mr = mbase + block_excl_scan<uint32_t, kResThreads>(mine, scan32, tot);
#pragma unroll
    for (int k = 0; k < kPlaceEpt; ++k) {
      if (vv[k] < 0) continue;
      if (mr < placed) {
        const int s = avail[mr];
        const int old = s_tag[s];
        if (old >= 0) {
          if (old < hkv * max_pages) umap[old] = -1;
          ++ev_local;
        }
        tags[s] = vv[k];
        stamps[s] = step;
        umap[vv[k]] = s;
        sel_phys[li[k]] = b * C + s;
        misses[(int64_t)b * C + mr] = MissRec{vv[k], s};
        if (miss_counts) {
          const int h = hh[k];
          const int64_t j = (int64_t)(b * hkv + h) * max_pages + (mr - head_miss[h]);
          miss_pages[j] = pp[k];
          miss_phys[j] = b * C + s;
        }
      } else {
        sel_phys[li[k]] = -1;
      }
      ++mr;
    }
    mbase += tot;
  }
  uint32_t evictions;
  block_excl_scan<uint32_t, kResThreads>(ev_local, scan32, evictions);
  if (miss_counts && tid < hkv) {
    // placed misses of head tid: its run of the request's misses, cut at
    // `placed` (the misses left without a slot are the last ones)
    const uint32_t lo = head_miss[tid];
    const uint32_t hi = (tid + 1 < hkv) ? head_miss[tid + 1] : M;
    miss_counts[b * hkv + tid] = (int32_t)(min(hi, placed) - min(lo, placed));
  }
  if (tid == 0) {
    stats[b * 4 + 0] = (int32_t)H;
    stats[b * 4 + 1] = (int32_t)M;
    stats[b * 4 + 2] = (int32_t)evictions;
    stats[b * 4 + 3] = (M > placed) ? 1 : 0;
    miss_count[b] = (int32_t)placed;
  }
  return placed;
}

// Workgroup (b, h, c) of the grid: list entries c * 1024 + tid,
// + nchunk * 1024, ... of unit (b, h).  Every workgroup stamps its hits and
// writes their slot ids; the request's last workgroup to finish (ticket)
// places the misses, or with none only writes the statistics.  With every
// access a hit, a step is one pass of parallel lookups: the list entries and
// the list length are loaded together, then the unit map.
//
// kFetch: the resolve of the one-pass call.  Each request's last workgroup
// then copies the request's placed misses itself (its 16 waves, from pinned
// host memory into the slots), and the last workgroup of the whole grid
// (a second ticket) advances the step counter -- every workgroup has read
// the step by then.  One launch instead of resolve + fetch.
template <bool kFetch>
__global__ __launch_bounds__(kResThreads) void resolve_kernel(
    const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages, int hkv,
    int max_pages, int C, int nchunk, int recency_shift, int32_t* __restrict__ step_counter,
    int32_t* __restrict__ slot_tag, int32_t* __restrict__ slot_stamp,
    int32_t* __restrict__ unit_slot, int32_t* __restrict__ sel_phys,
    int32_t* __restrict__ hit_phys, int32_t* __restrict__ stats, MissRec* __restrict__ misses,
    int32_t* __restrict__ miss_count, unsigned long long* __restrict__ tickets,
    int32_t* __restrict__ miss_counts, int32_t* __restrict__ miss_pages,
    int32_t* __restrict__ miss_phys, const uint16_t* __restrict__ host_kv,
    uint16_t* __restrict__ cache_kv, uint32_t* __restrict__ grid_ticket) {
  __shared__ unsigned long long scan64[kResThreads / 64];
  __shared__ unsigned long long s_tk;
  const int tid = threadIdx.x;
  const int per_req = hkv * nchunk;
  const int b = blockIdx.x / per_req;
  const int hc = blockIdx.x - b * per_req;
  const int h = hc / nchunk, c = hc - (hc / nchunk) * nchunk;
  const int u = b * hkv + h;
  const int64_t row = (int64_t)u * max_pages;
  int32_t* stamps = slot_stamp + (int64_t)b * C;
  const int32_t* umap = unit_slot + (int64_t)b * hkv * max_pages;

  // the first chunk's entries are loaded before the length is known: an
  // index past the row re-reads its last entry, and the entry is used only
  // if it lies inside the list
  int i = c * kResThreads + tid;
  int p = sel_pages[row + min(i, max_pages - 1)];
  const int n = min(max(sel_counts[u], 0), max_pages);
  const int step = *step_counter;
  uint32_t m_local = 0u, h_local = 0u;
  for (;;) {
    const bool in = i < n;
    const int v = (in && p >= 0 && p < max_pages) ? h * max_pages + p : -1;
    int s = umap[max(v, 0)];                 // unit 0's entry stands in when unused
    asm volatile("" : "+v"(s));              // keep the load ahead of the tests
    if (in) {
      int sk = (v >= 0) ? s : -2;
      if (sk >= C) sk = -2;                  // corrupt state: never index past the cache
      if (hit_phys) hit_phys[row + i] = (sk >= 0) ? b * C + sk : -1;
      if (sk >= 0) {
        ++h_local;
        stamps[sk] = step;
        sel_phys[row + i] = b * C + sk;
      } else if (sk == -1) {
        ++m_local;                           // placed by the request's last workgroup
      } else {
        sel_phys[row + i] = -1;              // page id out of range: an empty page
      }
    }
    i += nchunk * kResThreads;
    if (i - tid >= n) break;                 // (uniform across the workgroup)
    p = sel_pages[row + min(i, max_pages - 1)];
  }
  // every thread holds the step before the block's first barrier, so the
  // grid ticket below (taken after it) follows every read of the step
  asm volatile("" ::"v"(step));
  unsigned long long tot;
  block_excl_scan<unsigned long long, kResThreads>(
      ((unsigned long long)h_local << kTkHitShift) | m_local, scan64, tot);
  if (tid == 0) {
    const unsigned long long mine = tot | (1ull << kTkDoneShift);
    const unsigned long long old = atomicAdd(tickets + b, mine);
    s_tk = old + mine;
  }
  __syncthreads();
  const unsigned long long tk = s_tk;
  if ((int)(tk >> kTkDoneShift) == per_req) {           // the request's last workgroup
    const uint32_t M = (uint32_t)(tk & kTkCountMask);
    const uint32_t H = (uint32_t)((tk >> kTkHitShift) & kTkCountMask);
    if (tid == 0) __hip_atomic_store(tickets + b, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (M == 0u) {               // every requested unit is resident: nothing to place
      if (miss_counts && tid < hkv) miss_counts[b * hkv + tid] = 0;
      if (tid == 0) {
        stats[b * 4 + 0] = (int32_t)H;
        stats[b * 4 + 1] = 0;
        stats[b * 4 + 2] = 0;
        stats[b * 4 + 3] = 0;
        miss_count[b] = 0;
      }
    } else {
      const uint32_t placed = resolve_place(
          b, sel_counts, sel_pages, hkv, max_pages, C, recency_shift, step,
          slot_tag + (int64_t)b * C, stamps, unit_slot + (int64_t)b * hkv * max_pages, sel_phys,
          stats, misses, miss_count, M, H, miss_counts, miss_pages, miss_phys);
      if (kFetch) {
        __syncthreads();         // the miss records written above, visible to every wave
        for (int k = tid >> 6; k < (int)placed; k += kResThreads / 64)
          copy_request_miss(host_kv, cache_kv, hkv, max_pages, C, b,
                            misses[(int64_t)b * C + k]);
      }
    }
  }
  if (kFetch && tid == 0) {
    const uint32_t t = atomicAdd(grid_ticket, 1u);
    if (t == gridDim.x - 1u) {   // the grid's last workgroup: advance the step
      *step_counter = step + 1;
      __hip_atomic_store(grid_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The fetch runs in a few whole compute units that it keeps to itself: each
// workgroup is 8 waves and reserves the unit's entire LDS, so no other
// workgroup that uses LDS (the attention, merges, resolves) is placed beside
// it.  A fetch wave holds its PCIe reads in flight for microseconds, and
// workgroups sharing its compute unit were measured to stall behind them:
// attention launched beside a fetch ran up to 9x longer.  (8 waves per unit
// over 32 units fetched faster than 16 waves over 16.)
constexpr int kFetchThreads = 512;
constexpr int kFetchWavesPerGroup = kFetchThreads / 64;
constexpr int kFetchLdsWords = 40960;    // 160 KiB, the whole LDS of a compute unit

// Wave w of waves_per_req * B copies request b = w % B's misses
// w / B, w / B + waves_per_req, ...: 8 KiB each, from pinned host memory into
// the slot.
__global__ __launch_bounds__(kFetchThreads) void fetch_kernel(
    const uint16_t* __restrict__ host_kv, uint16_t* __restrict__ cache_kv, int hkv,
    int max_pages, int C, const MissRec* __restrict__ misses,
    const int32_t* __restrict__ miss_count, int B, int waves_per_req,
    int32_t* __restrict__ step_counter) {
  __shared__ uint32_t cu_reserve[kFetchLdsWords];
  // every resolve workgroup has read the step (the resolve kernel ran first on
  // this stream): advance it for the next call
  if (blockIdx.x == 0 && threadIdx.x == 0) *step_counter += 1;
  const int w = blockIdx.x * kFetchWavesPerGroup + (threadIdx.x >> 6);
  if (w >= waves_per_req * B) return;
  const int b = w % B;
  const int cnt = miss_count[b];
  if (cnt < 0) {                               // never taken; keeps the reservation
    cu_reserve[threadIdx.x] = 0u;
    asm volatile("" ::"v"(cu_reserve[threadIdx.x ^ 1u]));
  }
  for (int i = w / B; i < cnt; i += waves_per_req)
    copy_request_miss(host_kv, cache_kv, hkv, max_pages, C, b, misses[(int64_t)b * C + i]);
}


// ---- one pool shared by every request --------------------------------------
// Pooled unit id g = (b * Hkv + h) * max_pages + p; slots 0 .. S-1 belong to
// no request in particular.  The rules above apply over pooled ids: the
// requested set is the union over requests, and misses in ascending pooled
// id (so request by request) take the available slots in ascending order --
// a request holds as many slots as the pool-wide replacement leaves it.
//   pool_mark_kernel   one workgroup per request: hits (stamp, mark, slot id)
//                      and the request's hit and miss counts;
//   pool_scan_kernel   one workgroup per block of 1024 slots: the block's
//                      free slots counted, its victim candidates' keys
//                      compacted into the block's segment;
//   pool_select_kernel one workgroup: each request's miss-rank offset, the
//                      victims (radix select over the compacted keys), each
//                      block's offset in the list of available slots;
//   pool_avail_kernel  one workgroup per block: its available slots, in
//                      ascending order, at the block's offset; clears marks;
//   pool_place_kernel  one workgroup per request: its misses, ascending, take
//                      avail[offset + rank]; statistics;
//   pool_fetch_kernel  copies every placed miss from pinned host memory.
constexpr int kMaxPoolSlots = 1 << 22;

__global__ __launch_bounds__(kResThreads) void pool_mark_kernel(
    const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages, int hkv,
    int max_pages, int S, const int32_t* __restrict__ step_counter,
    int32_t* __restrict__ slot_stamp, const int32_t* __restrict__ unit_slot,
    int32_t* __restrict__ sel_phys, int32_t* __restrict__ hit_phys, uint8_t* __restrict__ req,
    int32_t* __restrict__ counts) {
  __shared__ int32_t head_off[kMaxKvHeads + 1];
  __shared__ unsigned long long scan64[kResThreads / 64];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int step = *step_counter;
  request_heads(sel_counts, b, hkv, max_pages, head_off);
  const int E = head_off[hkv];
  // kMarkEpt entries per thread per round, their loads issued together
  constexpr int kMarkEpt = 4;
  uint32_t m_local = 0u, h_local = 0u;
  for (int base = 0; base < E; base += kMarkEpt * kResThreads) {
    int ee[kMarkEpt], hh[kMarkEpt], pg[kMarkEpt], sk[kMarkEpt];
    int64_t li[kMarkEpt], v[kMarkEpt];
#pragma unroll
    for (int k = 0; k < kMarkEpt; ++k) ee[k] = min(base + k * kResThreads + tid, E - 1);
    entry_heads(ee, hh, head_off, hkv);
#pragma unroll
    for (int k = 0; k < kMarkEpt; ++k) {
      li[k] = (int64_t)(b * hkv + hh[k]) * max_pages + (ee[k] - head_off[hh[k]]);
      pg[k] = sel_pages[li[k]];
    }
#pragma unroll
    for (int k = 0; k < kMarkEpt; ++k) asm volatile("" : "+v"(pg[k]));
#pragma unroll
    for (int k = 0; k < kMarkEpt; ++k) {
      const bool in = base + k * kResThreads + tid < E;
      v[k] = (in && pg[k] >= 0 && pg[k] < max_pages)
                 ? (int64_t)(b * hkv + hh[k]) * max_pages + pg[k] : -1;
      sk[k] = unit_slot[max(v[k], (int64_t)0)];   // unit 0's entry stands in when unused
    }
#pragma unroll
    for (int k = 0; k < kMarkEpt; ++k) asm volatile("" : "+v"(sk[k]));
#pragma unroll
    for (int k = 0; k < kMarkEpt; ++k) {
      if (base + k * kResThreads + tid >= E) continue;
      int s_ = (v[k] >= 0) ? sk[k] : -2;
      if (s_ >= S) s_ = -2;                  // corrupt state: never index past the pool
      if (hit_phys) hit_phys[li[k]] = (s_ >= 0) ? s_ : -1;
      if (s_ >= 0) {
        ++h_local;
        req[s_] = 1;
        slot_stamp[s_] = step;
        sel_phys[li[k]] = s_;
      } else if (s_ == -1) {
        ++m_local;
      } else {
        sel_phys[li[k]] = -1;                // page id out of range: an empty page
      }
    }
  }
  unsigned long long tot;
  block_excl_scan<unsigned long long, kResThreads>(
      ((unsigned long long)h_local << 32) | m_local, scan64, tot);
  if (tid == 0) {
    counts[2 * b] = (int32_t)(tot >> 32);
    counts[2 * b + 1] = (int32_t)(uint32_t)tot;
  }
}

constexpr int kPoolBlk = 1024;          // slots per scan / avail workgroup
constexpr int kPoolBlkThreads = 256;    // 4 consecutive slots per thread

// Selection state handed from pool_select_kernel to pool_avail_kernel.
struct PoolSel {
  unsigned long long kappa;   // the r-th smallest candidate key
  uint32_t r;                 // victims to take
  uint32_t take_all;          // every candidate is a victim
  uint32_t placed;            // misses that get a slot
  uint32_t pad;
};

__global__ __launch_bounds__(kPoolBlkThreads) void pool_scan_kernel(
    int S, int recency_shift, int tag_bits, const int32_t* __restrict__ slot_tag,
    const int32_t* __restrict__ slot_stamp, const uint8_t* __restrict__ req,
    unsigned long long* __restrict__ ckeys, int32_t* __restrict__ cblk,
    int32_t* __restrict__ blk_free, uint32_t* __restrict__ totals) {
  __shared__ unsigned long long scan64[kPoolBlkThreads / 64];
  __shared__ uint32_t s_base;
  const int tid = threadIdx.x, blk = blockIdx.x;
  const int s0 = blk * kPoolBlk + 4 * tid;
  int tg[4], st[4];
  bool fr[4], cd[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool in = s0 + k < S;
    tg[k] = in ? slot_tag[s0 + k] : 0;
    st[k] = in ? slot_stamp[s0 + k] : 0;
    const uint8_t rq = in ? req[s0 + k] : 1;
    fr[k] = in && tg[k] < 0;
    cd[k] = in && tg[k] >= 0 && !rq;
  }
  uint32_t nf = 0u, nc = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    nf += fr[k] ? 1u : 0u;
    nc += cd[k] ? 1u : 0u;
  }
  unsigned long long tot;
  const unsigned long long ex = block_excl_scan<unsigned long long, kPoolBlkThreads>(
      ((unsigned long long)nc << 32) | nf, scan64, tot);
  // the block's candidates go to one contiguous run of the compacted list
  // (run order across blocks does not matter to the selection)
  if (tid == 0) {
    s_base = atomicAdd(&totals[0], (uint32_t)(tot >> 32));
    atomicAdd(&totals[1], (uint32_t)tot);
    blk_free[blk] = (int32_t)(uint32_t)tot;
  }
  __syncthreads();
  uint32_t at = s_base + (uint32_t)(ex >> 32);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (cd[k]) {
      ckeys[at] = lru_key(st[k], tg[k], recency_shift, tag_bits);
      cblk[at] = blk;
      ++at;
    }
}

__global__ __launch_bounds__(kResThreads) void pool_select_kernel(
    int B, int nblk, const int32_t* __restrict__ counts, int32_t* __restrict__ moff,
    const unsigned long long* __restrict__ ckeys, const int32_t* __restrict__ cblk,
    const int32_t* __restrict__ blk_free, uint32_t* __restrict__ totals,
    int32_t* __restrict__ blk_off, PoolSel* __restrict__ sel_out) {
  __shared__ SelectScratch sel;
  __shared__ uint32_t scan32[kResThreads / 64];
  __shared__ uint32_t s_vict[kMaxPoolSlots / kPoolBlk];
  const int tid = threadIdx.x;
  // each request's miss-rank offset: exclusive prefix of the miss counts
  uint32_t M = 0u;
  for (int base = 0; base < B; base += kResThreads) {
    const int b = base + tid;
    const uint32_t m = (b < B) ? (uint32_t)counts[2 * b + 1] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<uint32_t, kResThreads>(m, scan32, tot);
    if (b < B) moff[b] = (int32_t)(M + ex);
    M += tot;
  }
  const uint32_t NC = totals[0], F = totals[1];
  for (int k = tid; k < nblk; k += kResThreads) s_vict[k] = 0u;
  __syncthreads();
  const uint32_t r = (M > F) ? min(M - F, NC) : 0u;
  const bool take_all = r == NC;
  unsigned long long kappa = 0ull;
  if (r > 0u && !take_all) {
    kappa = select_rth_key<kResThreads>(
        (int)NC, r,
        [&](int i, unsigned long long& key) {
          key = ckeys[i];
          return true;
        },
        sel);
  }
  // victims per block: a block's keys are one contiguous run, so a wave's
  // lanes mostly share the block and hist_add_wave adds them with one atomic
  if (r > 0u) {
    for (int base = 0; base < (int)NC; base += kResThreads) {
      const int i = base + tid;
      const bool in = i < (int)NC;
      const bool v = in && (take_all || ckeys[i] <= kappa);
      hist_add_wave(s_vict, in ? cblk[i] : 0, v);
    }
  }
  __syncthreads();
  uint32_t A = 0u;
  for (int base = 0; base < nblk; base += kResThreads) {
    const int k = base + tid;
    const uint32_t a = (k < nblk) ? (uint32_t)blk_free[k] + s_vict[k] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<uint32_t, kResThreads>(a, scan32, tot);
    if (k < nblk) blk_off[k] = (int32_t)(A + ex);
    A += tot;
  }
  if (tid == 0) {
    *sel_out = PoolSel{kappa, r, take_all ? 1u : 0u, min(M, A), 0u};
    totals[0] = 0u;                            // re-armed for the next call
    totals[1] = 0u;
  }
}

__global__ __launch_bounds__(kPoolBlkThreads) void pool_avail_kernel(
    int S, int recency_shift, int tag_bits, const int32_t* __restrict__ slot_tag,
    const int32_t* __restrict__ slot_stamp, uint8_t* __restrict__ req,
    const PoolSel* __restrict__ sel_in, const int32_t* __restrict__ blk_off,
    int32_t* __restrict__ avail, int32_t* __restrict__ placed_out) {
  __shared__ uint32_t scan32[kPoolBlkThreads / 64];
  const int tid = threadIdx.x, blk = blockIdx.x;
  const PoolSel sl = *sel_in;
  const int s0 = blk * kPoolBlk + 4 * tid;
  bool av[4];
  uint32_t n = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int sk = s0 + k;
    av[k] = false;
    if (sk < S) {
      const int tg = slot_tag[sk];
      const uint8_t rq = req[sk];
      const int st = slot_stamp[sk];
      if (tg < 0) av[k] = true;
      else if (sl.r > 0u && !rq)
        av[k] = sl.take_all || lru_key(st, tg, recency_shift, tag_bits) <= sl.kappa;
      req[sk] = 0;                             // marks are read only here: clear them
    }
    n += av[k] ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t rank = (uint32_t)blk_off[blk] + block_excl_scan<uint32_t, kPoolBlkThreads>(n, scan32, tot);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (av[k]) avail[rank++] = s0 + k;
  if (blk == 0 && tid == 0) *placed_out = (int32_t)sl.placed;
}

__global__ __launch_bounds__(kResThreads) void pool_place_kernel(
    const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages, int hkv,
    int max_pages, const int32_t* __restrict__ step_counter, int32_t* __restrict__ slot_tag,
    int32_t* __restrict__ slot_stamp, int32_t* __restrict__ unit_slot,
    int32_t* __restrict__ sel_phys, int32_t* __restrict__ stats,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ moff,
    const int32_t* __restrict__ avail, const int32_t* __restrict__ placed_in,
    MissRec* __restrict__ misses) {
  __shared__ int32_t head_off[kMaxKvHeads + 1];
  __shared__ uint32_t scan32[kResThreads / 64];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int step = *step_counter;
  request_heads(sel_counts, b, hkv, max_pages, head_off);
  const int E = head_off[hkv];
  const uint32_t P = (uint32_t)*placed_in, off = (uint32_t)moff[b];
  const uint32_t Mb = (uint32_t)counts[2 * b + 1];
  const int64_t n_units = (int64_t)gridDim.x * hkv * max_pages;
  uint32_t ev_local = 0u, mbase = 0u;
  if (Mb > 0u) {
    // rounds of kPlaceEpt * 1024 entries; thread t ranks the blocked run of
    // kPlaceEpt entries from kPlaceEpt t, its loads issued together
    for (int base = 0; base < E; base += kPlaceEpt * kResThreads) {
      int ee[kPlaceEpt], hh[kPlaceEpt], pp[kPlaceEpt], sm[kPlaceEpt];
      int64_t li[kPlaceEpt], vv[kPlaceEpt];
#pragma unroll
      for (int k = 0; k < kPlaceEpt; ++k) ee[k] = min(base + kPlaceEpt * tid + k, E - 1);
      entry_heads(ee, hh, head_off, hkv);
#pragma unroll
      for (int k = 0; k < kPlaceEpt; ++k) {
        li[k] = (int64_t)(b * hkv + hh[k]) * max_pages + (ee[k] - head_off[hh[k]]);
        pp[k] = sel_pages[li[k]];
      }
#pragma unroll
      for (int k = 0; k < kPlaceEpt; ++k) asm volatile("" : "+v"(pp[k]));
#pragma unroll
      for (int k = 0; k < kPlaceEpt; ++k) {
        const bool in = base + kPlaceEpt * tid + k < E;
        vv[k] = (in && pp[k] >= 0 && pp[k] < max_pages)
                    ? (int64_t)(b * hkv + hh[k]) * max_pages + pp[k] : -1;
        sm[k] = unit_slot[max(vv[k], (int64_t)0)];
      }
#pragma unroll
      for (int k = 0; k < kPlaceEpt; ++k) asm volatile("" : "+v"(sm[k]));
      uint32_t mine = 0u;
#pragma unroll
      for (int k = 0; k < kPlaceEpt; ++k) {
        const bool miss = vv[k] >= 0 && sm[k] == -1;
        if (!miss) vv[k] = -1;
        mine += miss ? 1u : 0u;
      }
      uint32_t tot;
      uint32_t mr = off + mbase + block_excl_scan<uint32_t, kResThreads>(mine, scan32, tot);
#pragma unroll
      for (int k = 0; k < kPlaceEpt; ++k) {
        if (vv[k] < 0) continue;
        if (mr < P) {
          const int sl = avail[mr];
          const int old = slot_tag[sl];
          if (old >= 0) {
            if (old < n_units) unit_slot[old] = -1;
            ++ev_local;
          }
          slot_tag[sl] = (int32_t)vv[k];
          slot_stamp[sl] = step;
          unit_slot[vv[k]] = sl;
          sel_phys[li[k]] = sl;
          misses[mr] = MissRec{(int32_t)vv[k], sl};
        } else {
          sel_phys[li[k]] = -1;
        }
        ++mr;
      }
      mbase += tot;
    }
  }
  uint32_t evictions;
  block_excl_scan<uint32_t, kResThreads>(ev_local, scan32, evictions);
  if (tid == 0) {
    stats[b * 4 + 0] = counts[2 * b];
    stats[b * 4 + 1] = (int32_t)Mb;
    stats[b * 4 + 2] = (int32_t)evictions;
    stats[b * 4 + 3] = (off + Mb > P) ? 1 : 0;
  }
}

// The pool's fetch, in whole compute units like fetch_kernel: wave w copies
// the placed misses w, w + waves, ...
__global__ __launch_bounds__(kFetchThreads) void pool_fetch_kernel(
    const uint16_t* __restrict__ host_kv, uint16_t* __restrict__ cache_kv, int hkv,
    int max_pages, const MissRec* __restrict__ misses, const int32_t* __restrict__ placed_in,
    int waves, int32_t* __restrict__ step_counter) {
  __shared__ uint32_t cu_reserve[kFetchLdsWords];
  // every workgroup of the earlier kernels has read the step: advance it
  if (blockIdx.x == 0 && threadIdx.x == 0) *step_counter += 1;
  const int w = blockIdx.x * kFetchWavesPerGroup + (threadIdx.x >> 6);
  const int P = *placed_in;
  if (P < 0) {                                 // never taken; keeps the reservation
    cu_reserve[threadIdx.x] = 0u;
    asm volatile("" ::"v"(cu_reserve[threadIdx.x ^ 1u]));
  }
  for (int i = w; i < P; i += waves) copy_pooled_miss(host_kv, cache_kv, hkv, max_pages, misses[i]);
}

// One workgroup per (request, KV head) unit: the unit's list entries that
// were placed this step but were not resident before it (hit_phys < 0,
// sel_phys >= 0), compacted in list order -- ascending page order -- into
// the unit's miss list.
constexpr int kSplitThreads = 256;

__global__ __launch_bounds__(kSplitThreads) void split_misses_kernel(
    const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ hit_phys, int max_pages,
    int32_t* __restrict__ miss_counts, int32_t* __restrict__ miss_pages,
    int32_t* __restrict__ miss_phys) {
  __shared__ uint32_t scan32[kSplitThreads / 64];
  const int u = blockIdx.x, tid = threadIdx.x;
  const int n = min(max(sel_counts[u], 0), max_pages);
  const int64_t row = (int64_t)u * max_pages;
  uint32_t base = 0u;
  for (int i0 = 0; i0 < n; i0 += kSplitThreads) {
    const int i = i0 + tid;
    int page = -1, phys = -1;
    uint32_t miss = 0u;
    if (i < n) {
      page = sel_pages[row + i];
      phys = sel_phys[row + i];
      miss = (hit_phys[row + i] < 0 && phys >= 0) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t r = base + block_excl_scan<uint32_t, kSplitThreads>(miss, scan32, tot);
    if (miss) {
      miss_pages[row + r] = page;
      miss_phys[row + r] = phys;
    }
    base += tot;
  }
  if (tid == 0) miss_counts[u] = (int32_t)base;
}

}  // namespace sp

extern "C" size_t sparse_cache_workspace_bytes(const sparse_dims* dims, int32_t capacity) {
  if (sp::check_dims(dims) != SPARSE_OK || capacity < 1) return 0;
  return (size_t)dims->batch * (sizeof(unsigned long long) +
                                (size_t)capacity * sizeof(sp::MissRec) + sizeof(int32_t)) +
         sizeof(uint32_t) + 256;
}

namespace {

// Per-request workspace: the resolve's ticket words [B] (zero before the
// first call; every call leaves them zero), miss records [B][C], the
// per-request counts [B], then the one-pass resolve's grid ticket (zero
// before the first call, left zero).
// Pooled workspace (S rounded up to whole blocks of 1024 slots, nblk of
// them): marks [S], compacted candidate keys [S] and their blocks [S],
// avail [S], miss records [S], the selection state, two running totals, per
// block free counts and offsets, then counts [B][2], offsets [B], placed [1].
// The marks and the totals must be zero before the first call; every call
// leaves them zero.
size_t pooled_ws_bytes(int B, int S) {
  const size_t nblk = ((size_t)S + sp::kPoolBlk - 1) / sp::kPoolBlk;
  const size_t Sr = nblk * sp::kPoolBlk;
  return Sr + Sr * sizeof(unsigned long long) + Sr * sizeof(int32_t) + Sr * sizeof(int32_t) +
         Sr * sizeof(sp::MissRec) + sizeof(sp::PoolSel) + 2 * sizeof(uint32_t) +
         nblk * 2 * sizeof(int32_t) + (size_t)B * 3 * sizeof(int32_t) + sizeof(int32_t) + 256;
}

// Arguments of the resolve itself (lists, cache state, outputs).
sparse_status check_resolve_args(const sparse_dims* dims, const int32_t* sel_counts,
                                 const int32_t* sel_pages, int32_t capacity, int32_t* slot_tag,
                                 int32_t* slot_stamp, int32_t* unit_slot, int32_t* step_counter,
                                 int32_t* sel_phys, int32_t* stats) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!sel_counts || !sel_pages || !slot_tag || !slot_stamp || !unit_slot || !step_counter ||
      !sel_phys || !stats)
    return SPARSE_ERR_INVALID;
  if (capacity < 1) return SPARSE_ERR_INVALID;
  if (dims->num_kv_heads > sp::kMaxKvHeads) return SPARSE_ERR_UNSUPPORTED;
  return SPARSE_OK;
}

// Arguments of the fetch: the pinned host pool and the HBM cache pool.
sparse_status check_pool_args(const uint16_t* host_kv, const uint16_t* cache_kv) {
  if (!host_kv || !cache_kv) return SPARSE_ERR_INVALID;
  if (!sp::aligned(host_kv, 16) || !sp::aligned(cache_kv, 16)) return SPARSE_ERR_INVALID;
  return SPARSE_OK;
}

// About 256 fetching waves in all (each has one 8 KiB unit in flight; 32
// compute units in all) keep the PCIe link busy; more only take compute
// units from the attention that may run beside the fetch.
constexpr int kFetchWaves = SPARSE_FETCH_GROUPS * sp::kFetchWavesPerGroup;

// Per-request workspace views (layout above sparse_cache_workspace_bytes).
struct PerRequestWs {
  unsigned long long* tickets;
  sp::MissRec* misses;
  int32_t* miss_count;
  uint32_t* grid_ticket;
};
PerRequestWs per_request_ws(int B, int32_t capacity, void* ws) {
  unsigned long long* tickets = static_cast<unsigned long long*>(ws);
  sp::MissRec* misses = reinterpret_cast<sp::MissRec*>(tickets + B);
  int32_t* counts = reinterpret_cast<int32_t*>(misses + (size_t)B * capacity);
  return {tickets, misses, counts, reinterpret_cast<uint32_t*>(counts + B)};
}

// Optional per-unit lists of the misses placed this step (split schedule).
struct MissLists {
  int32_t* counts;
  int32_t* pages;
  int32_t* phys;
};

// Hit-pass workgroups per (request, KV head): enough 1024-entry chunks for
// the longest list the dims allow, but no more than about 512 workgroups in
// all (longer lists loop).
int resolve_chunks(const sparse_dims* dims) {
  const int want = (sp::list_cap(dims) + sp::kResThreads - 1) / sp::kResThreads;
  const int64_t units = (int64_t)dims->batch * dims->num_kv_heads;
  const int lim = (int)std::max<int64_t>(1, 512 / units);
  return std::max(1, std::min(want, lim));
}

// host_kv and cache_kv given: the one-pass resolve, which also copies the
// misses and advances the step (resolve_kernel<true>); else the resolve
// alone, for a fetch that follows.
sparse_status resolve_per_request(const sparse_dims* dims, int shift, const int32_t* sel_counts,
                                  const int32_t* sel_pages, int32_t capacity, int32_t* slot_tag,
                                  int32_t* slot_stamp, int32_t* unit_slot, int32_t* step_counter,
                                  int32_t* sel_phys, int32_t* hit_phys, int32_t* stats, void* ws,
                                  MissLists ml, const uint16_t* host_kv, uint16_t* cache_kv,
                                  hipStream_t s) {
  const int B = dims->batch, hkv = dims->num_kv_heads;
  const PerRequestWs w = per_request_ws(B, capacity, ws);
  const int nchunk = resolve_chunks(dims);
  const int64_t groups = (int64_t)B * hkv * nchunk;
  if (groups > INT32_MAX) return SPARSE_ERR_UNSUPPORTED;
  if (host_kv)
    hipLaunchKernelGGL(sp::resolve_kernel<true>, dim3((unsigned)groups), dim3(sp::kResThreads), 0,
                       s, sel_counts, sel_pages, hkv, dims->max_pages, capacity, nchunk, shift,
                       step_counter, slot_tag, slot_stamp, unit_slot, sel_phys, hit_phys, stats,
                       w.misses, w.miss_count, w.tickets, ml.counts, ml.pages, ml.phys, host_kv,
                       cache_kv, w.grid_ticket);
  else
    hipLaunchKernelGGL(sp::resolve_kernel<false>, dim3((unsigned)groups), dim3(sp::kResThreads),
                       0, s, sel_counts, sel_pages, hkv, dims->max_pages, capacity, nchunk, shift,
                       step_counter, slot_tag, slot_stamp, unit_slot, sel_phys, hit_phys, stats,
                       w.misses, w.miss_count, w.tickets, ml.counts, ml.pages, ml.phys, nullptr,
                       nullptr, w.grid_ticket);
  return sp::launch_status();
}

sparse_status fetch_per_request(const sparse_dims* dims, const uint16_t* host_kv,
                                uint16_t* cache_kv, int32_t capacity, int32_t* step_counter,
                                void* ws, hipStream_t s) {
  const int B = dims->batch, hkv = dims->num_kv_heads;
  const PerRequestWs w = per_request_ws(B, capacity, ws);
  const int waves_per_req = std::max(1, kFetchWaves / B);
  const int groups = (waves_per_req * B + sp::kFetchWavesPerGroup - 1) / sp::kFetchWavesPerGroup;
  hipLaunchKernelGGL(sp::fetch_kernel, dim3(groups), dim3(sp::kFetchThreads), 0, s, host_kv,
                     cache_kv, hkv, dims->max_pages, capacity, w.misses, w.miss_count, B,
                     waves_per_req, step_counter);
  return sp::launch_status();
}

// Pooled workspace views (layout above pooled_ws_bytes).
struct PooledWs {
  uint8_t* req;
  unsigned long long* ckeys;
  int32_t* cblk;
  int32_t* avail;
  sp::MissRec* misses;
  sp::PoolSel* psel;
  uint32_t* totals;
  int32_t* blk_free;
  int32_t* blk_off;
  int32_t* counts;
  int32_t* moff;
  int32_t* placed;
  int nblk;
};
PooledWs pooled_ws(int B, int32_t S, void* ws) {
  PooledWs w;
  w.nblk = (S + sp::kPoolBlk - 1) / sp::kPoolBlk;
  const size_t Sr = (size_t)w.nblk * sp::kPoolBlk;
  uint8_t* base = static_cast<uint8_t*>(ws);
  w.req = base;                                                  // Sr is a multiple of 1024
  w.ckeys = reinterpret_cast<unsigned long long*>(base + Sr);
  w.cblk = reinterpret_cast<int32_t*>(w.ckeys + Sr);
  w.avail = w.cblk + Sr;
  w.misses = reinterpret_cast<sp::MissRec*>(w.avail + Sr);
  w.psel = reinterpret_cast<sp::PoolSel*>(w.misses + Sr);
  w.totals = reinterpret_cast<uint32_t*>(w.psel + 1);
  w.blk_free = reinterpret_cast<int32_t*>(w.totals + 2);
  w.blk_off = w.blk_free + w.nblk;
  w.counts = w.blk_off + w.nblk;
  w.moff = w.counts + 2 * (size_t)B;
  w.placed = w.moff + B;
  return w;
}

sparse_status resolve_pooled(const sparse_dims* dims, int shift, const int32_t* sel_counts,
                             const int32_t* sel_pages, int32_t S, int32_t* slot_tag,
                             int32_t* slot_stamp, int32_t* unit_slot, int32_t* step_counter,
                             int32_t* sel_phys, int32_t* hit_phys, int32_t* stats, void* ws,
                             MissLists ml, hipStream_t s) {
  const int B = dims->batch, hkv = dims->num_kv_heads, MP = dims->max_pages;
  const PooledWs w = pooled_ws(B, S, ws);
  hipLaunchKernelGGL(sp::pool_mark_kernel, dim3(B), dim3(sp::kResThreads), 0, s, sel_counts,
                     sel_pages, hkv, MP, S, step_counter, slot_stamp, unit_slot, sel_phys,
                     hit_phys, w.req, w.counts);
  if (hipGetLastError() != hipSuccess) return SPARSE_ERR_HIP;
  // pooled unit ids: (b * Hkv + h) * max_pages + p
  const int tag_bits = sp::unit_tag_bits((long long)B * hkv * MP);
  hipLaunchKernelGGL(sp::pool_scan_kernel, dim3(w.nblk), dim3(sp::kPoolBlkThreads), 0, s, S,
                     shift, tag_bits, slot_tag, slot_stamp, w.req, w.ckeys, w.cblk, w.blk_free,
                     w.totals);
  if (hipGetLastError() != hipSuccess) return SPARSE_ERR_HIP;
  hipLaunchKernelGGL(sp::pool_select_kernel, dim3(1), dim3(sp::kResThreads), 0, s, B, w.nblk,
                     w.counts, w.moff, w.ckeys, w.cblk, w.blk_free, w.totals, w.blk_off, w.psel);
  if (hipGetLastError() != hipSuccess) return SPARSE_ERR_HIP;
  hipLaunchKernelGGL(sp::pool_avail_kernel, dim3(w.nblk), dim3(sp::kPoolBlkThreads), 0, s, S,
                     shift, tag_bits, slot_tag, slot_stamp, w.req, w.psel, w.blk_off, w.avail,
                     w.placed);
  if (hipGetLastError() != hipSuccess) return SPARSE_ERR_HIP;
  hipLaunchKernelGGL(sp::pool_place_kernel, dim3(B), dim3(sp::kResThreads), 0, s, sel_counts,
                     sel_pages, hkv, MP, step_counter, slot_tag, slot_stamp, unit_slot, sel_phys,
                     stats, w.counts, w.moff, w.avail, w.placed, w.misses);
  if (ml.counts) {
    if (hipGetLastError() != hipSuccess) return SPARSE_ERR_HIP;
    hipLaunchKernelGGL(sp::split_misses_kernel, dim3(B * hkv), dim3(sp::kSplitThreads), 0, s,
                       sel_counts, sel_pages, sel_phys, hit_phys, MP, ml.counts, ml.pages,
                       ml.phys);
  }
  return sp::launch_status();
}

sparse_status fetch_pooled(const sparse_dims* dims, const uint16_t* host_kv, uint16_t* cache_kv,
                           int32_t S, int32_t* step_counter, void* ws, hipStream_t s) {
  const PooledWs w = pooled_ws(dims->batch, S, ws);
  hipLaunchKernelGGL(sp::pool_fetch_kernel, dim3(kFetchWaves / sp::kFetchWavesPerGroup),
                     dim3(sp::kFetchThreads), 0, s, host_kv, cache_kv, dims->num_kv_heads,
                     dims->max_pages, w.misses, w.placed, kFetchWaves, step_counter);
  return sp::launch_status();
}

}  // namespace

extern "C" sparse_status sparse_hbm_cache_resolve(
    const sparse_dims* dims, const int32_t* sel_counts, const int32_t* sel_pages,
    const uint16_t* host_kv, uint16_t* cache_kv, int32_t capacity, int32_t* slot_tag,
    int32_t* slot_stamp, int32_t* unit_slot, int32_t* step_counter, int32_t* sel_phys,
    int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
  const sparse_cache_policy exact = {0, 0};
  return sparse_hbm_cache_resolve_policy(dims, &exact, sel_counts, sel_pages, host_kv, cache_kv,
                                         capacity, slot_tag, slot_stamp, unit_slot, step_counter,
                                         sel_phys, stats, ws, ws_bytes, stream);
}

extern "C" size_t sparse_cache_policy_workspace_bytes(const sparse_dims* dims,
                                                      const sparse_cache_policy* policy,
                                                      int32_t capacity) {
  if (!policy || sp::check_dims(dims) != SPARSE_OK || capacity < 1) return 0;
  if (policy->pooled) return pooled_ws_bytes(dims->batch, capacity);
  return sparse_cache_workspace_bytes(dims, capacity);
}

namespace {

// The policy and the capacity it allows (no workspace).
sparse_status check_policy_args(const sparse_dims* dims, const sparse_cache_policy* policy,
                                int32_t capacity) {
  if (!policy || policy->recency_shift < 0 || policy->recency_shift > 30 ||
      (policy->pooled != 0 && policy->pooled != 1))
    return SPARSE_ERR_INVALID;
  const int64_t units = (int64_t)dims->batch * dims->num_kv_heads * dims->max_pages;
  if (policy->pooled) {
    if (capacity > sp::kMaxPoolSlots || units > INT32_MAX) return SPARSE_ERR_UNSUPPORTED;
  } else if (capacity > sp::kMaxSlots) {
    return SPARSE_ERR_UNSUPPORTED;
  }
  return SPARSE_OK;
}

sparse_status check_policy(const sparse_dims* dims, const sparse_cache_policy* policy,
                           int32_t capacity, const void* ws, size_t ws_bytes) {
  const sparse_status st = check_policy_args(dims, policy, capacity);
  if (st != SPARSE_OK) return st;
  if (!ws || ws_bytes < sparse_cache_policy_workspace_bytes(dims, policy, capacity) ||
      !sp::aligned(ws, 8))
    return SPARSE_ERR_WORKSPACE;
  return SPARSE_OK;
}

sparse_status resolve_any(const sparse_dims* dims, const sparse_cache_policy* policy,
                          const int32_t* sel_counts, const int32_t* sel_pages, int32_t capacity,
                          int32_t* slot_tag, int32_t* slot_stamp, int32_t* unit_slot,
                          int32_t* step_counter, int32_t* sel_phys, int32_t* hit_phys,
                          int32_t* stats, void* ws, MissLists ml, hipStream_t s) {
  if (policy->pooled)
    return resolve_pooled(dims, policy->recency_shift, sel_counts, sel_pages, capacity, slot_tag,
                          slot_stamp, unit_slot, step_counter, sel_phys, hit_phys, stats, ws, ml,
                          s);
  return resolve_per_request(dims, policy->recency_shift, sel_counts, sel_pages, capacity,
                             slot_tag, slot_stamp, unit_slot, step_counter, sel_phys, hit_phys,
                             stats, ws, ml, nullptr, nullptr, s);
}

sparse_status fetch_any(const sparse_dims* dims, const sparse_cache_policy* policy,
                        const uint16_t* host_kv, uint16_t* cache_kv, int32_t capacity,
                        int32_t* step_counter, void* ws, hipStream_t s) {
  if (policy->pooled) return fetch_pooled(dims, host_kv, cache_kv, capacity, step_counter, ws, s);
  return fetch_per_request(dims, host_kv, cache_kv, capacity, step_counter, ws, s);
}

}  // namespace

extern "C" sparse_status sparse_hbm_cache_resolve_policy(
    const sparse_dims* dims, const sparse_cache_policy* policy, const int32_t* sel_counts,
    const int32_t* sel_pages, const uint16_t* host_kv, uint16_t* cache_kv, int32_t capacity,
    int32_t* slot_tag, int32_t* slot_stamp, int32_t* unit_slot, int32_t* step_counter,
    int32_t* sel_phys, int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
  sparse_status st = check_resolve_args(dims, sel_counts, sel_pages, capacity, slot_tag,
                                        slot_stamp, unit_slot, step_counter, sel_phys, stats);
  if (st != SPARSE_OK) return st;
  if ((st = check_pool_args(host_kv, cache_kv)) != SPARSE_OK) return st;
  if ((st = check_policy(dims, policy, capacity, ws, ws_bytes)) != SPARSE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (!policy->pooled)          // one launch: the resolve copies its requests' misses itself
    return resolve_per_request(dims, policy->recency_shift, sel_counts, sel_pages, capacity,
                               slot_tag, slot_stamp, unit_slot, step_counter, sel_phys, nullptr,
                               stats, ws, MissLists{nullptr, nullptr, nullptr}, host_kv,
                               cache_kv, s);
  if ((st = resolve_any(dims, policy, sel_counts, sel_pages, capacity, slot_tag, slot_stamp,
                        unit_slot, step_counter, sel_phys, nullptr, stats, ws,
                        MissLists{nullptr, nullptr, nullptr}, s)) != SPARSE_OK)
    return st;
  return fetch_any(dims, policy, host_kv, cache_kv, capacity, step_counter, ws, s);
}

extern "C" sparse_status sparse_hbm_cache_resolve_split(
    const sparse_dims* dims, const sparse_cache_policy* policy, const int32_t* sel_counts,
    const int32_t* sel_pages, int32_t capacity, int32_t* slot_tag, int32_t* slot_stamp,
    int32_t* unit_slot, int32_t* step_counter, int32_t* sel_phys, int32_t* hit_phys,
    int32_t* stats, int32_t* miss_counts, int32_t* miss_pages, int32_t* miss_phys, void* ws,
    size_t ws_bytes, void* stream) {
  sparse_status st = check_resolve_args(dims, sel_counts, sel_pages, capacity, slot_tag,
                                        slot_stamp, unit_slot, step_counter, sel_phys, stats);
  if (st != SPARSE_OK) return st;
  if (!hit_phys) return SPARSE_ERR_INVALID;
  const bool any = miss_counts || miss_pages || miss_phys;
  if (any && !(miss_counts && miss_pages && miss_phys)) return SPARSE_ERR_INVALID;
  if ((st = check_policy(dims, policy, capacity, ws, ws_bytes)) != SPARSE_OK) return st;
  return resolve_any(dims, policy, sel_counts, sel_pages, capacity, slot_tag, slot_stamp,
                     unit_slot, step_counter, sel_phys, hit_phys, stats, ws,
                     MissLists{miss_counts, miss_pages, miss_phys}, (hipStream_t)stream);
}

extern "C" sparse_status sparse_hbm_cache_fetch(const sparse_dims* dims,
                                                const sparse_cache_policy* policy,
                                                const uint16_t* host_kv, uint16_t* cache_kv,
                                                int32_t capacity, int32_t* step_counter,
                                                void* ws, size_t ws_bytes, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!step_counter || capacity < 1) return SPARSE_ERR_INVALID;
  if ((st = check_pool_args(host_kv, cache_kv)) != SPARSE_OK) return st;
  if (dims->num_kv_heads > sp::kMaxKvHeads) return SPARSE_ERR_UNSUPPORTED;
  if ((st = check_policy(dims, policy, capacity, ws, ws_bytes)) != SPARSE_OK) return st;
  return fetch_any(dims, policy, host_kv, cache_kv, capacity, step_counter, ws,
                   (hipStream_t)stream);
}

extern "C" sparse_status sparse_hbm_cache_fetch_attn(
    const sparse_dims* dims, const sparse_cache_policy* policy, const uint16_t* host_kv,
    uint16_t* cache_kv, int32_t capacity, int32_t* step_counter, const uint16_t* q,
    const int32_t* ctx_lens, const int32_t* sel_counts, const int32_t* sel_pages,
    const int32_t* hit_phys, const int32_t* miss_counts, const int32_t* miss_pages,
    const int32_t* miss_phys, float scale, int32_t workers, float* part_o, float* part_lse,
    int64_t max_parts, float* miss_part_o, float* miss_part_lse, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!step_counter || capacity < 1) return SPARSE_ERR_INVALID;
  if ((st = check_pool_args(host_kv, cache_kv)) != SPARSE_OK) return st;
  if ((st = check_policy_args(dims, policy, capacity)) != SPARSE_OK) return st;
  const int B = dims->batch;
  const int64_t slots = policy->pooled ? (int64_t)capacity : (int64_t)B * capacity;
  int wmax = 0;
  if ((st = sp::check_attn(dims, q, cache_kv, sp::kUnitElems, 0, slots, ctx_lens, sel_counts,
                           sel_pages, hit_phys, scale, workers, wmax)) != SPARSE_OK)
    return st;
  if (!part_o || !part_lse || !sp::aligned(part_o, 16)) return SPARSE_ERR_INVALID;
  if (max_parts != (int64_t)B * dims->num_kv_heads + wmax) return SPARSE_ERR_INVALID;
  if (!miss_counts || !miss_pages || !miss_phys || !miss_part_o || !miss_part_lse ||
      !sp::aligned(miss_part_o, 16))
    return SPARSE_ERR_INVALID;
  sp::enqueue_fetch_attn(dims, host_kv, cache_kv, slots, step_counter, q, ctx_lens, sel_counts,
                         sel_pages, hit_phys, miss_counts, miss_pages, miss_phys, scale, wmax,
                         part_o, part_lse, miss_part_o, miss_part_lse, (hipStream_t)stream);
  return sp::launch_status();
}

extern "C" sparse_status sparse_split_misses(const sparse_dims* dims, const int32_t* sel_counts,
                                             const int32_t* sel_pages, const int32_t* sel_phys,
                                             const int32_t* hit_phys, int32_t* miss_counts,
                                             int32_t* miss_pages, int32_t* miss_phys,
                                             void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!sel_counts || !sel_pages || !sel_phys || !hit_phys || !miss_counts || !miss_pages ||
      !miss_phys)
    return SPARSE_ERR_INVALID;
  const int U = dims->batch * dims->num_kv_heads;
  hipLaunchKernelGGL(sp::split_misses_kernel, dim3(U), dim3(sp::kSplitThreads), 0,
                     (hipStream_t)stream, sel_counts, sel_pages, sel_phys, hit_phys,
                     dims->max_pages, miss_counts, miss_pages, miss_phys);
  return sp::launch_status();
}
