// Victim selection of the host-tier cache resolvers: the r-th smallest
// replacement key among candidate slots, by radix select on LDS histograms.
#pragma once

#include "common.h"

namespace sp {

// Replacement order of resident units: stamps compared in buckets of
// 2^shift steps, then the unit id (shift 0 = exact LRU, ties to the lower id).
__device__ __forceinline__ unsigned long long lru_key(int32_t stamp, int32_t tag, int shift) {
  return ((unsigned long long)((uint32_t)stamp >> shift) << 32) | (uint32_t)tag;
}

// hist[bin] += 1 for every lane with `valid`.  Keys of resident units
// cluster (few distinct stamps), so in the first radix pass the lanes of a
// wave often all fall in one bin: then one atomic adds their count.  Every
// lane of the wave calls (wave-uniform control flow).
__device__ __forceinline__ void hist_add_wave(uint32_t* hist, int bin, bool valid) {
  const unsigned long long act = __ballot(valid);
  if (!act) return;
  const int l0 = __ffsll((long long)act) - 1;
  const int b0 = __shfl(bin, l0, 64);
  if ((__ballot(bin == b0) & act) == act) {
    if (lane_id() == l0) atomicAdd(&hist[b0], (uint32_t)__popcll(act));
  } else if (valid) {
    atomicAdd(&hist[bin], 1u);
  }
}

struct SelectScratch {
  uint32_t hist[2048];
  uint32_t scan32[16];
  unsigned long long red_lo[16], red_hi[16];
  int bin;
  uint32_t below;
};

// The r-th smallest key (1 <= r < number of candidates) over slots [0, C),
// where key_of(s, key) returns whether slot s is a candidate and its key.
// Keys must be distinct.  Every thread of the NT-thread workgroup calls;
// contains barriers.
template <int NT, typename KeyOf>
__device__ unsigned long long select_rth_key(int C, uint32_t r, KeyOf key_of, SelectScratch& sc) {
  const int tid = threadIdx.x;
  constexpr int kB = 8;   // slots per thread whose loads are issued together
  unsigned long long kmin = ~0ull, kmax = 0ull;
  for (int base = 0; base < C; base += kB * NT) {
    unsigned long long key[kB] = {};
    bool ok[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int s = base + k * NT + tid;
      ok[k] = (s < C) && key_of(s, key[k]);
    }
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (ok[k]) {
        kmin = min(kmin, key[k]);
        kmax = max(kmax, key[k]);
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (unsigned long long)__shfl_xor((long long)kmin, o, 64));
    kmax = max(kmax, (unsigned long long)__shfl_xor((long long)kmax, o, 64));
  }
  if (lane_id() == 0) {
    sc.red_lo[tid >> 6] = kmin;
    sc.red_hi[tid >> 6] = kmax;
  }
  __syncthreads();
  kmin = ~0ull;
  kmax = 0ull;
  for (int w = 0; w < NT / 64; ++w) {
    kmin = min(kmin, sc.red_lo[w]);
    kmax = max(kmax, sc.red_hi[w]);
  }
  const int top = 63 - __clzll(kmin ^ kmax);   // kmin != kmax: at least two candidates
  unsigned long long hi_mask = (top == 63) ? 0ull : ~((2ull << top) - 1ull);
  unsigned long long prefix = kmin & hi_mask;
  uint32_t need = r;                            // keys still to take, ascending
  int lo = top + 1;
  while (lo > 0) {
    const int width = min(11, lo);
    const int sh = lo - width, nb = 1 << width;
    for (int k = tid; k < nb; k += NT) sc.hist[k] = 0u;
    __syncthreads();
    // uniform trip count over the workgroup: the wave votes stay converged
    for (int base = 0; base < C; base += kB * NT) {
      unsigned long long key[kB] = {};
      bool ok[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int s = base + k * NT + tid;
        ok[k] = (s < C) && key_of(s, key[k]);
      }
#pragma unroll
      for (int k = 0; k < kB; ++k)
        hist_add_wave(sc.hist, (int)((key[k] >> sh) & (nb - 1)),
                      ok[k] && (key[k] & hi_mask) == prefix);
    }
    __syncthreads();
    // the bin where the count from the bottom reaches `need`
    const int b0 = 2 * tid, b1 = 2 * tid + 1;
    const uint32_t c0 = (b0 < nb) ? sc.hist[b0] : 0u, c1 = (b1 < nb) ? sc.hist[b1] : 0u;
    uint32_t tot;
    const uint32_t below0 = block_excl_scan<uint32_t, NT>(c0 + c1, sc.scan32, tot);
    const uint32_t below1 = below0 + c0;
    if (b0 < nb && below0 < need && need <= below0 + c0) {
      sc.bin = b0;
      sc.below = below0;
    }
    if (b1 < nb && below1 < need && need <= below1 + c1) {
      sc.bin = b1;
      sc.below = below1;
    }
    __syncthreads();
    need -= sc.below;
    prefix |= (unsigned long long)sc.bin << sh;
    hi_mask |= (unsigned long long)(nb - 1) << sh;
    lo = sh;
    __syncthreads();
  }
  return prefix;
}

}  // namespace sp
