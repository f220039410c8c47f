// Victim selection of the host-tier cache resolvers: the r-th smallest
// replacement key among candidate slots, by radix select on LDS histograms.
#pragma once

#include "common.h"

namespace sp {

// Replacement order of resident units: stamps compared in buckets of
// 2^shift steps, then the unit id (shift 0 = exact LRU, ties to the lower id).
// The unit id takes the low `tag_bits` bits (enough for every unit id of the
// cache), the stamp bucket the bits above: the keys of one cache then span
// only the bits in which recent stamps and unit ids differ, so the radix
// select below needs few passes.  Every user of one cache's keys must pass
// the same tag_bits.
__device__ __forceinline__ unsigned long long lru_key(int32_t stamp, int32_t tag, int shift,
                                                     int tag_bits) {
  return ((unsigned long long)((uint32_t)stamp >> shift) << tag_bits) | (uint32_t)tag;
}

// Bits that hold unit ids 0 .. n - 1 (n >= 1).
__host__ __device__ inline int unit_tag_bits(long long n) {
  int b = 1;
  while (b < 62 && (1ll << b) < n) ++b;
  return b;
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

constexpr int kSelDigitBits = 12;              // radix digit of the select
constexpr int kSelBins = 1 << kSelDigitBits;

struct SelectScratch {
  uint32_t hist[2][kSelBins];                   // alternate passes
  uint32_t wsum[16];
  unsigned long long red_lo[16], red_hi[16];
  int bin;
  uint32_t below;
};

// The r-th smallest key (1 <= r < number of candidates) over slots [0, C),
// where key_of(s, key) returns whether slot s is a candidate and its key.
// Keys must be distinct.  Every thread of the NT-thread workgroup calls;
// contains barriers.  Radix select from the highest bit in which the keys
// differ, 12 bits per pass, three barriers per pass: the histogram, the scan
// of its bins (wave scans, then the wave totals through LDS), and the bin
// that holds the r-th key.  The two histogram buffers alternate, so a pass
// clears the next one's while it fills its own.
template <int NT, typename KeyOf>
__device__ unsigned long long select_rth_key(int C, uint32_t r, KeyOf key_of, SelectScratch& sc) {
  static_assert(NT % 64 == 0 && NT / 64 <= 16 && kSelBins % NT == 0, "select workgroup size");
  constexpr int BPT = kSelBins / NT;            // bins per thread in the scan
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  constexpr int kB = 8;   // slots per thread whose loads are issued together
  for (int k = tid; k < kSelBins; k += NT) sc.hist[0][k] = 0u;
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
  if (lane == 0) {
    sc.red_lo[wv] = kmin;
    sc.red_hi[wv] = kmax;
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
  int lo = top + 1, buf = 0;
  while (lo > 0) {
    const int width = min(kSelDigitBits, lo);
    const int sh = lo - width, nb = 1 << width;
    uint32_t* hist = sc.hist[buf];
    // the next pass's buffer: its last readers finished before the previous
    // pass's final barrier
    for (int k = tid; k < kSelBins; k += NT) sc.hist[buf ^ 1][k] = 0u;
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
        hist_add_wave(hist, (int)((key[k] >> sh) & (nb - 1)),
                      ok[k] && (key[k] & hi_mask) == prefix);
    }
    __syncthreads();
    // thread t owns bins t * BPT .. t * BPT + BPT - 1 (bins past nb are 0)
    uint32_t c[BPT], sum = 0u;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      c[i] = hist[tid * BPT + i];
      sum += c[i];
    }
    const uint32_t incl = wave_incl_scan(sum);
    if (lane == 63) sc.wsum[wv] = incl;
    __syncthreads();
    uint32_t below = incl - sum;
    for (int w = 0; w < wv; ++w) below += sc.wsum[w];
    // the bin where the count from the bottom reaches `need` (one thread)
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (below < need && need <= below + c[i]) {
        sc.bin = tid * BPT + i;
        sc.below = below;
      }
      below += c[i];
    }
    __syncthreads();
    need -= sc.below;
    prefix |= (unsigned long long)sc.bin << sh;
    hi_mask |= (unsigned long long)(nb - 1) << sh;
    lo = sh;
    buf ^= 1;
  }
  return prefix;
}

}  // namespace sp
