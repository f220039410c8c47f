// The coverage rule with several workgroups per unit ("Adaptive DHiSparse:
// Speculative Decoding over a Load-Adaptive KV Hierarchy", MOIRA abstract,
// coverage-rule sentence: per request, layer, KV head and step, keep the
// fewest pages that together hold at least gamma of the estimated mass).
//
// The single-workgroup selection (select.hip) runs one workgroup per unit, a
// chain of block-wide steps on one compute unit; with few units (4 requests x
// 8 KV heads) most of the chip idles while it runs.  Here K workgroups of
// 1024 threads share a unit: member m owns the unit's logical pages
// [m P, (m + 1) P) and keeps their logits in its LDS, and the members agree on
// the unit-wide quantities through device memory:
//   1. per-head max and sum of exp over the member's pages -> partials;
//      every member combines the K partials (in member order: identical bits
//      everywhere) into the unit's normalisers M_g, S_g;
//   2. group masses m = (1/G) sum_g exp(x_g - M_g) / S_g, keys = fp32 bits,
//      fixed-point weights floor(m 2^52); the unit's key range;
//   3. mass-weighted radix passes over the key bits below the highest bit in
//      which the unit's keys differ: each member adds its histogram to the
//      unit's (integer atomics, order independent), every member then finds
//      the same crossing bin; once it holds at most 64 pages they are
//      gathered and sorted by (key desc, page asc) to fix the cut key tau and
//      the number of ties at tau to keep;
//   4. each member's kept and tied page counts -> every member places its
//      kept pages in the unit's ascending list.
// The cut is the one select.hip computes (same masses up to the summation
// order of S_g, same exact fixed-point sums, same tie rule).
//
// With SCORE = true the members also score their own pages from the page
// summaries (the Quest-style bound on the matrix cores, as score.hip), so the
// logits never leave the chip: scoring and selection in one kernel.
//
// Agreement between members: values are exchanged with device-scope atomic
// stores, loads and adds (coherent across the XCDs' separate L2 caches
// without a device-scope fence, which writes back and invalidates a whole L2
// and costs 5-7 us); a barrier waits for the member's stores to complete,
// then counts the member in with a device-scope atomic add and polls the
// count.  Every member of a unit must be resident at once: the host launches
// the cooperative form only when the whole grid fits the device.  A barrier
// that waits longer than ~100 ms gives up and sets the workspace's error
// word (outputs invalid) rather than hang.

#include <stddef.h>

#include "common.h"
#include "reduce.h"

namespace sp {

constexpr int kCoopThreads = 1024;
constexpr int kCoopWaves = kCoopThreads / 64;
constexpr int kCoopMaxK = 8;                 // workgroups per unit
constexpr int kCoopMaxPasses = 3;            // 11-bit radix passes over 32-bit keys
constexpr int kCoopMaxPages = 2048;          // pages per member
constexpr long long kCoopTimeoutTicks = 10000000;   // 100 ms of the 100 MHz clock

// One unit's exchange area in the workspace (zero-filled once by the
// caller; the last member of every unit to finish leaves it zeroed again).
struct CoopUnit {
  uint32_t sync;                 // arrivals at the unit's barriers
  uint32_t done;                 // members finished with the shared state
  uint32_t ncand;                // candidates appended in the final pass
  uint32_t pad0[13];
  float part_m[kCoopMaxK][kMaxGroup];
  float part_s[kCoopMaxK][kMaxGroup];
  uint32_t klo[kCoopMaxK], khi[kCoopMaxK];
  uint32_t above[kCoopMaxK], ties[kCoopMaxK];
  uint32_t cand_key[64], cand_page[64];
  uint32_t hc[kCoopMaxPasses][2048];
  unsigned long long hw[kCoopMaxPasses][2048];
};

struct CoopHeader {
  uint32_t err;                  // nonzero: a barrier timed out
  uint32_t pad[63];
};

__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev(unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier number s (1, 2, ...) of the unit's K members.  Every thread's
// earlier device-scope stores and atomics have completed before the member
// is counted in.  All threads of the workgroup call it.
__device__ __forceinline__ void coop_barrier(CoopUnit* cu, uint32_t s, int K, uint32_t* err) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&cu->sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t target = s * (uint32_t)K;
    const long long t0 = wall_clock64();
    while (ld_dev(&cu->sync) < target) {
      if (wall_clock64() - t0 > kCoopTimeoutTicks) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// SCORE: score the member's pages from the summaries (TPW 16-page tiles per
// wave); else read the unit's logits.  NPT = pages per thread in the select
// phases (the member's pages are TPW * 256 = NPT * 1024).
template <bool SCORE, int TPW>
__global__ __launch_bounds__(kCoopThreads) void coop_select_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ summ, int64_t pool_pages,
    const float* __restrict__ logits, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, float scale, float gamma, int hkv, int group,
    int max_pages, int K, unsigned char* __restrict__ ws, int32_t* __restrict__ sel_counts,
    int32_t* __restrict__ sel_pages, int32_t* __restrict__ sel_phys) {
  constexpr int PB = TPW * 16 * kCoopWaves;              // pages per member
  constexpr int NPT = (PB + kCoopThreads - 1) / kCoopThreads;
  static_assert(PB <= kCoopMaxPages, "member block");
  extern __shared__ float xl[];                          // [group][PB] logits
  __shared__ uint32_t hcnt[2048];
  __shared__ unsigned long long hwt[2048];
  __shared__ float red_f[kMaxGroup][kCoopWaves];
  __shared__ uint32_t red_u[2][kCoopWaves];
  __shared__ unsigned long long red64[kCoopWaves];
  __shared__ float s_loc[kMaxGroup], s_M[kMaxGroup], s_invS[kMaxGroup];
  __shared__ uint32_t s_cnt[2][kCoopMaxK];
  __shared__ uint32_t cand_key[64], cand_page[64];
  __shared__ int s_bin;
  __shared__ unsigned long long s_wgt;
  __shared__ uint32_t s_tau, s_need, s_last;

  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int u = blockIdx.x / K, m = blockIdx.x - (blockIdx.x / K) * K;
  const int b = u / hkv, h = u - (u / hkv) * hkv;
  uint32_t* err = &reinterpret_cast<CoopHeader*>(ws)->err;
  CoopUnit* cu = reinterpret_cast<CoopUnit*>(ws + sizeof(CoopHeader)) + u;
  const int32_t* pt = page_table + (int64_t)b * max_pages;
  const int L = min(max(ctx_lens[b], 0), max_pages * kP);
  const int n = (L + kP - 1) / kP;                       // the unit's pages
  if (n == 0) {                                          // the same for every member
    if (m == 0 && tid == 0) sel_counts[u] = 0;
    return;
  }
  const int p0 = m * PB;                                 // the member's first page
  const int nb = min(max(n - p0, 0), PB);                // its pages in the context

  // ---- scores (or logits) of the member's pages into LDS -------------------
  if constexpr (SCORE) {
    const int row = lane & 15, j = lane >> 4;
    // B operands: q- for the kmin half, q+ for the kmax half (as score.hip)
    bf16x8 qneg[4], qpos[4];
    {
      const int hq = h * group + min(row, group - 1);
      const uint32_t gmask = (row < group) ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 w = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * hkv * group + hq) * kD +
                                                  32 * s + 8 * j);
        w &= gmask;
        u32x4 neg, pos;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t sgn = (w[e] >> 15) & 0x00010001u;
          const uint32_t mk = sgn * 0xFFFFu;
          neg[e] = w[e] & mk;
          pos[e] = w[e] & ~mk;
        }
        qneg[s] = as_bf16x8(neg);
        qpos[s] = as_bf16x8(pos);
      }
    }
    // wave wv scores tiles wv, wv + 16, ...: page ids of all its tiles first
    // (unconditional loads, clamped to the context), then the summaries of
    // tile i + 1 in flight while the matrix cores work on tile i
    int xid[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int p = p0 + 16 * (wv + kCoopWaves * i) + row;
      const int x = pt[min(p, n - 1)];
      xid[i] = (p < n) ? x : -1;
    }
    const float ln16 = 2.772588722239781f;
    u32x4 a[2][8];
    bool oks[2];
    auto issue = [&](int i, int slot) {
      const int x = xid[i];
      const bool ok = (x >= 0) && (x < pool_pages);
      oks[slot] = ok;
      const uint16_t* src = summ + ((int64_t)(ok ? x : 0) * hkv + h) * (2 * kD) + 8 * j;
#pragma unroll
      for (int s = 0; s < 8; ++s) a[slot][s] = *reinterpret_cast<const u32x4*>(src + 32 * s);
    };
    issue(0, 0);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (i + 1 < TPW) issue(i + 1, (i + 1) & 1);
      const int slot = i & 1;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[slot][s]), qneg[s], acc, 0, 0,
                                                      0);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[slot][4 + s]), qpos[s], acc,
                                                      0, 0, 0);
      const unsigned long long okm = __ballot(oks[slot]);
      const int t16 = 16 * (wv + kCoopWaves * i);       // tile's first page in the block
      if (row < group) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pl = t16 + 4 * j + e;                // page within the block
          const int pg = p0 + pl;                        // logical page
          const bool ok = ((okm >> (4 * j + e)) & 1ull) && pg < n;
          const int nv = min(kP, L - kP * pg);
          const float lnv = (nv >= kP) ? ln16 : logf((float)max(nv, 1));
          xl[row * PB + pl] = ok ? fmaf(scale, acc[e], lnv) : -INFINITY;
        }
      }
    }
  } else {
    const float* X = logits + (int64_t)u * group * max_pages;
    for (int g = 0; g < group; ++g)
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int i = k * kCoopThreads + tid;
        if (i < PB) {
          const float v = X[(int64_t)g * max_pages + min(p0 + i, max_pages - 1)];
          xl[g * PB + i] = (i < nb) ? v : -INFINITY;
        }
      }
  }
  __syncthreads();

  // ---- 1. the unit's per-head normalisers ---------------------------------
  // thread t owns the member's pages t * NPT .. t * NPT + NPT - 1.  Per-head
  // values live in LDS (a head index known only at run time would put
  // per-thread arrays in scratch memory).
  const int pbase = tid * NPT;
  for (int g = 0; g < group; ++g) {
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      if (pbase + k < nb) mx = fmaxf(mx, xl[g * PB + pbase + k]);
    mx = wave_total_f32(mx, OpMax());
    if (lane == 0) red_f[g][wv] = mx;
  }
  __syncthreads();
  if (tid < group) {
    float mx = red_f[tid][0];
#pragma unroll
    for (int w = 1; w < kCoopWaves; ++w) mx = fmaxf(mx, red_f[tid][w]);
    s_loc[tid] = mx;                                   // member max of head tid
  }
  __syncthreads();
  for (int g = 0; g < group; ++g) {
    const float mg = s_loc[g];
    float se = 0.f;
    if (mg != -INFINITY) {
#pragma unroll
      for (int k = 0; k < NPT; ++k)
        if (pbase + k < nb) se += __expf(xl[g * PB + pbase + k] - mg);
    }
    se = wave_total_f32(se, OpAdd());
    if (lane == 0) red_f[g][wv] = se;
  }
  __syncthreads();
  if (tid < group) {
    float se = red_f[tid][0];
#pragma unroll
    for (int w = 1; w < kCoopWaves; ++w) se += red_f[tid][w];
    st_dev(&cu->part_m[m][tid], s_loc[tid]);
    st_dev(&cu->part_s[m][tid], se);
  }
  uint32_t bar = 1;
  coop_barrier(cu, bar++, K, err);
  if (tid < group) {
    // the unit's normalisers from the K partials, combined in member order
    // (identical bits in every member)
    float pm[kCoopMaxK], ps[kCoopMaxK];
#pragma unroll
    for (int mm = 0; mm < kCoopMaxK; ++mm) {
      pm[mm] = (mm < K) ? ld_dev(&cu->part_m[mm][tid]) : -INFINITY;
      ps[mm] = (mm < K) ? ld_dev(&cu->part_s[mm][tid]) : 0.f;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mm = 0; mm < kCoopMaxK; ++mm) mx = fmaxf(mx, pm[mm]);
    float S = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int mm = 0; mm < kCoopMaxK; ++mm)
        if (pm[mm] != -INFINITY) S += ps[mm] * __expf(pm[mm] - mx);
    }
    s_M[tid] = mx;
    s_invS[tid] = (S > 0.f) ? 1.f / S : 0.f;           // a head with no finite logit adds no mass
  }
  __syncthreads();

  // ---- 2. masses, keys and the unit's key range ---------------------------
  const float invg = 1.f / (float)group;
  uint32_t key[NPT];
  uint32_t klo = 0xFFFFFFFFu, khi = 0u;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = pbase + k;
    float ms = 0.f;
    if (i < nb) {
      for (int g = 0; g < group; ++g) {
        const float is = s_invS[g];
        if (is > 0.f) ms += __expf(xl[g * PB + i] - s_M[g]) * is;
      }
    }
    key[k] = __float_as_uint(ms * invg);
    if (i < nb) {
      klo = min(klo, key[k]);
      khi = max(khi, key[k]);
    }
  }
  klo = wave_total_u32(klo, OpMinU());
  khi = wave_total_u32(khi, OpMaxU());
  if (lane == 0) {
    red_u[0][wv] = klo;
    red_u[1][wv] = khi;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t lo = red_u[0][0], hi = red_u[1][0];
    for (int w = 1; w < kCoopWaves; ++w) {
      lo = min(lo, red_u[0][w]);
      hi = max(hi, red_u[1][w]);
    }
    st_dev(&cu->klo[m], lo);
    st_dev(&cu->khi[m], hi);
  }
  coop_barrier(cu, bar++, K, err);
  if (tid == 0) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int mm = 0; mm < K; ++mm) {
      lo = min(lo, ld_dev(&cu->klo[mm]));
      hi = max(hi, ld_dev(&cu->khi[mm]));
    }
    s_cnt[0][0] = lo;
    s_cnt[1][0] = hi;
  }
  __syncthreads();
  const uint32_t KLO = s_cnt[0][0], KHI = s_cnt[1][0];
  __syncthreads();

  // ---- 3. the cut ---------------------------------------------------------
  const bool all = !(gamma < 1.0f);
  uint32_t tau = 0u;
  unsigned long long need = 0ull;
  int passes = 0;
  if (!all) {
    auto target = [&](unsigned long long Z) {
      unsigned long long t = (unsigned long long)ceil((double)gamma * (double)Z);
      if (t > Z) t = Z;
      if (t < 1ull) t = 1ull;
      return t;
    };
    unsigned long long T = 0ull;
    unsigned long long w_tau = weight_of(KHI);
    if (KLO == KHI) {
      tau = KHI;                         // every page of the unit has the same mass
      T = target((unsigned long long)n * w_tau);
    } else {
      const int top = 31 - __clz(KLO ^ KHI);
      uint32_t hi_mask = ~((2u << top) - 1u);
      uint32_t prefix = KHI & hi_mask;
      int lo = top + 1;
      bool resolved = false, first = true;
      while (lo > 0 && passes < kCoopMaxPasses) {
        const int width = min(11, lo);
        const int sh = lo - width, nbins = 1 << width;
        const int ps = passes++;
        for (int k = tid; k < 2048; k += kCoopThreads) {
          hcnt[k] = 0u;
          hwt[k] = 0ull;
        }
        if (tid == 0) {
          s_bin = 0;
          s_wgt = 0ull;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          if (pbase + k < nb && (key[k] & hi_mask) == prefix) {
            const int bin = (key[k] >> sh) & (nbins - 1);
            atomicAdd(&hcnt[bin], 1u);
            atomicAdd(&hwt[bin], weight_of(key[k]));
          }
        }
        __syncthreads();
        for (int k = tid; k < nbins; k += kCoopThreads) {
          if (hcnt[k]) {
            __hip_atomic_fetch_add(&cu->hc[ps][k], hcnt[k], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&cu->hw[ps][k], hwt[k], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        coop_barrier(cu, bar++, K, err);
        {
          // every bin in one round of loads (bins past nbins are never
          // written, so they read 0)
          static_assert(2048 == 2 * kCoopThreads, "two bins per thread");
          uint32_t c0 = ld_dev(&cu->hc[ps][tid]), c1 = ld_dev(&cu->hc[ps][tid + kCoopThreads]);
          unsigned long long w0 = ld_dev(&cu->hw[ps][tid]);
          unsigned long long w1 = ld_dev(&cu->hw[ps][tid + kCoopThreads]);
          hcnt[tid] = c0;
          hcnt[tid + kCoopThreads] = c1;
          hwt[tid] = w0;
          hwt[tid + kCoopThreads] = w1;
        }
        __syncthreads();
        {
          // thread t owns bins 2t, 2t + 1; one barrier for the wave totals,
          // then only the wave whose bins hold the crossing scans them
          constexpr int BPT = 2048 / kCoopThreads;
          unsigned long long wb[BPT], wsum = 0ull;
#pragma unroll
          for (int i = 0; i < BPT; ++i) {
            wb[i] = hwt[BPT * tid + i];
            wsum += wb[i];
          }
          const unsigned long long wtot = wave_total_u64(wsum);
          if (lane == 0) red64[wv] = wtot;
          __syncthreads();
          if (first) {                   // the first pass holds every page: Z
            unsigned long long Z = 0ull;
#pragma unroll
            for (int w = 0; w < kCoopWaves; ++w) Z += red64[w];
            T = target(Z);
            first = false;
          }
          unsigned long long above = 0ull;
#pragma unroll
          for (int w = 0; w < kCoopWaves; ++w)
            if (w > wv) above += red64[w];
          if (above < T && T <= above + wtot) {
            unsigned long long gt = above + (wtot - wave_scan_u64(wsum));
#pragma unroll
            for (int i = BPT - 1; i >= 0; --i) {
              const int bi = BPT * tid + i;
              if (gt < T && T <= gt + wb[i]) {
                s_bin = bi;
                s_wgt = gt;
              }
              gt += wb[i];
            }
          }
        }
        __syncthreads();
        const int bin = s_bin & (nbins - 1);
        T -= s_wgt;
        prefix |= (uint32_t)bin << sh;
        hi_mask |= (uint32_t)(nbins - 1) << sh;
        const uint32_t cbin = hcnt[bin];
        if (sh == 0) {
          w_tau = cbin ? hwt[bin] / cbin : 1ull;   // every page at tau has one weight
          lo = 0;
          break;
        }
        lo = sh;
        if (cbin <= 64u) {
          // the few pages sharing the resolved high bits: gather, then one
          // wave sorts them by (key desc, page asc) and walks their weights
#pragma unroll
          for (int k = 0; k < NPT; ++k) {
            if (pbase + k < nb && (key[k] & hi_mask) == prefix) {
              const uint32_t at = __hip_atomic_fetch_add(&cu->ncand, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
              if (at < 64u) {
                st_dev(&cu->cand_key[at], key[k]);
                st_dev(&cu->cand_page[at], (uint32_t)(p0 + pbase + k));
              }
            }
          }
          coop_barrier(cu, bar++, K, err);
          const uint32_t nc = min(cbin, 64u);
          if (tid < (int)nc) {
            cand_key[tid] = ld_dev(&cu->cand_key[tid]);
            cand_page[tid] = ld_dev(&cu->cand_page[tid]);
          }
          __syncthreads();
          if (wv == 0) {
            const bool ok = (uint32_t)lane < nc;
            unsigned long long c =
                ok ? (((unsigned long long)(~cand_key[lane]) << 32) | cand_page[lane]) : ~0ull;
#pragma unroll
            for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
              for (int jj = kk >> 1; jj > 0; jj >>= 1) {
                const unsigned long long o =
                    (unsigned long long)__shfl_xor((long long)c, jj, 64);
                const bool up = (lane & kk) == 0, low = (lane & jj) == 0;
                c = (low == up) ? min(c, o) : max(c, o);
              }
            }
            const uint32_t kk = ~(uint32_t)(c >> 32);
            const unsigned long long wk = ok ? weight_of(kk) : 0ull;
            const unsigned long long cum = wave_scan_u64(wk);
            const unsigned long long reach = __ballot(ok && cum >= T);
            const int at = __ffsll((long long)reach) - 1;
            const uint32_t t_key = (uint32_t)__shfl((int)kk, at, 64);
            const unsigned long long eq = __ballot(ok && kk == t_key);
            const int first_eq = __ffsll((long long)eq) - 1;
            if (lane == 0) {
              s_tau = t_key;
              s_need = (uint32_t)(at - first_eq + 1);
            }
          }
          __syncthreads();
          resolved = true;
          break;
        }
      }
      if (resolved) {
        tau = s_tau;
        need = s_need;
      } else {
        tau = prefix;
      }
    }
    if (need == 0ull) {
      if (w_tau == 0ull) w_tau = 1ull;
      need = (T + w_tau - 1ull) / w_tau;   // pages at tau to keep (>= 1)
    }
  }

  // ---- 4. the unit's list in ascending page order --------------------------
  // high half: pages above tau (every page when gamma = 1); low half: ties
  uint32_t packed = 0u;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    if (pbase + k < nb) {
      if (all || key[k] > tau) packed += 0x10000u;
      else if (key[k] == tau) packed += 1u;
    }
  }
  const uint32_t incl = wave_scan_u32(packed);
  if (lane == 63) red_u[0][wv] = incl;
  __syncthreads();
  uint32_t before_w = 0u, mem_tot = 0u;
#pragma unroll
  for (int w = 0; w < kCoopWaves; ++w) {
    before_w += (w < wv) ? red_u[0][w] : 0u;
    mem_tot += red_u[0][w];
  }
  const uint32_t ex = before_w + incl - packed;
  if (tid == 0) {
    st_dev(&cu->above[m], mem_tot >> 16);
    st_dev(&cu->ties[m], mem_tot & 0xFFFFu);
  }
  coop_barrier(cu, bar++, K, err);
  if (tid < K) {
    s_cnt[0][tid] = ld_dev(&cu->above[tid]);
    s_cnt[1][tid] = ld_dev(&cu->ties[tid]);
  }
  __syncthreads();
  unsigned long long a_before = 0ull, t_before = 0ull, a_tot = 0ull, t_tot = 0ull;
  for (int mm = 0; mm < K; ++mm) {
    if (mm < m) {
      a_before += s_cnt[0][mm];
      t_before += s_cnt[1][mm];
    }
    a_tot += s_cnt[0][mm];
    t_tot += s_cnt[1][mm];
  }
  const unsigned long long keep_ties = min(t_tot, need);            // ties kept in the unit
  const unsigned long long mine = (keep_ties > t_before) ? keep_ties - t_before : 0ull;
  const unsigned long long base = a_before + min(t_before, keep_ties);
  int32_t* lp = sel_pages + (int64_t)u * max_pages;
  int32_t* lx = sel_phys + (int64_t)u * max_pages;
  uint32_t gtb = ex >> 16, tb = ex & 0xFFFFu;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = pbase + k;
    if (i >= nb) continue;
    long long pos = -1;
    if (all || key[k] > tau) {
      pos = (long long)(base + gtb + min((unsigned long long)tb, mine));
      ++gtb;
    } else if (key[k] == tau) {
      if ((unsigned long long)tb < mine) pos = (long long)(base + gtb + tb);
      ++tb;
    }
    if (pos >= 0 && pos < n) {
      lp[pos] = p0 + i;
      lx[pos] = pt[p0 + i];
    }
  }
  if (m == 0 && tid == 0) sel_counts[u] = (int32_t)min(a_tot + keep_ties, (unsigned long long)n);

  // ---- 5. the last member to finish leaves the exchange area zeroed --------
  __syncthreads();
  if (tid == 0) {
    const uint32_t d = __hip_atomic_fetch_add(&cu->done, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = (d == (uint32_t)(K - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (s_last) {
    // every member is past its last read of the area: the counters, the
    // exchanged values and the histograms of the passes used go back to 0
    uint32_t* words = reinterpret_cast<uint32_t*>(cu);
    constexpr int kSmallWords = (int)(offsetof(CoopUnit, hc) / sizeof(uint32_t));
    for (int k = tid; k < kSmallWords; k += kCoopThreads) st_dev(&words[k], 0u);
    for (int ps = 0; ps < passes; ++ps)
      for (int k = tid; k < 2048; k += kCoopThreads) {
        st_dev(&cu->hc[ps][k], 0u);
        __hip_atomic_store(&cu->hw[ps][k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  }
}

// Members per unit and pages per member for a step, or false when the
// cooperative form does not apply: rows longer than 8 members hold, a grid
// that does not fit the device at once, or too few pages to share.
struct CoopShape {
  int K, tpw, smem;
};

template <bool SCORE>
static bool coop_shape(const sparse_dims* d, CoopShape& cs) {
  const int hkv = d->num_kv_heads, group = d->num_q_heads / hkv;
  const int U = d->batch * hkv;
  if (d->max_pages < 1024) return false;      // short rows: one workgroup per unit is faster
  int dev = -1, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  for (int tpw = 1; tpw <= 8; tpw <<= 1) {
    const int pb = tpw * 16 * kCoopWaves;
    const int K = (d->max_pages + pb - 1) / pb;
    if (K > kCoopMaxK || K < 2) continue;
    const int smem = (int)sizeof(float) * group * pb;
    const void* fn = nullptr;
#define SP_FN(T)                                                                               \
  if (tpw == T) fn = reinterpret_cast<const void*>(&coop_select_kernel<SCORE, T>);
    SP_FN(1) SP_FN(2) SP_FN(4) SP_FN(8)
#undef SP_FN
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kCoopThreads, smem) !=
        hipSuccess)
      return false;
    if ((int64_t)U * K > (int64_t)per_cu * cus) continue;   // every member resident at once
    cs.K = K;
    cs.tpw = tpw;
    cs.smem = smem;
    return true;
  }
  return false;
}

template <bool SCORE>
static sparse_status coop_launch(const sparse_dims* d, const uint16_t* q, const uint16_t* summ,
                                 int64_t pool_pages, const float* logits,
                                 const int32_t* page_table, const int32_t* ctx_lens, float scale,
                                 float gamma, int32_t* sel_counts, int32_t* sel_pages,
                                 int32_t* sel_phys, void* ws, size_t ws_bytes, void* stream) {
  CoopShape cs;
  if (!coop_shape<SCORE>(d, cs)) return SPARSE_ERR_UNSUPPORTED;
  const int hkv = d->num_kv_heads, group = d->num_q_heads / hkv;
  const int U = d->batch * hkv;
  if (!ws || ws_bytes < sizeof(CoopHeader) + (size_t)U * sizeof(CoopUnit) || !aligned(ws, 16))
    return SPARSE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  unsigned char* w = static_cast<unsigned char*>(ws);
#define SP_COOP(T)                                                                              \
  hipLaunchKernelGGL((coop_select_kernel<SCORE, T>), dim3(U * cs.K), dim3(kCoopThreads),        \
                     cs.smem, s, q, summ, pool_pages, logits, page_table, ctx_lens, scale,      \
                     gamma, hkv, group, d->max_pages, cs.K, w, sel_counts, sel_pages, sel_phys)
  switch (cs.tpw) {
    case 1: SP_COOP(1); break;
    case 2: SP_COOP(2); break;
    case 4: SP_COOP(4); break;
    default: SP_COOP(8); break;
  }
#undef SP_COOP
  return launch_status();
}

}  // namespace sp

extern "C" size_t sparse_coop_workspace_bytes(const sparse_dims* dims) {
  if (sp::check_dims(dims) != SPARSE_OK) return 0;
  return sizeof(sp::CoopHeader) +
         (size_t)dims->batch * dims->num_kv_heads * sizeof(sp::CoopUnit);
}

extern "C" sparse_status sparse_select_coverage_coop(const sparse_dims* dims, const float* logits,
                                                     const int32_t* ctx_lens,
                                                     const int32_t* page_table, float gamma,
                                                     int32_t* sel_counts, int32_t* sel_pages,
                                                     int32_t* sel_phys, void* ws,
                                                     size_t ws_bytes, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!(gamma > 0.0f && gamma <= 1.0f)) return SPARSE_ERR_INVALID;
  if (!logits || !ctx_lens || !page_table || !sel_counts || !sel_pages || !sel_phys)
    return SPARSE_ERR_INVALID;
  return sp::coop_launch<false>(dims, nullptr, nullptr, 1, logits, page_table, ctx_lens, 1.f,
                                gamma, sel_counts, sel_pages, sel_phys, ws, ws_bytes, stream);
}

extern "C" sparse_status sparse_score_select_coverage(
    const sparse_dims* dims, const uint16_t* q, const uint16_t* summ, int64_t pool_pages,
    const int32_t* page_table, const int32_t* ctx_lens, float scale, float gamma,
    int32_t* sel_counts, int32_t* sel_pages, int32_t* sel_phys, void* ws, size_t ws_bytes,
    void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!(gamma > 0.0f && gamma <= 1.0f)) return SPARSE_ERR_INVALID;
  if (!q || !summ || !page_table || !ctx_lens || !sel_counts || !sel_pages || !sel_phys ||
      pool_pages < 1)
    return SPARSE_ERR_INVALID;
  if (!sp::aligned(q, 16) || !sp::aligned(summ, 16) || !isfinite(scale))
    return SPARSE_ERR_INVALID;
  return sp::coop_launch<true>(dims, q, summ, pool_pages, nullptr, page_table, ctx_lens, scale,
                               gamma, sel_counts, sel_pages, sel_phys, ws, ws_bytes, stream);
}
