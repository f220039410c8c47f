// The coverage rule: per (request, KV head) unit, the fewest pages that
// together hold at least gamma of the unit's estimated attention mass ("Adaptive
// DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", MOIRA
// abstract, coverage-rule sentence).
//
// One 1024-thread workgroup per unit.  Logits are read coalesced (thread t:
// pages t, t + 1024, ...); the page keys then pass through LDS so that for the
// cut thread t owns the blocked run [t*NPT, t*NPT + NPT).  Steps:
//   1. per query head g: (max, sum of exp) over the unit's pages (block
//      reduction of all heads at once), then m[p] += exp(x_g[p] - max_g) /
//      sum_g;  m /= G.
//   2. weights w[p] = floor(m[p] * 2^52) (exact 64-bit fixed point, so the
//      cut's sums are exact and order independent) and keys = fp32 bits of
//      m[p] (monotone for m >= 0).
//   3. target T = ceil(gamma * sum w); a mass-weighted radix select over the
//      key bits below the highest bit in which the unit's keys differ (up to
//      11 bits per pass; LDS histograms of counts and weights; one wave scans
//      the bins from the top) finds the key tau with
//      W(key > tau) < T <= W(key >= tau).
//   4. keep every page with key > tau plus the r lowest-index pages with key
//      == tau, r = ceil((T - W(key > tau)) / w_tau); compact in ascending page
//      order by one block prefix sum of packed (above, tie) counts.
//   5. the last workgroup to finish (device ticket) writes the prefix sums of
//      the counts and of the chunk counts over all units, then re-arms the
//      ticket -- the plan the attention kernel reads, made on the device.

#include "common.h"

extern "C" size_t sparse_select_workspace_bytes(const sparse_dims* dims);

namespace sp {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

struct PairMS {
  float m, s;
};

// fixed-point weight of a page from its fp32 mass bits: floor(m * 2^52)
__device__ __forceinline__ unsigned long long weight_of(uint32_t key) {
  return (unsigned long long)(__uint_as_float(key) * 4503599627370496.0f);
}

template <bool COUNT>
__device__ __forceinline__ unsigned long long wgt_of(uint32_t key) {
  if constexpr (COUNT) return 1ull;
  else return weight_of(key);
}

__device__ __forceinline__ PairMS combine(PairMS a, PairMS b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return {M, 0.f};
  const float sa = (a.m == -INFINITY) ? 0.f : a.s * __expf(a.m - M);
  const float sb = (b.m == -INFINITY) ? 0.f : b.s * __expf(b.m - M);
  return {M, sa + sb};
}

// COUNT = false: the coverage cut (page weight = its fixed-point mass, target
// ceil(gamma * total)).  COUNT = true: the fixed-budget variant (page weight 1,
// target min(k_pages, n)) -- the k highest-mass pages, ties to lower index.
template <int NPT, bool COUNT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ page_table, float gamma, int k_pages, int chunk_pages, int hkv,
    int group,
    int max_pages, int cap, int U, int32_t* __restrict__ sel_counts,
    int32_t* __restrict__ sel_offsets,
    int32_t* __restrict__ chunk_offsets, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ sel_phys, uint32_t* __restrict__ ticket) {
  // Page keys, staged so that loads are coalesced (thread t reads pages
  // t, t + 1024, ...) while the cut works on blocked runs (thread t owns
  // pages t*NPT .. t*NPT + NPT-1); later reused for the kept page list.
  __shared__ uint32_t keys_lds[NPT * kSelThreads];
  // radix histograms: two buffers (alternate passes) while LDS allows
  constexpr int kHistBufs = (NPT <= 16) ? 2 : 1;
  __shared__ uint32_t hcnt[kHistBufs][2048];
  __shared__ unsigned long long hw[kHistBufs][2048];
  __shared__ float red_m[kMaxGroup][kSelWaves], red_s[kMaxGroup][kSelWaves];
  __shared__ unsigned long long red_z[kSelWaves];
  __shared__ uint32_t red_lo[kSelWaves], red_hi[kSelWaves];
  __shared__ uint32_t scan32[kSelWaves];
  __shared__ unsigned long long scan64[kSelWaves];
  __shared__ int s_bin[2];
  __shared__ unsigned long long s_wgt[2];
  __shared__ int s_last;
  __shared__ uint32_t s_ncand, s_tau, s_need;
  __shared__ uint32_t cand_key[64], cand_page[64];

  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int u = blockIdx.x;
  const int b = u / hkv;
  const int L = min(max(ctx_lens[b], 0), max_pages * kP);
  const int n = (L + kP - 1) / kP;
  int count = 0;

  if (n > 0) {
    const float* X = logits + (int64_t)u * group * max_pages;

    // ---- 1. per-head softmax normalisers -----------------------------------
    // Logits of HPR heads at a time, every load issued before the first use.
    // (max, sum of exp) per head: thread-local, wave shuffles, then one lane
    // per head combines the wave partials.  When all heads fit one round the
    // values stay in registers for step 2; otherwise they are read again.
    constexpr int HPR = (NPT >= 32) ? 1 : 32 / NPT;
    const bool one_round = group <= HPR;
    float xv[HPR][NPT];
    for (int g0 = 0; g0 < group; g0 += HPR) {
#pragma unroll
      for (int hh = 0; hh < HPR; ++hh) {
        const float* Xg = X + (int64_t)(g0 + hh) * max_pages;
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          const int p = k * kSelThreads + tid;
          xv[hh][k] = (g0 + hh < group && p < n) ? Xg[p] : -INFINITY;
        }
      }
#pragma unroll
      for (int hh = 0; hh < HPR; ++hh) {
        if (g0 + hh >= group) break;
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < NPT; ++k) mx = fmaxf(mx, xv[hh][k]);
        float se = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int k = 0; k < NPT; ++k) se += __expf(xv[hh][k] - mx);
        }
        PairMS pr = {mx, se};
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          PairMS other = {__shfl_xor(pr.m, o, 64), __shfl_xor(pr.s, o, 64)};
          pr = combine(pr, other);
        }
        if (lane == 0) {
          red_m[g0 + hh][wv] = pr.m;
          red_s[g0 + hh][wv] = pr.s;
        }
      }
    }
    __syncthreads();
    if (wv == 0) {
      // lane l combines wave partial (l & 15) of head g0 + (l >> 4)
      for (int g0 = 0; g0 < group; g0 += 4) {
        const int g = g0 + (lane >> 4), w = lane & 15;
        PairMS pr = (g < group) ? PairMS{red_m[g][w], red_s[g][w]} : PairMS{-INFINITY, 0.f};
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
          PairMS other = {__shfl_xor(pr.m, o, 64), __shfl_xor(pr.s, o, 64)};
          pr = combine(pr, other);
        }
        if (w == 0 && g < group) {
          red_m[g][0] = pr.m;
          red_s[g][0] = 1.f / pr.s;
        }
      }
    }
    __syncthreads();

    // ---- 2. group mass, keys, fixed-point weights, total and key range ----
    float m[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) m[k] = 0.f;
    for (int g0 = 0; g0 < group; g0 += HPR) {
      if (!one_round) {
#pragma unroll
        for (int hh = 0; hh < HPR; ++hh) {
          const float* Xg = X + (int64_t)(g0 + hh) * max_pages;
#pragma unroll
          for (int k = 0; k < NPT; ++k) {
            const int p = k * kSelThreads + tid;
            xv[hh][k] = (g0 + hh < group && p < n) ? Xg[p] : -INFINITY;
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < HPR; ++hh) {
        if (g0 + hh >= group) break;
        const float M = red_m[g0 + hh][0], inv = red_s[g0 + hh][0];
        if (M == -INFINITY) continue;      // a head with no finite logit adds no mass
#pragma unroll
        for (int k = 0; k < NPT; ++k) m[k] += __expf(xv[hh][k] - M) * inv;
      }
    }
    const float invg = 1.f / (float)group;
    unsigned long long zl = 0ull;
    uint32_t klo = 0xFFFFFFFFu, khi = 0u;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int p = k * kSelThreads + tid;
      if (p < n) {
        const uint32_t key = __float_as_uint(m[k] * invg);
        keys_lds[p] = key;
        zl += wgt_of<COUNT>(key);
        klo = min(klo, key);
        khi = max(khi, key);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      zl += __shfl_xor(zl, o, 64);
      klo = min(klo, (uint32_t)__shfl_xor((int)klo, o, 64));
      khi = max(khi, (uint32_t)__shfl_xor((int)khi, o, 64));
    }
    if (lane == 0) {
      red_z[wv] = zl;
      red_lo[wv] = klo;
      red_hi[wv] = khi;
    }
    __syncthreads();
    if (wv == 0) {
      unsigned long long z = (lane < kSelWaves) ? red_z[lane] : 0ull;
      uint32_t lo2 = (lane < kSelWaves) ? red_lo[lane] : 0xFFFFFFFFu;
      uint32_t hi2 = (lane < kSelWaves) ? red_hi[lane] : 0u;
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        z += __shfl_xor(z, o, 64);
        lo2 = min(lo2, (uint32_t)__shfl_xor((int)lo2, o, 64));
        hi2 = max(hi2, (uint32_t)__shfl_xor((int)hi2, o, 64));
      }
      if (lane == 0) {
        red_z[0] = z;
        red_lo[0] = lo2;
        red_hi[0] = hi2;
      }
    }
    __syncthreads();
    const unsigned long long Z = red_z[0];
    const uint32_t KLO = red_lo[0], KHI = red_hi[0];
    // this thread's blocked run of keys
    const int pbase = tid * NPT;
    uint32_t key[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) key[i] = (pbase + i < n) ? keys_lds[pbase + i] : 0u;

    // ---- 3. the cut: key tau and the number of ties at tau to keep -------
    const bool all = COUNT ? (k_pages >= n) : !(gamma < 1.0f);
    uint32_t tau = 0u;
    unsigned long long need = 0ull;
    if (!all) {
      unsigned long long T = COUNT ? (unsigned long long)k_pages
                                   : (unsigned long long)ceil((double)gamma * (double)Z);
      if (T > Z) T = Z;
      if (T < 1ull) T = 1ull;
      unsigned long long w_tau = wgt_of<COUNT>(KHI);
      if (KLO == KHI) {
        tau = KHI;                          // every page has the same mass
      } else {
        // radix passes over the bits below the highest bit where keys differ
        const int top = 31 - __clz(KLO ^ KHI);
        uint32_t hi_mask = ~((2u << top) - 1u);
        uint32_t prefix = KHI & hi_mask;
        int lo = top + 1, buf = 0;
        bool resolved = false;
        while (lo > 0) {
          const int width = min(11, lo);
          const int sh = lo - width, nb = 1 << width;
          uint32_t* cnt = hcnt[buf];
          unsigned long long* wgt = hw[buf];
          for (int k = tid; k < nb; k += kSelThreads) {
            cnt[k] = 0u;
            wgt[k] = 0ull;
          }
          if (tid == 0) s_ncand = 0u;
          __syncthreads();
#pragma unroll
          for (int i = 0; i < NPT; ++i) {
            if (pbase + i < n && (key[i] & hi_mask) == prefix) {
              const int bin = (key[i] >> sh) & (nb - 1);
              atomicAdd(&cnt[bin], 1u);
              atomicAdd(&wgt[bin], wgt_of<COUNT>(key[i]));
            }
          }
          __syncthreads();
          {
            // thread t owns bins 2t, 2t+1; the weight of all bins above a
            // thread's comes from one block prefix sum
            const int b0 = 2 * tid, b1 = 2 * tid + 1;
            const unsigned long long w0 = (b0 < nb) ? wgt[b0] : 0ull;
            const unsigned long long w1 = (b1 < nb) ? wgt[b1] : 0ull;
            unsigned long long total;
            const unsigned long long ex =
                block_excl_scan<unsigned long long, kSelThreads>(w0 + w1, scan64, total);
            const unsigned long long gt1 = total - (ex + w0 + w1);  // weight above bin b1
            const unsigned long long gt0 = gt1 + w1;                // weight above bin b0
            if (b1 < nb && gt1 < T && T <= gt1 + w1) {
              s_bin[buf & 1] = b1;
              s_wgt[buf & 1] = gt1;
            }
            if (b0 < nb && gt0 < T && T <= gt0 + w0) {
              s_bin[buf & 1] = b0;
              s_wgt[buf & 1] = gt0;
            }
          }
          __syncthreads();
          const int bin = s_bin[buf & 1];
          T -= s_wgt[buf & 1];
          prefix |= (uint32_t)bin << sh;
          hi_mask |= (uint32_t)(nb - 1) << sh;
          if (sh == 0) {
            const unsigned long long c = cnt[bin];
            w_tau = c ? wgt[bin] / c : 1ull;   // every page with key tau has one weight
          }
          lo = sh;
          if (sh > 0 && cnt[bin] <= 64u) {
            // Few pages share the resolved high bits: one wave sorts them by
            // (key descending, page ascending) and walks their weights.
            for (int i = 0; i < NPT; ++i) {
              if (pbase + i < n && (key[i] & hi_mask) == prefix) {
                const uint32_t at = atomicAdd(&s_ncand, 1u);
                if (at < 64u) {
                  cand_key[at] = key[i];
                  cand_page[at] = (uint32_t)(pbase + i);
                }
              }
            }
            __syncthreads();
            if (wv == 0) {
              const uint32_t nc = s_ncand;
              const bool ok = (uint32_t)lane < nc;
              unsigned long long c =
                  ok ? (((unsigned long long)(~cand_key[lane]) << 32) | cand_page[lane]) : ~0ull;
#pragma unroll
              for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
                for (int jj = k >> 1; jj > 0; jj >>= 1) {
                  const unsigned long long o =
                      (unsigned long long)__shfl_xor((long long)c, jj, 64);
                  const bool up = (lane & k) == 0, low = (lane & jj) == 0;
                  c = (low == up) ? min(c, o) : max(c, o);
                }
              }
              const uint32_t kk = ~(uint32_t)(c >> 32);
              const unsigned long long wk = ok ? wgt_of<COUNT>(kk) : 0ull;
              const unsigned long long cum = wave_incl_scan(wk);
              const unsigned long long reach = __ballot(ok && cum >= T);
              const int at = __ffsll((long long)reach) - 1;     // first lane reaching T
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
          if constexpr (kHistBufs == 2) {
            buf ^= 1;
          } else {
            __syncthreads();                  // single buffer: wait before it is cleared
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
        need = (T + w_tau - 1ull) / w_tau;  // pages at tau to keep (>= 1)
      }
    }

    // ---- 4. compact in ascending page order: one scan of packed counts ----
    // high half: pages above tau (all pages when gamma = 1); low half: ties
    uint32_t packed = 0u;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (pbase + i < n) {
        if (all || key[i] > tau) packed += 0x10000u;
        else if (key[i] == tau) packed += 1u;
      }
    }
    uint32_t tot_packed;
    const uint32_t ex = block_excl_scan<uint32_t, kSelThreads>(packed, scan32, tot_packed);
    // every thread has its keys in registers by now: reuse keys_lds for the list
    uint32_t gtb = ex >> 16, tb = ex & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (pbase + i >= n) continue;
      int pos = -1;
      if (all || key[i] > tau) {
        pos = (int)(gtb + (uint32_t)min((unsigned long long)tb, need));
        ++gtb;
      } else if (key[i] == tau) {
        if ((unsigned long long)tb < need) pos = (int)(gtb + tb);
        ++tb;
      }
      if (pos >= 0) keys_lds[pos] = (uint32_t)(pbase + i);
    }
    count = (int)((tot_packed >> 16) + min((unsigned long long)(tot_packed & 0xFFFFu), need));
    __syncthreads();
    int32_t* lp = sel_pages + (int64_t)u * max_pages;
    int32_t* lx = sel_phys + (int64_t)u * max_pages;
    const int32_t* pt = page_table + (int64_t)b * max_pages;
    for (int i = tid; i < count; i += kSelThreads) {
      const int p = (int)keys_lds[i];
      lp[i] = p;
      lx[i] = pt[p];
    }
  }

  // ---- 5. optional: the last workgroup writes prefix sums over units ------
  if (sel_offsets == nullptr) {
    if (tid == 0) sel_counts[u] = count;
    return;
  }
  __syncthreads();   // every thread's list writes are issued before the ticket
  if (tid == 0) {
    sel_counts[u] = count;
    __threadfence();   // release this unit's list and count device-wide
    const uint32_t t = atomicAdd(ticket, 1u);
    s_last = (t == (uint32_t)(U - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();     // acquire every unit's count
  uint32_t run = 0u, runc = 0u;
  for (int base = 0; base < U; base += kSelThreads) {
    const int v = base + tid;
    uint32_t c = 0u;
    if (v < U) c = (uint32_t)__hip_atomic_load(sel_counts + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // chunks as the attention plans them: lists beyond the dims' bound are cut
    const uint32_t ch = (min(c, (uint32_t)cap) + (uint32_t)chunk_pages - 1u) / (uint32_t)chunk_pages;
    // both prefix sums in one scan: count in the high word, chunks in the low
    unsigned long long tot;
    const unsigned long long ex = block_excl_scan<unsigned long long, kSelThreads>(
        ((unsigned long long)c << 32) | ch, scan64, tot);
    if (v < U) {
      sel_offsets[v] = (int32_t)(run + (uint32_t)(ex >> 32));
      chunk_offsets[v] = (int32_t)(runc + (uint32_t)ex);
    }
    run += (uint32_t)(tot >> 32);
    runc += (uint32_t)tot;
  }
  if (tid == 0) {
    sel_offsets[U] = (int32_t)run;
    chunk_offsets[U] = (int32_t)runc;
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int NPT, bool COUNT>
static void launch_select(hipStream_t st, int U, const float* logits, const int32_t* ctx_lens,
                          const int32_t* page_table, float gamma, int k_pages, int chunk_pages,
                          int hkv, int group, int max_pages, int cap, int32_t* sel_counts,
                          int32_t* sel_offsets, int32_t* chunk_offsets, int32_t* sel_pages,
                          int32_t* sel_phys, uint32_t* ticket) {
  hipLaunchKernelGGL((select_kernel<NPT, COUNT>), dim3(U), dim3(kSelThreads), 0, st, logits,
                     ctx_lens, page_table, gamma, k_pages, chunk_pages, hkv, group, max_pages, cap,
                     U,
                     sel_counts, sel_offsets, chunk_offsets, sel_pages, sel_phys, ticket);
}

template <bool COUNT>
static sparse_status select_entry(const sparse_dims* dims, const float* logits,
                                  const int32_t* ctx_lens, const int32_t* page_table, float gamma,
                                  int k_pages, int32_t chunk_pages, int32_t* sel_counts,
                                  int32_t* sel_offsets, int32_t* chunk_offsets,
                                  int32_t* sel_pages, int32_t* sel_phys, void* ws,
                                  size_t ws_bytes, void* stream);

}  // namespace sp

extern "C" size_t sparse_select_workspace_bytes(const sparse_dims* dims) {
  (void)dims;
  return 256;  // the finishing ticket (one 32-bit counter), padded
}

namespace sp {

template <bool COUNT>
static sparse_status select_entry(const sparse_dims* dims, const float* logits,
                                  const int32_t* ctx_lens, const int32_t* page_table, float gamma,
                                  int k_pages, int32_t chunk_pages, int32_t* sel_counts,
                                  int32_t* sel_offsets, int32_t* chunk_offsets,
                                  int32_t* sel_pages, int32_t* sel_phys, void* ws,
                                  size_t ws_bytes, void* stream) {
  sparse_status st = check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!logits || !ctx_lens || !page_table || !sel_counts || !sel_pages || !sel_phys)
    return SPARSE_ERR_INVALID;
  if ((sel_offsets == nullptr) != (chunk_offsets == nullptr)) return SPARSE_ERR_INVALID;
  if (chunk_pages < 1 || chunk_pages > dims->max_pages) return SPARSE_ERR_INVALID;
  if (sel_offsets != nullptr &&
      (!ws || ws_bytes < sparse_select_workspace_bytes(dims) || !aligned(ws, 4)))
    return SPARSE_ERR_WORKSPACE;
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  const int npt = (dims->max_pages + kSelThreads - 1) / kSelThreads;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* ticket = static_cast<uint32_t*>(ws);
#define SP_SEL(N)                                                                           \
  launch_select<N, COUNT>(s, U, logits, ctx_lens, page_table, gamma, k_pages, chunk_pages, \
                          hkv, group, dims->max_pages, list_cap(dims), sel_counts,        \
                          sel_offsets,                                                      \
                          chunk_offsets, sel_pages, sel_phys, ticket)
  if (npt <= 1) SP_SEL(1);
  else if (npt <= 2) SP_SEL(2);
  else if (npt <= 4) SP_SEL(4);
  else if (npt <= 8) SP_SEL(8);
  else if (npt <= 16) SP_SEL(16);
  else SP_SEL(32);
#undef SP_SEL
  return launch_status();
}

}  // namespace sp

extern "C" sparse_status sparse_select_coverage(const sparse_dims* dims, const float* logits,
                                                const int32_t* ctx_lens, const int32_t* page_table,
                                                float gamma, int32_t chunk_pages,
                                                int32_t* sel_counts, int32_t* sel_offsets,
                                                int32_t* chunk_offsets, int32_t* sel_pages,
                                                int32_t* sel_phys, void* ws, size_t ws_bytes,
                                                void* stream) {
  if (!(gamma > 0.0f && gamma <= 1.0f)) return SPARSE_ERR_INVALID;
  return sp::select_entry<false>(dims, logits, ctx_lens, page_table, gamma, 0, chunk_pages,
                                 sel_counts, sel_offsets, chunk_offsets, sel_pages, sel_phys, ws,
                                 ws_bytes, stream);
}

extern "C" sparse_status sparse_select_topk(const sparse_dims* dims, const float* logits,
                                            const int32_t* ctx_lens, const int32_t* page_table,
                                            int32_t k_pages, int32_t chunk_pages,
                                            int32_t* sel_counts, int32_t* sel_offsets,
                                            int32_t* chunk_offsets, int32_t* sel_pages,
                                            int32_t* sel_phys, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (k_pages < 1) return SPARSE_ERR_INVALID;
  return sp::select_entry<true>(dims, logits, ctx_lens, page_table, 1.0f, k_pages, chunk_pages,
                                sel_counts, sel_offsets, chunk_offsets, sel_pages, sel_phys, ws,
                                ws_bytes, stream);
}
