// The coverage rule: per (request, KV head) unit, the fewest pages that
// together hold at least gamma of the unit's estimated attention mass ("Adaptive
// DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", MOIRA
// abstract, coverage-rule sentence).
//
// One workgroup of NT threads per unit (256, 512 or 1024, with at most 8
// pages per thread below 1024).  Logits are read coalesced (thread t: pages
// t, t + NT, ...); the page keys then pass through LDS so that for the cut
// thread t owns the blocked run [t*NPT, t*NPT + NPT).  Steps:
//   0. one round of loads: the context length, the logits and the request's
//      page-table row (staged in LDS for the list's physical ids).
//   1. per query head g: the max M_g over the unit's pages, then the sum S_g
//      of exp(x_g[p] - M_g) (two block reductions, each over all heads at
//      once); m[p] = (1/G) sum_g exp(x_g[p] - M_g) / S_g.
//   2. weights w[p] = floor(m[p] * 2^52) (exact 64-bit fixed point, so the
//      cut's sums are exact and order independent) and keys = fp32 bits of
//      m[p] (monotone for m >= 0).
//   3. target T = ceil(gamma * sum w) (the sum taken from the first radix
//      pass's histogram, which holds every page); a mass-weighted radix select over the
//      key bits below the highest bit in which the unit's keys differ (up to
//      11 bits per pass; LDS histograms of counts and weights; each wave
//      totals its share of the 2048 bins, and the wave whose bins hold the
//      crossing scans them) finds the key tau with
//      W(key > tau) < T <= W(key >= tau).
//   4. keep every page with key > tau plus the r lowest-index pages with key
//      == tau, r = ceil((T - W(key > tau)) / w_tau); compact in ascending page
//      order by one block prefix sum of packed (above, tie) counts.
//   5. optionally, the last workgroup to finish (device ticket) writes the
//      exclusive prefix sum of the counts over all units, then re-arms the
//      ticket (the attention and merge plan from the counts alone and do not
//      read it).

#include "common.h"
#include "reduce.h"

extern "C" size_t sparse_select_workspace_bytes(const sparse_dims* dims);

namespace sp {

constexpr int kSelThreads = 1024;              // the largest selection workgroup
constexpr int kSelWaves = kSelThreads / 64;    // its waves (LDS partial arrays)

template <bool COUNT>
__device__ __forceinline__ unsigned long long wgt_of(uint32_t key) {
  if constexpr (COUNT) return 1ull;
  else return weight_of(key);
}

// Logits of heads g0 .. g0 + HPR - 1 for this thread's pages (thread t:
// pages t, t + NT, ...); -inf for a page past the context or a head past
// the group.
template <int NPT, int HPR, int NT>
__device__ __forceinline__ void load_logits(const float* __restrict__ X, int g0, int group,
                                            int max_pages, int n, int tid,
                                            float (&xv)[HPR][NPT]) {
#pragma unroll
  for (int hh = 0; hh < HPR; ++hh) {
    const float* Xg = X + (int64_t)(g0 + hh) * max_pages;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int p = k * NT + tid;
      xv[hh][k] = (g0 + hh < group && p < n) ? Xg[p] : -INFINITY;
    }
  }
}

// The max (MAX) or sum over the NW wave partials part[g][w] of heads g0 ..
// g0 + H - 1, computed by every lane of the calling wave: four heads per LDS
// read (lane l takes head g0 + 4r + (l >> 4), partial l & 15, the identity
// past the NW partials), one row
// butterfly, then each head's total is read from its row.  The results are
// the same in every lane and every wave.
template <bool MAX, int H, int NW>
__device__ __forceinline__ void head_totals(const float (*part)[kSelWaves], int g0, int group,
                                            float (&out)[H]) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < (H + 3) / 4; ++r) {
    const int g = g0 + 4 * r + (lane >> 4);
    const float raw = part[min(g, kMaxGroup - 1)][lane & 15];
    float v = (g < group && (lane & 15) < NW) ? raw : (MAX ? -INFINITY : 0.f);
    v = MAX ? row16_f32(v, OpMax()) : row16_f32(v, OpAdd());
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * r + e < H) out[4 * r + e] = __uint_as_float(lane_u32(__float_as_uint(v), 16 * e));
  }
}

// COUNT = false: the coverage cut (page weight = its fixed-point mass, target
// ceil(gamma * total)).  COUNT = true: the fixed-budget variant (page weight 1,
// target min(k_pages, n)) -- the k highest-mass pages, ties to lower index.
template <int NPT, bool COUNT, int NT>
__global__ __launch_bounds__(NT) void select_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ page_table, float gamma, int k_pages, int hkv, int group,
    int max_pages, int U, int32_t* __restrict__ sel_counts,
    int32_t* __restrict__ sel_offsets, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ sel_phys, uint32_t* __restrict__ ticket) {
  // NT threads in NW waves; a workgroup takes rows of up to NPT * NT pages.
  constexpr int NW = NT / 64;
  static_assert(NT == 256 || NT == 512 || NT == 1024, "select workgroup size");
  // Page keys, staged so that loads are coalesced (thread t reads pages
  // t, t + NT, ...) while the cut works on blocked runs (thread t owns
  // pages t*NPT .. t*NPT + NPT-1); later reused for the kept page list.
  __shared__ __attribute__((aligned(16))) uint32_t keys_lds[NPT * NT];
  // The request's page-table row, staged while the logits load so that the
  // list's physical ids need no dependent global gather at the end (when the
  // row fits beside the keys and histograms in LDS).
  constexpr bool kStagePt = NPT * NT <= 8192;
  __shared__ int32_t ptl[kStagePt ? NPT * NT : 1];
  // radix histograms: two buffers (alternate passes) while LDS allows
  constexpr int kHistBufs = (NPT * NT <= 16384) ? 2 : 1;
  __shared__ uint32_t hcnt[kHistBufs][2048];
  __shared__ unsigned long long hw[kHistBufs][2048];
  __shared__ float red_m[kMaxGroup][kSelWaves], red_s[kMaxGroup][kSelWaves];
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
  const float* X = logits + (int64_t)u * group * max_pages;
  const int32_t* pt = page_table + (int64_t)b * max_pages;

  // Every load the selection starts from is issued in one round, before the
  // context length is known: the length, the first HPR heads' logits and
  // (when staged) the page-table row.  Indices are clamped to the row, so a
  // page past the context reads an in-bounds word that is masked below; the
  // empty asm statements keep the compiler from moving the loads under the
  // length test, where each would wait behind the length's round trip.
  // heads per round of loads: 32 logits per thread in a 1024-thread
  // workgroup, 64 in a smaller one (fewer waves per SIMD leave more registers)
  constexpr int kRegLogits = (NT == 1024) ? 32 : 64;
  constexpr int HPR = (NPT >= kRegLogits) ? 1 : kRegLogits / NPT;
  const int Lraw = ctx_lens[b];
  float xv[HPR][NPT];
#pragma unroll
  for (int hh = 0; hh < HPR; ++hh) {
    const float* Xg = X + (int64_t)min(hh, group - 1) * max_pages;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      xv[hh][k] = (hh < group) ? Xg[min(k * NT + tid, max_pages - 1)] : -INFINITY;
  }
  int ptv[kStagePt ? NPT : 1];
  if constexpr (kStagePt) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) ptv[k] = pt[min(k * NT + tid, max_pages - 1)];
  }
  // the first radix pass's histogram is cleared while the loads are in flight
  for (int k = tid; k < 2048; k += NT) {
    hcnt[0][k] = 0u;
    hw[0][k] = 0ull;
  }
  if (tid == 0) {
    s_ncand = 0u;
    s_bin[0] = s_bin[1] = 0;
    s_wgt[0] = s_wgt[1] = 0ull;
  }
#pragma unroll
  for (int hh = 0; hh < HPR; ++hh)
#pragma unroll
    for (int k = 0; k < NPT; ++k) asm volatile("" : "+v"(xv[hh][k]));
  if constexpr (kStagePt) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) asm volatile("" : "+v"(ptv[k]));
  }
  const int L = min(max(Lraw, 0), max_pages * kP);
  const int n = (L + kP - 1) / kP;
  int count = 0;

  if (n > 0) {
    // ---- 1. per-head softmax normalisers -----------------------------------
    // Two passes per head, neither spending an exp on combining partials:
    // the max M_g (thread-local, wave shuffles, one partial per wave in LDS),
    // then e = exp(x - M_g) and its sum S_g the same way.  After each
    // barrier every wave reduces the NW wave partials itself, so no second
    // barrier hands a result on.  Heads go HPR at a time (the first round
    // from the loads above); when all heads fit one round, e stays in
    // registers for step 2, otherwise the logits are read again.
    const bool one_round = group <= HPR;
    for (int g0 = 0; g0 < group; g0 += HPR) {
      if (g0 == 0) {
#pragma unroll
        for (int hh = 0; hh < HPR; ++hh)
#pragma unroll
          for (int k = 0; k < NPT; ++k)
            if (!(hh < group && k * NT + tid < n)) xv[hh][k] = -INFINITY;
      } else {
        load_logits<NPT, HPR, NT>(X, g0, group, max_pages, n, tid, xv);
      }
#pragma unroll
      for (int hh = 0; hh < HPR; ++hh) {
        if (g0 + hh >= group) break;
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < NPT; ++k) mx = fmaxf(mx, xv[hh][k]);
        mx = wave_total_f32(mx, OpMax());
        if (lane == 0) red_m[g0 + hh][wv] = mx;
      }
    }
    __syncthreads();
    for (int g0 = 0; g0 < group; g0 += HPR) {
      if (!one_round) load_logits<NPT, HPR, NT>(X, g0, group, max_pages, n, tid, xv);
      float Mh[4];
#pragma unroll
      for (int hh = 0; hh < HPR; ++hh) {
        if (g0 + hh >= group) break;
        if ((hh & 3) == 0) head_totals<true, 4, NW>(red_m, g0 + hh, group, Mh);
        const float M = Mh[hh & 3];
        float se = 0.f;
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          // a head with no finite logit (M = -inf) adds no mass
          xv[hh][k] = (M == -INFINITY) ? 0.f : __expf(xv[hh][k] - M);
          se += xv[hh][k];
        }
        se = wave_total_f32(se, OpAdd());
        if (lane == 0) red_s[g0 + hh][wv] = se;
      }
    }
    __syncthreads();

    // ---- 2. group mass, keys, fixed-point weights, total and key range ----
    float m[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) m[k] = 0.f;
    for (int g0 = 0; g0 < group; g0 += HPR) {
      if (!one_round) load_logits<NPT, HPR, NT>(X, g0, group, max_pages, n, tid, xv);
      float Sh[4], Mh[4];
#pragma unroll
      for (int hh = 0; hh < HPR; ++hh) {
        if (g0 + hh >= group) break;
        if ((hh & 3) == 0) {
          head_totals<false, 4, NW>(red_s, g0 + hh, group, Sh);
          if (!one_round) head_totals<true, 4, NW>(red_m, g0 + hh, group, Mh);
        }
        const float S = Sh[hh & 3];
        if (!(S > 0.f)) continue;            // no finite logit: no mass
        const float inv = 1.f / S;
        if (one_round) {
#pragma unroll
          for (int k = 0; k < NPT; ++k) m[k] += xv[hh][k] * inv;
        } else {
          const float M = Mh[hh & 3];
#pragma unroll
          for (int k = 0; k < NPT; ++k) m[k] += __expf(xv[hh][k] - M) * inv;
        }
      }
    }
    const float invg = 1.f / (float)group;
    uint32_t klo = 0xFFFFFFFFu, khi = 0u;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int p = k * NT + tid;
      if (p < n) {
        const uint32_t key = __float_as_uint(m[k] * invg);
        keys_lds[p] = key;
        if constexpr (kStagePt) ptl[p] = ptv[k];
        klo = min(klo, key);
        khi = max(khi, key);
      }
    }
    klo = wave_total_u32(klo, OpMinU());
    khi = wave_total_u32(khi, OpMaxU());
    if (lane == 0) {
      red_lo[wv] = klo;
      red_hi[wv] = khi;
    }
    __syncthreads();
    // every wave combines the NW wave partials itself (lane l: partial
    // l & (NW - 1); a repeated partial leaves a min or max unchanged)
    const uint32_t KLO = row16_u32(red_lo[lane & (NW - 1)], OpMinU());
    const uint32_t KHI = row16_u32(red_hi[lane & (NW - 1)], OpMaxU());
    // lane l of a row of 16 stands for wave l & 15 in the block-wide sums below
    const int wl = lane & 15;
    // this thread's blocked run of keys
    const int pbase = tid * NPT;
    uint32_t key[NPT];
    if constexpr (NPT >= 4) {
      // 16-byte LDS reads: the run's words are consecutive, so one read per
      // four keys instead of four bank-conflicting single-word reads
#pragma unroll
      for (int v = 0; v < NPT / 4; ++v) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(&keys_lds[pbase + 4 * v]);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * v + e] = (pbase + 4 * v + e < n) ? w[e] : 0u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPT; ++i) key[i] = (pbase + i < n) ? keys_lds[pbase + i] : 0u;
    }

    // ---- 3. the cut: key tau and the number of ties at tau to keep -------
    const bool all = COUNT ? (k_pages >= n) : !(gamma < 1.0f);
    uint32_t tau = 0u;
    unsigned long long need = 0ull;
    if (!all) {
      // target T from the total weight Z = sum of every page's weight
      auto target = [&](unsigned long long Z) {
        unsigned long long t = COUNT ? (unsigned long long)k_pages
                                     : (unsigned long long)ceil((double)gamma * (double)Z);
        if (t > Z) t = Z;
        if (t < 1ull) t = 1ull;
        return t;
      };
      unsigned long long T = 0ull;
      unsigned long long w_tau = wgt_of<COUNT>(KHI);
      if (KLO == KHI) {
        tau = KHI;                          // every page has the same mass
        T = target((unsigned long long)n * w_tau);
      } else {
        // radix passes over the bits below the highest bit where keys differ
        const int top = 31 - __clz(KLO ^ KHI);
        uint32_t hi_mask = ~((2u << top) - 1u);
        uint32_t prefix = KHI & hi_mask;
        int lo = top + 1, buf = 0;
        bool resolved = false, first = true, need_z = true;
        while (lo > 0) {
          const int width = min(11, lo);
          const int sh = lo - width, nb = 1 << width;
          uint32_t* cnt = hcnt[buf];
          unsigned long long* wgt = hw[buf];
          if (!first) {   // the first pass's buffer was cleared at the start
            for (int k = tid; k < nb; k += NT) {
              cnt[k] = 0u;
              wgt[k] = 0ull;
            }
            if (tid == 0) s_ncand = 0u;
            __syncthreads();
          }
          first = false;
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
            // thread t owns bins BPT t .. BPT t + BPT - 1, wave w the 64 BPT
            // bins from 64 BPT w.  One barrier for the wave totals; then only
            // the wave whose bins hold the crossing scans them.
            constexpr int BPT = 2048 / NT;
            unsigned long long wb[BPT], ws = 0ull;
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
              wb[i] = (BPT * tid + i < nb) ? wgt[BPT * tid + i] : 0ull;
              ws += wb[i];
            }
            const unsigned long long wtot = wave_total_u64(ws);
            if (lane == 0) scan64[wv] = wtot;
            __syncthreads();
            const unsigned long long tw = (wl < NW) ? scan64[wl] : 0ull;
            // The first pass takes in every page (all keys share the bits
            // above the first digit), so its bins sum to Z: the target is
            // set here instead of by a block reduction of its own.
            if (need_z) {
              T = target(row16_sum_u64(tw));
              need_z = false;
            }
            // weight of the bins of the waves above this one (same in every lane)
            const unsigned long long above = row16_sum_u64((wl > wv) ? tw : 0ull);
            if (above < T && T <= above + wtot) {
              // weight above this thread's highest bin, then down its bins
              unsigned long long gt = above + (wtot - wave_scan_u64(ws));
#pragma unroll
              for (int i = BPT - 1; i >= 0; --i) {
                const int bi = BPT * tid + i;
                if (bi < nb && gt < T && T <= gt + wb[i]) {
                  s_bin[buf & 1] = bi;
                  s_wgt[buf & 1] = gt;
                }
                gt += wb[i];
              }
            }
          }
          __syncthreads();
          const int bin = s_bin[buf & 1] & (nb - 1);
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
              // bitonic network, stopped once a sorted block covers the
              // candidates (lanes 0 .. nc-1, the rest hold the largest key)
#pragma unroll
              for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
                for (int jj = k >> 1; jj > 0; jj >>= 1) {
                  const unsigned long long o =
                      (unsigned long long)__shfl_xor((long long)c, jj, 64);
                  const bool up = (lane & k) == 0, low = (lane & jj) == 0;
                  c = (low == up) ? min(c, o) : max(c, o);
                }
                if ((uint32_t)k >= nc) break;
              }
              const uint32_t kk = ~(uint32_t)(c >> 32);
              const unsigned long long wk = ok ? wgt_of<COUNT>(kk) : 0ull;
              const unsigned long long cum = wave_scan_u64(wk);
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
    // block prefix sum with one barrier: wave scans, wave totals in LDS,
    // then every wave sums the totals of the waves before it
    const uint32_t incl = wave_scan_u32(packed);
    if (lane == 63) scan32[wv] = incl;
    __syncthreads();
    const uint32_t tq = (wl < NW) ? scan32[wl] : 0u;
    const uint32_t tot_packed = row16_u32(tq, OpAddU());
    const uint32_t ex =
        row16_u32((wl < wv) ? tq : 0u, OpAddU()) + incl - packed;
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
      if (pos >= 0 && pos < n) keys_lds[pos] = (uint32_t)(pbase + i);
    }
    count = min((int)((tot_packed >> 16) + min((unsigned long long)(tot_packed & 0xFFFFu), need)),
                n);
    __syncthreads();
    int32_t* lp = sel_pages + (int64_t)u * max_pages;
    int32_t* lx = sel_phys + (int64_t)u * max_pages;
    const int32_t* pt = page_table + (int64_t)b * max_pages;
    for (int i = tid; i < count; i += NT) {
      const int p = (int)keys_lds[i];
      lp[i] = p;
      if constexpr (kStagePt) lx[i] = ptl[p];
      else lx[i] = pt[p];
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
  unsigned long long run = 0ull;
  for (int base = 0; base < U; base += NT) {
    const int v = base + tid;
    unsigned long long c = 0ull;
    if (v < U)
      c = (unsigned long long)__hip_atomic_load(sel_counts + v, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long tot;
    const unsigned long long ex = block_excl_scan<unsigned long long, NT>(c, scan64, tot);
    if (v < U) sel_offsets[v] = (int32_t)(run + ex);
    run += tot;
  }
  if (tid == 0) {
    sel_offsets[U] = (int32_t)run;
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One workgroup per unit, NT threads, the smallest NPT with NPT * NT >=
// max_pages (select_threads keeps NPT <= 8 below 1024 threads and >= 8 at
// 1024, so only those forms are built).
// Returns false, launching nothing, when the row does not fit NPT * NT.
template <bool COUNT, int NT>
static bool launch_select(hipStream_t st, int U, const float* logits, const int32_t* ctx_lens,
                          const int32_t* page_table, float gamma, int k_pages, int hkv,
                          int group, int max_pages, int32_t* sel_counts,
                          int32_t* sel_offsets, int32_t* sel_pages,
                          int32_t* sel_phys, uint32_t* ticket) {
  const int npt = (max_pages + NT - 1) / NT;
#define SP_SEL(N)                                                                               \
  hipLaunchKernelGGL((select_kernel<N, COUNT, NT>), dim3(U), dim3(NT), 0, st, logits, ctx_lens, \
                     page_table, gamma, k_pages, hkv, group, max_pages, U, sel_counts,       \
                     sel_offsets, sel_pages, sel_phys, ticket)
  if constexpr (NT == 256) {
    if (npt <= 1) SP_SEL(1);
    else if (npt <= 2) SP_SEL(2);
    else if (npt <= 4) SP_SEL(4);
    else if (npt <= 8) SP_SEL(8);
    else return false;
  } else if constexpr (NT == 512) {
    if (npt <= 8) SP_SEL(8);
    else return false;
  } else {
    if (npt <= 8) SP_SEL(8);
    else if (npt <= 16) SP_SEL(16);
    else if (npt <= 32) SP_SEL(32);
    else return false;
  }
#undef SP_SEL
  return true;
}

// Threads per selection workgroup for rows of max_pages pages: the fewest of
// 256, 512 and 1024 that hold the row at 8 pages per thread.  The kernel is a
// chain of block-wide steps, and with fewer waves each barrier and each LDS
// combine is shorter; past 8 pages per thread the per-thread work costs more
// than that saves (timed at 256, 2048 and 8192 pages).
static int select_threads(int max_pages) {
  if (max_pages <= 8 * 256) return 256;
  if (max_pages <= 8 * 512) return 512;
  return kSelThreads;
}

template <bool COUNT>
static sparse_status select_entry(const sparse_dims* dims, const float* logits,
                                  const int32_t* ctx_lens, const int32_t* page_table, float gamma,
                                  int k_pages, int32_t* sel_counts, int32_t* sel_offsets,
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
                                  int k_pages, int32_t* sel_counts, int32_t* sel_offsets,
                                  int32_t* sel_pages, int32_t* sel_phys, void* ws,
                                  size_t ws_bytes, void* stream) {
  sparse_status st = check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!logits || !ctx_lens || !page_table || !sel_counts || !sel_pages || !sel_phys)
    return SPARSE_ERR_INVALID;
  if (sel_offsets != nullptr &&
      (!ws || ws_bytes < sparse_select_workspace_bytes(dims) || !aligned(ws, 4)))
    return SPARSE_ERR_WORKSPACE;
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* ticket = static_cast<uint32_t*>(ws);
#define SP_SEL(NT)                                                                              \
  launch_select<COUNT, NT>(s, U, logits, ctx_lens, page_table, gamma, k_pages, hkv, group,     \
                           dims->max_pages, sel_counts, sel_offsets, sel_pages, sel_phys, ticket)
  bool ok;
  switch (select_threads(dims->max_pages)) {
    case 256: ok = SP_SEL(256); break;
    case 512: ok = SP_SEL(512); break;
    default: ok = SP_SEL(1024); break;
  }
#undef SP_SEL
  if (!ok) return SPARSE_ERR_UNSUPPORTED;
  return launch_status();
}

}  // namespace sp

extern "C" sparse_status sparse_select_coverage(const sparse_dims* dims, const float* logits,
                                                const int32_t* ctx_lens, const int32_t* page_table,
                                                float gamma, int32_t* sel_counts,
                                                int32_t* sel_offsets, int32_t* sel_pages,
                                                int32_t* sel_phys, void* ws, size_t ws_bytes,
                                                void* stream) {
  if (!(gamma > 0.0f && gamma <= 1.0f)) return SPARSE_ERR_INVALID;
  return sp::select_entry<false>(dims, logits, ctx_lens, page_table, gamma, 0, sel_counts,
                                 sel_offsets, sel_pages, sel_phys, ws, ws_bytes, stream);
}

extern "C" sparse_status sparse_select_topk(const sparse_dims* dims, const float* logits,
                                            const int32_t* ctx_lens, const int32_t* page_table,
                                            int32_t k_pages, int32_t* sel_counts,
                                            int32_t* sel_offsets, int32_t* sel_pages,
                                            int32_t* sel_phys, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (k_pages < 1) return SPARSE_ERR_INVALID;
  return sp::select_entry<true>(dims, logits, ctx_lens, page_table, 1.0f, k_pages, sel_counts,
                                sel_offsets, sel_pages, sel_phys, ws, ws_bytes, stream);
}
