// The coverage rule: per (request, KV head) unit, the smallest page set whose
// estimated attention mass reaches a fraction gamma of the total ("Adaptive
// DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", MOIRA
// abstract, coverage-rule sentence).
//
// One 1024-thread workgroup per unit; thread t owns pages [t*NPT, t*NPT+NPT)
// in registers.  Steps:
//   1. per query head g: (max, sum of exp) over the unit's pages by one
//      block reduction, then m[p] += exp(x_g[p] - max_g) / sum_g;  m /= G.
//   2. weights w[p] = floor(m[p] * 2^52) (exact 64-bit fixed point, so the
//      cut's sums are exact and order independent) and keys = fp32 bits of
//      m[p] (monotone for m >= 0).
//   3. target T = ceil(gamma * sum w); a mass-weighted radix select over the
//      key bits (11 + 11 + 9 bits, LDS histograms of counts and weights,
//      suffix scans) finds the key tau with W(key > tau) < T <= W(key >= tau).
//   4. keep every page with key > tau plus the r lowest-index pages with key
//      == tau, r = ceil((T - W(key > tau)) / w_tau); compact in ascending page
//      order by a block prefix sum.
//   5. the last workgroup to finish (device ticket) writes the prefix sums of
//      the counts and of the chunk counts over all units, then re-arms the
//      ticket -- the plan the attention kernel reads, made on the device.

#include "common.h"

namespace sp {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

struct PairMS {
  float m, s;
};

__device__ __forceinline__ PairMS combine(PairMS a, PairMS b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return {M, 0.f};
  const float sa = (a.m == -INFINITY) ? 0.f : a.s * __expf(a.m - M);
  const float sb = (b.m == -INFINITY) ? 0.f : b.s * __expf(b.m - M);
  return {M, sa + sb};
}

template <int NPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ page_table, float gamma, int chunk_pages, int hkv, int group,
    int max_pages, int U, int32_t* __restrict__ sel_counts, int32_t* __restrict__ sel_offsets,
    int32_t* __restrict__ chunk_offsets, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ sel_phys, uint32_t* __restrict__ ticket) {
  __shared__ uint32_t hcnt[2048];
  __shared__ unsigned long long hw[2048];
  __shared__ float red_m[kSelWaves], red_s[kSelWaves];
  __shared__ unsigned long long scan64[kSelWaves];
  __shared__ uint32_t scan32[kSelWaves];
  __shared__ int s_bin;
  __shared__ unsigned long long s_wgt;
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int u = blockIdx.x;
  const int b = u / hkv;
  const int L = min(max(ctx_lens[b], 0), max_pages * kP);
  const int n = (L + kP - 1) / kP;
  const int pbase = tid * NPT;
  int count = 0;

  if (n > 0) {
    const float* X = logits + (int64_t)u * group * max_pages;
    float m[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) m[i] = 0.f;

    // ---- 1. per-head softmax normalisers, group mass --------------------
    for (int g = 0; g < group; ++g) {
      float xv[NPT];
      const float* Xg = X + (int64_t)g * max_pages;
#pragma unroll
      for (int i = 0; i < NPT; ++i) xv[i] = (pbase + i < n) ? Xg[pbase + i] : -INFINITY;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPT; ++i) mx = fmaxf(mx, xv[i]);
      float se = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) se += __expf(xv[i] - mx);
      }
      PairMS pr = {mx, se};
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        PairMS other = {__shfl_xor(pr.m, o, 64), __shfl_xor(pr.s, o, 64)};
        pr = combine(pr, other);
      }
      if (lane == 0) {
        red_m[wv] = pr.m;
        red_s[wv] = pr.s;
      }
      __syncthreads();
      PairMS tot = {red_m[0], red_s[0]};
#pragma unroll
      for (int w = 1; w < kSelWaves; ++w) tot = combine(tot, PairMS{red_m[w], red_s[w]});
      __syncthreads();
      const float inv = 1.f / tot.s;
#pragma unroll
      for (int i = 0; i < NPT; ++i)
        if (pbase + i < n) m[i] += __expf(xv[i] - tot.m) * inv;
    }
    const float invg = 1.f / (float)group;
    uint32_t key[NPT];
    unsigned long long wsum_local = 0ull;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const float mi = m[i] * invg;
      key[i] = (pbase + i < n) ? __float_as_uint(mi) : 0u;
      wsum_local += (unsigned long long)(__uint_as_float(key[i]) * 4503599627370496.0f);  // 2^52
    }
    const unsigned long long Z = block_sum<unsigned long long, kSelThreads>(wsum_local, scan64);

    // ---- 2-4. the cut ---------------------------------------------------
    uint32_t tau = 0u;
    unsigned long long need = 0ull, w_tau = 1ull;
    const bool all = !(gamma < 1.0f);
    if (!all) {
      unsigned long long T = (unsigned long long)ceil((double)gamma * (double)Z);
      if (T > Z) T = Z;
      if (T < 1ull) T = 1ull;
      uint32_t prefix = 0u, hi_mask = 0u;
      const int shifts[3] = {20, 9, 0};
      const int widths[3] = {11, 11, 9};
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        const int sh = shifts[pass], nb = 1 << widths[pass];
        for (int k = tid; k < nb; k += kSelThreads) {
          hcnt[k] = 0u;
          hw[k] = 0ull;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
          if (pbase + i < n && (key[i] & hi_mask) == prefix) {
            const int bin = (key[i] >> sh) & (nb - 1);
            atomicAdd(&hcnt[bin], 1u);
            atomicAdd(&hw[bin], (unsigned long long)(__uint_as_float(key[i]) * 4503599627370496.0f));
          }
        }
        __syncthreads();
        // thread t owns bins 2t, 2t+1; find the bin where the running weight
        // from the top crosses T.
        const int b0 = 2 * tid, b1 = 2 * tid + 1;
        const unsigned long long w0 = (b0 < nb) ? hw[b0] : 0ull;
        const unsigned long long w1 = (b1 < nb) ? hw[b1] : 0ull;
        unsigned long long total;
        const unsigned long long ex = block_excl_scan<unsigned long long, kSelThreads>(w0 + w1, scan64, total);
        const unsigned long long gt1 = total - (ex + w0 + w1);  // weight of bins > b1
        const unsigned long long gt0 = gt1 + w1;                // weight of bins > b0
        if (b1 < nb && gt1 < T && T <= gt1 + w1) {
          s_bin = b1;
          s_wgt = gt1;
        }
        if (b0 < nb && gt0 < T && T <= gt0 + w0) {
          s_bin = b0;
          s_wgt = gt0;
        }
        __syncthreads();
        const int bin = s_bin;
        T -= s_wgt;
        prefix |= (uint32_t)bin << sh;
        hi_mask |= (uint32_t)(nb - 1) << sh;
        if (pass == 2) {
          // every page with key tau has the same weight
          const unsigned long long cnt = hcnt[bin];
          w_tau = cnt ? hw[bin] / cnt : 1ull;
          if (w_tau == 0ull) w_tau = 1ull;
        }
        __syncthreads();
      }
      tau = prefix;
      need = (T + w_tau - 1ull) / w_tau;  // ties at tau to keep, >= 1
    }

    // ---- rank ties, compact in ascending page order ---------------------
    uint32_t ties_local = 0u;
    if (!all) {
#pragma unroll
      for (int i = 0; i < NPT; ++i) ties_local += (pbase + i < n && key[i] == tau) ? 1u : 0u;
    }
    uint32_t ties_total;
    const uint32_t tie_rank0 = block_excl_scan<uint32_t, kSelThreads>(ties_local, scan32, ties_total);
    uint32_t keep_mask = 0u, keep_local = 0u, tr = tie_rank0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      bool keep = false;
      if (pbase + i < n) {
        if (all) {
          keep = true;
        } else if (key[i] > tau) {
          keep = true;
        } else if (key[i] == tau) {
          keep = (unsigned long long)tr < need;
          ++tr;
        }
      }
      if (keep) {
        keep_mask |= 1u << i;
        ++keep_local;
      }
    }
    uint32_t kept_total;
    uint32_t pos = block_excl_scan<uint32_t, kSelThreads>(keep_local, scan32, kept_total);
    int32_t* lp = sel_pages + (int64_t)u * max_pages;
    int32_t* lx = sel_phys + (int64_t)u * max_pages;
    const int32_t* pt = page_table + (int64_t)b * max_pages;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (keep_mask & (1u << i)) {
        lp[pos] = pbase + i;
        lx[pos] = pt[pbase + i];
        ++pos;
      }
    }
    count = (int)kept_total;
  }

  // ---- 5. last workgroup: prefix sums over units --------------------------
  if (tid == 0) sel_counts[u] = count;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t t = atomicAdd(ticket, 1u);
    s_last = (t == (uint32_t)(U - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  uint32_t run = 0u, runc = 0u;
  for (int base = 0; base < U; base += kSelThreads) {
    const int v = base + tid;
    uint32_t c = 0u;
    if (v < U) c = (uint32_t)__hip_atomic_load(sel_counts + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ch = (c + (uint32_t)chunk_pages - 1u) / (uint32_t)chunk_pages;
    uint32_t t1, t2;
    const uint32_t e1 = block_excl_scan<uint32_t, kSelThreads>(c, scan32, t1);
    const uint32_t e2 = block_excl_scan<uint32_t, kSelThreads>(ch, scan32, t2);
    if (v < U) {
      sel_offsets[v] = (int32_t)(run + e1);
      chunk_offsets[v] = (int32_t)(runc + e2);
    }
    run += t1;
    runc += t2;
  }
  if (tid == 0) {
    sel_offsets[U] = (int32_t)run;
    chunk_offsets[U] = (int32_t)runc;
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int NPT>
static void launch_select(hipStream_t st, int U, const float* logits, const int32_t* ctx_lens,
                          const int32_t* page_table, float gamma, int chunk_pages, int hkv,
                          int group, int max_pages, int32_t* sel_counts, int32_t* sel_offsets,
                          int32_t* chunk_offsets, int32_t* sel_pages, int32_t* sel_phys,
                          uint32_t* ticket) {
  hipLaunchKernelGGL(select_kernel<NPT>, dim3(U), dim3(kSelThreads), 0, st, logits, ctx_lens,
                     page_table, gamma, chunk_pages, hkv, group, max_pages, U, sel_counts,
                     sel_offsets, chunk_offsets, sel_pages, sel_phys, ticket);
}

}  // namespace sp

extern "C" size_t sparse_select_workspace_bytes(const sparse_dims* dims) {
  (void)dims;
  return 256;  // the finishing ticket (one 32-bit counter), padded
}

extern "C" sparse_status sparse_select_coverage(const sparse_dims* dims, const float* logits,
                                                const int32_t* ctx_lens, const int32_t* page_table,
                                                float gamma, int32_t chunk_pages,
                                                int32_t* sel_counts, int32_t* sel_offsets,
                                                int32_t* chunk_offsets, int32_t* sel_pages,
                                                int32_t* sel_phys, void* ws, size_t ws_bytes,
                                                void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!logits || !ctx_lens || !page_table || !sel_counts || !sel_offsets || !chunk_offsets ||
      !sel_pages || !sel_phys)
    return SPARSE_ERR_INVALID;
  if (!(gamma > 0.0f && gamma <= 1.0f)) return SPARSE_ERR_INVALID;
  if (chunk_pages < 1 || chunk_pages > dims->max_pages) return SPARSE_ERR_INVALID;
  if (!ws || ws_bytes < sparse_select_workspace_bytes(dims) || !sp::aligned(ws, 4))
    return SPARSE_ERR_WORKSPACE;
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  const int npt = (dims->max_pages + sp::kSelThreads - 1) / sp::kSelThreads;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* ticket = static_cast<uint32_t*>(ws);
#define SP_SEL(N)                                                                             \
  sp::launch_select<N>(s, U, logits, ctx_lens, page_table, gamma, chunk_pages, hkv, group,   \
                       dims->max_pages, sel_counts, sel_offsets, chunk_offsets, sel_pages,   \
                       sel_phys, ticket)
  if (npt <= 1) SP_SEL(1);
  else if (npt <= 2) SP_SEL(2);
  else if (npt <= 4) SP_SEL(4);
  else if (npt <= 8) SP_SEL(8);
  else if (npt <= 16) SP_SEL(16);
  else SP_SEL(32);
#undef SP_SEL
  return sp::launch_status();
}
