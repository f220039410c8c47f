// Self-planning split-K decode attention over variable-length page lists
// ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
// Hierarchy", MOIRA abstract, sentence on self-planning attention: every block
// works out from the per-head list lengths which part it handles, so no plan
// is made on the host and the step stays inside the graph; and the sentence on
// FA3/FlashInfer, whose padded lists, unbalanced blocks or host-side plans this
// avoids).
//
// The grid is fixed (W workgroups, W chosen by the caller, typically one per
// compute unit).  Every workgroup reads the list lengths, lays the step's
// lists end to end and takes an even 1/W of all their entries -- a slice that
// may start in one unit's list and end in another's -- so every workgroup has
// the same number of pages whatever the lengths (balanced plan in common.h).
// It attends its slice one unit segment at a time; its 4 waves split a
// segment's pages and each runs an online softmax for the unit's G query
// heads on the bf16 matrix cores:
//   QK:  S^T[t][g] = K[t][:] . q[g][:]   v_mfma_f32_16x16x32_bf16, 4 k-slices
//        (A = K tile rows = tokens, read straight from HBM in 16-byte runs;
//         B = q of the group, columns = heads)
//   PV:  O^T[d][g] += V^T[d][t] P^T[t][g]  v_mfma_f32_16x16x16bf16_1k, 8 tiles
//        (A = the channel-major V tile, 8-byte token runs; B = P, which the
//         QK result layout already holds in the right lanes).  P is split
//        into a bf16 high part and a bf16 residual, two products, so the
//        weights keep ~16 significant bits.
// The 4 waves' (max, sum, O) are merged in LDS into one normalised partial
// and its log-sum-exp per head, written to slot u + w (unit u, worker w), so
// the merge finds a unit's partials from the same lengths.

#include "common.h"
#include "fetch.h"

namespace sp {

constexpr int kAttnWaves = 4;

struct PageFrag {
  u32x4 k[4];   // K tile: token (lane & 15), channels 32 s + 8 (lane >> 4) .. +7
  u32x2 v[8];   // V^T tile m: channel 16 m + (lane & 15), tokens 4 (lane >> 4) .. +3
  int valid;    // valid tokens (0 = skip page)
};

// Issue the loads of one page's K and V fragments.  p is the logical page,
// x its physical page (or cache slot); both are wave-uniform.  K/V are read
// once per step, so the loads are non-temporal (streaming).  The loads are
// unconditional: a page that is out of range or past the context reads page
// 0 of the pool instead (always in bounds) and is marked empty, so
// attend_page skips it.  (Zero-filling the registers instead would be a
// write that has to wait for every load still in flight.)
__device__ __forceinline__ void load_page(PageFrag& f, const uint16_t* __restrict__ kv,
                                          int64_t stride_page, int64_t stride_head,
                                          int64_t pool_pages, int h, int L, int p, int x) {
  const int lane = lane_id(), row = lane & 15, j = lane >> 4;
  const int nv = min(kP, L - kP * p);
  const bool ok = x >= 0 && x < pool_pages && p >= 0 && nv > 0;
  f.valid = ok ? nv : 0;
  const uint16_t* kt = kv + (int64_t)(ok ? x : 0) * stride_page + (int64_t)h * stride_head;
  const uint16_t* vt = kt + kTile;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    f.k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + row * kD + 32 * s + 8 * j));
#pragma unroll
  for (int m = 0; m < 8; ++m)
    f.v[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vt + (16 * m + row) * kP + 4 * j));
}

// One page of the online softmax: QK on the matrix cores, running max/sum
// update, PV with P split into bf16 high and residual parts.
__device__ __forceinline__ void attend_page(PageFrag& f, const bf16x8* qf, bool gok, int j,
                                            float scale_log2, float& m_run, float& l_run,
                                            floatx4* o) {
  if (f.valid == 0) return;
  floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.k[s]), qf[s], sacc, 0, 0, 0);
  // lane (g, j): logits of tokens 4j + e, in log2 units
  float xs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    xs[e] = (gok && 4 * j + e < f.valid) ? sacc[e] * scale_log2 : -INFINITY;
  float pm = fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3]));
  pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
  pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
  const float m_new = gok ? fmaxf(m_run, pm) : 0.f;
  const float alpha = gok ? exp2f(m_run - m_new) : 1.f;
  float pv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pv[e] = gok ? exp2f(xs[e] - m_new) : 0.f;
  l_run = l_run * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
  m_run = gok ? m_new : m_run;
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] *= alpha;
  if (f.valid < kP) {
    // zero V of tokens past the end of the context (they may hold anything)
    const int t0 = 4 * j;
    const uint32_t k0 = (t0 + 0 < f.valid ? 0x0000FFFFu : 0u) | (t0 + 1 < f.valid ? 0xFFFF0000u : 0u);
    const uint32_t k1 = (t0 + 2 < f.valid ? 0x0000FFFFu : 0u) | (t0 + 3 < f.valid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      f.v[m][0] &= k0;
      f.v[m][1] &= k1;
    }
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = f32_to_bf16_rne(pv[e]);
    lo[e] = f32_to_bf16_rne(pv[e] - __uint_as_float(hi[e] << 16));
  }
  const short4v phi = as_short4(u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)});
  const short4v plo = as_short4(u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)});
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_short4(f.v[m]), phi, o[m], 0, 0, 0);
    o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_short4(f.v[m]), plo, o[m], 0, 0, 0);
  }
}

// One unit segment of a workgroup's slice: unit u's list entries [i0, i1).
// seg_begin issues the segment's first loads (context length, the first 64
// list ids of each wave) in one round trip and returns without waiting for
// them.  Every load is unconditional (an index past the segment re-reads its
// last entry): a load under a condition becomes a branch that waits for it.
struct Seg {
  int u, b, h, L, i0, i1;
  int pl, xl;        // lane k: logical / physical id of this wave's k-th page of the batch
};

__device__ __forceinline__ void seg_begin(Seg& S, const int32_t* __restrict__ ctx_lens,
                                          const int32_t* __restrict__ sel_pages,
                                          const int32_t* __restrict__ sel_phys, int hkv,
                                          int max_pages, int u, int i0, int i1) {
  // (lane and thread index through empty asm statements: the lane-dependent
  // address parts are computed here rather than hoisted out of the segment
  // loop, where they would be live, or spilled, across the page loop)
  int lane = lane_id(), tid = threadIdx.x;
  asm volatile("" : "+v"(lane), "+v"(tid));
  const int wv = tid >> 6;
  S.u = u;
  S.b = u / hkv;
  S.h = u - S.b * hkv;
  S.i0 = i0;
  S.i1 = i1;
  S.L = __builtin_amdgcn_readfirstlane(min(max(ctx_lens[S.b], 0), max_pages * kP));
  const int64_t rowoff = (int64_t)u * max_pages;
  const int ie = min(i0 + wv + kAttnWaves * lane, i1 - 1);
  S.pl = sel_pages[rowoff + ie];
  S.xl = sel_phys[rowoff + ie];
}

// The segment's pages: each wave takes list entries i0 + wv + 4k and runs an
// online softmax over them (m_run, l_run, o).  The ids are read 64 at a time
// into lanes k and broadcast with readlane, so no KV load waits on a list
// load; each batch's ids are loaded while the previous batch is attended.
// The unit's queries are loaded here, beside the first page (their round
// trip overlaps the page's), so no register carries them between segments.
__device__ __forceinline__ void seg_pages(Seg& S, const uint16_t* __restrict__ q, int hkv,
                                          const uint16_t* __restrict__ kv,
                                          int64_t stride_page, int64_t stride_head,
                                          int64_t pool_pages,
                                          const int32_t* __restrict__ sel_pages,
                                          const int32_t* __restrict__ sel_phys, float scale_log2,
                                          int group, int max_pages, float& m_run, float& l_run,
                                          floatx4 (&o)[8]) {
  const int lane = lane_id(), wv = threadIdx.x >> 6, row = lane & 15, j = lane >> 4;
  const bool gok = row < group;
  const int h = S.h, L = S.L, i0 = S.i0, i1 = S.i1;
  const int32_t* lp = sel_pages + (int64_t)S.u * max_pages;
  const int32_t* lx = sel_phys + (int64_t)S.u * max_pages;
  int pl = S.pl, xl = S.xl;
  asm volatile("" : "+v"(pl), "+v"(xl));
  // B operand of QK: q of head g = row.  A padding column (g >= group)
  // re-reads the group's last head; its logits and weights are masked in
  // attend_page, so it is not zeroed (a select here would wait for the load).
  const uint16_t* qrow =
      q + ((int64_t)S.b * hkv * group + h * group + min(row, group - 1)) * kD + 8 * j;
  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * s));
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (i1 - i0 - wv + kAttnWaves - 1) / kAttnWaves;
  for (int base = 0; base < nk; base += 64) {
    const int cnt_k = min(64, nk - base);
    const int ie_next = min(i0 + wv + kAttnWaves * (base + 64 + lane), i1 - 1);
    const int pl_next = lp[ie_next];
    const int xl_next = lx[ie_next];
    // Two page buffers in turn, so a page's loads are in flight while the
    // other page is attended and no register copy waits on them.  In the
    // steady-state loop every load is unconditional (a branch around a load
    // makes the compiler wait for all loads where the paths meet); the last
    // one or two pages are handled after it.
    PageFrag fa, fb;
    load_page(fa, kv, stride_page, stride_head, pool_pages, h, L,
              __builtin_amdgcn_readlane(pl, 0), __builtin_amdgcn_readlane(xl, 0));
    int k = 0;
    for (; k + 2 < cnt_k; k += 2) {
      load_page(fb, kv, stride_page, stride_head, pool_pages, h, L,
                __builtin_amdgcn_readlane(pl, k + 1), __builtin_amdgcn_readlane(xl, k + 1));
      attend_page(fa, qf, gok, j, scale_log2, m_run, l_run, o);
      load_page(fa, kv, stride_page, stride_head, pool_pages, h, L,
                __builtin_amdgcn_readlane(pl, k + 2), __builtin_amdgcn_readlane(xl, k + 2));
      attend_page(fb, qf, gok, j, scale_log2, m_run, l_run, o);
    }
    if (k + 1 < cnt_k) {
      load_page(fb, kv, stride_page, stride_head, pool_pages, h, L,
                __builtin_amdgcn_readlane(pl, k + 1), __builtin_amdgcn_readlane(xl, k + 1));
      attend_page(fa, qf, gok, j, scale_log2, m_run, l_run, o);
      attend_page(fb, qf, gok, j, scale_log2, m_run, l_run, o);
    } else {
      attend_page(fa, qf, gok, j, scale_log2, m_run, l_run, o);
    }
    pl = pl_next;
    xl = xl_next;
  }
}

// A workgroup barrier that orders LDS accesses only.  __syncthreads() is a
// fence over all memory, which waits for every global load the wave has in
// flight; this one lets the next segment's loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Merge the 4 waves' (max, sum, O) in LDS into one normalised partial and
// its log-sum-exp per head, written to `slot`, in two calls made by all 256
// threads: seg_stage puts each wave's (max, sum, O) in LDS (after it the
// accumulators are free), seg_combine merges them.  Loads issued between
// the two stay in flight through seg_combine's barriers.
__device__ __forceinline__ void seg_stage(float m_run, float l_run, const floatx4 (&o)[8],
                                          int group, float* smem) {
  int lane = lane_id(), tid = threadIdx.x;       // (not hoisted: as in seg_begin)
  asm volatile("" : "+v"(lane), "+v"(tid));
  const int wv = tid >> 6, g = lane & 15, j = lane >> 4;
  const bool gok = g < group;
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  float* so = smem;                                   // [kAttnWaves][group][kD]
  float* sm = smem + kAttnWaves * group * kD;         // [kAttnWaves][group]
  float* sl = sm + kAttnWaves * group;
  if (gok) {
    float* dst = so + (wv * group + g) * kD;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *reinterpret_cast<floatx4*>(dst + 16 * m + 4 * j) = o[m];
    if (j == 0) {
      sm[wv * group + g] = m_run;
      sl[wv * group + g] = l_run;
    }
  }
}

__device__ __forceinline__ void seg_combine(int group, int64_t slot, const float* smem,
                                            float* __restrict__ part_o,
                                            float* __restrict__ part_lse) {
  const float* so = smem;
  const float* sm = smem + kAttnWaves * group * kD;
  const float* sl = sm + kAttnWaves * group;
  lds_barrier();
  const float ln2 = 0.6931471805599453f;
  // (the thread index passes through an empty asm statement so that the
  // addresses below are computed here, not hoisted out of the segment loop
  // and kept live, or spilled, across the page loop)
  int t0 = threadIdx.x;
  asm volatile("" : "+v"(t0));
  for (int idx = t0; idx < group * kD; idx += 256) {
    const int gg = idx / kD, d = idx - (idx / kD) * kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm[w * group + gg]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = sm[w * group + gg];
        if (mw == -INFINITY) continue;
        const float a = exp2f(mw - M);
        num += a * so[(w * group + gg) * kD + d];
        den += a * sl[w * group + gg];
      }
    }
    const int64_t r = slot * group + gg;
    part_o[r * kD + d] = (den > 0.f) ? num / den : 0.f;
    if (d == 0) part_lse[r] = (den > 0.f) ? (M + log2f(den)) * ln2 : -INFINITY;
  }
  lds_barrier();     // the LDS is reused by the workgroup's next segment
}

// Worker w of the balanced plan: its slice of the step's list entries, one
// unit segment at a time.  Uses the launch's dynamic LDS: [waves][group][128]
// O, then [waves][group] m and l.
__device__ __forceinline__ void attn_worker(
    int w, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t stride_page,
    int64_t stride_head, int64_t pool_pages, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_phys, float scale_log2, int hkv, int group, int max_pages,
    int cap, int U, int wmax, float* __restrict__ part_o, float* __restrict__ part_lse) {
  extern __shared__ float smem[];
  int x, e, u, off, len;
  {
    PlanSeg first;
    const int total = __builtin_amdgcn_readfirstlane(plan_total(sel_counts, U, cap, first));
    const int W = plan_workers(total, wmax);
    if (w >= W) return;                // the step has too few pages for this worker
    x = plan_start(w, W, total);
    e = plan_start(w + 1, W, total);
    plan_find(sel_counts, U, cap, first, x, u, off, len);
  }
  u = __builtin_amdgcn_readfirstlane(u);
  off = __builtin_amdgcn_readfirstlane(off);
  len = __builtin_amdgcn_readfirstlane(len);
  if (u < 0) return;                   // (x < T always lies in some unit)
  // Unit u's entries are its positions past the first kPlanUnitCost; the
  // worker's first unit always gives it some (its range is longer than that).
  constexpr int C = kPlanUnitCost;
  Seg cur;
  seg_begin(cur, ctx_lens, sel_pages, sel_phys, hkv, max_pages, u, max(x - off - C, 0),
            min(e, off + len) - off - C);
  // Segment by segment.  After the first, the next unit is u + 1 (its length
  // loaded at the segment's start), skipping empty lists.  x < e <= T, so a
  // later unit holds position x whenever the loop goes on; the u < U - 1
  // test only guards against lengths changed under the kernel.  A range that
  // ends within a unit's first C positions gives no entries there.  The next
  // segment's first loads are issued before this one's epilogue, whose
  // barriers order LDS only, so they are in flight while it runs.
  while (true) {
    const int next_raw = sel_counts[min(u + 1, U - 1)];
    float m_run, l_run;
    floatx4 o[8];
    seg_pages(cur, q, hkv, kv, stride_page, stride_head, pool_pages, sel_pages, sel_phys,
              scale_log2, group, max_pages, m_run, l_run, o);
    const int64_t slot = (int64_t)cur.u + w;
    bool more = off + C + cur.i1 < e;
    if (more) {
      off += len;
      ++u;
      len = plan_positions(next_raw, cap);
      while (len == 0 && u < U - 1) {
        ++u;
        len = plan_positions(sel_counts[u], cap);
      }
      more = len > 0 && e - off > C;
    }
    seg_stage(m_run, l_run, o, group, smem);
    if (more)
      seg_begin(cur, ctx_lens, sel_pages, sel_phys, hkv, max_pages, u, 0,
                min(e, off + len) - off - C);
    seg_combine(group, slot, smem, part_o, part_lse);
    if (!more) break;
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t stride_page,
    int64_t stride_head, int64_t pool_pages, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ sel_counts, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_phys, float scale_log2, int hkv, int group, int max_pages,
    int cap, int U, int wmax, float* __restrict__ part_o, float* __restrict__ part_lse) {
  attn_worker(blockIdx.x, q, kv, stride_page, stride_head, pool_pages, ctx_lens, sel_counts,
              sel_pages, sel_phys, scale_log2, hkv, group, max_pages, cap, U, wmax, part_o,
              part_lse);
}

// A host-tier miss on its way through a copying wave: read from pinned host
// memory as the plain copy reads it (lane l of read k holds bytes
// 1024 k + 16 l .. + 15 of the unit: every read is 1 KiB contiguous),
// written to its slot the same way, and staged in the wave's LDS tile to be
// read back in load_page's fragment layout.  K rows are padded to 272 bytes
// in LDS, so the fragment reads of 16 rows fall in distinct banks.
struct RawUnit {
  u32x4 t[8];
};
constexpr int kStageKRow = 2 * kD + 16;                   // bytes per padded K row
constexpr int kStageBytes = kP * kStageKRow + 2 * kTile;  // padded K tile + V tile

__device__ __forceinline__ void load_raw(RawUnit& r, const uint16_t* __restrict__ unit) {
  const u32x4* s = reinterpret_cast<const u32x4*>(unit);
  const int lane = lane_id();
#pragma unroll
  for (int k = 0; k < 8; ++k) r.t[k] = __builtin_nontemporal_load(s + k * 64 + lane);
}

__device__ __forceinline__ void store_raw(const RawUnit& r, uint16_t* __restrict__ unit) {
  u32x4* d = reinterpret_cast<u32x4*>(unit);
  const int lane = lane_id();
#pragma unroll
  for (int k = 0; k < 8; ++k) d[k * 64 + lane] = r.t[k];
}

// Through the wave's LDS tile into f (K token (lane & 15), V^T channels).
__device__ __forceinline__ void raw_to_frag(const RawUnit& r, char* tile, PageFrag& f) {
  const int lane = lane_id(), row = lane & 15, j = lane >> 4;
#pragma unroll
  for (int k = 0; k < 4; ++k)          // K: token 4k + (lane >> 4), channels 8 (lane & 15) ..
    *reinterpret_cast<u32x4*>(tile + (4 * k + j) * kStageKRow + 16 * row) = r.t[k];
  char* vt = tile + kP * kStageKRow;
#pragma unroll
  for (int k = 4; k < 8; ++k) *reinterpret_cast<u32x4*>(vt + (k - 4) * 1024 + 16 * lane) = r.t[k];
  // the wave's own LDS writes, read back by other lanes: complete them, and
  // keep the compiler from moving the reads above them
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int s = 0; s < 4; ++s)
    f.k[s] = *reinterpret_cast<const u32x4*>(tile + row * kStageKRow + 64 * s + 16 * j);
#pragma unroll
  for (int m = 0; m < 8; ++m)
    f.v[m] = *reinterpret_cast<const u32x2*>(vt + (16 * m + row) * 32 + 8 * j);
  asm volatile("" ::: "memory");     // the next unit's LDS writes stay after these reads
}

// A copying wave of the host tier's fetch: wave fw of FW is worker fw of the
// balanced plan over the per-unit miss lists (miss_counts, miss_pages,
// miss_phys), one worker per wave.  For each miss of its slice it reads the
// unit from pinned host memory into registers, writes it to its slot, and
// attends it from its LDS tile with the unit's queries (one online softmax
// per unit segment), so the misses are attended without being read back
// from HBM.  Uses kStageBytes of the launch's dynamic LDS per wave.
// Each segment's normalised partial and log-sum-exp go to slot u + fw of
// part_o / part_lse, where the merge finds them from miss_counts and FW as
// it finds the attention's.  A miss whose page or slot is out of range is
// neither copied nor attended.
__device__ __forceinline__ void miss_worker(
    int fw, int FW, const uint16_t* __restrict__ host_kv, uint16_t* __restrict__ cache_kv,
    int64_t pool_slots, const uint16_t* __restrict__ q, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ miss_counts, const int32_t* __restrict__ miss_pages,
    const int32_t* __restrict__ miss_phys, float scale_log2, int hkv, int group, int max_pages,
    int cap, int U, float* __restrict__ part_o, float* __restrict__ part_lse) {
  int x, e, u, off, len;
  {
    PlanSeg first;
    const int total = __builtin_amdgcn_readfirstlane(plan_total(miss_counts, U, cap, first));
    const int W = plan_workers(total, FW);
    if (fw >= W) return;               // nothing to copy, or too little for this wave
    x = plan_start(fw, W, total);
    e = plan_start(fw + 1, W, total);
    plan_find(miss_counts, U, cap, first, x, u, off, len);
  }
  u = __builtin_amdgcn_readfirstlane(u);
  off = __builtin_amdgcn_readfirstlane(off);
  len = __builtin_amdgcn_readfirstlane(len);
  if (u < 0) return;
  constexpr int C = kPlanUnitCost;
  const int lane = lane_id(), row = lane & 15, j = lane >> 4;
  const bool gok = row < group;
  extern __shared__ float smem[];
  char* tile = reinterpret_cast<char*>(smem) + (threadIdx.x >> 6) * kStageBytes;
  int i0 = max(x - off - C, 0);
  while (true) {
    const int i1 = min(e, off + len) - off - C;
    const int b = u / hkv, h = u - b * hkv;
    const int L = __builtin_amdgcn_readfirstlane(min(max(ctx_lens[b], 0), max_pages * kP));
    const uint16_t* qrow =
        q + ((int64_t)b * hkv * group + h * group + min(row, group - 1)) * kD + 8 * j;
    bf16x8 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 32 * s);
      qf[s] = as_bf16x8(gok ? w : u32x4{0u, 0u, 0u, 0u});
    }
    float m_run = -INFINITY, l_run = 0.f;
    floatx4 o[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int32_t* lp = miss_pages + (int64_t)u * max_pages;
    const int32_t* lx = miss_phys + (int64_t)u * max_pages;
    // 64 ids at a time into lanes k (read with readlane), and two units in
    // flight: the next unit's host read is issued before the current one is
    // stored and attended, so the wave keeps the link busy while it attends.
    // A miss out of range reads unit 0 of the pool (in bounds) and is
    // neither stored nor attended.
    for (int base = i0; base < i1; base += 64) {
      const int cnt = min(64, i1 - base);
      const int ie = min(base + lane, i1 - 1);
      int pl = lp[ie], xl = lx[ie];
      asm volatile("" : "+v"(pl), "+v"(xl));
      auto src = [&](int k) {
        const int p = __builtin_amdgcn_readlane(pl, k), x = __builtin_amdgcn_readlane(xl, k);
        const bool ok = p >= 0 && p < max_pages && x >= 0 && x < pool_slots;
        return host_kv + (ok ? (((int64_t)b * max_pages + p) * hkv + h) * kUnitElems : 0);
      };
      auto finish = [&](const RawUnit& r, int k) {
        const int p = __builtin_amdgcn_readlane(pl, k), x = __builtin_amdgcn_readlane(xl, k);
        if (p < 0 || p >= max_pages || x < 0 || x >= pool_slots) return;
        store_raw(r, cache_kv + (int64_t)x * kUnitElems);
        PageFrag f;
        raw_to_frag(r, tile, f);
        f.valid = max(min(kP, L - kP * p), 0);
        attend_page(f, qf, gok, j, scale_log2, m_run, l_run, o);
      };
      RawUnit ra, rb;
      load_raw(ra, src(0));
      int k = 0;
      for (; k + 2 < cnt; k += 2) {
        load_raw(rb, src(k + 1));
        finish(ra, k);
        load_raw(ra, src(k + 2));
        finish(rb, k + 1);
      }
      if (k + 1 < cnt) {
        load_raw(rb, src(k + 1));
        finish(ra, k);
        finish(rb, k + 1);
      } else {
        finish(ra, k);
      }
    }
    // the wave's partial: tokens 4j .. 4j + 3 of each page were summed in
    // lane (g, j); lane (g, j) holds channels 16 m + 4 j .. + 3 of head g
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (gok) {
      const int64_t r = ((int64_t)u + fw) * group + row;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        floatx4 v = o[m];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (l_run > 0.f) ? v[c] / l_run : 0.f;
        *reinterpret_cast<floatx4*>(part_o + r * kD + 16 * m + 4 * j) = v;
      }
      if (j == 0)
        part_lse[r] = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
    }
    if (off + len >= e) break;         // the slice ends in this unit
    off += len;
    ++u;
    len = 0;
    while (len == 0 && u < U) {
      len = plan_positions(miss_counts[u], cap);
      if (len == 0) ++u;
    }
    if (len == 0 || e - off <= C) break;
    i0 = 0;
  }
}

// The host tier's fetch with its attention, and the attention over the
// hits, in one launch.  The first nfetch workgroups are the copying waves
// (miss_worker, 4 waves each: they copy the step's placed misses into their
// slots and attend them); the others are the attention's workers over lists
// whose misses read as empty pages (hit_phys), so no worker reads a slot
// being written.  Every workgroup holds 96 KiB of LDS (dynamic, the
// attention workers use the first part of it), so a compute unit runs one
// of them at a time: a copying wave, whose host reads take microseconds,
// never shares its unit's memory pipeline with attention waves.  The copying
// workgroups come first in the grid and are placed first; attention workers
// beyond the free units start as units free up.  With nothing to copy, the
// copying waves exit after reading the miss counts.
constexpr size_t kFetchAttnLds = 96 * 1024;
// Copying workgroups: 64 of 4 waves, the 256 waves that keep the PCIe link
// busy (the copy waits on the link, not on the waves).
constexpr int kFetchAttnGroups = SPARSE_FETCH_ATTN_COPY_GROUPS;
static_assert(SPARSE_FETCH_ATTN_COPY_WAVES == kFetchAttnGroups * kAttnWaves,
              "copying waves: 4 per copying workgroup");
static_assert(kAttnWaves * kStageBytes <= kFetchAttnLds, "copying waves' LDS tiles");

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void fetch_attn_kernel(
    const uint16_t* __restrict__ host_kv, uint16_t* __restrict__ cache_kv, int64_t pool_slots,
    int nfetch, int32_t* __restrict__ step_counter, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ sel_counts,
    const int32_t* __restrict__ sel_pages, const int32_t* __restrict__ hit_phys,
    const int32_t* __restrict__ miss_counts, const int32_t* __restrict__ miss_pages,
    const int32_t* __restrict__ miss_phys, float scale_log2, int hkv, int group, int max_pages,
    int cap, int U, int wmax, float* __restrict__ part_o, float* __restrict__ part_lse,
    float* __restrict__ miss_part_o, float* __restrict__ miss_part_lse) {
  if ((int)blockIdx.x < nfetch) {
    // every resolve workgroup has read the step (the resolve ran first on
    // this stream): advance it for the next call
    if (blockIdx.x == 0 && threadIdx.x == 0) *step_counter += 1;
    miss_worker((int)blockIdx.x * kAttnWaves + (int)(threadIdx.x >> 6), nfetch * kAttnWaves,
                host_kv, cache_kv, pool_slots, q, ctx_lens, miss_counts, miss_pages, miss_phys,
                scale_log2, hkv, group, max_pages, cap, U, miss_part_o, miss_part_lse);
    return;
  }
  attn_worker((int)blockIdx.x - nfetch, q, cache_kv, kUnitElems, 0, pool_slots, ctx_lens,
              sel_counts, sel_pages, hit_phys, scale_log2, hkv, group, max_pages, cap, U, wmax,
              part_o, part_lse);
}

}  // namespace sp

extern "C" int64_t sparse_decode_max_parts(const sparse_dims* dims, int32_t workers) {
  if (sp::check_dims(dims) != SPARSE_OK || workers < 0) return -1;
  const int wmax = sp::resolve_workers(workers);
  if (wmax < 1) return -1;
  return (int64_t)dims->batch * dims->num_kv_heads + wmax;
}

namespace sp {

sparse_status check_attn(const sparse_dims* dims, const uint16_t* q, const uint16_t* kv,
                         int64_t stride_page, int64_t stride_head, int64_t pool_pages,
                         const int32_t* ctx_lens, const int32_t* sel_counts,
                         const int32_t* sel_pages, const int32_t* sel_phys, float scale,
                         int32_t workers, int& wmax) {
  sparse_status st = check_dims(dims);
  if (st != SPARSE_OK) return st;
  if ((st = check_pool(kv, stride_page, stride_head, pool_pages)) != SPARSE_OK) return st;
  if (!q || !ctx_lens || !sel_counts || !sel_pages || !sel_phys) return SPARSE_ERR_INVALID;
  if (!aligned(q, 16) || !isfinite(scale)) return SPARSE_ERR_INVALID;
  if (workers < 0 || workers > kMaxWorkers) return SPARSE_ERR_INVALID;
  if ((int64_t)dims->batch * dims->num_kv_heads * dims->max_pages > INT32_MAX)
    return SPARSE_ERR_UNSUPPORTED;
  wmax = resolve_workers(workers);
  return wmax < 1 ? SPARSE_ERR_HIP : SPARSE_OK;
}

void enqueue_attn(const sparse_dims* dims, const uint16_t* q, const uint16_t* kv,
                  int64_t stride_page, int64_t stride_head, int64_t pool_pages,
                  const int32_t* ctx_lens, const int32_t* sel_counts, const int32_t* sel_pages,
                  const int32_t* sel_phys, float scale, int wmax, float* part_o, float* part_lse,
                  hipStream_t stream) {
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  const size_t lds = sizeof(float) * (size_t)kAttnWaves * group * (kD + 2);
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)wmax), dim3(256), lds, stream, q, kv,
                     stride_page, stride_head, pool_pages, ctx_lens, sel_counts, sel_pages,
                     sel_phys, scale_log2, hkv, group, dims->max_pages, list_cap(dims), U, wmax,
                     part_o, part_lse);
}

void enqueue_fetch_attn(const sparse_dims* dims, const uint16_t* host_kv, uint16_t* cache_kv,
                        int64_t pool_slots, int32_t* step_counter, const uint16_t* q,
                        const int32_t* ctx_lens, const int32_t* sel_counts,
                        const int32_t* sel_pages, const int32_t* hit_phys,
                        const int32_t* miss_counts, const int32_t* miss_pages,
                        const int32_t* miss_phys, float scale, int wmax, float* part_o,
                        float* part_lse, float* miss_part_o, float* miss_part_lse,
                        hipStream_t stream) {
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(fetch_attn_kernel, dim3((unsigned)(kFetchAttnGroups + wmax)), dim3(256),
                     kFetchAttnLds, stream, host_kv, cache_kv, pool_slots, kFetchAttnGroups,
                     step_counter, q, ctx_lens, sel_counts, sel_pages, hit_phys, miss_counts,
                     miss_pages, miss_phys, scale_log2, hkv, group, dims->max_pages,
                     list_cap(dims), U, wmax, part_o, part_lse, miss_part_o, miss_part_lse);
}

}  // namespace sp

extern "C" sparse_status sparse_decode_attn(const sparse_dims* dims, const uint16_t* q,
                                            const uint16_t* kv, int64_t stride_page,
                                            int64_t stride_head, int64_t pool_pages,
                                            const int32_t* ctx_lens, const int32_t* sel_counts,
                                            const int32_t* sel_pages, const int32_t* sel_phys,
                                            float scale, int32_t workers, float* part_o,
                                            float* part_lse, int64_t max_parts, void* stream) {
  int wmax = 0;
  sparse_status st = sp::check_attn(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens,
                                    sel_counts, sel_pages, sel_phys, scale, workers, wmax);
  if (st != SPARSE_OK) return st;
  if (!part_o || !part_lse || !sp::aligned(part_o, 16)) return SPARSE_ERR_INVALID;
  if (max_parts != (int64_t)dims->batch * dims->num_kv_heads + wmax) return SPARSE_ERR_INVALID;
  sp::enqueue_attn(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens, sel_counts,
                   sel_pages, sel_phys, scale, wmax, part_o, part_lse, (hipStream_t)stream);
  return sp::launch_status();
}
