// Log-sum-exp merge of the per-segment attention partials of every unit:
//   lse = ln sum_c exp(lse_c),  o = sum_c exp(lse_c - lse) o_c,
// the identity that makes splitting a page list over several workgroups exact.

#include "common.h"

namespace sp {

constexpr int kMergeThreads = 256;
constexpr int kMergeSlots = kMergeThreads / 32;   // segments read side by side

// Merge segments of a unit under one plan: slot c0 + i for i < nseg.
struct MergeRun {
  int64_t c0;
  int nseg;
};

__device__ __forceinline__ MergeRun merge_run(const int32_t* __restrict__ sel_counts, int U,
                                              int cap, int wmax, int u) {
  int off, len, total;
  plan_unit(sel_counts, U, cap, u, off, len, total);
  off = __builtin_amdgcn_readfirstlane(off);
  len = __builtin_amdgcn_readfirstlane(len);
  total = __builtin_amdgcn_readfirstlane(total);
  int w_lo = 0, nseg = 0;
  if (len > 0) {                 // its entries: positions off + C .. off + len - 1
    const int W = plan_workers(total, wmax);
    w_lo = plan_owner(off + kPlanUnitCost, W, total);
    nseg = plan_owner(off + len - 1, W, total) - w_lo + 1;
  }
  return MergeRun{(int64_t)u + w_lo, nseg};   // segment i of the unit is slot c0 + i
}

// One 256-thread workgroup per (unit, query head).  The unit's partials are
// those of the workers its list entries fall to under the balanced plan: the
// slots u + w for w from the owner of its first entry's position to the owner
// of its last, found from the list lengths alone (one round of loads of the
// lengths, then one of the partials).  Thread t reads channel quad t % 32 of
// segments t / 32, t / 32 + 8, ... (each segment's 128 floats are one
// coalesced 512-byte read by 32 threads), keeping an online (max, sum,
// weighted sum); the 8 segment slots are then combined through LDS.  With
// kPair, the unit's segments under a second plan (lists sel_counts_b,
// partials part_o_b / part_lse_b, wmax_b workers) follow its segments under
// the first: attention over the union of two disjoint lists.
template <bool kPair>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ sel_counts, const float* __restrict__ part_o_b,
    const float* __restrict__ part_lse_b, const int32_t* __restrict__ sel_counts_b, int cap,
    int U, int wmax, int wmax_b, int hkv, int group, float* __restrict__ out,
    float* __restrict__ out_lse) {
  __shared__ floatx4 s_acc[kMergeSlots][32];
  __shared__ float s_m[kMergeSlots], s_s[kMergeSlots];
  const int u = blockIdx.x, g = blockIdx.y;
  const int b = u / hkv, h = u - (u / hkv) * hkv;
  const int slot = threadIdx.x >> 5, quad = threadIdx.x & 31;
  const MergeRun ra = merge_run(sel_counts, U, cap, wmax, u);
  MergeRun rb{0, 0};
  if (kPair) rb = merge_run(sel_counts_b, U, cap, wmax_b, u);
  const int nall = ra.nseg + rb.nseg;

  float m = -INFINITY, s = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = slot; i < nall; i += 2 * kMergeSlots) {
    // Both slots' loads are issued before any is used; an index past the
    // unit's segments is clamped to its last one (read, then discarded).  The
    // empty asm statements keep the compiler from moving a load under a test,
    // where it would become a branch that waits for it.
    const int i1 = i + kMergeSlots;
    const int j1 = min(i1, nall - 1);
    const bool b0 = kPair && i >= ra.nseg, b1 = kPair && j1 >= ra.nseg;
    const int64_t r0 = (b0 ? rb.c0 + (i - ra.nseg) : ra.c0 + i) * group + g;
    const int64_t r1 = (b1 ? rb.c0 + (j1 - ra.nseg) : ra.c0 + j1) * group + g;
    float l0 = (b0 ? part_lse_b : part_lse)[r0], l1 = (b1 ? part_lse_b : part_lse)[r1];
    floatx4 o0 = *reinterpret_cast<const floatx4*>((b0 ? part_o_b : part_o) + r0 * kD + 4 * quad);
    floatx4 o1 = *reinterpret_cast<const floatx4*>((b1 ? part_o_b : part_o) + r1 * kD + 4 * quad);
    asm volatile("" : "+v"(l0), "+v"(l1), "+v"(o0), "+v"(o1));
    if (i1 >= nall) l1 = -INFINITY;
    const float mn = fmaxf(m, fmaxf(l0, l1));
    if (mn == -INFINITY) continue;
    const float a = (m == -INFINITY) ? 0.f : __expf(m - mn);
    const float w0 = (l0 == -INFINITY) ? 0.f : __expf(l0 - mn);
    const float w1 = (l1 == -INFINITY) ? 0.f : __expf(l1 - mn);
    // a discarded slot's floats are never read as weights: w1 = 0 and its
    // values may be anything, so they are selected away, not multiplied
    acc = acc * a + o0 * w0 + ((l1 == -INFINITY) ? floatx4{0.f, 0.f, 0.f, 0.f} : o1 * w1);
    s = s * a + w0 + w1;
    m = mn;
  }
  s_acc[slot][quad] = acc;
  if (quad == 0) {
    s_m[slot] = m;
    s_s[slot] = s;
  }
  __syncthreads();
  if (slot != 0) return;
  float M = -INFINITY;
#pragma unroll 8
  for (int k = 0; k < kMergeSlots; ++k) M = fmaxf(M, s_m[k]);
  floatx4 tot = {0.f, 0.f, 0.f, 0.f};
  float S = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int k = 0; k < kMergeSlots; ++k) {
      if (s_m[k] == -INFINITY) continue;
      const float a = __expf(s_m[k] - M);
      tot += s_acc[k][quad] * a;
      S += s_s[k] * a;
    }
  }
  const int64_t row = (int64_t)b * hkv * group + h * group + g;
  const float inv = (S > 0.f) ? 1.f / S : 0.f;
  *reinterpret_cast<floatx4*>(out + row * kD + 4 * quad) = tot * inv;
  if (quad == 0) out_lse[row] = (S > 0.f) ? M + __logf(S) : -INFINITY;
}

}  // namespace sp

namespace sp {

void enqueue_merge(const sparse_dims* dims, const float* part_o, const float* part_lse,
                   const int32_t* sel_counts, int wmax, float* out, float* out_lse,
                   hipStream_t stream) {
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  hipLaunchKernelGGL(merge_kernel<false>, dim3(U, group), dim3(kMergeThreads), 0, stream, part_o,
                     part_lse, sel_counts, nullptr, nullptr, nullptr, list_cap(dims), U, wmax,
                     0, hkv, group, out, out_lse);
}

}  // namespace sp

namespace {

sparse_status check_merge(const sparse_dims* dims, const float* part_o, const float* part_lse,
                          const int32_t* sel_counts, int32_t workers, const float* out,
                          const float* out_lse, int& wmax) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!part_o || !part_lse || !sel_counts || !out || !out_lse)
    return SPARSE_ERR_INVALID;
  if (!sp::aligned(part_o, 16) || !sp::aligned(out, 16)) return SPARSE_ERR_INVALID;
  if (workers < 0 || workers > sp::kMaxWorkers) return SPARSE_ERR_INVALID;
  wmax = sp::resolve_workers(workers);
  return wmax < 1 ? SPARSE_ERR_HIP : SPARSE_OK;
}

}  // namespace

extern "C" sparse_status sparse_merge_splits(const sparse_dims* dims, const float* part_o,
                                             const float* part_lse, const int32_t* sel_counts,
                                             int32_t workers, float* out, float* out_lse,
                                             void* stream) {
  int wmax = 0;
  const sparse_status st =
      check_merge(dims, part_o, part_lse, sel_counts, workers, out, out_lse, wmax);
  if (st != SPARSE_OK) return st;
  sp::enqueue_merge(dims, part_o, part_lse, sel_counts, wmax, out, out_lse, (hipStream_t)stream);
  return sp::launch_status();
}

extern "C" sparse_status sparse_merge_splits_pair(
    const sparse_dims* dims, const float* part_o_a, const float* part_lse_a,
    const int32_t* sel_counts_a, int32_t workers_a, const float* part_o_b,
    const float* part_lse_b, const int32_t* sel_counts_b, int32_t workers_b, float* out,
    float* out_lse, void* stream) {
  int wmax_a = 0, wmax_b = 0;
  sparse_status st =
      check_merge(dims, part_o_a, part_lse_a, sel_counts_a, workers_a, out, out_lse, wmax_a);
  if (st != SPARSE_OK) return st;
  st = check_merge(dims, part_o_b, part_lse_b, sel_counts_b, workers_b, out, out_lse, wmax_b);
  if (st != SPARSE_OK) return st;
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  hipLaunchKernelGGL(sp::merge_kernel<true>, dim3(U, group), dim3(sp::kMergeThreads), 0,
                     (hipStream_t)stream, part_o_a, part_lse_a, sel_counts_a, part_o_b,
                     part_lse_b, sel_counts_b, sp::list_cap(dims), U, wmax_a, wmax_b, hkv, group,
                     out, out_lse);
  return sp::launch_status();
}

namespace sp {

// Two attention results over disjoint token sets, combined by the same
// identity: one 128-thread workgroup per (request, query head) row.
__global__ __launch_bounds__(kD) void lse_combine_kernel(
    const float* __restrict__ out_a, const float* __restrict__ lse_a,
    const float* __restrict__ out_b, const float* __restrict__ lse_b, float* __restrict__ out,
    float* __restrict__ out_lse) {
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float la = lse_a[row], lb = lse_b[row];
  const float m = fmaxf(la, lb);
  float o = 0.f, l = -INFINITY;
  if (m != -INFINITY) {
    const float wa = (la == -INFINITY) ? 0.f : __expf(la - m);
    const float wb = (lb == -INFINITY) ? 0.f : __expf(lb - m);
    const float s = wa + wb;
    o = (wa * out_a[row * kD + d] + wb * out_b[row * kD + d]) / s;
    l = m + __logf(s);
  }
  out[row * kD + d] = o;
  if (d == 0) out_lse[row] = l;
}

}  // namespace sp

extern "C" sparse_status sparse_lse_combine(const sparse_dims* dims, const float* out_a,
                                            const float* lse_a, const float* out_b,
                                            const float* lse_b, float* out, float* out_lse,
                                            void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!out_a || !lse_a || !out_b || !lse_b || !out || !out_lse) return SPARSE_ERR_INVALID;
  if (out_lse == lse_a || out_lse == lse_b) return SPARSE_ERR_INVALID;
  const int rows = dims->batch * dims->num_q_heads;
  hipLaunchKernelGGL(sp::lse_combine_kernel, dim3(rows), dim3(sp::kD), 0, (hipStream_t)stream,
                     out_a, lse_a, out_b, lse_b, out, out_lse);
  return sp::launch_status();
}
