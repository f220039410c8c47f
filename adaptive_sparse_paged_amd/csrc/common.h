// Internal helpers of the gfx950 sparse paged decode library (kernels + C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/sparse_paged.h"

namespace sp {

constexpr int kD = 128;            // head_dim
constexpr int kP = 16;             // tokens per page
constexpr int kTile = kP * kD;     // elements of one K (or V) tile
constexpr int kMaxGroup = 16;      // query heads per KV head
constexpr int kMaxPages = 32768;   // page-table row length limit

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ short4v as_short4(u32x2 v) { return __builtin_bit_cast(short4v, v); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---- wave (64-lane) reductions / scans -------------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64,
// at most 4096).  `scratch` holds NT/64 elements.  Returns the exclusive
// prefix of `v`; `total` receives the block total.  Contains barriers: every
// thread of the block must call it.
template <typename T, int NT>
__device__ __forceinline__ T block_excl_scan(T v, T* scratch, T& total) {
  constexpr int NW = NT / 64;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  T incl = wave_incl_scan(v);
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  if (w == 0) {
    T s = (lane < NW) ? scratch[lane] : T(0);
    s = wave_incl_scan(s);
    if (lane < NW) scratch[lane] = s;
  }
  __syncthreads();
  T base = (w > 0) ? scratch[w - 1] : T(0);
  total = scratch[NW - 1];
  __syncthreads();
  return base + incl - v;
}

template <typename T, int NT>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
  T total;
  block_excl_scan<T, NT>(v, scratch, total);
  return total;
}

// ---- the balanced plan, derived on the device from the list lengths -------
// Every unit with a nonempty list (k_u = min(count_u, cap) entries, cap the
// dims' list bound) takes c = kPlanUnitCost + k_u positions: c positions that
// stand for the fixed cost of starting a unit's segment, then its entries.
// The units are laid end to end in unit order: entry e of unit u sits at
// global position off_u + c + e, off_u the sum of the positions of the units
// before it; T is the total.  W workers share the positions evenly: worker w
// owns [floor(w T / W), floor((w + 1) T / W)), crossing unit boundaries where
// they fall, and writes one partial per unit whose entries its range meets,
// in slot u + w (unit and worker indices both grow along the positions, so
// the slots of distinct (unit, worker) pairs differ and every slot is below
// U + W).  A worker whose range crosses into a unit therefore gets c fewer
// entries for the segment it starts there.  W is the grid size the caller
// gave, cut to ceil(T / kMinWorkerPages) so short steps do not spread a few
// pages over hundreds of workgroups; every worker's range is then at least
// 16 positions, more than c, so its first unit always gives it entries.
// Everything here is computed by each wave from sel_counts alone: no host
// plan and no precomputed offsets.  The functions below work in positions;
// the attention and the merge turn them into entries.
constexpr int kPlanVU = 8;                  // units per lane in one scan segment
constexpr int kPlanSeg = 64 * kPlanVU;      // units per scan segment
constexpr int kMinWorkerPages = SPARSE_ATTN_MIN_WORKER_PAGES;
constexpr int kPlanUnitCost = SPARSE_ATTN_UNIT_COST_PAGES;
static_assert(kPlanUnitCost < kMinWorkerPages / 2, "a worker's first unit must give it entries");

// Positions a unit of `raw` list entries takes in the plan.
__device__ __forceinline__ int plan_positions(int raw, int cap) {
  const int k = min(max(raw, 0), cap);
  return k > 0 ? k + kPlanUnitCost : 0;
}

// Plan positions of units base .. base + kPlanVU - 1 (0 past the last unit).  The loads are unconditional -- an index past the
// last unit re-reads unit U-1 -- and all are issued before any is used.  The
// empty asm statement pins each loaded value in a register; without it the
// compiler moves each load under the `idx < U` test, and a load under a
// per-lane condition becomes a branch that waits for it: 8 round trips
// instead of one.
__device__ __forceinline__ void plan_counts8(const int32_t* __restrict__ counts, int base, int U,
                                             int cap, int (&k)[kPlanVU]) {
  int raw[kPlanVU];
#pragma unroll
  for (int v = 0; v < kPlanVU; ++v) raw[v] = counts[min(base + v, U - 1)];
#pragma unroll
  for (int v = 0; v < kPlanVU; ++v) {
    asm volatile("" : "+v"(raw[v]));
    k[v] = (base + v < U) ? plan_positions(raw[v], cap) : 0;
  }
}

// One scan segment of units seg .. seg + kPlanSeg - 1 held by a wave: lane l
// has the lengths of units seg + 8l .. seg + 8l + 7, their sum s and the
// inclusive wave prefix incl of s; total is the segment's sum (wave-uniform).
struct PlanSeg {
  int k[kPlanVU];
  int s, incl, total;
};

__device__ __forceinline__ void plan_load(PlanSeg& P, const int32_t* __restrict__ counts,
                                          int seg, int U, int cap) {
  plan_counts8(counts, seg + lane_id() * kPlanVU, U, cap, P.k);
  int s = 0;
#pragma unroll
  for (int v = 0; v < kPlanVU; ++v) s += P.k[v];
  P.s = s;
  P.incl = wave_incl_scan(s);
  P.total = __shfl(P.incl, 63, 64);
}

// If global position x falls in segment P (which starts at global position
// `before`), set the unit holding it, that unit's first position and its
// length (wave-uniform) and return true.
__device__ __forceinline__ bool plan_seg_find(const PlanSeg& P, int seg, int before, int x,
                                              int& unit, int& off, int& len) {
  if (x >= before + P.total) return false;
  const unsigned long long hit_mask = __ballot(before + P.incl > x);
  const int hit = __ffsll((long long)hit_mask) - 1;
  int acc = before + P.incl - P.s, fu = -1, fo = 0, fl = 0;
#pragma unroll
  for (int v = 0; v < kPlanVU; ++v) {
    if (fu < 0 && x < acc + P.k[v]) {
      fu = seg + lane_id() * kPlanVU + v;
      fo = acc;
      fl = P.k[v];
    }
    acc += P.k[v];
  }
  unit = __builtin_amdgcn_readlane(fu, hit);
  off = __builtin_amdgcn_readlane(fo, hit);
  len = __builtin_amdgcn_readlane(fl, hit);
  return true;
}

// T, the step's total positions.  `first` receives segment 0 (units
// 0 .. 511), which is all of them when U <= 512.
__device__ __forceinline__ int plan_total(const int32_t* __restrict__ counts, int U, int cap,
                                          PlanSeg& first) {
  plan_load(first, counts, 0, U, cap);
  int total = first.total;
  for (int seg = kPlanSeg; seg < U; seg += kPlanSeg) {
    PlanSeg P;
    plan_load(P, counts, seg, U, cap);
    total += P.total;
  }
  return total;
}

// The unit holding global position x < T (with its first position and
// length).  Segment 0 comes from registers; later segments are reloaded.
__device__ __forceinline__ void plan_find(const int32_t* __restrict__ counts, int U, int cap,
                                          const PlanSeg& first, int x, int& unit, int& off,
                                          int& len) {
  unit = -1;
  off = len = 0;
  if (plan_seg_find(first, 0, 0, x, unit, off, len)) return;
  int before = first.total;
  for (int seg = kPlanSeg; seg < U; seg += kPlanSeg) {
    PlanSeg P;
    plan_load(P, counts, seg, U, cap);
    if (plan_seg_find(P, seg, before, x, unit, off, len)) return;
    before += P.total;
  }
}

// Unit u's first global position, its positions and T (wave-uniform).
__device__ __forceinline__ void plan_unit(const int32_t* __restrict__ counts, int U, int cap,
                                          int u, int& off, int& len, int& total) {
  total = 0;
  off = len = 0;
  for (int seg = 0; seg < U; seg += kPlanSeg) {
    PlanSeg P;
    plan_load(P, counts, seg, U, cap);
    if (u >= seg && u < seg + kPlanSeg) {
      const int l = (u - seg) / kPlanVU, v = (u - seg) % kPlanVU;
      int pre = P.incl - P.s, mine = 0;
#pragma unroll
      for (int i = 0; i < kPlanVU; ++i) {
        pre += (i < v) ? P.k[i] : 0;
        mine = (i == v) ? P.k[i] : mine;
      }
      off = total + __builtin_amdgcn_readlane(pre, l);
      len = __builtin_amdgcn_readlane(mine, l);
    }
    total += P.total;
  }
}

// Workers the plan uses for T positions with a grid of wmax workgroups.
__device__ __forceinline__ int plan_workers(int total, int wmax) {
  if (total <= 0) return 0;
  return min(wmax, (total + kMinWorkerPages - 1) / kMinWorkerPages);
}

// First position owned by worker w (of W over T positions).
__device__ __forceinline__ int plan_start(int w, int W, int total) {
  return (int)(((int64_t)w * total) / W);
}

// The worker that owns position x (the largest w with plan_start(w) <= x).
__device__ __forceinline__ int plan_owner(int x, int W, int total) {
  return (int)((((int64_t)x + 1) * W - 1) / total);
}

// ---- host-side argument checks ----------------------------------------------
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline sparse_status check_dims(const sparse_dims* d) {
  if (!d) return SPARSE_ERR_INVALID;
  if (d->batch < 1 || d->num_kv_heads < 1 || d->num_q_heads < 1 || d->max_pages < 1)
    return SPARSE_ERR_INVALID;
  if (d->num_q_heads % d->num_kv_heads != 0) return SPARSE_ERR_INVALID;
  const int G = d->num_q_heads / d->num_kv_heads;
  // G in {1, 2, 4, 8, 16}: the kernels' head loops and row layouts assume a
  // power of two
  if (d->head_dim != kD || d->page_size != kP || G > kMaxGroup || (G & (G - 1)) != 0 ||
      d->max_pages > kMaxPages)
    return SPARSE_ERR_UNSUPPORTED;
  if (d->max_list_pages < 0 || d->max_list_pages > d->max_pages) return SPARSE_ERR_INVALID;
  return SPARSE_OK;
}

// The length every page list is clamped to (attention and merge).
inline int list_cap(const sparse_dims* d) {
  return d->max_list_pages > 0 ? d->max_list_pages : d->max_pages;
}

inline sparse_status check_pool(const void* kv, int64_t stride_page, int64_t stride_head,
                                int64_t pool_pages) {
  if (!kv || pool_pages < 1 || stride_page < 0 || stride_head < 0) return SPARSE_ERR_INVALID;
  if (!aligned(kv, 16) || (stride_page % 8) != 0 || (stride_head % 8) != 0)
    return SPARSE_ERR_INVALID;
  return SPARSE_OK;
}

// Attention workgroups for a caller's `workers`: itself when positive, else
// one per compute unit of the current device (queried once per device).
// Returns -1 when the device cannot be queried.
constexpr int kMaxWorkers = 1 << 20;
inline int resolve_workers(int workers) {
  if (workers > 0) return workers;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  static std::atomic<int> cus[64];
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n < 1) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      return -1;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Shared by the attention entry points (attn.hip, attn_merge.hip): host-side
// checks of the attention's arguments (sets wmax, the resolved grid), and the
// attention and merge launches without checks.
sparse_status check_attn(const sparse_dims* dims, const uint16_t* q, const uint16_t* kv,
                         int64_t stride_page, int64_t stride_head, int64_t pool_pages,
                         const int32_t* ctx_lens, const int32_t* sel_counts,
                         const int32_t* sel_pages, const int32_t* sel_phys, float scale,
                         int32_t workers, int& wmax);
void enqueue_attn(const sparse_dims* dims, const uint16_t* q, const uint16_t* kv,
                  int64_t stride_page, int64_t stride_head, int64_t pool_pages,
                  const int32_t* ctx_lens, const int32_t* sel_counts, const int32_t* sel_pages,
                  const int32_t* sel_phys, float scale, int wmax, float* part_o, float* part_lse,
                  hipStream_t stream);
void enqueue_merge(const sparse_dims* dims, const float* part_o, const float* part_lse,
                   const int32_t* sel_counts, int wmax, float* out, float* out_lse,
                   hipStream_t stream);

inline sparse_status launch_status() {
  return hipGetLastError() == hipSuccess ? SPARSE_OK : SPARSE_ERR_HIP;
}

}  // namespace sp
