// Internal helpers of the gfx950 sparse paged decode library (kernels + C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

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

// ---- the chunk plan, derived on the device from the list lengths ------------
// Unit u's list of k_u = min(count_u, cap) pages (cap: the dims' list bound)
// has ceil(k_u / chunk) chunks (the attention shares the list evenly over
// them).  Chunks are numbered over every unit's first floor(k_u / chunk)
// chunks (unit order), then the last chunk of each unit that chunk does not
// divide (unit order), so the grid's last workgroups -- the ones that run
// while the rest of the chip drains -- include every unit shorter than one
// chunk.  A wave derives where chunk c falls with one round of
// loads (lane l reads the counts of units l*8 .. l*8+7 of each 512-unit
// segment) and wave prefix sums -- no host plan and no precomputed offsets.
constexpr int kPlanVU = 8;

// List lengths of units base .. base + kPlanVU - 1, clamped to [0, cap]
// (0 past the last unit).  The loads are unconditional -- an index past the
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
    k[v] = (base + v < U) ? min(max(raw[v], 0), cap) : 0;
  }
}

// Within one 512-unit segment whose lane-l units (seg + 8l ..) hold ch[v]
// chunks of this numbering pass (per-lane sum s, inclusive wave prefix incl,
// `before` chunks numbered ahead of the segment): if chunk c falls in it,
// set unit and local (wave-uniform) and return true.
__device__ __forceinline__ bool plan_find(int c, int before, int seg, const int (&ch)[kPlanVU],
                                          const int (&k)[kPlanVU], int s, int incl, bool full,
                                          int chunk, int& unit, int& local) {
  const int lane = lane_id();
  if (c >= before + __shfl(incl, 63, 64)) return false;
  const unsigned long long hit_mask = __ballot(before + incl > c);
  const int hit = __ffsll((long long)hit_mask) - 1;
  int acc = before + incl - s, fu = -1, fl = 0;
#pragma unroll
  for (int v = 0; v < kPlanVU; ++v) {
    if (fu < 0 && c < acc + ch[v]) {
      fu = seg + lane * kPlanVU + v;
      fl = full ? c - acc : k[v] / chunk;
    }
    acc += ch[v];
  }
  unit = __builtin_amdgcn_readlane(fu, hit);
  local = __builtin_amdgcn_readlane(fl, hit);
  return true;
}

// Unit of global chunk c and the chunk's index within that unit (unit = -1
// when c is past the last chunk).  Wave-uniform results; every lane calls.
__device__ __forceinline__ void plan_locate(const int32_t* __restrict__ counts, int U,
                                            int cap, int chunk, int c, int& unit,
                                            int& local) {
  const int lane = lane_id();
  unit = -1;
  local = 0;
  int k[kPlanVU], ch[kPlanVU], cp[kPlanVU];
  if (U <= 64 * kPlanVU) {
    // one segment: a single round of loads serves both numbering passes
    plan_counts8(counts, lane * kPlanVU, U, cap, k);
    int sf = 0, sp = 0;
#pragma unroll
    for (int v = 0; v < kPlanVU; ++v) {
      ch[v] = k[v] / chunk;
      cp[v] = (k[v] % chunk != 0) ? 1 : 0;
      sf += ch[v];
      sp += cp[v];
    }
    const int inf = wave_incl_scan(sf), inp = wave_incl_scan(sp);
    const int full_total = __shfl(inf, 63, 64);
    if (plan_find(c, 0, 0, ch, k, sf, inf, true, chunk, unit, local)) return;
    plan_find(c, full_total, 0, cp, k, sp, inp, false, chunk, unit, local);
    return;
  }
  // pass 0: the full chunks of every unit; pass 1: one partial chunk per
  // unit whose length chunk does not divide
  int before = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int seg = 0; seg < U; seg += 64 * kPlanVU) {
      plan_counts8(counts, seg + lane * kPlanVU, U, cap, k);
      int s = 0;
#pragma unroll
      for (int v = 0; v < kPlanVU; ++v) {
        ch[v] = pass == 0 ? k[v] / chunk : (k[v] % chunk != 0 ? 1 : 0);
        s += ch[v];
      }
      const int incl = wave_incl_scan(s);
      if (plan_find(c, before, seg, ch, k, s, incl, pass == 0, chunk, unit, local)) return;
      before += __shfl(incl, 63, 64);
    }
  }
}

// ---- host-side argument checks ----------------------------------------------
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline sparse_status check_dims(const sparse_dims* d) {
  if (!d) return SPARSE_ERR_INVALID;
  if (d->batch < 1 || d->num_kv_heads < 1 || d->num_q_heads < 1 || d->max_pages < 1)
    return SPARSE_ERR_INVALID;
  if (d->num_q_heads % d->num_kv_heads != 0) return SPARSE_ERR_INVALID;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->head_dim != kD || d->page_size != kP || G > kMaxGroup || d->max_pages > kMaxPages)
    return SPARSE_ERR_UNSUPPORTED;
  if (d->max_list_pages < 0 || d->max_list_pages > d->max_pages) return SPARSE_ERR_INVALID;
  return SPARSE_OK;
}

// The length every page list is planned for (attention and merge).
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

inline sparse_status launch_status() {
  return hipGetLastError() == hipSuccess ? SPARSE_OK : SPARSE_ERR_HIP;
}

}  // namespace sp
