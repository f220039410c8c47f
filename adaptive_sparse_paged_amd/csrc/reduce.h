// Wave-level reductions and scans on the DPP crossbar and the fixed-point
// page weight, shared by the selection kernels.
#pragma once

#include "common.h"

namespace sp {

// fixed-point weight of a page from its fp32 mass bits: floor(m * 2^52)
__device__ __forceinline__ unsigned long long weight_of(uint32_t key) {
  return (unsigned long long)(__uint_as_float(key) * 4503599627370496.0f);
}

// ---- reductions on the DPP crossbar ----------------------------------------
// A lane-shuffle through __shfl_xor is an LDS permute; sixteen waves doing
// many of them queue on the LDS.  Within a row of 16 lanes the butterfly runs
// on DPP moves instead: quad swaps (lane ^ 1, lane ^ 2), then the half-row and
// row mirrors (i <-> 7 - i, i <-> 15 - i) -- after the quad steps a mirror
// pairs every lane with the other half's total.  Each step combines a and b
// as op(a, b) in one lane and op(b, a) in its partner; the ops are
// commutative, so every lane ends with the same bits.  Across the four rows,
// four readlanes and a fixed combination order.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  return (unsigned long long)dpp_u32<CTRL>((uint32_t)v) |
         ((unsigned long long)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32);
}

struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpAdd {
  __device__ float operator()(float a, float b) const { return a + b; }
  __device__ unsigned long long operator()(unsigned long long a, unsigned long long b) const {
    return a + b;
  }
};
struct OpAddU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMinU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct OpMaxU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

// every lane of a row of 16 ends with the row's total
template <typename Op>
__device__ __forceinline__ float row16_f32(float v, Op op) {
  v = op(v, dpp_f32<kDppXor1>(v));
  v = op(v, dpp_f32<kDppXor2>(v));
  v = op(v, dpp_f32<kDppHalfMirror>(v));
  v = op(v, dpp_f32<kDppMirror>(v));
  return v;
}
template <typename Op>
__device__ __forceinline__ uint32_t row16_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<kDppXor1>(v));
  v = op(v, dpp_u32<kDppXor2>(v));
  v = op(v, dpp_u32<kDppHalfMirror>(v));
  v = op(v, dpp_u32<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ unsigned long long row16_sum_u64(unsigned long long v) {
  v += dpp_u64<kDppXor1>(v);
  v += dpp_u64<kDppXor2>(v);
  v += dpp_u64<kDppHalfMirror>(v);
  v += dpp_u64<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// the wave's total, the same value in every lane
template <typename Op>
__device__ __forceinline__ float wave_total_f32(float v, Op op) {
  v = row16_f32(v, op);
  const float r0 = __uint_as_float(lane_u32(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(lane_u32(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(lane_u32(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(lane_u32(__float_as_uint(v), 48));
  return op(op(r0, r1), op(r2, r3));
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_total_u32(uint32_t v, Op op) {
  v = row16_u32(v, op);
  return op(op(lane_u32(v, 0), lane_u32(v, 16)), op(lane_u32(v, 32), lane_u32(v, 48)));
}
__device__ __forceinline__ unsigned long long wave_total_u64(unsigned long long v) {
  v = row16_sum_u64(v);
  unsigned long long t = 0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    t += (unsigned long long)lane_u32((uint32_t)v, 16 * r) |
         ((unsigned long long)lane_u32((uint32_t)(v >> 32), 16 * r) << 32);
  return t;
}

// Inclusive prefix sums over the wave on DPP: row_shr 1, 2, 4, 8 within each
// row of 16 (a lane whose source falls outside its row adds 0), then lane 15
// of rows 0 and 2 into rows 1 and 3 (row_bcast15), then lane 31 into rows 2
// and 3 (row_bcast31).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_upd_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_upd_u64(unsigned long long v) {
  return (unsigned long long)dpp_upd_u32<CTRL, ROWS>((uint32_t)v) |
         ((unsigned long long)dpp_upd_u32<CTRL, ROWS>((uint32_t)(v >> 32)) << 32);
}
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
  x += dpp_upd_u32<0x111, 0xF>(x);
  x += dpp_upd_u32<0x112, 0xF>(x);
  x += dpp_upd_u32<0x114, 0xF>(x);
  x += dpp_upd_u32<0x118, 0xF>(x);
  x += dpp_upd_u32<0x142, 0xA>(x);
  x += dpp_upd_u32<0x143, 0xC>(x);
  return x;
}
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long x) {
  x += dpp_upd_u64<0x111, 0xF>(x);
  x += dpp_upd_u64<0x112, 0xF>(x);
  x += dpp_upd_u64<0x114, 0xF>(x);
  x += dpp_upd_u64<0x118, 0xF>(x);
  x += dpp_upd_u64<0x142, 0xA>(x);
  x += dpp_upd_u64<0x143, 0xC>(x);
  return x;
}

}  // namespace sp
