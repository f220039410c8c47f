// Measurement helper, not a step of the decode path: read whole 8 KiB blocks
// of a KV pool in a given order, at the rate the memory system allows.
//
// The decode attention reads each kept (page, KV head) unit as one 8 KiB
// block (K tile + V tile) at a data-dependent address.  This kernel moves the
// same blocks in the same unit with nothing else to do -- no list lookups, no
// math, no partials -- so its rate on a random block order is the practical
// ceiling the attention kernel is compared against, and its rate in address
// order is the streaming-read ceiling.  The words are XOR-folded into one
// checksum so the loads cannot be elided and the result can be checked.

#include "common.h"

namespace sp {

constexpr int kReadWaves = 4;           // waves per workgroup
constexpr int kReadDepth = 2;           // blocks in flight per wave
constexpr int kReadGroups = SPARSE_READ_BLOCKS_GROUPS;   // workgroups (16 per compute unit)
constexpr int kBlockWords = 2048;       // 32-bit words per 8 KiB block

// Wave w reads blocks order[w], order[w + W], ... (W = all waves), two at a
// time.  The two ids come in one load (lane d holds the d-th) and are
// broadcast with readlane; then the 8 16-byte loads per lane of both blocks
// are issued before either is folded.  The block loads are unconditional --
// an id outside [0, pool_blocks) reads block 0 and its words are masked to
// zero afterwards -- because a load under a per-lane condition becomes a
// branch whose wait also drains the other block's loads.  Each workgroup
// ends with one plain store of its fold: a device-scope atomic there makes
// every workgroup wait for its round trip before the next one can start,
// which costs about 12% of the rate at this grid.  In random order the rate
// varies little with the grid (6.70-6.82 TB/s over 256-4096 workgroups on a
// 2 GiB pool); 4096, the fastest, is used so the ceiling is not understated.
__global__ __launch_bounds__(256) void read_blocks_kernel(const uint32_t* __restrict__ pool,
                                                          int64_t pool_blocks,
                                                          const int32_t* __restrict__ order,
                                                          int64_t n, uint32_t* __restrict__ xor_out) {
  __shared__ uint32_t fold[kReadWaves];
  const int64_t waves = (int64_t)gridDim.x * kReadWaves;
  const int64_t w = (int64_t)blockIdx.x * kReadWaves + (threadIdx.x >> 6);
  const int lane = lane_id();
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = w; i < n; i += waves * kReadDepth) {
    const int64_t jl = i + (int64_t)(lane % kReadDepth) * waves;
    const int xl = order[jl < n ? jl : i];
    int64_t xs[kReadDepth];
    uint32_t keep[kReadDepth];
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) {
      const int x = __builtin_amdgcn_readlane(xl, d);
      const bool ok = i + d * waves < n && x >= 0 && (int64_t)x < pool_blocks;
      xs[d] = ok ? x : 0;
      keep[d] = ok ? 0xFFFFFFFFu : 0u;
    }
    u32x4 t[kReadDepth][8];
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) {
      const u32x4* src = reinterpret_cast<const u32x4*>(pool + xs[d] * kBlockWords);
#pragma unroll
      for (int k = 0; k < 8; ++k) t[d][k] = __builtin_nontemporal_load(src + k * 64 + lane);
    }
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= t[d][k] & keep[d];
  }
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v ^= (uint32_t)__shfl_xor((int)v, o, 64);
  if (lane == 0) fold[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) xor_out[blockIdx.x] = fold[0] ^ fold[1] ^ fold[2] ^ fold[3];
}

}  // namespace sp

extern "C" sparse_status sparse_read_blocks(const uint16_t* pool, int64_t pool_blocks,
                                            const int32_t* order, int64_t n, uint32_t* xor_out,
                                            void* stream) {
  if (n < 0 || pool_blocks < 0) return SPARSE_ERR_INVALID;
  if (!pool || (!order && n > 0) || !xor_out || !sp::aligned(pool, 16) ||
      !sp::aligned(xor_out, 4))
    return SPARSE_ERR_INVALID;
  if (pool_blocks == 0) n = 0;   // no block to read: the loads below must not touch the pool
  hipLaunchKernelGGL(sp::read_blocks_kernel, dim3(sp::kReadGroups), dim3(256), 0,
                     (hipStream_t)stream, reinterpret_cast<const uint32_t*>(pool), pool_blocks,
                     order, n, xor_out);
  return sp::launch_status();
}
