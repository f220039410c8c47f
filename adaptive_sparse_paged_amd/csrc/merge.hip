// Log-sum-exp merge of the per-chunk attention partials of every unit:
//   lse = ln sum_c exp(lse_c),  o = sum_c exp(lse_c - lse) o_c,
// the identity that makes splitting a page list over several workgroups exact.

#include "common.h"

namespace sp {

// One 256-thread workgroup per unit.  Wave w computes (max, sum of exp) of the
// chunk lse values of heads g = w, w + 4, ...; then every thread accumulates
// its (head, channel) outputs over the unit's chunks.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    const int32_t* __restrict__ chunk_offsets,
                                                    int hkv, int group, float* __restrict__ out,
                                                    float* __restrict__ out_lse) {
  __shared__ float s_max[kMaxGroup], s_inv[kMaxGroup];
  const int u = blockIdx.x;
  const int b = u / hkv, h = u - (u / hkv) * hkv;
  const int c0 = chunk_offsets[u], c1 = chunk_offsets[u + 1];
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  for (int g = wv; g < group; g += 4) {
    float mx = -INFINITY;
    for (int c = c0 + lane; c < c1; c += 64) mx = fmaxf(mx, part_lse[(int64_t)c * group + g]);
    mx = wave_max(mx);
    float s = 0.f;
    if (mx != -INFINITY)
      for (int c = c0 + lane; c < c1; c += 64) {
        const float l = part_lse[(int64_t)c * group + g];
        if (l != -INFINITY) s += __expf(l - mx);
      }
    s = wave_sum(s);
    if (lane == 0) {
      s_max[g] = mx;
      s_inv[g] = (s > 0.f) ? 1.f / s : 0.f;
      out_lse[(int64_t)b * hkv * group + h * group + g] = (s > 0.f) ? mx + __logf(s) : -INFINITY;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < group * kD; idx += 256) {
    const int g = idx / kD, d = idx - (idx / kD) * kD;
    const float mx = s_max[g], inv = s_inv[g];
    float acc = 0.f;
    if (mx != -INFINITY)
      for (int c = c0; c < c1; ++c) {
        const float l = part_lse[(int64_t)c * group + g];
        if (l != -INFINITY) acc += __expf(l - mx) * part_o[((int64_t)c * group + g) * kD + d];
      }
    out[((int64_t)b * hkv * group + h * group + g) * kD + d] = acc * inv;
  }
}

}  // namespace sp

extern "C" sparse_status sparse_merge_splits(const sparse_dims* dims, const float* part_o,
                                             const float* part_lse, const int32_t* sel_counts,
                                             const int32_t* chunk_offsets, int32_t chunk_pages,
                                             float* out, float* out_lse, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!part_o || !part_lse || !sel_counts || !chunk_offsets || !out || !out_lse)
    return SPARSE_ERR_INVALID;
  if (chunk_pages < 1 || chunk_pages > dims->max_pages) return SPARSE_ERR_INVALID;
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  hipLaunchKernelGGL(sp::merge_kernel, dim3(U), dim3(256), 0, (hipStream_t)stream, part_o,
                     part_lse, chunk_offsets, hkv, group, out, out_lse);
  return sp::launch_status();
}
