// Page scoring: the estimated attention logit of every page, per query head.
//
// u = sum_d max(q_d kmin_d, q_d kmax_d) is the Quest-style bound on q.k_t
// over the page's tokens.  Since max(q a, q b) = q+ b + q- a for a <= b
// (q+ = max(q,0), q- = min(q,0)), u is the dot product of the 256-element
// summary row [kmin | kmax] with [q- | q+]: a 16-page x 256 x G contraction
// per tile, which runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with exact bf16 products and fp32 accumulation.  logit = scale*u +
// ln(valid tokens), the log of an upper bound of the page's unnormalised
// attention mass -- the estimate the coverage rule cuts on ("Adaptive
// DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", MOIRA
// abstract, coverage-rule sentence; the estimator itself is not given there).

#include "common.h"

namespace sp {

constexpr int kScoreTilesPerWave = 2;   // 16-page tiles per wave
constexpr int kScoreWaves = 4;          // waves per workgroup
constexpr int kScorePagesPerBlock = 16 * kScoreTilesPerWave * kScoreWaves;

// MFMA 16x16x32 bf16 operand layout (wave64): lane l supplies row (l & 15) of
// A and column (l & 15) of B, k-elements 8*(l >> 4) .. +7 of the 32-wide
// k-slice; the fp32 result in lane l is column (l & 15), rows 4*(l >> 4) + i.
// Here rows = pages of the tile, columns = query heads of the group, and
// k-slice s covers summary elements [32 s, 32 s + 32) (s < 4: kmin channels,
// s >= 4: kmax channels).
//
// Grid (KV head, page block, request): the KV heads of one request and page
// block are consecutive workgroups, so the Hkv summary rows of a physical
// page (adjacent 512-byte rows, one 4 KiB run) are read close together in
// time.  A wave loads the page ids of both its tiles, then the summaries of
// tile t + 1 while the matrix cores work on tile t.
__global__ __launch_bounds__(64 * kScoreWaves) void score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ summ, int64_t pool_pages,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ ctx_lens, float scale,
    float* __restrict__ logits, int hkv, int group, int max_pages) {
  const int h = blockIdx.x, b = blockIdx.z;
  const int u = b * hkv + h;
  const int L = min(max(ctx_lens[b], 0), max_pages * kP);
  const int n = (L + kP - 1) / kP;
  const int wave = blockIdx.y * kScoreWaves + (threadIdx.x >> 6);
  const int p_begin = wave * kScoreTilesPerWave * 16;
  if (p_begin >= n) return;
  const int lane = lane_id(), row = lane & 15, j = lane >> 4;
  const int32_t* pt = page_table + (int64_t)b * max_pages;

  // Every load below is unconditional (out-of-range rows read a valid
  // address and are discarded later): a load under a per-lane condition
  // becomes a branch, and where the paths meet the compiler waits for every
  // load in flight -- which would drain tile 1's loads before tile 0's math.
  int xs[kScoreTilesPerWave];
#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t) {
    const int p = p_begin + t * 16 + row;
    const int x = pt[min(p, n - 1)];
    xs[t] = (p < n) ? x : -1;
  }

  // B operands: q- for the kmin half, q+ for the kmax half (bf16 bit masks).
  bf16x8 qneg[4], qpos[4];
  {
    const int g = row;
    const int hq = h * group + min(g, group - 1);
    const uint32_t gmask = (g < group) ? 0xFFFFFFFFu : 0u;    // padding columns are zero
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * hkv * group + hq) * kD + 32 * s +
                                                8 * j);
      w &= gmask;
      u32x4 neg, pos;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // per 16-bit half: all-ones where the sign bit is set
        const uint32_t sgn = (w[e] >> 15) & 0x00010001u;
        const uint32_t m = sgn * 0xFFFFu;
        neg[e] = w[e] & m;
        pos[e] = w[e] & ~m;
      }
      qneg[s] = as_bf16x8(neg);
      qpos[s] = as_bf16x8(pos);
    }
  }

  const float ln16 = 2.772588722239781f;
  float* out = logits + (int64_t)u * group * max_pages;
  const bool vec_ok = (max_pages & 3) == 0 && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  u32x4 a[2][8];
  bool oks[2];
  // A row whose page is out of range reads page 0's summary (always in
  // bounds); MFMA rows are independent and that row's logit is written as
  // -inf, so the values it read never matter.
  auto issue = [&](int t, int slot) {
    const int x = xs[t];
    const bool ok = (x >= 0) && (x < pool_pages);
    oks[slot] = ok;
    const uint16_t* src = summ + ((int64_t)(ok ? x : 0) * hkv + h) * (2 * kD) + 8 * j;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[slot][s] = *reinterpret_cast<const u32x4*>(src + 32 * s);
  };
  issue(0, 0);
#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t) {
    const int p0 = p_begin + t * 16;
    if (p0 >= n) break;
    if (t + 1 < kScoreTilesPerWave) issue(t + 1, (t + 1) & 1);
    const int slot = t & 1;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[slot][s]), qneg[s], acc, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[slot][4 + s]), qpos[s], acc, 0, 0,
                                                    0);
    // Which of the tile's pages are in range: lane r < 16 holds page r's
    // flag, and a ballot hands it to every lane without an LDS permute.
    const unsigned long long okm = __ballot(oks[slot]);
    // lane (g = row, j) now holds u for pages p0 + 4j + i: one 16-byte store
    // of its 4 consecutive pages when they are all in range and aligned
    float val[4];
    bool okv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pi = p0 + 4 * j + i;
      okv[i] = (okm >> (4 * j + i)) & 1ull;
      const int nv = min(kP, L - kP * pi);
      const float lnv = (nv >= kP) ? ln16 : logf((float)max(nv, 1));
      val[i] = okv[i] ? fmaf(scale, acc[i], lnv) : -INFINITY;
    }
    if (row < group) {
      const int pq = p0 + 4 * j;
      if (vec_ok && pq + 4 <= n) {
        *reinterpret_cast<floatx4*>(out + (int64_t)row * max_pages + pq) =
            floatx4{val[0], val[1], val[2], val[3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (pq + i < n) out[(int64_t)row * max_pages + pq + i] = val[i];
      }
    }
  }
}

}  // namespace sp

extern "C" sparse_status sparse_score_pages(const sparse_dims* dims, const uint16_t* q,
                                            const uint16_t* summ, int64_t pool_pages,
                                            const int32_t* page_table, const int32_t* ctx_lens,
                                            float scale, float* logits, void* stream) {
  sparse_status st = sp::check_dims(dims);
  if (st != SPARSE_OK) return st;
  if (!q || !summ || !page_table || !ctx_lens || !logits || pool_pages < 1)
    return SPARSE_ERR_INVALID;
  if (!sp::aligned(q, 16) || !sp::aligned(summ, 16) || !isfinite(scale))
    return SPARSE_ERR_INVALID;
  const int hkv = dims->num_kv_heads, group = dims->num_q_heads / hkv;
  const int U = dims->batch * hkv;
  dim3 grid(hkv, (dims->max_pages + sp::kScorePagesPerBlock - 1) / sp::kScorePagesPerBlock,
            dims->batch);
  if (U < 1 || grid.z > 65535) return SPARSE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(sp::score_kernel, grid, dim3(64 * sp::kScoreWaves), 0, (hipStream_t)stream, q, summ,
                     pool_pages, page_table, ctx_lens, scale, logits, hkv, group,
                     dims->max_pages);
  return sp::launch_status();
}
