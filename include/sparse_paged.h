/*
 * sparse_paged.h -- C ABI of the MI355X (gfx950) sparse paged decode step.
 *
 * One decode step, per (request, KV head) "unit": score every KV page of the
 * request with a cheap upper bound of its attention mass, keep the fewest
 * pages holding at least gamma of the estimated mass, then run exact
 * attention for the unit's GQA group over that variable-length page list.
 * The attention's workgroups each take an even share of all the step's list
 * entries, found on the device from the prefix-summed list lengths, and the
 * per-segment partials are merged by log-sum-exp.
 *
 * Pages cited:
 *   [P1] "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
 *        Hierarchy" (thelatestinai.com/papers/2610.13708), MOIRA abstract.
 *   [P2] "HiSparse: Scaling Sparse Attention Decoding with Hierarchical KV
 *        Cache" (scholarbro.com/p/47450), abstract.
 *   [P3] "Unifying Sparse Attention with Hierarchical Memory for Scalable
 *        Long-Context LLM Serving" (thelatestinai.com/papers/2604.26837),
 *        the SPIN abstract.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *   buffer; the library never allocates, frees or synchronises, and every
 *   call only enqueues kernels on `stream` (a hipStream_t, or NULL for the
 *   default stream).  Any sequence of calls can therefore be captured into
 *   one HIP graph.
 * - Errors: a nonzero sparse_status comes only from synchronous host-side
 *   argument checks (or a failed launch).  On a nonzero return nothing was
 *   enqueued and no output was touched.  Device-resident values (context
 *   lengths, page ids) cannot be checked on the host; page ids outside
 *   [0, pool_pages) are treated as empty pages by every kernel (never read).
 * - Supported shapes: head_dim D = 128, page_size P = 16, GQA group
 *   G = num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}, max_pages <= 32768.
 *   Other shapes return SPARSE_ERR_UNSUPPORTED.
 * - bf16 values are passed as uint16_t bit patterns.
 * - Query head j = h * G + g belongs to KV head h.  Unit u = b * Hkv + h.
 * - Request b has ctx_lens[b] = L_b tokens in n_b = ceil(L_b / 16) logical
 *   pages; logical page p holds tokens [16p, min(16p + 16, L_b)).
 *   page_table[b][p] is the physical page id of logical page p.
 *
 * KV pool layout (one layer)
 * --------------------------
 * The K tile of (physical page x, KV head h) starts at element
 *   kv + x * stride_page + h * stride_head
 * and is token-major [16][128] bf16 (4 KiB).  The V tile follows it
 * immediately (element offset +2048) and is CHANNEL-major [128][16] bf16
 * (V transposed within the page), so that the products over tokens read
 * contiguous token runs.  The canonical pool is [Ppool][Hkv][2][2048] with
 * stride_head = 4096 and stride_page = Hkv * 4096.
 */
#ifndef SPARSE_PAGED_H
#define SPARSE_PAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARSE_OK = 0,
  SPARSE_ERR_INVALID = 1,     /* null pointer, bad size, gamma outside (0,1] */
  SPARSE_ERR_UNSUPPORTED = 2, /* shape outside the supported set above */
  SPARSE_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  SPARSE_ERR_HIP = 4          /* a kernel launch failed */
} sparse_status;

typedef struct {
  int32_t batch;        /* B: requests */
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv; Hq must be a multiple of it */
  int32_t head_dim;     /* D: 128 */
  int32_t page_size;    /* P: 16 */
  int32_t max_pages;    /* row length of page_table and of the page lists */
  int32_t max_list_pages; /* 0, or a bound 1..max_pages on every page list's
                             length: the attention and merge clamp each
                             list's count to it (entries past it are not
                             attended); 0 means max_pages */
} sparse_dims;

/* Library version string (host, static storage). */
const char* sparse_version(void);

/* Human-readable name of a status code (host, static storage). */
const char* sparse_status_string(int32_t status);

/*
 * sparse_build_page_summaries -- per-page, per-channel key summaries.
 *
 * For i < n, page x = pages[i] and every KV head h, writes
 *   summ[x][h][0][d] = min over the first valid[i] tokens t of K[t][d]
 *   summ[x][h][1][d] = max over the same tokens
 * (bf16, bit-exact; -0 orders below +0; NaN inputs are unsupported).
 * This is the Quest-style page summary ([P2], abstract, the evaluated
 * sparse-attention families include Quest); [P1] names no estimator.
 * valid[i] is clamped to [0, 16]; pages with 0 valid tokens are skipped.
 * Runs at prefill / append time, outside the decode step.
 *
 *   kv        bf16 KV pool (layout above), read only
 *   pages     int32 [n] physical page ids, each in [0, pool_pages)
 *   valid     int32 [n] valid tokens of each listed page
 *   summ      bf16 [pool_pages][Hkv][2][128], written for the listed pages
 */
sparse_status sparse_build_page_summaries(const sparse_dims* dims, const uint16_t* kv,
                                          int64_t stride_page, int64_t stride_head,
                                          int64_t pool_pages, const int32_t* pages,
                                          const int32_t* valid, int32_t n, uint16_t* summ,
                                          void* stream);

/*
 * sparse_score_pages -- estimated attention logit of every page, per query head.
 *
 * For every unit (b, h), query head g of its group and logical page
 * p < n_b, with x = page_table[b][p]:
 *   u = sum_d max(q[b][hG+g][d] * kmin[x][h][d], q[b][hG+g][d] * kmax[x][h][d])
 *   logits[b][h][g][p] = scale * u + ln(valid tokens of page p)
 * n_valid * exp(scale * u) bounds the page's unnormalised attention mass;
 * this is the estimate behind the coverage rule ([P1], abstract, sentence on
 * the coverage rule; the pages leave the estimator open).  Entries with
 * p >= n_b are not written.  fp32 accumulation.
 *
 *   q          bf16 [B][Hq][128]
 *   summ       bf16 [pool_pages][Hkv][2][128] (from sparse_build_page_summaries)
 *   page_table int32 [B][max_pages]
 *   ctx_lens   int32 [B], 0 <= L_b <= 16 * max_pages
 *   logits     fp32 [B][Hkv][G][max_pages]
 */
sparse_status sparse_score_pages(const sparse_dims* dims, const uint16_t* q, const uint16_t* summ,
                                 int64_t pool_pages, const int32_t* page_table,
                                 const int32_t* ctx_lens, float scale, float* logits,
                                 void* stream);

/* Bytes of workspace sparse_select_coverage needs (host; a helper of the
 * coverage rule, [P1], abstract, coverage-rule sentence). */
size_t sparse_select_workspace_bytes(const sparse_dims* dims);

/*
 * sparse_select_coverage -- the coverage rule, per unit ([P1], abstract,
 * coverage-rule sentence: keep the smallest page set whose estimated mass
 * reaches gamma).
 *
 * Per unit: pi_g = softmax over pages of logits[b][h][g][:n_b]; page mass
 * m = mean_g pi_g; the kept set is the first k* pages in (m descending, page
 * ascending) order, k* = min{k >= 1 : sum of the first k masses >= gamma * sum
 * of all masses}; gamma = 1 keeps every page.  Masses are fp32, the cut's sums
 * are exact 64-bit fixed point (weight = floor(m * 2^52)), found by a
 * mass-weighted radix select over the fp32 bit patterns with ties at the cut
 * filled by ascending page index.
 *
 * Outputs (unit u = b * Hkv + h; lists use a fixed stride of max_pages):
 *   sel_counts    int32 [U]            k* of each unit (0 when L_b = 0)
 *   sel_pages     int32 [U][max_pages] kept logical pages, ascending, first k* valid
 *   sel_phys      int32 [U][max_pages] page_table[b][sel_pages[..]]
 * Optional whole-batch prefix sum (NULL to skip):
 *   sel_offsets   int32 [U + 1]        exclusive prefix sum of sel_counts
 * It is written by whichever workgroup finishes last (a device-side ticket
 * in the workspace).  The attention and merge calls do not need it: they
 * derive their plan from sel_counts.
 *
 *   ws / ws_bytes  device workspace of at least sparse_select_workspace_bytes(),
 *                  needed only with the prefix sum (NULL otherwise); it must
 *                  be zero-filled ONCE before its first use and is left
 *                  zero-filled by every call.  Calls sharing one workspace
 *                  must not overlap in time.
 *   gamma          in (0, 1]
 */
sparse_status sparse_select_coverage(const sparse_dims* dims, const float* logits,
                                     const int32_t* ctx_lens, const int32_t* page_table,
                                     float gamma, int32_t* sel_counts, int32_t* sel_offsets,
                                     int32_t* sel_pages, int32_t* sel_phys, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * sparse_select_topk -- the fixed-budget selection the coverage rule is
 * argued against ([P1], abstract, sentence on fixed budgets): per unit keep
 * the min(k_pages, n_b) pages of highest group mass m (m as in
 * sparse_select_coverage), ties to the lower page index.  Same outputs,
 * workspace and prefix sum as sparse_select_coverage.  k_pages >= 1.
 */
sparse_status sparse_select_topk(const sparse_dims* dims, const float* logits,
                                 const int32_t* ctx_lens, const int32_t* page_table,
                                 int32_t k_pages, int32_t* sel_counts, int32_t* sel_offsets,
                                 int32_t* sel_pages, int32_t* sel_phys, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * sparse_append_tokens -- decode-time append of each request's new token,
 * with the refresh of its page's summary, so that the step's own token is
 * scored like every other: the coverage rule is applied anew at every decode
 * step over the whole context so far ([P1], abstract, coverage-rule
 * sentence: per request, layer, KV head and step).  For request b with L_b = ctx_lens[b] tokens, the token
 * goes to logical page p = L_b / 16, slot t = L_b % 16, of physical page
 * x = page_table[b][p] (allocated by the caller): row t of the K tile and
 * column t of the channel-major V tile, for every KV head.  The summary of
 * (x, h) becomes k itself when t = 0, else its per-channel min / max with k
 * (the total order of sparse_build_page_summaries: bit-exact with a rebuild
 * over the first t + 1 tokens).  ctx_lens[b] then advances by one.  A request
 * whose page is missing (p >= max_pages or x outside [0, pool_pages)) is left
 * untouched and its length is not advanced.
 *   k_new, v_new  bf16 [B][Hkv][128]
 */
sparse_status sparse_append_tokens(const sparse_dims* dims, const uint16_t* k_new,
                                   const uint16_t* v_new, uint16_t* kv, int64_t stride_page,
                                   int64_t stride_head, int64_t pool_pages,
                                   const int32_t* page_table, int32_t* ctx_lens, uint16_t* summ,
                                   void* stream);

/* Fewest plan positions the attention gives one workgroup: a step of T
 * positions runs on min(W, ceil(T / SPARSE_ATTN_MIN_WORKER_PAGES)) of its W
 * workgroups (see sparse_decode_attn). */
#define SPARSE_ATTN_MIN_WORKER_PAGES 32
/* Positions the attention's plan charges a unit on top of its entries: the
 * fixed cost, in pages, of starting a unit's segment (see sparse_decode_attn). */
#define SPARSE_ATTN_UNIT_COST_PAGES 12

/* Partial slots one step of sparse_decode_attn may write (host; a helper of
 * [P1]'s self-planning attention, abstract, self-planning sentence): U + W, with
 * U = batch * num_kv_heads and W = workers, or the current device's compute
 * unit count when workers = 0.  Returns -1 for invalid dims, workers < 0, or
 * workers = 0 when the current device cannot be queried. */
int64_t sparse_decode_max_parts(const sparse_dims* dims, int32_t workers);

/*
 * sparse_decode_attn -- self-planning split-K attention over the page lists
 * ([P1], abstract, sentence on self-planning attention: every block works
 * out from the per-head list lengths which part it handles, so no plan is
 * made on the host and the step stays inside the graph; and the sentence on
 * FA3/FlashInfer, which pad the lists, run unbalanced blocks or plan on the
 * host -- the even split below does none of these).
 *
 * The balanced plan.  Unit u has k_u = min(sel_counts[u], Lb) entries (Lb
 * the dims' list bound); a unit with k_u > 0 takes p_u = C + k_u positions,
 * C = SPARSE_ATTN_UNIT_COST_PAGES positions standing for the fixed cost of
 * starting a unit's segment, then one per entry.  Laid end to end in unit
 * order they are T = sum_u p_u global positions, entry e of unit u at
 * off_u + C + e with off_u = sum_{v<u} p_v.  The grid has W = workers
 * workgroups (0: one per compute unit of the current device), fixed at
 * enqueue time; the step uses W' = min(W, ceil(T /
 * SPARSE_ATTN_MIN_WORKER_PAGES)) of them (0 when T = 0), and worker w < W'
 * owns positions [floor(w T / W'), floor((w + 1) T / W')) -- the same work,
 * to within one page, for every worker whatever the list lengths (a worker
 * that starts a second unit's segment gets C fewer pages).  Each workgroup
 * derives T, W' and its units from sel_counts alone (wave prefix sums),
 * then, for every unit u whose entries its range meets, computes exact
 * attention of u's G query heads over the valid tokens of the pages at those
 * entries and writes, in slot c = u + w, for head g:
 *   part_o[c][g][:]  = sum_t softmax_t(scale * q.k_t) v_t   (normalised over the segment)
 *   part_lse[c][g]   = ln sum_t exp(scale * q.k_t)
 * (lse = -inf and o = 0 for a segment with no valid token).  Slots that no
 * (unit, worker) pair of this step uses are left as they were.
 * K/V are read from the pool at sel_phys (physical ids or cache slots).
 *
 *   part_o   fp32 [max_parts][G][128];  part_lse fp32 [max_parts][G]
 *   max_parts must equal sparse_decode_max_parts(dims, workers)
 *   workers  0 .. 2^20
 */
sparse_status sparse_decode_attn(const sparse_dims* dims, const uint16_t* q, const uint16_t* kv,
                                 int64_t stride_page, int64_t stride_head, int64_t pool_pages,
                                 const int32_t* ctx_lens, const int32_t* sel_counts,
                                 const int32_t* sel_pages, const int32_t* sel_phys, float scale,
                                 int32_t workers, float* part_o, float* part_lse,
                                 int64_t max_parts, void* stream);

/*
 * sparse_merge_splits -- log-sum-exp merge of each unit's segment partials:
 *   lse = ln sum_c exp(lse_c),  o = sum_c exp(lse_c - lse) * o_c,
 * the identity that makes exact the split of one page list over several
 * workgroups ([P1], abstract, sentence on self-planning attention: a list
 * is shared among the blocks that plan their own part of it).  Unit u's
 * partials are the slots u + w for the workers w from the owner of its first
 * entry's position (off_u + C) to the owner of its last (off_u + C + k_u - 1)
 * under the plan of sparse_decode_attn, found from sel_counts alone; workers and dims
 * must be those of the sparse_decode_attn call that wrote them.  Other slots
 * are not read as values.
 *   out      fp32 [B][Hq][128];  out_lse fp32 [B][Hq]
 * A unit with no kept page gets o = 0 and lse = -inf.
 */
sparse_status sparse_merge_splits(const sparse_dims* dims, const float* part_o,
                                  const float* part_lse, const int32_t* sel_counts,
                                  int32_t workers, float* out, float* out_lse, void* stream);

/*
 * sparse_merge_splits_pair -- the merge of sparse_merge_splits over two
 * disjoint sets of lists of the same rows: unit u's segments under the plan
 * of lists a (sel_counts_a, partials part_o_a / part_lse_a, written by
 * sparse_decode_attn with workers_a) and under the plan of lists b, all
 * merged by the same identity into one result -- attention over the union
 * of the two lists ([P1], abstract, sentence on self-planning attention, as
 * sparse_merge_splits).  The host tier's split step merges the hits' and the
 * misses' partials with it.  Arguments and errors as sparse_merge_splits,
 * per set.
 */
sparse_status sparse_merge_splits_pair(const sparse_dims* dims, const float* part_o_a,
                                       const float* part_lse_a, const int32_t* sel_counts_a,
                                       int32_t workers_a, const float* part_o_b,
                                       const float* part_lse_b, const int32_t* sel_counts_b,
                                       int32_t workers_b, float* out, float* out_lse,
                                       void* stream);

/*
 * sparse_decode_attn_merge -- sparse_decode_attn followed by
 * sparse_merge_splits on the same stream, in one call: attention of every
 * unit's G query heads over its page list ([P1], abstract, sentence on
 * self-planning attention), the per-segment partials passing through the
 * caller's part_o / part_lse (same layout, size and max_parts rule as
 * sparse_decode_attn), the merged result in out / out_lse (as
 * sparse_merge_splits).  Same kernels, so the outputs are bitwise those of
 * the two calls.  Errors as the two calls; nothing is enqueued on error.
 */
sparse_status sparse_decode_attn_merge(const sparse_dims* dims, const uint16_t* q,
                                       const uint16_t* kv, int64_t stride_page,
                                       int64_t stride_head, int64_t pool_pages,
                                       const int32_t* ctx_lens, const int32_t* sel_counts,
                                       const int32_t* sel_pages, const int32_t* sel_phys,
                                       float scale, int32_t workers, float* part_o,
                                       float* part_lse, int64_t max_parts, float* out,
                                       float* out_lse, void* stream);

/*
 * sparse_decode_attn_merge_noalloc -- sparse_decode_attn_merge for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same outputs, bitwise, but the partials live in a library-owned device
 * array of SPARSE_NOALLOC_SCRATCH_BYTES per GPU (a static __device__ array,
 * held until the process ends), so the caller passes only inputs and outputs
 * and the call allocates nothing.
 *
 * Limit: (U + W) * G * 129 * 4 bytes <= SPARSE_NOALLOC_SCRATCH_BYTES, with
 * U = batch * num_kv_heads, W the resolved workers (see sparse_decode_attn);
 * larger steps return SPARSE_ERR_WORKSPACE (use sparse_decode_attn_merge
 * with a caller workspace).  16 MiB holds e.g. 7800 units at G = 4 and
 * W = 256.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (on different streams) race and give wrong
 * outputs; calls ordered on one stream are safe.  Nothing in the array needs
 * clearing: a call reads only partials it wrote itself.  The first call made
 * with a device current resolves that device's array address (a host
 * query, no allocation); make it once before capturing a graph.  Errors as
 * sparse_decode_attn_merge; SPARSE_ERR_HIP if the address cannot be resolved.
 */
#define SPARSE_NOALLOC_SCRATCH_BYTES (16u << 20)
sparse_status sparse_decode_attn_merge_noalloc(const sparse_dims* dims, const uint16_t* q,
                                               const uint16_t* kv, int64_t stride_page,
                                               int64_t stride_head, int64_t pool_pages,
                                               const int32_t* ctx_lens,
                                               const int32_t* sel_counts,
                                               const int32_t* sel_pages,
                                               const int32_t* sel_phys, float scale,
                                               int32_t workers, float* out, float* out_lse,
                                               void* stream);

/* Bytes of workspace sparse_hbm_cache_resolve needs (host; the resolver of
 * [P2], abstract, sentence on the fused in-graph resolver): a ticket word per
 * request (the resolve's workgroups of one request count themselves in on
 * it), the per-request list of placed misses (kept for a separate fetch, see
 * sparse_hbm_cache_fetch) and a ticket for the whole grid.  Zero it once
 * before the first call; every call leaves the tickets zero. */
size_t sparse_cache_workspace_bytes(const sparse_dims* dims, int32_t capacity);

/*
 * sparse_hbm_cache_resolve -- host-resident KV tier behind a fixed-size HBM
 * page cache, resolved on the device inside the step ([P2], abstract: full KV
 * history in host memory, a small fixed-size GPU cache per request, and one
 * resolver inside the graph that finds hits, replaces least recently used
 * entries and fetches misses from the host; attention outputs stay the same
 * because only where KV lives changes).
 *
 * Cache unit = (logical page p, KV head h) of request b, unit id
 * v = h * max_pages + p.  Per request, the requested set R is the union of the
 * request's KV-head lists (sel_pages / sel_counts, as written by
 * sparse_select_coverage or supplied by the caller).  Units of R already
 * resident are hits (their stamp becomes the current step).  Misses, in ascending unit
 * id, take slots in ascending slot index from the available set: the lowest
 * free slots if they suffice, else every free slot plus the
 * r = misses - free least recently used resident units outside R, ordered by
 * (stamp, unit id) -- exact LRU with ties to the lower unit id.  Each placed
 * miss is copied (8 KiB: K tile then channel-major V tile) from host_kv into
 * its slot by device-initiated reads of pinned host memory.  Misses that find
 * no slot get sel_phys = -1 and set the overflow flag (attention treats them
 * as empty pages; the step's outputs are then not meaningful).
 *
 *   host_kv    bf16 [B][max_pages][Hkv][2][2048], pinned host memory the
 *              device can address (hipHostMalloc / torch pin_memory)
 *   cache_kv   bf16 [B * capacity][2][2048] device; attend it with
 *              sparse_decode_attn(kv = cache_kv, stride_page = 4096,
 *              stride_head = 0, pool_pages = B * capacity, sel_phys)
 *   slot_tag   int32 [B][capacity]  unit id held by each slot, -1 = free
 *   slot_stamp int32 [B][capacity]  step of last use (-1 when free)
 *   unit_slot  int32 [B][Hkv * max_pages]  slot of each unit, -1 = not resident
 *              (the caller initialises tags/stamps/unit_slot to -1 once; the
 *              library keeps them consistent afterwards)
 *   step_counter  int32 [1] device: the step number this call stamps with
 *              (start it at 0); the call advances it by one, so a captured
 *              graph replays with fresh steps
 *   sel_phys   int32 [U][max_pages] out: global slot id b * capacity + slot
 *   stats      int32 [B][4] out: hits, misses, evictions, overflow flag
 *   capacity   slots per request, 1..8192; num_kv_heads <= 64
 *   ws         see sparse_cache_workspace_bytes (zeroed once before use)
 * Enqueues one kernel: one 1024-thread workgroup per (request, KV head,
 * chunk of up to 1024 list entries); each stamps its hits and writes their
 * slot ids, and the last of a request's workgroups to finish places the
 * request's misses and copies them into their slots (or, with none, writes
 * only the statistics); the grid's last workgroup advances the step.  Calls
 * sharing cache state or a workspace must not overlap in time.
 */
sparse_status sparse_hbm_cache_resolve(const sparse_dims* dims, const int32_t* sel_counts,
                                       const int32_t* sel_pages, const uint16_t* host_kv,
                                       uint16_t* cache_kv, int32_t capacity, int32_t* slot_tag,
                                       int32_t* slot_stamp, int32_t* unit_slot,
                                       int32_t* step_counter, int32_t* sel_phys, int32_t* stats,
                                       void* ws, size_t ws_bytes, void* stream);

/*
 * Replacement policy of the host-tier cache (sparse_hbm_cache_resolve_policy).
 *
 * recency_shift -- bucketed LRU ([P3], abstract, technique (2): a
 *   GPU-friendly bucketed LRU policy; no bucket rule is given, this is the
 *   library's reading): resident units are ordered for eviction by
 *   (stamp >> recency_shift, unit id), i.e. stamps compared in buckets of
 *   2^recency_shift steps, the lower unit id first within a bucket.
 *   0 = exact LRU (sparse_hbm_cache_resolve).  0..30.
 * pooled -- 0: one cache of `capacity` slots per request (as
 *   sparse_hbm_cache_resolve).  1: one pool of `capacity` slots shared by all
 *   requests ([P3], abstract, same technique: per-request HBM budgets
 *   sized dynamically -- a request holds as many slots as the pool-wide
 *   replacement leaves it).  Pooled unit id g = (b * Hkv + h) * max_pages +
 *   p; every rule of sparse_hbm_cache_resolve applies over pooled ids (the
 *   requested set is the union over requests; misses in ascending pooled id
 *   take the available slots in ascending slot index).
 */
typedef struct {
  int32_t recency_shift;
  int32_t pooled;
} sparse_cache_policy;

/* Bytes of workspace sparse_hbm_cache_resolve_policy needs (host); 0 for
 * invalid arguments.  Per-request: as sparse_cache_workspace_bytes.  Pooled:
 * about 25 bytes per slot plus 12 per request. */
size_t sparse_cache_policy_workspace_bytes(const sparse_dims* dims,
                                           const sparse_cache_policy* policy,
                                           int32_t capacity);

/*
 * sparse_hbm_cache_resolve_policy -- sparse_hbm_cache_resolve under a
 * replacement policy (see sparse_cache_policy: [P3], abstract, technique
 * (2), bucketed LRU and per-request budgets sized dynamically).  Arguments as
 * sparse_hbm_cache_resolve, except when policy->pooled = 1:
 *   capacity   slots of the pool, 1 .. 2^22 (B * Hkv * max_pages < 2^31)
 *   cache_kv   bf16 [capacity][2][2048] device (stride_page 4096, stride_head
 *              0, pool_pages = capacity for sparse_decode_attn)
 *   slot_tag   int32 [capacity] pooled unit id held by each slot, -1 = free
 *   slot_stamp int32 [capacity]
 *   unit_slot  int32 [B][Hkv * max_pages] (the same shape: index = pooled id)
 *   sel_phys   int32 [U][max_pages] out: slot index
 *   stats      int32 [B][4] out: hits, misses, evictions made by that
 *              request's misses, overflow (one of its misses got no slot)
 *   ws         pooled: zero it once before the first call (it carries the
 *              requested-slot marks and two running totals, which every
 *              call leaves zero)
 * Pooled mode enqueues five resolve kernels (per request; per block of 1024
 * slots; one workgroup selecting the victims; per block; per request) and
 * one fetch kernel.  Lists must hold distinct pages (as the selection writes
 * them).  Errors: as sparse_hbm_cache_resolve; policy missing or out of
 * range -> INVALID.
 */
sparse_status sparse_hbm_cache_resolve_policy(const sparse_dims* dims,
                                              const sparse_cache_policy* policy,
                                              const int32_t* sel_counts,
                                              const int32_t* sel_pages, const uint16_t* host_kv,
                                              uint16_t* cache_kv, int32_t capacity,
                                              int32_t* slot_tag, int32_t* slot_stamp,
                                              int32_t* unit_slot, int32_t* step_counter,
                                              int32_t* sel_phys, int32_t* stats, void* ws,
                                              size_t ws_bytes, void* stream);

/*
 * The host tier in two halves, so that attention over the hits can run while
 * the misses are still crossing PCIe (the split the resolver's placement
 * rule allows: a hit's slot is never a victim of the same step, so the hits
 * are final once the resolve has run).  The resolver is [P2]'s (abstract:
 * hit detection, LRU replacement and host-to-device fetches inside the
 * decode graph; only KV placement changes, so outputs do not), and the
 * merge is the split-and-merge identity of [P1]'s self-planning attention
 * (abstract, self-planning sentence).  One step is:
 *   sparse_hbm_cache_resolve_split   hits, victims, slots, and each unit's
 *                                    placed misses as a short list; no copy
 *   sparse_hbm_cache_fetch_attn      the misses' copies, each attended in
 *                                    the copying wave as it arrives, beside
 *                                    attention over the hits; advances the
 *                                    step
 *   sparse_merge_splits_pair         both sets of partials into the output
 *                                    (attention over a partition of a list,
 *                                    merged by log-sum-exp, is attention
 *                                    over the list)
 * or, with the copy on its own (sparse_hbm_cache_fetch), attention over the
 * hits beside it and attention over the miss lists after it.  Cache state,
 * statistics and sel_phys equal those of sparse_hbm_cache_resolve_policy on
 * the same inputs.
 *
 * sparse_hbm_cache_resolve_split -- the resolve of
 * sparse_hbm_cache_resolve_policy without the fetch.  Arguments as there
 * (no pools: the resolve never reads them), plus
 *   hit_phys    int32 [U][max_pages] out: for list entry i of unit u, the slot
 *               (as in sel_phys) if the unit was resident before this step,
 *               else -1; entries past sel_counts[u] are not written
 *   miss_counts int32 [U] out, miss_pages, miss_phys int32 [U][max_pages]
 *               out: for each unit, the list entries placed this step (not
 *               resident before, given a slot), in list order -- lists that
 *               sparse_decode_attn takes as (sel_counts, sel_pages,
 *               sel_phys); entries past miss_counts[u] are not written.  All
 *               three NULL: not written.
 * The misses it placed are recorded in ws for the next
 * sparse_hbm_cache_fetch on the same ws, which must follow it in stream
 * order before ws is used again.  Errors as sparse_hbm_cache_resolve_policy;
 * NULL hit_phys, or some but not all of the miss-list pointers -> INVALID.
 */
sparse_status sparse_hbm_cache_resolve_split(const sparse_dims* dims,
                                             const sparse_cache_policy* policy,
                                             const int32_t* sel_counts,
                                             const int32_t* sel_pages, int32_t capacity,
                                             int32_t* slot_tag, int32_t* slot_stamp,
                                             int32_t* unit_slot, int32_t* step_counter,
                                             int32_t* sel_phys, int32_t* hit_phys,
                                             int32_t* stats, int32_t* miss_counts,
                                             int32_t* miss_pages, int32_t* miss_phys, void* ws,
                                             size_t ws_bytes, void* stream);

/*
 * The fetch kernels (of sparse_hbm_cache_fetch, and of the pooled
 * sparse_hbm_cache_resolve_policy) run SPARSE_FETCH_GROUPS workgroups of 8 waves (for
 * up to 256 requests; one more per 8 requests beyond), each holding a whole
 * compute unit's LDS so that no other workgroup shares its unit.  A caller
 * that runs attention on another stream while a fetch is in flight can size
 * the attention (sparse_decode_attn's workers) to leave that many units free.
 */
#define SPARSE_FETCH_GROUPS 32

/*
 * sparse_hbm_cache_fetch -- the host-to-device fetch of [P2]'s resolver
 * (abstract, fused-resolver sentence) on its own: copy every miss placed by the last
 * sparse_hbm_cache_resolve_split on this ws from host_kv into its slot of
 * cache_kv (device-initiated reads of pinned host memory), and advance
 * *step_counter.  Arguments as sparse_hbm_cache_resolve_policy.
 */
sparse_status sparse_hbm_cache_fetch(const sparse_dims* dims, const sparse_cache_policy* policy,
                                     const uint16_t* host_kv, uint16_t* cache_kv,
                                     int32_t capacity, int32_t* step_counter, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * sparse_hbm_cache_fetch_attn -- the copies of a step's placed misses with
 * the attention over them, and the attention over its hits, in one launch.
 *   - SPARSE_FETCH_ATTN_COPY_WAVES copying waves share the miss lists
 *     (miss_counts, miss_pages, miss_phys as written by
 *     sparse_hbm_cache_resolve_split) under the balanced plan of
 *     sparse_decode_attn with one worker per wave.  Each reads its misses
 *     from host_kv (device-initiated reads of pinned host memory), writes
 *     them to their slots of cache_kv, and attends them from registers with
 *     the unit's queries; its partial for unit u goes to slot u + wave of
 *     miss_part_o / miss_part_lse.  A miss whose page is outside
 *     0 .. max_pages - 1 or whose slot is outside the pool is skipped.
 *   - The attention's workers run sparse_decode_attn over (sel_counts,
 *     sel_pages, hit_phys) on the cache pool (kv = cache_kv, stride_page
 *     4096, stride_head 0, pool_pages = B * capacity, or capacity pooled).
 *     A hit's slot is never written by the same step, so the two run side by
 *     side.
 * The copying waves form SPARSE_FETCH_ATTN_COPY_GROUPS workgroups placed
 * first in the grid; every workgroup holds 96 KiB of LDS, so a compute unit
 * never mixes copying waves (whose host reads take microseconds) with
 * attention waves.  With nothing to copy the copying waves exit after
 * reading miss_counts.  sparse_merge_splits_pair(part_o, part_lse,
 * sel_counts, workers, miss_part_o, miss_part_lse, miss_counts,
 * SPARSE_FETCH_ATTN_COPY_WAVES) then gives the step's output.
 * Arguments: dims, policy, host_kv, cache_kv, capacity and step_counter as
 * sparse_hbm_cache_resolve_policy; q, ctx_lens, sel_counts, sel_pages,
 * scale, workers, part_o, part_lse, max_parts as sparse_decode_attn with
 * hit_phys as sel_phys;
 *   miss_counts  int32 [U]; miss_pages, miss_phys int32 [U][max_pages]
 *   miss_part_o  fp32 [U + SPARSE_FETCH_ATTN_COPY_WAVES][G][128] out,
 *                16-byte aligned
 *   miss_part_lse fp32 [U + SPARSE_FETCH_ATTN_COPY_WAVES][G] out
 * Advances *step_counter.  Errors: as sparse_decode_attn and
 * sparse_hbm_cache_resolve_policy (no workspace); a NULL miss list or miss
 * partial -> INVALID.
 */
#define SPARSE_FETCH_ATTN_COPY_GROUPS 64
#define SPARSE_FETCH_ATTN_COPY_WAVES (4 * SPARSE_FETCH_ATTN_COPY_GROUPS)
sparse_status sparse_hbm_cache_fetch_attn(
    const sparse_dims* dims, const sparse_cache_policy* policy, const uint16_t* host_kv,
    uint16_t* cache_kv, int32_t capacity, int32_t* step_counter, const uint16_t* q,
    const int32_t* ctx_lens, const int32_t* sel_counts, const int32_t* sel_pages,
    const int32_t* hit_phys, const int32_t* miss_counts, const int32_t* miss_pages,
    const int32_t* miss_phys, float scale, int32_t workers, float* part_o, float* part_lse,
    int64_t max_parts, float* miss_part_o, float* miss_part_lse, void* stream);

/*
 * sparse_split_misses -- a helper of the split host tier above ([P2],
 * abstract): for each unit u, the list entries i < sel_counts[u]
 * with hit_phys < 0 and sel_phys >= 0 (placed this step, not resident
 * before), in list order, as
 *   miss_counts int32 [U]              their number
 *   miss_pages  int32 [U][max_pages]   their logical pages (ascending)
 *   miss_phys   int32 [U][max_pages]   their slots
 * -- lists that sparse_decode_attn takes as (sel_counts, sel_pages,
 * sel_phys).  The same lists sparse_hbm_cache_resolve_split writes when given
 * the miss-list outputs; this is the separate pass over sel_phys and hit_phys.
 * Each sel_counts[u] is clamped to [0, max_pages]; entries past a unit's
 * miss count are left as they were.  One 256-thread workgroup per unit.
 */
sparse_status sparse_split_misses(const sparse_dims* dims, const int32_t* sel_counts,
                                  const int32_t* sel_pages, const int32_t* sel_phys,
                                  const int32_t* hit_phys, int32_t* miss_counts,
                                  int32_t* miss_pages, int32_t* miss_phys, void* stream);

/*
 * sparse_lse_combine -- two attention results over disjoint token sets of
 * the same rows, combined by the identity of sparse_merge_splits (the merge
 * behind [P1]'s self-planning attention, abstract, self-planning sentence):
 *   lse = ln(exp(lse_a) + exp(lse_b)),
 *   out = exp(lse_a - lse) * out_a + exp(lse_b - lse) * out_b
 * (a side with lse = -inf contributes nothing; both -inf gives out = 0 and
 * lse = -inf).  out_a, out_b, out fp32 [B][Hq][128]; lse_a, lse_b, out_lse
 * fp32 [B][Hq].  out may be out_a or out_b; out_lse must not be lse_a or
 * lse_b (INVALID).
 */
sparse_status sparse_lse_combine(const sparse_dims* dims, const float* out_a, const float* lse_a,
                                 const float* out_b, const float* lse_b, float* out,
                                 float* out_lse, void* stream);

/*
 * Measurement helper (not a step of the decode path).
 *
 * sparse_read_blocks -- read whole 8 KiB blocks of a pool in a given order,
 * with nothing else to do, to measure the read rate that the attention
 * kernel's own access unit (one (page, KV head) K+V block) allows.  Block i
 * is the 4096 bf16 values starting at element pool + i * 4096 (the canonical
 * pool [Ppool][Hkv][2][2048] has Ppool * Hkv blocks).  The kernel reads
 * blocks order[0 .. n) -- a random permutation gives the random-block
 * ceiling, ascending ids the streaming-read ceiling -- with
 * SPARSE_READ_BLOCKS_GROUPS workgroups of 4 waves, 2 blocks in flight per
 * wave and non-temporal loads.  Workgroup g writes the XOR of every 32-bit
 * word it read to xor_out[g]; the XOR of all SPARSE_READ_BLOCKS_GROUPS words
 * is the XOR over the listed blocks (a block listed twice cancels itself).
 * Ids outside [0, pool_blocks) are skipped.  Every call writes all of
 * xor_out.  order may be NULL when n == 0.
 *   xor_out  uint32 [SPARSE_READ_BLOCKS_GROUPS], 4-byte aligned
 * INVALID: n < 0, pool_blocks < 0, a NULL pool or xor_out (or order with
 * n > 0), pool not 16-byte aligned.
 */
#define SPARSE_READ_BLOCKS_GROUPS 4096
sparse_status sparse_read_blocks(const uint16_t* pool, int64_t pool_blocks,
                                 const int32_t* order, int64_t n, uint32_t* xor_out,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_PAGED_H */
