"""fp64 CPU oracle of one sparse paged decode step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and bench.py's CPU-baseline leg may import this
module.  It shares nothing with the HIP library.  Everything is NumPy float64;
bf16 inputs are decoded exactly (bits << 16 -> float32 -> float64).

Page keys used in citations: [P1] "Adaptive DHiSparse: Speculative Decoding over
a Load-Adaptive KV Hierarchy" (MOIRA abstract); [P2] "HiSparse: Scaling Sparse
Attention Decoding with Hierarchical KV Cache" (abstract); [P3] "Unifying Sparse
Attention with Hierarchical Memory for Scalable Long-Context LLM Serving" (SPIN
abstract and its RaBitQCache card).

What the pages fix and what is read into them:

* The coverage rule [P1, abstract, coverage-rule sentence]: per request, layer,
  KV head and step, keep the fewest pages that together hold at least gamma of
  the *estimated* attention mass.  The pages name no estimator.  Reading used here:
  the Quest-style per-channel min/max key bound (Quest is named as a family on
  [P2, abstract, evaluation sentence]), turned into a per-page mass by a
  softmax over s*u + ln(n_valid), averaged over the G query heads of the KV
  head's group, cut at cumulative mass >= gamma * total in (mass desc, page asc)
  order (the cumulative / top-p reading; [P3] RaBitQCache card: adaptive top-p).
* Exact attention over the selected pages [P1, abstract, self-planning
  sentence: the kernel attends over variable-length page lists]; split-K
  partials are merged by log-sum-exp (a plain identity, written out here as
  its definition).

Functions whose agreement with the pages' own (unprinted) estimator cannot be
checked are marked "parity unpinned" below (that agreement only: each is still
pinned to the mathematics).  Every function is pinned by a CPU test in
tests/test_oracle_pins.py against something other than itself:

  bf16_bits_to_f64, f64_to_bf16_bits  all 65536 patterns; ties to even; torch's rounding
  summaries                           brute-force loops with tails and signed zeros
  bound                               dominates the true max logit; loops; q >= 0 / q <= 0
                                      and identical-key closed forms
  page_logits, head_mass, group_mass  sum to one; equal the exact dense page masses when
                                      every token of a page shares its key; the
                                      hand-derived worked example (tests/golden)
  coverage_cut                        brute force over all subsets; monotone and nested in
                                      gamma; n = 1, ties, gamma = 1; tests/golden fixtures
  topk_cut                            brute force; agrees with the coverage cut at k = k*
  select_unit                         the worked example's masses and cuts from bf16 bits
  attend_tokens, attend_pages         brute-force loops; scipy logsumexp; one token,
                                      equal keys, page permutation; worked example
  dense_unit                          gamma = 1 against brute-force dense attention
  merge_partials                      any partition of the tokens merges to the whole
  list_accepted                       accepts exact lists, rejects planted defects
  (oracle/lru.py)                     a textbook OrderedDict LRU, an explicit bucket model
                                      and per-request caches without pool pressure
"""

import numpy as np

PAGE = 16  # tokens per page (the workloads' page size; the pages print none)


# ----------------------------------------------------------------------------
# bf16 <-> float64 (exact decode; round-to-nearest-even encode)
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (any integer dtype) exactly to float64."""
    b = (np.asarray(bits).astype(np.int64) & 0xFFFF).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 (round to nearest, ties to even) -> uint16.

    Written from the bf16 format itself: 8 significant bits, fp32's exponent
    range, subnormal spacing 2**-133, overflow to +-inf past 0x7F7F.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = f * 2**e, 0.5 <= |f| < 1
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    y = np.rint(x / quantum) * quantum      # rint: ties to even
    big = np.abs(y) > 3.3895313892515355e38  # largest finite bf16 (0x7F7F)
    y = np.where(big, np.copysign(np.inf, x), y)
    f32 = y.astype(np.float32)              # exact: y has <= 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# O1: per-page key summaries
# ----------------------------------------------------------------------------

def _total_order_key(bits):
    """Integer key that orders non-NaN bf16 values numerically, with -0 < +0
    (IEEE-754 totalOrder).  The signed-zero rule makes min/max a unique bit
    pattern, so summaries are defined bit-exactly."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    return np.where(b & 0x8000, 0xFFFF - b, b | 0x8000)


def summaries(k_pages_bits, n_valid):
    """kmin/kmax over the valid tokens of each page, per channel.

    k_pages_bits: [n][P][D] bf16 bits (token-major K tiles of one KV head).
    n_valid:      [n] valid tokens per page (1..P).
    Returns (kmin_bits, kmax_bits), each [n][D] uint16.

    The per-page per-channel min/max is the Quest-style page summary (Quest is
    named as an evaluated family, [P2, abstract, evaluation sentence]).
    """
    k = np.asarray(k_pages_bits).astype(np.int64) & 0xFFFF
    n, P, D = k.shape
    nv = np.asarray(n_valid, dtype=np.int64).reshape(n)
    if np.any(nv < 1) or np.any(nv > P):
        raise ValueError("every page needs 1..P valid tokens")
    key = _total_order_key(k)
    valid = (np.arange(P)[None, :] < nv[:, None])[:, :, None]       # [n][P][1]
    big = np.int64(1 << 20)
    imin = np.argmin(np.where(valid, key, big), axis=1)             # [n][D]
    imax = np.argmax(np.where(valid, key, -big), axis=1)
    kmin = np.take_along_axis(k, imin[:, None, :], axis=1)[:, 0, :]
    kmax = np.take_along_axis(k, imax[:, None, :], axis=1)[:, 0, :]
    return kmin.astype(np.uint16), kmax.astype(np.uint16)


# ----------------------------------------------------------------------------
# O2-O5: the estimate and the per-page mass (parity unpinned against the
# pages' own estimator, which they never name; pinned by invariants)
# ----------------------------------------------------------------------------

def bound(q, kmin, kmax):
    """u[g][p] = sum_d max(q[g,d]*kmin[p,d], q[g,d]*kmax[p,d]).

    q: [G][D] float64; kmin, kmax: [n][D] float64.  Since kmin <= k_t <= kmax
    channel-wise for every valid token t, u[g][p] >= q_g . k_t for all t in p.
    """
    q = np.asarray(q, dtype=np.float64)
    kmin = np.asarray(kmin, dtype=np.float64)
    kmax = np.asarray(kmax, dtype=np.float64)
    G = q.shape[0]
    n = kmin.shape[0]
    u = np.empty((G, n), dtype=np.float64)
    step = 2048
    for s0 in range(0, n, step):
        a = q[:, None, :] * kmin[None, s0:s0 + step, :]
        b = q[:, None, :] * kmax[None, s0:s0 + step, :]
        u[:, s0:s0 + step] = np.maximum(a, b).sum(axis=2)
    return u


def page_logits(u, n_valid, scale):
    """x[g][p] = scale*u[g][p] + ln(n_valid[p]).

    n_valid * exp(scale*u) bounds the page's unnormalised attention mass
    (every one of its n_valid tokens has logit <= scale*u), so x is the log of
    that bound.  Reading of "estimated attention mass" [P1, abstract,
    coverage-rule sentence]; parity unpinned against the pages' estimator.
    """
    nv = np.asarray(n_valid, dtype=np.float64)
    return scale * np.asarray(u, dtype=np.float64) + np.log(nv)[None, :]


def head_mass(x):
    """pi[g][p] = exp(x[g][p] - max_p x[g]) / sum_p exp(x[g][p] - max_p x[g])."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def group_mass(pi):
    """m[p] = (1/G) * sum_g pi[g][p]: one list serves the whole GQA group, so
    the group's page mass is the mean of its heads' normalised masses."""
    return np.asarray(pi, dtype=np.float64).mean(axis=0)


# ----------------------------------------------------------------------------
# O6-O7: the coverage rule [P1, abstract, coverage-rule sentence]
# ----------------------------------------------------------------------------

def coverage_cut(m, gamma):
    """Smallest page set whose mass reaches gamma of the total.

    Pages are ordered by (mass descending, page index ascending); the set is
    the first k* of that order with k* = min{k >= 1 : S_k >= gamma * Z}, where
    S_k is the sum of the first k masses and Z = S_n.  Taking the largest
    masses first gives the minimum cardinality.  gamma >= 1 keeps every page.
    Returns (sorted page list, k*, order, cumulative sums).
    """
    m = np.asarray(m, dtype=np.float64)
    n = m.shape[0]
    if n == 0:
        raise ValueError("a unit has at least one page")
    if not (gamma > 0.0):
        raise ValueError("gamma must be in (0, 1]")
    order = np.lexsort((np.arange(n), -m))
    S = np.cumsum(m[order])
    Z = S[-1]
    if gamma >= 1.0:
        k = n
    else:
        k = int(np.argmax(S >= gamma * Z)) + 1
    return np.sort(order[:k]), k, order, S


def topk_cut(m, k):
    """Fixed-budget selection (the baseline the coverage rule replaces,
    [P1, abstract, sentence on fixed budgets]): the min(k, n) pages of highest
    mass, ties to the lower page index, emitted ascending."""
    m = np.asarray(m, dtype=np.float64)
    n = m.shape[0]
    if k < 1:
        raise ValueError("k >= 1")
    order = np.lexsort((np.arange(n), -m))
    return np.sort(order[:min(k, n)])


def select_unit(q_bits, kmin_bits, kmax_bits, n_valid, scale, gamma):
    """Score, mass and cut for one (request, KV head) unit.

    q_bits [G][D] bf16 bits; kmin_bits/kmax_bits [n][D] bf16 bits.
    Returns dict with 'list', 'count', 'm', 'x', 'u'.
    """
    q = bf16_bits_to_f64(q_bits)
    kmin = bf16_bits_to_f64(kmin_bits)
    kmax = bf16_bits_to_f64(kmax_bits)
    u = bound(q, kmin, kmax)
    x = page_logits(u, n_valid, scale)
    m = group_mass(head_mass(x))
    lst, k, _, _ = coverage_cut(m, gamma)
    return {"list": lst, "count": k, "m": m, "x": x, "u": u}


# ----------------------------------------------------------------------------
# O8-O9: exact attention over the selected pages, and the split/merge identity
# ----------------------------------------------------------------------------

def attend_tokens(q, K, V, scale):
    """Exact softmax attention of G query rows over T tokens, in float64.

    q [G][D], K [T][D], V [T][D].  Returns o [G][D] and lse [G] with
    l_t = scale * q.k_t, lse = ln sum_t exp(l_t), o = sum_t exp(l_t - lse) v_t.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        raise ValueError("attention over an empty token set")
    logit = scale * (q @ K.T)
    mx = logit.max(axis=1, keepdims=True)
    w = np.exp(logit - mx)
    ssum = w.sum(axis=1, keepdims=True)
    lse = (mx + np.log(ssum))[:, 0]
    o = (w / ssum) @ V
    return o, lse


def attend_pages(q, K_pages, V_pages, n_valid, pages, scale):
    """Attention over the valid tokens of the listed pages.

    K_pages, V_pages: [n][P][D] float64, token-major; pages: logical indices.
    """
    pages = np.asarray(pages, dtype=np.int64)
    nv = np.asarray(n_valid, dtype=np.int64)
    Ks = [K_pages[p, :nv[p]] for p in pages]
    Vs = [V_pages[p, :nv[p]] for p in pages]
    return attend_tokens(q, np.concatenate(Ks, 0), np.concatenate(Vs, 0), scale)


def dense_unit(q, K_pages, V_pages, n_valid, scale):
    """Dense attention over every page of the unit (the gamma = 1 case)."""
    return attend_pages(q, K_pages, V_pages, n_valid, np.arange(K_pages.shape[0]), scale)


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint token sets.

    o_parts [C][G][D] (each normalised over its own set), lse_parts [C][G]:
    lse = ln sum_c exp(lse_c), o = sum_c exp(lse_c - lse) o_c.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0, keepdims=True)
    w = np.exp(lse_parts - mx)
    ssum = w.sum(axis=0, keepdims=True)
    lse = (mx + np.log(ssum))[0]
    o = ((w / ssum)[:, :, None] * o_parts).sum(axis=0)
    return o, lse


# ----------------------------------------------------------------------------
# Acceptance of a list computed in lower precision
# ----------------------------------------------------------------------------

def list_accepted(A, m, gamma, eps=1e-5):
    """Is page list A the coverage rule's output for masses within a relative
    eps of m?  (Exact agreement is required except where masses within eps of
    each other make several lists correct.)  Returns (ok, reason).

    Conservative checks, each under its own worst-case perturbation:
      P1 top set:  min_{A} m (1+eps) >= max_{not A} m (1-eps)
      P2 reaches:  (1-gamma)(1+eps) S(A) >= gamma (1-eps) (Z - S(A))
      P3 minimal:  (1-gamma)(1-eps)(S(A) - m_a) < gamma (1+eps)(Z - S(A) + m_a),
                   a = A's least-mass page.
    gamma >= 1 requires every page.
    """
    m = np.asarray(m, dtype=np.float64)
    n = m.shape[0]
    A = np.asarray(A, dtype=np.int64)
    if A.size == 0:
        return False, "empty list"
    if np.any(A < 0) or np.any(A >= n):
        return False, "page index out of range"
    if A.size > 1 and np.any(np.diff(A) <= 0):
        return False, "not strictly ascending"
    if gamma >= 1.0:
        return (A.size == n), ("gamma=1 needs all pages" if A.size != n else "ok")
    inA = np.zeros(n, dtype=bool)
    inA[A] = True
    S = m[inA].sum()
    Z = m.sum()
    R = Z - S
    if (~inA).any():
        if m[inA].min() * (1 + eps) < m[~inA].max() * (1 - eps):
            return False, "not a top set"
    if (1 - gamma) * (1 + eps) * S < gamma * (1 - eps) * R:
        return False, "does not reach gamma"
    ma = m[inA].min()
    if not ((1 - gamma) * (1 - eps) * (S - ma) < gamma * (1 + eps) * (R + ma)):
        return False, "not minimal"
    return True, "ok"
