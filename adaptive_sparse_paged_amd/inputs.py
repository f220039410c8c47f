"""Seeded synthetic inputs for the sparse paged decode step.

This module only *makes inputs*: it holds none of the method's arithmetic (no
scores, masses, cuts or attention).  The tests feed the same bytes to the HIP
library and to the fp64 CPU oracle, and the benchmark builds its KV pools here.

Random bits come from one counter-based generator, the splitmix64 output
function (Steele, Lea and Flood, "Fast Splittable Pseudorandom Number
Generators", OOPSLA 2014): output i of a stream with key k is
mix64(k + (i + 1) * 0x9E3779B97F4A7C15) mod 2**64.  It is written with torch
int64 tensor ops only (add, multiply, xor, shift, mask), so it produces the same
bits on the CPU and on the GPU; any single unit of a workload can therefore be
regenerated on the host without holding the whole pool.

Normal bf16 values: each 64-bit output gives four 16-bit uniforms u, mapped
through a fixed table T[u] = bf16(fp32(Phi^-1((u + 0.5) / 65536))) (65536
equiprobable standard-normal quantiles, tails cut at about +-4.3 sigma).

Workload shapes follow the five synthetic configurations the library is
measured on; see ``WORKLOADS``.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

PAGE = 16
HEAD_DIM = 128
_GOLDEN = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1


def _s64(c):
    """Unsigned 64-bit constant -> the signed int64 with the same bits."""
    c &= _M64
    return c - (1 << 64) if c >= (1 << 63) else c


def _srl(z, s):
    """Logical right shift of an int64 tensor (torch's >> is arithmetic)."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def mix64(z):
    """splitmix64 output mix on an int64 tensor (bits as unsigned)."""
    z = (z ^ _srl(z, 30)) * _s64(_C1)
    z = (z ^ _srl(z, 27)) * _s64(_C2)
    return z ^ _srl(z, 31)


def mix64_int(z):
    """The same mix on a Python int (used to derive stream keys)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * _C1) & _M64
    z = ((z ^ (z >> 27)) * _C2) & _M64
    return z ^ (z >> 31)


def splitmix64_stream(key, start, count, device="cpu"):
    """Outputs start .. start+count-1 of the splitmix64 stream with this key,
    as int64 tensors holding the unsigned bits."""
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return mix64(i * _s64(_GOLDEN) + _s64(key))


def stream_key(*parts):
    """Fold a tuple of small non-negative ints into one 64-bit stream key."""
    k = 0x5DEECE66D
    for p in parts:
        k = mix64_int(k ^ ((int(p) + 1) * _GOLDEN))
    return k


def _normal_table_bits():
    from scipy.special import ndtri
    q = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
    b = q.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16          # fp32 -> bf16, ties to even
    return b.astype(np.int64).astype(np.int16)


_TABLE_CPU = None
_TABLE_DEV = {}


def normal_table(device="cpu"):
    """The 65536-entry bf16 standard-normal quantile table (int16 bit patterns)."""
    global _TABLE_CPU
    if _TABLE_CPU is None:
        _TABLE_CPU = torch.from_numpy(_normal_table_bits())
    dev = torch.device(device)
    if dev.type == "cpu":
        return _TABLE_CPU
    key = str(dev)
    if key not in _TABLE_DEV:
        _TABLE_DEV[key] = _TABLE_CPU.to(dev)
    return _TABLE_DEV[key]


def normal_bf16(key, start, count, device="cpu"):
    """Elements start .. start+count-1 of the normal stream with this key, as
    bf16 bit patterns (torch.int16).  Element e uses 16-bit field e % 4 of
    splitmix64 output e // 4."""
    c0 = start // 4
    c1 = (start + count + 3) // 4
    z = splitmix64_stream(key, c0, c1 - c0, device)
    f = torch.stack([_srl(z, 16 * j) & 0xFFFF for j in range(4)], dim=1).reshape(-1)
    f = f[start - 4 * c0: start - 4 * c0 + count]
    return normal_table(device)[f]


def bf16_bits_to_float(bits):
    """int16 bf16 patterns -> float32 tensor (exact)."""
    return (bits.to(torch.int32) << 16).view(torch.float32)


def float_to_bf16_bits(x):
    """float tensor -> bf16 bit patterns (int16), via fp32 with ties to even."""
    return x.to(torch.float32).to(torch.bfloat16).view(torch.int16)


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """One synthetic decode-step workload."""
    name: str
    index: int
    batch: int
    q_heads: int
    kv_heads: int
    layers: int
    ctx: tuple            # ("fixed", L) | ("uniform", lo, hi)
    alpha: tuple          # ("fixed", a) | ("choice", (..)) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    targets: tuple        # ("fixed", t) | ("uniform", lo, hi)
    gammas: tuple = (0.99,)
    scale: float = 1.0 / math.sqrt(128.0)
    extra: dict = field(default_factory=dict, hash=False, compare=False)

    @property
    def group(self):
        return self.q_heads // self.kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 8, 2, 1, ("fixed", 4096), ("fixed", 2.0), ("fixed", 4)),
    "llama8b_32k": Workload("llama8b_32k", 1, 8, 32, 8, 1, ("fixed", 32768),
                            ("choice", (0.5, 1.0, 2.0, 4.0)), ("uniform", 1, 64)),
    "long_128k": Workload("long_128k", 2, 4, 32, 8, 32, ("fixed", 131072),
                          ("uniform", 0.25, 4.0), ("fixed", 4), gammas=(0.99, 0.98)),
    "serving_b64": Workload("serving_b64", 3, 64, 32, 8, 1, ("uniform", 4096, 131072),
                            ("loguniform", 0.25, 8.0), ("fixed", 4)),
    "host_tier_512k": Workload("host_tier_512k", 4, 16, 32, 8, 1, ("fixed", 524288),
                               ("uniform", 0.25, 4.0), ("fixed", 4),
                               extra={"capacity": 4096, "steps": 64, "drift": 0.10,
                                      "list_pages": 448}),
    # the host tier over several layers that share their page lists
    "host_tier_layers": Workload("host_tier_layers", 5, 16, 32, 8, 4, ("fixed", 131072),
                                 ("uniform", 0.25, 4.0), ("fixed", 4),
                                 extra={"capacity": 4096, "steps": 32, "drift": 0.10,
                                        "list_pages": 448}),
}


def custom_workload(name, batch, q_heads, kv_heads, ctx, layers=1, alpha=("fixed", 2.0),
                    targets=("fixed", 4), gammas=(0.99,), index=99):
    """A small workload of the same construction (used for parity tests)."""
    return Workload(name, index, batch, q_heads, kv_heads, layers, ctx, alpha, targets, gammas)


def _rng(w, *parts, seed=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.index, *parts])))


def context_lengths(w, seed=0):
    """Per-request context lengths (tokens)."""
    if w.ctx[0] == "fixed":
        return np.full(w.batch, w.ctx[1], dtype=np.int64)
    lo, hi = w.ctx[1], w.ctx[2]
    return _rng(w, 7, seed=seed).integers(lo, hi + 1, size=w.batch).astype(np.int64)


def pages_of(L):
    return (int(L) + PAGE - 1) // PAGE


def valid_tokens(L):
    """Valid tokens of each logical page of a context of L tokens."""
    n = pages_of(L)
    v = np.full(n, PAGE, dtype=np.int64)
    if n:
        v[-1] = int(L) - PAGE * (n - 1)
    return v


def unit_params(w, layer, b, h, n_pages, seed=0):
    """(alpha, target pages) of one (layer, request, KV head) unit."""
    r = _rng(w, 1, layer, b, h, seed=seed)
    a = w.alpha
    if a[0] == "fixed":
        alpha = float(a[1])
    elif a[0] == "choice":
        alpha = float(a[1][int(r.integers(0, len(a[1])))])
    elif a[0] == "uniform":
        alpha = float(r.uniform(a[1], a[2]))
    else:
        alpha = float(math.exp(r.uniform(math.log(a[1]), math.log(a[2]))))
    t = w.targets
    nt = int(t[1]) if t[0] == "fixed" else int(r.integers(t[1], t[2] + 1))
    nt = max(1, nt) if n_pages > 0 else 0
    nt = min(nt, n_pages)
    targets = np.sort(r.choice(n_pages, size=nt, replace=False))
    return alpha, targets


def kv_key(w, layer, b, h, which, seed=0):
    """Stream key of the K (which=0) or V (which=1) tokens of one unit."""
    return stream_key(seed, w.index, layer, b, h, which)


def unit_kv_bits(w, layer, b, h, n_pages, which, pages=None, device="cpu", seed=0):
    """Token-major K or V tiles [len(pages)][P][D] (bf16 bits) of one unit.
    Page p's tile is elements [p*P*D, (p+1)*P*D) of the unit's stream."""
    key = kv_key(w, layer, b, h, which, seed)
    if pages is None:
        return normal_bf16(key, 0, n_pages * PAGE * HEAD_DIM, device).view(n_pages, PAGE, HEAD_DIM)
    tiles = [normal_bf16(key, int(p) * PAGE * HEAD_DIM, PAGE * HEAD_DIM, device) for p in pages]
    return torch.stack(tiles).view(len(tiles), PAGE, HEAD_DIM)


def unit_query_bits(w, layer, b, h, L, seed=0):
    """Queries of the unit's G heads: q_j = alpha * mean(valid keys of the
    target pages) + N(0,1) noise drawn per query head, rounded to bf16.
    Returns int16 [G][D]."""
    n = pages_of(L)
    alpha, targets = unit_params(w, layer, b, h, n, seed)
    if len(targets):
        kt = bf16_bits_to_float(unit_kv_bits(w, layer, b, h, n, 0, pages=targets, seed=seed)).double()
        nv = valid_tokens(L)[targets]
        rows = torch.cat([kt[i, :int(nv[i])] for i in range(len(targets))], 0)
        mu = rows.mean(0)
    else:                                   # empty context: noise only
        mu = torch.zeros(HEAD_DIM, dtype=torch.float64)
    noise = torch.from_numpy(_rng(w, 2, layer, b, h, seed=seed).standard_normal((w.group, HEAD_DIM)))
    return float_to_bf16_bits(alpha * mu[None, :] + noise)


def page_placement(w, layer, lens, seed=0):
    """Physical page ids: a seeded permutation of the layer's pool, assigned
    to (request, logical page) in order.  Returns (page_table [B][max_pages]
    int32 with -1 past each context, pool_pages, max_pages)."""
    n = np.array([pages_of(L) for L in lens], dtype=np.int64)
    max_pages = int(n.max())
    total = int(n.sum())
    perm = _rng(w, 3, layer, seed=seed).permutation(total).astype(np.int32)
    table = np.full((w.batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(w.batch):
        table[b, :n[b]] = perm[off:off + n[b]]
        off += int(n[b])
    return table, total, max_pages


@dataclass
class LayerInputs:
    """One layer's device inputs in the library's layouts."""
    kv_pool: torch.Tensor       # int16 [Ppool][Hkv][2][P*D]: K token-major, V channel-major
    page_table: torch.Tensor    # int32 [B][max_pages]
    ctx_lens: torch.Tensor      # int32 [B]
    q: torch.Tensor             # int16 [B][Hq][D]
    page_valid: torch.Tensor    # int32 [Ppool] valid tokens of each physical page
    max_pages: int
    pool_pages: int


def build_layer(w, layer, device, seed=0, lens=None):
    """Generate one layer's pool, page table, lengths and queries on ``device``."""
    if lens is None:
        lens = context_lengths(w, seed)
    table, total, max_pages = page_placement(w, layer, lens, seed)
    H = w.kv_heads
    pool = torch.empty((total, H, 2, PAGE * HEAD_DIM), dtype=torch.int16, device=device)
    page_valid = np.zeros(total, dtype=np.int32)
    q = torch.empty((w.batch, w.q_heads, HEAD_DIM), dtype=torch.int16)
    for b in range(w.batch):
        n = pages_of(lens[b])
        phys = torch.from_numpy(table[b, :n].astype(np.int64)).to(device)
        page_valid[table[b, :n]] = valid_tokens(lens[b])
        for h in range(H):
            q[b, h * w.group:(h + 1) * w.group] = unit_query_bits(w, layer, b, h, lens[b], seed)
            if n == 0:
                continue
            k = unit_kv_bits(w, layer, b, h, n, 0, device=device, seed=seed)
            v = unit_kv_bits(w, layer, b, h, n, 1, device=device, seed=seed)
            pool[phys, h, 0] = k.reshape(n, PAGE * HEAD_DIM)
            pool[phys, h, 1] = v.transpose(1, 2).reshape(n, PAGE * HEAD_DIM)
            del k, v
    return LayerInputs(
        kv_pool=pool,
        page_table=torch.from_numpy(table).to(device),
        ctx_lens=torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(device),
        q=q.to(device),
        page_valid=torch.from_numpy(page_valid).to(device),
        max_pages=max_pages,
        pool_pages=total,
    )


def unit_host(w, layer, b, h, L, seed=0):
    """Everything the oracle needs for one unit, generated on the host:
    K and V tiles [n][P][D] (bf16 bits, token-major), q [G][D] bits and the
    valid tokens per page."""
    n = pages_of(L)
    k = unit_kv_bits(w, layer, b, h, n, 0, seed=seed).numpy()
    v = unit_kv_bits(w, layer, b, h, n, 1, seed=seed).numpy()
    q = unit_query_bits(w, layer, b, h, L, seed).numpy()
    return k, v, q, valid_tokens(L)


# ----------------------------------------------------------------------------
# Host-resident KV tier: host pool and drifting page lists
# ----------------------------------------------------------------------------

def drift_lists(w, n_pages, list_pages, steps, drift, seed=0, sizes=None):
    """Synthetic page lists for the host-tier workload: per (request, KV head)
    a list of `list_pages` distinct logical pages (sizes[b] for request b when
    given); each step replaces round(drift * size) of them, chosen uniformly,
    with pages drawn uniformly from those not in the list.  Returns int32
    [steps][B][Hkv][max size], each list ascending, padded with -1."""
    B, H = w.batch, w.kv_heads
    sizes = [int(list_pages)] * B if sizes is None else [int(x) for x in sizes]
    out = np.full((steps, B, H, max(sizes)), -1, dtype=np.int32)
    for b in range(B):
        size = sizes[b]
        k = int(round(drift * size))
        for h in range(H):
            r = _rng(w, 5, b, h, seed=seed)
            cur = r.choice(n_pages, size=size, replace=False)
            for t in range(steps):
                out[t, b, h, :size] = np.sort(cur)
                drop = r.choice(size, size=k, replace=False)
                keep = np.delete(cur, drop)
                pool = np.setdiff1d(np.arange(n_pages), cur)
                cur = np.concatenate([keep, r.choice(pool, size=k, replace=False)])
    return out


def spread_sizes(batch, list_pages, spread):
    """Per-request list lengths from list_pages * (1 - spread) up to
    list_pages * (1 + spread), evenly over the requests (mean list_pages)."""
    if batch == 1 or spread == 0:
        return [int(list_pages)] * batch
    return [int(round(list_pages * (1 + spread * (2 * b / (batch - 1) - 1))))
            for b in range(batch)]


def build_host_pool(w, layer=0, seed=0, lens=None, device="cuda"):
    """The full KV history in pinned host memory, layout
    [B][max_pages][Hkv][2][P*D] (K tile token-major, then V tile
    channel-major), generated on `device` one request at a time."""
    if lens is None:
        lens = context_lengths(w, seed)
    max_pages = int(max(pages_of(L) for L in lens))
    H = w.kv_heads
    host = torch.empty((w.batch, max_pages, H, 2, PAGE * HEAD_DIM), dtype=torch.int16,
                       pin_memory=True)
    for b in range(w.batch):
        n = pages_of(lens[b])
        dev = torch.zeros((max_pages, H, 2, PAGE * HEAD_DIM), dtype=torch.int16, device=device)
        for h in range(H):
            if n == 0:
                continue
            k = unit_kv_bits(w, layer, b, h, n, 0, device=device, seed=seed)
            v = unit_kv_bits(w, layer, b, h, n, 1, device=device, seed=seed)
            dev[:n, h, 0] = k.reshape(n, PAGE * HEAD_DIM)
            dev[:n, h, 1] = v.transpose(1, 2).reshape(n, PAGE * HEAD_DIM)
            del k, v
        host[b].copy_(dev)
        del dev
    return host, max_pages
