"""Benchmark of the sparse paged decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long_128k] [--gamma 0.99]

A step is one pass of the whole hot path -- for every layer: page scoring,
coverage selection, self-planning split-K attention and the split merge --
over one batch of synthetic, HBM-resident inputs, captured as one HIP graph.
Default workload: 4 requests of 131072 tokens, Llama-3-8B layer shape (32 query
heads / 8 KV heads, head_dim 128, 16-token pages), 32 independent seeded
layers, gamma 0.99.

Prints ONE JSON line.  `value` is the achieved HBM throughput in GB/s on the
bytes the step must move (page summaries, logits, page lists, the selected K/V
tokens, split partials, queries and outputs -- counted from the device's own
page counts); `us_per_layer` is the step time divided by the layers.
`roofline` covers the attention kernel (the dominant one), timed with HIP
events on its own stream; `cpu_baseline` times the fp64 oracle on layer 0 of
the same workload over the host's cores (one process per core), with the
one-thread figure beside it.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PAGE, D = 16, 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_128k")
    ap.add_argument("--gamma", type=float, default=0.99)
    ap.add_argument("--workers", type=int, default=0,
                    help="attention workgroups (default 0: one per compute unit); the step's "
                         "list entries are split evenly over them on the device")
    ap.add_argument("--groups", type=int, default=1,
                    help="request groups pipelined on separate streams")
    ap.add_argument("--layers", type=int, default=0, help="override the workload's layer count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", default="split", choices=("split", "one_pass"),
                    help="host tier: split = attention over the hits beside the fetch of the "
                         "misses (default); one_pass = resolve and fetch, then one attention")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="oracle processes for the multi-core CPU baseline (default: the "
                         "usable host cores, at most 16)")
    ap.add_argument("--cache-policy", default="exact",
                    help="host tier: exact | bucketed:S | pooled | pooled:S")
    ap.add_argument("--list-spread", type=float, default=0.0,
                    help="host tier: per-request list lengths spread +-f around the mean")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="only launch what the hardware-counter runs measure")
    return ap.parse_args()


def plan_segments(counts, workers, min_pages, unit_cost, cap=None):
    """Partials each unit's list is split into by the attention's balanced
    plan (the formulas of sparse_decode_attn in include/sparse_paged.h): a
    unit of k > 0 entries takes unit_cost + k positions (its entries are the
    last k), the units laid end to end, T positions over W' = min(workers,
    ceil(T / min_pages)) workers, worker w owning [floor(w T / W'),
    floor((w+1) T / W')).  Returns int64 [U]: the number of workers each
    unit's entries fall to."""
    k = np.asarray(counts, dtype=np.int64).clip(min=0)
    if cap is not None:
        k = np.minimum(k, cap)
    p = np.where(k > 0, k + int(unit_cost), 0)
    T = int(p.sum())
    out = np.zeros(k.shape[0], dtype=np.int64)
    if T == 0:
        return out
    W = min(int(workers), -(-T // int(min_pages)))
    off = np.concatenate([[0], np.cumsum(p)[:-1]])
    owner = lambda x: ((x + 1) * W - 1) // T
    nz = k > 0
    out[nz] = owner(off[nz] + p[nz] - 1) - owner(off[nz] + int(unit_cost)) + 1
    return out


def counted_bytes(n, k, tsel, G, Hkv, nseg):
    """Algorithmic bytes of one unit: n pages, k kept, tsel kept valid tokens,
    its list split into nseg attention partials."""
    return (512 * n                 # page summaries (kmin|kmax bf16)
            + 2 * 4 * G * n         # fp32 logits written and read
            + 4 * n / Hkv           # the request's page-table row, shared by its KV heads
            + 512 * tsel            # kept K and V tokens (bf16)
            + 16 * k                # kept logical/physical ids written and read
            + 2 * nseg * G * (D + 1) * 4                   # split partials written and read
            + 2 * G * D * 2 + G * D * 4 + G * 4)           # q read twice, out, lse


def attn_bytes(k, tsel, G, nseg):
    """Algorithmic bytes of the attention kernel alone for one unit."""
    return 512 * tsel + 8 * k + G * D * 2 + nseg * G * (D + 1) * 4


def kept_tokens(counts, pages, lens, Hkv, max_pages):
    U = counts.shape[0]
    tsel = np.zeros(U, dtype=np.int64)
    for u in range(U):
        b = u // Hkv
        k = int(counts[u])
        p = pages[u, :k].astype(np.int64)
        tsel[u] = np.minimum(PAGE, lens[b] - PAGE * p).clip(min=0).sum()
    return tsel


def read_ceiling(lib, pool, nblocks, reps, kept=None):
    """Read rate of one layer's KV pool in whole 8 KiB (page, KV head) blocks,
    the attention's access unit, with nothing else to do: in a seeded random
    order (the practical ceiling for the attention kernel) and in address
    order (the streaming-read ceiling), over the whole pool.  With `kept`,
    also `kept` distinct random blocks: a launch of the attention's own size,
    with the same share of start-up and drain.  HIP events around each
    launch."""
    import torch
    rng = np.random.default_rng(1234)
    perm = rng.permutation(nblocks)
    out = {}
    probes = [("random_8k_blocks_gbs", perm), ("sequential_8k_blocks_gbs", np.arange(nblocks))]
    if kept is not None and 0 < kept < nblocks:
        probes.append(("random_kept_blocks_gbs", perm[:kept]))
    for name, ids in probes:
        order = torch.from_numpy(ids.astype(np.int32)).cuda()
        sink = torch.empty(lib.READ_BLOCKS_GROUPS, dtype=torch.int32, device="cuda")
        lib.read_blocks(pool, nblocks, order, sink)
        marks = []
        for _ in range(max(reps, 3)):
            a, b = TimingEvent(), TimingEvent()
            a.record()
            lib.read_blocks(pool, nblocks, order, sink)
            b.record()
            marks.append((a, b))
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in marks]))
        out[name] = round(len(ids) * 8192 / (us * 1e-6) / 1e9, 1)
    out["bytes_per_launch"] = int(nblocks * 8192)
    if "random_kept_blocks_gbs" in out:
        out["kept_blocks"] = int(kept)
    return out


class TimingEvent:
    """A HIP timing event (the API of torch.cuda.Event(enable_timing=True))
    created with hipEventDisableSystemFence: a default event's record also
    writes back and invalidates the caches for the host, which puts about
    5 us of GPU time inside every interval it bounds.  These events only
    carry timestamps; the host reads nothing else through them."""

    _hip = None
    _DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            # the HIP runtime torch loaded (one copy per process, by its soname)
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        self._ct = ctypes
        self._ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self._ev),
                                               ctypes.c_uint(self._DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream=None):
        import torch
        s = torch.cuda.current_stream() if stream is None else stream
        rc = self._hip.hipEventRecord(self._ev, self._ct.c_void_p(s.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if getattr(self, "_ev", None) is not None and self._ev.value:
            self._hip.hipEventDestroy(self._ev)


def library_source_hash():
    """sha256 (first 16 hex digits) over the library's sources: the C ABI
    header and every file under csrc/, in name order."""
    csrc = os.path.join(ROOT, "adaptive_sparse_paged_amd", "csrc")
    files = [os.path.join(ROOT, "include", "sparse_paged.h")]
    files += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))
              if f.endswith((".hip", ".h"))]
    return source_hash(*files)


# attn.hip and the headers it includes (the C ABI header holds constants the
# kernel uses), in this order, relative to the repository root
ATTN_SOURCES = ("adaptive_sparse_paged_amd/csrc/attn.hip", "adaptive_sparse_paged_amd/csrc/common.h",
                "adaptive_sparse_paged_amd/csrc/fetch.h", "include/sparse_paged.h")


def source_hash(*paths):
    """First 16 hex digits of the sha256 over the given sources, in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one_thread():
    """Limit this process's BLAS / OpenMP / torch pools to one thread."""
    import torch
    torch.set_num_threads(1)
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:                      # pragma: no cover
        return None


def _oracle_unit_inputs(w, b, h, L):
    """One unit of layer 0 generated on the host (untimed): bf16 bits of q and
    the summaries, fp64 K, V, q, and the valid tokens per page."""
    import oracle as O
    from adaptive_sparse_paged_amd import inputs as I
    k, v, q, nv = I.unit_host(w, 0, b, h, L)
    lo, hi = O.summaries(k, nv)            # prefill-time, not timed
    return dict(q=q, lo=lo, hi=hi, nv=nv, qf=O.bf16_bits_to_f64(q), Kf=O.bf16_bits_to_f64(k),
                Vf=O.bf16_bits_to_f64(v))


def _oracle_step(w, un, gamma):
    """The timed oracle work for one unit: score, masses, cut, attention."""
    import oracle as O
    sel = O.select_unit(un["q"], un["lo"], un["hi"], un["nv"], w.scale, gamma)
    O.attend_pages(un["qf"], un["Kf"], un["Vf"], un["nv"], sel["list"], w.scale)
    return sel


def cpu_baseline(w, lens, gamma, budget_s):
    """Time the fp64 oracle (score, masses, cut, attention) on every
    (request, KV head) unit of layer 0, on one host thread.  Each unit is
    generated once (untimed) and its oracle call repeated R times, with R
    chosen from the first unit so the timed total is about budget_s; the mean
    per-unit time is scaled to one layer."""
    limiter = _one_thread()
    n_units = w.batch * w.kv_heads
    spent, calls, reps = 0.0, 0, None
    t_total = time.time()
    for b in range(w.batch):
        for h in range(w.kv_heads):
            un = _oracle_unit_inputs(w, b, h, int(lens[b]))
            r = 0
            while reps is None or r < reps:
                t0 = time.perf_counter()
                _oracle_step(w, un, gamma)
                dt = time.perf_counter() - t0
                spent += dt
                calls += 1
                r += 1
                if reps is None:
                    reps = int(min(16, max(1, round(budget_s / (dt * n_units)))))
            del un
            if time.time() - t_total > 8 * budget_s:
                break
        if time.time() - t_total > 8 * budget_s:
            break
    if limiter is not None:
        limiter.unregister()
    units = -(-calls // reps)
    us_layer = spent / calls * n_units * 1e6
    return {"value": round(us_layer, 1), "unit": "us/layer", "cores": 1, "kind": "oracle",
            "sample": f"{units} of {n_units} (request, KV head) units of layer 0, each run "
                      f"{reps} times: {spent:.1f} s of fp64 NumPy on one host thread, "
                      f"mean per unit scaled to one layer"}


def _pool_worker(w, lens, gamma, units, reps, barrier, results):
    """One oracle process of the multi-core baseline: generate its units
    (untimed), wait for every process, then run the oracle on its units reps
    times and report the elapsed time."""
    _one_thread()
    prepared = [_oracle_unit_inputs(w, b, h, int(lens[b])) for b, h in units]
    barrier.wait()
    t0 = time.perf_counter()
    for _ in range(reps):
        for un in prepared:
            _oracle_step(w, un, gamma)
    results.put(time.perf_counter() - t0)


def host_cores():
    """Host cores this process may run on, at most 16 (one GPU's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:                 # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_pool(w, lens, gamma, budget_s, procs):
    """The same oracle on every unit of layer 0, spread over `procs` processes
    (one thread each, units dealt round robin), all starting together once
    their inputs are generated; one layer's time is the slowest process's
    elapsed time over reps repetitions of its units, divided by reps.  reps
    is set so that the run takes about budget_s.  Processes are forked, so
    this must run before the process touches the GPU."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    procs = max(1, min(procs, len(units)))
    share = [units[i::procs] for i in range(procs)]
    # one calibration unit on this thread sets the repetition count
    limiter = _one_thread()
    un = _oracle_unit_inputs(w, *units[0], int(lens[units[0][0]]))
    t0 = time.perf_counter()
    _oracle_step(w, un, gamma)
    per_unit = time.perf_counter() - t0
    del un
    if limiter is not None:
        limiter.unregister()
    per_rep = per_unit * max(len(x) for x in share)
    reps = int(min(64, max(1, round(budget_s / per_rep))))
    barrier = ctx.Barrier(procs)
    results = ctx.Queue()
    ps = [ctx.Process(target=_pool_worker, args=(w, lens, gamma, share[i], reps, barrier,
                                                 results)) for i in range(procs)]
    for p in ps:
        p.start()
    times = [results.get() for _ in ps]
    for p in ps:
        p.join()
    layer_s = max(times) / reps
    return {"value": round(layer_s * 1e6, 1), "unit": "us/layer", "cores": procs,
            "kind": "oracle",
            "sample": f"all {len(units)} (request, KV head) units of layer 0 over {procs} "
                      f"processes (one thread each), {reps} repetitions: slowest process "
                      f"{max(times):.1f} s, per repetition = one layer"}


def oracle_check(w, lens, gamma, gpu):
    """Untimed check of what the timed run produced for layer 0, unit by
    unit against the oracle: gpu = (counts, pages, out).  Lists accepted by
    the coverage predicate, lists equal to the oracle's, and the max-abs
    error of attention on the GPU's own list."""
    import oracle as O
    counts, pages, out = gpu
    chk = {"units": 0, "accepted": 0, "exact": 0, "max_abs_err": 0.0}
    for b in range(w.batch):
        for h in range(w.kv_heads):
            un = _oracle_unit_inputs(w, b, h, int(lens[b]))
            sel = O.select_unit(un["q"], un["lo"], un["hi"], un["nv"], w.scale, gamma)
            u = b * w.kv_heads + h
            lst = pages[u, :int(counts[u])]
            ok, _ = O.list_accepted(lst, sel["m"], gamma, 1e-5)
            chk["units"] += 1
            chk["accepted"] += int(ok)
            chk["exact"] += int(len(lst) == sel["count"] and np.array_equal(lst, sel["list"]))
            o_ref, _ = O.attend_pages(un["qf"], un["Kf"], un["Vf"], un["nv"], lst, w.scale)
            o_gpu = out[b, h * w.group:(h + 1) * w.group].astype(np.float64)
            chk["max_abs_err"] = max(chk["max_abs_err"], float(np.abs(o_gpu - o_ref).max()))
            del un
    chk["max_abs_err"] = float(f"{chk['max_abs_err']:.3g}")
    chk["what"] = ("layer 0 of the timed run against the fp64 oracle: lists accepted by the "
                   "coverage predicate (1e-5 relative mass), lists equal to the oracle's, "
                   "max-abs error of attention on the GPU's lists (bar 1e-2)")
    return chk


# GPU clock cycles of the wait that lets the host run ahead of the all-hit
# steps (tens of milliseconds)
ALLHIT_HOST_LEAD_CYCLES = 100_000_000


def host_tier_bench(args):
    """Host-resident KV tier: 16 requests x 524288 tokens of bf16 KV in pinned
    host memory (32 GiB), a 4096-slot HBM cache per request, page lists of 448
    pages per (request, KV head) drifting 10% per step over 64 steps, each
    step timed with HIP events.  Schedule "split" (default): resolve, then the
    fetch of the misses (attended by the waves that copy them) beside
    attention over the hits, then one merge of both.  Schedule "one_pass": resolve
    and fetch, then attention + merge over whole lists, with the two phases
    timed apart.  Either way, then steps with every access a hit (no host
    IO), timed on the device: the one-pass resolve against its attention +
    merge, and with the split schedule the split step against the one-pass
    step.  Also the pinned host-to-device copy rate of the link for
    reference."""
    import torch
    from adaptive_sparse_paged_amd import inputs as I
    from adaptive_sparse_paged_amd import lib
    from adaptive_sparse_paged_amd.host_tier import HbmPageCache, SplitHostTierStep
    from adaptive_sparse_paged_amd.step import SparseDecodeStep

    lib.load()
    w = I.WORKLOADS["host_tier_512k"]
    ex = w.extra
    lens = I.context_lengths(w)
    t0 = time.time()
    host, MP = I.build_host_pool(w, 0, lens=lens)
    print(f"# host pool {host.numel() * 2 / 2**30:.0f} GiB pinned ({time.time() - t0:.0f} s)",
          file=sys.stderr, flush=True)
    steps, LP, C = ex["steps"], ex["list_pages"], ex["capacity"]
    B, H = w.batch, w.kv_heads
    U = B * H
    sizes = I.spread_sizes(B, LP, args.list_spread)
    lists = I.drift_lists(w, I.pages_of(lens[0]), LP, steps, ex["drift"], sizes=sizes)
    LM = lists.shape[-1]
    # every list holds at most LM pages: the attention plans for that
    dims = lib.make_dims(B, w.q_heads, H, MP, max_list_pages=LM)
    name, _, sh = args.cache_policy.partition(":")
    if name not in ("exact", "bucketed", "pooled"):
        raise SystemExit(f"unknown cache policy {args.cache_policy}")
    shift = int(sh or 0)
    pooled = name == "pooled"
    cap = B * C if pooled else C          # the same HBM either way
    cache = HbmPageCache(dims, host, cap, recency_shift=shift, pooled=pooled)
    st = SparseDecodeStep(dims, args.gamma, args.workers, scale=w.scale, scoring=False)
    q = torch.empty((B, w.q_heads, D), dtype=torch.int16)
    for b in range(B):
        for h in range(H):
            q[b, h * w.group:(h + 1) * w.group] = I.unit_query_bits(w, 0, b, h, int(lens[b]))
    q = q.cuda()
    ctx = torch.from_numpy(lens.astype(np.int32)).cuda()
    lists_dev = torch.from_numpy(lists.reshape(steps, U, LM)).cuda()
    counts0 = torch.tensor([sizes[u // H] for u in range(U)], dtype=torch.int32)
    st.buf.sel_counts.copy_(counts0)
    kv, s_page, s_head, ppages = cache.pool_args()
    spl = None
    if args.schedule == "split":
        spl = SplitHostTierStep(dims, cache, args.gamma, args.workers, scale=w.scale)
        spl.sel_counts.copy_(counts0)
        out_s = torch.empty((B, w.q_heads, D), dtype=torch.float32, device="cuda")
        lse_s = torch.empty((B, w.q_heads), dtype=torch.float32, device="cuda")

    def run_one(t, marks, phases=True):
        """phases=False: no event between the resolve and the attention (the
        step as it runs), e[0] -> e[1] is the whole step."""
        e = [TimingEvent() for _ in range(3)]
        st.buf.sel_pages[:, :LM].copy_(lists_dev[t])
        e[0].record()
        cache.resolve(st.buf.sel_counts, st.buf.sel_pages, st.buf.sel_phys)
        if phases:
            e[1].record()
        st.attend(q, kv, s_page, s_head, ppages, ctx)
        if not phases:
            e[1].record()
        e[2].record()
        marks.append(e)

    def run_split(t, marks):       # the phases overlap: only the whole step is timed
        e = [TimingEvent() for _ in range(3)]
        spl.sel_pages[:, :LM].copy_(lists_dev[t])
        e[0].record()
        spl.run(q, ctx, out_s, lse_s)
        e[1].record()
        e[2].record()
        marks.append(e)

    run_step = run_one if spl is None else run_split

    marks, stats = [], []
    for t in range(steps):
        run_step(t, marks)
        stats.append(cache.stats.clone())
    torch.cuda.synchronize()
    res_us = np.array([m[0].elapsed_time(m[1]) * 1e3 for m in marks])
    att_us = np.array([m[1].elapsed_time(m[2]) * 1e3 for m in marks])
    st_np = np.stack([s.cpu().numpy() for s in stats])          # [steps][B][4]
    hits, misses = st_np[:, :, 0].sum(1), st_np[:, :, 1].sum(1)
    overflow = int(st_np[:, :, 3].max())
    unit_bytes = 2 * 16 * 128 * 2
    h2d = misses[1:] * unit_bytes / (res_us[1:] * 1e-6) / 1e9
    # all-hit steps (no host IO): the last list again, after it is resident.
    # The GPU first runs a wait long enough for the host to enqueue every
    # step below, so the events time the device alone (an all-hit step is
    # shorter than the host's launches for it).  With the split schedule the
    # one-pass step runs after each split step, on the same cache.
    t_last = steps - 1
    torch.cuda.synchronize()
    torch.cuda._sleep(ALLHIT_HOST_LEAD_CYCLES)
    allhit, allhit_one, allhit_whole = [], [], []
    for k in range(args.steps):
        if spl is not None:
            run_split(t_last, allhit)
        run_one(t_last, allhit_one)
        run_one(t_last, allhit_whole, phases=False)
    torch.cuda.synchronize()
    allhit_res = np.array([m[0].elapsed_time(m[1]) * 1e3 for m in allhit_one])
    allhit_att = np.array([m[1].elapsed_time(m[2]) * 1e3 for m in allhit_one])
    allhit_step = np.array([m[0].elapsed_time(m[1]) * 1e3 for m in allhit_whole])
    if overflow == 0:           # with overflow some units can never be resident
        assert int(cache.stats[:, 1].sum().item()) == 0
    # the link: pinned host -> device copy of 1 GiB
    src = host.view(-1)[: 512 * 1024 * 1024]
    dst = torch.empty(src.shape, dtype=src.dtype, device="cuda")
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = TimingEvent(), TimingEvent()
    c0.record()
    dst.copy_(src, non_blocking=True)
    c1.record()
    torch.cuda.synchronize()
    link = src.numel() * 2 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    step_us = res_us[1:] + att_us[1:]
    kept_bytes = H * sum(sizes) * unit_bytes
    tags = cache.slot_tag.cpu().numpy()
    if pooled:
        held = np.bincount(tags[tags >= 0] // (H * MP), minlength=B)
    else:
        held = (tags >= 0).sum(1)
    result = {
        "metric": "host-tier sparse decode step us (resolve + attention + merge), 4096-slot HBM cache",
        "value": round(float(np.median(step_us)), 1),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps - 1,
        "warmup": 1,
        "ms_per_step": round(float(np.median(step_us)) / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "ctx": int(lens.max()), "kv_heads": H,
                   "q_heads": w.q_heads, "capacity_slots": C, "list_pages": LP,
                   "drift": ex["drift"], "attn_workers": st.max_parts - U,
                   "cache_policy": args.cache_policy, "list_spread": args.list_spread,
                   "list_pages_min_max": [min(sizes), max(sizes)],
                   "schedule": "split" if spl is not None else "one_pass"},
        "cold_step_us": round(float(res_us[0] + att_us[0]), 1),
        "slots_held_min_max": [int(held.min()), int(held.max())],
        "overflow_steps": int((st_np[:, :, 3].max(1) > 0).sum()),
        "resolve_fetch_us_median": round(float(np.median(res_us[1:])), 1),
        "attention_merge_us_median": round(float(np.median(att_us[1:])), 1),
        "hit_rate_steady": round(float(hits[1:].sum() / (hits[1:].sum() + misses[1:].sum())), 4),
        "misses_per_step_median": int(np.median(misses[1:])),
        "h2d_gbs_median": round(float(np.median(h2d)), 1),
        "pinned_copy_gbs": round(link, 1),
        "h2d_frac_of_link": round(float(np.median(h2d)) / link, 3),
        "attention_hbm_gbs": (round(kept_bytes / (float(np.median(att_us[1:])) * 1e-6) / 1e9, 1)
                              if spl is None else None),
        "overflow": overflow,
        "no_io": {"what": "every access a hit, device time: one-pass resolve + fetch and "
                          "attention + merge timed apart, and the one-pass step whole",
                  "resolve_us": round(float(np.median(allhit_res)), 1),
                  "attention_merge_us": round(float(np.median(allhit_att)), 1),
                  "resolve_share": round(float(np.median(allhit_res) /
                                               (np.median(allhit_res) + np.median(allhit_att))), 4),
                  "one_pass_step_us": round(float(np.median(allhit_step)), 1)},
    }
    if spl is not None:
        # the phases overlap: their separate figures do not exist in this schedule
        for k in ("resolve_fetch_us_median", "attention_merge_us_median", "h2d_gbs_median",
                  "h2d_frac_of_link", "attention_hbm_gbs"):
            result[k] = None
        allhit_split = np.array([m[0].elapsed_time(m[1]) * 1e3 for m in allhit])
        one = float(np.median(allhit_step))
        result["no_io"]["split_step_us"] = round(float(np.median(allhit_split)), 1)
        result["no_io"]["split_over_one_pass"] = round(float(np.median(allhit_split)) / one - 1, 4)
    print(json.dumps(result), flush=True)


def host_tier_layers_bench(args):
    """Layer-wise prefetch over the host tier: 16 requests x 131072 tokens,
    4 layers that share their page lists (448 pages per request and KV head,
    drifting 10% per step, 32 steps), each layer with its own pinned host
    pool (8 GiB) and 4096-slot HBM cache per request.  Times every step two
    ways on separate caches fed the same lists: layer by layer on one stream
    (resolve+fetch then attention+merge, with events between the phases) and
    pipelined (all resolves on a second stream, each layer's attention waiting
    for its own layer only)."""
    import torch
    from adaptive_sparse_paged_amd import inputs as I
    from adaptive_sparse_paged_amd import lib
    from adaptive_sparse_paged_amd.host_tier import LayeredHostTierStep

    lib.load()
    w = I.WORKLOADS["host_tier_layers"]
    ex = w.extra
    lens = I.context_lengths(w)
    nl = args.layers or w.layers
    t0 = time.time()
    hosts = [I.build_host_pool(w, l, lens=lens)[0] for l in range(nl)]
    MP = hosts[0].shape[1]
    print(f"# host pools {nl} x {hosts[0].numel() * 2 / 2**30:.0f} GiB pinned "
          f"({time.time() - t0:.0f} s)", file=sys.stderr, flush=True)
    steps, LP, C = ex["steps"], ex["list_pages"], ex["capacity"]
    lists = I.drift_lists(w, I.pages_of(lens[0]), LP, steps, ex["drift"])
    B, H = w.batch, w.kv_heads
    U = B * H
    dims = lib.make_dims(B, w.q_heads, H, MP, max_list_pages=LP)
    seq = LayeredHostTierStep(dims, hosts, C, args.gamma, args.workers, scale=w.scale,
                              prefetch=False)
    pre = LayeredHostTierStep(dims, hosts, C, args.gamma, args.workers, scale=w.scale,
                              prefetch=True)
    qs = []
    for l in range(nl):
        q = torch.empty((B, w.q_heads, D), dtype=torch.int16)
        for b in range(B):
            for h in range(H):
                q[b, h * w.group:(h + 1) * w.group] = I.unit_query_bits(w, l, b, h, int(lens[b]))
        qs.append(q.cuda())
    ctx = torch.from_numpy(lens.astype(np.int32)).cuda()
    lists_dev = torch.from_numpy(lists.reshape(steps, U, LP)).cuda()
    outs = [torch.empty((B, w.q_heads, D), dtype=torch.float32, device="cuda") for _ in range(nl)]
    lses = [torch.empty((B, w.q_heads), dtype=torch.float32, device="cuda") for _ in range(nl)]
    ev = lambda: TimingEvent()
    seq_io, seq_att, pre_step, misses = [], [], [], []
    for t in range(steps):
        for stp in (seq, pre):
            stp.sel_counts.fill_(LP)
            stp.sel_pages[:, :LP].copy_(lists_dev[t])
        # layer by layer, with the phases timed apart
        marks = []
        st = seq.attn
        for l, cache in enumerate(seq.caches):
            e = [ev(), ev(), ev()]
            e[0].record()
            cache.resolve(st.buf.sel_counts, st.buf.sel_pages, seq.sel_phys[l])
            e[1].record()
            kv, sp_, sh_, pp = cache.pool_args()
            st.attend(qs[l], kv, sp_, sh_, pp, ctx, outs[l], lses[l], sel_phys=seq.sel_phys[l])
            e[2].record()
            marks.append(e)
        p0, p1 = ev(), ev()
        p0.record()
        pre.run(qs, ctx, outs, lses)
        p1.record()
        torch.cuda.synchronize()
        seq_io.append(sum(m[0].elapsed_time(m[1]) for m in marks) * 1e3)
        seq_att.append(sum(m[1].elapsed_time(m[2]) for m in marks) * 1e3)
        pre_step.append(p0.elapsed_time(p1) * 1e3)
        misses.append(int(sum(int(c.stats[:, 1].sum()) for c in pre.caches)))
        for a, b_ in zip(seq.caches, pre.caches):
            assert torch.equal(a.stats, b_.stats)
    seq_io, seq_att, pre_step = (np.array(x[1:]) for x in (seq_io, seq_att, pre_step))
    seq_step = seq_io + seq_att
    hide = np.minimum(seq_io, seq_att)
    hidden = (seq_step - pre_step) / hide
    unit_bytes = 2 * PAGE * D * 2
    result = {
        "metric": "host-tier decode step us over 4 layers sharing page lists, layer-wise prefetch",
        "value": round(float(np.median(pre_step)), 1),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps - 1,
        "warmup": 1,
        "ms_per_step": round(float(np.median(pre_step)) / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "ctx": int(lens.max()), "layers": nl,
                   "kv_heads": H, "q_heads": w.q_heads, "capacity_slots": C,
                   "list_pages": LP, "drift": ex["drift"],
                   "attn_workers": seq.attn.max_parts - U},
        "sequential_step_us_median": round(float(np.median(seq_step)), 1),
        "sequential_resolve_fetch_us_median": round(float(np.median(seq_io)), 1),
        "sequential_attention_merge_us_median": round(float(np.median(seq_att)), 1),
        "prefetch_saving_us_median": round(float(np.median(seq_step - pre_step)), 1),
        "hidden_frac_of_overlappable_median": round(float(np.median(hidden)), 3),
        "misses_per_step_median": int(np.median(misses[1:])),
        "h2d_gbs_sequential_median": round(float(np.median(
            np.array(misses[1:]) * unit_bytes / (seq_io * 1e-6) / 1e9)), 1),
    }
    print(json.dumps(result), flush=True)


def attn_launch(lib, st, dims, li, stride_page, stride_head):
    """The step's attention launch alone (sparse_decode_attn, without its merge)."""
    b = st.buf
    lib.decode_attn(dims, li.q, li.kv_pool, stride_page, stride_head, li.pool_pages, li.ctx_lens,
                    b.sel_counts, b.sel_pages, b.sel_phys, st.scale, st.workers, b.part_o,
                    b.part_lse, st.max_parts)


def pmc_probe(args):
    """Launches for hardware-counter runs (rocprofv3 --pmc FETCH_SIZE, then
    WRITE_SIZE): a plain device copy of 1 GiB (known bytes, the calibration)
    and the attention kernel on layer 0 of the workload, three times each."""
    import torch
    from adaptive_sparse_paged_amd import inputs as I
    from adaptive_sparse_paged_amd import lib
    from adaptive_sparse_paged_amd.step import SparseDecodeStep, canonical_strides

    lib.load()
    w = I.WORKLOADS[args.workload]
    lens = I.context_lengths(w)
    li = I.build_layer(w, 0, "cuda", lens=lens)
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, li.max_pages)
    sp_, sh_ = canonical_strides(w.kv_heads)
    summ = torch.empty((li.pool_pages, w.kv_heads, 2, D), dtype=torch.int16, device="cuda")
    lib.build_page_summaries(dims, li.kv_pool, sp_, sh_, li.pool_pages,
                             torch.arange(li.pool_pages, dtype=torch.int32, device="cuda"),
                             li.page_valid, summ)
    st = SparseDecodeStep(dims, args.gamma, args.workers, scale=w.scale)
    st.score_select(li.q, summ, li.pool_pages, li.page_table, li.ctx_lens)
    torch.cuda.synchronize()
    c = st.buf.sel_counts.cpu().numpy()
    tsel = kept_tokens(c, st.buf.sel_pages.cpu().numpy(), lens, w.kv_heads, li.max_pages)
    nseg = plan_segments(c, st.max_parts - len(c), lib.ATTN_MIN_WORKER_PAGES,
                         lib.ATTN_UNIT_COST_PAGES)
    ab = sum(attn_bytes(int(c[u]), int(tsel[u]), w.group, int(nseg[u])) for u in range(len(c)))
    for _ in range(3):
        attn_launch(lib, st, dims, li, sp_, sh_)
    src = torch.empty(512 * 1024 * 1024, dtype=torch.int16, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"attn_algorithmic_bytes_per_launch": int(ab),
                      "calibration_copy_bytes_each_way": src.numel() * 2}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path here is single-GPU "
              "(requests and KV heads shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)
    if args.pmc_probe:
        pmc_probe(args)
        return
    if args.workload == "host_tier_512k":
        host_tier_bench(args)
        return
    if args.workload == "host_tier_layers":
        host_tier_layers_bench(args)
        return
    import torch
    from adaptive_sparse_paged_amd import inputs as I
    from adaptive_sparse_paged_amd import lib
    from adaptive_sparse_paged_amd.step import SparseDecodeStep, canonical_strides, capture

    w = I.WORKLOADS[args.workload]
    layers = args.layers or w.layers
    lens = I.context_lengths(w)
    base = None
    if not args.no_cpu_baseline:
        # CPU legs first: the pool forks, which must happen before any GPU use
        procs = args.cpu_procs or host_cores()
        print(f"# oracle baseline: 1 thread, then {procs} processes", file=sys.stderr,
              flush=True)
        single = cpu_baseline(w, lens, args.gamma, args.cpu_seconds)
        base = cpu_baseline_pool(w, lens, args.gamma, args.cpu_seconds, procs)
        base["single_core"] = single
    lib.load()
    dev = "cuda"
    t_gen = time.time()
    L_in, summs = [], []
    for layer in range(layers):
        li = I.build_layer(w, layer, dev, lens=lens)
        dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, li.max_pages)
        sp_, sh_ = canonical_strides(w.kv_heads)
        summ = torch.empty((li.pool_pages, w.kv_heads, 2, D), dtype=torch.int16, device=dev)
        lib.build_page_summaries(dims, li.kv_pool, sp_, sh_, li.pool_pages,
                                 torch.arange(li.pool_pages, dtype=torch.int32, device=dev),
                                 li.page_valid, summ)
        L_in.append(li)
        summs.append(summ)
        if layer % 8 == 7:
            print(f"# generated {layer + 1}/{layers} layers ({time.time() - t_gen:.0f} s)",
                  file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    stride_page, stride_head = canonical_strides(w.kv_heads)
    max_pages = L_in[0].max_pages
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, max_pages)
    groups = max(1, min(args.groups, w.batch))
    st = SparseDecodeStep(dims, args.gamma, args.workers, scale=w.scale, device=dev,
                          groups=groups, offsets=False)
    workers = st.max_parts - w.batch * w.kv_heads
    outs = [torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device=dev) for _ in range(layers)]
    lses = [torch.empty((w.batch, w.q_heads), dtype=torch.float32, device=dev) for _ in range(layers)]
    counts = [torch.empty_like(st.buf.sel_counts) for _ in range(layers)]

    def step_fn():
        for l, li in enumerate(L_in):
            st.run(li.q, summs[l], li.kv_pool, stride_page, stride_head, li.pool_pages,
                   li.page_table, li.ctx_lens, outs[l], lses[l])

    # one eager pass to record the per-layer selections (for byte accounting)
    sel_stats = []
    for l, li in enumerate(L_in):
        st.run(li.q, summs[l], li.kv_pool, stride_page, stride_head, li.pool_pages,
               li.page_table, li.ctx_lens, outs[l], lses[l])
        torch.cuda.synchronize()
        c = st.buf.sel_counts.cpu().numpy()
        pg = st.buf.sel_pages.cpu().numpy()
        sel_stats.append((c, kept_tokens(c, pg, lens, w.kv_heads, max_pages),
                          plan_segments(c, workers, lib.ATTN_MIN_WORKER_PAGES,
                                        lib.ATTN_UNIT_COST_PAGES)))
        if l == 0:
            layer0 = (c.copy(), pg.copy())
    graph = capture(step_fn)

    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        graph.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    per_replay = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    p10, p50, p90 = (float(np.percentile(per_replay, x)) for x in (10, 50, 90))
    # The device's own time per step: the GPU first runs a wait long enough
    # for the host to enqueue every replay, so these events time the device
    # alone.  A step shorter than the host's launch of its graph (the tiny
    # workload) is otherwise timed at the host's launch rate.
    torch.cuda.synchronize()
    torch.cuda._sleep(ALLHIT_HOST_LEAD_CYCLES)
    dv = [TimingEvent() for _ in range(2)]
    dv[0].record()
    for i in range(args.steps):
        graph.replay()
    dv[1].record()
    torch.cuda.synchronize()
    device_ms_step = dv[0].elapsed_time(dv[1]) / args.steps

    # bytes moved per step
    G, Hkv = w.group, w.kv_heads
    npages = np.array([I.pages_of(L) for L in lens])
    total_bytes, attn_total, kept, pages_all = 0.0, 0.0, 0, 0
    for c, tsel, nseg in sel_stats:
        for u in range(c.shape[0]):
            n = int(npages[u // Hkv])
            total_bytes += counted_bytes(n, int(c[u]), int(tsel[u]), G, Hkv, int(nseg[u]))
            attn_total += attn_bytes(int(c[u]), int(tsel[u]), G, int(nseg[u]))
            kept += int(c[u])
            pages_all += n
    gbs = total_bytes / (ms_step * 1e-3) / 1e9

    # attention kernel alone: eager passes over every layer with HIP events
    # around each attention launch, on the stream the launches run on
    stream = torch.cuda.current_stream()
    marks = []
    for _ in range(args.steps):
        for l, li in enumerate(L_in):
            st.score_select(li.q, summs[l], li.pool_pages, li.page_table, li.ctx_lens)
            a0 = TimingEvent()
            a1 = TimingEvent()
            a0.record(stream)
            attn_launch(lib, st, dims, li, stride_page, stride_head)
            a1.record(stream)
            lib.merge_splits(dims, st.buf.part_o, st.buf.part_lse, st.buf.sel_counts,
                             st.workers, outs[l], lses[l])
            marks.append((a0, a1))
    torch.cuda.synchronize()
    attn_us = sum(a.elapsed_time(b) for a, b in marks) * 1e3 / len(marks)
    attn_launch_bytes = 0.0
    for c, tsel, nseg in sel_stats:
        attn_launch_bytes += sum(attn_bytes(int(c[u]), int(tsel[u]), G, int(nseg[u]))
                                 for u in range(c.shape[0]))
    attn_launch_bytes /= layers
    attn_gbs = attn_launch_bytes / (attn_us * 1e-6) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "attn_kernel_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            rec = json.load(f)
        # the attention kernel is compiled from attn.hip and the headers it includes
        src_hash = source_hash(*(os.path.join(ROOT, f) for f in ATTN_SOURCES))
        if (rec.get("source_sha256_16") == src_hash and rec.get("workload") == w.name
                and rec.get("attn_workers") == workers and rec.get("gamma") == args.gamma):
            traffic = rec.get("bytes_per_launch")

    kept_blocks = int(round(sum(int(c.sum()) for c, _, _ in sel_stats) / len(sel_stats)))
    ceiling = read_ceiling(lib, L_in[0].kv_pool, L_in[0].pool_pages * w.kv_heads, args.steps,
                           kept=kept_blocks)

    result = {
        "metric": "sparse decode step \u00b5s/layer + achieved HBM GB/s vs peak at 128k ctx, \u03b3=0.99",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "us_per_layer": round(ms_step * 1e3 / layers, 2),
        "step_ms_p10_p50_p90": [round(p10, 4), round(p50, 4), round(p90, 4)],
        "device_ms_per_step": round(device_ms_step, 4),
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "ctx": int(lens.max()),
                   "layers": layers, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": D, "page_size": PAGE, "gamma": args.gamma,
                   "attn_workers": workers, "stream_groups": groups},
        "selected_fraction": round(kept / pages_all, 4),
        "bytes_per_step": int(total_bytes),
        "roofline": {"kernel": "attn_kernel", "bound": "hbm", "achieved": round(attn_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(attn_us, 2),
                     "bytes_per_launch": int(attn_launch_bytes)},
        "read_ceiling": dict(ceiling,
                             attn_frac_of_random=round(attn_gbs / ceiling["random_8k_blocks_gbs"], 4),
                             value_frac_of_random=round(gbs / ceiling["random_8k_blocks_gbs"], 4)),
    }
    if "random_kept_blocks_gbs" in ceiling:
        result["read_ceiling"]["attn_frac_of_random_kept"] = round(
            attn_gbs / ceiling["random_kept_blocks_gbs"], 4)
    result["env"] = {"hip": torch.version.hip, "library": lib.version(),
                     "device": torch.cuda.get_device_name(0),
                     "sources_sha256_16": library_source_hash()}
    if base is not None:
        torch.cuda.synchronize()
        result["cpu_baseline"] = base
        gpu0 = (layer0[0], layer0[1], outs[0].cpu().numpy())
        result["oracle_check"] = oracle_check(w, lens, args.gamma, gpu0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
