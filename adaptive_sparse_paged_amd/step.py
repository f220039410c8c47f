"""One sparse decode step (score -> select -> attention -> merge) on caller-owned
buffers, and its capture into a single HIP graph.

Buffers are torch tensors (device memory only); every operation is a call into
the HIP library.  The step is captured whole: nothing in it waits on the host,
and the page lists, their lengths and the attention's plan live on the device, so a
captured graph replays correctly after the queries, context lengths or page
tables change in place.
"""

from dataclasses import dataclass

import torch

from . import lib

PAGE = 16
HEAD_DIM = 128


@dataclass
class StepBuffers:
    logits: torch.Tensor        # fp32 [B][Hkv][G][max_pages]
    sel_counts: torch.Tensor    # int32 [U]
    sel_offsets: torch.Tensor   # int32 [U+1]
    sel_pages: torch.Tensor     # int32 [U][max_pages]
    sel_phys: torch.Tensor      # int32 [U][max_pages]
    ws: torch.Tensor            # uint8 workspace (zero-filled once)
    part_o: torch.Tensor        # fp32 [max_parts][G][D], max_parts = U + workers
    part_lse: torch.Tensor      # fp32 [max_parts][G]
    out: torch.Tensor           # fp32 [B][Hq][D]
    out_lse: torch.Tensor       # fp32 [B][Hq]


class SparseDecodeStep:
    """Fixed-shape decode step for one layer shape.

    dims: lib.Dims; gamma in (0, 1]; workers: the attention's grid (0 = one
    workgroup per compute unit of the device).  The attention splits all the
    step's list entries evenly over its workgroups on the device, whatever
    the list lengths, so no per-workload size is needed.  Intermediate
    buffers are shared by every layer run through this object; outputs can
    be given per call.

    groups > 1 splits the requests into that many contiguous groups, each on a
    stream of its own, where a group's scoring starts once the previous group's
    page lists are chosen.  Selection is latency-bound (one workgroup per
    unit) and attention is bandwidth-bound, so this lets one group's selection
    run under another group's attention.  Every unit's arithmetic is the same
    in both modes (bitwise); only the grouped mode leaves the whole-batch
    prefix sum (sel_offsets) unwritten.  Measured on MI355X
    (ROCm 7.2, graph replay) on 4 x 131072 tokens, 32 layers: 376 us/layer
    with one group, 414 with two and 591 with four.  Each group's kernels get
    a fraction of the grid, and the last group's attention has nothing left to
    run beside it, so the default is one group.
    """

    def __init__(self, dims, gamma, workers=0, scale=None, device="cuda", groups=1,
                 offsets=True, scoring=True):
        """offsets: also write the whole-batch prefix sum (sel_offsets) in the
        selection; the attention does not need it.  scoring=False: attention
        over lists the caller writes (sel_counts / sel_pages / sel_phys) only,
        so no logits buffer or selection workspace is allocated."""
        self.dims = dims
        self.offsets = bool(offsets)
        self.gamma = float(gamma)
        self.workers = int(workers)
        self.scale = float(scale if scale is not None else HEAD_DIM ** -0.5)
        B, Hq, Hkv, MP = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.max_pages
        G = Hq // Hkv
        U = B * Hkv
        self.max_parts = lib.decode_max_parts(dims, self.workers)
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.scoring = bool(scoring)
        self.buf = StepBuffers(
            logits=torch.empty((B, Hkv, G, MP) if scoring else (0,), **f32),
            sel_counts=torch.zeros(U, **i32),
            sel_offsets=torch.zeros(U + 1, **i32),
            sel_pages=torch.zeros((U, MP), **i32),
            sel_phys=torch.zeros((U, MP), **i32),
            ws=torch.zeros(lib.select_workspace_bytes(dims) if scoring else 0, dtype=torch.uint8,
                           device=device),
            part_o=torch.empty((self.max_parts, G, HEAD_DIM), **f32),
            part_lse=torch.empty((self.max_parts, G), **f32),
            out=torch.empty((B, Hq, HEAD_DIM), **f32),
            out_lse=torch.empty((B, Hq), **f32),
        )
        self.groups = []
        if groups > 1:
            if not scoring:
                raise ValueError("request groups score and select: scoring=False has none")
            self._make_groups(int(groups), device)

    def _make_groups(self, ngroups, device):
        d, b = self.dims, self.buf
        B, Hkv, G = d.batch, d.num_kv_heads, d.num_q_heads // d.num_kv_heads
        bounds = [round(i * B / ngroups) for i in range(ngroups + 1)]
        for g in range(ngroups):
            b0, b1 = bounds[g], bounds[g + 1]
            if b1 <= b0:
                continue
            dg = lib.make_dims(b1 - b0, d.num_q_heads, Hkv, d.max_pages)
            u0, u1 = b0 * Hkv, b1 * Hkv
            mp = lib.decode_max_parts(dg, self.workers)
            self.groups.append(dict(
                b0=b0, b1=b1, u0=u0, u1=u1, dims=dg, max_parts=mp,
                sel_offsets=torch.zeros(u1 - u0 + 1, dtype=torch.int32, device=device),
                ws=torch.zeros(lib.select_workspace_bytes(dg), dtype=torch.uint8, device=device),
                part_o=torch.empty((mp, G, HEAD_DIM), dtype=torch.float32, device=device),
                part_lse=torch.empty((mp, G), dtype=torch.float32, device=device),
                stream=torch.cuda.Stream(device=device),
                selected=torch.cuda.Event(),
            ))

    def _run_groups(self, q, summ, kv, stride_page, stride_head, pool_pages, page_table,
                    ctx_lens, out, out_lse):
        b = self.buf
        cur = torch.cuda.current_stream()
        prev = None
        for gr in self.groups:
            s = gr["stream"]
            s.wait_stream(cur)
            if prev is not None:
                s.wait_event(prev["selected"])
            b0, b1, u0, u1, dg = gr["b0"], gr["b1"], gr["u0"], gr["u1"], gr["dims"]
            with torch.cuda.stream(s):
                lib.score_pages(dg, q[b0:b1], summ, pool_pages, page_table[b0:b1],
                                ctx_lens[b0:b1], self.scale, b.logits[b0:b1], s)
                on = self.offsets
                lib.select_coverage(dg, b.logits[b0:b1], ctx_lens[b0:b1], page_table[b0:b1],
                                    self.gamma, b.sel_counts[u0:u1],
                                    gr["sel_offsets"] if on else None, b.sel_pages[u0:u1],
                                    b.sel_phys[u0:u1], gr["ws"] if on else None, s)
                gr["selected"].record(s)
                lib.decode_attn(dg, q[b0:b1], kv, stride_page, stride_head, pool_pages,
                                ctx_lens[b0:b1], b.sel_counts[u0:u1], b.sel_pages[u0:u1],
                                b.sel_phys[u0:u1], self.scale, self.workers, gr["part_o"],
                                gr["part_lse"], gr["max_parts"], s)
                lib.merge_splits(dg, gr["part_o"], gr["part_lse"], b.sel_counts[u0:u1],
                                 self.workers, out[b0:b1], out_lse[b0:b1], s)
            prev = gr
        for gr in self.groups:
            cur.wait_stream(gr["stream"])
        return out, out_lse

    def score_select(self, q, summ, pool_pages, page_table, ctx_lens, stream=None):
        if not self.scoring:
            raise ValueError("this step was made with scoring=False")
        d, b = self.dims, self.buf
        lib.score_pages(d, q, summ, pool_pages, page_table, ctx_lens, self.scale, b.logits, stream)
        on = self.offsets
        lib.select_coverage(d, b.logits, ctx_lens, page_table, self.gamma, b.sel_counts,
                            b.sel_offsets if on else None, b.sel_pages, b.sel_phys,
                            b.ws if on else None, stream)

    def attend(self, q, kv, stride_page, stride_head, pool_pages, ctx_lens, out=None,
               out_lse=None, stream=None, sel_pages=None, sel_phys=None):
        d, b = self.dims, self.buf
        out = b.out if out is None else out
        out_lse = b.out_lse if out_lse is None else out_lse
        sp = b.sel_pages if sel_pages is None else sel_pages
        sx = b.sel_phys if sel_phys is None else sel_phys
        lib.decode_attn_merge(d, q, kv, stride_page, stride_head, pool_pages, ctx_lens,
                              b.sel_counts, sp, sx, self.scale, self.workers, b.part_o,
                              b.part_lse, self.max_parts, out, out_lse, stream)
        return out, out_lse

    def run(self, q, summ, kv, stride_page, stride_head, pool_pages, page_table, ctx_lens,
            out=None, out_lse=None, stream=None):
        """Enqueue the whole step for one layer."""
        if self.groups:
            if stream is not None:
                raise ValueError("the grouped step runs on the current stream")
            out = self.buf.out if out is None else out
            out_lse = self.buf.out_lse if out_lse is None else out_lse
            return self._run_groups(q, summ, kv, stride_page, stride_head, pool_pages,
                                    page_table, ctx_lens, out, out_lse)
        self.score_select(q, summ, pool_pages, page_table, ctx_lens, stream)
        return self.attend(q, kv, stride_page, stride_head, pool_pages, ctx_lens, out, out_lse,
                           stream)


def canonical_strides(kv_heads):
    """(stride_page, stride_head) in elements of the pool [Ppool][Hkv][2][P*D]."""
    return kv_heads * 2 * PAGE * HEAD_DIM, 2 * PAGE * HEAD_DIM


def capture(fn, warmup=1):
    """Capture everything ``fn`` enqueues on a side stream into one graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g
