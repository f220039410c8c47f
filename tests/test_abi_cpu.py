"""The C ABI without a GPU: the library loads, exports every function the
header declares, and its host-side argument checks reject bad calls before
any HIP call is made."""

import ctypes
import os
import re
import subprocess

import pytest

from adaptive_sparse_paged_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_paged.h")


def _declared():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        from adaptive_sparse_paged_amd import build
        build.build(verbose=False)
    return lib.load()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_status_strings(L):
    assert "gfx950" in lib.version()
    assert L.sparse_status_string(0) == b"ok"
    assert L.sparse_status_string(3).startswith(b"workspace")


def _dims(**kw):
    d = dict(batch=2, q_heads=8, kv_heads=2, max_pages=64)
    d.update(kw)
    return lib.make_dims(d["batch"], d["q_heads"], d["kv_heads"], d["max_pages"],
                         d.get("head_dim", 128), d.get("page_size", 16))


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def test_max_parts_and_workspace(L):
    d = _dims()
    # U + W partial slots: 4 units, W workers
    assert L.sparse_decode_max_parts(ctypes.byref(d), 16) == 4 + 16
    assert L.sparse_decode_max_parts(ctypes.byref(d), 5) == 4 + 5
    assert L.sparse_decode_max_parts(ctypes.byref(d), -1) == -1
    # 0 = one worker per compute unit of the current device (-1 with no device)
    r0 = L.sparse_decode_max_parts(ctypes.byref(d), 0)
    assert r0 == -1 or r0 > 4
    assert L.sparse_select_workspace_bytes(ctypes.byref(d)) >= 4
    # the exact per-request cache's workspace is the {0, 0} policy's
    for cap in (1, 64, 4096):
        plain = lib.cache_workspace_bytes(d, cap)
        assert plain > 0
        assert plain == lib.cache_policy_workspace_bytes(d, lib.CachePolicy(0, 0), cap)
    # a bound on the list lengths clamps the lists, not the grid
    d.max_list_pages = 20
    assert L.sparse_decode_max_parts(ctypes.byref(d), 16) == 4 + 16
    d.max_list_pages = 64
    assert L.sparse_decode_max_parts(ctypes.byref(d), 16) == 4 + 16
    for bad in (-1, 65):
        d.max_list_pages = bad
        assert L.sparse_decode_max_parts(ctypes.byref(d), 16) == -1
        assert L.sparse_score_pages(ctypes.byref(d), FAKE, FAKE, 10, FAKE, FAKE, 0.1, FAKE,
                                    None) == lib.ERR_INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), lib.ERR_UNSUPPORTED),
    (dict(page_size=32), lib.ERR_UNSUPPORTED),
    (dict(q_heads=7), lib.ERR_INVALID),
    (dict(q_heads=64, kv_heads=2), lib.ERR_UNSUPPORTED),
    (dict(q_heads=6, kv_heads=2), lib.ERR_UNSUPPORTED),     # G = 3: not a power of two
    (dict(q_heads=20, kv_heads=4), lib.ERR_UNSUPPORTED),    # G = 5
    (dict(q_heads=24, kv_heads=2), lib.ERR_UNSUPPORTED),    # G = 12
    (dict(max_pages=40000), lib.ERR_UNSUPPORTED),
    (dict(batch=0), lib.ERR_INVALID),
])
def test_dims_rejected(L, kw, code):
    d = _dims(**kw)
    r = L.sparse_score_pages(ctypes.byref(d), FAKE, FAKE, 10, FAKE, FAKE, 0.1, FAKE, None)
    assert r == code


def test_null_and_value_checks(L):
    d = _dims()
    assert L.sparse_score_pages(None, FAKE, FAKE, 10, FAKE, FAKE, 0.1, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_score_pages(ctypes.byref(d), None, FAKE, 10, FAKE, FAKE, 0.1, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_score_pages(ctypes.byref(d), FAKE, FAKE, 10, FAKE, FAKE, float("nan"), FAKE, None) == lib.ERR_INVALID
    sel = lambda gamma, ws, wsb, offs=FAKE: L.sparse_select_coverage(
        ctypes.byref(d), FAKE, FAKE, FAKE, gamma, FAKE, offs, FAKE, FAKE, ws, wsb, None)
    assert sel(0.0, FAKE, 256) == lib.ERR_INVALID
    assert sel(1.5, FAKE, 256) == lib.ERR_INVALID
    assert sel(float("nan"), FAKE, 256) == lib.ERR_INVALID
    assert sel(0.99, None, 256) == lib.ERR_WORKSPACE              # prefix sum without workspace
    assert sel(0.99, FAKE, 1) == lib.ERR_WORKSPACE
    assert L.sparse_select_coverage(ctypes.byref(d), FAKE, FAKE, FAKE, 0.9, None, None, FAKE,
                                    FAKE, None, 0, None) == lib.ERR_INVALID   # no counts
    attn = lambda kvp, sp_, sh, mp, workers=16: L.sparse_decode_attn(
        ctypes.byref(d), FAKE, kvp, sp_, sh, 100, FAKE, FAKE, FAKE, FAKE, 0.1, workers, FAKE,
        FAKE, mp, None)
    assert attn(FAKE, 8192, 4096, 19) == lib.ERR_INVALID          # wrong max_parts (U + 16 = 20)
    assert attn(FAKE, 8192, 4096, 20, workers=-1) == lib.ERR_INVALID
    assert attn(FAKE, 8192, 4096, 20, workers=(1 << 20) + 1) == lib.ERR_INVALID
    assert attn(ctypes.c_void_p(0x10002), 8192, 4096, 20) == lib.ERR_INVALID  # misaligned pool
    assert attn(FAKE, 8191, 4096, 20) == lib.ERR_INVALID          # stride not 16-byte
    am = lambda mp, out=FAKE, workers=16: L.sparse_decode_attn_merge(
        ctypes.byref(d), FAKE, FAKE, 8192, 4096, 100, FAKE, FAKE, FAKE, FAKE, 0.1, workers, FAKE,
        FAKE, mp, out, FAKE, None)
    assert am(19) == lib.ERR_INVALID                              # wrong max_parts
    assert am(20, out=None) == lib.ERR_INVALID
    assert am(20, out=ctypes.c_void_p(0x10004)) == lib.ERR_INVALID   # out not 16-byte aligned
    assert am(20, workers=-3) == lib.ERR_INVALID
    na = lambda dd, out=FAKE: L.sparse_decode_attn_merge_noalloc(
        ctypes.byref(dd), FAKE, FAKE, 8192, 4096, 100, FAKE, FAKE, FAKE, FAKE, 0.1, 16, out,
        FAKE, None)
    assert na(d, out=None) == lib.ERR_INVALID
    # partials beyond the library's device array: (16384 + 16) * 4 * 129 * 4 bytes > 16 MiB
    assert na(_dims(batch=2048, q_heads=32, kv_heads=8)) == lib.ERR_WORKSPACE
    assert L.sparse_merge_splits(ctypes.byref(d), FAKE, FAKE, FAKE, -1, FAKE, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_merge_splits(ctypes.byref(d), FAKE, FAKE, None, 16, FAKE, FAKE, None) == lib.ERR_INVALID
    pair = lambda b_o=FAKE, b_l=FAKE, b_c=FAKE, workers=16, workers_b=8: L.sparse_merge_splits_pair(
        ctypes.byref(d), FAKE, FAKE, FAKE, workers, b_o, b_l, b_c, workers_b, FAKE, FAKE, None)
    assert pair(b_o=None) == lib.ERR_INVALID
    assert pair(b_l=None) == lib.ERR_INVALID
    assert pair(b_c=None) == lib.ERR_INVALID
    assert pair(b_o=ctypes.c_void_p(0x10004)) == lib.ERR_INVALID      # partials 16-byte aligned
    assert pair(workers=-1) == lib.ERR_INVALID
    assert pair(workers_b=-1) == lib.ERR_INVALID
    assert L.sparse_select_topk(ctypes.byref(d), FAKE, FAKE, FAKE, 0, FAKE, None,
                                FAKE, FAKE, None, 0, None) == lib.ERR_INVALID
    assert L.sparse_append_tokens(ctypes.byref(d), None, FAKE, FAKE, 8192, 4096, 100, FAKE,
                                  FAKE, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_hbm_cache_resolve(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 9000, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == lib.ERR_UNSUPPORTED
    assert L.sparse_hbm_cache_resolve(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == lib.ERR_WORKSPACE
    pol = lambda shift, pooled, cap, nb, ws=FAKE: L.sparse_hbm_cache_resolve_policy(
        ctypes.byref(d), ctypes.byref(lib.CachePolicy(shift, pooled)), FAKE, FAKE, FAKE, FAKE,
        cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nb, None)
    assert L.sparse_hbm_cache_resolve_policy(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, 64,
                                             FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                             None) == lib.ERR_INVALID
    assert pol(31, 0, 64, 1 << 30) == lib.ERR_INVALID
    assert pol(-1, 0, 64, 1 << 30) == lib.ERR_INVALID
    assert pol(0, 2, 64, 1 << 30) == lib.ERR_INVALID
    assert pol(0, 0, 9000, 1 << 30) == lib.ERR_UNSUPPORTED      # per-request slot limit
    assert pol(0, 1, (1 << 22) + 1, 1 << 40) == lib.ERR_UNSUPPORTED
    need = L.sparse_cache_policy_workspace_bytes(ctypes.byref(d), ctypes.byref(lib.CachePolicy(3, 1)), 9000)
    assert need >= 9000 * 13
    assert pol(3, 1, 9000, need - 1) == lib.ERR_WORKSPACE
    assert pol(3, 1, 9000, need, None) == lib.ERR_WORKSPACE
    assert L.sparse_build_page_summaries(ctypes.byref(d), FAKE, 8192, 4096, 100, FAKE, FAKE, -1, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_build_page_summaries(ctypes.byref(d), FAKE, 8192, 4096, 100, FAKE, FAKE, 0, FAKE, None) == lib.OK
    # the host tier in two halves
    split = lambda cap, ws_bytes, hit=FAKE, pol=lib.CachePolicy(0, 0), ml=(None, None, None): \
        L.sparse_hbm_cache_resolve_split(
            ctypes.byref(d), ctypes.byref(pol), FAKE, FAKE, cap, FAKE, FAKE, FAKE, FAKE, FAKE, hit,
            FAKE, *ml, FAKE, ws_bytes, None)
    assert split(64, 1 << 30, hit=None) == lib.ERR_INVALID
    # the miss lists: all three or none
    assert split(64, 1 << 30, ml=(FAKE, None, None)) == lib.ERR_INVALID
    assert split(64, 1 << 30, ml=(FAKE, FAKE, None)) == lib.ERR_INVALID
    assert split(64, 1 << 30, ml=(None, None, FAKE)) == lib.ERR_INVALID
    assert split(0, 1 << 30) == lib.ERR_INVALID
    assert split(9000, 1 << 30) == lib.ERR_UNSUPPORTED          # per-request slot limit
    assert split(64, 16) == lib.ERR_WORKSPACE
    assert split(64, 1 << 30, pol=lib.CachePolicy(0, 3)) == lib.ERR_INVALID
    fetch = lambda host, cache, ws_bytes: L.sparse_hbm_cache_fetch(
        ctypes.byref(d), ctypes.byref(lib.CachePolicy(0, 0)), host, cache, 64, FAKE, FAKE,
        ws_bytes, None)
    assert fetch(None, FAKE, 1 << 30) == lib.ERR_INVALID
    assert fetch(FAKE, ctypes.c_void_p(0x10002), 1 << 30) == lib.ERR_INVALID
    assert fetch(FAKE, FAKE, 16) == lib.ERR_WORKSPACE
    # the fetch with its attention beside the attention over the hits
    fa = lambda host=FAKE, cap=64, step=FAKE, pol=lib.CachePolicy(0, 0), ml=(FAKE, FAKE, FAKE), \
        mp=20, mo=FAKE, mlse=FAKE: L.sparse_hbm_cache_fetch_attn(
            ctypes.byref(d), ctypes.byref(pol), host, FAKE, cap, step, FAKE, FAKE, FAKE, FAKE,
            FAKE, *ml, 0.1, 16, FAKE, FAKE, mp, mo, mlse, None)
    assert fa(host=None) == lib.ERR_INVALID
    assert fa(cap=0) == lib.ERR_INVALID
    assert fa(cap=9000) == lib.ERR_UNSUPPORTED                   # per-request slot limit
    assert fa(step=None) == lib.ERR_INVALID
    assert fa(pol=lib.CachePolicy(0, 3)) == lib.ERR_INVALID
    assert fa(mp=19) == lib.ERR_INVALID                          # hits' partials: U + 16 = 20
    assert fa(ml=(None, FAKE, FAKE)) == lib.ERR_INVALID
    assert fa(ml=(FAKE, None, FAKE)) == lib.ERR_INVALID
    assert fa(ml=(FAKE, FAKE, None)) == lib.ERR_INVALID
    assert fa(mo=None) == lib.ERR_INVALID
    assert fa(mlse=None) == lib.ERR_INVALID
    assert fa(mo=ctypes.c_void_p(0x10004)) == lib.ERR_INVALID    # 16-byte aligned partials
    assert L.sparse_split_misses(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                 None) == lib.ERR_INVALID
    assert L.sparse_lse_combine(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                None) == lib.ERR_INVALID
    assert L.sparse_lse_combine(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.c_void_p(0x20000), FAKE,
                                ctypes.c_void_p(0x20000), None) == lib.ERR_INVALID   # lse aliased
    # the read-ceiling helper
    assert L.sparse_read_blocks(FAKE, 100, FAKE, -1, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_read_blocks(FAKE, -1, FAKE, 10, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_read_blocks(None, 100, FAKE, 10, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_read_blocks(FAKE, 100, FAKE, 10, None, None) == lib.ERR_INVALID
    assert L.sparse_read_blocks(ctypes.c_void_p(0x10002), 100, FAKE, 10, FAKE, None) == lib.ERR_INVALID
    assert L.sparse_read_blocks(FAKE, 100, FAKE, 10, ctypes.c_void_p(0x10002), None) == lib.ERR_INVALID


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        lib.load.__wrapped__ if hasattr(lib.load, "__wrapped__") else None
        saved = lib._lib
        try:
            lib._lib = None
            lib.load(str(tmp_path / "nope.so"))
        finally:
            lib._lib = saved


def test_binding_constants_match_header():
    """The binding's copies of the header's constants: the read probe's grid
    (it sizes xor_out), the attention plan's fewest pages per worker (the
    bench's partial count follows it) and the host tier's copying grid (it
    sizes the copying waves' partials)."""
    with open(HEADER) as f:
        text = f.read()
    m = re.search(r"#define SPARSE_READ_BLOCKS_GROUPS (\d+)", text)
    assert m and int(m.group(1)) == lib.READ_BLOCKS_GROUPS
    m = re.search(r"#define SPARSE_ATTN_MIN_WORKER_PAGES (\d+)", text)
    assert m and int(m.group(1)) == lib.ATTN_MIN_WORKER_PAGES
    m = re.search(r"#define SPARSE_ATTN_UNIT_COST_PAGES (\d+)", text)
    assert m and int(m.group(1)) == lib.ATTN_UNIT_COST_PAGES
    m = re.search(r"#define SPARSE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == lib.NOALLOC_SCRATCH_BYTES
    m = re.search(r"#define SPARSE_FETCH_ATTN_COPY_GROUPS (\d+)", text)
    assert m and int(m.group(1)) == lib.FETCH_ATTN_COPY_GROUPS
    m = re.search(r"#define SPARSE_FETCH_ATTN_COPY_WAVES \((\d+) \* SPARSE_FETCH_ATTN_COPY_GROUPS\)",
                  text)
    assert m and int(m.group(1)) * lib.FETCH_ATTN_COPY_GROUPS == lib.FETCH_ATTN_COPY_WAVES
    m = re.search(r"#define SPARSE_FETCH_GROUPS (\d+)", text)
    assert m and int(m.group(1)) == lib.FETCH_GROUPS
