"""The read-ceiling helper (sparse_read_blocks): it must read exactly the
listed 8 KiB blocks, which its XOR checksum shows against NumPy."""

import numpy as np
import pytest
import torch

from adaptive_sparse_paged_amd import lib

from _gpu_case import say

pytestmark = pytest.mark.gpu


def _xor_of(pool_np, ids, nblocks):
    words = pool_np.view(np.uint32).reshape(nblocks, 2048)
    acc = np.uint32(0)
    for x in ids:
        if 0 <= x < nblocks:
            acc ^= np.bitwise_xor.reduce(words[x])
    return int(acc)


@pytest.mark.parametrize("kind", ["permutation", "sequential", "dups_and_out_of_range", "short",
                                  "empty"])
def test_read_blocks_checksum(gpu_lib, kind):
    nblocks = 4096                                    # 32 MiB
    rng = np.random.default_rng(7)
    pool_np = rng.integers(-32768, 32768, size=nblocks * 4096, dtype=np.int16)
    if kind == "permutation":
        ids = rng.permutation(nblocks)
    elif kind == "sequential":
        ids = np.arange(nblocks)
    elif kind == "short":
        ids = rng.permutation(nblocks)[:5]
    elif kind == "empty":
        ids = np.zeros(0, dtype=np.int64)
    else:
        ids = np.concatenate([rng.integers(0, nblocks, 3000), [-1, nblocks, 1 << 30, -7]])
        rng.shuffle(ids)
    say(f"[read_blocks] {kind}: {len(ids)} ids over {nblocks} blocks")
    pool = torch.from_numpy(pool_np).cuda()
    order = torch.from_numpy(ids.astype(np.int32)).cuda() if len(ids) else \
        torch.zeros(1, dtype=torch.int32, device="cuda")[:0]
    folds = torch.full((lib.READ_BLOCKS_GROUPS,), -1, dtype=torch.int32, device="cuda")
    lib.read_blocks(pool, nblocks, order, folds)
    torch.cuda.synchronize()
    words = folds.cpu().numpy().view(np.uint32)
    got = int(np.bitwise_xor.reduce(words))
    assert got == _xor_of(pool_np, ids, nblocks)
    if kind == "empty":
        assert (words == 0).all()          # every fold is written, even with nothing to read
