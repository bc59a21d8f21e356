"""Pools larger than 4 GiB: block byte offsets past 2^32 must be formed in
64-bit arithmetic by every kernel that addresses the cache (decode in both
forms and both layouts, the chunk write, the prefix attention).

A small seeded problem is built in a compact pool, as everywhere else; its
blocks are then placed in a pool of 163 840 blocks (5 GiB per cache at 4 KV
heads x head size 256 in bf16), half of them beyond the 4 GiB mark and half at
their compact ids, with the rest of the large pool NaN.  The block table is
renumbered to match.  Placement changes no arithmetic, so each output must be
bitwise equal to the compact pool's output, and within tolerance of the
oracle."""

import sys

import numpy as np
import pytest
import torch

import decode_attention_paged_05_amd as pad
from decode_attention_paged_05_amd import inputs as gen
from tests import gpu_util as gu
from tests.test_gpu_prefill import DevicePrefill, _poison_chunk_slots, _upload

pytestmark = pytest.mark.gpu

BIG_BLOCKS = 163_840          # x 4 KV heads x 8 KB per (block, head) tile = 5 GiB per cache
FOUR_GIB_BLOCK = 131_072      # first block whose byte offset is 2^32 or more


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def placement(num_small: int) -> np.ndarray:
    """New id of every compact block: even ids go beyond the 4 GiB mark
    (counting down from the pool's last block, 3 apart), odd ids stay."""
    ids = np.arange(num_small, dtype=np.int64)
    far = BIG_BLOCKS - 1 - 3 * (ids // 2)
    new = np.where(ids % 2 == 0, far, ids)
    assert len(np.unique(new)) == num_small
    assert new[0::2].min() >= FOUR_GIB_BLOCK and new.max() < BIG_BLOCKS
    return new


def renumber(tables: torch.Tensor, new: np.ndarray) -> torch.Tensor:
    t = tables.cpu().numpy().astype(np.int64)
    valid = (t >= 0) & (t < len(new))
    t[valid] = new[t[valid]]
    return torch.from_numpy(t.astype(np.int32)).to(tables.device)


def spread(cache: torch.Tensor, new: np.ndarray) -> torch.Tensor:
    big = torch.full((BIG_BLOCKS,) + tuple(cache.shape[1:]), float("nan"), dtype=cache.dtype, device=cache.device)
    big.index_copy_(0, torch.from_numpy(new).to(cache.device), cache)
    return big


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_decode_pool_beyond_4gib(layout):
    lens = [700, 33, 1500]
    nb = sum(-(-L // 16) for L in lens) + 7
    spec = gen.ConfigSpec("large_pool", num_seqs=3, num_heads=24, num_kv_heads=4, head_size=256, block_size=16,
                          num_blocks=nb, max_blocks_per_seq=94, partition_size=256, dtype="bf16", seed=41,
                          seq_len_range=(1, 2))
    dp = gu.DeviceProblem(gen.make_problem(spec, seq_lens=lens), layouts=(layout,))
    ref = dp.oracle()
    new = placement(dp.p.num_blocks)
    kc, vc = spread(dp.kc, new), spread(dp.vc, new)
    assert kc.numel() * kc.element_size() > 2**32
    tables = renumber(dp.tables, new)
    # one-pass; the queue (94 partitions per head), the pool (47) and the plain split
    for P in (0, 16, 32, 256):
        log(f"[run] large pool {layout} P={P}")
        small = dp.run(partition_size=P)
        large = dp.run(partition_size=P, kc=kc, vc=vc, tables=tables)
        torch.cuda.synchronize()
        assert torch.equal(bits(large), bits(small)), f"{layout} P={P}: placement changed the output"
        gu.assert_close(large, ref, "bf16", f"large pool {layout} P={P}")
    del kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_chunk_write_and_prefill_pool_beyond_4gib(layout):
    spec = gen.PrefillSpec("large_pool", context_lens=(300, 0, 1000), query_lens=(100, 64, 130), num_heads=24,
                           num_kv_heads=4, head_size=256, dtype="bf16", seed=43)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp, layouts=(layout,))
    new = placement(pp.pool.num_blocks)
    tables = renumber(dp.dp.tables, new)
    # the cache without the chunk's rows, spread over the large pool; the chunk
    # write must fill exactly the rows the compact cache holds
    kc = spread(_upload(_poison_chunk_slots(dp.dp.kc_host, pp), layout, "bf16", "k"), new)
    vc = spread(_upload(_poison_chunk_slots(dp.dp.vc_host, pp), layout, "bf16", "v"), new)
    key, value = pp.chunk_kv()
    log(f"[run] large pool chunk write {layout}")
    pad.paged_attention_prefill_write_kv(kc, vc, gu.to_device(key, "bf16"), gu.to_device(value, "bf16"), tables,
                                         dp.qs, dp.ctx, 4, 16, pp.max_query_len)
    torch.cuda.synchronize()
    idx = torch.from_numpy(new).cuda()
    assert torch.equal(bits(kc.index_select(0, idx)), bits(dp.dp.kc)), "keys"
    assert torch.equal(bits(vc.index_select(0, idx)), bits(dp.dp.vc)), "values"
    if layout == "tiled":
        log("[run] large pool prefill")
        small = dp.run()
        large = dp.run(kc=kc, vc=vc, tables=tables)
        assert torch.equal(bits(large), bits(small)), "placement changed the prefill output"
        err = gu.max_err(large, dp.oracle())
        assert err <= gu.TOL["bf16"], err
    del kc, vc
    torch.cuda.empty_cache()
