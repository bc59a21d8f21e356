"""GPU edge cases against the oracle: ragged and empty sequences, every head
grouping (GQA, MHA, groups wider than 16 heads), head sizes 64/128/256 in both
element types, the one-wave one-pass variant, the separate phase entry points,
the workspace initialisation, and out-of-contract inputs (bad lengths, bad
block ids) that must give NaN rows without touching memory outside the pool."""

import sys

import numpy as np
import pytest
import torch

import decode_attention_paged_05_amd as pad
from decode_attention_paged_05_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def custom(lens, H=24, Hkv=4, D=256, dtype="bf16", W=None, P=512, seed=21, extra_blocks=7):
    lens = list(lens)
    W = W or max(1, max(-(-L // 16) for L in lens))
    nb = sum(-(-L // 16) for L in lens) + extra_blocks
    spec = gen.ConfigSpec("custom", num_seqs=len(lens), num_heads=H, num_kv_heads=Hkv, head_size=D, block_size=16,
                          num_blocks=nb, max_blocks_per_seq=W, partition_size=P, dtype=dtype, seed=seed,
                          seq_len_range=(1, 2))
    return gen.make_problem(spec, seq_lens=lens)


RAGGED = [0, 1, 15, 16, 17, 511, 512, 513, 1000]


@pytest.mark.parametrize("layout", gu.LAYOUTS)
@pytest.mark.parametrize("P", [0, 16, 512, 1024])
def test_ragged_and_empty(P, layout):
    dp = gu.DeviceProblem(custom(RAGGED, P=P)).use(layout)
    log(f"[run] ragged P={P} {layout}")
    out = dp.run()
    ref = dp.oracle()
    assert np.all(ref[0] == 0)
    gu.assert_close(out, ref, "bf16", f"ragged P={P}")
    assert torch.all(out[0] == 0)


SHAPES = [
    dict(H=32, Hkv=1, D=128, dtype="bf16"),   # 32 heads per KV head: two head chunks
    dict(H=8, Hkv=8, D=64, dtype="bf16"),     # MHA
    dict(H=12, Hkv=4, D=128, dtype="bf16"),   # 3 heads per KV head
    dict(H=20, Hkv=4, D=256, dtype="bf16"),   # 5 heads per KV head
    dict(H=64, Hkv=4, D=64, dtype="bf16"),    # 16 heads per KV head
    dict(H=4, Hkv=2, D=256, dtype="bf16"),    # 2 heads per KV head
    dict(H=16, Hkv=2, D=256, dtype="f32"),
    dict(H=16, Hkv=1, D=128, dtype="f32"),
    dict(H=6, Hkv=1, D=64, dtype="f32"),
    dict(H=40, Hkv=2, D=128, dtype="f32"),    # 20 heads per KV head
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"H{s['H']}kv{s['Hkv']}D{s['D']}{s['dtype']}")
@pytest.mark.parametrize("P", [0, 64])
def test_head_groupings(shape, P):
    dp = gu.DeviceProblem(custom([37, 300, 1, 129], P=P, **shape))
    ref = dp.oracle()
    for layout in gu.LAYOUTS:
        log(f"[run] {shape} P={P} {layout}")
        out = dp.use(layout).run()
        gu.assert_close(out, ref, shape["dtype"], f"{shape} P={P} {layout}")


def test_one_pass_one_wave_variant():
    # 256 sequences x 4 KV heads = 1024 workgroups: the one-wave one-pass kernel
    lens = np.random.default_rng(5).integers(1, 200, size=256).tolist()
    dp = gu.DeviceProblem(custom(lens, P=0))
    ref = dp.oracle()
    for layout in gu.LAYOUTS:
        log(f"[run] one-pass, 1024 workgroups, {layout}")
        out = dp.use(layout).run()
        gu.assert_close(out, ref, "bf16", f"one-pass one-wave {layout}")
        split = dp.run(partition_size=64)
        gu.assert_close(split, ref, "bf16", f"split P=64, 256 seqs {layout}")


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_phase_entry_points_match_combined_call(layout):
    dp = gu.DeviceProblem(custom([700, 33, 1500], P=256)).use(layout)
    p = dp.p
    combined = dp.run()
    ws = dp.workspace(256)
    out = torch.full_like(combined, float("nan"))
    pad.paged_attention_decode_phase1(dp.query, dp.kc, dp.vc, dp.tables, dp.lens, p.scale, p.num_kv_heads, 16, 256,
                                      ws)
    dims = pad.make_dims(dp.query, dp.kc, dp.tables)
    pad.paged_attention_decode_phase2(out, dp.lens, 16, 256, ws, dims)
    assert torch.equal(out, combined)


def test_workspace_init_contents():
    S, H, D, W, P = 3, 5, 128, 40, 64
    ws = torch.full((pad.paged_attention_decode_workspace_size(S, H, D, W, 16, P),), 0x55, dtype=torch.uint8,
                    device="cuda")
    pad.paged_attention_decode_workspace_init(ws, S, H, D, W, 16, P)
    torch.cuda.synchronize()
    NP = -(-W * 16 // P)
    ml, es, tmp = pad.paged_attention_decode_workspace_layout(S, H, D, W, 16, P)
    n = S * H * NP
    assert torch.all(ws[ml: ml + 4 * n].view(torch.float32) == float("-inf"))
    assert torch.all(ws[es: es + 4 * n].view(torch.float32) == 0)
    assert torch.all(ws[tmp: tmp + 4 * n * D].view(torch.float32) == 0)


@pytest.mark.parametrize("layout", gu.LAYOUTS)
@pytest.mark.parametrize("P", [0, 64])
def test_out_of_contract_inputs_give_nan_rows(P, layout):
    """A length beyond the table width and a block id outside the pool are
    caught inside the kernels: those rows become NaN, the other rows stay
    exact, and no load leaves the pool (bounded buffer loads)."""
    dp = gu.DeviceProblem(custom([100, 40, 50, 70], P=P, W=8)).use(layout)
    good = dp.run()
    ref = dp.oracle()
    lens = dp.lens.clone()
    lens[1] = 8 * 16 + 1  # longer than the table
    tables = dp.tables.clone()
    tables[2, 1] = dp.p.num_blocks + 3  # outside the pool
    tables[3, 0] = -5
    out = dp.run(lens=lens, tables=tables)
    o = out.cpu()
    assert torch.isnan(o[1]).all() and torch.isnan(o[2]).all() and torch.isnan(o[3]).all()
    gu.assert_close(out[:1], ref[:1], "bf16", "untouched row")
    assert torch.equal(out[0], good[0])
