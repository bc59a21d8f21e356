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
import oracle
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


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_skewed_batch_at_the_batch_rule_choice(layout):
    """64 sequences, one 16 times as long as the others: the batch rule turns
    the fixed rule's one-pass choice into a split; both against the oracle."""
    lens = [256] * 63 + [4096]
    P = pad.paged_attention_decode_choose_partition_for_batch(64, 24, 4, 256, "bf16", max(lens), sum(lens), 16, 256)
    assert pad.paged_attention_decode_choose_partition(64, 24, 4, max(lens), 16, 256) == 0
    assert P > 0
    dp = gu.DeviceProblem(custom(lens, P=P, seed=23)).use(layout)
    ref = dp.oracle()
    for part in (P, 0):
        log(f"[run] skewed batch P={part} {layout}")
        gu.assert_close(dp.run(partition_size=part), ref, "bf16", f"skewed batch P={part}")


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
    pad.paged_attention_decode_phase2(out, dp.lens, p.num_kv_heads, 16, 256, ws, dims)
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


def long_like(L, W=6272, seed=31):
    """1 sequence, 24 q / 4 KV heads, D 256, P 512 and a table 6272 blocks wide:
    4 x 196 partition slots, more than one workgroup per compute unit, as in the
    100K-token workload, so phase 1 runs the balanced split."""
    spec = gen.ConfigSpec("long_like", num_seqs=1, num_heads=24, num_kv_heads=4, head_size=256, block_size=16,
                          num_blocks=W + 5, max_blocks_per_seq=W, partition_size=512, dtype="bf16", seed=seed,
                          seq_len=L)
    return gen.make_problem(spec)


def garbage_workspace(dp, P):
    """A workspace of the right size filled with random bytes, launch record
    included (never initialised: phase 1 reads nothing from it)."""
    ws = dp.workspace(P, init=False)
    g = torch.Generator(device="cuda").manual_seed(99)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g))
    return ws


def run_checked(dp, P, what, expect_balanced=True):
    """Split run on a never-initialised workspace: the output against the
    oracle, every phase-1 entry against the oracle's Phase 1 over the tokens
    the host-side plan gives its slot (for a few heads), the plan's mode, and
    a second call bitwise equal."""
    p = dp.p
    ws = garbage_workspace(dp, P)
    out = dp.run(partition_size=P, workspace=ws)
    torch.cuda.synchronize()
    ref = dp.oracle()
    gu.assert_close(out, ref, p.dtype, what)
    plan = gu.entry_plan(p, P, layout=dp.layout)
    if gu.device_cus() == 256:
        assert plan[0] == expect_balanced, f"{what}: balanced split expected {expect_balanced}"
    for s in sorted({0, p.num_seqs - 1, p.num_seqs // 2}):
        L = int(p.seq_lens[s])
        if L <= 0 or L > p.max_blocks_per_seq * 16:
            continue
        K = oracle.widen(oracle.gather_sequence(dp.kc_host, p.block_tables[s], L, 16), p.dtype)
        V = oracle.widen(oracle.gather_sequence(dp.vc_host, p.block_tables[s], L, 16), p.dtype)
        q = oracle.widen(p.query[s], p.dtype)
        G = p.num_heads // p.num_kv_heads
        for h in sorted({0, p.num_heads - 1}):
            entries = gu.phase1_entries(ws, p, P, s, h, plan)
            tol = dict(tol_m=1e-5, tol_l=1e-5, tol_o=1e-5) if p.dtype == "f32" else {}
            gu.check_phase1_entries(entries, q[h], K[h // G], V[h // G], p.scale, **tol)
    again = dp.run(partition_size=P, workspace=ws)
    assert torch.equal(again, out), f"{what}: not repeatable"
    return out, ws


@pytest.mark.parametrize("layout", gu.LAYOUTS)
@pytest.mark.parametrize("L", [90000, 99000, 100352])
def test_long_balanced(L, layout):
    # 90000: ranges over a shorter context than the table; 99000: the last
    # range ends inside a block; 100352: every slot of the table's width full
    dp = gu.DeviceProblem(long_like(L)).use(layout)
    log(f"[run] long-like L={L} {layout}")
    run_checked(dp, 512, f"long-like L={L} {layout}")


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_long_balanced_every_entry(layout):
    # every entry of every head of a 99 000-token context equals the oracle's
    # Phase 1 over the tokens the plan gives its slot, and the entries tile the context
    dp = gu.DeviceProblem(long_like(99000)).use(layout)
    p = dp.p
    ws = garbage_workspace(dp, 512)
    dp.run(workspace=ws)
    torch.cuda.synchronize()
    plan = gu.entry_plan(p, 512, layout=layout)
    K = oracle.widen(oracle.gather_sequence(dp.kc_host, p.block_tables[0], 99000, 16), "bf16")
    V = oracle.widen(oracle.gather_sequence(dp.vc_host, p.block_tables[0], 99000, 16), "bf16")
    q = oracle.widen(p.query[0], "bf16")
    for h in range(24):
        entries = gu.phase1_entries(ws, p, 512, 0, h, plan)
        assert entries[0][0] == 0 and entries[-1][1] == 99000
        assert all(a[1] == b[0] for a, b in zip(entries, entries[1:])), "entries must tile the context"
        if gu.device_cus() == 256:
            # 512 ranges (two per compute unit, tiled) or 768 (three, rows) over 4 heads' equal shares
            assert len(entries) in ((128, 129) if layout == "tiled" else (192, 193))
        gu.check_phase1_entries(entries, q[h], K[h // 6], V[h // 6], p.scale)


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_long_balanced_phase_entry_points_match_combined_call(layout):
    # phase 2 on its own must find the entries phase 1 left, through the launch record
    dp = gu.DeviceProblem(long_like(100000)).use(layout)
    p = dp.p
    combined = dp.run()
    gu.assert_close(combined, dp.oracle(), "bf16", "long-like combined")
    ws = garbage_workspace(dp, 512)
    out = torch.full_like(combined, float("nan"))
    pad.paged_attention_decode_phase1(dp.query, dp.kc, dp.vc, dp.tables, dp.lens, p.scale, p.num_kv_heads, 16, 512,
                                      ws)
    dims = pad.make_dims(dp.query, dp.kc, dp.tables)
    pad.paged_attention_decode_phase2(out, dp.lens, p.num_kv_heads, 16, 512, ws, dims)
    assert torch.equal(out, combined)


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_phase2_without_matching_phase1_gives_nan(layout):
    """Phase 2 of a balanced-split launch reads phase 1's launch record; when
    the record does not match the call (phase 1 never ran on this workspace,
    or ran with other lengths) the rows are NaN, never a silent wrong value."""
    dp = gu.DeviceProblem(long_like(100000)).use(layout)
    p = dp.p
    dims = pad.make_dims(dp.query, dp.kc, dp.tables)
    out = torch.zeros((1, 24, 256), dtype=torch.float32, device="cuda")
    ws = garbage_workspace(dp, 512)
    pad.paged_attention_decode_phase2(out, dp.lens, p.num_kv_heads, 16, 512, ws, dims)
    assert torch.isnan(out).all(), "random launch record"
    ws = dp.workspace(512)  # initialised: an empty launch record
    out.zero_()
    pad.paged_attention_decode_phase2(out, dp.lens, p.num_kv_heads, 16, 512, ws, dims)
    assert torch.isnan(out).all(), "initialised workspace, phase 1 never run"
    # phase 1 with 99 000 tokens, phase 2 told 100 000
    lens2 = dp.lens.clone()
    lens2[0] = 99000
    pad.paged_attention_decode_phase1(dp.query, dp.kc, dp.vc, dp.tables, lens2, p.scale, p.num_kv_heads, 16, 512, ws)
    out.zero_()
    pad.paged_attention_decode_phase2(out, dp.lens, p.num_kv_heads, 16, 512, ws, dims)
    assert torch.isnan(out).all(), "launch record of other lengths"
    # and the workspace serves a correct call right after
    gu.assert_close(dp.run(workspace=ws), dp.oracle(), "bf16", "after the mismatched calls")


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_long_balanced_bad_block_in_the_last_range(layout):
    dp = gu.DeviceProblem(long_like(100352)).use(layout)
    tables = dp.tables.clone()
    tables[0, 6200] = dp.p.num_blocks + 11  # logical block 6200, in the last ranges of KV head 0..3
    out = dp.run(tables=tables)
    assert torch.isnan(out).all()
    good = dp.run()
    gu.assert_close(good, dp.oracle(), "bf16", "after the bad call")


BALANCED_SHAPES = [
    # (lens, H, Hkv, D, dtype, W, P): more partition slots than compute units
    ([17900, 16500], 24, 4, 256, "bf16", 1120, 512),   # 2 seqs: a range crosses from one sequence to the next
    ([20380], 8, 8, 128, "bf16", 1280, 512),           # MHA
    ([76793], 8, 2, 64, "f32", 4800, 512),             # fp32
    ([40000], 24, 4, 256, "f32", 2500, 128),           # fp32 at head 256, tiled: three ranges per CU (768)
    ([38397], 16, 2, 256, "bf16", 2400, 256),          # P 256
    ([300, 290, 17, 5], 8, 8, 64, "bf16", 40, 16),     # little work: ranges of 8 blocks, fewer than the grid
    ([1000] * 40, 8, 4, 128, "bf16", 64, 512),         # two slots per head: the entry cap sets the range count
    ([1000, 24, 1000, 999] * 10, 40, 2, 128, "f32", 63, 512),  # 20 heads per KV head (two head chunks), two slots
]


@pytest.mark.parametrize("layout", gu.LAYOUTS)
@pytest.mark.parametrize("shape", BALANCED_SHAPES,
                         ids=lambda s: f"S{len(s[0])}H{s[1]}kv{s[2]}D{s[3]}{s[4]}W{s[5]}P{s[6]}")
def test_balanced_shapes(shape, layout):
    lens, H, Hkv, D, dtype, W, P = shape
    dp = gu.DeviceProblem(custom(lens, H=H, Hkv=Hkv, D=D, dtype=dtype, W=W, P=P)).use(layout)
    log(f"[run] balanced shape {shape} {layout}")
    run_checked(dp, P, f"balanced {shape} {layout}")


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_graph_capture_replays(layout):
    """The split call (balanced split) and the one-pass call captured in a
    HIP graph: every replay, with eager work and synchronisation in between,
    equals the eager result bitwise (no memset nodes, no host state)."""
    dp = gu.DeviceProblem(long_like(100000)).use(layout)
    p = dp.p
    ws = dp.workspace(512)
    out = torch.empty((1, 24, 256), dtype=torch.float32, device="cuda")
    one = torch.empty_like(out)
    eager = dp.run(workspace=ws)
    eager_one = dp.run(partition_size=0)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        dp.run(workspace=ws, out=out)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            dp.run(workspace=ws, out=out)
            dp.run(partition_size=0, out=one)
    for r in range(4):
        out.fill_(float("nan"))
        one.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}: split result differs from eager"
        assert torch.equal(one, eager_one), f"replay {r}: one-pass result differs from eager"
        # eager work between replays, on the same workspace
        assert torch.equal(dp.run(workspace=ws), eager)
    gu.assert_close(out, dp.oracle(), "bf16", "graph replay vs oracle")


@pytest.mark.parametrize("layout", gu.LAYOUTS)
def test_balanced_ragged_batch(layout):
    """40 ragged sequences (some empty, one of a single token), P 256: the
    balanced split over the live blocks only; the two phases called
    separately; a length past the table makes that row NaN and leaves the
    others bitwise unchanged."""
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 5000, size=40)
    lens[[3, 17]] = 0
    lens[25] = 1
    dp = gu.DeviceProblem(custom(lens.tolist(), H=24, Hkv=4, D=128, P=256, W=313)).use(layout)
    p = dp.p
    log(f"[run] balanced ragged batch {layout}")
    out, ws = run_checked(dp, 256, f"ragged batch {layout}")
    assert torch.all(out[3] == 0) and torch.all(out[17] == 0)
    sep = torch.full_like(out, float("nan"))
    pad.paged_attention_decode_phase1(dp.query, dp.kc, dp.vc, dp.tables, dp.lens, p.scale, p.num_kv_heads, 16, 256,
                                      ws)
    pad.paged_attention_decode_phase2(sep, dp.lens, p.num_kv_heads, 16, 256, ws, pad.make_dims(dp.query, dp.kc,
                                                                                                dp.tables))
    assert torch.equal(sep, out)
    lens_bad = dp.lens.clone()
    lens_bad[7] = 313 * 16 + 5
    bad = dp.run(workspace=ws, lens=lens_bad)
    assert torch.isnan(bad[7]).all()
    keep = [i for i in range(40) if i != 7]
    # the other rows: within tolerance (the ranges move when sequence 7's blocks drop out)
    gu.assert_close(bad[keep], dp.oracle()[keep], "bf16", "rows next to an out-of-contract length")


@pytest.mark.parametrize("layout", gu.LAYOUTS)
@pytest.mark.parametrize("shape", [(16, 4, 64, "f32", 128), (8, 8, 256, "bf16", 512), (32, 2, 128, "f32", 64)],
                         ids=lambda s: f"H{s[0]}kv{s[1]}D{s[2]}{s[3]}P{s[4]}")
def test_balanced_many_sequences(shape, layout):
    H, Hkv, D, dtype, P = shape
    rng = np.random.default_rng(D + P)
    lens = rng.integers(1, 3000, size=24).tolist()
    W = -(-max(lens) // 16)
    dp = gu.DeviceProblem(custom(lens, H=H, Hkv=Hkv, D=D, dtype=dtype, P=P, W=W)).use(layout)
    log(f"[run] balanced {shape} {layout}")
    run_checked(dp, P, f"balanced {shape} {layout}")


def test_two_streams_two_workspaces():
    """Two split calls in flight at once on two streams, each with its own
    workspace: both exact."""
    a = gu.DeviceProblem(long_like(100000)).use("tiled")
    b = gu.DeviceProblem(custom(np.random.default_rng(3).integers(1, 6000, size=24).tolist(), P=512)).use("tiled")
    ra, rb = a.oracle(), b.oracle()
    wa, wb = a.workspace(512), b.workspace(512)
    oa = torch.empty((1, 24, 256), dtype=torch.float32, device="cuda")
    ob = torch.empty((24, 24, 256), dtype=torch.float32, device="cuda")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(sa):
            a.run(workspace=wa, out=oa)
        with torch.cuda.stream(sb):
            b.run(workspace=wb, out=ob)
    torch.cuda.synchronize()
    gu.assert_close(oa, ra, "bf16", "stream a")
    gu.assert_close(ob, rb, "bf16", "stream b")


@pytest.mark.parametrize("layout", gu.LAYOUTS)
@pytest.mark.parametrize("P", [0, 64, 512])
def test_strided_query_and_out(P, layout):
    """query as the query part of a fused QKV projection [S, (H + 2 Hkv) * D]
    and out as a slice of a wider buffer: bitwise equal to contiguous tensors,
    nothing written outside the slice (one-pass, one workgroup per partition,
    the balanced split; the phase entry points too)."""
    lens = [700, 33, 1500, 0, 2100, 16]
    dp = gu.DeviceProblem(custom(lens, P=P or 512, W=140)).use(layout)
    p = dp.p
    S, H, Hkv, D = p.num_seqs, p.num_heads, p.num_kv_heads, p.head_size
    ref = dp.run(partition_size=P)
    qkv = torch.full((S, (H + 2 * Hkv) * D), float("nan"), dtype=dp.query.dtype, device="cuda")
    qkv[:, :H * D] = dp.query.reshape(S, H * D)
    q_view = qkv[:, :H * D].view(S, H, D)
    wide = torch.full((S, H * D + 96), -3.0, dtype=torch.float32, device="cuda")
    out_view = wide[:, 32:32 + H * D].view(S, H, D)
    assert q_view.stride(0) == (H + 2 * Hkv) * D and out_view.stride(0) == H * D + 96
    ws = dp.workspace(P) if P else None
    pad.paged_attention_decode(out_view, q_view, dp.kc, dp.vc, dp.tables, dp.lens, p.scale, Hkv, 16, P, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_view, ref), f"strided views differ (P={P})"
    assert torch.all(wide[:, :32] == -3.0) and torch.all(wide[:, 32 + H * D:] == -3.0), "wrote outside the slice"
    gu.assert_close(out_view, dp.oracle(), "bf16", f"strided P={P}")
    if P:
        wide.fill_(-3.0)
        pad.paged_attention_decode_phase1(q_view, dp.kc, dp.vc, dp.tables, dp.lens, p.scale, Hkv, 16, P, ws)
        pad.paged_attention_decode_phase2(out_view, dp.lens, Hkv, 16, P, ws, pad.make_dims(q_view, dp.kc, dp.tables))
        torch.cuda.synchronize()
        assert torch.equal(out_view, ref), "phase entry points with strided views"
        assert torch.all(wide[:, :32] == -3.0) and torch.all(wide[:, 32 + H * D:] == -3.0)


def test_more_than_1024_sequences_split():
    """1 100 short sequences: more than the balanced split takes, so phase 1
    runs one workgroup per partition (and the merge counts ceil(L / P))."""
    rng = np.random.default_rng(17)
    lens = rng.integers(0, 200, size=1100).tolist()
    dp = gu.DeviceProblem(custom(lens, H=8, Hkv=2, D=64, P=64, W=13))
    p = dp.p
    bal, *_ = gu.entry_plan(p, 64)
    assert not bal
    ref = dp.oracle()
    for layout in gu.LAYOUTS:
        log(f"[run] 1100 sequences, P=64, {layout}")
        gu.assert_close(dp.use(layout).run(), ref, "bf16", f"1100 sequences {layout}")
