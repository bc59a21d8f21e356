"""The balanced split of the prefix attention on the GPU, against the oracle.

Every call goes through the C ABI (``paged_attention_prefill_split``): the
launch's walks are cut into equal ranges, cut walks leave pieces in the
workspace and a merge combines them.  The cases make the cuts fall everywhere:
walks cut into many pieces (more ranges than steps, so empty ranges too),
boundaries on walk starts, sequences without steps, and the two prefill
workloads the benchmark times.
"""

import numpy as np
import pytest
import torch

import decode_attention_paged_05_amd as pad
from decode_attention_paged_05_amd import inputs as gen
from tests.gpu_util import TOL
from tests.test_gpu_prefill import (PREFILL_SHAPES, DevicePrefill, _every_64th_and_edges, _edge_rows,
                                    _sampled_check, max_err)

pytestmark = pytest.mark.gpu


def run_split(dp: DevicePrefill, ws=None, out=None, tables=None, mql=None, scale=None):
    pp = dp.pp
    spec = pp.spec
    if ws is None:
        ws = pad.alloc_prefill_split_workspace(pp.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_size,
                                               pp.max_query_len if mql is None else mql, dp.dp.tables.shape[1])
    if out is None:
        out = torch.full(tuple(pp.query.shape), float("nan"), dtype=torch.float32, device="cuda")
    pad.paged_attention_prefill_split(out, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables if tables is None else tables,
                                      dp.qs, dp.ctx, pp.scale if scale is None else scale, spec.num_kv_heads, 16,
                                      pp.max_query_len if mql is None else mql, ws)
    torch.cuda.synchronize()
    return out


def test_split_small_ragged():
    dp = DevicePrefill(gen.make_prefill_problem("prefill_small"))
    assert max_err(run_split(dp), dp.oracle()) <= TOL["bf16"]


@pytest.mark.parametrize("H,Hkv,D,ctx,qn", PREFILL_SHAPES, ids=lambda v: str(v))
def test_split_shapes(H, Hkv, D, ctx, qn):
    """Every head grouping and head size; the split agrees with the oracle and
    with the one-walk-per-workgroup launch."""
    spec = gen.PrefillSpec("shape", context_lens=ctx, query_lens=qn, num_heads=H, num_kv_heads=Hkv, head_size=D,
                           dtype="bf16", seed=hash((H, Hkv, D, ctx, qn)) % 1000)
    dp = DevicePrefill(gen.make_prefill_problem(spec))
    got = run_split(dp)
    assert max_err(got, dp.oracle()) <= TOL["bf16"]
    assert float((got - dp.run()).abs().max()) <= TOL["bf16"]


@pytest.mark.parametrize("ctx,qn", [((5000,), (40,)), ((0, 3000, 0), (1, 17, 2)), ((70000,), (300,))],
                         ids=["one-walk", "tiny-walks", "long"])
def test_split_cuts_walks_into_many_pieces(ctx, qn):
    """Few, long walks against hundreds of ranges: each walk is cut into many
    pieces (ranges of one or two steps, some empty), all merged."""
    spec = gen.PrefillSpec("cuts", context_lens=ctx, query_lens=qn, num_heads=4, num_kv_heads=1, head_size=64,
                           dtype="bf16", seed=sum(ctx) % 997)
    dp = DevicePrefill(gen.make_prefill_problem(spec))
    assert max_err(run_split(dp), dp.oracle()) <= TOL["bf16"]


def test_split_pieces_mix_fp16_and_fallback():
    """A V value beyond fp16's range (1e6) in the middle of a 70 000-token
    context: the plan cuts each walk into pieces, the pieces holding the
    outlier fall back to the bf16 form and record their own reference, the
    others stay in fp16 and record theirs 2^7 lower, and the merge combines
    both kinds.  Every row attends to the outlier: each is within the
    tolerance of the oracle plus the bf16 form's relative precision."""
    spec = gen.PrefillSpec("mix", context_lens=(70000,), query_lens=(64,), num_heads=8, num_kv_heads=2,
                           head_size=128, dtype="bf16", seed=71)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp)
    g, d, pos = 1, 9, 35000
    blk, t = int(pp.pool.block_tables[0, pos // 16]), pos % 16
    big = torch.tensor(1e6, dtype=torch.bfloat16)
    dp.dp.vc[blk, g, d, t] = big.cuda()  # tiled V: [blocks, KV heads, D, 16]
    dp.dp.vc_host[blk, g, t, d] = big.view(torch.int16).numpy().astype(np.uint16)
    torch.cuda.synchronize()
    ws = pad.alloc_prefill_split_workspace(pp.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_size,
                                           pp.max_query_len, dp.dp.tables.shape[1])
    got = run_split(dp, ws=ws)
    assert int(ws[4:8].cpu().numpy().view(np.int32)[0]) > 0  # pieces listed
    want = dp.oracle()
    g_ = got.double().cpu().numpy()
    assert np.all(np.isfinite(g_))
    group = spec.num_heads // spec.num_kv_heads
    assert np.max(np.abs(want[:, g * group:(g + 1) * group, d])) > 1.0  # the outlier shows in every such row
    assert np.all(np.abs(g_ - want) <= TOL["bf16"] + 1e-4 * np.abs(want))


def test_split_sequences_without_work():
    """Empty chunks around the ones with work: their (no) rows, and the others exact."""
    spec = gen.PrefillSpec("empty", context_lens=(100, 0, 5000, 7, 0), query_lens=(0, 0, 129, 0, 33), num_heads=8,
                           num_kv_heads=2, head_size=128, dtype="bf16", seed=51)
    dp = DevicePrefill(gen.make_prefill_problem(spec))
    assert max_err(run_split(dp), dp.oracle()) <= TOL["bf16"]


def test_split_workspace_contents_do_not_matter():
    """Every workspace byte the call reads it writes first: NaN-filled and
    random workspaces, and a second call on the same one, give the same bits."""
    dp = DevicePrefill(gen.make_prefill_problem(gen.PrefillSpec(
        "ws", context_lens=(3000, 10, 700), query_lens=(100, 300, 64), num_heads=24, num_kv_heads=4, head_size=256,
        dtype="bf16", seed=52)))
    spec = dp.pp.spec
    ws = pad.alloc_prefill_split_workspace(dp.pp.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_size,
                                           dp.pp.max_query_len, dp.dp.tables.shape[1])
    ws.view(torch.uint8).fill_(0xFF)  # NaN floats, all-ones counters and offsets
    a = run_split(dp, ws=ws)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    b = run_split(dp, ws=ws)
    c = run_split(dp, ws=ws)
    assert torch.equal(a, b) and torch.equal(b, c)
    assert max_err(a, dp.oracle()) <= TOL["bf16"]


def test_split_ragged_batch_sampled():
    """The 4-sequence batch workload the benchmark times, same launch."""
    pp = gen.make_prefill_problem("prefill_batch")
    dp = DevicePrefill(pp, keep_host=False)
    got = run_split(dp)
    assert bool(torch.isfinite(got).all())
    assert _sampled_check(pp, got, _every_64th_and_edges, heads=(0, 5, 7, 12, 17, 23)) <= TOL["bf16"]


def test_split_full_size_sampled():
    """8192 new tokens over a 32768-token prefix: every 64th chunk token and the
    tile edges of all 24 heads against the oracle."""
    pp = gen.make_prefill_problem("prefill")
    dp = DevicePrefill(pp, keep_host=False)
    got = run_split(dp)
    assert bool(torch.isfinite(got).all())
    assert _sampled_check(pp, got, _every_64th_and_edges, heads=range(pp.spec.num_heads)) <= TOL["bf16"]


def test_split_out_of_contract_sequences():
    """A block id outside the pool makes that sequence's rows NaN (through the
    merge when its walks are cut); a chunk longer than max_query_len gets its
    first max_query_len rows NaN and the rest untouched; others exact."""
    pp = gen.make_prefill_problem("prefill_small")  # chunks (50, 1, 77, 128, 0)
    dp = DevicePrefill(pp)
    want = dp.oracle()
    tables = dp.dp.tables.clone()
    tables[0, 1] = pp.pool.num_blocks + 5
    got = run_split(dp, tables=tables)
    lo, hi = int(pp.query_start[0]), int(pp.query_start[1])
    assert bool(torch.isnan(got[lo:hi]).all())
    keep = np.r_[hi:pp.num_tokens]
    assert np.max(np.abs(got[keep].double().cpu().numpy() - want[keep])) <= TOL["bf16"]
    mq = 64
    out = torch.full(tuple(pp.query.shape), 7.0, dtype=torch.float32, device="cuda")
    run_split(dp, out=out, mql=mq)
    o = out.cpu()
    for s in (2, 3):  # 77 and 128 tokens
        lo, hi = int(pp.query_start[s]), int(pp.query_start[s + 1])
        assert bool(torch.isnan(o[lo:lo + mq]).all()), s
        assert bool((o[lo + mq:hi] == 7.0).all()), s
    keep = np.r_[0:int(pp.query_start[2])]
    assert np.max(np.abs(o[keep].double().numpy() - want[keep])) <= TOL["bf16"]


def test_split_rejects_a_small_workspace():
    dp = DevicePrefill(gen.make_prefill_problem("prefill_small"), keep_host=False)
    spec = dp.pp.spec
    need = pad.paged_attention_prefill_split_workspace_size(
        dp.pp.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_size, dp.pp.max_query_len,
        dp.dp.tables.shape[1], pad.paged_attention_prefill_split_ranges(spec.head_size, spec.num_heads,
                                                                          spec.num_kv_heads))
    with pytest.raises(pad.PadError):
        run_split(dp, ws=torch.empty(need - 256, dtype=torch.uint8, device="cuda"))


def test_split_graph_capture_replays():
    """The three kernels captured in a HIP graph: every replay, with eager work
    in between, equals the eager result bitwise."""
    dp = DevicePrefill(gen.make_prefill_problem("prefill_small"))
    pp, spec = dp.pp, dp.pp.spec
    ws = pad.alloc_prefill_split_workspace(pp.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_size,
                                           pp.max_query_len, dp.dp.tables.shape[1])
    eager = run_split(dp, ws=ws)
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()

    def step():
        pad.paged_attention_prefill_split(out, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables, dp.qs, dp.ctx, pp.scale,
                                          spec.num_kv_heads, 16, pp.max_query_len, ws)

    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            step()
    for r in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        assert torch.equal(run_split(dp, ws=ws), eager)


def test_split_more_sequences_than_the_plan_caches():
    """1 100 sequences: past the plan's 1 024 sequences in LDS, its tables live
    in the workspace and the sequences keep their given order."""
    rng = np.random.default_rng(61)
    S = 1100
    ctx = tuple(int(v) for v in rng.integers(0, 300, S))
    qn = tuple(int(v) for v in rng.integers(0, 9, S))
    spec = gen.PrefillSpec("many", context_lens=ctx, query_lens=qn, num_heads=8, num_kv_heads=2, head_size=128,
                           dtype="bf16", seed=61)
    dp = DevicePrefill(gen.make_prefill_problem(spec))
    assert max_err(run_split(dp), dp.oracle()) <= TOL["bf16"]


def test_split_many_cut_sequences():
    """400 sequences whose one walk each is cut: more (piece index, sequence)
    pairs than the plan's 1 024 threads, so its pair loop takes several rounds."""
    rng = np.random.default_rng(62)
    S = 400
    ctx = tuple(int(v) for v in rng.integers(1900, 2100, S))
    qn = tuple(int(v) for v in rng.integers(1, 4, S))
    spec = gen.PrefillSpec("cutmany", context_lens=ctx, query_lens=qn, num_heads=4, num_kv_heads=1, head_size=64,
                           dtype="bf16", seed=62)
    pp = gen.make_prefill_problem(spec)
    n_ranges = pad.paged_attention_prefill_split_ranges(64, 4, 1)
    assert pad.paged_attention_prefill_choose_split(pp.context_lens, pp.query_lens, 4, 1, 64, n_ranges)
    dp = DevicePrefill(pp)
    assert max_err(run_split(dp), dp.oracle()) <= TOL["bf16"]


def plan_model(ctx, qn, H, Hkv, N, mql):
    """The plan's decisions restated: C, the walks it cuts and the units it lists."""
    G = H // Hkv
    hc = 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    hg, tpw = G // hc, 256 // hc
    walks = []  # (sequence, tile, steps) of sequences inside the contract
    for s, (c, n) in enumerate(zip(ctx, qn)):
        if 0 < n <= mql:
            walks += [(s, t, -(-(c + min((t + 1) * tpw, n)) // 32)) for t in range(-(-n // tpw))]
    B = sum(st for _, _, st in walks) * Hkv * hg
    L = max((st for _, _, st in walks), default=0)
    C = max(-(-B // (4 * N)), -(-L // 32), 16)
    if L * 2 * N <= B:
        C = max(C, L)
    ks = [-(-st // C) for _, _, st in walks]
    cut = [k for k in ks if k > 1]
    pieces = Hkv * sum(cut)
    whole = Hkv * sum(1 for k in ks if k == 1)
    return {"units": pieces + whole, "pieces": pieces, "cut_walks": Hkv * len(cut), "C": C,
            "max_pieces": max(ks) if L > C else 1, "cut_seqs": len({s for (s, _, _), k in zip(walks, ks) if k > 1})}


@pytest.mark.parametrize("name", ["prefill_batch", "prefill", "prefill_small", "skewed"])
def test_split_plan_matches_model(name):
    """The plan's header (units, pieces, cut walks, C, most pieces of a walk,
    sequences with cut walks) against a restatement of its rule."""
    if name == "skewed":
        spec = gen.PrefillSpec("skewed", context_lens=(60000,) + (500,) * 15, query_lens=(1024,) + (256,) * 15,
                               num_heads=24, num_kv_heads=4, head_size=256, dtype="bf16", seed=63)
        pp = gen.make_prefill_problem(spec)
    else:
        pp = gen.make_prefill_problem(name)
    spec = pp.spec
    dp = DevicePrefill(pp, keep_host=False)
    ws = pad.alloc_prefill_split_workspace(pp.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_size,
                                           pp.max_query_len, dp.dp.tables.shape[1])
    run_split(dp, ws=ws)
    hdr = ws[:24].cpu().numpy().view(np.int32)
    N = pad.paged_attention_prefill_split_ranges(spec.head_size, spec.num_heads, spec.num_kv_heads)
    want = plan_model([int(v) for v in pp.context_lens], [int(v) for v in pp.query_lens], spec.num_heads,
                      spec.num_kv_heads, N, pp.max_query_len)
    got = dict(zip(["units", "pieces", "cut_walks", "C", "max_pieces", "cut_seqs"], [int(v) for v in hdr]))
    assert got == want


@pytest.mark.parametrize("H,Hkv,D,ctx,qn", [(24, 4, 256, (0, 37, 200, 16, 5), (50, 1, 77, 128, 0)),
                                            (8, 4, 128, (0, 64), (200, 17)), (10, 5, 64, (0,), (90,))],
                         ids=lambda v: str(v))
def test_split_without_cuts_gives_the_plain_bits(H, Hkv, D, ctx, qn):
    """Walks the split launch does not cut run the plain launch's walk code over
    the same steps: the same bits (the plan cuts nothing here; its header says
    so).  The split launch always takes the solo layout; a max_query_len of
    8192 makes the plain launch take it at head size 256 too."""
    spec = gen.PrefillSpec("nocut", context_lens=ctx, query_lens=qn, num_heads=H, num_kv_heads=Hkv, head_size=D,
                           dtype="bf16", seed=64)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp, keep_host=False)
    ws = pad.alloc_prefill_split_workspace(pp.num_seqs, H, Hkv, D, pp.max_query_len, dp.dp.tables.shape[1])
    got = run_split(dp, ws=ws)
    assert int(ws[4:8].cpu().numpy().view(np.int32)[0]) == 0  # pieces listed
    plain = torch.full(tuple(pp.query.shape), float("nan"), dtype=torch.float32, device="cuda")
    pad.paged_attention_prefill(plain, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables, dp.qs, dp.ctx, pp.scale, Hkv, 16,
                                8192)
    torch.cuda.synchronize()
    assert torch.equal(got, plain)
