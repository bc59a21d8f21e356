"""Prefix (chunked prefill) attention and the chunk write on the GPU, against the oracle.

Every call goes through the C ABI (``paged_attention_prefill``,
``paged_attention_prefill_write_kv``).  Small problems are compared row by
row with the full oracle; the 8192-token chunk over a 32768-token prefix (the
workload the benchmark times) and a ragged batch are compared on sampled
rows that the oracle computes one by one, plus properties of every row.
"""

import numpy as np
import pytest
import torch

import decode_attention_paged_05_amd as pad
import oracle
from decode_attention_paged_05_amd import inputs as gen
from tests.gpu_util import TOL, DeviceProblem, require_gpu, to_device

pytestmark = pytest.mark.gpu


class DevicePrefill:
    """A prefill problem on the GPU: packed queries, the cache holding every
    sequence's context and chunk (tiled layout unless asked otherwise)."""

    def __init__(self, pp: gen.PrefillProblem, keep_host=True, layouts=("tiled",)):
        require_gpu()
        self.pp = pp
        self.dp = DeviceProblem(pp.pool, keep_host=keep_host, layouts=layouts)
        self.query = to_device(pp.query, pp.spec.dtype)
        self.qs = torch.from_numpy(pp.query_start).cuda()
        self.ctx = torch.from_numpy(pp.context_lens).cuda()
        torch.cuda.synchronize()

    def run(self, kc=None, vc=None, tables=None, qs=None, ctx=None, out=None, scale=None):
        pp = self.pp
        if out is None:
            out = torch.full(tuple(pp.query.shape), float("nan"), dtype=torch.float32, device="cuda")
        pad.paged_attention_prefill(out, self.query, self.dp.kc if kc is None else kc,
                                    self.dp.vc if vc is None else vc, self.dp.tables if tables is None else tables,
                                    self.qs if qs is None else qs, self.ctx if ctx is None else ctx,
                                    pp.scale if scale is None else scale, pp.spec.num_kv_heads, 16, pp.max_query_len)
        torch.cuda.synchronize()
        return out

    def oracle(self, scale=None):
        pp = self.pp
        return oracle.prefill_attention(pp.query, self.dp.kc_host, self.dp.vc_host, pp.pool.block_tables,
                                        pp.query_start, pp.context_lens, pp.scale if scale is None else scale,
                                        pp.spec.num_kv_heads, 16, pp.spec.dtype)


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.double().cpu().numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want))) if want.size else 0.0


def test_prefill_small_ragged():
    """Five sequences: no context, a one-token chunk, several query tiles, an empty chunk."""
    dp = DevicePrefill(gen.make_prefill_problem("prefill_small"))
    got = dp.run()
    assert max_err(got, dp.oracle()) <= TOL["bf16"]


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 0.7])
def test_prefill_scale_sign_and_zero(scale):
    """The kernel applies the scale inside the exp2 argument and takes maxima over
    the raw logits, so the launcher turns a negative scale into a flipped query
    and 0 into a tiny positive one: each must still match the oracle (0 gives the
    mean of the visible values)."""
    dp = DevicePrefill(gen.make_prefill_problem("prefill_small"))
    got = dp.run(scale=scale)
    assert max_err(got, dp.oracle(scale=scale)) <= TOL["bf16"]


PREFILL_SHAPES = [
    # (H, Hkv, D, context_lens, query_lens): every head grouping the workgroup
    # shape distinguishes (1, 2 or 4 heads per workgroup) and every head size
    (4, 1, 64, (3, 100, 0), (70, 33, 129)),
    (8, 4, 128, (0, 64), (200, 17)),
    (6, 2, 256, (31, 5), (40, 96)),
    (8, 1, 128, (16, 250), (65, 31)),
    (32, 8, 64, (500,), (130,)),
    (24, 24, 128, (7, 0), (33, 64)),
    (24, 4, 256, (1000, 0, 1), (1, 1, 1)),
    # one sequence: the workgroup order that gives each XCD one KV head (or a
    # residue class of its token tiles, or every 8th head)
    (8, 1, 64, (0,), (512,)),
    (16, 2, 64, (50,), (256,)),
    (24, 24, 128, (300,), (200,)),
    # KV-head counts that neither divide 8 nor are a multiple of it: the
    # other workgroup order
    (12, 3, 128, (40, 7), (100, 64)),
    (10, 5, 64, (0,), (90,)),
]


@pytest.mark.parametrize("H,Hkv,D,ctx,qn", PREFILL_SHAPES, ids=lambda v: str(v))
def test_prefill_shapes(H, Hkv, D, ctx, qn):
    spec = gen.PrefillSpec("shape", context_lens=ctx, query_lens=qn, num_heads=H, num_kv_heads=Hkv, head_size=D,
                           dtype="bf16", seed=hash((H, Hkv, D, ctx, qn)) % 1000)
    dp = DevicePrefill(gen.make_prefill_problem(spec))
    assert max_err(dp.run(), dp.oracle()) <= TOL["bf16"]


def test_prefill_one_token_chunks_match_decode():
    """Chunks of one token are decode over the context plus that token: the
    prefill kernel agrees with the oracle and with the library's decode path."""
    spec = gen.PrefillSpec("one", context_lens=(1000, 0, 4097), query_lens=(1, 1, 1), num_heads=24, num_kv_heads=4,
                           head_size=256, dtype="bf16", seed=21)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp)
    got = dp.run()
    assert max_err(got, dp.oracle()) <= TOL["bf16"]
    dec = torch.full((3, 24, 256), float("nan"), dtype=torch.float32, device="cuda")
    pad.paged_attention_decode(dec, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables, dp.dp.lens, pp.scale, 4, 16, 0)
    torch.cuda.synchronize()
    assert float((got - dec).abs().max()) <= 2 * TOL["bf16"]


def _poison_chunk_slots(host_cache: np.ndarray, pp: gen.PrefillProblem) -> np.ndarray:
    c = host_cache.copy()
    nan = gen.poison_value(pp.spec.dtype)
    for s in range(pp.num_seqs):
        for i in range(int(pp.query_lens[s])):
            p = int(pp.context_lens[s]) + i
            c[int(pp.pool.block_tables[s, p // 16]), :, p % 16] = nan
    return c


def _upload(host_rows: np.ndarray, layout: str, dtype: str, kv: str):
    if layout == "rows":
        return to_device(host_rows, dtype)
    kt, vt = gen.to_tiled(host_rows, host_rows, dtype)
    return to_device(kt if kv == "k" else vt, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_write_kv_bitwise(dtype, layout):
    """The chunk write stores exactly the chunk's rows in their slots and changes nothing else."""
    spec = gen.PrefillSpec("write", context_lens=(0, 37, 16, 5), query_lens=(50, 1, 77, 0), num_heads=8,
                           num_kv_heads=2, head_size=128, dtype=dtype, seed=31)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp, layouts=(layout,))
    key, value = pp.chunk_kv()
    kc = _upload(_poison_chunk_slots(dp.dp.kc_host, pp), layout, dtype, "k")
    vc = _upload(_poison_chunk_slots(dp.dp.vc_host, pp), layout, dtype, "v")
    pad.paged_attention_prefill_write_kv(kc, vc, to_device(key, dtype), to_device(value, dtype), dp.dp.tables,
                                         dp.qs, dp.ctx, 2, 16, pp.max_query_len)
    torch.cuda.synchronize()
    iv = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(kc.view(iv), dp.dp.kc.view(iv)), "keys"
    assert torch.equal(vc.view(iv), dp.dp.vc.view(iv)), "values"


def test_write_then_prefill_matches_two_phase_form():
    """The whole step from the chunk's own rows (write, then attention) against
    the pages' two-phase form, which reads the chunk from those rows directly."""
    pp = gen.make_prefill_problem("prefill_small")
    dp = DevicePrefill(pp)
    key, value = pp.chunk_kv()
    kc_ctx = _poison_chunk_slots(dp.dp.kc_host, pp)
    vc_ctx = _poison_chunk_slots(dp.dp.vc_host, pp)
    kc = _upload(kc_ctx, "tiled", "bf16", "k")
    vc = _upload(vc_ctx, "tiled", "bf16", "v")
    pad.paged_attention_prefill_write_kv(kc, vc, to_device(key, "bf16"), to_device(value, "bf16"), dp.dp.tables,
                                         dp.qs, dp.ctx, 4, 16, pp.max_query_len)
    got = dp.run(kc=kc, vc=vc)
    want = oracle.prefix_attention_two_phase(pp.query, key, value, kc_ctx, vc_ctx, pp.pool.block_tables,
                                             pp.query_start, pp.context_lens, pp.scale, 4, 16, "bf16", 64)
    assert max_err(got, want) <= TOL["bf16"]


def _sampled_check(pp: gen.PrefillProblem, got: torch.Tensor, rows_per_seq, heads):
    """Oracle rows computed from the logical K/V of each sequence (one oracle
    call per (sequence, head) over the listed chunk tokens, on a thread pool)."""
    from concurrent.futures import ThreadPoolExecutor

    Hkv, H = pp.spec.num_kv_heads, pp.spec.num_heads
    G = H // Hkv
    g_host = got.double().cpu().numpy()
    jobs = []
    for s in range(pp.num_seqs):
        n, c, lo = int(pp.query_lens[s]), int(pp.context_lens[s]), int(pp.query_start[s])
        toks = np.array(sorted({t for t in rows_per_seq(n) if 0 <= t < n}), dtype=np.int64)
        if toks.size:
            jobs += [(s, h, n, c, lo, toks) for h in heads]
    kv = {}

    def rows_kv(s, g):
        if (s, g) not in kv:
            kv[(s, g)] = gen.sequence_kv(pp.pool, s, g)
        return kv[(s, g)]

    for s, g in sorted({(j[0], j[1] // G) for j in jobs}):
        rows_kv(s, g)

    def err(job):
        s, h, n, c, lo, toks = job
        K, V = kv[(s, h // G)]
        want = oracle.prefill_rows(pp.query[lo + toks, h], K, V, c, toks, pp.scale, pp.spec.dtype)
        return float(np.max(np.abs(g_host[lo + toks, h] - want)))

    with ThreadPoolExecutor(max_workers=gen.default_threads()) as ex:
        return max(ex.map(err, jobs), default=0.0)


def _edge_rows(n):
    return [0, 1, 15, 16, 31, 32, 33, 63, 64, 65, 127, 128, n // 2, n - 65, n - 64, n - 33, n - 32, n - 2, n - 1]


def _every_64th_and_edges(n):
    return list(range(0, n, 64)) + _edge_rows(n)


def test_prefill_full_size_sampled():
    """8192 new tokens over a 32768-token prefix (the timed workload, same launch):
    every row finite; every 64th chunk token and the tile edges of all 24 heads
    against the oracle (147 tokens x 24 heads)."""
    pp = gen.make_prefill_problem("prefill")
    dp = DevicePrefill(pp, keep_host=False)
    got = dp.run()
    assert bool(torch.isfinite(got).all())
    assert _sampled_check(pp, got, _every_64th_and_edges, heads=range(pp.spec.num_heads)) <= TOL["bf16"]


def test_prefill_ragged_batch_sampled():
    pp = gen.make_prefill_problem("prefill_batch")
    dp = DevicePrefill(pp, keep_host=False)
    got = dp.run()
    assert bool(torch.isfinite(got).all())
    assert _sampled_check(pp, got, _edge_rows, heads=(0, 7, 17, 23)) <= TOL["bf16"]


def test_prefill_repeatable():
    dp = DevicePrefill(gen.make_prefill_problem("prefill_small"), keep_host=False)
    a = dp.run()
    b = dp.run()
    assert torch.equal(a, b)


def test_prefill_sequence_order_does_not_change_rows():
    """Batches of up to 64 sequences are served heaviest first whatever their
    order: listing the same sequences in another order (tables, lengths and
    packed queries permuted together, same cache) gives every sequence
    bitwise the rows it had."""
    spec = gen.PrefillSpec("order", context_lens=(0, 300, 37, 2000, 5, 130), query_lens=(50, 1, 200, 77, 0, 64),
                           num_heads=8, num_kv_heads=2, head_size=256, dtype="bf16", seed=21)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp, keep_host=False)
    base = dp.run()
    qs = pp.query_start
    for perm in ([5, 4, 3, 2, 1, 0], [3, 0, 5, 1, 4, 2]):
        qn = pp.query_lens[perm]
        qs2 = np.zeros(len(perm) + 1, dtype=np.int32)
        qs2[1:] = np.cumsum(qn)
        rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in perm]).astype(np.int64)
        q2 = dp.query[torch.from_numpy(rows).cuda()].contiguous()
        out = torch.full(tuple(q2.shape), float("nan"), dtype=torch.float32, device="cuda")
        pad.paged_attention_prefill(out, q2, dp.dp.kc, dp.dp.vc, dp.dp.tables[torch.tensor(perm).cuda()].contiguous(),
                                    torch.from_numpy(qs2).cuda(), dp.ctx[torch.tensor(perm).cuda()].contiguous(),
                                    pp.scale, spec.num_kv_heads, 16, pp.max_query_len)
        torch.cuda.synchronize()
        assert torch.equal(out, base[torch.from_numpy(rows).cuda()]), f"order {perm}"


def test_prefill_batch_above_the_ordering_cap():
    """70 sequences: more than the on-device ordering ranks, so the given order
    is kept; every row against the oracle."""
    rng = np.random.default_rng(5)
    ctx = tuple(int(v) for v in rng.integers(0, 200, 70))
    qn = tuple(int(v) for v in rng.integers(0, 40, 70))
    spec = gen.PrefillSpec("many", context_lens=ctx, query_lens=qn, num_heads=4, num_kv_heads=2, head_size=128,
                           dtype="bf16", seed=22)
    dp = DevicePrefill(gen.make_prefill_problem(spec))
    assert max_err(dp.run(), dp.oracle()) <= TOL["bf16"]


def _run_mql(dp, mql, vc=None):
    pp = dp.pp
    out = torch.full(tuple(pp.query.shape), float("nan"), dtype=torch.float32, device="cuda")
    pad.paged_attention_prefill(out, dp.query, dp.dp.kc, dp.dp.vc if vc is None else vc, dp.dp.tables, dp.qs, dp.ctx,
                                pp.scale, pp.spec.num_kv_heads, 16, mql)
    torch.cuda.synchronize()
    return out


_LAYOUT_SPEC = gen.PrefillSpec("layouts", context_lens=(1000, 0, 37), query_lens=(700, 129, 300), num_heads=24,
                               num_kv_heads=4, head_size=256, dtype="bf16", seed=24)
_PAIRED_MQL, _SOLO_MQL = 700, 8192


def test_prefill_layouts_agree_bitwise():
    """Head size 256 has two layouts: paired (two waves share 32 rows, 128 rows
    per workgroup) and solo (a wave owns 32 rows over all of D, 256 rows).  The
    launcher picks by the longest chunk's workgroup count: with 24 / 4 heads a
    max_query_len of 700 gives 132 paired or 72 solo workgroups (one round of
    256 compute units either way: paired), 8192 gives 1536 or 768 (6 rounds
    against 3: solo).  Every output element sees the same matrix-core sequence
    in both, so one batch run with either bound gives the same bits, within
    the tolerance of the oracle."""
    pp = gen.make_prefill_problem(_LAYOUT_SPEC)
    dp = DevicePrefill(pp)
    paired, solo = _run_mql(dp, _PAIRED_MQL), _run_mql(dp, _SOLO_MQL)
    assert torch.equal(paired, solo)
    assert max_err(solo, dp.oracle()) <= TOL["bf16"]


def test_prefill_v_beyond_fp16_range_falls_back():
    """A V value beyond fp16's range (1e6, at sequence 1's last chunk position,
    which only that sequence's last row sees) makes the walks over it start
    over in the bf16 form: that row is within the bf16 form's relative
    precision of the oracle and the same in both layouts; every other row
    stays within the tolerance, and the rows of other sequences and KV heads,
    whose walks never read the outlier, keep the bits of a run without it."""
    pp = gen.make_prefill_problem(_LAYOUT_SPEC)
    dp = DevicePrefill(pp)
    s, g, d = 1, 1, 5
    clean = _run_mql(dp, _SOLO_MQL)
    pos = int(pp.context_lens[s] + pp.query_lens[s] - 1)
    blk, t = int(pp.pool.block_tables[s, pos // 16]), pos % 16
    big = torch.tensor(1e6, dtype=torch.bfloat16)
    dp.dp.vc[blk, g, d, t] = big.cuda()  # tiled V: [blocks, KV heads, D, 16]
    dp.dp.vc_host[blk, g, t, d] = big.view(torch.int16).numpy().astype(np.uint16)
    torch.cuda.synchronize()
    want = dp.oracle()
    paired, solo = _run_mql(dp, _PAIRED_MQL), _run_mql(dp, _SOLO_MQL)
    group = pp.spec.num_heads // pp.spec.num_kv_heads
    row, heads = int(pp.query_start[s + 1]) - 1, slice(g * group, (g + 1) * group)
    assert torch.equal(solo[row, heads], paired[row, heads])
    w = want[row, heads]
    got = solo[row, heads].double().cpu().numpy()
    assert np.max(np.abs(w)) > 100.0  # the outlier carries the row
    assert np.all(np.abs(got - w) <= TOL["bf16"] + 1e-4 * np.abs(w))
    keep = np.ones(want.shape[:2], dtype=bool)
    keep[row, heads] = False
    for out in (solo, paired):
        g_ = out.double().cpu().numpy()
        assert np.all(np.isfinite(g_))
        assert np.max(np.abs(g_ - want)[keep]) <= TOL["bf16"]
    # other sequences' walks and other KV heads never read the outlier: same bits
    others = torch.ones(solo.shape[:2], dtype=torch.bool, device=solo.device)
    others[int(pp.query_start[s]):int(pp.query_start[s + 1]), heads] = False
    assert torch.equal(solo[others], clean[others])


@pytest.mark.parametrize("D", [64, 256])
def test_prefill_peaked_row_keeps_its_tail(D):
    """One key 21.5 (log2 units) above 32 767 others, every V value 1: the
    weighted average must come out 1 (the oracle's definition, with every V
    equal, reduces to it).  With fp16 weights formed 2^7 below the reference
    the keys after the dominant one sit in fp16's subnormal range, holding
    about 1 % of the row's mass; were they flushed to zero, the rows would
    read 0.9905.  They read 0.9998: each step adds the tail's small weights to
    an fp32 accumulator holding the dominant one (128), and that rounding,
    the same in every step, is what is left.  Both launches."""
    spec = gen.PrefillSpec("peak", context_lens=(32767,), query_lens=(1,), num_heads=4, num_kv_heads=1,
                           head_size=D, dtype="bf16", seed=81)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp, keep_host=False)
    # logits: q . k = 8 * (-x) for every key but the dominant one (0): with scale
    # 1 / sqrt(D) the gap in log2 units is 8 x scale log2(e) = 21.46
    x = 21.46 / (8 * D ** -0.5 * 1.4426950408889634)
    q = torch.zeros_like(dp.query)
    q[:, :, 0] = 8.0
    kc = torch.zeros_like(dp.dp.kc)
    kc[:, :, 0, :, 0] = -x  # tiled K: [blocks, KV heads, D / 8, 16, 8]; dim 0
    dom = 5000
    kc[int(pp.pool.block_tables[0, dom // 16]), 0, 0, dom % 16, 0] = 0.0
    vc = torch.ones_like(dp.dp.vc)
    torch.cuda.synchronize()
    outs = []
    out = torch.full(tuple(pp.query.shape), float("nan"), dtype=torch.float32, device="cuda")
    pad.paged_attention_prefill(out, q, kc, vc, dp.dp.tables, dp.qs, dp.ctx, D ** -0.5, 1, 16, pp.max_query_len)
    outs.append(out)
    ws = pad.alloc_prefill_split_workspace(pp.num_seqs, 4, 1, D, pp.max_query_len, dp.dp.tables.shape[1])
    out2 = torch.full(tuple(pp.query.shape), float("nan"), dtype=torch.float32, device="cuda")
    pad.paged_attention_prefill_split(out2, q, kc, vc, dp.dp.tables, dp.qs, dp.ctx, D ** -0.5, 1, 16,
                                      pp.max_query_len, ws)
    outs.append(out2)
    torch.cuda.synchronize()
    for o in outs:
        assert float((o - 1.0).abs().max()) <= TOL["bf16"]


def test_prefill_tail_slots_do_not_reach_rows():
    """The cache slots past each sequence's last token (the tail of its last
    block) hold 1e30 instead of NaN: the solo walk zeroes them before its
    range check and P.V, so the rows keep their bits (an fp16 range failure
    there would have sent the walk to the bf16 form, with other bits)."""
    pp = gen.make_prefill_problem(_LAYOUT_SPEC)
    dp = DevicePrefill(pp, keep_host=False)
    base = _run_mql(dp, _SOLO_MQL)
    vc = dp.dp.vc.clone()
    for s in range(pp.num_seqs):
        end = int(pp.context_lens[s] + pp.query_lens[s])
        for pos in range(end, -(-end // 16) * 16):
            vc[int(pp.pool.block_tables[s, pos // 16]), :, :, pos % 16] = 1e30
    got = _run_mql(dp, _SOLO_MQL, vc=vc)
    assert torch.equal(got, base)


def test_prefill_block_outside_pool_gives_nan_rows():
    """A block id outside the pool (out of contract) makes that sequence's rows
    NaN and leaves the other sequences exact; nothing faults."""
    pp = gen.make_prefill_problem("prefill_small")
    dp = DevicePrefill(pp)
    tables = dp.dp.tables.clone()
    tables[2, 3] = pp.pool.num_blocks + 5
    got = dp.run(tables=tables)
    want = dp.oracle()
    lo, hi = int(pp.query_start[2]), int(pp.query_start[3])
    assert bool(torch.isnan(got[lo:hi]).all())
    keep = np.r_[0:lo, hi:pp.num_tokens]
    g = got[keep].double().cpu().numpy()
    assert np.max(np.abs(g - want[keep])) <= TOL["bf16"]


def test_prefill_chunk_longer_than_max_query_len():
    """A chunk longer than max_query_len is out of contract: the attention
    makes the rows the grid covers NaN and leaves the rest untouched, the
    chunk write writes none of its tokens; the other sequences are exact."""
    pp = gen.make_prefill_problem("prefill_small")  # chunks (50, 1, 77, 128, 0)
    dp = DevicePrefill(pp)
    want = dp.oracle()
    mq = 64  # the grid covers 64 tokens a sequence (heads 24 / 4, D 256: 64 per workgroup)
    out = torch.full(tuple(pp.query.shape), 7.0, dtype=torch.float32, device="cuda")
    pad.paged_attention_prefill(out, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables, dp.qs, dp.ctx, pp.scale, 4, 16, mq)
    torch.cuda.synchronize()
    o = out.cpu()
    for s in (2, 3):  # 77 and 128 tokens
        lo, hi = int(pp.query_start[s]), int(pp.query_start[s + 1])
        assert bool(torch.isnan(o[lo:lo + mq]).all()), s
        assert bool((o[lo + mq:hi] == 7.0).all()), s
    keep = np.r_[0:int(pp.query_start[2])]
    assert np.max(np.abs(o[keep].double().numpy() - want[keep])) <= TOL["bf16"]
    # the chunk write: sequences 2 and 3 untouched, 0 and 1 written
    key, value = pp.chunk_kv()
    kc_ctx = _poison_chunk_slots(dp.dp.kc_host, pp)
    vc_ctx = _poison_chunk_slots(dp.dp.vc_host, pp)
    kc = _upload(kc_ctx, "tiled", "bf16", "k")
    vc = _upload(vc_ctx, "tiled", "bf16", "v")
    before = kc.clone()
    pad.paged_attention_prefill_write_kv(kc, vc, to_device(key, "bf16"), to_device(value, "bf16"), dp.dp.tables,
                                         dp.qs, dp.ctx, 4, 16, mq)
    torch.cuda.synchronize()
    full_k = _upload(dp.dp.kc_host, "tiled", "bf16", "k")
    for s in range(4):
        ids = torch.as_tensor(sorted({int(pp.pool.block_tables[s, p // 16]) for p in
                                      range(int(pp.context_lens[s]), int(pp.context_lens[s] + pp.query_lens[s]))}),
                              dtype=torch.long, device="cuda")
        if s in (2, 3):
            assert torch.equal(kc[ids].view(torch.int16), before[ids].view(torch.int16)), f"sequence {s} written"
        elif ids.numel():
            assert torch.equal(kc[ids].view(torch.int16), full_k[ids].view(torch.int16)), f"sequence {s} not written"


def test_prefill_rejects_unsupported():
    pp = gen.make_prefill_problem("prefill_small")
    dp = DevicePrefill(pp, layouts=("rows",), keep_host=False)
    out = torch.empty(tuple(pp.query.shape), dtype=torch.float32, device="cuda")
    with pytest.raises(pad.PadError):
        pad.paged_attention_prefill(out, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables, dp.qs, dp.ctx, pp.scale, 4, 16,
                                    pp.max_query_len)


def test_prefill_graph_capture_replays():
    """The chunk write and the prefix attention captured in a HIP graph: every
    replay, with eager work and synchronisation in between, equals the eager
    result bitwise (no memset nodes, no host-side state)."""
    pp = gen.make_prefill_problem("prefill_small")
    dp = DevicePrefill(pp)
    key, value = pp.chunk_kv()
    kd, vd = to_device(key, "bf16"), to_device(value, "bf16")
    eager = dp.run()
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()

    def step():
        pad.paged_attention_prefill_write_kv(dp.dp.kc, dp.dp.vc, kd, vd, dp.dp.tables, dp.qs, dp.ctx, 4, 16,
                                             pp.max_query_len)
        pad.paged_attention_prefill(out, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables, dp.qs, dp.ctx, pp.scale, 4,
                                    16, pp.max_query_len)

    with torch.cuda.stream(stream):
        step()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            step()
    for r in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager result"
        assert torch.equal(dp.run(), eager)
    assert max_err(out, dp.oracle()) <= TOL["bf16"]


def test_prefill_two_streams():
    """Two prefill calls in flight at once on two streams: both exact."""
    a = DevicePrefill(gen.make_prefill_problem("prefill_small"))
    b = DevicePrefill(gen.make_prefill_problem(gen.PrefillSpec(
        "b", context_lens=(300, 0, 77), query_lens=(200, 333, 64), num_heads=24, num_kv_heads=4, head_size=256,
        dtype="bf16", seed=41)))
    ra, rb = a.oracle(), b.oracle()
    oa = torch.empty(tuple(a.pp.query.shape), dtype=torch.float32, device="cuda")
    ob = torch.empty(tuple(b.pp.query.shape), dtype=torch.float32, device="cuda")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        for dp, o, st in ((a, oa, sa), (b, ob, sb)):
            with torch.cuda.stream(st):
                pp = dp.pp
                pad.paged_attention_prefill(o, dp.query, dp.dp.kc, dp.dp.vc, dp.dp.tables, dp.qs, dp.ctx, pp.scale,
                                            4, 16, pp.max_query_len)
    torch.cuda.synchronize()
    assert max_err(oa, ra) <= TOL["bf16"]
    assert max_err(ob, rb) <= TOL["bf16"]


def test_prefill_long_chunk_no_context_sampled():
    """A 16384-token chunk with no cached context (the raised batched-token
    budget of the serving configuration): plain causal attention, the largest
    launch grid; sampled rows against the oracle."""
    spec = gen.PrefillSpec("chunk16k", context_lens=(0,), query_lens=(16384,), num_heads=24, num_kv_heads=4,
                           head_size=256, dtype="bf16", seed=42)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp, keep_host=False)
    got = dp.run()
    assert bool(torch.isfinite(got).all())
    assert _sampled_check(pp, got, _edge_rows, heads=(0, 11, 23)) <= TOL["bf16"]


@pytest.mark.parametrize("H,Hkv,D", [(64, 8, 64), (32, 8, 128), (16, 16, 128)])
def test_prefill_long_walks_small_heads_sampled(H, Hkv, D):
    """Head sizes 64 and 128 (the one-wave-per-row-group layout) over walks of
    hundreds of blocks: a 5000-token context with a 700-token chunk, and a
    second sequence with a 2000-token chunk over 1000 cached.  Sampled rows
    against the oracle, every row finite."""
    spec = gen.PrefillSpec(f"long_d{D}", context_lens=(5000, 1000), query_lens=(700, 2000), num_heads=H,
                           num_kv_heads=Hkv, head_size=D, dtype="bf16", seed=44)
    pp = gen.make_prefill_problem(spec)
    dp = DevicePrefill(pp, keep_host=False)
    got = dp.run()
    assert bool(torch.isfinite(got).all())
    G = H // Hkv
    heads = sorted({0, G - 1, G, H // 2, H - 1})
    assert _sampled_check(pp, got, _edge_rows, heads=heads) <= TOL["bf16"]
