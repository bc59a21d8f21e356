"""The C-ABI library on the host: exports, validation, workspace layout, the
one-pass/split choice and error strings.  No GPU work is enqueued here: every
call that takes device pointers is given arguments that fail validation, which
happens before any HIP call."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

import decode_attention_paged_05_amd as pad
from decode_attention_paged_05_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("paged_attention_decode.h", "paged_attention_prefill.h")]
GOLDEN = os.path.join(ROOT, "tests", "golden")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def header_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(paged_attention_\w+)\s*\(", text))
    return sorted(names)


def test_every_header_is_checked():
    assert sorted(os.path.basename(h) for h in HEADERS) == sorted(os.listdir(os.path.join(ROOT, "include")))


def test_header_symbols_exported():
    names = header_functions()
    assert names == sorted(B.EXPORTED)
    for n in names:
        assert hasattr(B.LIB, n), n
        assert callable(getattr(pad, n)), n


def dims(**kw):
    d = dict(dtype=1, num_seqs=1, num_heads=24, head_size=256, num_blocks=100, max_blocks_per_seq=10)
    d.update(kw)
    return B.PadDims(**d)


def call(partition=512, scale=0.0625, kv=4, bs=16, ws=FAKE, ws_bytes=1 << 30, d=None, ptrs=None):
    p = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, t=FAKE, l=FAKE)
    if ptrs:
        p.update(ptrs)
    return B.LIB.paged_attention_decode(p["out"], p["q"], p["k"], p["v"], p["t"], p["l"], scale, kv, bs, partition,
                                        ws, ws_bytes, ctypes.byref(d or dims()), None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=dims(dtype=7)), -2),
    (dict(d=dims(kv_layout=2)), -2),
    (dict(d=dims(num_heads=24), kv=5), -3),
    (dict(d=dims(num_seqs=-1)), -3),
    (dict(d=dims(num_blocks=0)), -3),
    (dict(d=dims(max_blocks_per_seq=0)), -3),
    (dict(scale=float("nan")), -3),
    (dict(scale=float("inf")), -3),
    (dict(d=dims(head_size=96)), -4),
    (dict(bs=32), -4),
    (dict(partition=500), -5),
    (dict(partition=-16), -5),
    (dict(ptrs=dict(q=0)), -1),
    (dict(ptrs=dict(out=0)), -1),
    (dict(ptrs=dict(t=0)), -1),
    (dict(ptrs=dict(k=FAKE + 8)), -7),
    (dict(ptrs=dict(l=FAKE + 2)), -7),
    (dict(ws=0), -6),
    (dict(ws_bytes=100), -6),
])
def test_argument_errors(kw, status):
    assert call(**kw) == status
    assert B.strerror(status) and "unknown" not in B.strerror(status)


def test_null_dims_and_phase_errors():
    assert B.LIB.paged_attention_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 4, 16, 0, None, 0, None, None) == -1
    d = dims()
    # phase 1 requires a split
    assert B.LIB.paged_attention_decode_phase1(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 4, 16, 0, FAKE, 1 << 30,
                                               ctypes.byref(d), None) == -5
    assert B.LIB.paged_attention_decode_phase1(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 4, 16, 512, FAKE, 10,
                                               ctypes.byref(d), None) == -6
    assert B.LIB.paged_attention_decode_phase2(FAKE, FAKE, 4, 16, 0, FAKE, 1 << 30, ctypes.byref(d), None) == -5
    assert B.LIB.paged_attention_decode_phase2(0, FAKE, 4, 16, 512, FAKE, 1 << 30, ctypes.byref(d), None) == -1
    assert B.LIB.paged_attention_decode_phase2(FAKE, FAKE, 4, 16, 512, FAKE, 10, ctypes.byref(d), None) == -6
    # the KV-head count must be that of phase 1: positive and a divisor of num_heads
    assert B.LIB.paged_attention_decode_phase2(FAKE, FAKE, 0, 16, 512, FAKE, 1 << 30, ctypes.byref(d), None) == -3
    assert B.LIB.paged_attention_decode_phase2(FAKE, FAKE, 5, 16, 512, FAKE, 1 << 30, ctypes.byref(d), None) == -3
    assert B.LIB.paged_attention_decode_workspace_init(FAKE, 10, 1, 24, 256, 10, 16, 512, None) == -6
    assert B.LIB.paged_attention_decode_workspace_init(FAKE, 1 << 30, 1, 24, 256, 10, 16, 100, None) == -5


def test_empty_batch_is_a_noop():
    # zero sequences: valid, nothing to do, no pointer needed
    assert B.LIB.paged_attention_decode(None, None, None, None, None, None, 1.0, 4, 16, 512, None, 0,
                                        ctypes.byref(dims(num_seqs=0)), None) == 0


def test_workspace_size_and_layout():
    S, H, D, W, bs, P = 1, 24, 256, 6250, 16, 512
    np_ = -(-W * bs // P)
    assert np_ == 196
    ml, es, tmp = pad.paged_attention_decode_workspace_layout(S, H, D, W, bs, P)
    assert ml == 0 and es % 256 == 0 and tmp % 256 == 0
    assert es >= S * H * np_ * 4 and tmp - es >= S * H * np_ * 4
    size = pad.paged_attention_decode_workspace_size(S, H, D, W, bs, P)
    # then the balanced split's launch record: 1029 words, 4352 bytes
    assert size == tmp + S * H * np_ * D * 4 + 4352 and size % 256 == 0
    assert pad.paged_attention_decode_workspace_size(S, H, D, W, bs, 0) == 0
    with pytest.raises(ValueError):
        pad.paged_attention_decode_workspace_size(S, H, D, W, bs, 100)


def test_workspace_matches_page_figures():
    """The second page's workspace message sizes tmp_output, exp_sums and
    max_logits for one sequence, 24 heads, 200 partitions and head size 256."""
    with open(os.path.join(GOLDEN, "partition_counts.json")) as f:
        g = json.load(f)["workspace_elements"][0]
    P, bs = 512, 16
    W = g["num_partitions"] * P // bs  # a table width that gives 200 partitions
    ml, es, tmp = pad.paged_attention_decode_workspace_layout(g["num_seqs"], g["num_heads"], g["head_size"], W, bs, P)
    size = pad.paged_attention_decode_workspace_size(g["num_seqs"], g["num_heads"], g["head_size"], W, bs, P)
    f32 = 4
    assert es - ml == -(-g["max_logits"] * f32 // 256) * 256
    assert tmp - es == -(-g["exp_sums"] * f32 // 256) * 256
    assert size - tmp == -(-g["tmp_output"] * f32 // 256) * 256 + 4352


def test_partition_counts_from_pages():
    with open(os.path.join(GOLDEN, "partition_counts.json")) as f:
        cases = json.load(f)["partition_counts"]
    for c in cases:
        # a table exactly as wide as the sequence gives the page's partition count
        W = -(-c["seq_len"] // 16)
        ml, es, tmp = pad.paged_attention_decode_workspace_layout(1, 1, 64, W, 16, c["partition_size"])
        assert (es - ml) // 4 >= c["num_partitions"] > (es - ml - 256) // 4


@pytest.mark.parametrize("S,H,Hkv,ctx,expect", [
    # split sizes: the largest P with (ceil(ctx / P) - 1) x S x workgroups per sequence >= 4 x 256
    (1, 24, 4, 100000, 256),      # 390 x 4 = 1560 >= 1024 (512: 195 x 4 = 780 is too few)
    (1, 24, 4, 32768, 128),       # none reaches 1024 (128: 255 x 4 = 1020): the smallest
    (1, 24, 4, 8192, 128),
    (4, 24, 4, 100000, 1024),     # 97 x 16 (2048: 48 x 16 = 768)
    (16, 24, 4, 2048, 128),       # none: the smallest
    (16, 24, 4, 8192, 256),       # 31 x 64 (512: 15 x 64 = 960)
    (64, 24, 4, 8192, 0),         # 256 (seq, KV head) workgroups: one per compute unit -> one-pass
    (256, 24, 4, 2048, 0),        # large batch
    (8, 24, 24, 131072, 2048),    # MHA: 63 x 8 x 24
    (32, 24, 4, 32768, 2048),     # 15 x 128
    (4, 24, 4, 512, 0),           # one partition's worth of context
    (1, 24, 4, 200, 0),
    (0, 24, 4, 100, 0),
])
def test_choose_partition(S, H, Hkv, ctx, expect):
    assert pad.paged_attention_decode_choose_partition(S, H, Hkv, ctx, 16, 256) == expect


def test_choose_partition_invalid():
    with pytest.raises(pad.PadError):
        pad.paged_attention_decode_choose_partition(1, 24, 5, 100, 16, 256)
    with pytest.raises(pad.PadError):
        pad.paged_attention_decode_choose_partition(1, 24, 4, 100, 32, 256)


# (S, max, total, expected): the batch rule's choices on the batches it was
# timed on (24 q / 4 KV heads, head 256, bf16, 256 compute units)
@pytest.mark.parametrize("S,mx,total,expect", [
    (256, 2048, 256 * 2048, 0),                 # equal lengths: one-pass
    (64, 8192, 64 * 8192, 0),
    (1024, 512, 1024 * 512, 0),
    (256, 65536, 255 * 1024 + 65536, 1024),     # one-pass 3421 us, split 279 us
    (132, 32768, 128 * 2048 + 4 * 32768, 1024),  # 781 us against 284 us
    (64, 3072, 63 * 1024 + 3072, 128),          # one-pass 91 us
    (64, 2048, 63 * 1024 + 2048, 0),            # 75 us; the best split 72 us
    (256, 2048, 255 * 1024 + 2048, 512),        # 231 us against 218 us
    (256, 32202, 1659008, 2048),                # log-uniform lengths: 2057 us against 1111 us
    (1, 100000, 100000, 256),
])
def test_choose_partition_for_batch(S, mx, total, expect):
    assert pad.paged_attention_decode_choose_partition_for_batch(S, 24, 4, 256, "bf16", mx, total, 16, 256) == expect


def test_choose_partition_for_batch_equal_lengths_and_slots():
    rng = np.random.default_rng(8)
    for _ in range(300):
        S = int(rng.integers(1, 600))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        H = Hkv * int(rng.choice([1, 2, 6, 20]))
        mx = int(rng.integers(1, 200000))
        fixed = pad.paged_attention_decode_choose_partition(S, H, Hkv, mx, 16, 256)
        # equal lengths: the fixed rule's choice
        assert pad.paged_attention_decode_choose_partition_for_batch(S, H, Hkv, 128, "bf16", mx, S * mx, 16,
                                                                     256) == fixed
        total = int(rng.integers(mx, S * mx + 1))
        P = pad.paged_attention_decode_choose_partition_for_batch(S, H, Hkv, 128, "bf16", mx, total, 16, 256)
        assert P in (0, 128, 256, 512, 1024, 2048)
        if fixed == 0 and mx <= 512:
            assert P == 0
        if P:
            wgs = Hkv * -(-(H // Hkv) // 16)
            ok = lambda p: (-(-mx // p) - 1) * total * wgs >= 4 * 256 * mx and -(-mx // p) >= 2
            # the largest size whose slots let the split launch its full width (else 128)
            assert ok(P) or P == 128
            assert all(not ok(q) for q in (256, 512, 1024, 2048) if q > P)


def test_choose_partition_for_batch_invalid():
    f = pad.paged_attention_decode_choose_partition_for_batch
    with pytest.raises(pad.PadError):
        f(4, 24, 4, 256, "bf16", 1000, 999, 16, 256)       # total below the maximum
    with pytest.raises(pad.PadError):
        f(4, 24, 4, 256, "bf16", 1000, 4001, 16, 256)      # total above S x maximum
    with pytest.raises(pad.PadError):
        f(4, 24, 4, 96, "bf16", 1000, 2000, 16, 256)       # head size
    with pytest.raises(pad.PadError):
        f(4, 24, 5, 256, "bf16", 1000, 2000, 16, 256)      # heads not a multiple of KV heads
    with pytest.raises(ValueError):
        f(4, 24, 4, 256, "f16", 1000, 2000, 16, 256)
    assert B.LIB.paged_attention_decode_choose_partition_for_batch(4, 24, 4, 256, 7, 1000, 2000, 16, 256) < 0


def test_strerror_never_null():
    for s in list(range(-8, 1)) + [1, 98, 12345]:
        assert isinstance(B.strerror(s), str) and B.strerror(s)


def test_one_hip_runtime_in_process():
    """libpad.so must share torch's HIP runtime (streams and memory are its
    objects); a second libamdhip64 in the process breaks every launch."""
    maps = open("/proc/self/maps").read().splitlines()
    runtimes = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(runtimes) == 1, runtimes


def pdims(**kw):
    d = dict(dtype=1, num_seqs=2, num_tokens=100, num_heads=24, head_size=256, max_query_len=64, num_blocks=100,
             max_blocks_per_seq=10, kv_layout=1)
    d.update(kw)
    return B.PadPrefillDims(**d)


def prefill_call(d=None, kv=4, bs=16, scale=0.0625, ptrs=None):
    p = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, t=FAKE, qs=FAKE, c=FAKE)
    if ptrs:
        p.update(ptrs)
    return B.LIB.paged_attention_prefill(p["out"], p["q"], p["k"], p["v"], p["t"], p["qs"], p["c"], scale, kv, bs,
                                         ctypes.byref(d or pdims()), None)


def write_call(d=None, kv=4, bs=16, ptrs=None):
    p = dict(kc=FAKE, vc=FAKE, k=FAKE, v=FAKE, t=FAKE, qs=FAKE, c=FAKE)
    if ptrs:
        p.update(ptrs)
    return B.LIB.paged_attention_prefill_write_kv(p["kc"], p["vc"], p["k"], p["v"], p["t"], p["qs"], p["c"], kv, bs,
                                                  ctypes.byref(d or pdims()), None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=pdims(dtype=0)), -4),            # the attention kernels are bf16
    (dict(d=pdims(kv_layout=0)), -4),        # and tiled
    (dict(d=pdims(dtype=3)), -2),
    (dict(d=pdims(kv_layout=2)), -2),
    (dict(kv=5), -3),
    (dict(d=pdims(num_tokens=-1)), -3),
    (dict(d=pdims(max_query_len=-1)), -3),
    (dict(d=pdims(num_blocks=0)), -3),
    (dict(d=pdims(head_size=96)), -4),
    (dict(bs=32), -4),
    (dict(scale=float("nan")), -3),
    (dict(d=pdims(num_tokens=1 << 20)), -4),  # 32-bit offsets inside the kernel
    (dict(ptrs=dict(qs=0)), -1),
    (dict(ptrs=dict(out=0)), -1),
    (dict(ptrs=dict(k=FAKE + 8)), -7),
    (dict(ptrs=dict(c=FAKE + 2)), -7),
])
def test_prefill_argument_errors(kw, status):
    assert prefill_call(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(d=pdims(dtype=3)), -2),
    (dict(d=pdims(head_size=48)), -4),
    (dict(kv=0), -3),
    (dict(ptrs=dict(kc=0)), -1),
    (dict(ptrs=dict(v=FAKE + 4)), -7),
])
def test_prefill_write_argument_errors(kw, status):
    assert write_call(**kw) == status


def split_call(ws=FAKE, ws_bytes=1 << 30, d=None, ptrs=None):
    p = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, t=FAKE, qs=FAKE, c=FAKE)
    if ptrs:
        p.update(ptrs)
    return B.LIB.paged_attention_prefill_split(p["out"], p["q"], p["kc"], p["vc"], p["t"], p["qs"], p["c"], 0.1, 4,
                                               16, ctypes.byref(d or pdims()), ws, ws_bytes, None)


def test_prefill_split_argument_errors():
    """Validation of the split launch, all before any HIP call: the prefill
    checks, then the workspace pointer and its alignment."""
    assert split_call(d=pdims(head_size=96)) == -4
    assert split_call(d=pdims(dtype=0)) == -4
    assert split_call(ptrs=dict(q=0)) == -1
    assert split_call(ws=None) == -6
    assert split_call(ws=FAKE + 8) == -7
    assert split_call(ws=None, d=pdims(num_seqs=0)) == 0  # nothing to do: no workspace needed


def walk_steps(ctx, n, tpw):
    """32-key steps of every token tile's walk: the tile's last row sees
    positions 0 .. ctx + min((t + 1) tpw, n) - 1."""
    return [-(-(ctx + min((t + 1) * tpw, n)) // 32) for t in range(-(-n // tpw))]


@pytest.mark.parametrize("seed", range(6))
def test_prefill_choose_split_rule(seed):
    """The split is chosen for a batch (more than one sequence with chunk
    tokens), and for one sequence exactly when its longest walk is more than
    half of a resident workgroup's share of all walks' steps (every KV head
    and head chunk walks the same steps)."""
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 40))
    ctx = rng.integers(0, 40000, S) * (rng.random(S) < 0.8)
    qn = rng.integers(0, 3000, S)
    H, Hkv, D, N = [(24, 4, 256, 256), (32, 8, 128, 256), (64, 8, 64, 512), (12, 12, 128, 256)][seed % 4]
    G = H // Hkv
    hc = 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    tpw = 256 // hc
    steps = [st for c, n in zip(ctx, qn) for st in walk_steps(int(c), int(n), tpw)]
    busy = int(np.count_nonzero(qn))
    want = busy > 1 or (bool(steps) and max(steps) * 2 * N > sum(steps) * Hkv * (G // hc))
    assert pad.paged_attention_prefill_choose_split(ctx, qn, H, Hkv, D, N) == want
    # one sequence alone: the cut rule decides
    for s in range(min(S, 8)):
        one = walk_steps(int(ctx[s]), int(qn[s]), tpw)
        want1 = bool(one) and max(one) * 2 * N > sum(one) * Hkv * (G // hc)
        assert pad.paged_attention_prefill_choose_split(ctx[s:s + 1], qn[s:s + 1], H, Hkv, D, N) == want1


def test_prefill_choose_split_workloads():
    """One chunk over a long prefix: its walks are short beside the total (no
    cut, the plain launch); the ragged batch: the split; one short chunk over a
    long context (few, long walks): the split, which cuts them."""
    from decode_attention_paged_05_amd import inputs as gen

    for name, want in (("prefill", False), ("prefill_batch", True)):
        pp = gen.make_prefill_problem(name)
        s = pp.spec
        assert pad.paged_attention_prefill_choose_split(pp.context_lens, pp.query_lens, s.num_heads, s.num_kv_heads,
                                                        s.head_size, 256) == want, name
    assert pad.paged_attention_prefill_choose_split([100000], [256], 24, 4, 256, 256)
    assert pad.paged_attention_prefill_choose_split([100000, 7], [256, 0], 24, 4, 128, 256)  # one busy: cut
    assert not pad.paged_attention_prefill_choose_split([32768, 7], [8192, 0], 24, 4, 256, 256)  # one busy: no cut
    with pytest.raises(pad.PadError):
        pad.paged_attention_prefill_choose_split([5, -1], [3, 3], 24, 4, 256, 256)


def test_prefill_split_workspace_size():
    size = pad.paged_attention_prefill_split_workspace_size
    base = size(4, 24, 4, 256, 3000, 2063, 256)  # the ragged batch: contexts up to 33 000 positions
    assert base > 0
    assert size(8, 24, 4, 256, 3000, 2063, 256) > base  # more sequences: more whole walks listed
    assert size(4, 24, 4, 128, 3000, 2063, 256) < base  # smaller partial slots
    # the batch's 376 pieces x 3 head chunks fit: 1 128 slots of 256 rows x 256 floats
    assert base >= 1128 * 256 * 256 * 4
    # no walk of a 16-block table can be cut (at most 8 steps): no partial slots at all
    assert size(4, 24, 4, 256, 3000, 16, 256) < 1 << 20
    with pytest.raises(pad.PadError):
        size(4, 24, 5, 256, 3000, 2063, 256)


def test_prefill_empty_is_a_noop():
    assert B.LIB.paged_attention_prefill(None, None, None, None, None, None, None, 1.0, 4, 16,
                                         ctypes.byref(pdims(num_seqs=0)), None) == 0
    assert B.LIB.paged_attention_prefill(None, None, None, None, None, None, None, 1.0, 4, 16,
                                         ctypes.byref(pdims(num_tokens=0)), None) == 0
    assert B.LIB.paged_attention_prefill_write_kv(None, None, None, None, None, None, None, 4, 16,
                                                  ctypes.byref(pdims(max_query_len=0)), None) == 0


# ---------------------------------------------------------------------------
# where phase 1 puts its entries (the host copy of the device rule)
# ---------------------------------------------------------------------------

def check_entry_plan(lens, H, Hkv, W, P, cus=256, layout="tiled", D=256, dtype="bf16"):
    """The invariants phase 2 relies on, for any lengths: every (sequence, head)
    with a valid non-empty length has entries that tile [0, L) in slot order,
    each a run of whole blocks (the last cut at L), no more than NP of them;
    the heads of one KV head share them."""
    import numpy as np

    bal, cnt, lo, hi = pad.paged_attention_decode_entry_ranges(lens, H, Hkv, W, 16, P, cus, layout, D, dtype)
    NP = -(-W * 16 // P)
    G = H // Hkv
    for s, L in enumerate(lens):
        for h in range(H):
            n = int(cnt[s, h])
            if L == 0:
                assert n == 0
                continue
            if L < 0 or L > W * 16:
                assert n == -1
                continue
            assert 1 <= n <= NP, (s, h, n, NP)
            b, e = lo[s, h, :n], hi[s, h, :n]
            assert b[0] == 0 and e[-1] == L and np.all(b[1:] == e[:-1]) and np.all(e > b), (s, h)
            assert np.all(b % 16 == 0)
            if not bal:
                assert np.array_equal(b, np.arange(n) * P)
            assert np.array_equal(cnt[s, h], cnt[s, (h // G) * G])
            assert np.array_equal(b, lo[s, (h // G) * G, :n])
    items = len(lens) * Hkv * NP
    expect_bal = items > cus and len(lens) <= 1024 and NP >= 2
    assert bal == expect_bal
    return bal, cnt, lo, hi


@pytest.mark.parametrize("seed", range(40))
def test_entry_plan_random_batches(seed):
    import numpy as np

    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 70))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    H = Hkv * int(rng.choice([1, 3, 6, 8]))
    W = int(rng.integers(1, 3000))
    P = int(rng.choice([16, 64, 256, 512, 1024]))
    lens = rng.integers(0, W * 16 + 1, size=S)
    lens[rng.random(S) < 0.1] = 0
    if S > 3:
        lens[1] = W * 16 + 7  # out of contract
    check_entry_plan(lens.tolist(), H, Hkv, W, P, cus=int(rng.choice([80, 256, 304])),
                     layout=str(rng.choice(["tiled", "rows"])), D=int(rng.choice([64, 128, 256])),
                     dtype=str(rng.choice(["bf16", "f32"])))


def test_entry_plan_long_context():
    # one 100 000-token sequence, 24 q / 4 KV heads, P 512: 196 partition slots;
    # 512 ranges (two per compute unit) of 48 or 49 blocks; each KV head's 6250
    # blocks are exactly a quarter of the 25 000 units, so every head gets 128
    # entries
    bal, cnt, lo, hi = check_entry_plan([100000], 24, 4, 6250, 512)
    assert bal
    assert set(cnt[0].tolist()) == {128} and cnt.sum() // 6 == 512
    sizes = (hi[0, 0, :cnt[0, 0]] - lo[0, 0, :cnt[0, 0]])
    assert set(((sizes + 15) // 16).tolist()) <= {48, 49} and sizes.max() <= 49 * 16
    # the rows layout launches three workgroups per compute unit: 768 ranges of 32 or 33 blocks
    bal, cnt, lo, hi = check_entry_plan([100000], 24, 4, 6250, 512, layout="rows")
    assert bal and set(cnt[0].tolist()) == {192} and cnt.sum() // 6 == 768
    # smaller heads in the tiled layout, four: 1024 ranges of 48 or 49 blocks (P 256 leaves the slots)
    bal, cnt, lo, hi = check_entry_plan([100000], 64, 8, 6250, 256, D=64)
    assert bal and set(cnt[0].tolist()) == {128} and cnt.sum() // 8 == 1024
    # fp32 in the tiled layout at head size 256, three: 768 ranges, as the rows layout
    bal, cnt, lo, hi = check_entry_plan([100000], 24, 4, 6250, 512, dtype="f32")
    assert bal and set(cnt[0].tolist()) == {192} and cnt.sum() // 6 == 768


def test_entry_plan_workloads():
    from decode_attention_paged_05_amd import inputs as gen

    for name in ("tiny", "short", "long", "mixed", "stress"):
        p = gen.make_problem(name)
        if p.partition_size:
            check_entry_plan(p.seq_lens.tolist(), p.num_heads, p.num_kv_heads, p.max_blocks_per_seq,
                             p.partition_size)


def test_entry_plan_argument_errors():
    with pytest.raises(pad.PadError):
        pad.paged_attention_decode_entry_ranges([10], 24, 4, 10, 16, 0)
    with pytest.raises(pad.PadError):
        pad.paged_attention_decode_entry_ranges([10], 24, 5, 10, 16, 512)
    with pytest.raises(pad.PadError):
        pad.paged_attention_decode_entry_ranges([10], 24, 4, 10, 16, 512, num_cus=0)
    with pytest.raises(ValueError):
        pad.paged_attention_decode_entry_ranges([10], 24, 4, 10, 16, 512, layout="nhd")
    with pytest.raises(pad.PadError):
        pad.paged_attention_decode_entry_ranges([10], 24, 4, 10, 16, 512, head_size=96)
    with pytest.raises(ValueError):
        pad.paged_attention_decode_entry_ranges([10], 24, 4, 10, 16, 512, dtype="f16")
    lens = (ctypes.c_int32 * 1)(10)
    out = (ctypes.c_int32 * 64)()
    assert B.LIB.paged_attention_decode_entry_ranges(lens, 1, 24, 4, 256, 1, 10, 16, 512, 7, 256, out, out, out) < 0
    assert B.LIB.paged_attention_decode_entry_ranges(lens, 1, 24, 4, 256, 9, 10, 16, 512, 1, 256, out, out,
                                                     out) == -2


def test_no_alloc_rejects_what_does_not_fit():
    """The allocation-free entry point checks its workspace need against the
    static 64 MiB before any HIP call; other errors are those of
    paged_attention_decode."""
    def na(d, partition=512, ptrs=None):
        p = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, t=FAKE, l=FAKE)
        if ptrs:
            p.update(ptrs)
        return B.LIB.paged_attention_decode_no_alloc(p["out"], p["q"], p["k"], p["v"], p["t"], p["l"], 0.0625, 4, 16,
                                                     partition, ctypes.byref(d), None)
    big = dims(max_blocks_per_seq=100000)  # 3125 partition slots x 24 heads x 258 floats: 77 MB
    assert pad.paged_attention_decode_workspace_size(1, 24, 256, 100000, 16, 512) > 64 << 20
    assert na(big) == -8
    assert "64 MiB" in B.strerror(-8)
    assert na(dims(num_seqs=3, max_blocks_per_seq=40000)) == -8
    assert na(dims(num_seqs=6, max_blocks_per_seq=100000), partition=16) == -8  # the GPU test's case
    assert na(dims(dtype=7)) == -2
    assert na(dims(), partition=500) == -5
    assert na(dims(), ptrs=dict(out=0)) == -1
    assert na(dims(), ptrs=dict(q=FAKE + 4)) == -7
    assert B.LIB.paged_attention_decode_no_alloc(None, None, None, None, None, None, 1.0, 4, 16, 512,
                                                 ctypes.byref(dims(num_seqs=0)), None) == 0


def test_source_folders_hold_sources_only():
    """The build id hashes every file under csrc/ and include/: a stray object or
    listing there gives a library whose id no clean checkout reproduces."""
    for d, exts in ((os.path.join(ROOT, "decode_attention_paged_05_amd", "csrc"), (".hip", ".hpp", ".h", ".cpp")),
                    (os.path.join(ROOT, "include"), (".h",))):
        stray = [n for n in os.listdir(d) if not n.endswith(exts)]
        assert not stray, f"{d}: {stray}"


def test_library_built_from_these_sources():
    """The loaded library's build id is the hash of csrc/ and include/ as they
    stand (a stale build fails here before any GPU run)."""
    bid = pad.check_build()
    assert len(bid) == 16 and int(bid, 16) >= 0


def test_sequence_strides_validated():
    """query_seq_stride / out_seq_stride: 0 (contiguous) or at least one
    sequence's rows, and a whole number of 16-byte units."""
    row = 24 * 256
    assert call(d=dims(query_seq_stride=row - 8)) == -3
    assert call(d=dims(out_seq_stride=row - 4)) == -3
    assert call(d=dims(query_seq_stride=-row)) == -3
    assert call(d=dims(query_seq_stride=row + 4)) == -7  # 8 bytes past a multiple of 16 (bf16)
    assert call(d=dims(out_seq_stride=row + 2)) == -7
    d = dims(out_seq_stride=row - 4)
    assert B.LIB.paged_attention_decode_phase2(FAKE, FAKE, 4, 16, 512, FAKE, 1 << 30, ctypes.byref(d), None) == -3


def _model_entry_plan(lens, H, Hkv, W, P, cus, wgs_per_cu=2, min_blocks=8):
    """The balanced split written out in Python from its description: the live
    (block, head group) units laid end to end, N equal ranges, one entry per
    (range, head group) they share, slot = range - owner of the head group's
    first unit.  Returns (balanced, {(s, h): [(lo, hi), ...]})."""
    import math

    G = H // Hkv
    chunks = -(-G // 16)
    gyc = Hkv * chunks
    NP = -(-W * 16 // P)
    S = len(lens)
    if not (S * gyc * NP > cus and S <= 1024 and NP >= 2 and S * W < 2**31):
        plan = {}
        for s, L in enumerate(lens):
            if 0 < L <= W * 16:
                for h in range(H):
                    plan[(s, h)] = [(e * P, min((e + 1) * P, L)) for e in range(-(-L // P))]
        return False, plan
    nb = [(-(-L // 16) if 0 < L <= W * 16 else 0) for L in lens]
    B = gyc * sum(nb)
    if B == 0:
        return True, {}
    nmax = max(nb)
    n = wgs_per_cu * cus
    n = min(n, (NP - 1) * B // nmax)            # at most NP entries a head group
    n = min(n, -(-B // min_blocks))             # at least min_blocks units a range
    if n > cus:
        n = n // cus * cus
    N = max(n, 1)
    starts = [j * B // N for j in range(N + 1)]
    plan = {}
    off = 0
    for s in range(S):
        for gy in range(gyc):
            g0, g1 = off, off + nb[s]
            off = g1
            if nb[s] == 0:
                continue
            pieces = []
            for j in range(N):
                a, b = max(starts[j], g0), min(starts[j + 1], g1)
                if a < b:
                    pieces.append((j, (a - g0) * 16, min((b - g0) * 16, lens[s])))
            first = pieces[0][0]
            assert all(j - first == k for k, (j, _, _) in enumerate(pieces))
            g = gy // chunks
            hc = gy % chunks
            for h in range(g * G + hc * 16, g * G + min(G, hc * 16 + 16)):
                plan[(s, h)] = [(lo, hi) for _, lo, hi in pieces]
    return True, plan


@pytest.mark.parametrize("seed", range(25))
def test_entry_plan_matches_model(seed):
    """The library's host plan equals the Python model of the balanced split
    (and of one workgroup per partition) slot for slot."""
    import numpy as np

    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(1, 50))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    H = Hkv * int(rng.choice([1, 3, 6, 20]))
    W = int(rng.integers(1, 2500))
    P = int(rng.choice([16, 64, 512, 1024]))
    cus = int(rng.choice([80, 256, 304]))
    layout = ("tiled", "rows")[seed % 2]
    D = (64, 128, 256)[seed % 3]
    lens = rng.integers(0, W * 16 + 1, size=S)
    lens[rng.random(S) < 0.15] = 0
    bal, cnt, lo, hi = pad.paged_attention_decode_entry_ranges(lens, H, Hkv, W, 16, P, cus, layout, D)
    # workgroups per compute unit: tiled 2 at head size 256 and 4 below, rows 3
    wpc = 3 if layout == "rows" else (2 if D == 256 else 4)
    mbal, model = _model_entry_plan(lens.tolist(), H, Hkv, W, P, cus, wgs_per_cu=wpc)
    assert bal == mbal
    for s in range(S):
        for h in range(H):
            want = model.get((s, h), [])
            n = int(cnt[s, h])
            assert n == (len(want) if lens[s] > 0 else 0), (s, h)
            assert [(int(lo[s, h, e]), int(hi[s, h, e])) for e in range(n)] == want, (s, h)
