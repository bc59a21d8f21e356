"""Checks that pin the prefix-attention (prefill) oracle to things other than itself.

Each ``pin_*`` function takes the ``oracle.prefill`` module and raises
``AssertionError`` when it disagrees with what the pages or the mathematics
fix:

* brute force: pure-Python loops over unpaged rows (context followed by the
  chunk) with the causal rule written out, no block table, no NumPy arithmetic;
* the pages' own two-phase form (context tiles from the cache, then the
  chunk's tiles under the causal mask) for several tile sizes;
* reduction to decode: a chunk of one token is single-token decode over the
  context plus that token;
* a library special case: float64 ``scaled_dot_product_attention`` with the
  explicit prefix-causal mask (and ``is_causal`` with no context);
* closed forms: a zero query gives the running mean of V, the first token of
  a chunk with no context gives V_0;
* invariants: physical-block permutation (bitwise), causality (later chunk
  rows never change earlier outputs, bitwise), splitting a chunk in two
  (bitwise);
* the chunk write: every chunk row lands in the slot of its position, and
  nothing else changes.
"""

from __future__ import annotations

import math

import numpy as np

import oracle.attention as dec
from tests.oracle_pins import decode_bits, store


def make_case(rng, dtype, ctx_lens, n_lens, H, Hkv, D, bs, extra_blocks=3, identity=False, spread=1.0):
    """A paged problem whose cache holds every sequence's context and chunk rows.

    Returns a dict with the storage-format arrays, the logical rows per
    sequence (``lk[s]``, ``lv[s]`` [Hkv, ctx + n, D]), the packed query [T, H, D]
    and the chunk's own key / value rows [T, Hkv, D].
    """
    S = len(ctx_lens)
    tot = [c + n for c, n in zip(ctx_lens, n_lens)]
    lk = [store(rng.standard_normal((Hkv, L, D)), dtype) for L in tot]
    lv = [store(rng.standard_normal((Hkv, L, D)), dtype) for L in tot]
    qs = np.zeros(S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(n_lens)
    T = int(qs[-1])
    q = store(rng.standard_normal((T, H, D)) * spread, dtype)
    key = np.concatenate([lk[s][:, ctx_lens[s]:].transpose(1, 0, 2) for s in range(S)], axis=0) if T else \
        store(np.zeros((0, Hkv, D)), dtype)
    value = np.concatenate([lv[s][:, ctx_lens[s]:].transpose(1, 0, 2) for s in range(S)], axis=0) if T else \
        store(np.zeros((0, Hkv, D)), dtype)
    nbs = [-(-L // bs) for L in tot]
    NB = sum(nbs) + extra_blocks
    W = max(max(nbs), 1)
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    sd = np.float32 if dtype == "f32" else np.uint16
    kc = np.full((NB, Hkv, bs, D), nan, dtype=sd)
    vc = np.full((NB, Hkv, bs, D), nan, dtype=sd)
    ids = np.arange(NB) if identity else rng.permutation(NB)
    tables = np.full((S, W), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        for j in range(nbs[s]):
            b = int(ids[off]); off += 1
            tables[s, j] = b
            lo, hi = j * bs, min((j + 1) * bs, tot[s])
            kc[b, :, : hi - lo] = lk[s][:, lo:hi]
            vc[b, :, : hi - lo] = lv[s][:, lo:hi]
    return dict(q=q, key=key, value=value, kc=kc, vc=vc, tables=tables, qs=qs,
                ctx=np.asarray(ctx_lens, dtype=np.int32), lk=lk, lv=lv, H=H, Hkv=Hkv, D=D, bs=bs, dtype=dtype)


def run(orc, c, scale):
    return orc.prefill_attention(c["q"], c["kc"], c["vc"], c["tables"], c["qs"], c["ctx"], scale,
                                 c["Hkv"], c["bs"], c["dtype"])


def brute_force(c, scale):
    """Pure-Python prefix attention over the logical rows: chunk token i of
    sequence s sees positions 0 .. ctx + i."""
    conv = (lambda x: float(x)) if c["dtype"] == "f32" else decode_bits
    q, qs, ctx = c["q"], c["qs"], c["ctx"]
    H, D = c["H"], c["D"]
    group = H // c["Hkv"]
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(len(ctx)):
        for i in range(int(qs[s + 1]) - int(qs[s])):
            t = int(qs[s]) + i
            for h in range(H):
                g = h // group
                qq = [conv(q[t, h, d]) for d in range(D)]
                logits = []
                for j in range(int(ctx[s]) + i + 1):
                    acc = 0.0
                    for d in range(D):
                        acc += qq[d] * conv(c["lk"][s][g, j, d])
                    logits.append(scale * acc)
                mx = max(logits)
                ws = [math.exp(x - mx) for x in logits]
                tot = math.fsum(ws)
                for d in range(D):
                    out[t, h, d] = math.fsum(ws[j] * conv(c["lv"][s][g, j, d]) for j in range(len(ws))) / tot
    return out


SHAPES = [
    dict(dtype="f32", ctx=(5, 0), n=(3, 4), H=4, Hkv=2, D=6, bs=4),
    dict(dtype="bf16", ctx=(9,), n=(6,), H=6, Hkv=2, D=4, bs=4),
    dict(dtype="bf16", ctx=(0, 16, 3), n=(1, 5, 0), H=3, Hkv=3, D=5, bs=16),
    dict(dtype="f32", ctx=(2, 7), n=(7, 1), H=2, Hkv=1, D=3, bs=2),
]


def pin_prefill_brute_force(orc):
    rng = np.random.default_rng(21)
    for sh in SHAPES:
        c = make_case(rng, sh["dtype"], sh["ctx"], sh["n"], sh["H"], sh["Hkv"], sh["D"], sh["bs"])
        got = run(orc, c, 0.41)
        want = brute_force(c, float(np.float32(0.41)))
        assert np.all(np.isfinite(got)), "oracle output not finite"
        assert np.max(np.abs(got - want)) <= 1e-12, (sh, np.max(np.abs(got - want)))


def pin_prefill_two_phase(orc):
    """The pages' tiled two-phase form reaches the plain result for every tile size."""
    rng = np.random.default_rng(22)
    for dtype in ("f32", "bf16"):
        c = make_case(rng, dtype, (13, 0, 40), (9, 6, 17), 6, 2, 8, 4, spread=2.0)
        plain = run(orc, c, 0.7)
        for tile in (1, 3, 4, 16, 64):
            got = orc.prefix_attention_two_phase(c["q"], c["key"], c["value"], c["kc"], c["vc"], c["tables"],
                                                 c["qs"], c["ctx"], 0.7, c["Hkv"], c["bs"], dtype, tile)
            assert np.max(np.abs(got - plain)) <= 1e-12, ("two-phase", tile)


def pin_prefill_decode_reduction(orc):
    """One chunk token is decode over the context plus that token."""
    rng = np.random.default_rng(23)
    for dtype in ("f32", "bf16"):
        c = make_case(rng, dtype, (11, 0, 32), (1, 1, 1), 4, 2, 8, 4)
        got = run(orc, c, 0.3)
        lens = c["ctx"] + 1
        want = dec.decode_attention(c["q"], c["kc"], c["vc"], c["tables"], lens, 0.3, c["Hkv"], c["bs"], dtype)
        assert np.max(np.abs(got - want)) <= 1e-12, "decode reduction"


def pin_prefill_sdpa(orc):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(24)
    for dtype in ("f32", "bf16"):
        for ctx in (0, 10):
            n, H, Hkv, D, bs = 7, 6, 2, 16, 4
            c = make_case(rng, dtype, (ctx,), (n,), H, Hkv, D, bs, identity=True)
            got = run(orc, c, 0.25)
            qt = torch.from_numpy(dec.widen(c["q"], dtype)).permute(1, 0, 2).unsqueeze(0)     # [1, H, n, D]
            kt = torch.from_numpy(dec.widen(c["lk"][0], dtype)).unsqueeze(0)                  # [1, Hkv, ctx+n, D]
            vt = torch.from_numpy(dec.widen(c["lv"][0], dtype)).unsqueeze(0)
            if ctx == 0:
                ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.25, is_causal=True, enable_gqa=True)
            else:
                mask = torch.arange(ctx + n)[None, :] <= (ctx + torch.arange(n))[:, None]
                ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.25, enable_gqa=True)
            ref = ref[0].permute(1, 0, 2).numpy()
            assert np.max(np.abs(got - ref)) <= 1e-12, ("float64 SDPA special case", ctx)


def pin_prefill_closed_forms(orc):
    rng = np.random.default_rng(25)
    for dtype in ("f32", "bf16"):
        c = make_case(rng, dtype, (6, 0), (5, 4), 4, 2, 6, 4)
        c["q"] = store(np.zeros(c["q"].shape), dtype)
        got = run(orc, c, 0.5)
        for s in range(2):
            for i in range(int(c["qs"][s + 1] - c["qs"][s])):
                for h in range(4):
                    vv = dec.widen(c["lv"][s][h // 2, : int(c["ctx"][s]) + i + 1], dtype)
                    assert np.max(np.abs(got[int(c["qs"][s]) + i, h] - vv.mean(axis=0))) <= 1e-12, "running mean"
        # first chunk token of a sequence with no context sees only itself
        c = make_case(rng, dtype, (0,), (3,), 2, 1, 5, 4)
        got = run(orc, c, 0.5)
        for h in range(2):
            assert np.array_equal(got[0, h], dec.widen(c["lv"][0][0, 0], dtype)), "first token"


def pin_prefill_invariants(orc):
    rng = np.random.default_rng(26)
    for dtype in ("f32", "bf16"):
        c = make_case(rng, dtype, (14, 3), (10, 7), 6, 2, 8, 4)
        base = run(orc, c, 0.4)
        # physical permutation of the pool: bitwise identical output
        NB = c["kc"].shape[0]
        perm = rng.permutation(NB)
        inv = np.empty_like(perm); inv[perm] = np.arange(NB)
        c2 = dict(c, kc=c["kc"][perm], vc=c["vc"][perm],
                  tables=np.where(c["tables"] >= 0, inv[np.maximum(c["tables"], 0)], -1).astype(np.int32))
        assert np.array_equal(run(orc, c2, 0.4), base), "physical block permutation"
        # causality: new values at chunk rows >= 4 of sequence 0 leave its rows < 4 unchanged
        kc, vc = c["kc"].copy(), c["vc"].copy()
        ctx0 = int(c["ctx"][0])
        for p in range(ctx0 + 4, ctx0 + 10):
            b = int(c["tables"][0, p // 4])
            kc[b, :, p % 4] = store(rng.standard_normal(kc[b, :, p % 4].shape) * 5, dtype)
            vc[b, :, p % 4] = store(rng.standard_normal(vc[b, :, p % 4].shape) * 5, dtype)
        got = run(orc, dict(c, kc=kc, vc=vc), 0.4)
        assert np.array_equal(got[:4], base[:4]), "causality"
        assert not np.array_equal(got[4:10], base[4:10]), "later rows do see the change"
        # splitting a chunk: rows 4.. of sequence 0 equal a chunk of those rows
        # over a context 4 tokens longer (the cache already holds them)
        qs2 = np.array([0, 6, 6 + 7], dtype=np.int32)
        c3 = dict(c, q=np.concatenate([c["q"][4:10], c["q"][10:]]), qs=qs2,
                  ctx=np.array([ctx0 + 4, int(c["ctx"][1])], dtype=np.int32))
        got = run(orc, c3, 0.4)
        assert np.array_equal(got[:6], base[4:10]) and np.array_equal(got[6:], base[10:]), "chunk split"


def pin_write_chunk(orc):
    rng = np.random.default_rng(27)
    for dtype in ("f32", "bf16"):
        c = make_case(rng, dtype, (5, 0, 16), (6, 3, 2), 4, 2, 3, 4)
        # a cache holding only the context: chunk slots poisoned with a marker
        kc, vc = c["kc"].copy(), c["vc"].copy()
        marker = np.float32(-7.0) if dtype == "f32" else np.uint16(0xC0E0)
        for s in range(3):
            for i in range(int(c["qs"][s + 1] - c["qs"][s])):
                p = int(c["ctx"][s]) + i
                kc[int(c["tables"][s, p // 4]), :, p % 4] = marker
                vc[int(c["tables"][s, p // 4]), :, p % 4] = marker
        k2, v2 = orc.write_chunk(kc, vc, c["key"], c["value"], c["tables"], c["qs"], c["ctx"], 4)
        # bitwise equal to the cache built directly from the logical rows (NaN tails included)
        assert np.array_equal(k2.view(np.uint32 if dtype == "f32" else np.uint16),
                              c["kc"].view(np.uint32 if dtype == "f32" else np.uint16)), "chunk keys"
        assert np.array_equal(v2.view(np.uint32 if dtype == "f32" else np.uint16),
                              c["vc"].view(np.uint32 if dtype == "f32" else np.uint16)), "chunk values"
        # the inputs are not modified
        assert (kc == marker).any(), "write_chunk must not modify its input"
        # and the prefill over the written cache equals the two-phase form from the chunk rows
        a = orc.prefill_attention(c["q"], k2, v2, c["tables"], c["qs"], c["ctx"], 0.6, 2, 4, dtype)
        b = orc.prefix_attention_two_phase(c["q"], c["key"], c["value"], kc, vc, c["tables"], c["qs"], c["ctx"],
                                           0.6, 2, 4, dtype, 4)
        assert np.max(np.abs(a - b)) <= 1e-12, "written cache vs chunk rows"


def pin_prefill_rows(orc):
    """The sampled-row helper equals the plain prefix attention and pure-Python
    brute force, row for row, for windows of chunk rows that start past the
    chunk's first token and end before its last (so a causal bound that is off
    by one either way changes the answer), with and without context."""
    rng = np.random.default_rng(28)
    scale = 0.1  # not a float32 value: whether the scale is rounded to float32 shows at ~1e-9
    for sh in (dict(dtype="f32", ctx=(5, 0), n=(9, 8), H=4, Hkv=2, D=6, bs=4),
               dict(dtype="bf16", ctx=(17, 3), n=(7, 10), H=6, Hkv=3, D=4, bs=4)):
        c = make_case(rng, sh["dtype"], sh["ctx"], sh["n"], sh["H"], sh["Hkv"], sh["D"], sh["bs"], spread=2.0)
        full = run(orc, c, scale)
        want = brute_force(c, float(np.float32(scale)))
        group = sh["H"] // sh["Hkv"]
        for s in range(len(sh["ctx"])):
            lo, n, ctx = int(c["qs"][s]), sh["n"][s], sh["ctx"][s]
            for first, m in ((0, 1), (1, 3), (2, n - 3), (n - 1, 1)):
                rows = slice(lo + first, lo + first + m)
                for h in range(sh["H"]):
                    g = h // group
                    got = orc.prefill_rows(c["q"][rows, h], c["lk"][s][g], c["lv"][s][g], ctx, first, scale,
                                           sh["dtype"])
                    assert got.shape == (m, sh["D"])
                    assert np.max(np.abs(got - full[rows, h])) <= 1e-12, ("prefill_rows vs plain", s, first, h)
                    assert np.max(np.abs(got - want[rows, h])) <= 1e-12, ("prefill_rows vs brute force", s, h)
            # a list of token indices in any order: each row as the plain oracle gives it
            toks = np.array([n - 2, 0, 3, 1])
            for h in range(sh["H"]):
                g = h // group
                got = orc.prefill_rows(c["q"][lo + toks, h], c["lk"][s][g], c["lv"][s][g], ctx, toks, scale,
                                       sh["dtype"])
                assert np.max(np.abs(got - full[lo + toks, h])) <= 1e-12, ("prefill_rows at listed tokens", s, h)
                assert np.max(np.abs(got - want[lo + toks, h])) <= 1e-12, ("listed tokens vs brute force", s, h)


ALL_PINS = [pin_prefill_brute_force, pin_prefill_two_phase, pin_prefill_decode_reduction, pin_prefill_sdpa,
            pin_prefill_closed_forms, pin_prefill_invariants, pin_write_chunk, pin_prefill_rows]


def failing_pins(orc):
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(orc)
        except Exception:  # noqa: BLE001 - any failure is a rejection
            bad.append(pin.__name__)
    return bad
