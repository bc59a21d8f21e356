"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function takes the oracle module and raises ``AssertionError``
when the oracle disagrees with what the pages or the mathematics fix:

* brute force: pure-Python loops over unpaged rows built without any block
  table, with an independent bfloat16 decoding (``struct``);
* hand-worked fixtures in ``tests/golden/hand_cases.json``;
* closed forms: zero query or identical keys give the mean of V, one token
  gives V_0, a dominant logit gives that row, two tokens give the logistic form;
* invariants: physical-block permutation (bitwise), logical token order,
  logit shift, affine maps of V;
* the log-sum-exp merge identity: the split form equals the plain form for
  every partition size, including one partition;
* the partition counts the pages print (``tests/golden/partition_counts.json``);
* a library special case: float64 ``torch.nn.functional.scaled_dot_product_attention``
  with an identity block table.

``tests/test_oracle.py`` runs every pin against the oracle, and runs the whole
set against oracles with planted mistakes to show that each mistake is caught.
"""

from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# small-problem construction (tests only)
# ---------------------------------------------------------------------------

def _bits_of(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits by truncation-free RNE using integer math."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def store(x, dtype):
    return np.asarray(x, dtype=np.float32) if dtype == "f32" else _bits_of(np.asarray(x, np.float32))


def paged(logical_k, logical_v, block_size, dtype, rng, extra_blocks=3, identity=False):
    """Lay per-sequence logical rows [Hkv, L_s, D] (storage format) into a pool
    with random distinct physical blocks; tail slots and spare blocks hold NaN."""
    S = len(logical_k)
    Hkv, _, D = logical_k[0].shape
    lens = [k.shape[1] for k in logical_k]
    nbs = [-(-L // block_size) for L in lens]
    NB = sum(nbs) + extra_blocks
    W = max(max(nbs), 1)
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    sd = np.float32 if dtype == "f32" else np.uint16
    kc = np.full((NB, Hkv, block_size, D), nan, dtype=sd)
    vc = np.full((NB, Hkv, block_size, D), nan, dtype=sd)
    ids = np.arange(NB) if identity else rng.permutation(NB)
    tables = np.full((S, W), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        for j in range(nbs[s]):
            b = int(ids[off]); off += 1
            tables[s, j] = b
            lo, hi = j * block_size, min((j + 1) * block_size, lens[s])
            kc[b, :, : hi - lo] = logical_k[s][:, lo:hi]
            vc[b, :, : hi - lo] = logical_v[s][:, lo:hi]
    return kc, vc, tables, np.asarray(lens, dtype=np.int32)


def random_case(rng, dtype="f32", S=2, H=4, Hkv=2, D=8, lens=(7, 13), block_size=4, spread=1.0):
    q = store(rng.standard_normal((S, H, D)) * spread, dtype)
    lk = [store(rng.standard_normal((Hkv, L, D)), dtype) for L in lens]
    lv = [store(rng.standard_normal((Hkv, L, D)), dtype) for L in lens]
    return q, lk, lv


def decode_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def brute_force(q, lk, lv, scale, num_kv_heads, dtype):
    """Pure-Python decode attention over unpaged rows (math module, no NumPy arithmetic)."""
    conv = (lambda x: float(x)) if dtype == "f32" else decode_bits
    S, H, D = q.shape
    group = H // num_kv_heads
    out = np.zeros((S, H, D))
    for s in range(S):
        L = lk[s].shape[1]
        for h in range(H):
            g = h // group
            qq = [conv(q[s, h, d]) for d in range(D)]
            logits = []
            for t in range(L):
                acc = 0.0
                for d in range(D):
                    acc += qq[d] * conv(lk[s][g, t, d])
                logits.append(scale * acc)
            if L == 0:
                continue
            mx = max(logits)
            ws = [math.exp(x - mx) for x in logits]
            tot = math.fsum(ws)
            for d in range(D):
                out[s, h, d] = math.fsum(ws[t] * conv(lv[s][g, t, d]) for t in range(L)) / tot
    return out


def run(orc, q, kc, vc, tables, lens, scale, Hkv, bs, dtype):
    return orc.decode_attention(q, kc, vc, tables, lens, scale, Hkv, bs, dtype)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_brute_force(orc):
    rng = np.random.default_rng(11)
    shapes = [
        dict(dtype="f32", S=2, H=4, Hkv=2, D=8, lens=(7, 13), block_size=4),
        dict(dtype="bf16", S=2, H=6, Hkv=2, D=4, lens=(1, 9), block_size=4),
        dict(dtype="bf16", S=1, H=3, Hkv=3, D=5, lens=(16,), block_size=16),
        dict(dtype="f32", S=3, H=2, Hkv=1, D=3, lens=(5, 0, 2), block_size=2),
    ]
    for sh in shapes:
        dtype, bs = sh["dtype"], sh["block_size"]
        q, lk, lv = random_case(rng, dtype, sh["S"], sh["H"], sh["Hkv"], sh["D"], sh["lens"], bs)
        kc, vc, tables, lens = paged(lk, lv, bs, dtype, rng)
        scale = 0.37
        got = run(orc, q, kc, vc, tables, lens, scale, sh["Hkv"], bs, dtype)
        want = brute_force(q, lk, lv, float(np.float32(scale)), sh["Hkv"], dtype)
        assert np.all(np.isfinite(got)), "oracle output not finite"
        assert np.max(np.abs(got - want)) <= 1e-12, (sh, np.max(np.abs(got - want)))


def _case_arrays(c):
    dtype = c["dtype"]

    def arr(x):
        if dtype == "f32":
            return np.asarray(x, dtype=object).astype(np.float32)
        return np.asarray(x, dtype=np.uint16)
    return (arr(c["query"]), arr(c["key_cache"]), arr(c["value_cache"]),
            np.asarray(c["block_tables"], dtype=np.int32), np.asarray(c["seq_lens"], dtype=np.int32))


def load_hand_cases():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        return json.load(f)


def pin_hand_cases(orc):
    data = load_hand_cases()
    for c in data["cases"]:
        q, kc, vc, tables, lens = _case_arrays(c)
        got = run(orc, q, kc, vc, tables, lens, c["scale"], c["num_kv_heads"], c["block_size"], c["dtype"])
        want = np.asarray(c["expected"], dtype=np.float64)
        assert got.shape == want.shape, c["name"]
        assert np.all(np.abs(got - want) <= c["tol"]), (c["name"], got, want)
    for c in data["split_cases"]:
        q, kc, vc, tables, lens = _case_arrays(c)
        out, stats = orc.decode_attention_split(q, kc, vc, tables, lens, c["scale"], c["num_kv_heads"],
                                                c["block_size"], c["dtype"], c["partition_size"])
        m, l, o = stats[(0, 0)]
        tol = c["tol"]
        assert np.allclose(m, c["expected_m"], atol=tol, rtol=0), (c["name"], m)
        assert np.allclose(l, c["expected_l"], atol=tol, rtol=0), (c["name"], l)
        assert np.allclose(o, c["expected_o"], atol=tol, rtol=0), (c["name"], o)
        assert np.allclose(out, c["expected"], atol=tol, rtol=0), (c["name"], out)


def pin_closed_forms(orc):
    rng = np.random.default_rng(12)
    D, Hkv, H, bs = 6, 2, 4, 4
    for dtype in ("f32", "bf16"):
        # zero query -> mean of V over the valid tokens
        lens = (9, 3)
        q = store(np.zeros((2, H, D)), dtype)
        _, lk, lv = random_case(rng, dtype, 2, H, Hkv, D, lens, bs)
        kc, vc, tables, L = paged(lk, lv, bs, dtype, rng)
        got = run(orc, q, kc, vc, tables, L, 0.5, Hkv, bs, dtype)
        for s in range(2):
            for h in range(H):
                vv = orc.widen(lv[s][h // (H // Hkv)], dtype)
                assert np.max(np.abs(got[s, h] - vv.mean(axis=0))) <= 1e-12, "zero query"
        # identical keys -> mean of V
        q = store(rng.standard_normal((1, H, D)), dtype)
        k_one = store(rng.standard_normal((Hkv, 1, D)), dtype)
        lk = [np.repeat(k_one, 11, axis=1)]
        lv = [store(rng.standard_normal((Hkv, 11, D)), dtype)]
        kc, vc, tables, L = paged(lk, lv, bs, dtype, rng)
        got = run(orc, q, kc, vc, tables, L, 0.3, Hkv, bs, dtype)
        for h in range(H):
            vv = orc.widen(lv[0][h // (H // Hkv)], dtype)
            assert np.max(np.abs(got[0, h] - vv.mean(axis=0))) <= 1e-12, "identical keys"
        # one token -> V_0
        q, lk, lv = random_case(rng, dtype, 1, H, Hkv, D, (1,), bs)
        kc, vc, tables, L = paged(lk, lv, bs, dtype, rng)
        got = run(orc, q, kc, vc, tables, L, 0.3, Hkv, bs, dtype)
        for h in range(H):
            assert np.array_equal(got[0, h], orc.widen(lv[0][h // (H // Hkv), 0], dtype)), "one token"
    # dominant logit -> that row (logit gap 1000; exp(-1000) underflows to 0)
    D, L = 4, 10
    q = np.zeros((1, 1, D), np.float32); q[0, 0, 0] = 1.0
    k = np.zeros((1, L, D), np.float32); k[0, 6, 0] = 1000.0; k[0, 2, 0] = 999.0 - 1000.0
    v = rng.standard_normal((1, L, D)).astype(np.float32)
    kc, vc, tables, lens = paged([k], [v], 4, "f32", rng)
    got = run(orc, q, kc, vc, tables, lens, 1.0, 1, 4, "f32")
    assert np.array_equal(got[0, 0], v[0, 6].astype(np.float64)), "dominant logit"
    # two tokens: out = sigmoid(x0 - x1) v0 + sigmoid(x1 - x0) v1
    for _ in range(5):
        D = 3
        q = rng.standard_normal((1, 1, D)).astype(np.float32)
        k = rng.standard_normal((1, 2, D)).astype(np.float32)
        v = rng.standard_normal((1, 2, D)).astype(np.float32)
        kc, vc, tables, lens = paged([k], [v], 2, "f32", rng)
        sc = 0.7
        got = run(orc, q, kc, vc, tables, lens, sc, 1, 2, "f32")
        x0 = float(np.float32(sc)) * float(np.dot(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64)))
        x1 = float(np.float32(sc)) * float(np.dot(q[0, 0].astype(np.float64), k[0, 1].astype(np.float64)))
        a = 1.0 / (1.0 + math.exp(x1 - x0))
        want = a * v[0, 0].astype(np.float64) + (1 - a) * v[0, 1].astype(np.float64)
        assert np.max(np.abs(got[0, 0] - want)) <= 1e-12, "two-token logistic form"


def pin_invariants(orc):
    rng = np.random.default_rng(13)
    for dtype in ("f32", "bf16"):
        H, Hkv, D, bs = 6, 2, 8, 4
        lens = (14, 5, 8)
        q, lk, lv = random_case(rng, dtype, 3, H, Hkv, D, lens, bs)
        kc, vc, tables, L = paged(lk, lv, bs, dtype, rng)
        base = run(orc, q, kc, vc, tables, L, 0.4, Hkv, bs, dtype)
        # physical permutation of the pool: bitwise identical output
        NB = kc.shape[0]
        perm = rng.permutation(NB)
        inv = np.empty_like(perm); inv[perm] = np.arange(NB)
        kc2, vc2 = kc[perm], vc[perm]            # new block i = old block perm[i]
        t2 = np.where(tables >= 0, inv[np.maximum(tables, 0)], -1).astype(np.int32)
        got = run(orc, q, kc2, vc2, t2, L, 0.4, Hkv, bs, dtype)
        assert np.array_equal(got, base), "physical block permutation"
        # logical token order
        lk2, lv2 = [], []
        for s in range(3):
            p = rng.permutation(lens[s])
            lk2.append(lk[s][:, p]); lv2.append(lv[s][:, p])
        kc3, vc3, t3, L3 = paged(lk2, lv2, bs, dtype, rng)
        got = run(orc, q, kc3, vc3, t3, L3, 0.4, Hkv, bs, dtype)
        assert np.max(np.abs(got - base)) <= 1e-12, "token order"
    # logit shift: adding c*q/|q|^2 to every key adds c*scale to every logit
    H, Hkv, D, bs = 2, 1, 4, 4
    q = np.zeros((1, H, D), np.float32); q[0, :, 1] = 2.0
    # keys on a 2^-10 grid so that k + 3 is exact in float32
    k = (np.round(rng.standard_normal((1, 9, D)) * 1024) / 1024).astype(np.float32)
    v = (np.round(rng.standard_normal((1, 9, D)) * 1024) / 1024).astype(np.float32)
    kc, vc, tables, lens = paged([k], [v], bs, "f32", rng)
    a = run(orc, q, kc, vc, tables, lens, 0.5, Hkv, bs, "f32")
    k2 = k.copy(); k2[0, :, 1] += np.float32(3.0)
    kc, vc, tables, lens = paged([k2], [v], bs, "f32", rng)
    b = run(orc, q, kc, vc, tables, lens, 0.5, Hkv, bs, "f32")
    assert np.max(np.abs(a - b)) <= 1e-12, "logit shift"
    # affine map of V: out(alpha V + beta) = alpha out(V) + beta (weights sum to one);
    # V on a 2^-10 grid so 2v + 0.5 is exact in float32
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    v2 = (v * np.float32(2.0) + np.float32(0.5)).astype(np.float32)
    kc, vc, tables, lens = paged([k], [v], bs, "f32", rng)
    a = run(orc, q, kc, vc, tables, lens, 0.5, Hkv, bs, "f32")
    kc, vc, tables, lens = paged([k], [v2], bs, "f32", rng)
    b = run(orc, q, kc, vc, tables, lens, 0.5, Hkv, bs, "f32")
    assert np.max(np.abs(b - (2.0 * a + 0.5))) <= 1e-12, "affine V"
    # output lies in the per-dimension hull of the valid V rows
    assert np.all(a[0] <= v[0].max(axis=0) + 1e-12) and np.all(a[0] >= v[0].min(axis=0) - 1e-12), "hull"


def pin_lse_identity(orc):
    rng = np.random.default_rng(14)
    for dtype in ("f32", "bf16"):
        H, Hkv, D, bs = 4, 2, 8, 4
        lens = (37, 4, 16, 1)
        q, lk, lv = random_case(rng, dtype, 4, H, Hkv, D, lens, bs, spread=3.0)
        kc, vc, tables, L = paged(lk, lv, bs, dtype, rng)
        full = run(orc, q, kc, vc, tables, L, 0.9, Hkv, bs, dtype)
        for P in (4, 8, 12, 16, 36, 40, 64):
            out, stats = orc.decode_attention_split(q, kc, vc, tables, L, 0.9, Hkv, bs, dtype, P)
            assert np.max(np.abs(out - full)) <= 1e-12, ("LSE merge", P)
            for s in range(4):
                m, l, o = stats[(s, 0)]
                assert m.shape[0] == -(-int(L[s]) // P), "partition count"
                assert np.all(l >= 1.0 - 1e-15), "each partition exp-sum includes exp(0) = 1"
            if P >= max(lens):
                # one partition: its normalised output is the answer
                for s in range(4):
                    for h in range(H):
                        m, l, o = stats[(s, h)]
                        assert np.max(np.abs(o[0] - full[s, h])) <= 1e-12, "single partition"


def pin_partition_counts(orc):
    with open(os.path.join(GOLDEN, "partition_counts.json")) as f:
        data = json.load(f)
    for c in data["partition_counts"]:
        L, P = c["seq_len"], c["partition_size"]
        # keys that make every logit zero: the Phase-1 count is what is checked
        D = 1
        K = np.zeros((L, D)); V = np.zeros((L, D)); q = np.zeros(D)
        m, l, o = orc.partition_stats(q, K, V, 1.0, P)
        assert m.shape[0] == c["num_partitions"], c
        assert l[-1] == L - (c["num_partitions"] - 1) * P, "last partition holds the remainder"


def pin_library_sdpa(orc):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(15)
    for dtype in ("f32", "bf16"):
        S, H, Hkv, D, bs, L = 1, 6, 2, 16, 4, 23
        q, lk, lv = random_case(rng, dtype, S, H, Hkv, D, (L,), bs)
        kc, vc, tables, lens = paged(lk, lv, bs, dtype, rng, identity=True)
        got = run(orc, q, kc, vc, tables, lens, 0.25, Hkv, bs, dtype)
        qt = torch.from_numpy(orc.widen(q, dtype)).reshape(1, H, 1, D)
        kt = torch.from_numpy(orc.widen(lk[0], dtype)).reshape(1, Hkv, L, D)
        vt = torch.from_numpy(orc.widen(lv[0], dtype)).reshape(1, Hkv, L, D)
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.25, enable_gqa=True)
        ref = ref.reshape(S, H, D).numpy()
        assert np.max(np.abs(got - ref)) <= 1e-12, "float64 SDPA special case"


def pin_attend_logical(orc):
    """The one-row helper used for sampled checks equals pure-Python brute force
    and the paged oracle, row for row, in both storage formats, with ordinary
    keys and with large-logit outliers (keys x 20 at a few positions)."""
    rng = np.random.default_rng(16)
    scale = 0.1  # not a float32 value: whether the scale is rounded to float32 shows at ~1e-9
    for dtype in ("f32", "bf16"):
        for outliers in (False, True):
            H, Hkv, D, bs = 6, 2, 8, 4
            lens = (13, 1, 6)
            S = len(lens)
            q = store(rng.standard_normal((S, H, D)) * 2.0, dtype)
            lk, lv = [], []
            for L in lens:
                k = rng.standard_normal((Hkv, L, D))
                if outliers:
                    k[:, rng.random(L) < 0.3] *= 20.0
                lk.append(store(k, dtype))
                lv.append(store(rng.standard_normal((Hkv, L, D)), dtype))
            kc, vc, tables, L = paged(lk, lv, bs, dtype, rng)
            want = brute_force(q, lk, lv, float(np.float32(scale)), Hkv, dtype)
            full = run(orc, q, kc, vc, tables, L, scale, Hkv, bs, dtype)
            for s in range(S):
                for h in range(H):
                    g = h // (H // Hkv)
                    got = orc.attend_logical(q[s, h], lk[s][g], lv[s][g], scale, dtype)
                    assert got.shape == (D,)
                    assert np.max(np.abs(got - want[s, h])) <= 1e-12, ("attend_logical vs brute force", s, h)
                    assert np.max(np.abs(got - full[s, h])) <= 1e-12, ("attend_logical vs decode_attention", s, h)


ALL_PINS = [pin_brute_force, pin_hand_cases, pin_closed_forms, pin_invariants,
            pin_lse_identity, pin_partition_counts, pin_library_sdpa, pin_attend_logical]


def failing_pins(orc):
    """Names of the pins that reject ``orc`` (an exception counts as a rejection)."""
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(orc)
        except Exception:  # noqa: BLE001 - any failure is a rejection
            bad.append(pin.__name__)
    return bad
