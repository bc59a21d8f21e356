"""The prefix-attention oracle against its pins, and the pins against planted mistakes."""

import numpy as np
import pytest

import oracle.attention as dec
import oracle.prefill as orc
from tests import oracle_pins_prefill as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(orc)


def _prefill_with(visible_of, q_shift=0):
    """prefill_attention with a planted mistake in the causal rule or the query rows."""
    def f(query, key_cache, value_cache, block_tables, query_start, context_lens, scale, num_kv_heads,
          block_size, dtype):
        T, H, D = query.shape
        out = np.zeros((T, H, D))
        sc = float(np.float32(scale))
        for s in range(len(context_lens)):
            lo, hi = int(query_start[s]), int(query_start[s + 1])
            ctx = int(context_lens[s])
            K = dec.widen(dec.gather_sequence(key_cache, block_tables[s], ctx + hi - lo, block_size), dtype)
            V = dec.widen(dec.gather_sequence(value_cache, block_tables[s], ctx + hi - lo, block_size), dtype)
            for i in range(hi - lo):
                a, b = visible_of(ctx, i)
                qi = dec.widen(query[min(lo + i + q_shift, T - 1)], dtype)
                for h in range(H):
                    g = dec.kv_head_for(h, H, num_kv_heads)
                    out[lo + i, h] = dec.attend(qi[h], K[g, a:b], V[g, a:b], sc)
        return out
    return f


def _two_phase_with(no_corr=False, strict_mask=False, skip_context=False):
    def f(query, key, value, key_cache, value_cache, block_tables, query_start, context_lens, scale,
          num_kv_heads, block_size, dtype, tile):
        T, H, D = query.shape
        out = np.zeros((T, H, D))
        sc = float(np.float32(scale))
        for s in range(len(context_lens)):
            lo, hi = int(query_start[s]), int(query_start[s + 1])
            n, ctx = hi - lo, int(context_lens[s])
            if n == 0:
                continue
            Kc = dec.widen(dec.gather_sequence(key_cache, block_tables[s], ctx, block_size), dtype)
            Vc = dec.widen(dec.gather_sequence(value_cache, block_tables[s], ctx, block_size), dtype)
            Kn = dec.widen(key[lo:hi], dtype).transpose(1, 0, 2)
            Vn = dec.widen(value[lo:hi], dtype).transpose(1, 0, 2)
            q = dec.widen(query[lo:hi], dtype)
            for h in range(H):
                g = dec.kv_head_for(h, H, num_kv_heads)
                for i in range(n):
                    m, l, acc = -np.inf, 0.0, np.zeros(D)
                    tiles = [] if skip_context else [(Kc[g, a:a + tile], Vc[g, a:a + tile]) for a in range(0, ctx, tile)]
                    last = i if strict_mask else i + 1
                    tiles += [(Kn[g, a:min(a + tile, last)], Vn[g, a:min(a + tile, last)])
                              for a in range(0, last, tile)]
                    for Kt, Vt in tiles:
                        if Kt.shape[0] == 0:
                            continue
                        x = sc * (Kt @ q[i, h])
                        m_new = max(m, x.max())
                        corr = 1.0 if no_corr else np.exp(m - m_new)
                        w = np.exp(x - m_new)
                        l = l * corr + w.sum()
                        acc = acc * corr + w @ Vt
                        m = m_new
                    out[lo + i, h] = acc / l if l > 0 else 0.0
        return out
    return f


def _write_off_by_one(key_cache, value_cache, key, value, block_tables, query_start, context_lens, block_size):
    kc, vc = key_cache.copy(), value_cache.copy()
    for s in range(len(context_lens)):
        for i in range(int(query_start[s + 1]) - int(query_start[s])):
            p = int(context_lens[s]) + i + 1
            b = int(block_tables[s, min(p // block_size, block_tables.shape[1] - 1)])
            kc[b, :, p % block_size] = key[int(query_start[s]) + i]
            vc[b, :, p % block_size] = value[int(query_start[s]) + i]
    return kc, vc


def _write_ignoring_context(key_cache, value_cache, key, value, block_tables, query_start, context_lens, block_size):
    kc, vc = key_cache.copy(), value_cache.copy()
    for s in range(len(context_lens)):
        for i in range(int(query_start[s + 1]) - int(query_start[s])):
            b = int(block_tables[s, i // block_size])
            kc[b, :, i % block_size] = key[int(query_start[s]) + i]
            vc[b, :, i % block_size] = value[int(query_start[s]) + i]
    return kc, vc


def _rows_with(visible_of=None, swap=False, unrounded=False):
    """prefill_rows with a planted mistake: the causal bound, K/V swapped, or
    the scale used without its float32 rounding."""
    def f(query_rows, K_rows, V_rows, ctx, first, scale, dtype):
        q = dec.widen(query_rows, dtype)
        K = dec.widen(V_rows if swap else K_rows, dtype)
        V = dec.widen(K_rows if swap else V_rows, dtype)
        sc = float(scale) if unrounded else float(np.float32(scale))
        toks = (np.arange(q.shape[0]) + int(first)) if np.ndim(first) == 0 else np.asarray(first)
        out = np.empty((q.shape[0], K.shape[1]))
        for r in range(q.shape[0]):
            visible = visible_of(ctx, int(toks[r]), r) if visible_of else ctx + int(toks[r]) + 1
            out[r] = dec.attend(q[r], K[:visible], V[:visible], sc)
        return out
    return f


MUTANTS = [
    ("prefill_attention", _prefill_with(lambda ctx, i: (0, ctx + i)), "excludes its own token"),
    ("prefill_attention", _prefill_with(lambda ctx, i: (0, i + 1)), "causal rule without the context offset"),
    ("prefill_attention", _prefill_with(lambda ctx, i: (ctx, ctx + i + 1)), "context ignored"),
    ("prefill_attention", _prefill_with(lambda ctx, i: (0, ctx + i + 2)), "one token into the future"),
    ("prefill_attention", _prefill_with(lambda ctx, i: (0, ctx + i + 1), q_shift=1), "query rows shifted"),
    ("prefix_attention_two_phase", _two_phase_with(no_corr=True), "no running-max correction"),
    ("prefix_attention_two_phase", _two_phase_with(strict_mask=True), "chunk mask excludes the diagonal"),
    ("prefix_attention_two_phase", _two_phase_with(skip_context=True), "context phase skipped"),
    ("write_chunk", _write_off_by_one, "chunk written one slot late"),
    ("write_chunk", _write_ignoring_context, "chunk written from position 0"),
    ("prefill_rows", _rows_with(lambda ctx, t, r: ctx + t + 2), "rows: one token into the future"),
    ("prefill_rows", _rows_with(lambda ctx, t, r: ctx + t), "rows: own token excluded"),
    ("prefill_rows", _rows_with(lambda ctx, t, r: ctx + r + 1), "rows: window start ignored"),
    ("prefill_rows", _rows_with(swap=True), "rows: keys and values swapped"),
    ("prefill_rows", _rows_with(unrounded=True), "rows: scale not rounded to float32"),
]


def test_pins_accept_oracle():
    assert pins.failing_pins(orc) == []


@pytest.mark.parametrize("name,fn,what", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, what):
    monkeypatch.setattr(orc, name, fn)
    assert pins.failing_pins(orc), f"no pin rejects the planted mistake: {what}"
