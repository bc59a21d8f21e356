"""Plain fp64 CPU oracle for prefix (chunked prefill) attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the GPU library and imports nothing from it.

What it computes.  The first page's prefill note (the path that replaced the
Triton context-attention kernel) and the second page's prefix-attention
messages (the allocator-reuse message and the rewrite that gathers the whole
context's K/V before attending) describe prefill for a sequence that already
holds ``ctx`` tokens in the paged cache and receives a chunk of ``n`` new
tokens: every new token attends to all cached context tokens and, causally,
to the chunk's tokens up to and including itself.  The pages compute it as a K-tiled online softmax in
two phases, context tiles first (keys gathered from the cache through the
block table once), then the chunk's own tiles under the causal mask.

* :func:`prefill_attention` is the plain definition: query token ``i`` of
  sequence ``s`` sits at absolute position ``ctx[s] + i`` and takes softmax
  attention over cache positions ``0 .. ctx[s] + i`` of its sequence, the
  chunk's keys and values having been stored at positions ``ctx[s] ..
  ctx[s] + n - 1`` (:func:`write_chunk`).
* :func:`prefix_attention_two_phase` follows the pages' method step by step
  (context phase from the cache, chunk phase from the chunk's own key and
  value rows, one running max / exp-sum / accumulator per query row).  It
  reaches the plain result up to rounding; the pins check that it does.
* :func:`write_chunk` stores the chunk's keys and values in the cache slots of
  their positions (a plain scatter through the block table).

Readings where the pages are silent: the GQA mapping and the bf16 widening
are those of the decode oracle; a chunk of ``n == 0`` tokens produces nothing;
the context may be empty (plain causal self-attention over the chunk).

All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

from .attention import attend, gather_sequence, kv_head_for, widen


def chunk_bounds(query_start, s: int):
    """Rows [lo, hi) of sequence s in the packed query (cumulative offsets, length S + 1)."""
    return int(query_start[s]), int(query_start[s + 1])


def prefill_attention(query, key_cache, value_cache, block_tables, query_start, context_lens, scale,
                      num_kv_heads, block_size, dtype) -> np.ndarray:
    """fp64 output [T, H, D] of prefix attention, everything read from the cache.

    query [T, H, D] (storage format of ``dtype``), the chunk's rows of all
    sequences packed one after another; key_cache, value_cache [NB, Hkv, bs, D]
    holding, for sequence s, positions 0 .. context_lens[s] + n_s - 1;
    block_tables [S, W]; query_start [S + 1] cumulative row offsets;
    context_lens [S].
    """
    T, H, D = query.shape
    out = np.zeros((T, H, D), dtype=np.float64)
    scale = float(np.float32(scale))
    for s in range(len(context_lens)):
        lo, hi = chunk_bounds(query_start, s)
        ctx = int(context_lens[s])
        total = ctx + (hi - lo)
        K = widen(gather_sequence(key_cache, block_tables[s], total, block_size), dtype)
        V = widen(gather_sequence(value_cache, block_tables[s], total, block_size), dtype)
        q = widen(query[lo:hi], dtype)
        for i in range(hi - lo):
            visible = ctx + i + 1   # causal: positions up to and including the token's own
            for h in range(H):
                g = kv_head_for(h, H, num_kv_heads)
                out[lo + i, h] = attend(q[i, h], K[g, :visible], V[g, :visible], scale)
    return out


def prefill_rows(query_rows, K_rows, V_rows, ctx: int, first, scale, dtype) -> np.ndarray:
    """Outputs of chosen chunk tokens of one (sequence, head) from unpaged rows.

    query_rows [m, D] are the rows of chunk tokens ``first .. first + m - 1``
    (``first`` an int), or of the chunk tokens listed in ``first`` (a sequence
    of m token indices); K_rows, V_rows [>= ctx + last token + 1, D] the
    sequence's logical keys and values of its KV head.  Chunk token t sees
    positions 0 .. ctx + t.  Used for sampled checks at sizes where the full
    oracle is too slow.
    """
    q = widen(query_rows, dtype)
    K = widen(K_rows, dtype)
    V = widen(V_rows, dtype)
    sc = float(np.float32(scale))
    tokens = (np.arange(q.shape[0]) + int(first)) if np.ndim(first) == 0 else np.asarray(first, dtype=np.int64)
    if tokens.shape != (q.shape[0],):
        raise ValueError("one token index per query row")
    out = np.empty((q.shape[0], K.shape[1]))
    for r in range(q.shape[0]):
        visible = ctx + int(tokens[r]) + 1
        out[r] = attend(q[r], K[:visible], V[:visible], sc)
    return out


def write_chunk(key_cache, value_cache, key, value, block_tables, query_start, context_lens, block_size):
    """Caches with the chunk's rows stored: row lo + i of sequence s (key [T, Hkv, D],
    value likewise) goes to position context_lens[s] + i, that is to block
    block_tables[s, p // block_size], slot p % block_size.  Returns new arrays."""
    kc = key_cache.copy()
    vc = value_cache.copy()
    for s in range(len(context_lens)):
        lo, hi = chunk_bounds(query_start, s)
        for i in range(hi - lo):
            p = int(context_lens[s]) + i
            b = int(block_tables[s, p // block_size])
            kc[b, :, p % block_size] = key[lo + i]
            vc[b, :, p % block_size] = value[lo + i]
    return kc, vc


def prefix_attention_two_phase(query, key, value, key_cache, value_cache, block_tables, query_start,
                               context_lens, scale, num_kv_heads, block_size, dtype, tile) -> np.ndarray:
    """The pages' prefill method: K-tiled online softmax, context then chunk.

    The context keys and values come from the cache (gathered once per
    sequence); the chunk's come from ``key`` / ``value`` [T, Hkv, D] directly.
    For each query row the running max m, exp-sum l and accumulator acc are
    updated tile by tile: m_new = max(m, tile max), corr = exp(m - m_new),
    l = l * corr + sum exp(x - m_new), acc = acc * corr + exp(x - m_new) V.
    In the chunk phase key j of the chunk is masked (logit -inf) for query
    rows i < j.  The result is acc / l.
    """
    T, H, D = query.shape
    out = np.zeros((T, H, D), dtype=np.float64)
    sc = float(np.float32(scale))
    for s in range(len(context_lens)):
        lo, hi = chunk_bounds(query_start, s)
        n = hi - lo
        if n == 0:
            continue
        ctx = int(context_lens[s])
        Kc = widen(gather_sequence(key_cache, block_tables[s], ctx, block_size), dtype)
        Vc = widen(gather_sequence(value_cache, block_tables[s], ctx, block_size), dtype)
        Kn = widen(key[lo:hi], dtype).transpose(1, 0, 2)      # [Hkv, n, D]
        Vn = widen(value[lo:hi], dtype).transpose(1, 0, 2)
        q = widen(query[lo:hi], dtype)                        # [n, H, D]
        rows = np.arange(n)
        for h in range(H):
            g = kv_head_for(h, H, num_kv_heads)
            m = np.full(n, -np.inf)
            l = np.zeros(n)
            acc = np.zeros((n, D))

            def update(x, Vt):
                nonlocal m, l, acc
                m_new = np.maximum(m, x.max(axis=1))
                corr = np.exp(m - m_new)
                w = np.exp(x - m_new[:, None])
                l = l * corr + w.sum(axis=1)
                acc = acc * corr[:, None] + w @ Vt
                m = m_new

            for a in range(0, ctx, tile):                     # context phase: no mask
                b = min(a + tile, ctx)
                update(sc * (q[:, h] @ Kc[g, a:b].T), Vc[g, a:b])
            for a in range(0, n, tile):                       # chunk phase: causal
                b = min(a + tile, n)
                x = sc * (q[:, h] @ Kn[g, a:b].T)
                cols = np.arange(a, b)
                x = np.where(cols[None, :] <= rows[:, None], x, -np.inf)
                # rows that see none of this tile keep their state
                seen = cols[0] <= rows
                if not seen.any():
                    continue
                m_keep, l_keep, acc_keep = m.copy(), l.copy(), acc.copy()
                update(np.where(seen[:, None], x, 0.0), Vn[g, a:b])
                m = np.where(seen, m, m_keep)
                l = np.where(seen, l, l_keep)
                acc = np.where(seen[:, None], acc, acc_keep)
            out[lo:hi, h] = acc / l[:, None]
    return out
