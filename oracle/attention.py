"""Plain fp64 CPU oracle for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the GPU library and imports nothing from it.

What it computes (the two-pass decode method on the second page, "paged_attn
rewrite" and "V2 implementation" messages, and the first page's two-pass
message):

* The result is plain softmax attention of one query row per head over the
  sequence's cached keys and values, gathered through the block table
  (:func:`decode_attention`).  The split method reaches exactly this result up
  to rounding order, so the plain definition is the oracle.
* Phase 1 / Phase 2 of the split form are also written out
  (:func:`partition_stats`, :func:`merge_partitions`) so that the
  log-sum-exp merge identity can be checked and the GPU's per-partition
  workspace can be compared entry by entry.

Readings where the pages are silent (each is listed with the others in the
design notes):
* query head h reads KV head ``h // (num_heads // num_kv_heads)``;
* only tokens ``t < seq_len`` count; tail slots of the last block and blocks
  the table does not reference are never read;
* ``seq_len == 0`` gives an all-zero output row;
* the per-partition output is normalised by its own exp-sum, and the merge
  weights are ``exp_sum_p * exp(max_p - global_max)`` divided by their total.

All arithmetic is float64.  bfloat16 inputs are widened exactly (the 16 bits
are the high half of an IEEE float32).
"""

from __future__ import annotations

import numpy as np


def widen(values: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored elements ("f32" floats or "bf16" uint16 bit patterns)."""
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(values, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kv_head_for(h: int, num_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: heads are grouped contiguously, G = H / Hkv per KV head."""
    return h // (num_heads // num_kv_heads)


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, seq_len: int, block_size: int) -> np.ndarray:
    """Logical [num_kv_heads, seq_len, head_size] rows of one sequence from a pool
    [num_blocks, num_kv_heads, block_size, head_size], following its block table."""
    nb = -(-seq_len // block_size)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = cache[ids]                                   # [nb, Hkv, bs, D]
    hkv, d = cache.shape[1], cache.shape[3]
    rows = blocks.transpose(1, 0, 2, 3).reshape(hkv, nb * block_size, d)
    return rows[:, :seq_len]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) weighted sum of the rows of V, for one query row (fp64).

    q: [D], K: [L, D], V: [L, D] -> [D].  An empty K gives zeros.
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    x = scale * (K @ q)
    w = np.exp(x - x.max())
    return (w @ V) / w.sum()


def decode_attention(query, key_cache, value_cache, block_tables, seq_lens, scale,
                     num_kv_heads, block_size, dtype) -> np.ndarray:
    """fp64 output [num_seqs, num_heads, head_size] of single-token decode attention.

    query [S, H, D]; key_cache, value_cache [NB, Hkv, bs, D] (storage format of
    ``dtype``); block_tables int [S, W]; seq_lens int [S]; scale float.
    """
    S, H, D = query.shape
    out = np.zeros((S, H, D), dtype=np.float64)
    scale = float(np.float32(scale))
    for s in range(S):
        L = int(seq_lens[s])
        # widen only the blocks this sequence references
        K = widen(gather_sequence(key_cache, block_tables[s], L, block_size), dtype)
        V = widen(gather_sequence(value_cache, block_tables[s], L, block_size), dtype)
        q = widen(query[s], dtype)
        for h in range(H):
            g = kv_head_for(h, H, num_kv_heads)
            out[s, h] = attend(q[h], K[g], V[g], scale)
    return out


# ---------------------------------------------------------------------------
# Split form: Phase 1 (per partition) and Phase 2 (log-sum-exp merge)
# ---------------------------------------------------------------------------

def partition_stats(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, partition_size: int):
    """Phase 1 for one (sequence, head): per partition of ``partition_size`` tokens,
    the max logit m_p, the exp-sum l_p = sum exp(x - m_p), and the partition
    output o_p = sum exp(x - m_p) v / l_p.

    Returns (m [NP], l [NP], o [NP, D]) with NP = ceil(L / partition_size).
    """
    L, D = K.shape
    n_part = -(-L // partition_size)
    m = np.empty(n_part)
    l = np.empty(n_part)
    o = np.empty((n_part, D))
    for p in range(n_part):
        lo, hi = p * partition_size, min((p + 1) * partition_size, L)
        x = scale * (K[lo:hi] @ q)
        m[p] = x.max()
        w = np.exp(x - m[p])
        l[p] = w.sum()
        o[p] = (w @ V[lo:hi]) / l[p]
    return m, l, o


def merge_partitions(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Phase 2: global max over partitions, rescale each partition's exp-sum by
    exp(m_p - global max), and take the rescaled sums' share of each partition output."""
    if m.shape[0] == 0:
        return np.zeros(o.shape[1], dtype=np.float64)
    gmax = m.max()
    rescale = np.exp(m - gmax) * l
    return (rescale / rescale.sum()) @ o


def decode_attention_split(query, key_cache, value_cache, block_tables, seq_lens, scale,
                           num_kv_heads, block_size, dtype, partition_size):
    """Split-form result and its Phase 1 intermediates.

    Returns ``(out [S,H,D], stats)`` where ``stats[(s, h)] = (m, l, o)`` holds the
    per-partition max logit, exp-sum and normalised partition output.
    """
    if partition_size <= 0 or partition_size % block_size:
        raise ValueError("partition_size must be a positive multiple of block_size")
    S, H, D = query.shape
    out = np.zeros((S, H, D), dtype=np.float64)
    stats = {}
    scale = float(np.float32(scale))
    for s in range(S):
        L = int(seq_lens[s])
        K = widen(gather_sequence(key_cache, block_tables[s], L, block_size), dtype)
        V = widen(gather_sequence(value_cache, block_tables[s], L, block_size), dtype)
        q = widen(query[s], dtype)
        for h in range(H):
            g = kv_head_for(h, H, num_kv_heads)
            m, l, o = partition_stats(q[h], K[g], V[g], scale, partition_size)
            stats[(s, h)] = (m, l, o)
            out[s, h] = merge_partitions(m, l, o)
    return out, stats


def attend_logical(q_row, K_rows, V_rows, scale, dtype) -> np.ndarray:
    """One (sequence, head) output from unpaged rows in storage format; used for
    sampled checks at sizes where gathering the whole pool is not needed."""
    return attend(widen(q_row, dtype), widen(K_rows, dtype), widen(V_rows, dtype),
                  float(np.float32(scale)))
