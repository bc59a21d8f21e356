"""Seeded synthetic inputs for single-token paged decode attention.

This module draws values and lays them out; it holds none of the attention
arithmetic.  It serves both the tests (which feed the same arrays to the CPU
oracle and to the GPU library) and the benchmark.

Storage formats on the host:
  * ``"f32"``  -> ``numpy.float32``
  * ``"bf16"`` -> ``numpy.uint16`` holding the bfloat16 bit pattern

The KV pool layout is ``[num_blocks, num_kv_heads, block_size, head_size]``
for both K and V (the 4-D layout the second page's hardware-test message
reports as accepted for the split kernel).  ``block_tables[s, j]`` names the
physical block that holds logical tokens ``[j*block_size, (j+1)*block_size)``
of sequence ``s``; unused entries hold -1.

Every random stream is derived from one integer seed through
``numpy.random.SeedSequence(seed, spawn_key=(stream, ...))`` so that any
(sequence, KV head) slice can be regenerated on its own, in any order and on
any number of threads, with identical bits.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# stream identifiers for SeedSequence spawn keys
_S_TABLE, _S_LENS, _S_QUERY, _S_KEY, _S_VALUE, _S_OUTLIER = range(6)


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    """Shape and value recipe of one synthetic workload."""

    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int           # physical blocks in the pool
    max_blocks_per_seq: int   # block-table width W
    partition_size: int       # 0 = one-pass
    dtype: str                # "f32" | "bf16"
    seed: int
    seq_len: Optional[int] = None          # fixed length for every sequence
    seq_len_range: Optional[tuple] = None  # inclusive (lo, hi) uniform integers
    outlier_rate: float = 0.0              # Bernoulli rate of outlier key positions
    outlier_scale: float = 1.0             # multiplier of K at outlier positions
    scale: Optional[float] = None          # default 1/sqrt(head_size)

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(self.scale if self.scale is not None
                                else 1.0 / math.sqrt(self.head_size)))


# The five workloads.  Shapes follow the model attention shape the pages
# describe (24 query heads, 4 KV heads, head size 256) and their 100K-token
# long-context case; the value distributions are synthetic N(0, 1).
CONFIGS: Dict[str, ConfigSpec] = {
    "tiny": ConfigSpec("tiny", num_seqs=1, num_heads=4, num_kv_heads=1, head_size=64,
                       block_size=16, num_blocks=16, max_blocks_per_seq=7,
                       partition_size=32, dtype="f32", seed=1, seq_len=100,
                       scale=0.125),
    "short": ConfigSpec("short", num_seqs=1, num_heads=24, num_kv_heads=4, head_size=256,
                        block_size=16, num_blocks=1024, max_blocks_per_seq=512,
                        partition_size=0, dtype="bf16", seed=2, seq_len=8192),
    "long": ConfigSpec("long", num_seqs=1, num_heads=24, num_kv_heads=4, head_size=256,
                       block_size=16, num_blocks=12500, max_blocks_per_seq=6250,
                       partition_size=512, dtype="bf16", seed=3, seq_len=100000),
    "mixed": ConfigSpec("mixed", num_seqs=32, num_heads=24, num_kv_heads=4, head_size=256,
                        block_size=16, num_blocks=65536, max_blocks_per_seq=2048,
                        partition_size=512, dtype="bf16", seed=4,
                        seq_len_range=(1, 32768)),
    "stress": ConfigSpec("stress", num_seqs=8, num_heads=24, num_kv_heads=24, head_size=256,
                         block_size=16, num_blocks=65536, max_blocks_per_seq=8192,
                         partition_size=1024, dtype="bf16", seed=5, seq_len=131072,
                         outlier_rate=0.01, outlier_scale=20.0),
    # Large-batch, short-context serving decode: 256 concurrent sequences of 2048
    # tokens (the serving configuration on the second page moves to 128-256
    # concurrent sequences); one-pass, the form the dispatch rule picks here.
    "batch256": ConfigSpec("batch256", num_seqs=256, num_heads=24, num_kv_heads=4, head_size=256,
                           block_size=16, num_blocks=32768, max_blocks_per_seq=128,
                           partition_size=0, dtype="bf16", seed=6, seq_len=2048),
}


@dataclasses.dataclass
class Problem:
    """Host-side metadata and the small arrays of one decode step.

    The KV pool is not stored here: it is produced on demand by
    :func:`build_pool` (whole pool) or :func:`fill_pool` (streamed per
    sequence), so that very large pools need not sit in host memory twice.
    """

    spec: ConfigSpec
    seq_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray  # int32 [S, W], -1 where unused
    query: np.ndarray         # [S, H, D] storage format

    # convenient aliases
    @property
    def num_seqs(self): return self.spec.num_seqs
    @property
    def num_heads(self): return self.spec.num_heads
    @property
    def num_kv_heads(self): return self.spec.num_kv_heads
    @property
    def head_size(self): return self.spec.head_size
    @property
    def block_size(self): return self.spec.block_size
    @property
    def num_blocks(self): return self.spec.num_blocks
    @property
    def max_blocks_per_seq(self): return self.spec.max_blocks_per_seq
    @property
    def partition_size(self): return self.spec.partition_size
    @property
    def dtype(self): return self.spec.dtype
    @property
    def scale(self): return self.spec.softmax_scale

    def kv_bytes(self) -> int:
        """Bytes of K and V that one decode step must read (each element once)."""
        elem = 4 if self.dtype == "f32" else 2
        return int(self.seq_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_size * 2 * elem


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def poison_value(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else BF16_NAN


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def make_problem(spec: ConfigSpec | str, seq_lens: Optional[Sequence[int]] = None,
                 seed: Optional[int] = None, **overrides) -> Problem:
    """Build metadata, block tables and queries for a workload.

    ``seq_lens`` and ``seed`` override the spec's; other keyword arguments
    replace spec fields (e.g. ``partition_size=0``).
    """
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if seed is not None:
        overrides["seed"] = seed
    if overrides:
        spec = dataclasses.replace(spec, **overrides)
    S, W, bs = spec.num_seqs, spec.max_blocks_per_seq, spec.block_size
    if seq_lens is None:
        if spec.seq_len is not None:
            lens = np.full(S, spec.seq_len, dtype=np.int64)
        else:
            lo, hi = spec.seq_len_range
            lens = _rng(spec.seed, _S_LENS).integers(lo, hi + 1, size=S)
    else:
        lens = np.asarray(seq_lens, dtype=np.int64)
        if lens.shape != (S,):
            raise ValueError("seq_lens must have num_seqs entries")
    if (lens < 0).any() or (lens > W * bs).any():
        raise ValueError("seq_lens must lie in [0, max_blocks_per_seq*block_size]")
    nblk = (lens + bs - 1) // bs
    if int(nblk.sum()) > spec.num_blocks:
        raise ValueError("pool too small for the sequences")
    perm = _rng(spec.seed, _S_TABLE).permutation(spec.num_blocks)
    tables = np.full((S, W), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        n = int(nblk[s])
        tables[s, :n] = perm[off:off + n]
        off += n
    q = _rng(spec.seed, _S_QUERY).standard_normal(
        (S, spec.num_heads, spec.head_size), dtype=np.float32)
    return Problem(spec=spec, seq_lens=lens.astype(np.int32), block_tables=tables,
                   query=to_storage(q, spec.dtype))


def sequence_kv_f32(problem: Problem, s: int, kv_head: int):
    """Logical K and V rows of (sequence s, KV head g) as float32, before rounding.

    Returns two arrays of shape [seq_len, head_size].
    """
    spec = problem.spec
    L, D = int(problem.seq_lens[s]), spec.head_size
    k = _rng(spec.seed, _S_KEY, s, kv_head).standard_normal((L, D), dtype=np.float32)
    v = _rng(spec.seed, _S_VALUE, s, kv_head).standard_normal((L, D), dtype=np.float32)
    if spec.outlier_rate > 0.0:
        mask = outlier_positions(problem, s)
        k[mask] *= np.float32(spec.outlier_scale)
    return k, v


def outlier_positions(problem: Problem, s: int) -> np.ndarray:
    """Boolean [seq_len] mask of the key positions scaled as outliers (shared by all KV heads)."""
    spec = problem.spec
    L = int(problem.seq_lens[s])
    if spec.outlier_rate <= 0.0:
        return np.zeros(L, dtype=bool)
    return _rng(spec.seed, _S_OUTLIER, s).random(L) < spec.outlier_rate


def sequence_kv(problem: Problem, s: int, kv_head: int):
    """Logical K and V rows of (s, kv_head) in storage format, shape [seq_len, head_size]."""
    k, v = sequence_kv_f32(problem, s, kv_head)
    return to_storage(k, problem.dtype), to_storage(v, problem.dtype)


def _head_rows(problem: Problem, s: int, g: int, poison: bool):
    """K and V rows of (s, g) padded to whole blocks: [nblk*bs, D] each, tail slots poisoned or zero."""
    D, bs = problem.head_size, problem.block_size
    L = int(problem.seq_lens[s])
    nb = (L + bs - 1) // bs
    sd = storage_dtype(problem.dtype)
    fill = poison_value(problem.dtype) if poison else sd(0)
    k, v = sequence_kv(problem, s, g)
    if nb * bs == L:
        return k, v
    kp = np.full((nb * bs, D), fill, dtype=sd)
    vp = np.full((nb * bs, D), fill, dtype=sd)
    kp[:L] = k
    vp[:L] = v
    return kp, vp


def _assemble(problem: Problem, s: int, rows):
    """Per-head padded rows -> (block ids, K blocks, V blocks) with blocks [nblk, Hkv, bs, D]."""
    Hkv, D, bs = problem.num_kv_heads, problem.head_size, problem.block_size
    nb = (int(problem.seq_lens[s]) + bs - 1) // bs
    sd = storage_dtype(problem.dtype)
    kb = np.empty((nb, Hkv, bs, D), dtype=sd)
    vb = np.empty((nb, Hkv, bs, D), dtype=sd)
    for g, (k, v) in enumerate(rows):
        kb[:, g] = k.reshape(nb, bs, D)
        vb[:, g] = v.reshape(nb, bs, D)
    return problem.block_tables[s, :nb].copy(), kb, vb


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_pool(problem: Problem, sink: Callable[[np.ndarray, np.ndarray, np.ndarray], None],
              poison: bool = True, threads: Optional[int] = None) -> None:
    """Stream the pool contents sequence by sequence.

    ``sink(block_ids, k_blocks, v_blocks)`` receives int32 [n] physical ids and
    the matching [n, Hkv, bs, D] blocks.  Blocks that no table references are
    never passed; the caller decides their contents (poison in the tests).
    (sequence, KV head) slices are generated on a thread pool, at most two
    sequences ahead of the one being handed to ``sink`` (called from the
    calling thread, in sequence order).
    """
    threads = threads or default_threads()
    S, Hkv = problem.num_seqs, problem.num_kv_heads
    if threads <= 1:
        for s in range(S):
            sink(*_assemble(problem, s, [_head_rows(problem, s, g, poison) for g in range(Hkv)]))
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        pending = {}

        def submit(s):
            if s < S:
                pending[s] = [ex.submit(_head_rows, problem, s, g, poison) for g in range(Hkv)]

        submit(0)
        submit(1)
        for s in range(S):
            submit(s + 2)
            rows = [f.result() for f in pending.pop(s)]
            sink(*_assemble(problem, s, rows))


def to_tiled(k_blocks: np.ndarray, v_blocks: np.ndarray, dtype: str):
    """Rows-layout blocks [n, Hkv, bs, D] -> the tiled layout: K [n, Hkv, D/x, bs, x]
    with x = 16 bytes of elements, V [n, Hkv, D, bs].  A pure permutation."""
    n, hkv, bs, d = k_blocks.shape
    x = 16 // np.dtype(storage_dtype(dtype)).itemsize
    kt = np.ascontiguousarray(k_blocks.reshape(n, hkv, bs, d // x, x).transpose(0, 1, 3, 2, 4))
    vt = np.ascontiguousarray(v_blocks.transpose(0, 1, 3, 2))
    return kt, vt


def build_pool(problem: Problem, poison: bool = True, threads: Optional[int] = None):
    """Whole K and V pools on the host, unreferenced blocks filled with poison (NaN)."""
    shape = (problem.num_blocks, problem.num_kv_heads, problem.block_size, problem.head_size)
    sd = storage_dtype(problem.dtype)
    fill = poison_value(problem.dtype) if poison else sd(0)
    kc = np.full(shape, fill, dtype=sd)
    vc = np.full(shape, fill, dtype=sd)

    def sink(ids, kb, vb):
        kc[ids] = kb
        vc[ids] = vb

    fill_pool(problem, sink, poison=poison, threads=threads)
    return kc, vc


def logical_kv(problem: Problem, s: int) -> List[tuple]:
    """[(K_g, V_g) for each KV head] of sequence s in storage format."""
    return [sequence_kv(problem, s, g) for g in range(problem.num_kv_heads)]


# ---------------------------------------------------------------------------
# Prefix (chunked prefill) attention inputs
# ---------------------------------------------------------------------------

_S_PREFILL_QUERY = 6


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    """Shape and value recipe of one prefill workload: per sequence, a cached
    context of ``context_lens[s]`` tokens and a chunk of ``query_lens[s]`` new
    tokens (whose keys and values also go into the cache)."""

    name: str
    context_lens: tuple
    query_lens: tuple
    num_heads: int
    num_kv_heads: int
    head_size: int
    dtype: str
    seed: int
    block_size: int = 16
    num_blocks: Optional[int] = None  # default: twice the blocks the sequences need
    scale: Optional[float] = None     # default 1/sqrt(head_size)

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(self.scale if self.scale is not None
                                else 1.0 / math.sqrt(self.head_size)))


# Shapes are the pages' model attention shape (24 query / 4 KV heads, head
# 256).  "prefill" is one chunk of 8192 new tokens (the serving
# configuration's batched-token budget on the second page) over a 32768-token
# cached prefix; the others are ragged batches that span several query tiles,
# empty chunks and empty contexts.
PREFILL_CONFIGS: Dict[str, PrefillSpec] = {
    "prefill_small": PrefillSpec("prefill_small", context_lens=(0, 37, 200, 16, 5), query_lens=(50, 1, 77, 128, 0),
                                 num_heads=24, num_kv_heads=4, head_size=256, dtype="bf16", seed=11),
    "prefill": PrefillSpec("prefill", context_lens=(32768,), query_lens=(8192,), num_heads=24, num_kv_heads=4,
                           head_size=256, dtype="bf16", seed=12),
    "prefill_batch": PrefillSpec("prefill_batch", context_lens=(0, 5000, 12345, 30000),
                                 query_lens=(2048, 1000, 777, 3000), num_heads=24, num_kv_heads=4, head_size=256,
                                 dtype="bf16", seed=13),
}


@dataclasses.dataclass
class PrefillProblem:
    """A prefill step: the packed chunk queries and the paged cache holding, per
    sequence, its context followed by its chunk (an inner decode
    :class:`Problem` whose sequence lengths are context + chunk supplies the
    block tables and the K/V generator)."""

    spec: PrefillSpec
    pool: Problem                # seq_lens = context + chunk; block tables, K/V streams
    context_lens: np.ndarray     # int32 [S]
    query_lens: np.ndarray       # int32 [S]
    query_start: np.ndarray      # int32 [S + 1]
    query: np.ndarray            # [T, H, D] storage format

    @property
    def num_seqs(self): return len(self.context_lens)
    @property
    def num_tokens(self): return int(self.query_start[-1])
    @property
    def max_query_len(self): return int(self.query_lens.max()) if len(self.query_lens) else 0
    @property
    def scale(self): return self.spec.softmax_scale

    def chunk_kv(self):
        """The chunk's own key and value rows [T, Hkv, D] (storage format): positions
        context .. context + n - 1 of each sequence."""
        T, Hkv, D = self.num_tokens, self.spec.num_kv_heads, self.spec.head_size
        sd = storage_dtype(self.spec.dtype)
        key = np.empty((T, Hkv, D), dtype=sd)
        value = np.empty((T, Hkv, D), dtype=sd)
        for s in range(self.num_seqs):
            lo, hi = int(self.query_start[s]), int(self.query_start[s + 1])
            c = int(self.context_lens[s])
            for g in range(Hkv):
                k, v = sequence_kv(self.pool, s, g)
                key[lo:hi, g] = k[c:c + hi - lo]
                value[lo:hi, g] = v[c:c + hi - lo]
        return key, value

    def flops(self) -> int:
        """Algorithmic flops: 4 H D per (query row, visible key) pair."""
        per_row = 0
        for s in range(self.num_seqs):
            c, n = int(self.context_lens[s]), int(self.query_lens[s])
            per_row += n * c + n * (n + 1) // 2
        return 4 * self.spec.num_heads * self.spec.head_size * per_row


def make_prefill_problem(spec: PrefillSpec | str, **overrides) -> PrefillProblem:
    if isinstance(spec, str):
        spec = PREFILL_CONFIGS[spec]
    if overrides:
        spec = dataclasses.replace(spec, **overrides)
    ctx = np.asarray(spec.context_lens, dtype=np.int64)
    qn = np.asarray(spec.query_lens, dtype=np.int64)
    if ctx.shape != qn.shape or (ctx < 0).any() or (qn < 0).any():
        raise ValueError("context_lens and query_lens must be non-negative and of one length")
    S, bs = len(ctx), spec.block_size
    total = ctx + qn
    W = max(1, int(((total + bs - 1) // bs).max()) if S else 1)
    need = int(((total + bs - 1) // bs).sum())
    NB = spec.num_blocks or max(2 * need, 1)
    inner = ConfigSpec(spec.name, num_seqs=S, num_heads=spec.num_heads, num_kv_heads=spec.num_kv_heads,
                       head_size=spec.head_size, block_size=bs, num_blocks=NB, max_blocks_per_seq=W,
                       partition_size=0, dtype=spec.dtype, seed=spec.seed, scale=spec.scale)
    pool = make_problem(inner, seq_lens=total)
    qs = np.zeros(S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(qn)
    q = _rng(spec.seed, _S_PREFILL_QUERY).standard_normal((int(qs[-1]), spec.num_heads, spec.head_size),
                                                          dtype=np.float32)
    return PrefillProblem(spec=spec, pool=pool, context_lens=ctx.astype(np.int32), query_lens=qn.astype(np.int32),
                          query_start=qs, query=to_storage(q, spec.dtype))
