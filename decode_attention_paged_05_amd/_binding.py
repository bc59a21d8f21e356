"""ctypes binding of ``libpad.so``: argument marshalling only.

Every entry point of ``include/paged_attention_decode.h`` and
``include/paged_attention_prefill.h`` has a Python function of the same name.  Tensors are torch tensors on the current CUDA (HIP) device;
torch supplies device memory and the stream, all arithmetic runs in the
library's HIP kernels.  A missing library raises at import of this module, and
a non-zero status raises ``RuntimeError`` with the library's message.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpad.so")

PAD_DTYPE_F32 = 0
PAD_DTYPE_BF16 = 1
PAD_KV_ROWS = 0
PAD_KV_TILED = 1

STATUS = {
    0: "PAD_OK", -1: "PAD_ERR_NULL", -2: "PAD_ERR_DTYPE", -3: "PAD_ERR_SHAPE",
    -4: "PAD_ERR_UNSUPPORTED", -5: "PAD_ERR_PARTITION", -6: "PAD_ERR_WORKSPACE", -7: "PAD_ERR_ALIGN",
    -8: "PAD_ERR_TOO_LARGE",
}

EXPORTED = [
    "paged_attention_decode",
    "paged_attention_decode_no_alloc",
    "paged_attention_decode_phase1",
    "paged_attention_decode_phase2",
    "paged_attention_decode_workspace_size",
    "paged_attention_decode_workspace_layout",
    "paged_attention_decode_workspace_init",
    "paged_attention_decode_choose_partition",
    "paged_attention_decode_choose_partition_for_batch",
    "paged_attention_decode_strerror",
    "paged_attention_decode_entry_ranges",
    "paged_attention_decode_build_id",
    "paged_attention_prefill",
    "paged_attention_prefill_choose_split",
    "paged_attention_prefill_split",
    "paged_attention_prefill_split_ranges",
    "paged_attention_prefill_split_workspace_size",
    "paged_attention_prefill_write_kv",
]


class PadDims(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("query_seq_stride", ctypes.c_int64),
        ("out_seq_stride", ctypes.c_int64),
    ]


class PadPrefillDims(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("max_query_len", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
    ]


class PadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {strerror(status)}")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    # torch's HIP runtime must be the one libpad.so binds to: streams and
    # device memory are objects of that runtime.  Loading torch first makes
    # the dynamic linker resolve libpad's libamdhip64.so.7 to torch's copy
    # instead of loading a second runtime from /opt/rocm.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python decode_attention_paged_05_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    dims = ctypes.POINTER(PadDims)
    lib.paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, sz, dims, vp]
    lib.paged_attention_decode.restype = i32
    lib.paged_attention_decode_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, dims, vp]
    lib.paged_attention_decode_no_alloc.restype = i32
    lib.paged_attention_decode_phase1.argtypes = [vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, sz, dims, vp]
    lib.paged_attention_decode_phase1.restype = i32
    lib.paged_attention_decode_phase2.argtypes = [vp, vp, i32, i32, i32, vp, sz, dims, vp]
    lib.paged_attention_decode_phase2.restype = i32
    lib.paged_attention_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_attention_decode_workspace_size.restype = sz
    lib.paged_attention_decode_workspace_layout.argtypes = [i32, i32, i32, i32, i32, i32,
                                                             ctypes.POINTER(sz), ctypes.POINTER(sz),
                                                             ctypes.POINTER(sz)]
    lib.paged_attention_decode_workspace_layout.restype = i32
    lib.paged_attention_decode_workspace_init.argtypes = [vp, sz, i32, i32, i32, i32, i32, i32, vp]
    lib.paged_attention_decode_workspace_init.restype = i32
    lib.paged_attention_decode_choose_partition.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_attention_decode_choose_partition.restype = i32
    lib.paged_attention_decode_choose_partition_for_batch.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, i32]
    lib.paged_attention_decode_choose_partition_for_batch.restype = i32
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.paged_attention_decode_entry_ranges.argtypes = [ip, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, ip, ip,
                                                        ip]
    lib.paged_attention_decode_entry_ranges.restype = i32
    lib.paged_attention_decode_build_id.argtypes = []
    lib.paged_attention_decode_build_id.restype = ctypes.c_char_p
    lib.paged_attention_decode_strerror.argtypes = [i32]
    lib.paged_attention_decode_strerror.restype = ctypes.c_char_p
    pdims = ctypes.POINTER(PadPrefillDims)
    lib.paged_attention_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, pdims, vp]
    lib.paged_attention_prefill.restype = i32
    lib.paged_attention_prefill_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, pdims, vp, sz, vp]
    lib.paged_attention_prefill_split.restype = i32
    lib.paged_attention_prefill_choose_split.argtypes = [ip, ip, i32, i32, i32, i32, i32]
    lib.paged_attention_prefill_choose_split.restype = i32
    lib.paged_attention_prefill_split_ranges.argtypes = [i32, i32, i32]
    lib.paged_attention_prefill_split_ranges.restype = i32
    lib.paged_attention_prefill_split_workspace_size.argtypes = [pdims, i32, i32]
    lib.paged_attention_prefill_split_workspace_size.restype = sz
    lib.paged_attention_prefill_write_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, pdims, vp]
    lib.paged_attention_prefill_write_kv.restype = i32
    del i64
    return lib


LIB = _load()


def strerror(status: int) -> str:
    return LIB.paged_attention_decode_strerror(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PadError(status, where)


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PAD_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return PAD_DTYPE_BF16
    raise TypeError(f"query/key/value must be float32 or bfloat16, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _seq_rows_ptr(t) -> Optional[int]:
    """Pointer of a [S, H, D] tensor whose [H, D] rows are contiguous; the
    sequence stride (passed in pad_dims_t) may be wider."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2] or (t.shape[0] > 1 and
                                                                          t.stride(0) < t.shape[1] * t.shape[2]):
        raise ValueError("query / out must be [S, H, D] with contiguous [H, D] rows")
    return t.data_ptr()


def _seq_stride(t) -> int:
    return int(t.stride(0)) if t is not None and t.shape[0] > 1 else 0


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def cache_layout(key_cache, value_cache) -> int:
    """PAD_KV_ROWS for 4-D K [NB,Hkv,bs,D]; PAD_KV_TILED for 5-D K [NB,Hkv,D/x,bs,x] with V [NB,Hkv,D,bs]."""
    if key_cache.dim() == 4:
        return PAD_KV_ROWS
    if key_cache.dim() == 5 and value_cache.dim() == 4:
        return PAD_KV_TILED
    raise ValueError("key_cache must be 4-D (rows layout) or 5-D (tiled layout)")


def make_dims(query, key_cache, block_tables, value_cache=None, out=None) -> PadDims:
    """Sizes of a decode call; the sequence strides of query (and out, when
    given) go into query_seq_stride / out_seq_stride."""
    if query.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("expected query [S,H,D] and block_tables [S,W]")
    S, H, D = query.shape
    layout = PAD_KV_TILED if key_cache.dim() == 5 else PAD_KV_ROWS
    return PadDims(_dtype_code(query), S, H, D, key_cache.shape[0], block_tables.shape[1], layout,
                   _seq_stride(query), _seq_stride(out))


def _check_tensors(out, query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, block_size):
    torch = _torch()
    if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
        raise TypeError("query, key_cache and value_cache must share a dtype")
    S, H, D = query.shape
    layout = cache_layout(key_cache, value_cache)
    NB = key_cache.shape[0]
    if layout == PAD_KV_ROWS:
        want_k = want_v = (NB, num_kv_heads, block_size, D)
    else:
        x = 16 // query.element_size()
        want_k = (NB, num_kv_heads, D // x, block_size, x)
        want_v = (NB, num_kv_heads, D, block_size)
    if tuple(key_cache.shape) != want_k or tuple(value_cache.shape) != want_v:
        raise ValueError(f"caches must be K {want_k} and V {want_v}, got {tuple(key_cache.shape)} and "
                         f"{tuple(value_cache.shape)}")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if block_tables.shape[0] != S or tuple(seq_lens.shape) != (S,):
        raise ValueError("block_tables / seq_lens disagree with num_seqs")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (S, H, D)):
        raise ValueError("out must be float32 [num_seqs, num_heads, head_size]")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def paged_attention_decode(out, query, key_cache, value_cache, block_tables, seq_lens, scale: float,
                           num_kv_heads: int, block_size: int, partition_size: int, workspace=None,
                           stream=None) -> None:
    """Decode attention into ``out`` (float32 [S, H, D]); see the C header for the contract."""
    _check_tensors(out, query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, block_size)
    dims = make_dims(query, key_cache, block_tables, out=out)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.paged_attention_decode(_seq_rows_ptr(out), _seq_rows_ptr(query), _ptr(key_cache), _ptr(value_cache),
                                    _ptr(block_tables), _ptr(seq_lens), float(scale), int(num_kv_heads),
                                    int(block_size), int(partition_size), ws_ptr, ws_bytes,
                                    ctypes.byref(dims), _stream(stream))
    _check(st, "paged_attention_decode")


def paged_attention_decode_no_alloc(out, query, key_cache, value_cache, block_tables, seq_lens, scale: float,
                                    num_kv_heads: int, block_size: int, partition_size: int, stream=None) -> None:
    """Decode attention with the library's static workspace (no allocation); see the C header."""
    _check_tensors(out, query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, block_size)
    dims = make_dims(query, key_cache, block_tables, out=out)
    st = LIB.paged_attention_decode_no_alloc(_seq_rows_ptr(out), _seq_rows_ptr(query), _ptr(key_cache),
                                             _ptr(value_cache),
                                             _ptr(block_tables), _ptr(seq_lens), float(scale), int(num_kv_heads),
                                             int(block_size), int(partition_size), ctypes.byref(dims),
                                             _stream(stream))
    _check(st, "paged_attention_decode_no_alloc")


def paged_attention_decode_phase1(query, key_cache, value_cache, block_tables, seq_lens, scale: float,
                                  num_kv_heads: int, block_size: int, partition_size: int, workspace,
                                  stream=None) -> None:
    _check_tensors(None, query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, block_size)
    dims = make_dims(query, key_cache, block_tables)
    st = LIB.paged_attention_decode_phase1(_seq_rows_ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                                           _ptr(seq_lens), float(scale), int(num_kv_heads), int(block_size),
                                           int(partition_size), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), ctypes.byref(dims),
                                           _stream(stream))
    _check(st, "paged_attention_decode_phase1")


def paged_attention_decode_phase2(out, seq_lens, num_kv_heads: int, block_size: int, partition_size: int, workspace,
                                  dims: PadDims, stream=None) -> None:
    """Phase 2 into ``out``; ``dims`` as for phase 1 (its out_seq_stride is taken from ``out``)."""
    dims = PadDims(*[getattr(dims, f) for f, _ in PadDims._fields_])
    dims.out_seq_stride = _seq_stride(out)
    st = LIB.paged_attention_decode_phase2(_seq_rows_ptr(out), _ptr(seq_lens), int(num_kv_heads), int(block_size),
                                           int(partition_size),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           ctypes.byref(dims), _stream(stream))
    _check(st, "paged_attention_decode_phase2")


def paged_attention_decode_workspace_size(num_seqs: int, num_heads: int, head_size: int, max_blocks_per_seq: int,
                                          block_size: int, partition_size: int) -> int:
    n = LIB.paged_attention_decode_workspace_size(num_seqs, num_heads, head_size, max_blocks_per_seq, block_size,
                                                  partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace-size arguments")
    return int(n)


def paged_attention_decode_workspace_layout(num_seqs, num_heads, head_size, max_blocks_per_seq, block_size,
                                            partition_size):
    """(max_logits, exp_sums, tmp_output) byte offsets inside the workspace."""
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = LIB.paged_attention_decode_workspace_layout(num_seqs, num_heads, head_size, max_blocks_per_seq,
                                                     block_size, partition_size, ctypes.byref(a), ctypes.byref(b),
                                                     ctypes.byref(c))
    _check(st, "paged_attention_decode_workspace_layout")
    return a.value, b.value, c.value


def paged_attention_decode_workspace_init(workspace, num_seqs, num_heads, head_size, max_blocks_per_seq, block_size,
                                          partition_size, stream=None) -> None:
    st = LIB.paged_attention_decode_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   num_seqs, num_heads, head_size, max_blocks_per_seq, block_size,
                                                   partition_size, _stream(stream))
    _check(st, "paged_attention_decode_workspace_init")


def paged_attention_decode_choose_partition(num_seqs, num_heads, num_kv_heads, max_context_len, block_size,
                                            num_cus=256) -> int:
    r = LIB.paged_attention_decode_choose_partition(num_seqs, num_heads, num_kv_heads, max_context_len, block_size,
                                                    num_cus)
    if r < 0:
        raise PadError(r, "paged_attention_decode_choose_partition")
    return int(r)


def paged_attention_decode_choose_partition_for_batch(num_seqs, num_heads, num_kv_heads, head_size, dtype: str,
                                                      max_context_len, total_context_len, block_size,
                                                      num_cus=256) -> int:
    """Partition size for a batch of (possibly) unequal lengths: ``dtype`` is
    "bf16" or "f32", ``total_context_len`` the sum of the sequence lengths."""
    code = {"f32": PAD_DTYPE_F32, "bf16": PAD_DTYPE_BF16}.get(dtype)
    if code is None:
        raise ValueError(f"dtype must be 'bf16' or 'f32', not {dtype!r}")
    r = LIB.paged_attention_decode_choose_partition_for_batch(num_seqs, num_heads, num_kv_heads, head_size, code,
                                                              max_context_len, total_context_len, block_size,
                                                              num_cus)
    if r < 0:
        raise PadError(r, "paged_attention_decode_choose_partition_for_batch")
    return int(r)


def paged_attention_decode_strerror(status: int) -> str:
    return strerror(status)


def paged_attention_decode_build_id() -> str:
    return LIB.paged_attention_decode_build_id().decode()


def check_build() -> str:
    """Raise unless the loaded libpad.so was built from the sources in this tree
    (its build id equals the hash of csrc/ and include/); returns the id."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("_pad_build_hash", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    want, got = mod.source_hash(), paged_attention_decode_build_id()
    if want != got:
        raise RuntimeError(f"{LIB_PATH} was built from other sources (build id {got}, sources {want}); rebuild it")
    return got


def paged_attention_decode_entry_ranges(seq_lens, num_heads: int, num_kv_heads: int, max_blocks_per_seq: int,
                                        block_size: int, partition_size: int, num_cus: int = 256,
                                        layout: str = "tiled", head_size: int = 256, dtype: str = "bf16"):
    """Where phase 1 puts each (sequence, head)'s results, for host lengths,
    heads of ``head_size``, elements of ``dtype`` ("bf16" or "f32") and a cache
    in ``layout`` ("tiled" or "rows").

    Returns ``(balanced, count [S, H], begin [S, H, NP], end [S, H, NP])`` as
    NumPy int32 arrays: slot e < count[s, h] of (s, h) holds tokens
    [begin, end); count is 0 for an empty sequence and -1 for a length outside
    the table.
    """
    import numpy as np

    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    S = int(lens.shape[0])
    kv_layout = {"rows": PAD_KV_ROWS, "tiled": PAD_KV_TILED}.get(layout)
    if kv_layout is None:
        raise ValueError(f"layout must be 'tiled' or 'rows', not {layout!r}")
    code = {"f32": PAD_DTYPE_F32, "bf16": PAD_DTYPE_BF16}.get(dtype)
    if code is None:
        raise ValueError(f"dtype must be 'bf16' or 'f32', not {dtype!r}")
    if partition_size <= 0 or partition_size % block_size:
        raise PadError(-5, "paged_attention_decode_entry_ranges")
    NP = -(-max_blocks_per_seq * block_size // partition_size)
    count = np.zeros((S, num_heads), dtype=np.int32)
    begin = np.zeros((S, num_heads, NP), dtype=np.int32)
    end = np.zeros((S, num_heads, NP), dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int32)
    r = LIB.paged_attention_decode_entry_ranges(lens.ctypes.data_as(ip), S, int(num_heads), int(num_kv_heads),
                                                int(head_size), code, int(max_blocks_per_seq), int(block_size),
                                                int(partition_size),
                                                kv_layout, int(num_cus), count.ctypes.data_as(ip),
                                                begin.ctypes.data_as(ip),
                                                end.ctypes.data_as(ip))
    if r < 0:
        raise PadError(r, "paged_attention_decode_entry_ranges")
    return bool(r), count, begin, end


def alloc_workspace(num_seqs, num_heads, head_size, max_blocks_per_seq, block_size, partition_size, device=None,
                    init=True, stream=None):
    """Allocate (torch, uint8) and optionally initialise a workspace for split calls."""
    torch = _torch()
    n = paged_attention_decode_workspace_size(num_seqs, num_heads, head_size, max_blocks_per_seq, block_size,
                                              partition_size)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")
    if init and n:
        paged_attention_decode_workspace_init(ws, num_seqs, num_heads, head_size, max_blocks_per_seq, block_size,
                                              partition_size, stream)
    return ws


# ---------------------------------------------------------------------------
# prefix (chunked prefill) attention
# ---------------------------------------------------------------------------

def make_prefill_dims(query, key_cache, block_tables, max_query_len: int, num_tokens=None) -> PadPrefillDims:
    """Sizes of a prefill call; ``query`` is [T, H, D] (or the chunk keys [T, Hkv, D] for the write)."""
    if query.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("expected rows [T, heads, D] and block_tables [S, W]")
    T, H, D = query.shape
    layout = PAD_KV_TILED if key_cache.dim() == 5 else PAD_KV_ROWS
    return PadPrefillDims(_dtype_code(query), block_tables.shape[0], T if num_tokens is None else num_tokens, H, D,
                          int(max_query_len), key_cache.shape[0], block_tables.shape[1], layout)


def _check_prefill(query, key_cache, value_cache, block_tables, query_start, context_lens, num_kv_heads,
                   block_size, heads_of_rows):
    torch = _torch()
    if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
        raise TypeError("rows and caches must share a dtype")
    T, _, D = query.shape
    layout = cache_layout(key_cache, value_cache)
    NB = key_cache.shape[0]
    if layout == PAD_KV_ROWS:
        want_k = want_v = (NB, num_kv_heads, block_size, D)
    else:
        x = 16 // query.element_size()
        want_k = (NB, num_kv_heads, D // x, block_size, x)
        want_v = (NB, num_kv_heads, D, block_size)
    if tuple(key_cache.shape) != want_k or tuple(value_cache.shape) != want_v:
        raise ValueError(f"caches must be K {want_k} and V {want_v}, got {tuple(key_cache.shape)} and "
                         f"{tuple(value_cache.shape)}")
    S = block_tables.shape[0]
    for name, t in (("block_tables", block_tables), ("query_start", query_start), ("context_lens", context_lens)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if tuple(query_start.shape) != (S + 1,) or tuple(context_lens.shape) != (S,):
        raise ValueError("query_start must be [num_seqs + 1] and context_lens [num_seqs]")
    if heads_of_rows is not None and query.shape[1] != heads_of_rows:
        raise ValueError(f"rows must have {heads_of_rows} heads")


def paged_attention_prefill(out, query, key_cache, value_cache, block_tables, query_start, context_lens,
                            scale: float, num_kv_heads: int, block_size: int, max_query_len: int,
                            stream=None) -> None:
    """Prefix attention of the chunk rows ``query`` [T, H, D] into ``out`` (float32 [T, H, D])."""
    torch = _torch()
    _check_prefill(query, key_cache, value_cache, block_tables, query_start, context_lens, num_kv_heads,
                   block_size, None)
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must be float32 with the shape of query")
    dims = make_prefill_dims(query, key_cache, block_tables, max_query_len)
    st = LIB.paged_attention_prefill(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                     _ptr(block_tables), _ptr(query_start), _ptr(context_lens), float(scale),
                                     int(num_kv_heads), int(block_size), ctypes.byref(dims), _stream(stream))
    _check(st, "paged_attention_prefill")


def paged_attention_prefill_split_ranges(head_size: int, num_heads: int, num_kv_heads: int) -> int:
    """Ranges the balanced split cuts a prefill launch into on the current device."""
    n = LIB.paged_attention_prefill_split_ranges(int(head_size), int(num_heads), int(num_kv_heads))
    _check(n if n < 0 else 0, "paged_attention_prefill_split_ranges")
    return n


def paged_attention_prefill_choose_split(context_lens, query_lens, num_heads: int, num_kv_heads: int,
                                         head_size: int, num_ranges: int) -> bool:
    """Whether the split launch serves these lengths (host sequences of ints) better than the plain one."""
    import numpy as np
    c = np.ascontiguousarray(context_lens, dtype=np.int32)
    q = np.ascontiguousarray(query_lens, dtype=np.int32)
    if c.shape != q.shape or c.ndim != 1:
        raise ValueError("context_lens and query_lens must be 1-D of one length")
    ip = ctypes.POINTER(ctypes.c_int32)
    r = LIB.paged_attention_prefill_choose_split(c.ctypes.data_as(ip), q.ctypes.data_as(ip), int(c.size),
                                                 int(num_heads), int(num_kv_heads), int(head_size), int(num_ranges))
    _check(r if r < 0 else 0, "paged_attention_prefill_choose_split")
    return r == 1


def paged_attention_prefill_split_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                                                 max_query_len: int, max_blocks_per_seq: int, num_ranges: int) -> int:
    dims = PadPrefillDims(PAD_DTYPE_BF16, int(num_seqs), 0, int(num_heads), int(head_size), int(max_query_len), 1,
                          int(max_blocks_per_seq), PAD_KV_TILED)
    n = LIB.paged_attention_prefill_split_workspace_size(ctypes.byref(dims), int(num_kv_heads), int(num_ranges))
    if n == ctypes.c_size_t(-1).value:
        raise PadError(-3, "paged_attention_prefill_split_workspace_size (sizes out of range)")
    return n


def alloc_prefill_split_workspace(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                                  max_query_len: int, max_blocks_per_seq: int, device=None):
    """Allocate (torch, uint8) a workspace for paged_attention_prefill_split on the current device."""
    torch = _torch()
    n = paged_attention_prefill_split_workspace_size(
        num_seqs, num_heads, num_kv_heads, head_size, max_query_len, max_blocks_per_seq,
        paged_attention_prefill_split_ranges(head_size, num_heads, num_kv_heads))
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def paged_attention_prefill_split(out, query, key_cache, value_cache, block_tables, query_start, context_lens,
                                  scale: float, num_kv_heads: int, block_size: int, max_query_len: int, workspace,
                                  stream=None) -> None:
    """paged_attention_prefill with the launch's work cut into equal ranges (``workspace``: uint8 tensor)."""
    torch = _torch()
    _check_prefill(query, key_cache, value_cache, block_tables, query_start, context_lens, num_kv_heads,
                   block_size, None)
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must be float32 with the shape of query")
    dims = make_prefill_dims(query, key_cache, block_tables, max_query_len)
    st = LIB.paged_attention_prefill_split(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                           _ptr(block_tables), _ptr(query_start), _ptr(context_lens), float(scale),
                                           int(num_kv_heads), int(block_size), ctypes.byref(dims), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "paged_attention_prefill_split")


def paged_attention_prefill_write_kv(key_cache, value_cache, key, value, block_tables, query_start, context_lens,
                                     num_kv_heads: int, block_size: int, max_query_len: int, stream=None) -> None:
    """Store the chunk rows ``key`` / ``value`` [T, Hkv, D] in the cache at their positions."""
    _check_prefill(key, key_cache, value_cache, block_tables, query_start, context_lens, num_kv_heads,
                   block_size, num_kv_heads)
    if value.shape != key.shape or value.dtype != key.dtype:
        raise ValueError("key and value must have one shape and dtype")
    dims = make_prefill_dims(key, key_cache, block_tables, max_query_len)
    st = LIB.paged_attention_prefill_write_kv(_ptr(key_cache), _ptr(value_cache), _ptr(key), _ptr(value),
                                              _ptr(block_tables), _ptr(query_start), _ptr(context_lens),
                                              int(num_kv_heads), int(block_size), ctypes.byref(dims),
                                              _stream(stream))
    _check(st, "paged_attention_prefill_write_kv")
