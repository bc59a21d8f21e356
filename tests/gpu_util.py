"""Upload of seeded problems to the GPU and the oracle comparisons the GPU tests share."""

from __future__ import annotations

import numpy as np
import torch

import decode_attention_paged_05_amd as pad
import oracle
from decode_attention_paged_05_amd import inputs as gen

TOL = {"f32": 1e-5, "bf16": 2e-3}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (run with -m 'not gpu' on a CPU-only host)")
    pad.check_build()  # the library under test was built from these sources


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def torch_dtype(dtype: str):
    return torch.float32 if dtype == "f32" else torch.bfloat16


LAYOUTS = ("rows", "tiled")


def tiled_shapes(problem: gen.Problem):
    x = 16 // np.dtype(gen.storage_dtype(problem.dtype)).itemsize
    NB, Hkv, bs, D = problem.num_blocks, problem.num_kv_heads, problem.block_size, problem.head_size
    return (NB, Hkv, D // x, bs, x), (NB, Hkv, D, bs)


class DeviceProblem:
    """A problem's inputs on the GPU in one or both cache layouts (pool
    poisoned with NaN outside referenced rows), optionally with the host pool
    (rows layout) kept for the oracle."""

    def __init__(self, problem: gen.Problem, keep_host: bool = True, device="cuda", layouts=LAYOUTS):
        require_gpu()
        self.p = problem
        shape = (problem.num_blocks, problem.num_kv_heads, problem.block_size, problem.head_size)
        td = torch_dtype(problem.dtype)
        self.caches = {}
        if "rows" in layouts:
            self.caches["rows"] = (torch.full(shape, float("nan"), dtype=td, device=device),
                                   torch.full(shape, float("nan"), dtype=td, device=device))
        if "tiled" in layouts:
            ks, vs = tiled_shapes(problem)
            self.caches["tiled"] = (torch.full(ks, float("nan"), dtype=td, device=device),
                                    torch.full(vs, float("nan"), dtype=td, device=device))
        self.layout = layouts[0]
        self.kc_host = self.vc_host = None
        if keep_host:
            sd = gen.storage_dtype(problem.dtype)
            fill = gen.poison_value(problem.dtype)
            self.kc_host = np.full(shape, fill, dtype=sd)
            self.vc_host = np.full(shape, fill, dtype=sd)

        def sink(ids, kb, vb):
            idx = torch.from_numpy(ids.astype(np.int64)).to(device)
            if "rows" in self.caches:
                k, v = self.caches["rows"]
                k.index_copy_(0, idx, to_device(kb, problem.dtype, device))
                v.index_copy_(0, idx, to_device(vb, problem.dtype, device))
            if "tiled" in self.caches:
                kt, vt = gen.to_tiled(kb, vb, problem.dtype)
                k, v = self.caches["tiled"]
                k.index_copy_(0, idx, to_device(kt, problem.dtype, device))
                v.index_copy_(0, idx, to_device(vt, problem.dtype, device))
            if keep_host:
                self.kc_host[ids] = kb
                self.vc_host[ids] = vb

        gen.fill_pool(problem, sink)
        self.query = to_device(problem.query, problem.dtype, device)
        self.tables = torch.from_numpy(problem.block_tables).to(device)
        self.lens = torch.from_numpy(problem.seq_lens).to(device)
        torch.cuda.synchronize()

    @property
    def kc(self):
        return self.caches[self.layout][0]

    @property
    def vc(self):
        return self.caches[self.layout][1]

    def use(self, layout: str) -> "DeviceProblem":
        self.layout = layout
        return self

    def workspace(self, partition_size: int, init: bool = True):
        p = self.p
        return pad.alloc_workspace(p.num_seqs, p.num_heads, p.head_size, p.max_blocks_per_seq, p.block_size,
                                   partition_size, init=init)

    def run(self, partition_size: int | None = None, workspace=None, out=None, kc=None, vc=None, tables=None,
            lens=None) -> torch.Tensor:
        p = self.p
        P = p.partition_size if partition_size is None else partition_size
        if out is None:
            out = torch.full((p.num_seqs, p.num_heads, p.head_size), float("nan"), dtype=torch.float32,
                             device=self.query.device)
        if P and workspace is None:
            workspace = self.workspace(P)
        pad.paged_attention_decode(out, self.query, self.kc if kc is None else kc, self.vc if vc is None else vc,
                                   self.tables if tables is None else tables, self.lens if lens is None else lens,
                                   p.scale, p.num_kv_heads, p.block_size, P, workspace)
        return out

    def oracle(self) -> np.ndarray:
        p = self.p
        return oracle.decode_attention(p.query, self.kc_host, self.vc_host, p.block_tables, p.seq_lens, p.scale,
                                       p.num_kv_heads, p.block_size, p.dtype)

    def oracle_split(self, partition_size: int):
        p = self.p
        return oracle.decode_attention_split(p.query, self.kc_host, self.vc_host, p.block_tables, p.seq_lens,
                                             p.scale, p.num_kv_heads, p.block_size, p.dtype, partition_size)


def max_err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape
    assert np.isfinite(g).all(), f"non-finite GPU output at {np.argwhere(~np.isfinite(g))[:5].tolist()}"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def assert_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str = ""):
    err = max_err(gpu, ref)
    tol = TOL[dtype]
    if err > tol:
        g = gpu.detach().cpu().numpy().astype(np.float64)
        idx = np.unravel_index(np.argmax(np.abs(g - ref)), ref.shape)
        raise AssertionError(f"{what}: max |gpu - oracle| = {err:.3e} > {tol:.0e} at {idx}: "
                             f"gpu {g[idx]!r} oracle {ref[idx]!r}")
    return err


def workspace_views(ws: torch.Tensor, p: gen.Problem, partition_size: int):
    """(max_logits [S,H,NP], exp_sums [S,H,NP], tmp_output [S,H,NP,D]) float32 views of a workspace."""
    ml, es, tmp = pad.paged_attention_decode_workspace_layout(p.num_seqs, p.num_heads, p.head_size,
                                                              p.max_blocks_per_seq, p.block_size, partition_size)
    NP = -(-p.max_blocks_per_seq * p.block_size // partition_size)
    S, H, D = p.num_seqs, p.num_heads, p.head_size
    n = S * H * NP
    f = lambda off, count: ws[off: off + 4 * count].view(torch.float32)
    return (f(ml, n).view(S, H, NP), f(es, n).view(S, H, NP), f(tmp, n * D).view(S, H, NP, D))


def device_cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def entry_plan(p: gen.Problem, partition_size: int, lens=None, layout: str = "tiled"):
    """(balanced, count [S, H], begin [S, H, NP], end [S, H, NP]): which tokens
    each phase-1 entry slot holds, from the library's host-side plan for a
    cache in `layout`."""
    lens = p.seq_lens if lens is None else lens
    return pad.paged_attention_decode_entry_ranges(lens, p.num_heads, p.num_kv_heads, p.max_blocks_per_seq,
                                                   p.block_size, partition_size, device_cus(), layout,
                                                   p.head_size, p.dtype)


def phase1_entries(ws: torch.Tensor, p: gen.Problem, partition_size: int, s: int, h: int, plan=None,
                   layout: str = "tiled"):
    """Phase-1 results of (sequence s, head h) as [(token lo, token hi, max, exp-sum, row)],
    max in natural-log units, in slot order (the plan of a cache in `layout`)."""
    _, cnt, lo, hi = plan if plan is not None else entry_plan(p, partition_size, layout=layout)
    ml, es, tmp = workspace_views(ws, p, partition_size)
    n = int(cnt[s, h])
    m = ml[s, h, :n].cpu().numpy().astype(np.float64)
    l = es[s, h, :n].cpu().numpy().astype(np.float64)
    o = tmp[s, h, :n].cpu().numpy().astype(np.float64)
    return [(int(lo[s, h, e]), int(hi[s, h, e]), m[e], l[e], o[e]) for e in range(n)]


def check_phase1_entries(entries, q, K, V, scale, tol_m=1e-4, tol_l=1e-4, tol_o=2e-3):
    """Each phase-1 entry against the oracle's Phase 1 over the same tokens
    (an empty token range must hold max -inf and exp-sum 0)."""
    for lo, hi, m, l, o in entries:
        if hi <= lo:
            assert m == -np.inf and l == 0.0, (lo, hi, m, l)
            continue
        om, ol, oo = oracle.partition_stats(q, K[lo:hi], V[lo:hi], scale, hi - lo)
        assert abs(m - om[0]) < tol_m, (lo, hi, m, om[0])
        assert abs(l / ol[0] - 1) < tol_l, (lo, hi, l, ol[0])
        assert np.max(np.abs(o - oo[0])) < tol_o, (lo, hi)
