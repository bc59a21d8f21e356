"""The seeded input generator: determinism, layout, rounding and poison placement."""

import numpy as np
import pytest
import torch

from decode_attention_paged_05_amd import inputs as gen


def test_same_seed_same_bits():
    a = gen.make_problem("mixed")
    b = gen.make_problem("mixed")
    assert np.array_equal(a.seq_lens, b.seq_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.query, b.query)
    small = dict(seq_lens=[300] * 32)
    ka, va = gen.sequence_kv(gen.make_problem("mixed", **small), 3, 1)
    kb, vb = gen.sequence_kv(gen.make_problem("mixed", **small), 3, 1)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    c = gen.make_problem("mixed", seed=99)
    assert not np.array_equal(a.seq_lens, c.seq_lens)


def test_config_shapes():
    p = gen.make_problem("long")
    assert p.block_tables.shape == (1, 6250)
    assert int(p.seq_lens[0]) == 100000
    assert p.query.shape == (1, 24, 256) and p.query.dtype == np.uint16
    assert p.kv_bytes() == 409_600_000
    t = gen.make_problem("tiny")
    assert t.query.dtype == np.float32 and t.block_tables.shape == (1, 7)
    assert (t.block_tables[0] >= 0).all() and len(set(t.block_tables[0].tolist())) == 7
    assert t.scale == 0.125
    assert gen.make_problem("short").scale == 0.0625


def test_mixed_tables_disjoint_and_lengths_in_range():
    p = gen.make_problem("mixed")
    assert p.seq_lens.min() >= 1 and p.seq_lens.max() <= 32768
    used = []
    for s in range(p.num_seqs):
        nb = -(-int(p.seq_lens[s]) // 16)
        row = p.block_tables[s]
        assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
        used.extend(row[:nb].tolist())
    assert len(used) == len(set(used))
    assert max(used) < p.num_blocks


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]  # ties round to even
    ours = gen.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_outlier_rate_and_placement():
    p = gen.make_problem("stress", seq_lens=[20000] * 8, num_blocks=8 * 1250, max_blocks_per_seq=1250)
    m = gen.outlier_positions(p, 0)
    assert 0.008 < m.mean() < 0.012
    k0, _ = gen.sequence_kv_f32(p, 0, 0)
    k5, _ = gen.sequence_kv_f32(p, 0, 5)
    # outliers are shared by every KV head and scale the whole row
    big = np.abs(k0).max(axis=1) > 8
    assert big[~m].sum() == 0 or big[~m].mean() < 1e-3
    assert np.abs(k5[m]).mean() > 10 * np.abs(k5[~m]).mean()


def test_pool_poison_and_placement():
    p = gen.make_problem("tiny")
    kc, vc = gen.build_pool(p)
    ids = p.block_tables[0]
    unused = sorted(set(range(p.num_blocks)) - set(ids.tolist()))
    assert np.isnan(kc[unused]).all() and np.isnan(vc[unused]).all()
    L = int(p.seq_lens[0])
    last = ids[-1]
    tail = L - 16 * (len(ids) - 1)
    assert np.isnan(kc[last, :, tail:]).all() and not np.isnan(kc[last, :, :tail]).any()
    k, v = gen.sequence_kv(p, 0, 0)
    for j, b in enumerate(ids):
        lo, hi = 16 * j, min(16 * j + 16, L)
        assert np.array_equal(kc[b, 0, : hi - lo], k[lo:hi])
        assert np.array_equal(vc[b, 0, : hi - lo], v[lo:hi])


def test_threads_do_not_change_bits():
    p = gen.make_problem("mixed", seq_lens=[40, 1, 300, 17] + [16] * 28, num_blocks=100,
                         max_blocks_per_seq=19)
    a = gen.build_pool(p, threads=1)
    b = gen.build_pool(p, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bad_lengths_rejected():
    with pytest.raises(ValueError):
        gen.make_problem("tiny", seq_lens=[113])


@pytest.mark.parametrize("dtype,x", [("bf16", 8), ("f32", 4)])
def test_tiled_layout_is_the_documented_permutation(dtype, x):
    rng = np.random.default_rng(3)
    sd = gen.storage_dtype(dtype)
    kb = rng.integers(0, 60000, size=(3, 2, 16, 64)).astype(sd)
    vb = rng.integers(0, 60000, size=(3, 2, 16, 64)).astype(sd)
    kt, vt = gen.to_tiled(kb, vb, dtype)
    assert kt.shape == (3, 2, 64 // x, 16, x) and vt.shape == (3, 2, 64, 16)
    for n, g, t, d in [(0, 0, 0, 0), (2, 1, 15, 63), (1, 0, 7, 9), (2, 1, 3, x)]:
        assert kt[n, g, d // x, t, d % x] == kb[n, g, t, d]
        assert vt[n, g, d, t] == vb[n, g, t, d]
