"""The CPU oracle against its pins, and the pins against planted mistakes."""

import numpy as np
import pytest

import oracle.attention as orc
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(orc)


# Plausible mistakes, each planted in one step of the oracle.  Every one must be
# rejected by at least one pin; otherwise the pins would not protect the oracle.
def _mut_gqa_modulo(h, H, Hkv):
    return h % Hkv


def _mut_gqa_wrong_divisor(h, H, Hkv):
    return min(h // Hkv, Hkv - 1)


def _mut_no_scale(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    x = K @ q
    w = np.exp(x - x.max())
    return (w @ V) / w.sum()


def _mut_sign(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    x = scale * (K @ q)
    w = np.exp(x.min() - x)
    return (w @ V) / w.sum()


def _mut_no_max_subtraction(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    w = np.exp(scale * (K @ q))
    return (w @ V) / w.sum()


def _mut_divide_by_len(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    x = scale * (K @ q)
    w = np.exp(x - x.max())
    return (w @ V) / len(w)


def _mut_keys_as_values(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    x = scale * (K @ q)
    w = np.exp(x - x.max())
    return (w @ K) / w.sum()


def _mut_ignore_table(cache, table_row, seq_len, block_size):
    nb = -(-seq_len // block_size)
    ids = np.arange(nb)
    rows = cache[ids].transpose(1, 0, 2, 3).reshape(cache.shape[1], nb * block_size, cache.shape[3])
    return rows[:, :seq_len]


def _mut_no_transpose(cache, table_row, seq_len, block_size):
    nb = -(-seq_len // block_size)
    blocks = cache[np.asarray(table_row[:nb], dtype=np.int64)]
    rows = blocks.reshape(cache.shape[1], nb * block_size, cache.shape[3])
    return rows[:, :seq_len]


def _mut_one_extra_token(cache, table_row, seq_len, block_size):
    return orc_gather(cache, table_row, seq_len + 1 if seq_len % block_size else seq_len, block_size)


def _mut_one_token_short(cache, table_row, seq_len, block_size):
    return orc_gather(cache, table_row, max(seq_len - 1, 0), block_size)


def _mut_merge_no_expsum(m, l, o):
    if m.shape[0] == 0:
        return np.zeros(o.shape[1])
    r = np.exp(m - m.max())
    return (r / r.sum()) @ o


def _mut_merge_sign(m, l, o):
    if m.shape[0] == 0:
        return np.zeros(o.shape[1])
    r = np.exp(m.max() - m) * l
    return (r / r.sum()) @ o


def _mut_partition_unnormalised(q, K, V, scale, P):
    m, l, o = orc_partition_stats(q, K, V, scale, P)
    return m, l, o * l[:, None]


def _mut_widen_shift(values, dtype):
    if dtype == "bf16":
        bits = np.asarray(values, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return orc_widen(values, dtype)


def _mut_logical_kv_swapped(q_row, K_rows, V_rows, scale, dtype):
    return orc_attend(orc_widen(q_row, dtype), orc_widen(V_rows, dtype), orc_widen(K_rows, dtype),
                      float(np.float32(scale)))


def _mut_logical_scale_unrounded(q_row, K_rows, V_rows, scale, dtype):
    return orc_attend(orc_widen(q_row, dtype), orc_widen(K_rows, dtype), orc_widen(V_rows, dtype), float(scale))


def _mut_logical_one_token_short(q_row, K_rows, V_rows, scale, dtype):
    n = max(K_rows.shape[0] - 1, 1)
    return orc_attend(orc_widen(q_row, dtype), orc_widen(K_rows[:n], dtype), orc_widen(V_rows[:n], dtype),
                      float(np.float32(scale)))


orc_attend = orc.attend
orc_gather = orc.gather_sequence
orc_partition_stats = orc.partition_stats
orc_widen = orc.widen

MUTANTS = [
    ("kv_head_for", _mut_gqa_modulo),
    ("kv_head_for", _mut_gqa_wrong_divisor),
    ("attend", _mut_no_scale),
    ("attend", _mut_sign),
    ("attend", _mut_no_max_subtraction),
    ("attend", _mut_divide_by_len),
    ("attend", _mut_keys_as_values),
    ("gather_sequence", _mut_ignore_table),
    ("gather_sequence", _mut_no_transpose),
    ("gather_sequence", _mut_one_extra_token),
    ("gather_sequence", _mut_one_token_short),
    ("merge_partitions", _mut_merge_no_expsum),
    ("merge_partitions", _mut_merge_sign),
    ("partition_stats", _mut_partition_unnormalised),
    ("widen", _mut_widen_shift),
    ("attend_logical", _mut_logical_kv_swapped),
    ("attend_logical", _mut_logical_scale_unrounded),
    ("attend_logical", _mut_logical_one_token_short),
]


def test_pins_accept_oracle():
    assert pins.failing_pins(orc) == []


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f.__name__ for _, f in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(orc, name, fn)
    assert pins.failing_pins(orc), f"no pin rejects the planted mistake {fn.__name__} in {name}"
