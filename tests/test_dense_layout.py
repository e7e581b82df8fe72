"""The dense (packed varlen) K/V layout of the dense prefill sibling, on the CPU:
the generator's packed rows are the paged rows of the same keys, the identity
table that lets the oracle read the packed layout addresses row
cu_seqlens_k[s] + k, and the oracle's result does not depend on the layout."""
import numpy as np
import pytest

import oracle
from varlen_attention_serving_amd import workloads as W


@pytest.mark.parametrize("kv", [W.DT_BF16, W.DT_FP8_E4M3])
def test_packed_rows_are_the_paged_rows(kv):
    w = W.random_small(71, num_seqs=5, max_q=30, max_k=150, kv_dtype=kv)
    d = W.to_dense(w)
    assert d.dense and d.block_size == 1
    cu = d.cu_seqlens_k
    assert cu[0] == 0 and np.array_equal(np.diff(cu), w.seq_lens)
    for s in range(w.num_seqs):
        sk = int(w.seq_lens[s])
        key = np.arange(sk)
        phys = w.block_table[s, key // w.block_size]
        slot = key % w.block_size
        assert np.array_equal(d.k_cache[cu[s]:cu[s] + sk, 0], w.k_cache[phys, slot])
        assert np.array_equal(d.v_cache[cu[s]:cu[s] + sk, 0], w.v_cache[phys, slot])
        assert np.array_equal(d.block_table[s, :sk], cu[s] + key)
    # rows past the last sequence hold NaN, so a stray read would show
    assert np.all(d.k_cache[cu[-1]:].view(np.uint8).any(axis=-1))


def test_oracle_is_layout_independent():
    w = W.random_small(72, num_seqs=4, max_q=40, max_k=120, num_q_heads=4, num_kv_heads=2,
                       use_alibi=True, softcap=10.0)
    assert np.array_equal(oracle.attention(W.to_dense(w)), oracle.attention(w))


def test_generator_dense_layout_is_contiguous_per_sequence():
    w = W.build("dense", 73, [3, 7, 0, 5], [10, 7, 4, 30], num_q_heads=4, num_kv_heads=2,
                head_dim=64, block_size=1, dense=True)
    cu = w.cu_seqlens_k
    for s in range(w.num_seqs):
        sk = int(w.seq_lens[s])
        assert np.array_equal(w.block_table[s, :sk], cu[s] + np.arange(sk))
    with pytest.raises(ValueError):
        W.build("dense", 73, [1], [4], num_q_heads=4, num_kv_heads=2, head_dim=64,
                block_size=16, dense=True)
