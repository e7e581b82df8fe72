"""HIP path vs the fp64 oracle, through the C boundary, on an MI355X.

Small batches are compared element by element (several tiles, ragged tails,
every flag, both strategies forced); the five named workloads at full size are
compared on sampled rows the oracle computes one by one, in the launch
configuration the benchmark times.  The bar is max-abs <= 2e-2 and relative
RMS <= 5e-3 against the oracle, and bitwise agreement where the result must
not depend on physical placement or on the run."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import LSE_TOL, compare, compare_rows, full_rows, run_hip, say
from varlen_attention_serving_amd import binding as B
from varlen_attention_serving_amd import device as D
from varlen_attention_serving_amd import workloads as W

pytestmark = pytest.mark.gpu

FORCE = {"auto": 0, "2d": B.UA_FLAG_FORCE_2D, "3d": B.UA_FLAG_FORCE_3D,
         "3d_seg": B.UA_FLAG_FORCE_3D}
SEG_TILES = {"3d_seg": 2}  # a segment override selects the segmented split


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _full_check(w, force="auto", what=None):
    what = what or f"{w.name}/{force}"
    say(f"[gpu] {what}: T_q={w.total_q} H={w.num_q_heads}/{w.num_kv_heads} d={w.head_dim} "
        f"b={w.block_size}")
    o, plan = run_hip(w, FORCE[force], split_segment_tiles=SEG_TILES.get(force, 0))
    say(f"  plan path={plan.path} split={plan.class_split} stream_k={plan.stream_k} waves={plan.waves} "
        f"tile_n={plan.tile_n} segments={plan.num_segments} tps={plan.tiles_per_segment} "
        f"grid={list(plan.grid)}")
    if force == "2d":
        assert plan.path == 2
    if force in ("3d", "3d_seg"):
        assert plan.path == 3
    if force == "3d_seg":
        assert plan.stream_k == 0
    compare(o, oracle.attention(w), what)
    return o, plan


@pytest.mark.parametrize("force", ["auto", "2d", "3d"])
def test_tiny_varlen(force):
    _full_check(W.tiny_varlen(), force)


SMALL_CASES = [
    ("plain", dict()),
    ("noncausal", dict(causal=False)),
    ("softcap", dict(softcap=3.0)),
    ("alibi", dict(use_alibi=True)),
    ("window", dict(window=37)),
    ("window_noncausal", dict(window=29, causal=False)),
    # the narrowest window: a causal row sees its own key only; a non-causal
    # row sees its own key and every later one
    ("window1", dict(window=1)),
    ("window1_noncausal_sinks", dict(window=1, causal=False, use_sinks=True)),
    ("sinks", dict(use_sinks=True)),
    ("all_flags", dict(softcap=5.0, use_alibi=True, window=45, use_sinks=True)),
    ("f16", dict(q_dtype=W.DT_F16, kv_dtype=W.DT_F16)),
    ("fp8_bf16q", dict(kv_dtype=W.DT_FP8_E4M3)),
    ("fp8_f16q_all", dict(q_dtype=W.DT_F16, kv_dtype=W.DT_FP8_E4M3, use_alibi=True,
                          use_sinks=True, window=50, softcap=20.0)),
]
SHAPES = [
    # (H_q, H_k, d, b): GQA groups 1, 2, 4, 8, 16; head dims 64/128/256; blocks 8..64
    (4, 2, 64, 16),
    (8, 2, 128, 32),
    (16, 2, 256, 64),
    (32, 2, 128, 16),
    (6, 6, 64, 8),
]


@pytest.mark.parametrize("force", ["auto", "2d", "3d", "3d_seg"])
@pytest.mark.parametrize("shape", range(len(SHAPES)))
@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_small_batches(case, shape, force):
    name, flags = SMALL_CASES[case]
    hq, hk, d, b = SHAPES[shape]
    w = W.random_small(1000 + 17 * case + shape, num_seqs=5, max_q=70, max_k=300,
                       num_q_heads=hq, num_kv_heads=hk, head_dim=d, block_size=b, **flags)
    _full_check(w, force, f"{name}/{SHAPES[shape]}/{force}")


@pytest.mark.parametrize("force", ["auto", "2d", "3d", "3d_seg"])
def test_decode_only_batch(force):
    """Single-query rows, S_k from 1 up to several tiles (the decode geometry)."""
    rng = np.random.default_rng(7)
    sk = np.concatenate([[1, 2, 31, 32, 33, 64, 65], rng.integers(1, 700, size=20)])
    w = W.build("decode_small", 7, np.ones(sk.size), sk, num_q_heads=32, num_kv_heads=8,
                head_dim=128, block_size=16, rng=rng)
    _full_check(w, force)


@pytest.mark.parametrize("hk", [1, 2, 8])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_stream_k_ragged_decode(seed, hk):
    """Decode-shaped batches with lengths from 1 to many tiles, empty
    sequences in between and short multi-row chunks: the stream-K workers'
    ranges start and end inside pairs, cross several pairs, or are empty."""
    rng = np.random.default_rng(300 + seed)
    n = [3, 40, 150][seed]
    sk = rng.integers(1, [70, 3000, 1200][seed], size=n, endpoint=True)
    ql = np.minimum(sk, rng.integers(0, 3, size=n, endpoint=True))  # 0..3 rows
    w = W.build(f"sk_{seed}_{hk}", 300 + seed, ql, sk, num_q_heads=4 * hk, num_kv_heads=hk,
                head_dim=128, block_size=16, rng=rng, use_sinks=seed == 1,
                use_alibi=seed == 2, softcap=30.0 if seed == 2 else 0.0)
    _, plan = _full_check(w, "3d")
    assert plan.stream_k == 1


SK_HEAD_GROUPS = [
    # (H_k, g, d, kv dtype): workers take the largest of 8, 4, 2, 1 kv heads
    # dividing H_k (1 for 3, 2 for 6, 4 for 12, 8 for 16 and 32)
    (3, 4, 128, W.DT_BF16), (6, 2, 128, W.DT_BF16), (12, 2, 64, W.DT_BF16),
    (16, 2, 128, W.DT_FP8_E4M3), (32, 1, 64, W.DT_BF16), (6, 4, 256, W.DT_BF16),
    (12, 2, 256, W.DT_FP8_E4M3), (4, 8, 256, W.DT_BF16),
]


@pytest.mark.parametrize("i", range(len(SK_HEAD_GROUPS)))
def test_stream_k_head_groups(i):
    """Stream-K workers of several waves, one kv head each, over every group
    size the launch can pick (and the single-head fallback for odd H_k), on
    both engines, ragged lengths with empty sequences."""
    hk, g, d, kv = SK_HEAD_GROUPS[i]
    rng = np.random.default_rng(500 + i)
    n = 25
    sk = rng.integers(1, 1500, size=n, endpoint=True)
    sk[::7] = 0
    ql = np.minimum(sk, 1)
    w = W.build(f"skg_{hk}_{g}_{d}", 500 + i, ql, sk, num_q_heads=g * hk, num_kv_heads=hk,
                head_dim=d, block_size=16, kv_dtype=kv, rng=rng, use_sinks=i % 2 == 1)
    _, plan = _full_check(w, "auto")
    assert plan.stream_k == 1


DECODE16 = [
    # (H_q, H_k, kv dtype, flags): d = 256 decode-shaped batches on the 16-row engine
    (4, 4, W.DT_BF16, dict()),
    (16, 4, W.DT_BF16, dict(use_sinks=True, window=700)),
    (16, 2, W.DT_FP8_E4M3, dict(use_alibi=True, use_sinks=True, window=2048, q_dtype=W.DT_F16)),
    (16, 1, W.DT_FP8_E4M3, dict(softcap=30.0)),
]


@pytest.mark.parametrize("i", range(len(DECODE16)))
def test_decode16_ragged(i):
    """d = 256 decode rows (and short chunks that still fit 16 rows) on the
    16-row stream-K engine: lengths from 1 to many tiles, empty sequences."""
    hq, hk, kv, flags = DECODE16[i]
    g = hq // hk
    rng = np.random.default_rng(600 + i)
    n = 40
    sk = rng.integers(1, 2500, size=n, endpoint=True)
    ql = np.minimum(sk, rng.integers(0, max(16 // g, 1), size=n, endpoint=True))
    w = W.build(f"decode16_{i}", 600 + i, ql, sk, num_q_heads=hq, num_kv_heads=hk, head_dim=256,
                block_size=32, rng=rng, kv_dtype=kv, **flags)
    _, plan = _full_check(w, "auto")
    assert plan.stream_k == 1 and plan.block_m == 16


MIXED = [
    # (name, flags, shape, class split expected)
    ("plain", dict(), (32, 8, 128, 16), 0),
    ("window_softcap", dict(window=300, softcap=30.0), (32, 8, 128, 32), 0),
    ("fp8_alibi_sinks_window", dict(q_dtype=W.DT_F16, kv_dtype=W.DT_FP8_E4M3, use_alibi=True,
                                    use_sinks=True, window=200), (16, 2, 256, 64), 1),
    ("d64_g2", dict(use_sinks=True), (8, 4, 64, 16), 0),
    ("fp8_d128_softcap", dict(kv_dtype=W.DT_FP8_E4M3, softcap=20.0), (32, 8, 128, 16), 1),
    ("bf16_d256_window", dict(window=150, use_sinks=True), (16, 4, 256, 32), 1),
    ("fp8_d64_g4", dict(kv_dtype=W.DT_FP8_E4M3), (16, 4, 64, 16), 1),
    # blocks of 2 keys are below one ring copy's 4 rows: register path, split
    ("bf16_d128_b2", dict(use_sinks=True), (16, 4, 128, 2), 1),
    ("bf16_d256_softcap", dict(softcap=25.0), (16, 8, 256, 16), 1),
]


@pytest.mark.parametrize("i", range(len(MIXED)))
def test_mixed_decode_and_chunks(i):
    """Decode rows and multi-row chunks in one batch.  On the register-staged
    wide path the decode-shaped sequences run in the concurrent stream-K
    launch and the rest in the wide launch (class split); on the LDS ring the
    batch stays one launch."""
    name, flags, (hq, hk, d, b), want_split = MIXED[i]
    rng = np.random.default_rng(400 + i)
    n_dec, n_chunk = 9, 3
    dec_k = rng.integers(1, 900, size=n_dec, endpoint=True)
    ctx = rng.integers(0, 600, size=n_chunk, endpoint=True)
    ch_q = rng.integers(40, 200, size=n_chunk, endpoint=True)
    q_lens = np.concatenate([np.ones(n_dec, np.int64), ch_q])
    sk = np.concatenate([dec_k, ctx + ch_q])
    order = rng.permutation(q_lens.size)
    w = W.build(f"mixed_{name}", 400 + i, q_lens[order], sk[order], num_q_heads=hq,
                num_kv_heads=hk, head_dim=d, block_size=b, rng=rng, **flags)
    _, plan = _full_check(w, "auto")
    assert plan.class_split == want_split


D256_RING_FLAGS = [dict(use_sinks=True, window=400),
                   dict(use_alibi=True, use_sinks=True),
                   dict(softcap=15.0, window=300),
                   dict(softcap=30.0, use_alibi=True)]


@pytest.mark.parametrize("i", range(len(D256_RING_FLAGS)))
def test_d256_ring_batch_in_one_launch(i):
    """A d = 256 16-bit batch (with or without softcap and ALiBi) whose full
    grid fills a resident round stays one 2D launch on the two-stage LDS
    ring, decode q-blocks and chunks together."""
    rng = np.random.default_rng(420 + i)
    n_dec = 96
    dec_k = rng.integers(1, 500, size=n_dec, endpoint=True)
    ch_q = rng.integers(40, 120, size=4, endpoint=True)
    ctx = rng.integers(0, 300, size=4, endpoint=True)
    q_lens = np.concatenate([np.ones(n_dec, np.int64), ch_q])
    order = rng.permutation(q_lens.size)
    w = W.build(f"d256_ring_mixed{i}", 420 + i, q_lens[order], np.concatenate([dec_k, ctx + ch_q])[order],
                num_q_heads=16, num_kv_heads=8, head_dim=256, block_size=16, rng=rng,
                **D256_RING_FLAGS[i])
    _, plan = _full_check(w, "auto")
    assert plan.path == 2 and plan.class_split == 0


D256_RING_XF = [
    # (name, shape (H_q, H_k, d, b), flags, force)
    ("2d_alibi", (16, 4, 256, 16), dict(use_alibi=True), "2d"),
    ("2d_softcap_f16_b64", (16, 4, 256, 64), dict(softcap=20.0, q_dtype=W.DT_F16, kv_dtype=W.DT_F16), "2d"),
    ("2d_softcap_alibi_b2", (8, 2, 256, 2), dict(softcap=5.0, use_alibi=True, use_sinks=True), "2d"),
    ("seg_softcap_alibi_noncausal", (16, 2, 256, 32), dict(softcap=30.0, use_alibi=True, causal=False),
     "3d_seg"),
    ("seg_alibi_window_sinks", (8, 2, 256, 16), dict(use_alibi=True, window=90, use_sinks=True), "3d_seg"),
]


@pytest.mark.parametrize("i", range(len(D256_RING_XF)))
def test_d256_ring_score_transforms(i):
    """The two-stage d = 256 ring with softcap and ALiBi, in one launch and
    on the segmented split: full tiles, the diagonal's masked tiles and each
    sequence's partial last tile (ragged lengths), blocks from the smallest
    the ring takes (2 keys) to 64."""
    name, (hq, hk, d, b), flags, force = D256_RING_XF[i]
    w = W.random_small(980 + i, num_seqs=5, max_q=150, max_k=420, num_q_heads=hq,
                       num_kv_heads=hk, head_dim=d, block_size=b, **flags)
    _full_check(w, force, f"d256_ring/{name}/{force}")


FP8_D256_WIDE = [
    # (name, shape (H_q, H_k, d, b), flags, force): four-wave fp8 d = 256 tiles
    ("2d_b4_alibi_sinks", (16, 2, 256, 4), dict(use_alibi=True, use_sinks=True), "2d"),
    ("2d_b2_registers", (16, 2, 256, 2), dict(softcap=10.0), "2d"),
    ("seg_b16_window_noncausal", (8, 2, 256, 16), dict(window=70, causal=False), "3d_seg"),
    ("seg_b64_bf16q_softcap", (16, 4, 256, 64), dict(softcap=25.0, q_dtype=W.DT_BF16), "3d_seg"),
    ("2d_b8_qq", (8, 2, 256, 8), dict(use_qq_bias=True), "2d"),
]


@pytest.mark.parametrize("i", range(len(FP8_D256_WIDE)))
def test_fp8_d256_wide_tiles(i):
    """fp8 K/V at d = 256 in four-wave q-blocks without a concurrent
    stream-K launch (the register-staged gather converting each tile to the
    Q type in LDS): the 2D path and the segmented split, every score
    transform, blocks of 2 to 64 keys, ragged last tiles."""
    name, (hq, hk, d, b), flags, force = FP8_D256_WIDE[i]
    kw = dict(q_dtype=W.DT_F16, kv_dtype=W.DT_FP8_E4M3)
    kw.update(flags)
    w = W.random_small(1000 + i, num_seqs=5, max_q=150, max_k=420, num_q_heads=hq,
                       num_kv_heads=hk, head_dim=d, block_size=b, **kw)
    _, plan = _full_check(w, force, f"fp8_d256_wide/{name}/{force}")
    assert plan.class_split == 0


@pytest.mark.parametrize("d,b", [(64, 1), (64, 4), (128, 2), (128, 4), (64, 8)])
def test_small_block_sizes(d, b):
    """Blocks smaller than the key rows one wave-wide LDS copy fills keep the
    register-staged gather; the rest take the LDS ring."""
    w = W.random_small(500 + d + b, num_seqs=4, max_q=60, max_k=200, num_q_heads=8,
                       num_kv_heads=2, head_dim=d, block_size=b, use_sinks=True)
    for force in ("2d", "3d"):
        _full_check(w, force, f"b={b}/d={d}/{force}")


@pytest.mark.parametrize("d,b,kv", [(64, 1024, W.DT_BF16), (128, 256, W.DT_BF16),
                                     (128, 512, W.DT_FP8_E4M3), (256, 128, W.DT_FP8_E4M3)])
def test_large_block_sizes(d, b, kv):
    """Blocks up to the largest size the descriptor accepts (1024 keys): a
    sequence spans one or two blocks and a tile lies inside one block."""
    w = W.random_small(540 + d + b, num_seqs=5, max_q=80, max_k=1500, num_q_heads=8,
                       num_kv_heads=2, head_dim=d, block_size=b, kv_dtype=kv, use_sinks=True)
    for force in ("2d", "3d"):
        _full_check(w, force, f"b={b}/d={d}/{force}")


MANY_SEQS = [
    # (sequences, H_k, d, kv dtype, force)
    (700, 2, 128, W.DT_BF16, "3d"),
    (700, 2, 128, W.DT_BF16, "2d"),
    (1500, 1, 64, W.DT_BF16, "3d"),
    (600, 2, 256, W.DT_FP8_E4M3, "3d"),
]


@pytest.mark.parametrize("i", range(len(MANY_SEQS)))
def test_many_sequences(i):
    """Batches of hundreds to thousands of short sequences (some empty, some of
    two rows): the stream-K workers' and the reduce's sequence scans take
    several rounds of 256 sequences, and the 2D grid maps many q-blocks."""
    n, hk, d, kv, force = MANY_SEQS[i]
    rng = np.random.default_rng(700 + i)
    sk = rng.integers(0, 300, size=n, endpoint=True)
    ql = np.minimum(sk, rng.integers(0, 2, size=n, endpoint=True))
    w = W.build(f"many_{n}_{d}", 700 + i, ql, sk, num_q_heads=4 * hk, num_kv_heads=hk,
                head_dim=d, block_size=16, kv_dtype=kv, rng=rng, use_sinks=i % 2 == 0)
    _, plan = _full_check(w, force, f"n={n}/d={d}/{force}")
    if force == "3d":
        assert plan.stream_k == 1


QQ_CASES = [
    # (name, shape (H_q, H_k, d, b), flags, force)
    ("2d_ring", (8, 2, 128, 16), dict(), "2d"),
    ("seg_ring_noncausal_alibi", (8, 2, 64, 16), dict(causal=False, use_alibi=True), "3d_seg"),
    ("2d_registers_fp8_sinks", (8, 2, 128, 32), dict(kv_dtype=W.DT_FP8_E4M3, use_sinks=True), "2d"),
    ("d256_softcap_window", (16, 4, 256, 32), dict(softcap=20.0, window=40), "auto"),
    ("stream_k_chunks", (32, 8, 128, 16), dict(use_sinks=True), "3d"),
]


@pytest.mark.parametrize("i", range(len(QQ_CASES)))
def test_qq_bias(i):
    """QQ-bias on the query section ([UA] section 1, step 4) on the 2D ring and
    register kernels, the segmented split, d = 256 and stream-K (short
    chunks)."""
    name, (hq, hk, d, b), flags, force = QQ_CASES[i]
    max_q = 3 if force == "3d" and name.startswith("stream_k") else 60
    w = W.random_small(950 + i, num_seqs=5, max_q=max_q, max_k=260, num_q_heads=hq,
                       num_kv_heads=hk, head_dim=d, block_size=b, use_qq_bias=True, **flags)
    _full_check(w, force, f"qq/{name}/{force}")


QQ_D256_CASES = [
    # (name, q dtype, kv dtype, force, stream-K expected)
    ("bf16_auto", W.DT_BF16, W.DT_BF16, "auto", 0),
    ("bf16_forced_3d", W.DT_BF16, W.DT_BF16, "3d", 0),
    ("f16_forced_3d", W.DT_F16, W.DT_F16, "3d", 0),
    ("fp8_forced_3d", W.DT_BF16, W.DT_FP8_E4M3, "3d", 1),
]


@pytest.mark.parametrize("i", range(len(QQ_D256_CASES)))
def test_qq_bias_d256_28_row_blocks(i):
    """QQ-bias at d = 256 on decode-shaped q-blocks of 17-32 rows (short
    chunks of up to 7 positions at g = 4).  With 16-bit K/V the 32-row
    stream-K kernel of this configuration is not built (the compiler dropped
    a register copy of a spilled Q fragment, so every row's scores were
    wrong): the plan takes the segmented split; fp8 K/V keeps the stream-K
    engine."""
    name, qdt, kvdt, force, sk = QQ_D256_CASES[i]
    w = W.build(f"qq_d256_{name}", 970 + i, [7, 3, 7, 1, 5], [438, 300, 1200, 90, 777],
                num_q_heads=16, num_kv_heads=4, head_dim=256, block_size=16, q_dtype=qdt,
                kv_dtype=kvdt, use_qq_bias=True, rng=np.random.default_rng(970 + i))
    _, plan = _full_check(w, force, f"qq_d256/{name}/{force}")
    assert plan.path == 3 and plan.stream_k == sk
    if sk:
        assert plan.block_m == 32


DENSE_CASES = [
    # (name, shape (H_q, H_k, d, paged b), workload flags, force, max_q)
    ("2d_ring", (8, 2, 128, 16), dict(), "2d", 300),
    ("2d_ring_d64_window_alibi", (8, 2, 64, 16), dict(window=50, use_alibi=True), "2d", 90),
    ("seg_ring_softcap_sinks", (8, 2, 128, 16), dict(softcap=20.0, use_sinks=True), "3d_seg", 90),
    ("2d_registers_fp8_qq", (8, 2, 128, 32), dict(kv_dtype=W.DT_FP8_E4M3, use_qq_bias=True),
     "2d", 90),
    ("d256_noncausal", (16, 4, 256, 32), dict(causal=False), "auto", 60),
    ("stream_k_decode", (32, 8, 128, 16), dict(use_sinks=True), "3d", 1),
    ("2d_fp8_d256", (16, 4, 256, 32), dict(q_dtype=W.DT_F16, kv_dtype=W.DT_FP8_E4M3,
                                                  use_alibi=True), "2d", 90),
    ("stream_k_16rows_d256_fp8", (16, 2, 256, 32), dict(kv_dtype=W.DT_FP8_E4M3, window=70),
     "auto", 1),
]


@pytest.mark.parametrize("i", range(len(DENSE_CASES)))
def test_dense_layout(i):
    """K/V packed per sequence and addressed through cu_seqlens_k (the dense
    sibling of [UA] section 8) on every path: the 2D ring and register
    kernels, the segmented split, d = 256 and both stream-K engines.  The
    oracle reads the same rows through the identity table of block size 1;
    the same batch in its paged layout gives bitwise the same output."""
    name, (hq, hk, d, b), flags, force, max_q = DENSE_CASES[i]
    w = W.random_small(960 + i, num_seqs=6, max_q=max_q, max_k=400, num_q_heads=hq,
                       num_kv_heads=hk, head_dim=d, block_size=b, **flags)
    wd = W.to_dense(w)
    o, plan = _full_check(wd, force, f"dense/{name}/{force}")
    paged, plan_p = run_hip(w, FORCE[force], split_segment_tiles=SEG_TILES.get(force, 0))
    assert (plan.path, plan.stream_k, plan.class_split) == \
        (plan_p.path, plan_p.stream_k, plan_p.class_split)
    assert np.array_equal(o, paged)



LSE_CASES = [
    # (name, workload maker, force)
    ("2d_ring", lambda: W.random_small(900, num_seqs=5, max_q=70, max_k=300, num_q_heads=8,
                                       num_kv_heads=2, head_dim=128, block_size=16), "2d"),
    ("seg_ring_sinks_softcap", lambda: W.random_small(901, num_seqs=5, max_q=70, max_k=300,
                                                      num_q_heads=8, num_kv_heads=2, head_dim=64,
                                                      block_size=16, use_sinks=True,
                                                      softcap=8.0), "3d_seg"),
    ("2d_registers_fp8_alibi", lambda: W.random_small(902, num_seqs=4, max_q=50, max_k=260,
                                                      num_q_heads=8, num_kv_heads=2, head_dim=128,
                                                      block_size=16, kv_dtype=W.DT_FP8_E4M3,
                                                      use_alibi=True), "2d"),
    ("stream_k_32rows_window", lambda: W.build(
        "lse_sk32", 903, np.ones(30, np.int64), np.random.default_rng(903).integers(1, 900, 30),
        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, window=200,
        use_sinks=True), "auto"),
    # softcap alone: its tile max is taken over 1 / (1 + e^{2y}) and folded
    # into the exponent; the LSE checks that bookkeeping exactly
    ("2d_ring_softcap_window", lambda: W.random_small(905, num_seqs=5, max_q=90, max_k=400,
                                                      num_q_heads=16, num_kv_heads=4,
                                                      head_dim=128, block_size=32, softcap=12.0,
                                                      window=150), "2d"),
    ("stream_k_32rows_softcap_sinks", lambda: W.build(
        "lse_sk32_cap", 906, np.ones(30, np.int64), np.random.default_rng(906).integers(1, 1500, 30),
        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, softcap=25.0,
        use_sinks=True), "auto"),
    # the d = 256 ring with softcap and ALiBi, one launch and segmented
    ("2d_ring_d256_softcap_alibi", lambda: W.random_small(907, num_seqs=5, max_q=90, max_k=400,
                                                          num_q_heads=16, num_kv_heads=4,
                                                          head_dim=256, block_size=16, softcap=20.0,
                                                          use_alibi=True, use_sinks=True), "2d"),
    ("seg_ring_d256_alibi", lambda: W.random_small(908, num_seqs=5, max_q=90, max_k=400,
                                                   num_q_heads=8, num_kv_heads=2, head_dim=256,
                                                   block_size=32, use_alibi=True,
                                                   use_sinks=True), "3d_seg"),
    ("stream_k_16rows_fp8_d256", lambda: W.build(
        "lse_sk16", 904, np.ones(30, np.int64), np.random.default_rng(904).integers(1, 900, 30),
        num_q_heads=16, num_kv_heads=2, head_dim=256, block_size=32, kv_dtype=W.DT_FP8_E4M3,
        q_dtype=W.DT_F16, use_sinks=True), "auto"),
]


@pytest.mark.parametrize("i", range(len(LSE_CASES)))
def test_row_lse_matches_oracle(i):
    """The optional row log-sum-exp output on each path (2D ring and register
    kernels, the segmented split, both stream-K engines) against the oracle's
    natural-log LSE, sinks included."""
    name, make, force = LSE_CASES[i]
    w = make()
    o, plan, lse = run_hip(w, FORCE[force], split_segment_tiles=SEG_TILES.get(force, 0), lse=True)
    ref_o, ref_lse = oracle.attention(w, return_lse=True)
    compare(o, ref_o, f"lse/{name} O")
    both_inf = np.isinf(lse) & np.isinf(ref_lse) & (np.sign(lse) == np.sign(ref_lse))
    err = np.where(both_inf, 0.0, np.abs(lse - ref_lse))
    say(f"  lse/{name}: path={plan.path} stream_k={plan.stream_k} max_abs={float(np.max(err)):.3e}")
    assert not np.isnan(lse).any()
    assert float(np.max(err)) <= LSE_TOL


@pytest.mark.parametrize("force", ["auto", "2d", "3d"])
def test_prefill_ragged(force):
    """Self-attention prefill with lengths that are not tile multiples."""
    lens = [1, 63, 64, 65, 127, 200]
    w = W.build("prefill_ragged", 8, lens, lens, num_q_heads=16, num_kv_heads=2, head_dim=128,
                block_size=32)
    _full_check(w, force)


def test_empty_and_zero_length_sequences():
    """Sequences with q_len 0 own no q-block; the others are unaffected."""
    w = W.build("with_empty", 9, [0, 3, 0, 1, 5], [10, 40, 7, 1, 90], num_q_heads=8,
                num_kv_heads=4, head_dim=64, block_size=16)
    _full_check(w)


def test_empty_batch_is_a_no_op():
    w = W.tiny_varlen()
    batch = D.DeviceBatch(w)
    ua = D.UnifiedAttention(D.problem_desc(w))
    args = batch.run_args(ua.workspace)
    args.num_seqs = 0
    args.total_q = 0
    args.max_seqlen_q = 0
    B.ua_run(ua.handle, args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.count_nonzero(batch.o).item() == 0


def test_block_table_permutation_is_bitwise_invariant():
    w = W.random_small(44, num_seqs=4, max_q=40, max_k=400, num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16)
    for force in ("2d", "3d"):
        base, _ = run_hip(w, FORCE[force])
        rng = np.random.default_rng(5)
        perm = rng.permutation(w.num_blocks)
        w2 = W.Workload(**{**w.__dict__})
        w2.k_cache = np.empty_like(w.k_cache)
        w2.v_cache = np.empty_like(w.v_cache)
        w2.k_cache[perm] = w.k_cache
        w2.v_cache[perm] = w.v_cache
        w2.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)],
                                  -1).astype(np.int32)
        moved, _ = run_hip(w2, FORCE[force])
        say(f"[gpu] permutation invariance ({force})")
        assert np.array_equal(base, moved)


BIG_POOL_CASES = [
    # (name, H_q, H_k, d, kv dtype, q lengths): blocks placed past 2^31 bytes
    ("ring_prefill", 8, 8, 128, W.DT_BF16, (40, 70, 1, 3)),
    ("stream_k_decode", 32, 8, 128, W.DT_BF16, (1, 1, 1, 1, 1)),
    ("registers_fp8", 8, 8, 128, W.DT_FP8_E4M3, (40, 70, 1, 3)),
    ("decode16_d256", 16, 4, 256, W.DT_BF16, (1, 1, 2)),
]


@pytest.mark.parametrize("i", range(len(BIG_POOL_CASES)))
def test_blocks_beyond_2gib_of_pool(i):
    """[UA] section 7.2: pools above 2^31 bytes need 64-bit addresses.  The
    batch's blocks are moved to physical ids whose byte offsets lie past
    2^31 (and past 2^32 for the last ones) in a pool of that size; the output
    must equal the compact pool's bit for bit."""
    name, hq, hk, d, kv, ql = BIG_POOL_CASES[i]
    rng = np.random.default_rng(600 + i)
    ql = np.asarray(ql)
    sk = ql + rng.integers(0, 400, size=ql.size)
    w = W.build(f"big_{name}", 600 + i, ql, sk, num_q_heads=hq, num_kv_heads=hk, head_dim=d,
                block_size=16, kv_dtype=kv, rng=rng)
    small, plan = run_hip(w)
    compare(small, oracle.attention(w), f"big pool/{name} (compact)")
    esz = 1 if kv == W.DT_FP8_E4M3 else 2
    block_bytes = 16 * hk * d * esz
    first = (1 << 31) // block_bytes + 7           # the first moved block starts past 2^31
    spread = (1 << 32) // block_bytes - first + 64  # and the ids reach past 2^32
    used = np.unique(w.block_table[w.block_table >= 0])
    new_id = np.full(w.num_blocks, -1, dtype=np.int64)
    new_id[used] = first + np.sort(rng.choice(spread, size=used.size, replace=False))
    pool = int(new_id.max()) + 1
    say(f"[gpu] big pool/{name}: {pool} blocks of {block_bytes} B "
        f"({pool * block_bytes / 2**30:.2f} GiB per cache)")
    batch = D.DeviceBatch(w)
    big_k = torch.empty((pool,) + tuple(batch.k.shape[1:]), dtype=batch.k.dtype, device="cuda")
    big_v = torch.empty_like(big_k)
    idx = torch.from_numpy(new_id[used]).cuda()
    src = torch.from_numpy(used.astype(np.int64)).cuda()
    big_k[idx] = batch.k[src]
    big_v[idx] = batch.v[src]
    table = np.where(w.block_table >= 0, new_id[np.maximum(w.block_table, 0)], -1)
    batch.k, batch.v = big_k, big_v
    batch.block_table = torch.from_numpy(table.astype(np.int32)).cuda()
    desc = D.problem_desc(w)
    desc.num_blocks = pool
    ua = D.UnifiedAttention(desc)
    info = ua.plan(w)
    assert info.use_i64_kv == 1 and (info.path, info.stream_k) == (plan.path, plan.stream_k)
    moved, _ = run_hip(w, batch=batch, ua=ua)
    assert np.array_equal(moved, small)
    del big_k, big_v, batch
    torch.cuda.empty_cache()


def test_run_to_run_determinism():
    w = W.random_small(45, num_seqs=4, max_q=60, max_k=500, num_q_heads=16, num_kv_heads=4,
                       head_dim=128, block_size=32, use_sinks=True)
    for force in ("2d", "3d"):
        a, _ = run_hip(w, FORCE[force])
        b, _ = run_hip(w, FORCE[force])
        assert np.array_equal(a, b)


def test_nan_poison_in_unused_blocks_and_tails_never_reaches_output():
    w = W.random_small(46, num_seqs=6, max_q=30, max_k=250, num_q_heads=8, num_kv_heads=2,
                       head_dim=64, block_size=64)
    assert np.isnan(oracle.attention(w)).sum() == 0
    for force in ("2d", "3d"):
        o, _ = run_hip(w, FORCE[force])
        assert not np.isnan(o).any()


# ---------------------------------------------------------------------------
# GQA groups outside the powers of two, and the widest groups
# ---------------------------------------------------------------------------

GQA_SHAPES = [
    # (H_q, H_k, d, b, workload flags).  Groups that do not divide a q-block's
    # rows leave rows_used < block_m on every geometry (128 / g and 32 / g
    # positions, 16 / g on the 16-row engine); above 32 no single-wave
    # q-block exists and stream-K is off.
    (24, 8, 128, 16, dict()),                                   # g = 3
    (10, 2, 64, 32, dict(use_sinks=True)),                      # g = 5
    (12, 2, 256, 64, dict(q_dtype=W.DT_F16, kv_dtype=W.DT_FP8_E4M3, use_alibi=True,
                          use_sinks=True, window=300)),          # g = 6, class split
    (28, 4, 128, 16, dict(softcap=30.0)),                       # g = 7
    (24, 2, 256, 32, dict(window=200, use_sinks=True)),         # g = 12, 16-row engine
    (48, 2, 128, 16, dict(kv_dtype=W.DT_FP8_E4M3)),             # g = 24, class split
    (64, 2, 64, 16, dict(use_alibi=True)),                      # g = 32
    (64, 1, 128, 16, dict(use_sinks=True)),                     # g = 64
    (128, 1, 128, 64, dict()),                                  # g = 128
    (128, 2, 256, 64, dict(kv_dtype=W.DT_FP8_E4M3, window=250)),  # g = 64, d = 256 fp8
]


def _gqa_batch(i, kind):
    """kind "mixed": decode rows, short chunks that fit a single-wave q-block
    and longer chunks / prefill in one ragged batch; kind "decode": single
    query rows over contexts up to 1500 keys with empty sequences."""
    hq, hk, d, b, flags = GQA_SHAPES[i]
    g = hq // hk
    seed = 1200 + 10 * i + (kind == "decode")
    rng = np.random.default_rng(seed)
    if kind == "decode":
        sk = rng.integers(1, 1500, size=20, endpoint=True)
        sk[::6] = 0
        ql = np.minimum(sk, 1)
    else:
        dec_k = rng.integers(1, 700, size=6, endpoint=True)
        sq = rng.integers(2, max(2, 32 // g), size=3, endpoint=True)
        sh_k = sq + rng.integers(0, 400, size=3, endpoint=True)
        lq = rng.integers(30, 120, size=3, endpoint=True)
        lk = lq + rng.integers(0, 200, size=3, endpoint=True)
        ql = np.concatenate([np.ones(6, np.int64), sq, lq])
        sk = np.concatenate([dec_k, sh_k, lk])
        order = rng.permutation(ql.size)
        ql, sk = ql[order], sk[order]
    return W.build(f"gqa{g}_{kind}", seed, ql, sk, num_q_heads=hq, num_kv_heads=hk,
                   head_dim=d, block_size=b, rng=rng, **flags)


@pytest.mark.parametrize("force", ["auto", "2d", "3d", "3d_seg"])
@pytest.mark.parametrize("i", range(len(GQA_SHAPES)))
def test_gqa_groups_mixed_batch(i, force):
    """[UA] section 0 (g = H_q / H_k) and section 4 (rows are (position, head)
    pairs of one GQA group) for groups 3 to 128: every path against the oracle
    on a batch of decode rows, short chunks and prefill rows."""
    w = _gqa_batch(i, "mixed")
    _, plan = _full_check(w, force, f"gqa g={w.group} d={w.head_dim} mixed/{force}")
    if force == "auto" and w.group in (6, 12, 24):
        assert plan.class_split == 1  # decode rows on stream-K beside the wide launch


@pytest.mark.parametrize("force", ["auto", "3d", "3d_seg"])
@pytest.mark.parametrize("i", range(len(GQA_SHAPES)))
def test_gqa_groups_decode_batch(i, force):
    """The same groups on decode-shaped batches: stream-K on the 32-row engine
    (g <= 32), on the 16-row engine at d = 256 (g <= 16), the segmented split
    and, above g = 32, the four-wave geometry with one or two positions per
    q-block."""
    w = _gqa_batch(i, "decode")
    _, plan = _full_check(w, force, f"gqa g={w.group} d={w.head_dim} decode/{force}")
    if force == "3d":
        assert plan.stream_k == (1 if w.group <= 32 else 0)
        if w.head_dim == 256 and w.group <= 16:
            assert plan.block_m == 16


# ---------------------------------------------------------------------------
# the named workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["decode_batch", "chunked_prefill_mix", "long_prefill",
                                  "variant_mix", "dense_prefill", "mha_prefill",
                                  "d256_prefill", "decode_large"])
def test_named_workload_full_size(name):
    """The benchmark's launch configuration at full size.  O starts as NaN and
    must come back finite everywhere (run_hip); every (token, head) row of the
    decode-shaped sequences and every token of the others (against every kv
    head the oracle budget allows, the query head rotating through the group)
    is compared with the oracle."""
    say(f"[gpu] {name}: generating")
    w = W.NAMED[name]()
    batch = D.DeviceBatch(w)
    ua = D.UnifiedAttention(D.problem_desc(w))
    o, plan = run_hip(w, batch=batch, ua=ua)
    say(f"  plan path={plan.path} split={plan.class_split} stream_k={plan.stream_k} "
        f"waves={plan.waves} tile_n={plan.tile_n} segments={plan.num_segments} "
        f"tps={plan.tiles_per_segment} grid={list(plan.grid)}")
    rows, m = full_rows(w)
    say(f"  comparing {rows.size} rows ({m} of {w.num_kv_heads} kv heads per prefill token)")
    compare_rows(o, w, rows, f"{name} ({rows.size} rows)")
    # a second run in the same configuration is bitwise identical
    o2, _ = run_hip(w, batch=batch, ua=ua)
    assert np.array_equal(o, o2)
