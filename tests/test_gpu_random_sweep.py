"""Seeded random configurations through the C boundary against the fp64 oracle.

Each case draws its own head dim, GQA group (powers of two and not), block
size, Q and K/V types, flag set (causal, softcap, ALiBi, window, sinks,
query-section bias), K/V layout (paged or dense), length mix (decode rows,
short multi-row sequences, chunks with context, an occasional empty
sequence) and path (the plan's own choice, or 2D, 3D, or the segmented split
forced), so that combinations the hand-written cases do not name are
compared element by element too.  The draws are fixed by the case index."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, compare_rows, full_rows, run_hip, say
from varlen_attention_serving_amd import binding as B
from varlen_attention_serving_amd import workloads as W

pytestmark = pytest.mark.gpu

N_CASES = 256
FORCES = ("auto", "auto", "2d", "3d", "3d_seg")
FLAG = {"auto": 0, "2d": B.UA_FLAG_FORCE_2D, "3d": B.UA_FLAG_FORCE_3D,
        "3d_seg": B.UA_FLAG_FORCE_3D}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def draw(i, medium=False):
    """Workload, forced path and segment override of case i, and a label.
    Medium cases take longer sequences (up to 700 queries over 3000 keys) and
    more decode rows, so chains span many tiles, segments and workers."""
    rng = np.random.default_rng((95_000 if medium else 90_000) + i)
    d = int(rng.choice([64, 128, 256]))
    g = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    hk = int(rng.choice([1, 2, 4]))
    dense = rng.random() < 0.1
    b = 1 if dense else int(rng.choice([8, 16, 32, 64]))
    q_dtype = int(rng.choice([W.DT_BF16, W.DT_F16]))
    kv_dtype = W.DT_FP8_E4M3 if rng.random() < 0.3 else q_dtype
    flags = dict(causal=bool(rng.random() < 0.8),
                 softcap=float(rng.choice([3.0, 20.0])) if rng.random() < 0.3 else 0.0,
                 use_alibi=bool(rng.random() < 0.3),
                 window=int(rng.integers(1, 1500 if medium else 200)) if rng.random() < 0.3 else 0,
                 use_sinks=bool(rng.random() < 0.3),
                 use_qq_bias=bool(rng.random() < 0.1))
    max_ctx_dec, max_q, max_ctx = (3000, 700, 2300) if medium else (400, 91, 300)
    n_dec = int(rng.integers(0, 33 if medium else 9))
    n_long = int(rng.integers(0, 4))
    if n_dec + n_long == 0:
        n_long = 1
    q_lens, seq_lens = [], []
    for _ in range(n_dec):
        ql = int(rng.integers(1, 3))
        q_lens.append(ql)
        seq_lens.append(ql + int(rng.integers(0, max_ctx_dec)))
    for _ in range(n_long):
        ql = int(rng.integers(3, max_q))
        q_lens.append(ql)
        seq_lens.append(ql + int(rng.integers(0, max_ctx)))
    if rng.random() < 0.15:
        pos = int(rng.integers(0, len(q_lens) + 1))
        q_lens.insert(pos, 0)
        seq_lens.insert(pos, int(rng.integers(0, 50)))
    order = rng.permutation(len(q_lens))
    q_lens = np.array(q_lens, np.int64)[order]
    seq_lens = np.array(seq_lens, np.int64)[order]
    force = FORCES[int(rng.integers(0, len(FORCES)))]
    seg = 2 if force == "3d_seg" else 0
    w = W.build(f"{'medium' if medium else 'sweep'}{i}", 90_000 + i, q_lens, seq_lens, num_q_heads=g * hk, num_kv_heads=hk,
                head_dim=d, block_size=16 if dense else b, q_dtype=q_dtype, kv_dtype=kv_dtype,
                rng=rng, **flags)
    if dense:
        w = W.to_dense(w)
    on = [k for k, v in flags.items() if v and k != "causal"]
    label = (f"case {i}: d={d} g={g} H_k={hk} b={w.block_size}{' dense' if dense else ''} "
             f"q={W.DTYPE_NAMES[q_dtype]} kv={W.DTYPE_NAMES[kv_dtype]} "
             f"{'causal' if flags['causal'] else 'noncausal'} {' '.join(on)} "
             f"q_lens={q_lens.tolist()} S_k={seq_lens.tolist()} force={force}")
    return w, force, seg, label


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    w, force, seg, label = draw(i)
    say(f"[gpu] {label}")
    o, plan = run_hip(w, FLAG[force], split_segment_tiles=seg)
    say(f"  plan path={plan.path} split={plan.class_split} stream_k={plan.stream_k} "
        f"waves={plan.waves} block_m={plan.block_m} segments={plan.num_segments}")
    if force == "2d":
        assert plan.path == 2
    if force in ("3d", "3d_seg"):
        assert plan.path == 3
    compare(o, oracle.attention(w), f"sweep {i}")


N_MEDIUM = 64


@pytest.mark.parametrize("i", range(N_MEDIUM))
def test_random_medium_configuration(i):
    """Longer random batches, compared on every decode row and, for the
    longer sequences, on every token with the query head rotating through
    its group (every q-block of every kv head visited)."""
    w, force, seg, label = draw(i, medium=True)
    say(f"[gpu] medium {label}")
    o, plan = run_hip(w, FLAG[force], split_segment_tiles=seg)
    say(f"  plan path={plan.path} split={plan.class_split} stream_k={plan.stream_k} "
        f"waves={plan.waves} block_m={plan.block_m} segments={plan.num_segments}")
    if force == "2d":
        assert plan.path == 2
    if force in ("3d", "3d_seg"):
        assert plan.path == 3
    rows, m = full_rows(w, budget_flops=2e10)
    compare_rows(o, w, rows, f"medium {i} ({rows.size} rows, {m} kv heads per token)")
