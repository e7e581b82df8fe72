"""The persistent schedule of the 2D launch (UA_FLAG_PERSISTENT; the two
grids of [UA] section 8.2): resident workgroups draw q-blocks from per-XCD
work queues instead of one workgroup per q-block.  Each q-block is computed
exactly as on the default grid, so the output must be bitwise that of the
default grid, and within the bar against the oracle; problems the schedule
does not apply to keep the default grid."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, run_hip, say
from varlen_attention_serving_amd import binding as B
from varlen_attention_serving_amd import device as D
from varlen_attention_serving_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _prefill(seed, hq, hk, d, b, lens, **kw):
    lens = np.asarray(lens)
    return W.build(f"persist_{seed}", seed, lens, lens, num_q_heads=hq, num_kv_heads=hk,
                   head_dim=d, block_size=b, **kw)


CASES = [
    # (name, workload): LDS-ring 2D launches of four-wave q-blocks
    ("d128_g16_ragged", lambda: _prefill(1, 128, 8, 128, 64, [1100, 300, 7, 513])),
    ("d128_g4_softcap_sinks", lambda: _prefill(2, 32, 8, 128, 32, [900, 64, 65, 1],
                                               softcap=20.0, use_sinks=True)),
    ("d64_alibi_window_h3", lambda: _prefill(3, 12, 3, 64, 16, [700, 250, 33],
                                             use_alibi=True, window=200)),
    ("d256_plain", lambda: _prefill(4, 16, 8, 256, 64, [800, 130, 40])),
    ("d128_qq_bias_noncausal", lambda: _prefill(5, 16, 4, 128, 16, [300, 120],
                                                causal=False, use_qq_bias=True)),
    ("dense_d128", lambda: W.to_dense(_prefill(6, 32, 8, 128, 16, [600, 77]))),
    ("chunks_and_decode", lambda: W.build("persist_mix", 7, np.array([1, 1, 200, 90, 1]),
                                          np.array([400, 30, 700, 90, 900]), num_q_heads=32,
                                          num_kv_heads=8, head_dim=128, block_size=16,
                                          use_sinks=True)),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_persistent_schedule_is_bitwise_the_default_grid(i):
    name, make = CASES[i]
    w = make()
    o_def, plan = run_hip(w, B.UA_FLAG_FORCE_2D)
    o_per, plan_p = run_hip(w, B.UA_FLAG_FORCE_2D | B.UA_FLAG_PERSISTENT)
    say(f"[gpu] persistent {name}: path={plan.path} waves={plan.waves} grid={list(plan.grid)}")
    assert plan.path == 2 and plan_p.path == 2
    compare(o_per, oracle.attention(w), f"persistent {name}")
    assert np.array_equal(o_per, o_def)
    # a second run (the queues are reset by the library each run)
    o2, _ = run_hip(w, B.UA_FLAG_FORCE_2D | B.UA_FLAG_PERSISTENT)
    assert np.array_equal(o2, o_def)


def test_persistent_schedule_without_allocation():
    """The queue counters live in the caller's workspace, or in the
    library's scratch for ua_run_no_alloc."""
    w = CASES[0][1]()
    batch = D.DeviceBatch(w)
    ua = D.UnifiedAttention(D.problem_desc(w, B.UA_FLAG_FORCE_2D | B.UA_FLAG_PERSISTENT))
    assert B.ua_workspace_size(ua.handle) >= 256
    want, _ = run_hip(w, B.UA_FLAG_FORCE_2D)
    batch.o.fill_(0x7FC0)
    B.ua_run_no_alloc(ua.handle, batch.run_args(None), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = batch.output().float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)


def test_persistent_flag_leaves_other_launches_alone():
    """fp8 K/V (register-staged kernel) and decode batches (stream-K) keep
    their own launches under the flag and match the oracle."""
    w = _prefill(8, 16, 4, 128, 16, [300, 40], kv_dtype=W.DT_FP8_E4M3)
    o, _ = run_hip(w, B.UA_FLAG_FORCE_2D | B.UA_FLAG_PERSISTENT)
    compare(o, oracle.attention(w), "persistent flag, fp8 register path")
    rng = np.random.default_rng(9)
    sk = rng.integers(1, 2000, size=20)
    wd = W.build("persist_decode", 9, np.ones(20), sk, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, block_size=16, rng=rng)
    o, plan = run_hip(wd, B.UA_FLAG_PERSISTENT)
    assert plan.stream_k == 1
    compare(o, oracle.attention(wd), "persistent flag, stream-K decode")
