"""ua_run_no_alloc, the entry point for callers that cannot allocate (graph
capture, tight serving loops): the same kernels as ua_run with the split-KV
partials in the library's per-GPU scratch.  Each case runs two calls in a row
through the C boundary, the second on a smaller batch of the same problem,
and checks each against ua_run with a caller workspace (bitwise when the
stream-K worker count is not capped by the scratch) and against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare, poison_output, say
from varlen_attention_serving_amd import binding as B
from varlen_attention_serving_amd import device as D
from varlen_attention_serving_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _decode(seed, n, hq, hk, d, max_k, **kw):
    rng = np.random.default_rng(seed)
    sk = rng.integers(1, max_k, size=n, endpoint=True)
    sk[::9] = 0
    return W.build(f"na_dec_{seed}", seed, np.minimum(sk, 1), sk, num_q_heads=hq, num_kv_heads=hk,
                   head_dim=d, block_size=16, rng=rng, **kw)


def _mixed(seed, n_dec, hq, hk, d, b, max_chunk=150, **kw):
    rng = np.random.default_rng(seed)
    dec_k = rng.integers(1, 900, size=n_dec, endpoint=True)
    ch_q = rng.integers(40, max_chunk, size=3, endpoint=True)
    ctx = rng.integers(0, 500, size=3, endpoint=True)
    ql = np.concatenate([np.ones(n_dec, np.int64), ch_q])
    sk = np.concatenate([dec_k, ctx + ch_q])
    order = rng.permutation(ql.size)
    return W.build(f"na_mix_{seed}", seed, ql[order], sk[order], num_q_heads=hq, num_kv_heads=hk,
                   head_dim=d, block_size=b, rng=rng, **kw)


def _first(w, n):
    """The batch of w's first n sequences over the same pool (same fp8
    scales): a smaller input for the same problem."""
    cu = w.cu_seqlens_q[:n + 1].copy()
    return W.Workload(**{**w.__dict__, "name": f"{w.name}_first{n}", "q_lens": w.q_lens[:n].copy(),
                         "seq_lens": w.seq_lens[:n].copy(), "cu_seqlens_q": cu,
                         "block_table": w.block_table[:n].copy(),
                         "q": w.q[:int(cu[-1])].copy()})


CASES = [
    # (name, big batch, small batch, extra flags, segment tiles, expect bitwise)
    # (name, batch, sequences of the second call, extra flags, segment tiles,
    #  expect bitwise)
    ("stream_k_32rows", lambda: _decode(1, 60, 32, 8, 128, 3000), 13, 0, 0, True),
    ("stream_k_16rows_d256_fp8", lambda: _decode(3, 50, 16, 2, 256, 2500, kv_dtype=W.DT_FP8_E4M3,
                                                 q_dtype=W.DT_F16, use_sinks=True), 7, 0, 0, True),
    ("segmented", lambda: _decode(5, 40, 32, 8, 128, 2000), 9, B.UA_FLAG_FORCE_3D, 4, True),
    ("class_split_serial", lambda: _mixed(7, 30, 16, 2, 256, 64, kv_dtype=W.DT_FP8_E4M3,
                                          use_alibi=True, use_sinks=True, window=300),
     20, 0, 0, True),
    ("two_d_no_scratch", lambda: _mixed(9, 10, 32, 8, 128, 16), 8, B.UA_FLAG_FORCE_2D, 0, True),
    # 900 decode sequences leave the scratch room for about 860 stream-K
    # worker waves: fewer workers than ua_run's, so a different fp32 merge
    # order (tolerance, not bitwise)
    ("stream_k_capped_workers", lambda: _decode(11, 900, 32, 8, 128, 400), 300,
     B.UA_FLAG_FORCE_3D, 0, False),
    # 1100 decode sequences: their stream-K slots (140 MiB) exceed the scratch,
    # so ua_run_no_alloc plans the 2D path where ua_run streams them; the
    # second call's 300 fit (tolerance: different plans)
    ("decode_beyond_scratch_2d", lambda: _decode(13, 1100, 32, 8, 128, 700), 300, 0, 0, False),
]


def _call(ua, batch, no_alloc):
    poison_output(batch)
    stream = torch.cuda.current_stream().cuda_stream
    if no_alloc:
        B.ua_run_no_alloc(ua.handle, batch.run_args(None), stream)
    else:
        B.ua_run(ua.handle, batch.run_args(ua.workspace), stream)
    torch.cuda.synchronize()
    o = batch.output()
    assert bool(torch.isfinite(o).all()), "rows left unwritten"
    return o.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_no_alloc_matches_ua_run_on_two_calls(i):
    name, make, n_small, flags, seg, bitwise = CASES[i]
    big = make()
    small = _first(big, n_small)
    ua = D.UnifiedAttention(D.problem_desc(big, flags, split_segment_tiles=seg))
    assert 0 < small.total_q < big.total_q
    for w in (big, small):  # the second call is the smaller batch
        plan = ua.plan(w)
        say(f"[gpu] no-alloc {name}: {w.name} T_q={w.total_q} path={plan.path} "
            f"stream_k={plan.stream_k} split={plan.class_split}")
        batch = D.DeviceBatch(w)
        want = _call(ua, batch, no_alloc=False)
        got = _call(ua, batch, no_alloc=True)
        compare(got, oracle.attention(w), f"no-alloc {name} {w.name} vs oracle")
        if bitwise:
            assert np.array_equal(got, want), f"{name}: differs from ua_run"
        else:
            compare(got, want, f"no-alloc {name} {w.name} vs ua_run")


def test_no_alloc_rejects_what_does_not_fit():
    """A segmented split whose partials exceed the scratch, and a caller
    workspace, are refused before anything is enqueued: O keeps its poison."""
    w = W.random_small(77, num_seqs=4, max_q=60, max_k=300, num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16)
    desc = D.problem_desc(w, B.UA_FLAG_FORCE_3D, split_segment_tiles=1, max_total_q=600_000)
    handle = B.ua_create_problem(desc)  # no workspace: this entry point takes none
    try:
        batch = D.DeviceBatch(w)
        args = batch.run_args(None)
        args.total_q = 600_000  # a host shape whose partials need far more than the scratch
        poison_output(batch)
        stream = torch.cuda.current_stream().cuda_stream
        with pytest.raises(B.UaError) as e:
            B.ua_run_no_alloc(handle, args, stream)
        assert e.value.status == B.UA_ERR_WORKSPACE and "scratch" in B.ua_last_error()
        ws = torch.empty(256, dtype=torch.uint8, device="cuda")
        with pytest.raises(B.UaError) as e:
            B.ua_run_no_alloc(handle, batch.run_args(ws), stream)
        assert e.value.status == B.UA_ERR_INVALID_ARG
        torch.cuda.synchronize()
        assert not bool(torch.isfinite(batch.output()).any())
    finally:
        B.ua_destroy_problem(handle)
