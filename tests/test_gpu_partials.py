"""Split partials in caller memory, their merge, and bf16 partials.

* UA_FLAG_BF16_PARTIALS keeps the split-KV partial o in bf16 in the workspace
  (the AITER sparse-attention change stores split-K accumulator partials in
  bf16): every split path stays within the bar against the oracle.
* Partial-output mode (ua_run_args_t.partial_o) writes each row's merge-ready
  state over the call's keys, without sinks; ua_merge joins sets of them and
  the sinks once ([UA] section 5's log-sum-exp re-base).  A batch whose
  sequences share a prefix of cached keys is run as two calls, the shared
  prefix (every key visible to every query) and the per-sequence suffixes
  (causal), merged, and compared with the oracle over the union of keys."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import LSE_TOL, compare, run_hip, say
from varlen_attention_serving_amd import binding as B
from varlen_attention_serving_amd import device as D
from varlen_attention_serving_amd import workloads as W

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _decode(seed, n, hq, hk, d, b, max_k, **kw):
    rng = np.random.default_rng(seed)
    sk = rng.integers(1, max_k, size=n, endpoint=True)
    sk[::7] = 0
    ql = np.minimum(sk, rng.integers(1, 2, size=n, endpoint=True))
    return W.build(f"part_dec_{seed}", seed, ql, sk, num_q_heads=hq, num_kv_heads=hk, head_dim=d,
                   block_size=b, rng=rng, **kw)


def _mixed(seed, hq, hk, d, b, **kw):
    rng = np.random.default_rng(seed)
    dec_k = rng.integers(1, 1200, size=12, endpoint=True)
    ch_q = rng.integers(30, 120, size=3, endpoint=True)
    ctx = rng.integers(0, 900, size=3, endpoint=True)
    ql = np.concatenate([np.ones(12, np.int64), ch_q])
    sk = np.concatenate([dec_k, ctx + ch_q])
    order = rng.permutation(ql.size)
    return W.build(f"part_mix_{seed}", seed, ql[order], sk[order], num_q_heads=hq,
                   num_kv_heads=hk, head_dim=d, block_size=b, rng=rng, **kw)


BF16_PARTIAL_CASES = [
    # (name, workload, extra flags, segment tiles, expected path / stream-K / split)
    ("stream_k_32rows", lambda: _decode(1, 40, 32, 8, 128, 16, 3000, use_sinks=True), 0, 0),
    ("stream_k_16rows_d256_fp8", lambda: _decode(2, 40, 16, 2, 256, 64, 3000,
                                                 kv_dtype=W.DT_FP8_E4M3, use_alibi=True), 0, 0),
    ("segmented_decode", lambda: _decode(3, 40, 32, 8, 128, 16, 3000), B.UA_FLAG_FORCE_3D, 8),
    ("segmented_wide_softcap", lambda: _mixed(4, 16, 4, 64, 16, softcap=20.0, use_sinks=True),
     B.UA_FLAG_FORCE_3D, 0),
    ("class_split_fp8", lambda: _mixed(5, 16, 2, 256, 64, kv_dtype=W.DT_FP8_E4M3,
                                       q_dtype=W.DT_F16, use_sinks=True, window=500), 0, 0),
]


@pytest.mark.parametrize("i", range(len(BF16_PARTIAL_CASES)))
def test_bf16_partials(i):
    """bf16 partial o on every split path: within the bar against the oracle,
    and close to the f32-partial run (each partial rounded to 2^-9 relative)."""
    name, make, flags, seg = BF16_PARTIAL_CASES[i]
    w = make()
    ref = oracle.attention(w)
    o32, plan = run_hip(w, flags, split_segment_tiles=seg)
    o16, plan16 = run_hip(w, flags | B.UA_FLAG_BF16_PARTIALS, split_segment_tiles=seg)
    assert (plan.path, plan.stream_k, plan.class_split) == \
        (plan16.path, plan16.stream_k, plan16.class_split)
    assert plan.path == 3 or plan.class_split == 1
    say(f"[gpu] bf16 partials {name}: path={plan.path} stream_k={plan.stream_k} "
        f"split={plan.class_split} segments={plan.num_segments}")
    compare(o32, ref, f"{name} f32 partials")
    compare(o16, ref, f"{name} bf16 partials")
    compare(o16, o32, f"{name} bf16 vs f32 partials")


def _partial_run(w, flags=0, seg=0, dtype=B.UA_PARTIAL_F32, stream=None):
    """Run w in partial-output mode; returns (partial o tensor, lse tensor, plan)."""
    batch = D.DeviceBatch(w)
    ua = D.UnifiedAttention(D.problem_desc(w, flags, split_segment_tiles=seg))
    shape = (w.total_q, w.num_q_heads, w.head_dim)
    po = torch.full(shape, float("nan"), device="cuda",
                    dtype=torch.float32 if dtype == B.UA_PARTIAL_F32 else torch.bfloat16)
    pl = torch.full(shape[:2], float("nan"), device="cuda", dtype=torch.float32)
    args = batch.run_args(ua.workspace)
    args.o = None
    args.partial_o = po.data_ptr()
    args.partial_lse = pl.data_ptr()
    args.partial_dtype = dtype
    B.ua_run(ua.handle, args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(po).all()) and not bool(torch.isnan(pl).any())
    plan = ua.plan(w)
    ua.close()
    return po, pl, plan


def _merge(w, sets, dtype, sinks=None):
    """ua_merge of partial sets [(o, lse)] into O (w.q_dtype) and its LSE."""
    o = torch.full((w.total_q, w.num_q_heads, w.head_dim), float("nan"), device="cuda",
                   dtype=torch.bfloat16 if w.q_dtype == W.DT_BF16 else torch.float16)
    lse = torch.full((w.total_q, w.num_q_heads), float("nan"), device="cuda")
    a = B.ua_merge_args_t(num_sets=len(sets), partial_dtype=dtype, total_q=w.total_q,
                          num_q_heads=w.num_q_heads, head_dim=w.head_dim, o_dtype=w.q_dtype,
                          o_stride_tok=w.num_q_heads * w.head_dim, o=o.data_ptr(),
                          lse=lse.data_ptr(), sinks=None if sinks is None else sinks.data_ptr())
    for i, (po, pl) in enumerate(sets):
        a.partial_o[i] = po.data_ptr()
        a.partial_lse[i] = pl.data_ptr()
    B.ua_merge(a, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _lse_check(lse, ref_lse, what):
    both_inf = np.isinf(lse) & np.isinf(ref_lse) & (np.sign(lse) == np.sign(ref_lse))
    err = np.where(both_inf, 0.0, np.abs(lse - ref_lse))
    say(f"  {what}: LSE max_abs={float(np.max(err)):.3e}")
    assert not np.isnan(lse).any()
    assert float(np.max(err)) <= LSE_TOL


SINGLE_CASES = [
    ("2d_ring", lambda: _mixed(20, 16, 4, 128, 16, use_sinks=True), B.UA_FLAG_FORCE_2D, 0),
    ("stream_k", lambda: _decode(21, 30, 32, 8, 128, 16, 2000, use_sinks=True), 0, 0),
    ("segmented", lambda: _mixed(22, 8, 2, 64, 32, use_sinks=True, softcap=10.0),
     B.UA_FLAG_FORCE_3D, 0),
    ("class_split_fp8_d256", lambda: _mixed(23, 16, 2, 256, 64, kv_dtype=W.DT_FP8_E4M3,
                                            use_sinks=True, use_alibi=True, window=600), 0, 0),
    ("2d_ring_d256_softcap_alibi", lambda: _mixed(24, 16, 4, 256, 32, use_sinks=True,
                                                  use_alibi=True, softcap=30.0),
     B.UA_FLAG_FORCE_2D, 0),
]


@pytest.mark.parametrize("dtype", [B.UA_PARTIAL_F32, B.UA_PARTIAL_BF16])
@pytest.mark.parametrize("i", range(len(SINGLE_CASES)))
def test_one_partial_set_merged_with_sinks(i, dtype):
    """A partial-output run (sinks left out) merged alone with the sinks gives
    the oracle's O and LSE on each path: the partial is the row's exact state."""
    name, make, flags, seg = SINGLE_CASES[i]
    w = make()
    po, pl, plan = _partial_run(w, flags, seg, dtype)
    sinks = torch.from_numpy(w.sinks).cuda()
    o, lse = _merge(w, [(po, pl)], dtype, sinks)
    ref_o, ref_lse = oracle.attention(w, return_lse=True)
    say(f"[gpu] single set {name} dtype={dtype}: path={plan.path} stream_k={plan.stream_k} "
        f"split={plan.class_split}")
    compare(o, ref_o, f"{name} merged O")
    _lse_check(lse, ref_lse, name)


def _views(full, prefix):
    """The prefix and suffix views of a batch whose sequences share their
    first `prefix` keys: the prefix view has S_k = prefix and sees every key
    (its queries all lie past the prefix); the suffix view keeps the causal
    mask over each sequence's own keys."""
    b = full.block_size
    nb = prefix // b
    kw = {**full.__dict__, "use_sinks": False, "sinks": None}
    pre = W.Workload(**{**kw, "name": full.name + "_prefix", "causal": False,
                        "seq_lens": np.full(full.num_seqs, prefix, np.int32),
                        "block_table": np.ascontiguousarray(full.block_table[:, :nb])})
    suf = W.Workload(**{**kw, "name": full.name + "_suffix",
                        "seq_lens": (full.seq_lens - prefix).astype(np.int32),
                        "block_table": np.ascontiguousarray(full.block_table[:, nb:])})
    return pre, suf


def _shared_prefix_batch(seed, hq, hk, d, b, prefix, kv=W.DT_BF16, q_dtype=W.DT_BF16, **kw):
    rng = np.random.default_rng(seed)
    n = 10
    ql = np.concatenate([np.ones(6, np.int64), rng.integers(2, 40, size=4, endpoint=True)])
    suffix = ql + rng.integers(0, 300, size=n, endpoint=True)
    full = W.build(f"cascade_{seed}", seed, ql, prefix + suffix, num_q_heads=hq, num_kv_heads=hk,
                   head_dim=d, block_size=b, rng=rng, kv_dtype=kv, q_dtype=q_dtype,
                   use_sinks=True, **kw)
    # every sequence's prefix blocks are sequence 0's
    nb = prefix // b
    full.block_table[1:, :nb] = full.block_table[0, :nb]
    return full, prefix


CASCADE_CASES = [
    # (name, full batch, prefix flags, suffix flags)
    ("bf16_d128", lambda: _shared_prefix_batch(30, 32, 8, 128, 16, 512), 0, 0),
    ("softcap_d64_segmented_prefix", lambda: _shared_prefix_batch(31, 8, 2, 64, 32, 1024,
                                                                  softcap=15.0),
     B.UA_FLAG_FORCE_3D, 0),
    ("fp8_d256", lambda: _shared_prefix_batch(32, 16, 2, 256, 64, 768, kv=W.DT_FP8_E4M3,
                                              q_dtype=W.DT_F16), 0, B.UA_FLAG_FORCE_3D),
]


@pytest.mark.parametrize("dtype", [B.UA_PARTIAL_F32, B.UA_PARTIAL_BF16])
@pytest.mark.parametrize("i", range(len(CASCADE_CASES)))
def test_shared_prefix_as_two_calls_merged(i, dtype):
    """Shared prefix + per-sequence suffixes as two partial-output calls over
    disjoint key sets, merged with the sinks: O within 2e-2 / 5e-3 and LSE
    within 4e-3 of the oracle over the union."""
    name, make, f_pre, f_suf = CASCADE_CASES[i]
    full, prefix = make()
    pre, suf = _views(full, prefix)
    po1, pl1, plan1 = _partial_run(pre, f_pre, 0, dtype)
    po2, pl2, plan2 = _partial_run(suf, f_suf, 0, dtype)
    say(f"[gpu] cascade {name} dtype={dtype}: prefix {prefix} keys path={plan1.path} "
        f"stream_k={plan1.stream_k}; suffix path={plan2.path} stream_k={plan2.stream_k}")
    sinks = torch.from_numpy(full.sinks).cuda()
    o, lse = _merge(full, [(po1, pl1), (po2, pl2)], dtype, sinks)
    ref_o, ref_lse = oracle.attention(full, return_lse=True)
    compare(o, ref_o, f"cascade {name} merged O")
    _lse_check(lse, ref_lse, f"cascade {name}")


def test_merge_of_empty_sets_and_no_sinks():
    """Rows whose sets are all empty (-inf LSE) get O = 0 and LSE = -inf; a
    sink alone gives O = 0 and LSE = sink."""
    w = W.tiny_varlen()
    rows = (w.total_q, w.num_q_heads, w.head_dim)
    po = torch.zeros(rows, device="cuda", dtype=torch.float32)
    pl = torch.full(rows[:2], float("-inf"), device="cuda")
    o, lse = _merge(w, [(po, pl), (po, pl)], B.UA_PARTIAL_F32)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    sinks = torch.linspace(-1, 1, w.num_q_heads, device="cuda")
    o, lse = _merge(w, [(po, pl)], B.UA_PARTIAL_F32, sinks)
    assert np.all(o == 0)
    assert np.allclose(lse, np.broadcast_to(sinks.cpu().numpy(), lse.shape), atol=1e-6)
