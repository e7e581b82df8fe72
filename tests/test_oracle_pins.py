"""Pins for the fp64 oracle against things other than itself: library decoders,
closed forms, torch's fp64 SDPA, a dense numpy brute force, limits and
invariants.  None of these tests needs a GPU."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from refs import brute_force, decode, dense_kv
from varlen_attention_serving_amd import workloads as W

TOL = 1e-12


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1.0, float(np.max(np.abs(b)))))


# ---------------------------------------------------------------------------
# exact decoders of the stored types
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [W.DT_BF16, W.DT_F16])
def test_decoder_all_16bit_codes(dtype):
    bits = np.arange(65536, dtype=np.uint32)
    ref = decode(bits.astype(np.uint16), dtype)
    got = np.array([oracle.decode(dtype, int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_decoder_all_e4m3fn_codes():
    bits = np.arange(256, dtype=np.uint32)
    ref = decode(bits.astype(np.uint8), W.DT_FP8_E4M3)
    got = np.array([oracle.decode(W.DT_FP8_E4M3, int(b)) for b in bits])
    nan = np.isnan(ref)
    assert nan.sum() == 2                      # 0x7F and 0xFF only
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# ---------------------------------------------------------------------------
# dense brute force (full score matrix + explicit mask matrix)
# ---------------------------------------------------------------------------

def test_tiny_varlen_vs_brute_force():
    w = W.tiny_varlen()
    o, lse = oracle.attention(w, return_lse=True)
    ob, lseb = brute_force(w)
    assert not np.isnan(o).any()
    assert _rel(o, ob) < TOL
    assert np.max(np.abs(lse - lseb)) < 1e-10


FLAG_CASES = [
    dict(),
    dict(causal=False),
    dict(softcap=3.0),
    dict(use_alibi=True),
    dict(window=7),
    dict(window=7, causal=False),
    dict(use_sinks=True),
    dict(softcap=2.0, use_alibi=True, window=9, use_sinks=True),
    dict(q_dtype=W.DT_F16, kv_dtype=W.DT_F16, use_sinks=True),
    dict(q_dtype=W.DT_F16, kv_dtype=W.DT_FP8_E4M3, use_alibi=True, use_sinks=True, window=11),
    dict(kv_dtype=W.DT_FP8_E4M3),
    dict(use_qq_bias=True),
    dict(use_qq_bias=True, causal=False, use_alibi=True, softcap=2.0, window=9, use_sinks=True),
]


@pytest.mark.parametrize("case", range(len(FLAG_CASES)))
@pytest.mark.parametrize("shape", [(4, 2, 64, 16), (8, 2, 32, 8), (6, 3, 16, 4), (2, 2, 128, 32)])
def test_random_flags_vs_brute_force(case, shape):
    hq, hk, d, b = shape
    w = W.random_small(100 + case, num_seqs=4, max_q=20, max_k=70, num_q_heads=hq,
                       num_kv_heads=hk, head_dim=d, block_size=b, **FLAG_CASES[case])
    o, lse = oracle.attention(w, return_lse=True)
    ob, lseb = brute_force(w)
    assert not np.isnan(o).any()
    assert _rel(o, ob) < TOL
    assert np.max(np.abs(lse - lseb)) < 1e-10


def test_window_reading_is_w_keys_not_w_plus_one():
    """The brute force with one extra window key must disagree: the oracle's
    window reading (W keys) is decided, not accidental."""
    w = W.random_small(7, num_seqs=3, max_q=20, max_k=70, window=5)
    o = oracle.attention(w)
    assert _rel(o, brute_force(w)[0]) < TOL
    assert _rel(o, brute_force(w, window_extra_key=1)[0]) > 1e-3


# ---------------------------------------------------------------------------
# torch fp64 SDPA (library routine) for the flag subsets it can express
# ---------------------------------------------------------------------------

def _sdpa_seq(w, s, float_mask=None, is_causal=False):
    ql, t0 = int(w.q_lens[s]), int(w.cu_seqlens_q[s])
    q = torch.from_numpy(decode(w.q[t0:t0 + ql], w.q_dtype)).permute(1, 0, 2)  # [Hq, ql, d]
    k, v = dense_kv(w, s)
    g = w.group
    k = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)        # [Hq, sk, d]
    v = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=float_mask, is_causal=is_causal,
                                       scale=w.scale)
    return o.permute(1, 0, 2).numpy()


def test_decode_vs_sdpa():
    rng = np.random.default_rng(11)
    sk = rng.integers(1, 300, size=6, endpoint=True)
    w = W.build("dec", 11, np.ones(6), sk, num_q_heads=8, num_kv_heads=2, head_dim=64,
                block_size=16, rng=rng)
    o = oracle.attention(w)
    for s in range(w.num_seqs):
        t0 = int(w.cu_seqlens_q[s])
        assert _rel(o[t0:t0 + 1], _sdpa_seq(w, s)) < TOL


def test_prefill_causal_vs_sdpa():
    lens = [1, 17, 64, 65]
    w = W.build("pf", 12, lens, lens, num_q_heads=6, num_kv_heads=3, head_dim=32, block_size=16)
    o = oracle.attention(w)
    for s in range(w.num_seqs):
        t0, ql = int(w.cu_seqlens_q[s]), int(w.q_lens[s])
        assert _rel(o[t0:t0 + ql], _sdpa_seq(w, s, is_causal=True)) < TOL


@pytest.mark.parametrize("causal", [True, False])
def test_window_and_alibi_vs_sdpa_float_mask(causal):
    """ALiBi enters SDPA as slope * (k - q_abs), a row-constant shift of the
    oracle's slope * (k - ctx): equal outputs by shift invariance."""
    rng = np.random.default_rng(13)
    sk = rng.integers(20, 120, size=4, endpoint=True)
    ql = np.minimum(sk, rng.integers(1, 30, size=4, endpoint=True))
    w = W.build("wa", 13, ql, sk, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                window=9, use_alibi=True, causal=causal, rng=rng)
    o = oracle.attention(w)
    for s in range(w.num_seqs):
        t0, q_len, s_k = int(w.cu_seqlens_q[s]), int(w.q_lens[s]), int(w.seq_lens[s])
        ctx = s_k - q_len
        qa = ctx + np.arange(q_len)[:, None]
        kp = np.arange(s_k)[None, :]
        keep = kp > qa - w.window
        if causal:
            keep &= kp <= qa
        slopes = w.alibi_slopes.astype(np.float64)[:, None, None]
        bias = slopes * (kp - qa)[None]
        mask = torch.from_numpy(np.where(keep[None], bias, -np.inf))
        assert _rel(o[t0:t0 + q_len], _sdpa_seq(w, s, float_mask=mask)) < 1e-11


@pytest.mark.parametrize("causal", [True, False])
def test_qq_bias_vs_sdpa_float_mask(causal):
    """QQ-bias is an additive float mask over the query section: keys
    ctx .. S_k - 1 of local query row i get bias[i, k - ctx]."""
    rng = np.random.default_rng(14)
    sk = rng.integers(20, 120, size=4, endpoint=True)
    ql = np.minimum(sk, rng.integers(1, 30, size=4, endpoint=True))
    w = W.build("qq", 14, ql, sk, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                causal=causal, rng=rng, use_qq_bias=True)
    o = oracle.attention(w)
    for s in range(w.num_seqs):
        t0, q_len, s_k = int(w.cu_seqlens_q[s]), int(w.q_lens[s]), int(w.seq_lens[s])
        ctx = s_k - q_len
        bias = np.zeros((q_len, s_k))
        bias[:, ctx:] = w.qq_bias[:q_len, :q_len]
        if causal:
            qa = ctx + np.arange(q_len)[:, None]
            bias = np.where(np.arange(s_k)[None, :] <= qa, bias, -np.inf)
        mask = torch.from_numpy(np.broadcast_to(bias, (w.num_q_heads, q_len, s_k)).copy())
        assert _rel(o[t0:t0 + q_len], _sdpa_seq(w, s, float_mask=mask)) < 1e-11


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _identical_keys(w, rng):
    kvec = W.f32_to_bf16_bits(rng.standard_normal(w.head_dim).astype(np.float32))
    w.k_cache[...] = kvec
    return w


def _visible(w, s, i):
    s_k, q_len = int(w.seq_lens[s]), int(w.q_lens[s])
    q_abs = s_k - q_len + i
    k = np.arange(s_k)
    keep = np.ones(s_k, dtype=bool)
    if w.causal:
        keep &= k <= q_abs
    if w.window > 0:
        keep &= k > q_abs - w.window
    return keep


@pytest.mark.parametrize("flags", [dict(), dict(window=5), dict(window=5, causal=False),
                                   dict(window=1)])
def test_identical_keys_give_mean_of_visible_values(flags):
    rng = np.random.default_rng(21)
    w = _identical_keys(W.build("ik", 21, [1, 4, 9], [9, 30, 50], num_q_heads=4, num_kv_heads=2,
                                head_dim=64, block_size=8, **flags), rng)
    o = oracle.attention(w)
    for s in range(w.num_seqs):
        _, v = dense_kv(w, s)
        for i in range(int(w.q_lens[s])):
            keep = _visible(w, s, i)
            t = int(w.cu_seqlens_q[s]) + i
            for h in range(w.num_q_heads):
                expect = v[keep, h // w.group, :].mean(axis=0)
                assert np.max(np.abs(o[t, h] - expect)) < 1e-12
            if w.window:
                s_k, q_abs = int(w.seq_lens[s]), int(w.seq_lens[s]) - int(w.q_lens[s]) + i
                hi = q_abs + 1 if w.causal else s_k
                assert keep.sum() == hi - max(0, q_abs - w.window + 1)


def test_identical_keys_with_alibi_give_geometric_weights():
    rng = np.random.default_rng(22)
    w = _identical_keys(W.build("ika", 22, [3], [40], num_q_heads=4, num_kv_heads=1,
                                head_dim=64, block_size=16, use_alibi=True), rng)
    o = oracle.attention(w)
    _, v = dense_kv(w, 0)
    for i in range(3):
        keep = _visible(w, 0, i)
        kk = np.nonzero(keep)[0]
        for h in range(4):
            r = math.exp(float(w.alibi_slopes[h]))
            wt = r ** (kk - kk.max())
            expect = (wt[:, None] * v[kk, 0, :]).sum(0) / wt.sum()
            assert np.max(np.abs(o[i, h] - expect)) < 1e-12


def test_identical_keys_with_qq_bias_weigh_the_query_section():
    """With every key equal, the weights are e^bias[i, k - ctx] on the query
    section and 1 on the context: the bias's row is the query, its column
    the key (an asymmetric matrix tells the two apart)."""
    rng = np.random.default_rng(24)
    w = _identical_keys(W.build("ikq", 24, [5, 3], [17, 3], num_q_heads=2, num_kv_heads=1,
                                head_dim=32, block_size=4, causal=False, use_qq_bias=True,
                                rng=rng), rng)
    assert np.max(np.abs(w.qq_bias - w.qq_bias.T)) > 0.1
    o = oracle.attention(w)
    for s in range(2):
        _, v = dense_kv(w, s)
        q_len, s_k = int(w.q_lens[s]), int(w.seq_lens[s])
        ctx = s_k - q_len
        for i in range(q_len):
            wt = np.ones(s_k)
            wt[ctx:] = np.exp(w.qq_bias[i, :q_len].astype(np.float64))
            expect = (wt[:, None] * v[:, 0, :]).sum(0) / wt.sum()
            t = int(w.cu_seqlens_q[s]) + i
            for h in range(2):
                assert np.max(np.abs(o[t, h] - expect)) < 1e-12


def test_identical_keys_with_sinks():
    """Sinks are an extra softmax column with no value row: the real weights
    sum to n e^x / (n e^x + e^sink) < 1."""
    rng = np.random.default_rng(23)
    w = _identical_keys(W.build("iks", 23, [2, 1], [12, 33], num_q_heads=2, num_kv_heads=2,
                                head_dim=32, block_size=4, use_sinks=True), rng)
    w.sinks = np.array([0.5, 3.0], dtype=np.float32)
    o = oracle.attention(w)
    qd = decode(w.q, w.q_dtype)
    kvec = decode(w.k_cache[0, 0, 0], w.kv_dtype)
    for s in range(2):
        _, v = dense_kv(w, s)
        for i in range(int(w.q_lens[s])):
            t = int(w.cu_seqlens_q[s]) + i
            keep = _visible(w, s, i)
            n = int(keep.sum())
            for h in range(2):
                x = w.scale * float(qd[t, h] @ kvec)
                frac = n * math.exp(x) / (n * math.exp(x) + math.exp(float(w.sinks[h])))
                assert frac < 1.0
                expect = frac * v[keep, h, :].mean(axis=0)
                assert np.max(np.abs(o[t, h] - expect)) < 1e-12


@pytest.mark.parametrize("softcap", [0.0, 4.0])
def test_one_dominant_logit(softcap):
    """Q = alpha e0, K_t = e0, every other key orthogonal to e0: exactly
    O = (e^{x_t} V_t + sum_others V_k) / (e^{x_t} + n - 1), x_t = tau alpha
    (capped to c tanh(tau alpha / c) under softcap)."""
    rng = np.random.default_rng(24)
    d, sk, target = 64, 45, 17
    w = W.build("dom", 24, [1], [sk], num_q_heads=1, num_kv_heads=1, head_dim=d, block_size=16,
                softcap=softcap, causal=True)
    alpha = 64.0
    qv = np.zeros(d, np.float32)
    qv[0] = alpha
    w.q[0, 0] = W.f32_to_bf16_bits(qv)
    kf = rng.standard_normal((sk, d)).astype(np.float32)
    kf[:, 0] = 0.0
    kf[target] = 0.0
    kf[target, 0] = 1.0
    for k in range(sk):
        w.k_cache[w.block_table[0, k // 16], k % 16, 0] = W.f32_to_bf16_bits(kf[k])
    o = oracle.attention(w)
    _, v = dense_kv(w, 0)
    xt = w.scale * alpha
    if softcap:
        xt = softcap * math.tanh(xt / softcap)
    others = np.delete(np.arange(sk), target)
    expect = (math.exp(xt) * v[target, 0] + v[others, 0].sum(0)) / (math.exp(xt) + sk - 1)
    assert np.max(np.abs(o[0, 0] - expect)) < 1e-12
    # and the dominant row is selected within the bound (n-1) e^{-x_t} max|V|
    if not softcap:
        bound = (sk - 1) * math.exp(-xt) * 2 * np.abs(v[:, 0]).max()
        assert np.max(np.abs(o[0, 0] - v[target, 0])) <= bound


# ---------------------------------------------------------------------------
# limits, special cases, invariants
# ---------------------------------------------------------------------------

def test_softcap_limit_is_no_softcap():
    w = W.random_small(31, num_seqs=3)
    base = oracle.attention(w)
    w.softcap = 1e12
    assert _rel(oracle.attention(w), base) < 1e-9


def test_window_covering_everything_is_no_window():
    w = W.random_small(32, num_seqs=3, max_k=60)
    base = oracle.attention(w)
    w.window = 60
    assert np.array_equal(oracle.attention(w), base)


def test_softcap_is_exercised_when_scores_reach_the_cap():
    """Scaled Q makes |s| ~ c: capped and uncapped outputs must then differ."""
    w = W.random_small(33, num_seqs=2, softcap=2.0)
    big = decode(w.q, w.q_dtype) * 40.0
    w.q[...] = W.f32_to_bf16_bits(big.astype(np.float32))
    capped = oracle.attention(w)
    assert _rel(capped, brute_force(w)[0]) < TOL
    w.softcap = 0.0
    assert _rel(capped, oracle.attention(w)) > 1e-2


def test_block_table_permutation_invariance():
    w = W.random_small(34, num_seqs=4, max_k=90)
    base = oracle.attention(w)
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_blocks)            # new physical slot of each block
    k2 = np.empty_like(w.k_cache)
    v2 = np.empty_like(w.v_cache)
    k2[perm] = w.k_cache
    v2[perm] = w.v_cache
    bt = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w.k_cache, w.v_cache, w.block_table = k2, v2, bt
    assert np.array_equal(oracle.attention(w), base)


def test_poisoned_slots_never_reach_output():
    for name in ("tiny_varlen",):
        w = W.NAMED[name]()
        assert np.isnan(decode(w.k_cache, w.kv_dtype)).any()
        assert not np.isnan(oracle.attention(w)).any()


def test_rows_match_full_attention():
    w = W.random_small(35, num_seqs=3, use_sinks=True, use_alibi=True)
    full, lse = oracle.attention(w, return_lse=True)
    rows = np.array([0, 5, w.total_q * w.num_q_heads - 1, 7])
    o, l = oracle.rows(w, rows, return_lse=True)
    flat = full.reshape(-1, w.head_dim)
    assert np.array_equal(o, flat[rows])
    assert np.array_equal(l, lse.reshape(-1)[rows])


# ---------------------------------------------------------------------------
# the streaming recurrence and the split merge reproduce the oracle
# ---------------------------------------------------------------------------

def _scores(w, s, i, h):
    k, _ = dense_kv(w, s)
    qd = decode(w.q, w.q_dtype)
    t = int(w.cu_seqlens_q[s]) + i
    x = w.scale * (k[:, h // w.group, :] @ qd[t, h])
    if w.softcap > 0:
        x = w.softcap * np.tanh(x / w.softcap)
    if w.use_alibi:
        ctx = int(w.seq_lens[s]) - int(w.q_lens[s])
        x = x + float(w.alibi_slopes[h]) * (np.arange(x.size) - ctx)
    return np.where(_visible(w, s, i), x, -np.inf)


def _stream(x, v, cuts, base2):
    """(m, l, o) over the tiles between `cuts`, in e- or 2-based exponentials."""
    lg = math.log2(math.e) if base2 else 1.0
    ex = np.exp2 if base2 else np.exp
    m, l, o = -np.inf, 0.0, np.zeros(v.shape[1])
    for a, b in zip(cuts[:-1], cuts[1:]):
        t = x[a:b] * lg
        m_new = max(m, float(t.max())) if b > a else m
        if m_new == -np.inf:
            continue
        alpha = ex(m - m_new) if m > -np.inf else 0.0
        p = ex(t - m_new)
        l = alpha * l + p.sum()
        o = alpha * o + p @ v[a:b]
        m = m_new
    return m, l, o


def _merge(parts, base2):
    ex = np.exp2 if base2 else np.exp
    live = [p for p in parts if p[0] > -np.inf]
    if not live:
        return -np.inf, 0.0, None
    mg = max(p[0] for p in live)
    l = sum(p[1] * ex(p[0] - mg) for p in live)
    o = sum(p[2] * ex(p[0] - mg) for p in live)
    return mg, l, o


@pytest.mark.parametrize("base2", [False, True])
def test_streaming_and_split_merge_equal_oracle(base2):
    rng = np.random.default_rng(41)
    w = W.random_small(41, num_seqs=3, max_k=120, softcap=5.0, use_alibi=True, window=40,
                       use_sinks=True)
    o = oracle.attention(w)
    lg = math.log2(math.e) if base2 else 1.0
    for s in range(w.num_seqs):
        _, v = dense_kv(w, s)
        for i in range(int(w.q_lens[s])):
            for h in range(w.num_q_heads):
                x = _scores(w, s, i, h)
                vv = v[:, h // w.group, :]
                n = x.size
                cuts = np.unique(np.concatenate([[0, n], rng.integers(0, n + 1, 5)]))
                segs = np.unique(np.concatenate([[0, n], rng.integers(0, n + 1, 3)]))
                parts = [_stream(x[a:b], vv[a:b], np.unique(np.r_[0, b - a,
                                 rng.integers(0, b - a + 1, 2)]), base2)
                         for a, b in zip(segs[:-1], segs[1:])]
                # the sink is one more (m = sink, l = 1, o = 0) partial
                parts.append((float(w.sinks[h]) * lg, 1.0, np.zeros(v.shape[2])))
                for m, l, acc in (_merge([_stream(x, vv, cuts, base2), parts[-1]], base2),
                                  _merge(parts, base2)):
                    t = int(w.cu_seqlens_q[s]) + i
                    assert np.max(np.abs(acc / l - o[t, h])) < 1e-12
