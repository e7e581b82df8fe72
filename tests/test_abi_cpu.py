"""The C boundary without a GPU: the library loads, exports every function
include/ua.h declares, rejects invalid descriptors and run arguments with a
status code and a message (before touching a device), sizes its workspace and
plans each named workload on the path the shape rule gives."""
import ctypes
import os
import re

import numpy as np
import pytest

from varlen_attention_serving_amd import binding as B
from varlen_attention_serving_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ua.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(ua_\w+)\s*\(", text, flags=re.M)))


def test_header_declarations_are_all_exported():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_empty_error():
    assert re.match(r"^\d+\.\d+\.\d+$", B.ua_version())
    h = B.ua_create_problem(_desc())
    assert B.ua_last_error() == ""
    B.ua_destroy_problem(h)
    B.ua_destroy_problem(None)


def _desc(**kw):
    d = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
             q_dtype=B.UA_DTYPE_BF16, kv_dtype=B.UA_DTYPE_BF16, flags=B.UA_FLAG_CAUSAL,
             scale=0.088, softcap=0.0, window=0, k_scale=1.0, v_scale=1.0, num_blocks=100,
             max_num_seqs=8, max_blocks_per_seq=64, max_total_q=512, max_seqlen_k=1024)
    d.update(kw)
    return B.ua_problem_desc_t(**d)


BAD_DESCS = [
    (dict(num_q_heads=0), B.UA_ERR_INVALID_ARG, "head counts"),
    (dict(num_q_heads=6, num_kv_heads=4), B.UA_ERR_INVALID_ARG, "multiple"),
    (dict(num_q_heads=256, num_kv_heads=1), B.UA_ERR_UNSUPPORTED, "GQA group"),
    (dict(head_dim=96), B.UA_ERR_UNSUPPORTED, "head_dim"),
    (dict(head_dim=-1), B.UA_ERR_INVALID_ARG, "head_dim"),
    (dict(block_size=24), B.UA_ERR_INVALID_ARG, "block_size"),
    (dict(q_dtype=B.UA_DTYPE_FP8_E4M3), B.UA_ERR_UNSUPPORTED, "q_dtype"),
    (dict(kv_dtype=B.UA_DTYPE_F16), B.UA_ERR_UNSUPPORTED, "kv_dtype"),
    (dict(flags=1 << 20), B.UA_ERR_INVALID_ARG, "unknown flag"),
    (dict(flags=B.UA_FLAG_FORCE_2D | B.UA_FLAG_FORCE_3D), B.UA_ERR_INVALID_ARG, "exclusive"),
    (dict(scale=0.0), B.UA_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("inf")), B.UA_ERR_INVALID_ARG, "scale"),
    (dict(flags=B.UA_FLAG_SOFTCAP, softcap=0.0), B.UA_ERR_INVALID_ARG, "softcap"),
    (dict(flags=B.UA_FLAG_WINDOW, window=0), B.UA_ERR_INVALID_ARG, "window"),
    (dict(kv_dtype=B.UA_DTYPE_FP8_E4M3, k_scale=0.0), B.UA_ERR_INVALID_ARG, "k_scale"),
    (dict(num_blocks=0), B.UA_ERR_INVALID_ARG, "num_blocks"),
    (dict(max_seqlen_k=2048, max_blocks_per_seq=64), B.UA_ERR_INVALID_ARG, "max_blocks_per_seq"),
    (dict(flags=B.UA_FLAG_DENSE_KV), B.UA_ERR_INVALID_ARG, "needs block_size 1"),
]


@pytest.mark.parametrize("i", range(len(BAD_DESCS)))
def test_invalid_descriptors_are_rejected(i):
    kw, status, text = BAD_DESCS[i]
    with pytest.raises(B.UaError) as e:
        B.ua_create_problem(_desc(**kw))
    assert e.value.status == status
    assert text in B.ua_last_error()


def test_null_pointers_are_rejected():
    h = ctypes.c_void_p()
    assert B.lib.ua_create_problem(None, ctypes.byref(h)) == B.UA_ERR_INVALID_ARG
    assert B.lib.ua_run(None, None, None) == B.UA_ERR_INVALID_ARG
    assert B.lib.ua_query_plan(None, 0, 0, 0, 0, None) == B.UA_ERR_INVALID_ARG


def _args(**kw):
    fake = 1 << 20  # aligned non-null placeholder; validation fails before any use
    a = dict(q=fake, k_cache=fake, v_cache=fake, o=fake, block_table=fake, seq_lens=fake,
             cu_seqlens_q=fake, alibi_slopes=None, sinks=None, workspace=None, workspace_bytes=0,
             num_seqs=2, max_seqlen_q=4, total_q=8, max_seqlen_k=512, block_table_stride=64,
             q_stride_tok=1024, o_stride_tok=1024)
    a.update(kw)
    return B.ua_run_args_t(**a)


BAD_ARGS = [
    (dict(num_seqs=9), B.UA_ERR_INVALID_ARG, "num_seqs"),
    (dict(total_q=513), B.UA_ERR_INVALID_ARG, "total_q"),
    (dict(max_seqlen_k=1025), B.UA_ERR_INVALID_ARG, "max_seqlen_k"),
    (dict(max_seqlen_q=600), B.UA_ERR_INVALID_ARG, "max_seqlen_q"),
    (dict(q_stride_tok=1000), B.UA_ERR_INVALID_ARG, "strides"),
    (dict(o_stride_tok=1028), B.UA_ERR_INVALID_ARG, "multiples of 8"),
    (dict(block_table_stride=8), B.UA_ERR_INVALID_ARG, "block_table_stride"),
    (dict(q=None), B.UA_ERR_INVALID_ARG, "null required"),
    (dict(cu_seqlens_q=None), B.UA_ERR_INVALID_ARG, "null required"),
    (dict(o=(1 << 20) + 2), B.UA_ERR_INVALID_ARG, "aligned"),
    (dict(lse=(1 << 20) + 2), B.UA_ERR_INVALID_ARG, "lse must be 4-byte aligned"),
]


@pytest.mark.parametrize("i", range(len(BAD_ARGS)))
def test_invalid_run_arguments_are_rejected(i):
    kw, status, text = BAD_ARGS[i]
    h = B.ua_create_problem(_desc())
    try:
        with pytest.raises(B.UaError) as e:
            B.ua_run(h, _args(**kw), None)
        assert e.value.status == status
        assert text in B.ua_last_error()
    finally:
        B.ua_destroy_problem(h)


def test_flagged_inputs_need_their_pointers():
    for flag, text in ((B.UA_FLAG_ALIBI, "alibi_slopes"), (B.UA_FLAG_SINKS, "sinks"),
                       (B.UA_FLAG_QQ_BIAS, "qq_bias is null")):
        h = B.ua_create_problem(_desc(flags=B.UA_FLAG_CAUSAL | flag))
        with pytest.raises(B.UaError, match=text):
            B.ua_run(h, _args(), None)
        B.ua_destroy_problem(h)


def test_qq_bias_must_cover_the_query_rows():
    h = B.ua_create_problem(_desc(flags=B.UA_FLAG_CAUSAL | B.UA_FLAG_QQ_BIAS))
    try:
        with pytest.raises(B.UaError, match="qq_bias_stride"):
            B.ua_run(h, _args(qq_bias=1 << 20, qq_bias_stride=3), None)  # max_seqlen_q = 4
        with pytest.raises(B.UaError, match="qq_bias must be 4-byte aligned"):
            B.ua_run(h, _args(qq_bias=(1 << 20) + 2, qq_bias_stride=4), None)
    finally:
        B.ua_destroy_problem(h)


def _dense_desc(extra=0):
    return _desc(flags=B.UA_FLAG_CAUSAL | B.UA_FLAG_DENSE_KV | extra, block_size=1,
                 num_blocks=4096, max_blocks_per_seq=0)


def test_dense_layout_needs_cu_seqlens_k_and_no_table():
    no_table = dict(block_table=None, seq_lens=None, block_table_stride=0)
    h = B.ua_create_problem(_dense_desc())
    try:
        with pytest.raises(B.UaError, match="cu_seqlens_k"):
            B.ua_run(h, _args(**no_table), None)
        with pytest.raises(B.UaError, match="cu_seqlens_k"):
            B.ua_run(h, _args(cu_seqlens_k=(1 << 20) + 2, **no_table), None)
    finally:
        B.ua_destroy_problem(h)
    # with cu_seqlens_k given, the table arguments are not validated: a forced
    # split run gets as far as the workspace check
    h = B.ua_create_problem(_dense_desc(B.UA_FLAG_FORCE_3D))
    try:
        with pytest.raises(B.UaError) as e:
            B.ua_run(h, _args(cu_seqlens_k=1 << 20, **no_table), None)
        assert e.value.status == B.UA_ERR_WORKSPACE
    finally:
        B.ua_destroy_problem(h)


def test_split_path_needs_workspace():
    h = B.ua_create_problem(_desc(flags=B.UA_FLAG_CAUSAL | B.UA_FLAG_FORCE_3D))
    assert B.ua_workspace_size(h) > 0
    with pytest.raises(B.UaError) as e:
        B.ua_run(h, _args(), None)
    assert e.value.status == B.UA_ERR_WORKSPACE
    B.ua_destroy_problem(h)


def test_empty_batch_returns_ok_without_launch():
    h = B.ua_create_problem(_desc())
    B.ua_run(h, _args(num_seqs=0, total_q=0, max_seqlen_q=0, q=None), None)
    B.ua_destroy_problem(h)


def _named_plan(name, extra=0, split_segment_tiles=0):
    sp = W.named_spec(name)
    kw = sp["kw"]
    ql = np.asarray(sp["q_lens"])
    sk = np.asarray(sp["seq_lens"])
    b = kw["block_size"]
    flags = B.UA_FLAG_CAUSAL | extra
    if kw.get("softcap", 0) > 0:
        flags |= B.UA_FLAG_SOFTCAP
    if kw.get("window", 0) > 0:
        flags |= B.UA_FLAG_WINDOW
    if kw.get("use_alibi"):
        flags |= B.UA_FLAG_ALIBI
    if kw.get("use_sinks"):
        flags |= B.UA_FLAG_SINKS
    d = B.ua_problem_desc_t(
        num_q_heads=kw["num_q_heads"], num_kv_heads=kw["num_kv_heads"], head_dim=kw["head_dim"],
        block_size=b, q_dtype=kw.get("q_dtype", 0), kv_dtype=kw.get("kv_dtype", 0), flags=flags,
        scale=kw.get("scale", kw["head_dim"] ** -0.5), softcap=kw.get("softcap", 0.0),
        window=kw.get("window", 0), k_scale=0.01, v_scale=0.01,
        num_blocks=int(((sk + b - 1) // b).sum()) + 16, max_num_seqs=len(ql),
        max_blocks_per_seq=int((sk.max() + b - 1) // b), max_total_q=int(ql.sum()),
        max_seqlen_k=int(sk.max()), split_segment_tiles=split_segment_tiles)
    h = B.ua_create_problem(d)
    try:
        return B.ua_query_plan(h, len(ql), int(ql.sum()), int(ql.max()), int(sk.max())), \
            B.ua_workspace_size(h)
    finally:
        B.ua_destroy_problem(h)


@pytest.mark.parametrize("name,path,split", [("tiny_varlen", 2, 0), ("decode_batch", 3, 0),
                                             ("chunked_prefill_mix", 2, 0),
                                             ("long_prefill", 2, 0), ("variant_mix", 2, 1),
                                             ("decode_large", 3, 0)])
def test_shape_rule(name, path, split):
    """2D when the q-block x kv-head grid of wide q-blocks fills the device or
    a q-block visits few keys (short context or a short window); otherwise
    the split path, and stream-K for decode-shaped batches of any size.
    Wide batches on the register-staged path (fp8 K/V, d = 256) send their
    decode-shaped sequences to a stream-K launch and keep the rest as one
    unsegmented 2D launch beside it; on the LDS ring a batch whose full grid
    fills one resident round stays one 2D launch."""
    plan, ws = _named_plan(name)
    assert plan.path == path
    assert plan.class_split == split
    if name in ("decode_batch", "decode_large"):
        assert plan.stream_k == 1 and plan.waves == 1 and plan.tile_n == 32
    if split:
        assert plan.waves == 4 and plan.stream_k == 1
    if path == 2:
        assert plan.num_segments == 1 and plan.grid[2] == 1
    assert ws < (3 << 30)


RING_POLICY = [
    # (H_q, H_k, d, b, extra flags, decode rows, class split expected)
    (32, 8, 128, 16, 0, 40, 0),                  # d <= 128 ring: one launch
    (32, 8, 128, 2, 0, 40, 1),                   # blocks below one copy's 4 rows
    (16, 8, 256, 32, 0, 96, 0),                  # d = 256 ring, grid fills a round
    (16, 2, 256, 32, 0, 64, 1),                  # d = 256 ring, grid too small
    (16, 8, 256, 32, B.UA_FLAG_SOFTCAP, 96, 0),  # d = 256 ring with softcap or ALiBi
    (16, 8, 256, 32, B.UA_FLAG_ALIBI, 96, 0),
    (16, 2, 256, 32, B.UA_FLAG_ALIBI, 64, 1),    # ... grid too small
    (16, 8, 256, 32, B.UA_FLAG_QQ_BIAS, 96, 1),  # d = 256 with the QQ bias: register path
    (16, 8, 256, 32, B.UA_FLAG_ALIBI | B.UA_FLAG_QQ_BIAS, 96, 1),
]


@pytest.mark.parametrize("i", range(len(RING_POLICY)))
def test_mixed_batch_policy(i):
    """Decode rows plus four 512-query chunks: LDS-ring batches (16-bit K/V,
    blocks of at least 512 / d keys, at d = 256 not with the QQ bias) stay
    one 2D launch when their full grid fills a resident
    round; other wide batches, and d = 256 ring batches that do not fill it,
    send the decode rows to the concurrent stream-K launch.  A d <= 128 ring
    batch never splits."""
    hq, hk, d, b, extra, n_dec, want = RING_POLICY[i]
    sk_max = 8192
    desc = _desc(num_q_heads=hq, num_kv_heads=hk, head_dim=d, block_size=b,
                 flags=B.UA_FLAG_CAUSAL | extra, softcap=30.0 if extra & B.UA_FLAG_SOFTCAP else 0.0,
                 num_blocks=(n_dec + 4) * sk_max // b, max_num_seqs=n_dec + 4,
                 max_blocks_per_seq=sk_max // b, max_total_q=n_dec + 4 * 512, max_seqlen_k=sk_max)
    h = B.ua_create_problem(desc)
    try:
        plan = B.ua_query_plan(h, n_dec + 4, n_dec + 4 * 512, 512, sk_max)
    finally:
        B.ua_destroy_problem(h)
    assert plan.path == 2 and plan.class_split == want
    if want:
        assert plan.stream_k == 1


@pytest.mark.parametrize("q_lens,want", [((1024, 1024), 0), ((1024, 1024, 1), 1),
                                          ((1024, 1024, 2), 1), ((1024, 1024, 3), 0)])
def test_no_class_split_without_a_decode_shaped_sequence(q_lens, want):
    """An fp8 d = 256 batch (H 16/2: the 16-row stream-K q-blocks hold two
    query positions) splits off its decode-shaped sequences only when one can
    exist: the shortest sequence holds at least total_q - (n - 1) * max_q
    queries."""
    sk_max = 4096
    n, total, mx = len(q_lens), sum(q_lens), max(q_lens)
    desc = _desc(num_q_heads=16, num_kv_heads=2, head_dim=256, block_size=64, q_dtype=B.UA_DTYPE_F16,
                 kv_dtype=B.UA_DTYPE_FP8_E4M3, flags=B.UA_FLAG_CAUSAL | B.UA_FLAG_ALIBI,
                 num_blocks=n * sk_max // 64, max_num_seqs=n, max_blocks_per_seq=sk_max // 64,
                 max_total_q=total, max_seqlen_k=sk_max)
    h = B.ua_create_problem(desc)
    try:
        plan = B.ua_query_plan(h, n, total, mx, sk_max)
    finally:
        B.ua_destroy_problem(h)
    assert plan.class_split == want
    if not want:
        assert plan.path == 3 and plan.stream_k == 0  # the wide rule: a segmented split


QQ_D256_PLANS = [
    # (H_q, H_k, kv dtype, QQ, max_q, forced 3D (or a sequence count in place of
    # the default 16), (path, stream_k, block_m) expected)
    (16, 4, B.UA_DTYPE_BF16, True, 7, False, (3, 0, 32)),    # 28-row blocks: segmented split
    (16, 4, B.UA_DTYPE_BF16, True, 7, True, (3, 0, 32)),     # forced: the segmented split
    (16, 4, B.UA_DTYPE_F16, True, 7, True, (3, 0, 32)),
    (16, 4, B.UA_DTYPE_BF16, False, 7, False, (3, 1, 32)),   # without the QQ bias it streams
    (16, 4, B.UA_DTYPE_FP8_E4M3, True, 7, False, (3, 1, 32)),  # fp8 K/V: built
    (16, 4, B.UA_DTYPE_BF16, True, 4, False, (3, 1, 16)),    # 16-row blocks: the 16-row engine
    (32, 1, B.UA_DTYPE_BF16, True, 1, False, (3, 0, 32)),    # g = 32: 32-row blocks
    (16, 4, B.UA_DTYPE_BF16, True, 7, 256, (2, 0, 32)),      # 256 sequences: the grid fills
]


@pytest.mark.parametrize("i", range(len(QQ_D256_PLANS)))
def test_qq_bias_d256_keeps_off_the_unbuilt_engine(i):
    """At d = 256 with 16-bit K/V and the QQ bias, q-blocks of more than 16
    rows never take the 32-row stream-K engine (not built for that
    configuration): the batch takes the segmented split, or the 2D path once
    its grid fills the device; the other configurations keep the engine."""
    hq, hk, kvdt, qq, max_q, f3, (path, sk, bm) = QQ_D256_PLANS[i]
    n = 16
    if f3 not in (True, False):
        n, f3 = f3, False
    q_dtype = B.UA_DTYPE_F16 if kvdt == B.UA_DTYPE_F16 else B.UA_DTYPE_BF16
    flags = B.UA_FLAG_CAUSAL | (B.UA_FLAG_QQ_BIAS if qq else 0) | (B.UA_FLAG_FORCE_3D if f3 else 0)
    h = B.ua_create_problem(_desc(num_q_heads=hq, num_kv_heads=hk, head_dim=256, block_size=16,
                                  q_dtype=q_dtype, kv_dtype=kvdt, flags=flags, num_blocks=4096,
                                  max_num_seqs=256, max_blocks_per_seq=256, max_total_q=2048,
                                  max_seqlen_k=4096))
    try:
        plan = B.ua_query_plan(h, n, n * max_q, max_q, 4000)
    finally:
        B.ua_destroy_problem(h)
    assert (plan.path, plan.stream_k, plan.block_m) == (path, sk, bm)
    assert plan.class_split == 0


def test_segment_override_selects_the_segmented_split():
    plan, _ = _named_plan("decode_batch", split_segment_tiles=16)
    assert plan.path == 3 and plan.stream_k == 0 and plan.tiles_per_segment == 16
    assert plan.num_segments * 16 * plan.tile_n >= 8138
    assert list(plan.grid)[1:] == [8, plan.num_segments]
    with pytest.raises(B.UaError):
        B.ua_create_problem(_desc(split_segment_tiles=-1))


def test_forced_paths_and_geometry():
    plan, _ = _named_plan("long_prefill", B.UA_FLAG_FORCE_3D)
    assert plan.path == 3 and plan.waves == 4 and plan.block_q == 8 and plan.class_split == 0
    plan, _ = _named_plan("variant_mix", B.UA_FLAG_FORCE_2D)
    assert plan.path == 2 and plan.class_split == 0
    plan, _ = _named_plan("decode_batch", B.UA_FLAG_FORCE_2D)
    assert plan.path == 2 and plan.waves == 1 and plan.block_m == 32


def test_i64_addressing_reported_above_2gib():
    small, _ = _named_plan("decode_batch")
    assert small.use_i64_kv == 0
    h = B.ua_create_problem(_desc(num_blocks=600_000))  # 600K * 16 * 2 * 128 * 2 B > 2^31
    p = B.ua_query_plan(h, 2, 8, 4, 512)
    assert p.use_i64_kv == 1
    B.ua_destroy_problem(h)


def test_shape_rule_scales_with_the_compute_units():
    """[UA] section 6 states the 2D threshold in workgroups per compute unit
    (4 per CU): one 2528-query prefill chunk of 8192 keys at H_k = 8 has a
    640-workgroup 2D grid, which a part with half the CUs takes as it is,
    while the full MI355X (256 CUs, the default when no device is queried)
    cuts it into segments to fill its round."""
    kw = dict(num_q_heads=32, num_kv_heads=8, num_blocks=20000, max_num_seqs=64,
              max_blocks_per_seq=512, max_total_q=4096, max_seqlen_k=8192)
    for cus, path in ((128, 2), (256, 3), (0, 3)):
        h = B.ua_create_problem(_desc(num_cus=cus, **kw))
        try:
            plan = B.ua_query_plan(h, 1, 2528, 2528, 8192)
            assert plan.path == path and plan.stream_k == 0 and plan.waves == 4, (cus, plan.path)
        finally:
            B.ua_destroy_problem(h)
    with pytest.raises(B.UaError) as e:
        B.ua_create_problem(_desc(num_cus=-1))
    assert "num_cus" in B.ua_last_error()


def test_decode_batches_stream_at_any_size():
    """Decode-shaped batches (every q-block one wave) take the stream-K
    split whatever their count once their keys are not short; at or below
    512 keys a q-block has few tiles and the 2D path keeps them."""
    h = B.ua_create_problem(_desc(num_q_heads=32, num_kv_heads=8, num_blocks=80000,
                                  max_num_seqs=1024, max_blocks_per_seq=512, max_total_q=1024,
                                  max_seqlen_k=8192))
    try:
        for n, sk in ((64, 8138), (128, 8192), (512, 8192), (1024, 4096)):
            plan = B.ua_query_plan(h, n, n, 1, sk)
            assert (plan.path, plan.stream_k, plan.waves) == (3, 1, 1), (n, sk)
        plan = B.ua_query_plan(h, 512, 512, 1, 500)
        assert (plan.path, plan.stream_k) == (2, 0)
    finally:
        B.ua_destroy_problem(h)


def test_bf16_partials_halve_the_split_workspace():
    """UA_FLAG_BF16_PARTIALS stores the partial o in bf16: the workspace of
    the decode batch's segmented split (and of its stream-K slots) shrinks
    by (2 d + 8) / (4 d + 8) = 264 / 520 at d = 128."""
    kw = dict(num_q_heads=32, num_kv_heads=8, num_blocks=20000, max_num_seqs=64,
              max_blocks_per_seq=512, max_total_q=64, max_seqlen_k=8192, split_segment_tiles=16)
    sizes = []
    for extra in (0, B.UA_FLAG_BF16_PARTIALS):
        h = B.ua_create_problem(_desc(flags=B.UA_FLAG_CAUSAL | B.UA_FLAG_FORCE_3D | extra, **kw))
        try:
            assert B.ua_query_plan(h, 64, 64, 1, 8138).path == 3
            sizes.append(B.ua_workspace_size(h))
        finally:
            B.ua_destroy_problem(h)
    assert abs(sizes[1] / sizes[0] - 264 / 520) < 1e-3, sizes


MERGE_BAD = [
    (dict(num_sets=0), "num_sets"),
    (dict(num_sets=9), "num_sets"),
    (dict(partial_dtype=5), "partial_dtype"),
    (dict(head_dim=96), "head_dim"),
    (dict(o_dtype=B.UA_DTYPE_FP8_E4M3), "o_dtype"),
    (dict(o_stride_tok=100), "o_stride_tok"),
    (dict(o=8), "o must be"),
]


@pytest.mark.parametrize("i", range(len(MERGE_BAD)))
def test_merge_rejects_invalid_arguments(i):
    kw, text = MERGE_BAD[i]
    base = dict(num_sets=2, partial_dtype=B.UA_PARTIAL_F32, total_q=4, num_q_heads=8,
                head_dim=128, o_dtype=B.UA_DTYPE_BF16, o_stride_tok=1024, o=4096)
    base.update(kw)
    a = B.ua_merge_args_t(**base)
    for j in range(2):
        a.partial_o[j] = 8192
        a.partial_lse[j] = 8192
    with pytest.raises(B.UaError) as e:
        B.ua_merge(a, None)
    assert text in B.ua_last_error()


def test_merge_rejects_a_missing_set_and_partial_mode_needs_lse():
    a = B.ua_merge_args_t(num_sets=2, partial_dtype=B.UA_PARTIAL_F32, total_q=4, num_q_heads=8,
                          head_dim=128, o_dtype=B.UA_DTYPE_BF16, o_stride_tok=1024, o=4096)
    a.partial_o[0] = 8192
    a.partial_lse[0] = 8192
    with pytest.raises(B.UaError):
        B.ua_merge(a, None)
    assert "partial set 1" in B.ua_last_error()
    h = B.ua_create_problem(_desc())
    try:
        args = B.ua_run_args_t(q=16, k_cache=16, v_cache=16, o=None, block_table=16,
                               seq_lens=16, cu_seqlens_q=16, num_seqs=2, max_seqlen_q=4,
                               total_q=8, max_seqlen_k=512, block_table_stride=32,
                               q_stride_tok=8 * 128, o_stride_tok=8 * 128, partial_o=256)
        with pytest.raises(B.UaError):
            B.ua_run(h, args, None)
        assert "partial_lse" in B.ua_last_error()
    finally:
        B.ua_destroy_problem(h)


def test_ceiling_probe_library_loads_and_exports_its_probes():
    """The test-only ceiling probes (built by __graft_entry__.build) load on a
    host without a GPU; nothing is launched."""
    import ceilings
    L = ceilings.lib()
    for name in ("uac_stream_read", "uac_paged_read", "uac_issue_rate"):
        assert hasattr(L, name), name
