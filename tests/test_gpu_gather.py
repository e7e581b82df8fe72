"""The K/V tile gathers, bit for bit: the kernels' own gather routines (the
LDS ring's copies and the register-staged loader) run through a test-only
probe that copies each gathered tile out of LDS, and every visited key must
hold exactly the stored cache row of block_table[s][k >> log2 b], slot
k & (b - 1), head h_k ([UA] §0's layout).  Keys past S_k hold slot S_k - 1's
row on both paths (finite data whose scores the kernels mask)."""
import numpy as np
import pytest
import torch

import gather_probe as P
from gpu_common import say
from varlen_attention_serving_amd import device as D
from varlen_attention_serving_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _tiles(w, limit=None, seed=0):
    """Every (sequence, kv-head, 32-key tile) below S_k, or a seeded sample."""
    t = [(s, h, i) for s in range(w.num_seqs) for h in range(w.num_kv_heads)
         for i in range((int(w.seq_lens[s]) + 31) // 32)]
    t = np.array(t, dtype=np.int32).reshape(-1, 3)
    if limit is not None and len(t) > limit:
        t = t[np.random.default_rng(seed).choice(len(t), limit, replace=False)]
    return t


def _host_rows(w, tiles, cache, past_end):
    """Host gather: [n, 32, d] rows of `cache` (already in 16-bit bits)."""
    b = w.block_size
    out = np.zeros((len(tiles), 32, w.head_dim), dtype=np.int16)
    for n, (s, h, t) in enumerate(tiles):
        s_k = int(w.seq_lens[s])
        for r in range(32):
            k = 32 * int(t) + r
            if k >= s_k:
                if past_end == "zero":
                    continue
                k = s_k - 1
            out[n, r] = cache[w.block_table[s, k // b], k % b, h]
    return out


def _as16(w, cache, fp8_to):
    if fp8_to == P.TO_16BIT:
        return np.ascontiguousarray(cache).view(np.int16)
    t = torch.from_numpy(np.ascontiguousarray(cache)).view(torch.float8_e4m3fn)
    t = t.to(torch.bfloat16 if fp8_to == P.FP8_TO_BF16 else torch.float16)
    return t.view(torch.int16).numpy()


def _check(w, path, waves=4, fp8_to=P.TO_16BIT, limit=None, what=""):
    batch = D.DeviceBatch(w)
    tiles = _tiles(w, limit)
    say(f"[gpu] gather {what}: path={path} waves={waves} fp8_to={fp8_to} tiles={len(tiles)}")
    gk, gv = P.gather(batch, torch.from_numpy(tiles).cuda(), path, waves, fp8_to)
    past = "last"
    for name, got, cache in (("K", gk, w.k_cache), ("V", gv, w.v_cache)):
        want = _host_rows(w, tiles, _as16(w, cache, fp8_to), past)
        got = got.cpu().numpy()
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{what} {name}: {len(bad)} mismatching elements, first {bad[:3]}"


RING_CASES = [(64, 8), (64, 16), (128, 4), (128, 16), (128, 32), (64, 64), (256, 2), (256, 16),
              (256, 64)]


@pytest.mark.parametrize("d,b", RING_CASES)
def test_ring_gather_is_bit_exact(d, b):
    w = W.random_small(700 + d + b, num_seqs=6, max_q=8, max_k=400, num_q_heads=8,
                       num_kv_heads=4, head_dim=d, block_size=b)
    _check(w, P.RING, what=f"ring d={d} b={b}")


REG_CASES = [(1, 64, 16, P.TO_16BIT), (4, 64, 1, P.TO_16BIT), (4, 128, 4, P.TO_16BIT),
             (1, 256, 64, P.TO_16BIT), (4, 256, 32, P.TO_16BIT),
             (1, 64, 16, P.FP8_TO_BF16), (1, 128, 32, P.FP8_TO_F16),
             (4, 128, 16, P.FP8_TO_BF16), (4, 256, 64, P.FP8_TO_F16)]


@pytest.mark.parametrize("i", range(len(REG_CASES)))
def test_register_gather_is_bit_exact(i):
    waves, d, b, fp8_to = REG_CASES[i]
    kw = dict(kv_dtype=W.DT_FP8_E4M3) if fp8_to != P.TO_16BIT else {}
    if fp8_to == P.FP8_TO_F16:
        kw["q_dtype"] = W.DT_F16
    w = W.random_small(800 + i, num_seqs=5, max_q=8, max_k=300, num_q_heads=4, num_kv_heads=2,
                       head_dim=d, block_size=b, **kw)
    _check(w, P.REGISTERS, waves, fp8_to, what=f"registers waves={waves} d={d} b={b}")


def test_ring_gather_full_size_sample():
    """The long-prefill pool (64-token blocks) at full size, 3000 sampled tiles."""
    w = W.NAMED["long_prefill"]()
    _check(w, P.RING, limit=3000, what="long_prefill sample")


LOADER16_CASES = [
    # (block size, fp8_to): the 16-row engine (d = 256) reads K straight into
    # its MFMA operand registers and V rows into padded LDS; blocks of 16 keys
    # and more take each V row's block id from its K half-tile (BIG), smaller
    # blocks read one id per V row
    (2, P.TO_16BIT), (8, P.TO_16BIT), (16, P.TO_16BIT), (64, P.TO_16BIT),
    (2, P.FP8_TO_BF16), (16, P.FP8_TO_BF16), (64, P.FP8_TO_F16), (4, P.FP8_TO_F16),
    (32, P.FP8_TO_F16),
]


@pytest.mark.parametrize("i", range(len(LOADER16_CASES)))
def test_loader16_gather_is_bit_exact(i):
    """Every tile below S_k of a ragged batch (lengths that end inside a
    half-tile, on a half-tile boundary and inside a block), including the
    clamp of keys past S_k to slot S_k - 1."""
    b, fp8_to = LOADER16_CASES[i]
    kw = dict(kv_dtype=W.DT_FP8_E4M3) if fp8_to != P.TO_16BIT else {}
    if fp8_to == P.FP8_TO_F16:
        kw["q_dtype"] = W.DT_F16
    rng = np.random.default_rng(900 + i)
    sk = np.concatenate([[1, 15, 16, 17, 31, 32, 33], rng.integers(1, 300, size=4)])
    w = W.build(f"loader16_{b}_{fp8_to}", 900 + i, np.ones(sk.size), sk, num_q_heads=8,
                num_kv_heads=4, head_dim=256, block_size=b, rng=rng, **kw)
    _check(w, P.LOADER16, 1, fp8_to, what=f"loader16 b={b}")


def test_transposing_lds_read_lane_map():
    """ds_read_b64_tr_b16 over all 64 lanes ('Replace the per-MFMA V transpose
    with CDNA4's transposing LDS read', architecture notes): lane 16 g + 4 a + b
    receives element b of what lanes 16 g + 4 j + a (j = 0..3) address, i.e.
    out(16g+4a+b)[j] = in(16g+4j+a)[b].  Checked for the kernels' own lane
    addresses (the padded 32-row and 16-row V tiles, the swizzled ring tile
    inside its 4096-element window) and for random addresses."""
    lanes = np.arange(64)
    g16, a4, b4 = lanes >> 4, (lanes & 15) >> 2, lanes & 3
    patterns = {
        # padded 32-row tile at d = 64 (row stride 64 + 32 elements)
        "padded32": (4 * (g16 >> 1) + a4) * (64 + 32) + 16 * (g16 & 1) + 4 * b4,
        # the 16-row engine's V tile at d = 256 (row stride 256 + 16), first d block
        "padded16": (4 * g16 + a4) * (256 + 16) + 4 * b4,
        # the swizzled ring tile at d = 64: row base, column half and chunk swizzle
        "swizzled": (4 * (g16 >> 1) + a4) * 64 + 8 * (2 * (g16 & 1) + (b4 >> 1)) + 4 * (b4 & 1),
        "random": 4 * np.random.default_rng(11).integers(0, 4096 // 4, size=64),
    }
    for name, addr in patterns.items():
        addr = np.asarray(addr, dtype=np.int64)
        assert np.all(addr % 4 == 0) and np.all(addr >= 0) and np.all(addr + 3 < 4096), name
        got = P.read_tr(torch.from_numpy(addr.astype(np.int32)).cuda()).astype(np.int64)
        want = np.empty((64, 4), dtype=np.int64)
        for lane in range(64):
            g, a, b = lane >> 4, (lane & 15) >> 2, lane & 3
            for j in range(4):
                want[lane, j] = addr[16 * g + 4 * j + a] + b
        say(f"[gpu] ds_read_b64_tr_b16 lane map, {name} addresses")
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name}: lanes {bad[:4].tolist()} differ"
    # the page's lane-0 figure: lanes 4 j read row j of a matrix of 64-element
    # rows (lanes 16 g + 4 j + a at row j, column 16 g + 4 a), so lane 0
    # receives {0, 64, 128, 192} where a plain 8-byte read gives its own row
    rows = P.read_tr(torch.from_numpy((64 * ((lanes & 15) >> 2) + 16 * (lanes >> 4) +
                                       4 * (lanes & 3)).astype(np.int32)).cuda())
    assert rows[0].tolist() == [0, 64, 128, 192]


def test_fp8_conversion_of_every_code():
    """[UA] section 7.3 (OCP e4m3fn K/V dequantised to 16 bits): the kernels'
    conversion of each of the 256 codes equals torch's float8_e4m3fn cast to
    bf16 and to f16 bit for bit (both NaN codes give NaN), and the oracle's
    exact decoder of the code."""
    import oracle
    got_bf, got_h = P.fp8_codes()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    want_bf = codes.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want_h = codes.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    vals_bf = torch.from_numpy(got_bf.view(np.int16)).view(torch.bfloat16).double().numpy()
    vals_h = got_h.view(np.float16).astype(np.float64)
    for c in range(256):
        ref = oracle.decode(W.DT_FP8_E4M3, c)
        if np.isnan(ref):
            assert np.isnan(vals_bf[c]) and np.isnan(vals_h[c]), c
            continue
        assert got_bf[c] == want_bf[c] and got_h[c] == want_h[c], (c, got_bf[c], want_bf[c])
        assert vals_bf[c] == ref and vals_h[c] == ref, (c, vals_bf[c], vals_h[c], ref)
    say("[gpu] fp8: 256 codes bit-exact against torch and the oracle decoder")
