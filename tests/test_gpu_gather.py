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
