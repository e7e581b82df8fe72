"""Seeded synthetic inputs for unified paged attention.

This module only draws and stores inputs: sequence lengths, a randomly permuted
paged KV pool with its block table, Q/K/V values and the per-head ALiBi slopes
and sink logits.  It holds none of the attention arithmetic, so both the HIP
path and the fp64 oracle can consume the same bytes.

Layouts follow the unified paged attention page ("Unified paged attention on
gfx950, from the math up", section 0 Notation): Q and O are packed varlen
[total_q, H_q, d]; the K and V caches are [num_blocks, block_size, H_k, d];
the block table maps a sequence's logical block to a physical block;
``cu_seqlens_q`` packs the ragged query rows; ``seq_lens`` holds S_k per
sequence (query rows are the last ``q_len`` key positions, ctx = S_k - q_len).

Recipe (same for every workload):
  * RNG is ``numpy.random.default_rng(seed)``; draw order is lengths ->
    physical permutation -> Q -> K -> V -> sinks (slopes are deterministic).
  * Values are N(0, 1) float32, rounded to nearest-even into the storage type
    (bf16 / fp16); fp8 K/V are e4m3fn codes of x / scale with a per-tensor
    scale = amax / 448 (rounded to fp16 first, then to e4m3fn).  Large
    tensors are drawn in 16M-value chunks, chunk i from child i of one seed
    drawn from the workload's generator (thread-count independent).
  * The pool holds sum(ceil(S_k / b)) used blocks plus max(16, 1%) slack
    blocks, in a random physical order.  Unused blocks and the tail slots of
    each sequence's last block are filled with NaN; unused block-table
    entries are -1.  A correct kernel never lets those reach O.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np

# Storage-type codes shared with the C boundary (plain integers, no arithmetic).
DT_BF16, DT_F16, DT_FP8_E4M3 = 0, 1, 2
DTYPE_NAMES = {DT_BF16: "bf16", DT_F16: "f16", DT_FP8_E4M3: "fp8_e4m3"}

_NAN_BITS = {DT_BF16: 0x7FC0, DT_F16: 0x7E00, DT_FP8_E4M3: 0x7F}
_CHUNK = 1 << 24  # elements per RNG draw, bounds peak host memory


@dataclasses.dataclass
class Workload:
    """One batch of paged attention inputs (host copies, raw storage bits)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: int
    kv_dtype: int
    causal: bool
    softcap: float           # 0 = off
    window: int              # 0 = off; otherwise keep the last `window` keys
    use_alibi: bool
    use_sinks: bool
    scale: float
    q_lens: np.ndarray       # int32 [N]
    seq_lens: np.ndarray     # int32 [N]   (S_k)
    cu_seqlens_q: np.ndarray  # int32 [N+1]
    block_table: np.ndarray  # int32 [N, max_blocks_per_seq], -1 where unused
    num_blocks: int
    q: np.ndarray            # uint16 [T_q, H_q, d] (bf16 / fp16 bits)
    k_cache: np.ndarray      # uint16 or uint8 [num_blocks, b, H_k, d]
    v_cache: np.ndarray
    alibi_slopes: Optional[np.ndarray]  # float32 [H_q] or None
    sinks: Optional[np.ndarray]         # float32 [H_q] or None
    k_scale: float = 1.0
    v_scale: float = 1.0
    qq_bias: Optional[np.ndarray] = None  # float32 [max_q, max_q] query-section bias, or None
    dense: bool = False                  # keys contiguous per sequence (block size 1, identity)

    @property
    def cu_seqlens_k(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.seq_lens)
        return cu

    @property
    def num_seqs(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def token_seq(self) -> np.ndarray:
        """Sequence index of each packed query token."""
        return np.repeat(np.arange(self.num_seqs, dtype=np.int64), self.q_lens)

    def select(self, seqs, name: Optional[str] = None) -> "Workload":
        """The batch of sequences ``seqs`` alone (same cache pool, same values;
        queries repacked in the given order).  Paged layouts only."""
        if self.dense:
            raise ValueError("select() needs a paged workload")
        idx = np.asarray(seqs, dtype=np.int64)
        ql = self.q_lens[idx].astype(np.int32)
        cu = np.zeros(len(idx) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(ql)
        parts = [self.q[self.cu_seqlens_q[s]:self.cu_seqlens_q[s + 1]] for s in idx]
        q = np.concatenate(parts) if parts else self.q[:0]
        return dataclasses.replace(
            self, name=name or f"{self.name}[{len(idx)} seqs]", q_lens=ql,
            seq_lens=self.seq_lens[idx].astype(np.int32), cu_seqlens_q=cu,
            block_table=self.block_table[idx].copy(), q=q)


# ----------------------------------------------------------------------------
# storage-type rounding (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) via torch's cast."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


_E4M3_LUT = None


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn codes: round to fp16 first (nearest-even), then to
    the nearest e4m3fn value (nearest-even, saturating at +-448) through a
    65536-entry table built once with torch's float8 cast."""
    global _E4M3_LUT
    if _E4M3_LUT is None:
        import torch
        halves = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
        halves = np.clip(np.nan_to_num(halves, nan=0.0), -448.0, 448.0)
        _E4M3_LUT = torch.from_numpy(halves).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    h = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0).astype(np.float16)
    return _E4M3_LUT[h.view(np.uint16)]


def _store(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == DT_BF16:
        return f32_to_bf16_bits(x)
    if dtype == DT_F16:
        return f32_to_f16_bits(x)
    raise ValueError(dtype)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _parallel_normal(rng: np.random.Generator, n: int, out: np.ndarray, convert) -> None:
    """Fill out[0:n] with convert(N(0,1) float32 draws).  Chunk i draws from its
    own child of one seed taken from ``rng``, so the values do not depend on
    the number of threads."""
    chunks = (n + _CHUNK - 1) // _CHUNK
    seeds = np.random.SeedSequence(int(rng.integers(0, 2**63))).spawn(max(chunks, 1))

    def work(i):
        s = i * _CHUNK
        e = min(n, s + _CHUNK)
        x = np.random.default_rng(seeds[i]).standard_normal(e - s, dtype=np.float32)
        out[s:e] = convert(x)

    with cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(chunks)))


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _parallel_normal(rng, n, out, lambda x: x)
    return out.reshape(shape)


def _normal_stored(rng, shape, dtype) -> np.ndarray:
    """N(0,1) drawn chunk by chunk straight into the 16-bit storage type."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _parallel_normal(rng, n, out, lambda x: _store(x, dtype))
    return out.reshape(shape)


def _amax(x: np.ndarray) -> float:
    flat = x.reshape(-1)
    spans = [(s, min(flat.size, s + _CHUNK)) for s in range(0, flat.size, _CHUNK)]
    with cf.ThreadPoolExecutor(_threads()) as ex:
        return max([0.0] + list(ex.map(lambda se: float(np.abs(flat[se[0]:se[1]]).max()), spans)))


def _encode_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    flat = x.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint8)
    inv = np.float32(scale)

    def work(se):
        out[se[0]:se[1]] = f32_to_e4m3_codes(flat[se[0]:se[1]] / inv)

    with cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, [(s, min(flat.size, s + _CHUNK)) for s in range(0, flat.size, _CHUNK)]))
    return out.reshape(x.shape)


def alibi_slopes(num_q_heads: int) -> np.ndarray:
    """Geometric ALiBi slopes 2^(-8 h / H_q) for h = 1 .. H_q."""
    h = np.arange(1, num_q_heads + 1, dtype=np.float64)
    return np.exp2(-8.0 * h / num_q_heads).astype(np.float32)


# ----------------------------------------------------------------------------
# generic builder
# ----------------------------------------------------------------------------

def build(name: str, seed: int, q_lens, seq_lens, *, num_q_heads: int, num_kv_heads: int,
          head_dim: int, block_size: int, q_dtype: int = DT_BF16, kv_dtype: int = DT_BF16,
          causal: bool = True, softcap: float = 0.0, window: int = 0, use_alibi: bool = False,
          use_sinks: bool = False, scale: Optional[float] = None, num_blocks: Optional[int] = None,
          rng: Optional[np.random.Generator] = None, poison: bool = True,
          table_slack_cols: int = 0, use_qq_bias: bool = False, dense: bool = False) -> Workload:
    """Draw one workload.  ``q_lens``/``seq_lens`` are already drawn by the caller
    (from ``rng`` when random) so the lengths come first in the draw order.
    ``dense`` lays every sequence's keys out contiguously, in sequence order
    (block size 1, identity table): the dense K/V layout [total_k, H_k, d]."""
    if rng is None:
        rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if q_lens.shape != seq_lens.shape:
        raise ValueError("q_lens and seq_lens differ in length")
    if np.any(q_lens > seq_lens) or np.any(q_lens < 0):
        raise ValueError("need 0 <= q_len <= S_k")
    n = q_lens.shape[0]
    b = block_size
    nb_seq = (seq_lens.astype(np.int64) + b - 1) // b
    used = int(nb_seq.sum())
    if num_blocks is None:
        num_blocks = used + max(16, (used + 99) // 100)
    if num_blocks < used:
        raise ValueError("pool smaller than the blocks in use")
    max_blocks = int(nb_seq.max()) + table_slack_cols if n else 1
    max_blocks = max(max_blocks, 1)

    if dense and b != 1:
        raise ValueError("a dense layout has block size 1")
    perm = (np.arange(num_blocks) if dense else rng.permutation(num_blocks)).astype(np.int32)
    block_table = np.full((n, max_blocks), -1, dtype=np.int32)
    off = 0
    for s in range(n):
        k = int(nb_seq[s])
        block_table[s, :k] = perm[off:off + k]
        off += k

    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    t_q = int(cu[-1])

    q = _normal_stored(rng, (t_q, num_q_heads, head_dim), q_dtype)
    cache_shape = (num_blocks, b, num_kv_heads, head_dim)
    k_scale = v_scale = 1.0
    if kv_dtype == DT_FP8_E4M3:
        kf = _normal(rng, cache_shape)
        vf = _normal(rng, cache_shape)
        # per-tensor scales: amax over the pool, kept exactly representable in f32
        k_scale = float(np.float32(_amax(kf) / 448.0))
        v_scale = float(np.float32(_amax(vf) / 448.0))
        k_cache = _encode_e4m3(kf, k_scale)
        del kf
        v_cache = _encode_e4m3(vf, v_scale)
        del vf
    else:
        k_cache = _normal_stored(rng, cache_shape, kv_dtype)
        v_cache = _normal_stored(rng, cache_shape, kv_dtype)

    slopes = alibi_slopes(num_q_heads) if use_alibi else None
    sinks = rng.standard_normal(num_q_heads, dtype=np.float32) if use_sinks else None
    # one query-section bias matrix for every head and sequence, drawn last
    mq = max(1, int(np.max(q_lens)) if len(q_lens) else 1)
    qq_bias = rng.standard_normal((mq, mq), dtype=np.float32) if use_qq_bias else None

    if poison:
        nan = _NAN_BITS[kv_dtype]
        in_use = np.zeros(num_blocks, dtype=bool)
        for s in range(n):
            k = int(nb_seq[s])
            in_use[block_table[s, :k]] = True
            tail = int(seq_lens[s]) - (k - 1) * b if k else b
            if k and tail < b:
                last = block_table[s, k - 1]
                k_cache[last, tail:] = nan
                v_cache[last, tail:] = nan
        k_cache[~in_use] = nan
        v_cache[~in_use] = nan

    return Workload(
        name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=b, q_dtype=q_dtype, kv_dtype=kv_dtype, causal=causal, softcap=float(softcap),
        window=int(window), use_alibi=use_alibi, use_sinks=use_sinks,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
        q_lens=q_lens, seq_lens=seq_lens, cu_seqlens_q=cu, block_table=block_table,
        num_blocks=num_blocks, q=q, k_cache=k_cache, v_cache=v_cache, alibi_slopes=slopes,
        sinks=sinks, k_scale=k_scale, v_scale=v_scale, qq_bias=qq_bias, dense=dense)



def to_dense(w: Workload) -> Workload:
    """The same batch with its K/V rows packed per sequence (the dense layout):
    row cu_seqlens_k[s] + k holds the cached row of key k.  Pure data movement;
    the slack rows past the last sequence are NaN."""
    if w.dense:
        return w
    n, b = w.num_seqs, w.block_size
    cu_k = w.cu_seqlens_k
    total = int(cu_k[-1])
    rows = total + 16
    shape = (rows, 1) + w.k_cache.shape[2:]
    nan = _NAN_BITS[w.kv_dtype]
    k = np.full(shape, nan, dtype=w.k_cache.dtype)
    v = np.full(shape, nan, dtype=w.v_cache.dtype)
    table = np.full((n, max(1, int(w.seq_lens.max()) if n else 1)), -1, dtype=np.int32)
    for s in range(n):
        sk = int(w.seq_lens[s])
        key = np.arange(sk)
        phys = w.block_table[s, key // b]
        k[cu_k[s]:cu_k[s] + sk, 0] = w.k_cache[phys, key % b]
        v[cu_k[s]:cu_k[s] + sk, 0] = w.v_cache[phys, key % b]
        table[s, :sk] = cu_k[s] + key
    return Workload(**{**w.__dict__, "name": w.name + "_dense", "block_size": 1,
                       "num_blocks": rows, "block_table": table, "k_cache": k, "v_cache": v,
                       "dense": True})


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

def _spec_tiny_varlen(seed):
    """4 sequences, q_lens {1,1,3,8}, S_k {17,40,64,100}, H_q=4, H_k=2, d=64,
    b=16, a 32-block pool, bf16, causal."""
    return dict(q_lens=[1, 1, 3, 8], seq_lens=[17, 40, 64, 100], rng=None,
                kw=dict(num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                        num_blocks=32))


def _spec_decode_batch(seed):
    """64 decode sequences, S_k ~ U{512..8192}, H_q=32, H_k=8, d=128, b=16, bf16, causal."""
    rng = np.random.default_rng(seed)
    sk = rng.integers(512, 8192, size=64, endpoint=True)
    return dict(q_lens=np.ones(64, np.int32), seq_lens=sk, rng=rng,
                kw=dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16))


def _spec_decode_large(seed):
    """256 decode sequences, S_k ~ U{512..8192}, H_q=32, H_k=8, d=128, b=16, bf16,
    causal: the decode batch's shape at a serving batch four times larger."""
    rng = np.random.default_rng(seed)
    sk = rng.integers(512, 8192, size=256, endpoint=True)
    return dict(q_lens=np.ones(256, np.int32), seq_lens=sk, rng=rng,
                kw=dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16))


def _spec_chunked_prefill_mix(seed):
    """32 decode sequences (S_k ~ U{1024..8192}) then 4 chunks of 512 queries with
    ctx ~ U{2048..6144}; H_q=32, H_k=8, d=128, b=32, bf16, causal, softcap 50,
    window 4096."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(1024, 8192, size=32, endpoint=True)
    ctx = rng.integers(2048, 6144, size=4, endpoint=True)
    return dict(q_lens=np.concatenate([np.ones(32, np.int64), np.full(4, 512)]),
                seq_lens=np.concatenate([dec, ctx + 512]), rng=rng,
                kw=dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=32,
                        softcap=50.0, window=4096))


def _spec_long_prefill(seed):
    """1 sequence S_q=S_k=8192 plus 4 of 2048; H_q=128, H_k=8, d=128, b=64, bf16, causal."""
    lens = [8192, 2048, 2048, 2048, 2048]
    return dict(q_lens=lens, seq_lens=lens, rng=None,
                kw=dict(num_q_heads=128, num_kv_heads=8, head_dim=128, block_size=64))


def _spec_variant_mix(seed):
    """128 decode sequences (S_k ~ U{1024..16384}) plus 2 prefill sequences of 1024;
    H_q=16, H_k=2, d=256, b=64; fp16 Q, fp8-e4m3 K/V with per-tensor scales;
    ALiBi, per-head sinks, window 2048, causal, tau = 1/16."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(1024, 16384, size=128, endpoint=True)
    return dict(q_lens=np.concatenate([np.ones(128, np.int64), np.full(2, 1024)]),
                seq_lens=np.concatenate([dec, np.full(2, 1024)]), rng=rng,
                kw=dict(num_q_heads=16, num_kv_heads=2, head_dim=256, block_size=64,
                        q_dtype=DT_F16, kv_dtype=DT_FP8_E4M3, window=2048, use_alibi=True,
                        use_sinks=True, scale=1.0 / 16.0))


def _spec_dense_prefill(seed):
    """The dense sibling's shape: 1 sequence S_q = S_k = 8192, H_q=128, H_k=8,
    d=128, bf16, causal, K/V packed per sequence (no block table)."""
    return dict(q_lens=[8192], seq_lens=[8192], rng=None,
                kw=dict(num_q_heads=128, num_kv_heads=8, head_dim=128, block_size=1,
                        dense=True))


def _spec_mha_prefill(seed):
    """The transposed-V-read benchmark shape: 1 sequence S_q = S_k = 4096, MHA
    H_q = H_k = 32, d=128, bf16, not causal, K/V packed per sequence."""
    return dict(q_lens=[4096], seq_lens=[4096], rng=None,
                kw=dict(num_q_heads=32, num_kv_heads=32, head_dim=128, block_size=1,
                        causal=False, dense=True))


def _spec_d256_prefill(seed):
    """Causal prefill at head dim 256: 1 sequence S_q = S_k = 8192 plus 4 of
    2048, H_q=16, H_k=8 (g=2), d=256, b=64, bf16, no other flags."""
    lens = [8192, 2048, 2048, 2048, 2048]
    return dict(q_lens=lens, seq_lens=lens, rng=None,
                kw=dict(num_q_heads=16, num_kv_heads=8, head_dim=256, block_size=64))


NAMED_SPECS = {
    "tiny_varlen": (1, _spec_tiny_varlen),
    "decode_batch": (2, _spec_decode_batch),
    "chunked_prefill_mix": (3, _spec_chunked_prefill_mix),
    "long_prefill": (4, _spec_long_prefill),
    "variant_mix": (5, _spec_variant_mix),
    "dense_prefill": (6, _spec_dense_prefill),
    "mha_prefill": (7, _spec_mha_prefill),
    "d256_prefill": (8, _spec_d256_prefill),
    "decode_large": (9, _spec_decode_large),
}


def named_spec(name: str, seed: Optional[int] = None) -> dict:
    """Lengths and parameters of a named workload, without drawing any values."""
    default_seed, fn = NAMED_SPECS[name]
    return fn(default_seed if seed is None else seed)


def named(name: str, seed: Optional[int] = None) -> Workload:
    default_seed, fn = NAMED_SPECS[name]
    seed = default_seed if seed is None else seed
    sp = fn(seed)
    return build(name, seed, sp["q_lens"], sp["seq_lens"], rng=sp["rng"], **sp["kw"])


def tiny_varlen(seed: int = 1) -> Workload:
    return named("tiny_varlen", seed)


def decode_batch(seed: int = 2) -> Workload:
    return named("decode_batch", seed)


def chunked_prefill_mix(seed: int = 3) -> Workload:
    return named("chunked_prefill_mix", seed)


def long_prefill(seed: int = 4) -> Workload:
    return named("long_prefill", seed)


def variant_mix(seed: int = 5) -> Workload:
    return named("variant_mix", seed)


NAMED = {
    "tiny_varlen": tiny_varlen,
    "decode_batch": decode_batch,
    "chunked_prefill_mix": chunked_prefill_mix,
    "long_prefill": long_prefill,
    "variant_mix": variant_mix,
    "dense_prefill": lambda seed=6: named("dense_prefill", seed),
    "mha_prefill": lambda seed=7: named("mha_prefill", seed),
    "d256_prefill": lambda seed=8: named("d256_prefill", seed),
    "decode_large": lambda seed=9: named("decode_large", seed),
}


def random_small(seed: int, *, num_seqs: int = 3, max_q: int = 40, max_k: int = 130,
                 num_q_heads: int = 4, num_kv_heads: int = 2, head_dim: int = 64,
                 block_size: int = 16, **kw) -> Workload:
    """A small ragged batch (oracle finishes in well under a second)."""
    rng = np.random.default_rng(seed)
    sk = rng.integers(1, max_k, size=num_seqs, endpoint=True)
    ql = np.minimum(sk, rng.integers(1, max_q, size=num_seqs, endpoint=True))
    return build(f"random_small_{seed}", seed, ql, sk, num_q_heads=num_q_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                 rng=rng, **kw)
