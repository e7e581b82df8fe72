"""Shared helpers of the GPU parity tests: run the HIP path through the C
boundary and compare with the fp64 oracle element by element."""
import numpy as np
import torch

import oracle
from varlen_attention_serving_amd import binding as B
from varlen_attention_serving_amd import device as D

# acceptance bar: bf16/fp16 outputs against the fp64 oracle
MAX_ABS = 2e-2
REL_RMS = 5e-3
# row LSE against the oracle's: the denominator sums 16-bit-rounded p, about
# 2^-9 relative
LSE_TOL = 4e-3


def say(msg):
    print(msg, flush=True)


# NaN bit patterns of the output types: O is filled with them before a run,
# so a row that no workgroup writes shows up as NaN
_NAN16 = {B.UA_DTYPE_BF16: 0x7FC0, B.UA_DTYPE_F16: 0x7E00}


def poison_output(batch):
    batch.o.fill_(_NAN16[batch.w.q_dtype])


def run_hip(w, extra_flags=0, batch=None, ua=None, repeat=1, split_segment_tiles=0, lse=False):
    """Run the HIP path on workload w; returns (O as float64 numpy, plan), and
    the row LSE [total_q, H_q] as a third item when `lse` is set.  O (and the
    LSE) start as NaN, and every element of O must come back finite: each
    row of the batch belongs to some workgroup's q-block."""
    if batch is None:
        batch = D.DeviceBatch(w)
    if ua is None:
        ua = D.UnifiedAttention(D.problem_desc(w, extra_flags,
                                               split_segment_tiles=split_segment_tiles))
    plan = ua.plan(w)
    lse_buf = batch.lse_buffer() if lse else None
    for _ in range(repeat):
        poison_output(batch)
        if lse_buf is not None:
            lse_buf.fill_(float("nan"))
        ua.run(batch, lse=lse_buf)
    torch.cuda.synchronize()
    finite = torch.isfinite(batch.output())
    if not bool(finite.all()):
        bad = torch.nonzero(~finite.all(dim=2))[:4].tolist()
        raise AssertionError(f"{w.name}: {int((~finite).sum())} output elements not written "
                             f"or not finite; first (token, head) {bad}")
    o = batch.output().float().cpu().numpy().astype(np.float64)
    if lse:
        return o, plan, lse_buf.cpu().numpy().astype(np.float64)
    return o, plan


def compare(o_gpu, o_ref, what=""):
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in the output"
    diff = o_gpu - o_ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    ref_norm = float(np.linalg.norm(o_ref))
    rel_rms = float(np.linalg.norm(diff) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(diff))
    say(f"  {what}: max_abs={max_abs:.3e} rel_rms={rel_rms:.3e}")
    assert max_abs <= MAX_ABS, f"{what}: max_abs {max_abs}"
    assert rel_rms <= REL_RMS, f"{what}: rel_rms {rel_rms}"
    return max_abs, rel_rms


def sample_rows(w, n_random=256, seed=0):
    """Random (token, head) rows plus the first and last token of every
    sequence for a spread of heads."""
    rng = np.random.default_rng(seed)
    total = w.total_q * w.num_q_heads
    rows = set(rng.integers(0, total, size=min(n_random, total)).tolist())
    heads = sorted({0, w.num_q_heads - 1, w.num_q_heads // 2})
    for s in range(w.num_seqs):
        lo, hi = int(w.cu_seqlens_q[s]), int(w.cu_seqlens_q[s + 1])
        if hi > lo:
            for t in {lo, hi - 1, (lo + hi) // 2}:
                for h in heads:
                    rows.add(t * w.num_q_heads + h)
    return np.array(sorted(rows), dtype=np.int64)


def compare_rows(o_gpu, w, rows, what=""):
    ref = oracle.rows(w, rows)
    flat = o_gpu.reshape(-1, w.head_dim)[rows]
    return compare(flat, ref, what)


def visible_counts(w, s):
    """Keys visible to each local query row of sequence s (causal / window)."""
    ql, sk = int(w.q_lens[s]), int(w.seq_lens[s])
    q_abs = sk - ql + np.arange(ql, dtype=np.int64)
    kmax = np.minimum(q_abs, sk - 1) if w.causal else np.full(ql, sk - 1)
    kmin = np.maximum(q_abs - w.window + 1, 0) if w.window > 0 else np.zeros(ql, np.int64)
    return np.maximum(kmax - kmin + 1, 0)


def full_rows(w, budget_flops=1.5e11, decode_rows=32):
    """Rows for a full-size check.  Sequences whose rows fit one single-wave
    q-block (q_len * g <= decode_rows) are compared on every (token, head).
    For the others every token is compared against m of the H_k kv heads,
    rotating with the token (m as large as the oracle budget allows, all H_k
    when it fits), with the query head rotating through the group:
    h = h_k * g + ((i + j) mod g) for local row i and pass j.  Every q-block
    of every kv head and every wave's rows are then visited."""
    g, hq, hk = w.group, w.num_q_heads, w.num_kv_heads
    rows = []
    long_cost = 0
    longs = []
    for s in range(w.num_seqs):
        lo, hi = int(w.cu_seqlens_q[s]), int(w.cu_seqlens_q[s + 1])
        if hi == lo:
            continue
        if (hi - lo) * g <= decode_rows:
            t = np.arange(lo, hi, dtype=np.int64)
            rows.append((t[:, None] * hq + np.arange(hq)[None, :]).reshape(-1))
        else:
            longs.append((s, lo, hi))
            long_cost += int(visible_counts(w, s).sum()) * 4 * w.head_dim
    m = hk if long_cost == 0 else int(max(1, min(hk, budget_flops // long_cost)))
    step = max(1, hk // m)
    for s, lo, hi in longs:
        i = np.arange(hi - lo, dtype=np.int64)
        for j in range(m):
            h_k = (i + j * step) % hk
            head = h_k * g + (i + j) % g
            rows.append((lo + i) * hq + head)
    rows = np.unique(np.concatenate(rows)) if rows else np.zeros(0, np.int64)
    return rows, m
