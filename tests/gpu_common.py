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


def say(msg):
    print(msg, flush=True)


def run_hip(w, extra_flags=0, batch=None, ua=None, repeat=1, split_segment_tiles=0, lse=False):
    """Run the HIP path on workload w; returns (O as float64 numpy, plan), and
    the row LSE [total_q, H_q] as a third item when `lse` is set."""
    if batch is None:
        batch = D.DeviceBatch(w)
    if ua is None:
        ua = D.UnifiedAttention(D.problem_desc(w, extra_flags,
                                               split_segment_tiles=split_segment_tiles))
    plan = ua.plan(w)
    lse_buf = batch.lse_buffer() if lse else None
    for _ in range(repeat):
        ua.run(batch, lse=lse_buf)
    torch.cuda.synchronize()
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
