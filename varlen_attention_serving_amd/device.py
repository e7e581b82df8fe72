"""Device-memory plumbing for the C boundary: torch tensors hold the inputs,
outputs and workspace; ``UnifiedAttention`` owns a problem handle and calls
``ua_run`` on the current torch stream.  No arithmetic happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_TORCH_VIEW = {B.UA_DTYPE_BF16: torch.bfloat16, B.UA_DTYPE_F16: torch.float16}


def problem_desc(w, extra_flags: int = 0, max_total_q=None, max_seqlen_k=None,
                 max_num_seqs=None, split_segment_tiles: int = 0) -> B.ua_problem_desc_t:
    """Descriptor of workload ``w`` (a ``workloads.Workload``)."""
    flags = extra_flags
    if w.causal:
        flags |= B.UA_FLAG_CAUSAL
    if w.softcap > 0:
        flags |= B.UA_FLAG_SOFTCAP
    if w.use_alibi:
        flags |= B.UA_FLAG_ALIBI
    if w.window > 0:
        flags |= B.UA_FLAG_WINDOW
    if w.use_sinks:
        flags |= B.UA_FLAG_SINKS
    if getattr(w, "qq_bias", None) is not None:
        flags |= B.UA_FLAG_QQ_BIAS
    if getattr(w, "dense", False):
        flags |= B.UA_FLAG_DENSE_KV
    return B.ua_problem_desc_t(
        num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
        block_size=w.block_size, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, flags=flags,
        scale=w.scale, softcap=w.softcap, window=w.window, k_scale=w.k_scale, v_scale=w.v_scale,
        num_blocks=w.num_blocks,
        max_num_seqs=max(1, w.num_seqs if max_num_seqs is None else max_num_seqs),
        max_blocks_per_seq=int(w.block_table.shape[1]),
        max_total_q=max(1, w.total_q if max_total_q is None else max_total_q),
        max_seqlen_k=max(1, w.max_seqlen_k if max_seqlen_k is None else max_seqlen_k),
        split_segment_tiles=split_segment_tiles)


class DeviceBatch:
    """Device copies of one workload's inputs plus an output buffer."""

    def __init__(self, w, device="cuda"):
        dev = torch.device(device)
        self.w = w
        as16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        self.q = as16(w.q)
        if w.kv_dtype == B.UA_DTYPE_FP8_E4M3:
            self.k = torch.from_numpy(np.ascontiguousarray(w.k_cache)).to(dev)
            self.v = torch.from_numpy(np.ascontiguousarray(w.v_cache)).to(dev)
        else:
            self.k = as16(w.k_cache)
            self.v = as16(w.v_cache)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        self.dense = bool(getattr(w, "dense", False))
        # the dense layout is addressed by cu_seqlens_k alone: no table, no S_k array
        self.block_table = None if self.dense else i32(w.block_table)
        self.seq_lens = None if self.dense else i32(w.seq_lens)
        self.cu_seqlens_k = i32(w.cu_seqlens_k) if self.dense else None
        self.cu_seqlens_q = i32(w.cu_seqlens_q)
        f32 = lambda a: None if a is None else torch.from_numpy(
            np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        self.alibi_slopes = f32(w.alibi_slopes)
        self.sinks = f32(w.sinks)
        self.qq_bias = f32(getattr(w, "qq_bias", None))
        self.o = torch.zeros_like(self.q)

    def output(self) -> torch.Tensor:
        """O viewed in its storage dtype (bf16 / f16)."""
        return self.o.view(_TORCH_VIEW[self.w.q_dtype])

    def lse_buffer(self) -> torch.Tensor:
        """A float32 [total_q, H_q] buffer for the optional row LSE output."""
        if getattr(self, "lse", None) is None:
            self.lse = torch.full((self.w.total_q, self.w.num_q_heads), float("nan"),
                                  dtype=torch.float32, device=self.o.device)
        return self.lse

    def run_args(self, workspace=None, lse=None) -> B.ua_run_args_t:
        w = self.w
        ptr = lambda t: None if t is None else t.data_ptr()
        return B.ua_run_args_t(lse=ptr(lse),
            q=ptr(self.q), k_cache=ptr(self.k), v_cache=ptr(self.v), o=ptr(self.o),
            block_table=ptr(self.block_table), seq_lens=ptr(self.seq_lens),
            cu_seqlens_q=ptr(self.cu_seqlens_q), alibi_slopes=ptr(self.alibi_slopes),
            sinks=ptr(self.sinks),
            workspace=None if workspace is None else workspace.data_ptr(),
            workspace_bytes=0 if workspace is None else workspace.numel(),
            num_seqs=w.num_seqs, max_seqlen_q=w.max_seqlen_q, total_q=w.total_q,
            max_seqlen_k=w.max_seqlen_k,
            block_table_stride=0 if self.dense else int(w.block_table.shape[1]),
            cu_seqlens_k=ptr(self.cu_seqlens_k),
            q_stride_tok=w.num_q_heads * w.head_dim, o_stride_tok=w.num_q_heads * w.head_dim,
            qq_bias=ptr(self.qq_bias),
            qq_bias_stride=0 if self.qq_bias is None else int(self.qq_bias.shape[1]))


class UnifiedAttention:
    """A problem handle plus its workspace (allocated once, through torch)."""

    def __init__(self, desc: B.ua_problem_desc_t, device="cuda"):
        self.desc = desc
        self.handle = B.ua_create_problem(desc)
        n = B.ua_workspace_size(self.handle)
        self.workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
        if self.workspace.data_ptr() % 256:
            raise RuntimeError("workspace allocation is not 256-byte aligned")

    def plan(self, w) -> B.ua_plan_info_t:
        return B.ua_query_plan(self.handle, w.num_seqs, w.total_q, w.max_seqlen_q,
                               w.max_seqlen_k)

    def run(self, batch: DeviceBatch, stream=None, lse=None) -> None:
        s = torch.cuda.current_stream() if stream is None else stream
        B.ua_run(self.handle, batch.run_args(self.workspace, lse), s.cuda_stream)

    def close(self):
        if self.handle:
            B.ua_destroy_problem(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
