"""Test-side helpers that are independent of the oracle: library decoders of the
stored bits, a dense numpy gather of the paged cache, and a brute-force dense
attention (full score matrix, explicit mask matrix, sinks as an extra column)."""
import numpy as np
import torch

from varlen_attention_serving_amd import workloads as W


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Decode stored bits to float64 with torch / numpy conversions."""
    if dtype == W.DT_BF16:
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).double().numpy()
    if dtype == W.DT_F16:
        return np.ascontiguousarray(bits).view(np.float16).astype(np.float64)
    if dtype == W.DT_FP8_E4M3:
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).double().numpy()
    raise ValueError(dtype)


def dense_kv(w, s):
    """K, V of sequence s as dense float64 [S_k, H_k, d] (fp8 scaled)."""
    sk = int(w.seq_lens[s])
    pos = np.arange(sk)
    phys = w.block_table[s, pos // w.block_size]
    slot = pos % w.block_size
    k = decode(w.k_cache[phys, slot], w.kv_dtype)
    v = decode(w.v_cache[phys, slot], w.kv_dtype)
    if w.kv_dtype == W.DT_FP8_E4M3:
        k = k * w.k_scale
        v = v * w.v_scale
    return k, v


def brute_force(w, window_extra_key=0):
    """Dense float64 attention for every row of w; returns (O, LSE)."""
    g = w.group
    q_all = decode(w.q, w.q_dtype)
    out = np.zeros((w.total_q, w.num_q_heads, w.head_dim))
    lse = np.full((w.total_q, w.num_q_heads), -np.inf)
    for s in range(w.num_seqs):
        ql, sk = int(w.q_lens[s]), int(w.seq_lens[s])
        if ql == 0:
            continue
        t0 = int(w.cu_seqlens_q[s])
        k, v = dense_kv(w, s)
        ctx = sk - ql
        qpos = ctx + np.arange(ql)[:, None]          # [ql, 1]
        kpos = np.arange(sk)[None, :]                # [1, sk]
        allowed = np.ones((ql, sk), dtype=bool)
        if w.causal:
            allowed &= kpos <= qpos
        if w.window > 0:
            allowed &= kpos > qpos - w.window - window_extra_key
        for h in range(w.num_q_heads):
            hk = h // g
            qh = q_all[t0:t0 + ql, h, :]               # [ql, d]
            s_mat = w.scale * (qh @ k[:, hk, :].T)     # [ql, sk]
            if w.softcap > 0:
                s_mat = w.softcap * np.tanh(s_mat / w.softcap)
            if w.use_alibi:
                s_mat = s_mat + float(w.alibi_slopes[h]) * (kpos - ctx)
            if getattr(w, "qq_bias", None) is not None:
                # the query section: keys ctx .. S_k - 1, biased by bias[i, k - ctx]
                s_mat = s_mat.copy()
                s_mat[:, ctx:] += w.qq_bias[:ql, :ql].astype(np.float64)
            s_mat = np.where(allowed, s_mat, -np.inf)
            cols = [s_mat]
            if w.use_sinks:
                cols.append(np.full((ql, 1), float(w.sinks[h])))
            full = np.concatenate(cols, axis=1)
            m = full.max(axis=1, keepdims=True)
            m_safe = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(full - m_safe)
            z = e.sum(axis=1, keepdims=True)
            p = e[:, :sk] / np.where(z > 0, z, 1.0)
            has = allowed.any(axis=1)
            o = p @ v[:, hk, :]
            o[~has] = 0.0
            out[t0:t0 + ql, h, :] = o
            with np.errstate(divide="ignore"):
                l = (m_safe + np.log(z))[:, 0]
            l[~has & (not w.use_sinks)] = -np.inf
            if w.use_sinks:
                l[~has] = float(w.sinks[h])
            lse[t0:t0 + ql, h] = l
    return out, lse
