"""Softmax attention over paged KV (decode) and over the FP16 workspace (prefill).

The method reaches a result with a plain definition, so this is that
definition written out in float64:

  s_t  = sm_scale * sum_d q[h, d] * k[t, g, d]          (g = KV head of h)
  p_t  = exp(s_t - max s) / sum_u exp(s_u - max s)
  o[h] = sum_t p_t * v[t, g, :]
  lse  = max s + ln sum_u exp(s_u - max s)               (natural log)

Grouped-query attention: query head h reads KV head h // (Hq / Hkv).

Decode: [asym] "What changes in vLLM's prefill routing?" (decode prefix
reads persistent FP16 keys and FP8 values; value scales still apply in
attention) and [ekv] section 3.2 (TARGET and compact pages in one batch, both
produce the same output interface).  Reading taken: ``seq_lens[b]`` counts
the token being decoded, whose K/V is already in the cache; the query attends
to tokens [0, len).  A sequence of length 0 yields o = 0, lse = -inf.

Prefill: [asym] same section: fresh whole prompts with no cached prefix,
causal attention, no sliding window, sinks or soft cap, FP16 Q/K/V from the
workspace.  Reading taken: key j is visible to query i of the same prompt iff
j <= i (q_len == kv_len); ``causal = 0`` makes all of the prompt's keys
visible.  Each prompt's keys start at workspace row ``kv_start[p]``.
"""
import numpy as np

from .paged import sequence_kv


def attention_rows(q, K, V, sm_scale):
    """Attention of query rows q [Hq, D] over keys/values [n, Hkv, D] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hq, d = q.shape
    n, hkv, _ = K.shape
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    lse = np.full(hq, -np.inf, dtype=np.float64)
    if n == 0:
        return out, lse
    for h in range(hq):
        g = h // group
        s = sm_scale * (K[:, g, :] @ q[h])
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        out[h] = (e @ V[:, g, :]) / z
        lse[h] = m + np.log(z)
    return out, lse


def decode_attention(q, k_target, v_target, k_compact, v_compact, v_scale,
                     page_table, fidelity, seq_lens, sm_scale):
    """One query token per sequence over its paged KV.  Returns out [B, Hq, D], lse [B, Hq]."""
    B, hq, d = q.shape
    out = np.zeros((B, hq, d), dtype=np.float64)
    lse = np.full((B, hq), -np.inf, dtype=np.float64)
    for b in range(B):
        K, V = sequence_kv(k_target, v_target, k_compact, v_compact, v_scale,
                           page_table[b], fidelity[b], seq_lens[b])
        out[b], lse[b] = attention_rows(q[b], K, V, sm_scale)
    return out, lse


def prefill_attention(q, k, v, cu_seqlens_q, kv_start, causal, sm_scale, rows=None,
                      block=256):
    """Causal (or full) attention of packed prompts over workspace rows.

    q: [T, Hq, D]; k, v: [R, Hkv, D]; cu_seqlens_q: [n + 1]; kv_start: [n].
    ``rows`` optionally lists packed query rows to compute (others stay 0).
    Rows are independent, so they are evaluated ``block`` at a time with the
    same definition in matrix form (masked keys get probability 0).
    Returns out [T, Hq, D] float64 and lse [T, Hq].
    """
    q = np.asarray(q)
    T, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((T, hq, d), dtype=np.float64)
    lse = np.full((T, hq), -np.inf, dtype=np.float64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    wanted = None if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
    for p in range(cu.shape[0] - 1):
        start, end = int(cu[p]), int(cu[p + 1])
        L = end - start
        if L == 0:
            continue
        if wanted is None:
            local = np.arange(L)
        else:
            local = wanted[(wanted >= start) & (wanted < end)] - start
            if local.size == 0:
                continue
        k0 = int(kv_start[p])
        Kp = np.asarray(k[k0:k0 + L], dtype=np.float64)
        Vp = np.asarray(v[k0:k0 + L], dtype=np.float64)
        for b0 in range(0, local.size, block):
            i = local[b0:b0 + block]                      # query positions in the prompt
            n = int(i.max()) + 1 if causal else L         # keys any row of the block can see
            Qb = np.asarray(q[start + i], dtype=np.float64)   # [r, Hq, D]
            visible = (np.arange(n)[None, :] <= i[:, None]) if causal else \
                np.ones((i.size, n), dtype=bool)
            for h in range(hq):
                g = h // group
                s = sm_scale * (Qb[:, h, :] @ Kp[:n, g, :].T)    # [r, n]
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                out[start + i, h] = (e @ Vp[:n, g, :]) / z
                lse[start + i, h] = (m + np.log(z))[:, 0]
    return out, lse
