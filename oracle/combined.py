"""CPU fp64 oracle for attention with variable sequence lengths, grouped key/value heads and
dropout on the probabilities, together (any subset of the three).

TEST INFRASTRUCTURE ONLY (like oracle/attention.py): nothing in the product path may import,
call or execute this module; it shares no code with the HIP kernels.

Each part follows the reading already fixed for it on its own:
  * variable lengths (oracle.attention.forward_varlen): sequence b is the single-sequence
    definition of [MW] "Attention'ın Cebiri" on its first seq_lens_q[b] query rows and first
    seq_lens_k[b] keys of the padded tensors, with the causal mask of [MW] "Maskeleme ve Dropout"
    aligned per sequence (visible_varlen); rows past the length, or with no visible key, give
    o = 0, lse = -inf and zero gradients, and keys past the length get zero dK, dV;
  * grouped query heads (oracle.attention.kv_head_of): query head h attends with key/value head
    h // (H / H_kv), and the key/value gradients are the sums over the group (the chain rule
    through a shared input);
  * dropout (oracle.dropout): O = (P Z / (1 - p)) V with Z = dropout_keep of query head
    b H + h; the keep counters index query rows and keys of the padded layout, which for a
    sequence coincide with its own row and key indices; L is that of the scores (the softmax is
    normalised before dropout); gradients hold Z fixed.
"""
from __future__ import annotations

import numpy as np

from . import attention as A
from . import dropout as DR


def _live_probs(qs, ks, mask, scale):
    """Softmax rows of scale qs ks^T over the visible keys (mask), rows with at least one visible
    key only: (P [rows, n_k], lse [rows])."""
    s = np.where(mask, scale * (qs @ ks.T), -np.inf)
    return A.softmax_rows(s)


def forward_combined(q, k, v, seq_lens_q, seq_lens_k, scale: float, causal: bool, p: float,
                     seed: int, offset: int):
    """q [B,H,N_q,d]; k, v [B,H_kv,N_k,d] (H a multiple of H_kv); seq_lens_q, seq_lens_k [B]
    (None: every sequence has the full extent); p = 0: no dropout.
    Returns (o [B,H,N_q,d_v], lse [B,H,N_q]) fp64."""
    B, H, n_q, _ = np.shape(q)
    H_kv, n_k = np.shape(k)[1], np.shape(k)[2]
    lq_all = [n_q] * B if seq_lens_q is None else seq_lens_q
    lk_all = [n_k] * B if seq_lens_k is None else seq_lens_k
    o = np.zeros((B, H, n_q, np.shape(v)[3]), dtype=np.float64)
    lse = np.full((B, H, n_q), -np.inf, dtype=np.float64)
    for b in range(B):
        lq, lk = A._clamp_len(lq_all[b], n_q), A._clamp_len(lk_all[b], n_k)
        mask = A.visible_varlen(lq, lk, causal)
        live = np.flatnonzero(mask.any(axis=1))
        if live.size == 0:
            continue
        for h in range(H):
            g = A.kv_head_of(h, H, H_kv)
            kh = np.asarray(k[b, g, :lk], np.float64)
            vh = np.asarray(v[b, g, :lk], np.float64)
            P, l_ = _live_probs(np.asarray(q[b, h, :lq], np.float64)[live], kh, mask[live], scale)
            if p > 0:
                P = P * DR.dropout_keep(seed, offset, b * H + h, lq, lk, p)[live] / (1.0 - p)
            o[b, h, live] = P @ vh
            lse[b, h, live] = l_
    return o, lse


def backward_combined(q, k, v, do, seq_lens_q, seq_lens_k, scale: float, causal: bool, p: float,
                      seed: int, offset: int):
    """Gradients of forward_combined's O given dO, by the chain rule of [MW] "Geri Yayılım":
    with Pd = P Z / (1 - p): dV = Pd^T dO; dP = (dO V^T) Z / (1 - p);
    dS = P (dP - rowsum(P dP)); dQ = scale dS K; dK = scale dS^T Q; dK and dV of a key/value head
    summed over its query heads. Returns (dq, dk, dv) fp64, zero on padding."""
    B, H, n_q, _ = np.shape(q)
    H_kv, n_k = np.shape(k)[1], np.shape(k)[2]
    lq_all = [n_q] * B if seq_lens_q is None else seq_lens_q
    lk_all = [n_k] * B if seq_lens_k is None else seq_lens_k
    dq = np.zeros(np.shape(q), dtype=np.float64)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(B):
        lq, lk = A._clamp_len(lq_all[b], n_q), A._clamp_len(lk_all[b], n_k)
        mask = A.visible_varlen(lq, lk, causal)
        live = np.flatnonzero(mask.any(axis=1))
        if live.size == 0:
            continue
        for h in range(H):
            g = A.kv_head_of(h, H, H_kv)
            qh = np.asarray(q[b, h, :lq], np.float64)[live]
            doh = np.asarray(do[b, h, :lq], np.float64)[live]
            kh = np.asarray(k[b, g, :lk], np.float64)
            vh = np.asarray(v[b, g, :lk], np.float64)
            P, _ = _live_probs(qh, kh, mask[live], scale)
            zs = np.ones_like(P)
            if p > 0:
                zs = DR.dropout_keep(seed, offset, b * H + h, lq, lk, p)[live] / (1.0 - p)
            dv[b, g, :lk] += (P * zs).T @ doh
            dP = (doh @ vh.T) * zs
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[b, h, live] = scale * (dS @ kh)
            dk[b, g, :lk] += scale * (dS.T @ qh)
    return dq, dk, dv
