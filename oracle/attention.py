"""Plain CPU fp64 oracle for exact scaled-dot-product attention (forward, backward, decode).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this module;
only the tests, the package's smoke check and the benchmark's CPU-baseline leg use it. It shares
no code with the HIP kernels: it takes plain float arrays and returns fp64 arrays.

Sources. Five web pages on FlashAttention; the arithmetic below follows
  [MW]  "Bellek Duvarının Fiziği: Standart Attention'dan FlashAttention'a" (webturing Principia):
        "Attention'ın Cebiri" (the definition S = QK^T/sqrt(d_k), P = row softmax(S), O = PV),
        "Softmax'ın Kalesi" (softmax with the row maximum subtracted),
        "O(N²) Çıkmazı" (the standard implementation materialises S and P),
        "Maskeleme ve Dropout" (causal: query i sees keys j <= i, masked entries are -inf before
        the row maximum),
        "Geri Yayılım" (the stored per-row log-sum-exp L, P = exp(S - L), and the softmax
        gradient identity dsoftmax = p * (dp - <dp>)),
        "Decode Aşaması: Flash-Decoding" (decode is the same function with one query row).
  [EN]  "FlashAttention'ı Anlamak Bölüm 1", section 0.2 (notation: Q in R^{N_q x d},
        K, V in R^{N_k x d}, optional mask/bias added to the scores).

Because FlashAttention computes exact attention (it differs from the textbook only in rounding
order, [MW] "Online Softmax"), this oracle is the textbook definition written out, not the tiled
algorithm: it materialises the full score matrix S and probability matrix P of every head, one
head at a time, in fp64.

Readings where the pages are silent (each also listed in the design notes):
  * the scale is a caller argument (the pages use 1/sqrt(d_k));
  * for N_q != N_k the causal mask is aligned bottom-right: key j is visible to query i iff
    j <= i + N_k - N_q (identical to "j <= i" when N_q == N_k); N_q > N_k is rejected so that
    no row is empty;
  * the stored statistic is the natural-log log-sum-exp of the scaled, masked scores,
    L_i = ln sum_j exp(S_ij);
  * d_v = d;
  * grouped query heads: H query heads, H_kv key/value heads, H a multiple of H_kv, query head
    h attends with key/value head h // (H // H_kv); dK and dV of a key/value head are the sums
    of the gradients its query heads send to it;
  * a batch of different-length sequences (padded tensors plus per-sequence lengths) is the
    single-sequence definition applied to each sequence's own rows and keys, causal alignment
    per sequence; a row that sees no key (padding, or causal with more queries than keys) has
    o = 0 and lse = -inf and contributes no gradient.

Every function here is pinned by tests that do not reuse its formulas: brute-force per-row
softmax in pure Python, rows of P summing to one, bitwise causal invariance to future keys,
central finite differences of the gradients, closed forms (Q = 0, one key, first causal row),
shift and permutation invariances, gradient sum rules, and agreement with PyTorch's CPU
scaled_dot_product_attention and autograd in float64.
"""
from __future__ import annotations

import numpy as np

# Rows of one head processed together. Rows are independent, so splitting them changes no
# arithmetic on any row; it only bounds host memory for long sequences (N_q * N_k large).
_ROW_BLOCK_ELEMS = 1 << 26


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible(n_q: int, n_k: int, causal: bool) -> np.ndarray:
    """Boolean [n_q, n_k]: True where key j may be attended by query i.

    [MW] "Maskeleme ve Dropout": under the causal mask query i sees only keys j <= i.
    With N_q < N_k the queries are taken to be the last N_q positions (bottom-right).
    """
    if causal and n_q > n_k:
        raise ValueError("causal attention needs n_q <= n_k")
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i + (n_k - n_q)


def scores(q, k, scale: float, causal: bool, rows=None) -> np.ndarray:
    """S = scale * Q K^T with masked entries set to -inf, for one head ([MW] "Attention'ın Cebiri").

    q: [n_q, d], k: [n_k, d]. `rows` selects a subset of query rows (default: all).
    """
    q = _f64(q)
    k = _f64(k)
    n_q, n_k = q.shape[0], k.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    s = scale * (q[rows] @ k.T)
    mask = visible(n_q, n_k, causal)[rows]
    s[~mask] = -np.inf
    return s


def softmax_rows(s: np.ndarray):
    """Row softmax with the row maximum subtracted ([MW] "Softmax'ın Kalesi").

    Returns (P, L) with P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i) and the log-sum-exp
    L_i = m_i + ln sum_j exp(S_ij - m_i) ([MW] "Geri Yayılım"). Every row must hold at least
    one finite score.
    """
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    p = e / z
    lse = (m + np.log(z))[:, 0]
    return p, lse


def forward_head(q, k, v, scale: float, causal: bool, rows=None):
    """O = P V and L for one head; q [n_q, d], k/v [n_k, d]. Returns (o [r, d], lse [r])."""
    v = _f64(v)
    n_q, n_k = np.shape(q)[0], np.shape(k)[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    block = max(1, _ROW_BLOCK_ELEMS // max(1, n_k))
    o = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for r0 in range(0, len(rows), block):
        sel = rows[r0:r0 + block]
        p, l_ = softmax_rows(scores(q, k, scale, causal, sel))
        o[r0:r0 + len(sel)] = p @ v
        lse[r0:r0 + len(sel)] = l_
    return o, lse


def forward(q, k, v, scale: float, causal: bool):
    """Batched forward: q [B,H,n_q,d], k/v [B,H,n_k,d] -> (o [B,H,n_q,d], lse [B,H,n_q])."""
    B, H, n_q, d = np.shape(q)
    o = np.empty((B, H, n_q, np.shape(v)[3]), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def backward_head(q, k, v, do, scale: float, causal: bool):
    """Gradients of O with respect to Q, K, V for one head, by the textbook chain rule.

    [MW] "Geri Yayılım": with P materialised, dV = P^T dO; dP = dO V^T; the softmax gradient
    identity gives dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik); and since S = scale * Q K^T,
    dQ = scale * dS K and dK = scale * dS^T Q. The row term is taken from P and dP here, not
    from rowsum(dO * O), so that it is independent of the GPU's preprocess.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, _ = softmax_rows(scores(q, k, scale, causal))
    dv = p.T @ do
    dp = do @ v.T
    row = np.sum(p * dp, axis=1, keepdims=True)
    ds = p * (dp - row)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward(q, k, v, do, scale: float, causal: bool):
    """Batched backward: returns (dq, dk, dv) shaped like (q, k, v), fp64."""
    B, H = np.shape(q)[:2]
    dq = np.empty(np.shape(q), dtype=np.float64)
    dk = np.empty(np.shape(k), dtype=np.float64)
    dv = np.empty(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(q[b, h], k[b, h], v[b, h], do[b, h],
                                                         scale, causal)
    return dq, dk, dv


def kv_head_of(h: int, H: int, H_kv: int) -> int:
    """Key/value head of query head h with grouped query heads ([MW] "Duvarın Ötesi: KV Cache,
    Uzun Bağlam ve Yaklaşık Attention" names GQA/MQA; the reading used throughout: H a multiple
    of H_kv, consecutive groups of H // H_kv query heads share one key/value head)."""
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("the query head count must be a multiple of the key/value head count")
    return h // (H // H_kv)


def forward_gqa(q, k, v, scale: float, causal: bool):
    """Forward with grouped query heads: q [B,H,n_q,d], k/v [B,H_kv,n_k,d] -> (o [B,H,n_q,d],
    lse [B,H,n_q]); each query head is forward_head against its key/value head."""
    B, H, n_q, _ = np.shape(q)
    H_kv = np.shape(k)[1]
    o = np.empty((B, H, n_q, np.shape(v)[3]), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, H_kv)
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, g], v[b, g], scale, causal)
    return o, lse


def backward_gqa(q, k, v, do, scale: float, causal: bool):
    """Gradients of forward_gqa's o. A key/value head enters the outputs of all query heads of its
    group, so by the chain rule its dK and dV are the sums of the per-query-head gradients of
    backward_head ([MW] "Geri Yayılım"); dQ is per query head. Returns (dq, dk, dv) shaped like
    (q, k, v), fp64."""
    B, H = np.shape(q)[:2]
    H_kv = np.shape(k)[1]
    dq = np.empty(np.shape(q), dtype=np.float64)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, H_kv)
            dq[b, h], gk, gv = backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dk[b, g] += gk
            dv[b, g] += gv
    return dq, dk, dv


def decode(q, k, v, scale: float):
    """Decode step: one query row per (b, h) against the whole KV cache.

    [MW] "Decode Aşaması: Flash-Decoding": the split-KV scheme computes the same function as
    the forward pass with a single query, so the oracle is the forward with n_q = 1 and no split.
    q [B,H,1,d], k/v [B,H,n_k,d] -> (o [B,H,1,d], lse [B,H,1]).
    """
    if np.shape(q)[2] != 1:
        raise ValueError("decode takes exactly one query row per (b, h)")
    return forward(q, k, v, scale, causal=False)


def gather_paged(cache, block_table_row, seq_len: int, kv_head: int) -> np.ndarray:
    """Positions 0 .. seq_len-1 of one sequence and one key/value head of a paged cache.

    cache [num_blocks, H_kv, block_size, d]; position j of the sequence lives in block
    block_table_row[j // block_size] at row j % block_size (the paged-cache reading of
    [MW] "Duvarın Ötesi: KV Cache, Uzun Bağlam ve Yaklaşık Attention", which names PagedAttention
    without defining it). Returns fp64 [seq_len, d].
    """
    cache = np.asarray(cache)
    bs = cache.shape[2]
    j = np.arange(seq_len)
    blocks = np.asarray(block_table_row)[j // bs]
    return _f64(cache[blocks, kv_head, j % bs])


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale: float):
    """Decode step over a paged KV cache with grouped query heads.

    [MW] "Duvarın Ötesi: KV Cache, ...": query heads may share key/value heads (GQA/MQA); the
    reading used here: with H query heads and H_kv key/value heads (H a multiple of H_kv), query
    head h uses key/value head h // (H // H_kv). Each (b, h) is the decode function of
    [MW] "Decode Aşaması: Flash-Decoding" (one query row, every position visible) over the
    sequence's seq_lens[b] positions gathered from the cache. A sequence with no position gives
    o = 0 and lse = -inf.
    q [B,H,d]; k_cache/v_cache [num_blocks,H_kv,block_size,d]; block_table [B,max_blocks];
    seq_lens [B] -> (o [B,H,d], lse [B,H]) fp64.
    """
    B, H, d = np.shape(q)
    H_kv = np.shape(k_cache)[1]
    if H % H_kv != 0:
        raise ValueError("the query head count must be a multiple of the key/value head count")
    group = H // H_kv
    o = np.zeros((B, H, np.shape(v_cache)[3]), dtype=np.float64)
    lse = np.full((B, H), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        for kvh in range(H_kv):
            kk = gather_paged(k_cache, block_table[b], n, kvh)
            vv = gather_paged(v_cache, block_table[b], n, kvh)
            for h in range(kvh * group, (kvh + 1) * group):
                ob, lb = forward_head(np.asarray(q[b, h])[None, :], kk, vv, scale, causal=False)
                o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def _clamp_len(x, n: int) -> int:
    return min(max(int(x), 0), n)


def visible_varlen(l_q: int, l_k: int, causal: bool) -> np.ndarray:
    """Boolean [l_q, l_k] visibility for one sequence of a variable-length batch.

    Same bottom-right causal alignment as `visible`, key j visible to query i iff
    j <= i + l_k - l_q, but l_q > l_k is allowed: the first l_q - l_k query rows then see no
    key at all (reading: such a row has no softmax, it gets o = 0 and lse = -inf).
    """
    if not causal:
        return np.ones((l_q, l_k), dtype=bool)
    i = np.arange(l_q)[:, None]
    j = np.arange(l_k)[None, :]
    return j <= i + (l_k - l_q)


def _varlen_probs(qs, ks, mask, scale):
    # scores of the rows that see at least one key, masked entries -inf, then the row softmax
    s = scale * (qs @ ks.T)
    s[~mask] = -np.inf
    return softmax_rows(s)


def forward_varlen(q, k, v, seq_lens_q, seq_lens_k, scale: float, causal: bool):
    """Forward over a batch of sequences of different lengths held in padded tensors.

    q [B,H,N_q,d], k/v [B,H,N_k,d]; sequence b uses its first seq_lens_q[b] query rows and
    first seq_lens_k[b] key rows (lengths clamped to [0, N]). The pages define attention for one
    sequence ([MW] "Attention'ın Cebiri"); the reading for a batch is that definition on each
    sequence's own rows and keys, with the causal mask of [MW] "Maskeleme ve Dropout" aligned
    per sequence (`visible_varlen`). Padding rows, and rows that see no key, get o = 0 and
    lse = -inf. Returns (o [B,H,N_q,d_v], lse [B,H,N_q]) fp64.
    """
    B, H, n_q, _ = np.shape(q)
    n_k = np.shape(k)[2]
    o = np.zeros((B, H, n_q, np.shape(v)[3]), dtype=np.float64)
    lse = np.full((B, H, n_q), -np.inf, dtype=np.float64)
    for b in range(B):
        lq, lk = _clamp_len(seq_lens_q[b], n_q), _clamp_len(seq_lens_k[b], n_k)
        mask = visible_varlen(lq, lk, causal)
        live = np.flatnonzero(mask.any(axis=1))
        if live.size == 0:
            continue
        for h in range(H):
            p, l_ = _varlen_probs(_f64(q[b, h, :lq])[live], _f64(k[b, h, :lk]), mask[live], scale)
            o[b, h, live] = p @ _f64(v[b, h, :lk])
            lse[b, h, live] = l_
    return o, lse


def backward_varlen(q, k, v, do, seq_lens_q, seq_lens_k, scale: float, causal: bool):
    """Gradients of forward_varlen's o with respect to q, k, v (the chain rule of
    [MW] "Geri Yayılım" on each sequence's live rows and keys). Padding rows and keys, and
    rows that see no key, have zero gradient: o does not depend on them (the o = 0 of an
    empty row is a constant). Returns (dq, dk, dv) fp64, shaped like (q, k, v).
    """
    B, H, n_q, _ = np.shape(q)
    n_k = np.shape(k)[2]
    dq = np.zeros(np.shape(q), dtype=np.float64)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(B):
        lq, lk = _clamp_len(seq_lens_q[b], n_q), _clamp_len(seq_lens_k[b], n_k)
        mask = visible_varlen(lq, lk, causal)
        live = np.flatnonzero(mask.any(axis=1))
        if live.size == 0:
            continue
        for h in range(H):
            qs, ks = _f64(q[b, h, :lq])[live], _f64(k[b, h, :lk])
            vs, dos = _f64(v[b, h, :lk]), _f64(do[b, h, :lq])[live]
            p, _ = _varlen_probs(qs, ks, mask[live], scale)
            dv[b, h, :lk] = p.T @ dos
            dp = dos @ vs.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h, live] = scale * (ds @ ks)
            dk[b, h, :lk] = scale * (ds.T @ qs)
    return dq, dk, dv


def forward_bias(q, k, v, bias, scale: float, causal: bool):
    """Forward with an additive bias on the scores (notation section 0.2 of "FlashAttention'ı
    Anlamak Bölüm 1": S = Q K^T / sqrt(d) + B, B an optional mask or bias; here the scale is a
    caller argument): S = scale Q K^T + bias, masked entries -inf. bias broadcasts to
    [B, H, n_q, n_k] and may hold -inf (a mask). A row with no finite score has no softmax
    (reading as for variable lengths): o = 0, lse = -inf. Returns (o, lse) fp64."""
    B, H, n_q, _ = np.shape(q)
    n_k = np.shape(k)[2]
    bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, H, n_q, n_k))
    o = np.zeros((B, H, n_q, np.shape(v)[3]), dtype=np.float64)
    lse = np.full((B, H, n_q), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, h], scale, causal) + bias[b, h]
            live = np.flatnonzero(np.any(np.isfinite(s), axis=1))
            if live.size == 0:
                continue
            p, l_ = softmax_rows(s[live])
            o[b, h, live] = p @ _f64(v[b, h])
            lse[b, h, live] = l_
    return o, lse


def backward_bias(q, k, v, do, bias, scale: float, causal: bool):
    """Gradients of forward_bias's o with respect to q, k, v (the bias is a constant input; no
    gradient is formed for it), by the chain rule of [MW] "Geri Yayılım" on the rows that have a
    softmax; rows without one contribute nothing."""
    B, H, n_q, _ = np.shape(q)
    n_k = np.shape(k)[2]
    bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, H, n_q, n_k))
    dq = np.zeros(np.shape(q), dtype=np.float64)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h])
            s = scores(qh, kh, scale, causal) + bias[b, h]
            live = np.flatnonzero(np.any(np.isfinite(s), axis=1))
            if live.size == 0:
                continue
            p, _ = softmax_rows(s[live])
            dv[b, h] = p.T @ doh[live]
            dp = doh[live] @ vh.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h, live] = scale * (ds @ kh)
            dk[b, h] = scale * (ds.T @ qh[live])
    return dq, dk, dv
