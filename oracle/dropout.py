"""CPU fp64 oracle for attention with dropout on the probabilities, and the counter-based random
generator that decides which probabilities are dropped.

TEST INFRASTRUCTURE ONLY (like oracle/attention.py): nothing in the product path may import,
call or execute this module; it shares no code with the HIP kernels.

Sources.
  [MW] "Bellek Duvarının Fiziği" (webturing Principia), section "Maskeleme ve Dropout": the
       classic implementation applies dropout to P; FlashAttention never stores P, so it cannot
       store the mask either; the kernel drives a counter-based generator (Philox on CUDA) from a
       seed and an offset and regenerates the same mask in the backward pass instead of saving it.
  [PX] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): the
       Philox family of counter-based generators. Philox-4xW-R maps a counter of four W-bit words
       and a key of two W-bit words through R rounds; each round multiplies words 0 and 2 by two
       fixed odd constants into (hi, lo) halves, and returns (hi of word 2's product xor word 1
       xor key 0, lo of word 2's product, hi of word 0's product xor word 3 xor key 1, lo of
       word 0's product); between rounds both key words are advanced by the Weyl constants
       (the fractional parts of the golden ratio and of sqrt(3), scaled to W bits).

Readings (where the pages leave the method open; each is also in the design notes):
  * generator: Philox-4x32-10 ([PX]'s recommended 32-bit member); key = (seed mod 2^32,
    seed div 2^32) of a 64-bit seed;
  * counter of the call that decides the dropout of scores (i, j) of head bh = b*H + h:
    (j div 8, i, bh, offset); its four 32-bit output words hold eight 16-bit numbers, and key j
    uses number j mod 8: word (j mod 8) div 2, low half for even j, high half for odd j;
  * keep (i, j) iff that 16-bit number u satisfies u < t with t = floor((1 - p) * 65536),
    computed in double precision (the drop probability p is in [0, 1));
  * inverted dropout: kept probabilities are multiplied by 1 / (1 - p); the softmax is
    normalised over all keys before dropout (the dropout acts on P, [MW]), so the log-sum-exp L
    is that of the scores, unchanged by dropout;
  * gradients are those of O = (P * Z / (1 - p)) V with the mask Z held fixed.
"""
from __future__ import annotations

import math

import numpy as np

from . import attention as A

# Multipliers of Philox-4x32 and Philox-4x64 ([PX], the published constants).
PHILOX_M = {32: (0xD2511F53, 0xCD9E8D57), 64: (0xD2E7470EE14C6C93, 0xCA5A826395121157)}
# Weyl key increments: floor(2^W (golden ratio - 1)) and floor(2^W (sqrt(3) - 1)).
PHILOX_W = {32: (0x9E3779B9, 0xBB67AE85), 64: (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)}

def philox(counters, key, word_bits: int = 32, rounds: int = 10) -> np.ndarray:
    """Philox-4xW-R of [PX] on many counters at once.

    counters: non-negative integer array [n, 4]; key: two W-bit integers. Returns [n, 4] output
    words. For W = 32 the words are held in uint64, so a 32 x 32-bit product is exact; for W = 64
    they are Python integers (object arrays), exact as well. The round below serves both sizes.
    """
    mask = (1 << word_bits) - 1
    if word_bits == 32:
        conv = np.uint64
        c = np.asarray(counters, dtype=np.uint64).reshape(-1, 4) & conv(mask)
    else:
        conv = int
        c = np.array([[int(x) & mask for x in row] for row in np.asarray(counters, dtype=object)
                      .reshape(-1, 4)], dtype=object).reshape(-1, 4)
    c = [c[:, w] for w in range(4)]
    m0, m1 = conv(PHILOX_M[word_bits][0]), conv(PHILOX_M[word_bits][1])
    sh, lo = conv(word_bits), conv(mask)
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    for r in range(rounds):
        if r > 0:  # advance the key by the Weyl constants between rounds
            k0 = (k0 + PHILOX_W[word_bits][0]) & mask
            k1 = (k1 + PHILOX_W[word_bits][1]) & mask
        p0, p1 = c[0] * m0, c[2] * m1
        c = [(p1 >> sh) ^ c[1] ^ conv(k0), p1 & lo, (p0 >> sh) ^ c[3] ^ conv(k1), p0 & lo]
    return np.stack(c, axis=1)


def keep_threshold(p: float) -> int:
    """t = floor((1 - p) * 2^16) in double precision; a 16-bit number u keeps iff u < t."""
    if not (0.0 <= p < 1.0):
        raise ValueError("the drop probability must lie in [0, 1)")
    return int(math.floor((1.0 - float(p)) * 65536.0))


def dropout_keep(seed: int, offset: int, bh: int, n_q: int, n_k: int, p: float) -> np.ndarray:
    """Boolean [n_q, n_k] keep mask of head bh: True where the probability survives."""
    t = keep_threshold(p)
    ngroups = (n_k + 7) // 8
    i, g = np.meshgrid(np.arange(n_q), np.arange(ngroups), indexing="ij")
    ctr = np.stack([g.ravel(), i.ravel(), np.full(i.size, bh), np.full(i.size, offset)], axis=1)
    words = philox(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).astype(np.uint64)
    words = words.reshape(n_q, ngroups, 4)
    u = np.empty((n_q, ngroups, 8), dtype=np.int64)
    u[:, :, 0::2] = (words & np.uint64(0xFFFF)).astype(np.int64)
    u[:, :, 1::2] = (words >> np.uint64(16)).astype(np.int64)
    return u.reshape(n_q, ngroups * 8)[:, :n_k] < t


def _head_ids(B: int, H: int, head_ids):
    return np.arange(B * H).reshape(B, H) if head_ids is None else np.asarray(head_ids)


def forward_dropout(q, k, v, scale: float, causal: bool, p: float, seed: int, offset: int,
                    head_ids=None):
    """O = (P * Z / (1 - p)) V and the (dropout-free) L per head; q [B,H,n_q,d], k/v [B,H,n_k,d].
    P and L as in oracle.attention (the textbook definition, [MW] "Attention'ın Cebiri");
    Z = dropout_keep of the head ([MW] "Maskeleme ve Dropout"). head_ids [B, H]: the generator's
    head index of each head (default b*H + h; a caller checking a slice of a larger batch passes
    the slice's own indices)."""
    B, H, n_q, _ = np.shape(q)
    n_k = np.shape(k)[2]
    ids = _head_ids(B, H, head_ids)
    o = np.empty((B, H, n_q, np.shape(v)[3]), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            P, lse[b, h] = A.softmax_rows(A.scores(q[b, h], k[b, h], scale, causal))
            Z = dropout_keep(seed, offset, int(ids[b, h]), n_q, n_k, p)
            o[b, h] = (P * Z / (1.0 - p)) @ np.asarray(v[b, h], dtype=np.float64)
    return o, lse


def backward_dropout(q, k, v, do, scale: float, causal: bool, p: float, seed: int, offset: int,
                     head_ids=None):
    """Gradients of forward_dropout's O with the mask fixed, by the chain rule of [MW]
    "Geri Yayılım" through the extra elementwise factor Z / (1 - p):
    dV = Pd^T dO with Pd = P Z / (1 - p); dP = (dO V^T) Z / (1 - p);
    dS = P (dP - rowsum(P dP)); dQ = scale dS K; dK = scale dS^T Q."""
    B, H, n_q, _ = np.shape(q)
    n_k = np.shape(k)[2]
    ids = _head_ids(B, H, head_ids)
    dq = np.empty(np.shape(q), dtype=np.float64)
    dk = np.empty(np.shape(k), dtype=np.float64)
    dv = np.empty(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            qh, kh = np.asarray(q[b, h], np.float64), np.asarray(k[b, h], np.float64)
            vh, doh = np.asarray(v[b, h], np.float64), np.asarray(do[b, h], np.float64)
            P, _ = A.softmax_rows(A.scores(qh, kh, scale, causal))
            zs = dropout_keep(seed, offset, int(ids[b, h]), n_q, n_k, p) / (1.0 - p)
            dv[b, h] = (P * zs).T @ doh
            dP = (doh @ vh.T) * zs
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ kh)
            dk[b, h] = scale * (dS.T @ qh)
    return dq, dk, dv
