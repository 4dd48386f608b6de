"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests and the benchmark.

This module holds no attention arithmetic. It only draws numbers and rounds them to bfloat16,
so that the oracle and the HIP kernels consume the very same bf16 values.

Recipe (one stream per slice, so any single head can be regenerated on its own):
    Generator(PCG64(SeedSequence([seed, tensor_id, b, h]))).standard_normal((N, d), float32)
then fp32 -> bf16 by round-to-nearest-even on the bit pattern. Tensor ids: Q=0, K=1, V=2, dO=3.
The values are iid N(0,1), the distribution every workload on the attention pages assumes for
its synthetic inputs.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from numpy.random import PCG64, Generator, SeedSequence

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generators below never draw a non-finite value).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    return bf16_to_f32(u).astype(np.float64)


def slice_bf16(seed: int, tensor: str, b: int, h: int, n: int, d: int) -> np.ndarray:
    """One (b, h) slice [n, d] of a tensor as bf16 bit patterns."""
    g = Generator(PCG64(SeedSequence([seed, TENSOR_ID[tensor], b, h])))
    return bf16_round(g.standard_normal((n, d), dtype=np.float32))


def tensor_bf16(seed: int, tensor: str, B: int, H: int, n: int, d: int,
                threads: int | None = None) -> np.ndarray:
    """The whole [B, H, n, d] tensor as bf16 bit patterns, drawn slice by slice."""
    out = np.empty((B, H, n, d), dtype=np.uint16)

    def fill(bh: int) -> None:
        b, h = divmod(bh, H)
        out[b, h] = slice_bf16(seed, tensor, b, h, n, d)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if B * H == 1 or nthreads == 1:
        for bh in range(B * H):
            fill(bh)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(B * H)))
    return out


def long_head_bf16(seed: int, tensor: str, n: int, d: int, parts: int = 32,
                   threads: int | None = None) -> np.ndarray:
    """One very long head [1, 1, n, d] as bf16 bit patterns, drawn in `parts` runs of rows with
    one stream each, SeedSequence([seed, tensor_id, 0, 0, part]), so that the draw runs on
    several threads (a single stream of 2^30 values takes half a minute)."""
    out = np.empty((1, 1, n, d), dtype=np.uint16)
    step = (n + parts - 1) // parts

    def fill(i: int) -> None:
        r0, r1 = i * step, min(n, (i + 1) * step)
        if r0 < r1:
            g = Generator(PCG64(SeedSequence([seed, TENSOR_ID[tensor], 0, 0, i])))
            out[0, 0, r0:r1] = bf16_round(g.standard_normal((r1 - r0, d), dtype=np.float32))

    with ThreadPoolExecutor(threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(parts)))
    return out


def qkv_bf16(seed: int, B: int, H: int, n_q: int, n_k: int, d: int, with_do: bool = False):
    """Q [B,H,n_q,d], K and V [B,H,n_k,d] (and dO [B,H,n_q,d]) as bf16 bit patterns."""
    q = tensor_bf16(seed, "q", B, H, n_q, d)
    k = tensor_bf16(seed, "k", B, H, n_k, d)
    v = tensor_bf16(seed, "v", B, H, n_k, d)
    if with_do:
        return q, k, v, tensor_bf16(seed, "do", B, H, n_q, d)
    return q, k, v


def paged_kv_bf16(seed: int, B: int, H_kv: int, seq_lens, d: int, block_size: int,
                  max_blocks: int, spare_blocks: int = 3):
    """A paged KV cache holding, for sequence b and key/value head h, the rows of
    slice_bf16(seed, "k"/"v", b, h, seq_lens[b], d), scattered over shuffled physical blocks.

    Returns (k_cache, v_cache [num_blocks, H_kv, block_size, d] uint16, block_table
    [B, max_blocks] int32, seq_lens [B] int32). num_blocks = B * max_blocks + spare_blocks; the
    table lists every block of a sequence (also those past its length), drawn without
    repetition from a seeded permutation; unused rows hold a fixed filler pattern (bf16 1.0).
    """
    lens = np.asarray(seq_lens, dtype=np.int32)
    if np.any(lens > max_blocks * block_size):
        raise ValueError("a sequence does not fit in max_blocks blocks")
    num_blocks = B * max_blocks + spare_blocks
    perm = Generator(PCG64(SeedSequence([seed, 7, B, max_blocks]))).permutation(num_blocks)
    table = perm[: B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    kc = np.full((num_blocks, H_kv, block_size, d), 0x3F80, dtype=np.uint16)
    vc = np.full((num_blocks, H_kv, block_size, d), 0x3F80, dtype=np.uint16)
    for b in range(B):
        n = int(lens[b])
        j = np.arange(n)
        blocks, rows = table[b][j // block_size], j % block_size
        for h in range(H_kv):
            kc[blocks, h, rows] = slice_bf16(seed, "k", b, h, n, d)
            vc[blocks, h, rows] = slice_bf16(seed, "v", b, h, n, d)
    return kc, vc, table, lens


def varlen_lengths(seed: int, B: int, n_min: int, n_max: int) -> np.ndarray:
    """Per-sequence lengths of a variable-length batch: int32 [B], uniform on [n_min, n_max]."""
    g = Generator(PCG64(SeedSequence([seed, 11, B, n_min, n_max])))
    return g.integers(n_min, n_max + 1, size=B).astype(np.int32)


BF16_NAN = 0x7FC0


def fill_padding(u16: np.ndarray, lens, pattern: int = BF16_NAN) -> np.ndarray:
    """Copy of a [B, H, n, d] bf16 tensor with rows n >= lens[b] of batch entry b set to a bit
    pattern (default: a quiet NaN), so that a test can show those rows are never used."""
    out = np.array(u16, copy=True)
    for b, n in enumerate(np.asarray(lens)):
        out[b, :, max(int(n), 0):] = pattern
    return out


def outlier_bf16(seed: int, tensor: str, B: int, H: int, n: int, d: int, frac: float = 1e-2,
                 mag: float = 10.0) -> np.ndarray:
    """Synthetic outlier features as bf16 bit patterns [B, H, n, d]: N(0, 1) entries, a random
    fraction `frac` of them plus N(0, mag^2)."""
    out = np.empty((B, H, n, d), dtype=np.uint16)
    for b in range(B):
        for h in range(H):
            g = Generator(PCG64(SeedSequence([seed, TENSOR_ID[tensor], b, h, 13])))
            x = g.standard_normal((n, d))
            hit = g.random((n, d)) < frac
            x[hit] += mag * g.standard_normal(int(hit.sum()))
            out[b, h] = bf16_round(x.astype(np.float32))
    return out


def rising_keys(q_u16: np.ndarray, k_u16: np.ndarray, per_key: float, q_value: float = 3.0):
    """Copies of Q [.., n_q, d] and K [.., n_k, d] (bf16 bit patterns) with column 0 overwritten:
    Q[.., 0] = q_value and K[.., j, 0] = per_key * j (rounded to bf16), so that every query's
    score grows with the key index and a running row maximum rises on every block of keys."""
    q = np.array(q_u16, copy=True)
    k = np.array(k_u16, copy=True)
    q[..., 0] = bf16_round(np.full(q.shape[:-1], q_value, dtype=np.float32))
    n_k = k.shape[-2]
    ramp = (np.arange(n_k, dtype=np.float64) * per_key).astype(np.float32)
    k[..., 0] = bf16_round(np.broadcast_to(ramp, k.shape[:-1]))
    return q, k


def rising_keys_paged(q_u16: np.ndarray, k_cache: np.ndarray, block_table, seq_lens,
                      per_key: float, q_value: float = 3.0):
    """rising_keys for a paged cache (paged_kv_bf16's layout): q [B, H, d] gets column 0 =
    q_value, and position j of sequence b (block block_table[b, j // bs], row j % bs) gets
    K column 0 = per_key * j in every K/V head."""
    q = np.array(q_u16, copy=True)
    kc = np.array(k_cache, copy=True)
    q[..., 0] = bf16_round(np.full(q.shape[:-1], q_value, dtype=np.float32))
    bs = kc.shape[2]
    for b, n in enumerate(np.asarray(seq_lens)):
        j = np.arange(int(n))
        vals = bf16_round((j * per_key).astype(np.float32))
        blocks, rows = np.asarray(block_table)[b][j // bs], j % bs
        for h in range(kc.shape[1]):
            kc[blocks, h, rows, 0] = vals
    return q, kc
