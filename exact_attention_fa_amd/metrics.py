"""Work and traffic counts used to turn measured times into the reported rates.

Conventions (the attention pages' own accounting):
  * forward FLOPs are 4 * N_q * N_k * d per head: 2 N_q N_k d for QK^T and as many for PV
    ("Bellek Duvarının Fiziği", section "Attention'ın Cebiri");
  * a causal mask halves them ("Maskeleme ve Dropout": roughly half the matrix is computed;
    the factor is taken as exactly 1/2);
  * the backward pass costs 2.5 times the forward ("Geri Yayılım");
  * decode is bandwidth-bound, so it is measured in bytes: K and V are read once.
"""
from __future__ import annotations

MI355X_BF16_DENSE_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 bf16 FLOP per CU-clock
MI355X_FP8_DENSE_TFLOPS = 5033.2  # twice the bf16 rate (dense, no sparsity)
MI355X_HBM_GBPS = 8000.0


def attention_flops(B: int, H: int, n_q: int, n_k: int, d: int, causal: bool = False,
                    backward: bool = False) -> float:
    """Algorithmic FLOPs of one attention pass (the forward, or the backward when asked)."""
    f = 4.0 * B * H * n_q * n_k * d
    if causal:
        f *= 0.5
    if backward:
        f *= 2.5
    return f


def executed_bwd_flops(B: int, H: int, n_q: int, n_k: int, d: int, causal: bool) -> float:
    """FLOPs the backward kernels execute: seven N_q x N_k x d products (S and dP are rebuilt in
    both the dK/dV pass and the dQ pass), against the five the 2.5x convention counts."""
    f = 7 * 2.0 * B * H * n_q * n_k * d
    return f * 0.5 if causal else f


def score_matrix_bytes(n: int, elem_bytes: int) -> int:
    """Bytes of one N x N score or probability matrix ("O(N²) Çıkmazı")."""
    return n * n * elem_bytes


def standard_attention_hbm_bytes(n: int, elem_bytes: int = 2) -> int:
    """The dominant N^2 HBM traffic of materialising attention: S written, S read and P written,
    P read: about 4 N^2 elements ("Bellek Duvarının Fiziği" section of the same page)."""
    return 4 * n * n * elem_bytes


def kv_cache_bytes_per_token(d_model: int, n_layers: int, elem_bytes: int) -> int:
    """K and V of one token across all layers ("Duvarın Ötesi")."""
    return 2 * d_model * n_layers * elem_bytes


def decode_bytes(B: int, H: int, n_k: int, d: int, elem_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one decode step: every K and V element read once, plus the
    query read and the output and log-sum-exp written."""
    kv = 2 * B * H * n_k * d * elem_bytes
    q_o = 2 * B * H * d * elem_bytes
    lse = B * H * 4
    return kv + q_o + lse


def fwd_compulsory_bytes(B: int, H: int, n_q: int, n_k: int, d: int, elem_bytes: int = 2) -> int:
    """Bytes a fused forward must move at least once: Q, K, V read, O and LSE written."""
    return (2 * B * H * n_q * d + 2 * B * H * n_k * d) * elem_bytes + B * H * n_q * 4
