"""CPU oracle for the FP8 forward with incoherent processing.

TEST INFRASTRUCTURE ONLY (like oracle/attention.py): nothing in the product path may import,
call or execute this module; it shares no code with the HIP kernels.

Sources.
  [FA3] "FlashAttention-3 (TR)" (systems-analysis.info wiki), section "Kuantizasyon Hatasını
        Azaltarak Düşük Hassasiyet (FP8) Kullanımı": before attention, Q and K are multiplied by
        a random orthogonal matrix (a Hadamard matrix, for example); this spreads outlier
        magnitudes over all coordinates; then Q and K are quantized to FP8; because the matrix is
        orthogonal it cancels in Q K^T. Reported effect: about 2.6x lower attention error than
        plain FP8.
  [MW]  "Bellek Duvarının Fiziği", section on FlashAttention-3: FP8 with block-wise scaling and
        incoherent processing (random sign multipliers).

The method is an approximation, so this oracle takes its steps in that order:
  1. incoherent processing: Q~ = Q M and K~ = K M with M = diag(sigma) H_d / sqrt(d), H_d the
     Sylvester-Hadamard matrix and sigma random signs (V is not rotated: it is not part of Q K^T);
  2. block-wise FP8 quantization of Q~, K~ and V;
  3. attention on the dequantized tensors, with the probabilities also quantized to FP8 for the
     P V product.

Readings (each also in the design notes):
  * FP8 = OCP E4M3 (4 exponent bits, bias 7, 3 mantissa bits, largest finite 448, subnormals down
    to 2^-9, round to nearest even); values are clamped to +-448 before rounding;
  * the orthogonal matrix: M = diag(sigma) H_d / sqrt(d) with H_d the Sylvester-Hadamard matrix
    (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]); the rotated rows x M are formed here as an
    fp64 matrix product (exact up to fp64 rounding, far below any E4M3 step);
  * signs: sigma_i = -1 iff bit i of the 128-bit output of Philox-4x32-10 (oracle.dropout.philox)
    with counter (0, 0, 0, 0) and key (seed mod 2^32, seed div 2^32) is set (bit i = bit i mod 32
    of word i div 32);
  * block scales: Q per 32 rows, K per 64 rows, V per head; s = amax / 448 computed in fp64 from
    the block's largest |x| and stored as the nearest fp32 value (s = 1 if amax = 0); the code of
    x is E4M3(clamp(x / s, -448, 448)) with x / s an fp64 quotient, rounded once. An
    implementation that evaluates these steps in fp32 reaches the same codes except where the
    quotient lies within its fp32 evaluation error of a midpoint between two E4M3 values; there
    the code may be the neighbouring one (quantize_head returns the quotients so that a test can
    tell such ties apart);
  * probabilities: P = exp(S - m) with m the row maximum of the scores of the dequantized
    Q and K; the P V product uses E4M3(256 P) / 256 (2^8 puts P's range [0, 1] into E4M3's
    normal range); O = sum_j P^_j V^_j / sum_j P_j (normaliser from the unquantized P);
    L = m + ln sum_j P_j. A streaming implementation quantizes P relative to a running maximum,
    which may sit below the final one (up to 2^0.5 in P), so its P codes may sit on a shifted
    grid: O is compared with a tolerance derived from the E4M3 step (o_tolerance), not bit for
    bit.
"""
from __future__ import annotations

import math

import numpy as np

from . import attention as A
from . import dropout as DR

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
Q_BLOCK_ROWS = 32
K_BLOCK_ROWS = 64
P_SCALE = 256.0


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to even; |x| > 448 (after rounding) gives NaN, as
    the conversion does without saturation. fp64 in, fp64 out."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a >= E4M3_MIN_NORMAL, np.exp2(e - 3), E4M3_SUBNORMAL_STEP)
    r = np.rint(a / step) * step  # np.rint rounds half to even
    r = np.where(r > E4M3_MAX, np.nan, r)
    return np.copysign(r, x)


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 bit patterns (uint8): sign, 4-bit exponent (bias 7), 3-bit mantissa;
    exponent 0 is subnormal; 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def e4m3_encode(x) -> np.ndarray:
    """Bit patterns of e4m3_round(x) (x finite and within +-448 after rounding)."""
    r = e4m3_round(x)
    a = np.abs(r)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    normal = a >= E4M3_MIN_NORMAL
    m_sub = np.rint(a / E4M3_SUBNORMAL_STEP).astype(np.int64)
    m_norm = np.rint((a / np.exp2(e) - 1.0) * 8.0).astype(np.int64)
    code = np.where(normal, ((e.astype(np.int64) + 7) << 3) | m_norm, m_sub)
    return (code | np.where(np.signbit(r), 0x80, 0)).astype(np.uint8)


def hadamard_signs(seed: int, d: int) -> np.ndarray:
    """+-1 signs sigma_0 .. sigma_{d-1} (reading above), d <= 128."""
    w = DR.philox([[0, 0, 0, 0]], (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))[0]
    bits = [(int(w[i // 32]) >> (i % 32)) & 1 for i in range(d)]
    return np.where(np.array(bits) == 1, -1.0, 1.0)


def sylvester_hadamard(d: int) -> np.ndarray:
    """H_d by the Sylvester recursion H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]] (d a power of
    two), as fp64 entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(signs) -> np.ndarray:
    """M = diag(signs) H_d / sqrt(d), fp64 (orthogonal)."""
    sg = np.asarray(signs, dtype=np.float64)
    d = sg.shape[0]
    return (sg[:, None] * sylvester_hadamard(d)) / math.sqrt(d)


def rotate(x, signs) -> np.ndarray:
    """Rows of x times M = diag(signs) H_d / sqrt(d), as an fp64 matrix product."""
    return np.asarray(x, dtype=np.float64) @ rotation_matrix(signs)


def block_scale(rows) -> np.float32:
    """s = amax / 448 of one block (fp64 quotient, stored as the nearest fp32); 1 if amax = 0."""
    amax = float(np.max(np.abs(rows))) if np.size(rows) else 0.0
    return np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)


def quantize_rows(x, block_rows: int | None):
    """E4M3 codes and fp32 scales of [n, d] rows, one scale per block of block_rows rows (None:
    one scale for all rows). Returns (codes uint8 [n, d], scales float32 [nblocks], quotients
    fp64 [n, d]): the code of x is E4M3(clamp(x / s, -448, 448)), x / s taken in fp64."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    br = n if block_rows is None else block_rows
    nb = max(1, -(-n // br)) if n else 0
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.ones(nb, dtype=np.float32)
    quot = np.zeros(x.shape, dtype=np.float64)
    for blk in range(nb):
        rows = x[blk * br:(blk + 1) * br]
        s = block_scale(rows)
        scales[blk] = s
        y = rows / np.float64(s)
        quot[blk * br:(blk + 1) * br] = y
        codes[blk * br:(blk + 1) * br] = e4m3_encode(np.clip(y, -E4M3_MAX, E4M3_MAX))
    return codes, scales, quot


def dequantize_rows(codes, scales, block_rows: int | None) -> np.ndarray:
    v = e4m3_decode(codes)
    n = v.shape[0]
    br = n if block_rows is None else block_rows
    s = np.repeat(np.asarray(scales, dtype=np.float64), br)[:n]
    return v * s[:, None]


def prepare_head(q, k, v, incoherent: bool, seed: int):
    """Steps 1 and 2 for one head: a dict of codes and scales (q8, sq, k8, sk, v8, sv), the
    quantized quotients x / s (qy, ky, vy) and the rows before quantization (qr, kr: rotated
    when incoherent, vr), all fp64."""
    d = np.shape(q)[-1]
    qr = np.asarray(q, dtype=np.float64)
    kr = np.asarray(k, dtype=np.float64)
    vr = np.asarray(v, dtype=np.float64)
    if incoherent:
        sg = hadamard_signs(seed, d)
        qr, kr = rotate(qr, sg), rotate(kr, sg)
    q8, sq, qy = quantize_rows(qr, Q_BLOCK_ROWS)
    k8, sk, ky = quantize_rows(kr, K_BLOCK_ROWS)
    v8, sv, vy = quantize_rows(vr, None)
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv, qy=qy, ky=ky, vy=vy, qr=qr, kr=kr,
                vr=vr)


def e4m3_tie_distance(y) -> np.ndarray:
    """Distance of each |y| (<= 448) to the nearest midpoint between two adjacent non-negative
    E4M3 values, i.e. how far y is from a point where its rounding would change."""
    vals = np.sort(e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))  # 0 .. 448, 127 values
    mids = (vals[1:] + vals[:-1]) / 2
    a = np.minimum(np.abs(np.asarray(y, dtype=np.float64)), E4M3_MAX)
    i = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    return np.minimum(np.abs(a - mids[i - 1]), np.abs(a - mids[i]))


def e4m3_code_index(codes) -> np.ndarray:
    """Signed position of each code on the ordered E4M3 value line (0 for both zeros), so that
    two codes of adjacent values differ by exactly one."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 0x7F  # magnitudes are ordered like their bit patterns
    return np.where(c & 0x80, -mag, mag)


def attention_from_codes(prep, scale: float, causal: bool, p_shift=0.0):
    """Step 3 for one head from prepare_head's codes: (o [n_q, d], lse [n_q]) in fp64.

    p_shift (default 0; a scalar or one value per row, in log2 units) quantizes each row's
    probabilities relative to a reference that sits p_shift below its maximum, as a streaming
    implementation with a running maximum does: P^ = E4M3(256 2^p_shift P) / (256 2^p_shift).
    The normaliser and L use the unquantized P either way."""
    qh = dequantize_rows(prep["q8"], prep["sq"], Q_BLOCK_ROWS)
    kh = dequantize_rows(prep["k8"], prep["sk"], K_BLOCK_ROWS)
    vh = dequantize_rows(prep["v8"], prep["sv"], None)
    s = A.scores(qh, kh, scale, causal)
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    z = np.sum(p, axis=1, keepdims=True)
    g = P_SCALE * np.exp2(np.reshape(np.asarray(p_shift, dtype=np.float64), (-1, 1)))
    p_hat = e4m3_round(g * p) / g
    o = (p_hat @ vh) / z
    return o, (m + np.log(z))[:, 0]


def forward_fp8(q, k, v, scale: float, causal: bool, incoherent: bool, seed: int):
    """Batched FP8 forward: q [B,H,n_q,d], k/v [B,H,n_k,d] (floats, normally bf16 values) ->
    (o, lse, preps) with preps[b][h] the codes and scales of each head."""
    B, H, n_q, d = np.shape(q)
    o = np.empty((B, H, n_q, np.shape(v)[3]), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    preps = []
    for b in range(B):
        row = []
        for h in range(H):
            pr = prepare_head(q[b, h], k[b, h], v[b, h], incoherent, seed)
            o[b, h], lse[b, h] = attention_from_codes(pr, scale, causal)
            row.append(pr)
        preps.append(row)
    return o, lse, preps


def o_tolerance(prep, scale: float, causal: bool) -> np.ndarray:
    """Per-element bound [n_q, d] on |O' - O| between this oracle's O (attention_from_codes) and
    an O' computed from the same codes whose probabilities were quantized on another grid (a
    reference maximum up to 2^0.5 away in P, see p_shift) and then rounded to bf16. Each
    quantized probability lies within half an E4M3 step of P: relative 2^-4 in the normal range,
    at most 2^0.5 2^-10 / 256 absolute below it. Both outputs carry such an error per key, so
    |O' - O| <= 2 (2^-4 sum_j P_j |v_j| + 2^0.5 (2^-10 / 256) sum_j |v_j|) / sum_j P_j,
    plus the bf16 rounding of O' (2^-8 |O|, above half a bf16 step)."""
    qh = dequantize_rows(prep["q8"], prep["sq"], Q_BLOCK_ROWS)
    kh = dequantize_rows(prep["k8"], prep["sk"], K_BLOCK_ROWS)
    vh = np.abs(dequantize_rows(prep["v8"], prep["sv"], None))
    s = A.scores(qh, kh, scale, causal)
    p = np.exp(s - np.max(s, axis=1, keepdims=True))
    z = np.sum(p, axis=1, keepdims=True)
    vis = np.isfinite(s).astype(np.float64)
    rel = 2.0 ** -4 * (p @ vh)
    sub = 2.0 ** -10 / P_SCALE * math.sqrt(2.0) * (vis @ vh)
    o = np.abs((e4m3_round(P_SCALE * p) / P_SCALE) @ dequantize_rows(prep["v8"], prep["sv"], None)) / z
    return 2.0 * (rel + sub) / z + 2.0 ** -8 * o + 1e-6
