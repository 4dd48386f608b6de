"""The CPU oracle against its pins, and planted mistakes in the oracle that the pins must catch."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.attention as A
import oracle.dropout as DR
import oracle.fp8 as F8
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_batched_matches_per_head():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 3, 9, 8))
    k = rng.standard_normal((2, 3, 13, 8))
    v = rng.standard_normal((2, 3, 13, 8))
    do = rng.standard_normal((2, 3, 9, 8))
    o, lse = oracle.forward(q, k, v, 0.3, True)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.3, True)
    for b in range(2):
        for h in range(3):
            oh, lh = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.3, True)
            assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, lse[b, h])
            gh = oracle.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.3, True)
            for x, y in zip(gh, (dq[b, h], dk[b, h], dv[b, h])):
                assert np.array_equal(x, y)


def test_row_subset_and_row_blocks(monkeypatch):
    """Rows computed alone, or in small row blocks, agree with the whole head."""
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((40, 8)), rng.standard_normal((50, 8)), rng.standard_normal((50, 8)))
    o, lse = oracle.forward_head(q, k, v, 0.4, True)
    rows = np.array([0, 7, 39])
    o2, lse2 = oracle.forward_head(q, k, v, 0.4, True, rows=rows)
    np.testing.assert_allclose(o2, o[rows], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse2, lse[rows], rtol=1e-14, atol=1e-15)
    monkeypatch.setattr(A, "_ROW_BLOCK_ELEMS", 3 * 50)
    o3, lse3 = oracle.forward_head(q, k, v, 0.4, True)
    np.testing.assert_allclose(o3, o, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse3, lse, rtol=1e-14, atol=1e-15)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.visible(5, 4, True)
    with pytest.raises(ValueError):
        oracle.decode(np.zeros((1, 1, 2, 4)), np.zeros((1, 1, 3, 4)), np.zeros((1, 1, 3, 4)), 1.0)


# ---- planted mistakes (in the oracle, on the CPU): each one must make some pin fail ----------

_orig_scores = A.scores
_orig_softmax = A.softmax_rows
_orig_visible = A.visible


def _scores_no_scale(q, k, scale, causal, rows=None):
    return _orig_scores(q, k, 1.0, causal, rows)


def _scores_transposed(q, k, scale, causal, rows=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (k @ q.T)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = s[rows]
    s[~_orig_visible(q.shape[0], k.shape[0], causal)[rows]] = -np.inf
    return s


def _visible_off_by_one(n_q, n_k, causal):
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i + (n_k - n_q) + 1


def _visible_top_left(n_q, n_k, causal):
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    return np.arange(n_k)[None, :] <= np.arange(n_q)[:, None]


def _softmax_lse_without_max(s):
    p, lse = _orig_softmax(s)
    m = np.max(s, axis=1)
    return p, lse - m


def _softmax_columns(s):
    m = np.max(s, axis=0, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=0, keepdims=True)
    return e / z, (m + np.log(z))[0, : s.shape[0]] if s.shape[0] <= s.shape[1] else np.zeros(s.shape[0])


def _bwd_factory(variant):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        p, _ = A.softmax_rows(A.scores(q, k, scale, causal))
        dv = p.T @ do
        dp = do @ v.T
        row = np.sum(p * dp, axis=1, keepdims=True)
        ds = p * (dp - row)
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if variant == "no_row_term":
            ds = p * dp
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        elif variant == "sign":
            ds = p * (row - dp)
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        elif variant == "dk_no_scale":
            dk = ds.T @ q
        elif variant == "dv_no_transpose":
            dv = (p @ do) if p.shape[0] == p.shape[1] else dv * 0.5
        elif variant == "dq_uses_v":
            dq = scale * (ds @ v)
        return dq, dk, dv
    return bwd


_orig_gather = A.gather_paged


def _gather_block_and_row_swapped(cache, block_table_row, seq_len, kv_head):
    cache = np.asarray(cache)
    bs = cache.shape[2]
    j = np.arange(seq_len)
    blocks = np.asarray(block_table_row)[np.minimum(j % bs, len(block_table_row) - 1)]
    return np.asarray(cache[blocks, kv_head, np.minimum(j // bs, bs - 1)], dtype=np.float64)


def _gather_physical_order(cache, block_table_row, seq_len, kv_head):
    # ignores the block table: reads blocks 0, 1, 2, ... in physical order
    cache = np.asarray(cache)
    bs = cache.shape[2]
    j = np.arange(seq_len)
    return np.asarray(cache[j // bs, kv_head, j % bs], dtype=np.float64)


def _decode_paged_head_modulo(q, k_cache, v_cache, block_table, seq_lens, scale):
    # query head h reads key/value head h % H_kv instead of h // (H // H_kv)
    B, H, d = np.shape(q)
    H_kv = np.shape(k_cache)[1]
    o = np.zeros((B, H, d))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        for h in range(H):
            kk = A.gather_paged(k_cache, block_table[b], n, h % H_kv)
            vv = A.gather_paged(v_cache, block_table[b], n, h % H_kv)
            ob, lb = A.forward_head(np.asarray(q[b, h])[None, :], kk, vv, scale, causal=False)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


_orig_fwd_varlen = A.forward_varlen
_orig_bwd_varlen = A.backward_varlen


def _visible_varlen_top_left(l_q, l_k, causal):
    if not causal:
        return np.ones((l_q, l_k), dtype=bool)
    return np.arange(l_k)[None, :] <= np.arange(l_q)[:, None]


def _visible_varlen_padded_shift(l_q, l_k, causal):
    # empty causal rows wrongly see the first key (a clamped shift)
    m = _orig_visible_varlen(l_q, l_k, causal)
    if causal and l_k > 0:
        m[:, 0] = True
    return m


def _fwd_varlen_full_keys(q, k, v, seq_lens_q, seq_lens_k, scale, causal):
    return _orig_fwd_varlen(q, k, v, seq_lens_q, np.full(len(seq_lens_k), np.shape(k)[2]),
                            scale, causal)


def _bwd_varlen_do_unaligned(q, k, v, do, seq_lens_q, seq_lens_k, scale, causal):
    # takes dO from the first rows of the sequence instead of the live rows
    do = np.array(do, dtype=np.float64)
    for b in range(np.shape(q)[0]):
        lq = min(max(int(seq_lens_q[b]), 0), np.shape(q)[2])
        lk = min(max(int(seq_lens_k[b]), 0), np.shape(k)[2])
        r0 = max(0, lq - lk) if causal else 0
        if lk > 0 and r0 > 0:
            do[b, :, r0:lq] = do[b, :, :lq - r0].copy()
    return _orig_bwd_varlen(q, k, v, do, seq_lens_q, seq_lens_k, scale, causal)


_orig_visible_varlen = A.visible_varlen


_orig_philox = DR.philox
_orig_keep = DR.dropout_keep
_orig_fwd_drop = DR.forward_dropout
_orig_bwd_drop = DR.backward_dropout


def _philox_no_key_schedule(counters, key, word_bits=32, rounds=10):
    saved = DR.PHILOX_W[word_bits]
    DR.PHILOX_W[word_bits] = (0, 0)
    try:
        return _orig_philox(counters, key, word_bits, rounds)
    finally:
        DR.PHILOX_W[word_bits] = saved


def _philox_outputs_reversed(counters, key, word_bits=32, rounds=10):
    return _orig_philox(counters, key, word_bits, rounds)[:, ::-1]


def _keep_transposed(seed, offset, bh, n_q, n_k, p):
    return _orig_keep(seed, offset, bh, n_k, n_q, p).T


def _keep_high_half_first(seed, offset, bh, n_q, n_k, p):
    n8 = (n_k + 7) // 8 * 8
    m = _orig_keep(seed, offset, bh, n_q, n8, p)
    m = m.reshape(n_q, n8 // 2, 2)[:, :, ::-1].reshape(n_q, n8)
    return m[:, :n_k]


def _keep_threshold_rounded(p):
    if not (0.0 <= p < 1.0):
        raise ValueError
    return int(round((1.0 - p) * 65536.0))


def _fwd_drop_renormalised(q, k, v, scale, causal, p, seed, offset):
    B, H, n_q, _ = np.shape(q)
    n_k = np.shape(k)[2]
    o = np.empty((B, H, n_q, np.shape(v)[3]))
    lse = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            P, lse[b, h] = A.softmax_rows(A.scores(q[b, h], k[b, h], scale, causal))
            Pz = P * DR.dropout_keep(seed, offset, b * H + h, n_q, n_k, p)
            o[b, h] = (Pz / np.maximum(Pz.sum(axis=1, keepdims=True), 1e-300)) @ v[b, h]
    return o, lse


def _fwd_drop_no_inverse_scale(q, k, v, scale, causal, p, seed, offset):
    o, lse = _orig_fwd_drop(q, k, v, scale, causal, p, seed, offset)
    return o * (1.0 - p), lse


def _bwd_drop_unmasked_dp(q, k, v, do, scale, causal, p, seed, offset):
    # the mask applied to dV only, not to dP
    dq, dk, dv = _orig_bwd_drop(q, k, v, do, scale, causal, p, seed, offset)
    gq, gk, _ = A.backward(q, k, v, do, scale, causal)
    return gq, gk, dv


_orig_e4m3_round = F8.e4m3_round
_orig_rotate = F8.rotate
_orig_att_codes = F8.attention_from_codes


def _e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)
    r = np.floor(a / step + 0.5) * step
    return np.copysign(np.where(r > 448, np.nan, r), x)


def _rotate_unnormalised(x, signs):
    return _orig_rotate(x, signs) * np.sqrt(np.shape(x)[-1])


def _hadamard_other_recursion(d):
    # [[H, H], [-H, H]]: also orthogonal, but not the Sylvester matrix
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [-h, h]])
    return h


def _block_scale_from_fp32_amax_halved(rows):
    amax = float(np.max(np.abs(rows))) if np.size(rows) else 0.0
    return np.float32(amax / 224.0) if amax > 0 else np.float32(1.0)


_orig_tol = F8.o_tolerance


def _o_tolerance_no_normaliser(prep, scale, causal):
    # the bound without its division by sum(P): far too loose
    qh = F8.dequantize_rows(prep["q8"], prep["sq"], F8.Q_BLOCK_ROWS)
    kh = F8.dequantize_rows(prep["k8"], prep["sk"], F8.K_BLOCK_ROWS)
    s = A.scores(qh, kh, scale, causal)
    z = np.sum(np.exp(s - np.max(s, axis=1, keepdims=True)), axis=1, keepdims=True)
    return _orig_tol(prep, scale, causal) * z


def _rotate_no_signs(x, signs):
    return _orig_rotate(x, np.ones_like(np.asarray(signs)))


def _att_codes_unshifted_p(prep, scale, causal):
    saved = F8.P_SCALE
    F8.P_SCALE = 1.0
    try:
        return _orig_att_codes(prep, scale, causal)
    finally:
        F8.P_SCALE = saved


def _att_codes_quantized_normaliser(prep, scale, causal):
    qh = F8.dequantize_rows(prep["q8"], prep["sq"], F8.Q_BLOCK_ROWS)
    kh = F8.dequantize_rows(prep["k8"], prep["sk"], F8.K_BLOCK_ROWS)
    vh = F8.dequantize_rows(prep["v8"], prep["sv"], None)
    s = A.scores(qh, kh, scale, causal)
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    ph = F8.e4m3_round(256 * p) / 256
    return (ph @ vh) / ph.sum(axis=1, keepdims=True), (m + np.log(p.sum(axis=1, keepdims=True)))[:, 0]


_orig_fwd_bias = A.forward_bias
_orig_bwd_bias = A.backward_bias


def _fwd_bias_scaled(q, k, v, bias, scale, causal):
    # the bias multiplied by the scale as well
    return _orig_fwd_bias(q, k, v, np.asarray(bias, dtype=np.float64) * scale, scale, causal)


def _fwd_bias_transposed(q, k, v, bias, scale, causal):
    b = np.asarray(bias, dtype=np.float64)
    n_q, n_k = np.shape(q)[2], np.shape(k)[2]
    b = np.broadcast_to(b, (np.shape(q)[0], np.shape(q)[1], n_q, n_k))
    if n_q == n_k:
        b = np.swapaxes(b, -1, -2)
    return _orig_fwd_bias(q, k, v, b, scale, causal)


_orig_fwd_gqa = A.forward_gqa
_orig_bwd_gqa = A.backward_gqa


def _fwd_gqa_head_modulo(q, k, v, scale, causal):
    # query head h paired with key/value head h % H_kv instead of h // (H // H_kv)
    B, H = np.shape(q)[:2]
    H_kv = np.shape(k)[1]
    o = np.empty(np.shape(q))
    lse = np.empty(np.shape(q)[:3])
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = A.forward_head(q[b, h], k[b, h % H_kv], v[b, h % H_kv], scale,
                                                causal)
    return o, lse


def _bwd_gqa_last_head_only(q, k, v, do, scale, causal):
    # the group's key/value gradients overwritten by each query head instead of summed
    B, H = np.shape(q)[:2]
    H_kv = np.shape(k)[1]
    dq = np.empty(np.shape(q))
    dk = np.zeros(np.shape(k))
    dv = np.zeros(np.shape(v))
    for b in range(B):
        for h in range(H):
            g = h // (H // H_kv)
            dq[b, h], dk[b, g], dv[b, g] = A.backward_head(q[b, h], k[b, g], v[b, g], do[b, h],
                                                           scale, causal)
    return dq, dk, dv


import oracle.combined as OC  # noqa: E402

_orig_fwd_comb = OC.forward_combined
_orig_bwd_comb = OC.backward_combined


def _fwd_comb_mask_of_kv_head(q, k, v, seq_lens_q, seq_lens_k, scale, causal, p, seed, offset):
    # the keep mask drawn for the key/value head instead of the query head
    B, H = np.shape(q)[:2]
    H_kv = np.shape(k)[1]
    saved = DR.dropout_keep
    DR.dropout_keep = lambda sd, off, bh, n_q, n_k, p_: saved(
        sd, off, (bh // H) * H_kv + (bh % H) // (H // H_kv), n_q, n_k, p_)
    try:
        return _orig_fwd_comb(q, k, v, seq_lens_q, seq_lens_k, scale, causal, p, seed, offset)
    finally:
        DR.dropout_keep = saved


def _bwd_comb_last_head_only(q, k, v, do, seq_lens_q, seq_lens_k, scale, causal, p, seed, offset):
    # the key/value gradients overwritten by each query head instead of summed over the group
    H, H_kv = np.shape(q)[1], np.shape(k)[1]
    G = H // H_kv
    dq, dk, dv = _orig_bwd_comb(q, k, v, do, seq_lens_q, seq_lens_k, scale, causal, p, seed,
                                offset)
    keep = [h for h in range(H) if h % G == G - 1]
    _, dk1, dv1 = _orig_bwd_comb(q[:, keep], k, v, do[:, keep], seq_lens_q, seq_lens_k, scale,
                                 causal, p, seed, offset)
    return dq, dk1, dv1


def _fwd_comb_first_lengths(q, k, v, seq_lens_q, seq_lens_k, scale, causal, p, seed, offset):
    # every sequence given the lengths of the first one
    B = np.shape(q)[0]
    lq = None if seq_lens_q is None else [seq_lens_q[0]] * B
    lk = None if seq_lens_k is None else [seq_lens_k[0]] * B
    return _orig_fwd_comb(q, k, v, lq, lk, scale, causal, p, seed, offset)


MUTANTS = {
    "gqa_head_modulo_fwd": ("forward_gqa", _fwd_gqa_head_modulo),
    "gqa_bwd_not_summed": ("backward_gqa", _bwd_gqa_last_head_only),
    "paged_block_and_row_swapped": ("gather_paged", _gather_block_and_row_swapped),
    "paged_ignores_block_table": ("gather_paged", _gather_physical_order),
    "gqa_head_modulo": ("decode_paged", _decode_paged_head_modulo),
    "varlen_mask_top_left": ("visible_varlen", _visible_varlen_top_left),
    "varlen_empty_rows_see_key0": ("visible_varlen", _visible_varlen_padded_shift),
    "varlen_ignores_key_lengths": ("forward_varlen", _fwd_varlen_full_keys),
    "varlen_bwd_do_unaligned": ("backward_varlen", _bwd_varlen_do_unaligned),
    "philox_no_key_schedule": ("philox", _philox_no_key_schedule, DR),
    "philox_outputs_reversed": ("philox", _philox_outputs_reversed, DR),
    "dropout_mask_transposed": ("dropout_keep", _keep_transposed, DR),
    "dropout_high_half_first": ("dropout_keep", _keep_high_half_first, DR),
    "dropout_threshold_rounded": ("keep_threshold", _keep_threshold_rounded, DR),
    "dropout_renormalised": ("forward_dropout", _fwd_drop_renormalised, DR),
    "dropout_no_inverse_scale": ("forward_dropout", _fwd_drop_no_inverse_scale, DR),
    "dropout_bwd_unmasked_dp": ("backward_dropout", _bwd_drop_unmasked_dp, DR),
    "fp8_ties_away_from_zero": ("e4m3_round", _e4m3_ties_away, F8),
    "bias_scaled_with_scores": ("forward_bias", _fwd_bias_scaled),
    "bias_transposed": ("forward_bias", _fwd_bias_transposed),
    "fp8_rotation_unnormalised": ("rotate", _rotate_unnormalised, F8),
    "fp8_rotation_without_signs": ("rotate", _rotate_no_signs, F8),
    "fp8_hadamard_other_recursion": ("sylvester_hadamard", _hadamard_other_recursion, F8),
    "fp8_scale_amax_over_224": ("block_scale", _block_scale_from_fp32_amax_halved, F8),
    "fp8_tolerance_without_normaliser": ("o_tolerance", _o_tolerance_no_normaliser, F8),
    "fp8_q_blocks_of_64": ("Q_BLOCK_ROWS", 64, F8),
    "fp8_p_unshifted": ("attention_from_codes", _att_codes_unshifted_p, F8),
    "fp8_normaliser_from_quantized_p": ("attention_from_codes", _att_codes_quantized_normaliser, F8),
    "scores_no_scale": ("scores", _scores_no_scale),
    "scores_transposed": ("scores", _scores_transposed),
    "mask_off_by_one": ("visible", _visible_off_by_one),
    "mask_top_left": ("visible", _visible_top_left),
    "lse_without_max": ("softmax_rows", _softmax_lse_without_max),
    "softmax_over_columns": ("softmax_rows", _softmax_columns),
    "bwd_no_row_term": ("backward_head", _bwd_factory("no_row_term")),
    "bwd_sign": ("backward_head", _bwd_factory("sign")),
    "bwd_dk_no_scale": ("backward_head", _bwd_factory("dk_no_scale")),
    "bwd_dv_no_transpose": ("backward_head", _bwd_factory("dv_no_transpose")),
    "bwd_dq_uses_v": ("backward_head", _bwd_factory("dq_uses_v")),
    "combined_mask_of_kv_head": ("forward_combined", _fwd_comb_mask_of_kv_head, OC),
    "combined_dkdv_not_summed": ("backward_combined", _bwd_comb_last_head_only, OC),
    "combined_first_lengths": ("forward_combined", _fwd_comb_first_lengths, OC),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn, *mod = MUTANTS[name]
    monkeypatch.setattr(mod[0] if mod else A, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # an assertion, or the mistake breaking a shape
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
