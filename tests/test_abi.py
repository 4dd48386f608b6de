"""The C ABI on the host: libfa.so loads without a GPU, exports every entry point include/fa.h
declares, and rejects bad arguments before anything reaches the device (no compute calls)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from exact_attention_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from exact_attention_fa_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names == sorted(_lib.SIGNATURES), "binding and header disagree"
    for n in names:
        assert hasattr(lib, n), f"{n} not exported by libfa.so"
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.fa_status_string(code).decode().startswith(name)
    assert lib.fa_status_string(1234).decode() == "FA_ERR_UNKNOWN"


FAKE = 1 << 20  # a 16-byte aligned non-null value; never dereferenced on error paths


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=8, Nk=8, d=64, scale=0.125,
         causal=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, None)


def test_fwd_validation(lib):
    assert _fwd(lib, q=None) == 1
    assert _fwd(lib, lse=None) == 1
    assert _fwd(lib, B=0) == 2
    assert _fwd(lib, Nq=0) == 2
    assert _fwd(lib, Nk=-1) == 2
    assert _fwd(lib, B=1 << 16, H=1 << 8, Nq=1 << 8) == 2  # B*H*Nq reaches 2^31
    assert _fwd(lib, d=96) == 3
    assert _fwd(lib, d=256) == 3
    assert _fwd(lib, scale=0.0) == 7
    assert _fwd(lib, scale=float("nan")) == 7
    assert _fwd(lib, scale=float("inf")) == 7
    assert _fwd(lib, scale=-1.0) == 7
    assert _fwd(lib, Nq=9, Nk=8, causal=1) == 5
    assert _fwd(lib, q=FAKE + 8) == 4
    assert _fwd(lib, o=FAKE + 2) == 4


def test_per_head_extent_validation(lib):
    """One head whose rows span 2^31 bytes or more (N_k = 2^24 at d = 128, or 2^23 at d = 128 is
    the first size that does) is rejected before any launch: the kernels address inside a head
    with 32-bit byte offsets. Every call here gets fake pointers, so reaching a launch would
    fail differently."""
    big = 1 << 23                                  # 2^23 rows x 128 x 2 bytes = 2^31
    assert _fwd(lib, Nk=1 << 24, d=128) == 2
    assert _fwd(lib, Nk=big, d=128) == 2
    assert _fwd(lib, Nq=big, Nk=big, d=128) == 2
    assert _fwd(lib, Nk=1 << 24, d=64) == 2        # 2^24 x 64 x 2 = 2^31
    ws = lib.fa_bwd_workspace_bytes(1, 1, 8, big, 128)
    assert lib.fa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 1, 1, 8,
                      big, 128, 0.125, 0, None) == 2
    assert lib.fa_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 8, 1 << 24, 128, 0.125, 0,
                          None) == 2
    assert lib.fa_fwd_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 1 << 24, 128, 0.125, 0,
                              0.1, 1, 0, None) == 2
    # d_v wider than d: V's rows decide
    assert lib.fa_fwd_dv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, big, 64, 128, 0.125, 0,
                         None) == 2
    assert lib.fa_bwd_dv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 1, 1,
                         8, big, 64, 128, 0.125, 0, None) == 2
    wsd = lib.fa_decode_workspace_bytes(1, 1, 1 << 24, 128, 4)
    assert lib.fa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsd, 1, 1, 1, 1 << 24, 128, 0.125,
                         0, 4, None) == 2


def test_bwd_validation(lib):
    ws = lib.fa_bwd_workspace_bytes(2, 3, 100, 50, 64)
    assert ws >= 2 * 3 * 100 * 4 and ws % 16 == 0
    assert lib.fa_bwd_workspace_bytes(0, 3, 100, 50, 64) == 0

    def call(ws_ptr=FAKE, ws_bytes=ws, d=64, causal=0, Nq=100, Nk=50, dq=FAKE):
        return lib.fa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, ws_ptr, ws_bytes,
                          2, 3, Nq, Nk, d, 0.125, causal, None)
    assert call(dq=None) == 1
    assert call(d=80) == 3
    assert call(causal=1) == 5
    assert call(ws_ptr=None) == 6
    assert call(ws_bytes=ws - 16) == 6
    assert call(ws_ptr=FAKE + 4) == 4
    assert call(dq=FAKE + 2) == 4


def test_varlen_validation(lib):
    def fwd(lq=FAKE, lk=FAKE, q=FAKE, d=64, B=2, scale=0.125, causal=1):
        return lib.fa_fwd_varlen(q, FAKE, FAKE, FAKE, FAKE, lq, lk, B, 3, 9, 8, d, scale,
                                 causal, None)
    assert fwd(lq=None) == 1
    assert fwd(lk=None) == 1
    assert fwd(q=None) == 1
    assert fwd(lq=FAKE + 2) == 4
    assert fwd(lk=FAKE + 1) == 4
    assert fwd(q=FAKE + 8) == 4
    assert fwd(d=96) == 3
    assert fwd(B=0) == 2
    assert fwd(scale=-1.0) == 7
    ws = lib.fa_bwd_workspace_bytes(2, 3, 9, 8, 64)

    def bwd(lq=FAKE, lk=FAKE, ws_bytes=ws, dk=FAKE, d=64):
        return lib.fa_bwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dk, FAKE, lq, lk,
                                 FAKE, ws_bytes, 2, 3, 9, 8, d, 0.125, 1, None)
    assert bwd(lq=None) == 1
    assert bwd(lk=FAKE + 2) == 4
    assert bwd(dk=None) == 1
    assert bwd(dk=FAKE + 2) == 4
    assert bwd(ws_bytes=ws - 16) == 6
    assert bwd(d=32) == 3


def test_dropout_validation(lib):
    def fwd(p=0.1, q=FAKE, d=64, causal=0, Nq=8):
        return lib.fa_fwd_dropout(q, FAKE, FAKE, FAKE, FAKE, 1, 2, Nq, 8, d, 0.125, causal, p,
                                  2**64 - 1, 7, None)
    assert fwd(p=-0.1) == 8
    assert fwd(p=1.0) == 8
    assert fwd(p=float("nan")) == 8
    assert fwd(p=float("inf")) == 8
    assert fwd(q=None) == 1
    assert fwd(d=96) == 3
    assert fwd(causal=1, Nq=9) == 5
    assert fwd(q=FAKE + 4) == 4
    ws = lib.fa_bwd_workspace_bytes(1, 2, 8, 8, 64)

    def bwd(p=0.1, ws_bytes=ws, dv=FAKE):
        return lib.fa_bwd_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dv, FAKE,
                                  ws_bytes, 1, 2, 8, 8, 64, 0.125, 0, p, 1, 0, None)
    assert bwd(p=1.5) == 8
    assert bwd(dv=None) == 1
    assert bwd(ws_bytes=ws - 16) == 6


def test_fp8_validation(lib):
    ws = lib.fa_fwd_fp8_workspace_bytes(2, 3, 100, 130, 128)
    assert ws >= 2 * 3 * (100 + 130 + 128 * 192) and ws % 256 == 0
    assert lib.fa_fwd_fp8_workspace_bytes(2, 3, 100, 130, 96) == 0
    assert lib.fa_fwd_fp8_workspace_bytes(0, 3, 100, 130, 64) == 0

    def call(q=FAKE, ws_ptr=FAKE, ws_bytes=ws, d=128, causal=0, Nq=100, scale=0.1):
        return lib.fa_fwd_fp8(q, FAKE, FAKE, FAKE, FAKE, 2, 3, Nq, 130, d, scale, causal, 1,
                              2**64 - 1, ws_ptr, ws_bytes, None)
    assert call(q=None) == 1
    assert call(d=96) == 3
    assert call(causal=1, Nq=131) == 5
    assert call(scale=0.0) == 7
    assert call(ws_ptr=None) == 6
    assert call(ws_bytes=ws - 1) == 6
    assert call(ws_ptr=FAKE + 8) == 4
    assert call(q=FAKE + 2) == 4


def test_bias_validation(lib):
    def fwd(bias=FAKE, sb=0, sh=0, sq=64, q=FAKE, d=64):
        return lib.fa_fwd_bias(q, FAKE, FAKE, FAKE, FAKE, bias, sb, sh, sq, 1, 2, 8, 8, d, 0.125,
                               0, None)
    assert fwd(bias=None) == 1
    assert fwd(bias=FAKE + 8) == 4
    assert fwd(sq=12) == 8
    assert fwd(sh=-8) == 8
    assert fwd(sb=4) == 8
    assert fwd(q=None) == 1
    assert fwd(d=80) == 3
    assert lib.fa_fwd_bias(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 1 << 28, 1, 1, 8, 8, 64,
                           0.125, 0, None) == 2
    ws = lib.fa_bwd_workspace_bytes(1, 2, 8, 8, 64)

    def bwd(bias=FAKE, sq=8, ws_bytes=ws):
        return lib.fa_bwd_bias(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bias, 0, 0, sq,
                               FAKE, ws_bytes, 1, 2, 8, 8, 64, 0.125, 1, None)
    assert bwd(bias=None) == 1
    assert bwd(sq=3) == 8
    assert bwd(ws_bytes=ws - 16) == 6


def test_dv_validation(lib):
    def fwd(dv_=64, d=128, q=FAKE):
        return lib.fa_fwd_dv(q, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 8, d, dv_, 0.125, 0, None)
    assert fwd(dv_=96) == 3
    assert fwd(d=80) == 3
    assert fwd(q=None) == 1
    assert fwd(q=FAKE + 4) == 4
    ws = lib.fa_bwd_workspace_bytes(1, 2, 8, 8, 128)
    assert lib.fa_bwd_dv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 8,
                         8, 128, 32, 0.125, 0, None) == 3
    assert lib.fa_bwd_dv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 16, 1,
                         2, 8, 8, 128, 64, 0.125, 0, None) == 6


def test_gqa_validation(lib):
    def fwd(H=4, Hkv=2, q=FAKE, causal=0, nq=8):
        return lib.fa_fwd_gqa(q, FAKE, FAKE, FAKE, FAKE, 1, H, Hkv, nq, 8, 64, 0.125, causal, None)
    assert fwd(H=4, Hkv=3) == 8      # H not a multiple of H_kv
    assert fwd(Hkv=0) == 8
    assert fwd(H=0) == 2
    assert fwd(q=None) == 1
    assert fwd(q=FAKE + 4) == 4
    assert fwd(causal=1, nq=9) == 5
    ws = lib.fa_bwd_gqa_workspace_bytes(1, 4, 2, 8, 8, 64)
    # one K/V tile per head: too few workgroups, so fp32 partial rows of dK and dV per query head
    assert ws == lib.fa_bwd_workspace_bytes(1, 4, 8, 8, 64) + 2 * 4 * 8 * 64 * 4
    assert lib.fa_bwd_gqa_workspace_bytes(1, 4, 3, 8, 8, 64) == 0
    # 8 K/V heads x 256 key tiles = 2048 workgroups: no partial rows
    assert (lib.fa_bwd_gqa_workspace_bytes(1, 32, 8, 64, 32768, 64)
            == lib.fa_bwd_workspace_bytes(1, 32, 64, 32768, 64))

    def bwd(H=4, Hkv=2, ws_bytes=ws, d=64):
        return lib.fa_bwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              ws_bytes, 1, H, Hkv, 8, 8, d, 0.125, 0, None)
    assert bwd(Hkv=3) == 8
    assert bwd(Hkv=0) == 8
    assert bwd(ws_bytes=ws - 16) == 6
    assert bwd(d=96) == 3


def test_decode_gqa_validation(lib):
    assert lib.fa_decode_gqa_num_splits(8, 32, 8, 65536, 128) == lib.fa_decode_paged_num_splits(
        8, 32, 8, 4096, 16, 128)
    assert lib.fa_decode_gqa_num_splits(8, 32, 32, 65536, 128) == lib.fa_decode_num_splits(
        8, 32, 65536, 128)
    ws = lib.fa_decode_gqa_workspace_bytes(2, 8, 2, 100, 64, 4)
    assert ws == 2 * 8 * 4 * 64 * 4 + 2 * 8 * 4 * 4
    assert lib.fa_decode_gqa_workspace_bytes(2, 8, 2, 100, 96, 4) == 0

    def dec(H=8, Hkv=2, q=FAKE, ws_bytes=ws, splits=4, nk=100, d=64):
        return lib.fa_decode_gqa(q, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, 2, H, Hkv, nk, d,
                                 0.125, splits, None)
    assert dec(Hkv=3) == 8       # H not a multiple of H_kv
    assert dec(Hkv=0) == 8
    assert dec(H=0) == 2
    assert dec(q=None) == 1
    assert dec(q=FAKE + 4) == 4
    assert dec(d=96) == 3
    assert dec(splits=101) == 8  # more splits than positions
    assert dec(splits=-1) == 8
    assert dec(ws_bytes=ws - 16) == 6


def test_bwd_phase_validation(lib):
    ws = lib.fa_bwd_workspace_bytes(1, 2, 64, 64, 128)
    assert ws == 2 * 2 * 64 * 4
    assert lib.fa_bwd_preprocess(None, FAKE, FAKE, FAKE, ws, 1, 2, 64, 64, 128, None) == 1
    assert lib.fa_bwd_preprocess(FAKE, None, FAKE, FAKE, ws, 1, 2, 64, 64, 128, None) == 1
    assert lib.fa_bwd_preprocess(FAKE, FAKE, FAKE, FAKE, ws - 16, 1, 2, 64, 64, 128, None) == 6
    assert lib.fa_bwd_preprocess(FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 64, 64, 48, None) == 3
    assert lib.fa_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, 1, 2, 64, 64, 128,
                           0.1, 0, None) == 1
    assert lib.fa_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 65, 64, 128,
                           0.1, 1, None) == 5
    assert lib.fa_bwd_dq(FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, 1, 2, 64, 64, 128, 0.1, 0,
                         None) == 1
    assert lib.fa_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, ws, 1, 2, 64, 64, 128, 0.1,
                         0, None) == 4


def test_decode_validation(lib):
    c = lib.fa_decode_num_splits(8, 32, 65536, 128)
    assert 1 <= c <= 1024
    assert lib.fa_decode_num_splits(1, 1, 10, 64) >= 1
    ws = lib.fa_decode_workspace_bytes(8, 32, 65536, 128, 0)
    assert ws == lib.fa_decode_workspace_bytes(8, 32, 65536, 128, c)
    assert ws >= 8 * 32 * c * (128 + 1) * 4
    assert lib.fa_decode_workspace_bytes(8, 32, 65536, 96, 0) == 0

    def call(Nq=1, splits=0, ws_bytes=ws, d=128, Nk=65536):
        return lib.fa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, 8, 32, Nq, Nk, d,
                             0.08, 0, splits, None)
    assert call(Nq=2) == 8
    assert call(splits=-1) == 8
    assert call(splits=1025) == 8
    assert call(splits=11, Nk=10) == 8
    assert call(ws_bytes=ws - 1) == 6
    assert call(d=32) == 3


def test_ext_validation(lib):
    """fa_fwd_ext / fa_bwd_ext: lengths both or neither, H a multiple of H_kv, p_drop in [0, 1),
    causal N_q > N_k only with lengths, the workspace of fa_bwd_ext_workspace_bytes."""
    def fwd(lq=FAKE, lk=FAKE, Hkv=2, Nq=8, Nk=8, causal=1, p=0.1, q=FAKE):
        return lib.fa_fwd_ext(q, FAKE, FAKE, FAKE, FAKE, lq, lk, 2, 4, Hkv, Nq, Nk, 64, 0.125,
                              causal, p, 1, 0, None)
    assert fwd(q=None) == 1
    assert fwd(lk=None) == 8 and fwd(lq=None) == 8
    assert fwd(Hkv=3) == 8 and fwd(Hkv=0) == 8
    assert fwd(p=1.0) == 8 and fwd(p=-0.1) == 8
    assert fwd(lq=None, lk=None, Nq=9, Nk=8) == 5
    assert fwd(lq=FAKE + 2) == 4
    ws = lib.fa_bwd_ext_workspace_bytes(2, 4, 2, 8, 8, 64)
    assert ws >= lib.fa_bwd_workspace_bytes(2, 4, 8, 8, 64) and ws % 16 == 0
    assert lib.fa_bwd_ext_workspace_bytes(2, 4, 3, 8, 8, 64) == 0

    def bwd(ws_bytes=ws, lk=FAKE, Hkv=2, p=0.1):
        return lib.fa_bwd_ext(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, lk,
                              FAKE, ws_bytes, 2, 4, Hkv, 8, 8, 64, 0.125, 1, p, 1, 0, None)
    assert bwd(ws_bytes=ws - 16) == 6
    assert bwd(lk=None) == 8
    assert bwd(Hkv=3) == 8
    assert bwd(p=2.0) == 8


def test_decode_noalloc_validation(lib):
    """fa_decode_noalloc validates like fa_decode and refuses, before any device call, a split
    count whose partials exceed its fixed 16 MiB array."""
    def call(q=FAKE, B=2, H=4, Nq=1, Nk=1000, d=128, splits=0):
        return lib.fa_decode_noalloc(q, FAKE, FAKE, FAKE, FAKE, B, H, Nq, Nk, d, 0.125, 0,
                                     splits, None)
    assert call(q=None) == 1
    assert call(Nq=2) == 8
    assert call(splits=1001) == 8
    assert call(d=96) == 3
    assert call(q=FAKE + 2) == 4
    # B8 H32 d128 at 1024 splits: 8 * 32 * 1024 * 129 * 4 bytes > 16 MiB
    assert lib.fa_decode_workspace_bytes(8, 32, 65536, 128, 1024) > (16 << 20)
    assert call(B=8, H=32, Nk=65536, splits=1024) == 6
    assert lib.fa_decode_workspace_bytes(8, 32, 65536, 128, 16) <= (16 << 20)


def test_decode_paged_validation(lib):
    # B8 H32 H_kv8, 512 blocks of 16 positions per sequence, d128
    c = lib.fa_decode_paged_num_splits(8, 32, 8, 512, 16, 128)
    assert 1 <= c <= 1024
    assert lib.fa_decode_paged_num_splits(1, 4, 3, 4, 16, 64) == 1  # H not a multiple of H_kv
    ws = lib.fa_decode_paged_workspace_bytes(8, 32, 8, 512, 16, 128, 0)
    assert ws == lib.fa_decode_paged_workspace_bytes(8, 32, 8, 512, 16, 128, c)
    assert ws >= 8 * 32 * c * (128 + 1) * 4 and ws % 16 == 0
    assert lib.fa_decode_paged_workspace_bytes(8, 32, 8, 512, 16, 96, 0) == 0

    def call(q=FAKE, table=FAKE, lens=FAKE, lse=FAKE, ws_ptr=FAKE, ws_bytes=ws, B=8, H=32,
             H_kv=8, d=128, bs=16, nblocks=4096, max_blocks=512, scale=0.08, splits=0):
        return lib.fa_decode_paged(q, FAKE, FAKE, table, lens, FAKE, lse, ws_ptr, ws_bytes, B, H,
                                   H_kv, d, bs, nblocks, max_blocks, scale, splits, None)
    assert call(q=None) == 1
    assert call(table=None) == 1
    assert call(lens=None) == 1
    assert call(B=0) == 2
    assert call(H_kv=0) == 2
    assert call(nblocks=0) == 2
    assert call(max_blocks=0) == 2
    assert call(d=80) == 3
    assert call(scale=0.0) == 7
    assert call(H=30) == 8                     # not a multiple of H_kv
    assert call(bs=24) == 8                    # not a power of two
    assert call(bs=8192) == 8
    assert call(splits=1025) == 8
    assert call(splits=-1) == 8
    assert call(splits=9, bs=1, max_blocks=8) == 8  # more splits than positions
    assert call(q=FAKE + 8) == 4
    assert call(table=FAKE + 2) == 4
    assert call(lse=FAKE + 1) == 4
    assert call(ws_ptr=None) == 6
    assert call(ws_bytes=ws - 16) == 6
