"""The Python binding rejects caller-supplied outputs and workspaces that do not match the
call (shape, dtype, contiguity, device) with ValueError before anything reaches the library, so
a wrong buffer can never be written out of bounds on the device."""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu


def _t(shape, dtype="bf16", dev="cuda"):
    import torch
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32}[dtype]
    return torch.zeros(shape, dtype=dt, device=dev)


def _bad_variants(shape, dtype):
    """(tensor, what) pairs that must be rejected where a tensor of `shape` and `dtype` is due."""
    import torch
    wrong_shape = list(shape)
    wrong_shape[-1] += 1
    other = "f32" if dtype == "bf16" else "bf16"
    big = _t(tuple(shape[:-1]) + (2 * shape[-1],), dtype)
    return [(_t(tuple(wrong_shape), dtype), "shape"), (_t(shape, other), "dtype"),
            (big[..., ::2], "strides"), (_t(shape, dtype, "cpu"), "device")]


def test_forward_outputs_rejected(gpu):
    B, H, N, d = 1, 2, 64, 64
    q, k, v = (_t((B, H, N, d)) for _ in range(3))
    lse = _t((B, H, N), "f32")
    calls = {
        "fwd": lambda out: gpu.fwd(q, k, v, out=out),
        "fwd_bias": lambda out: gpu.fwd_bias(q, k, v, _t((N, N)), out=out),
        "fwd_dv": lambda out: gpu.fwd_dv(q, k, v, out=out),
        "fwd_gqa": lambda out: gpu.fwd_gqa(q, k, v, out=out),
        "fwd_dropout": lambda out: gpu.fwd_dropout(q, k, v, 0.1, 1, out=out),
    }
    for name, call in calls.items():
        for bad, what in _bad_variants((B, H, N, d), "bf16"):
            with pytest.raises(ValueError):
                call((bad, lse))
        for bad, what in _bad_variants((B, H, N), "f32"):
            with pytest.raises(ValueError):
                call((_t((B, H, N, d)), bad))


def test_backward_outputs_and_workspace_rejected(gpu):
    B, H, N, d = 1, 2, 64, 64
    q, k, v, o, do = (_t((B, H, N, d)) for _ in range(5))
    lse = _t((B, H, N), "f32")
    calls = {
        "bwd": lambda out, ws=None: gpu.bwd(q, k, v, o, lse, do, out=out, workspace=ws),
        "bwd_bias": lambda out, ws=None: gpu.bwd_bias(q, k, v, o, lse, do, _t((N, N)), out=out,
                                                      workspace=ws),
        "bwd_dv": lambda out, ws=None: gpu.bwd_dv(q, k, v, o, lse, do, out=out, workspace=ws),
        "bwd_gqa": lambda out, ws=None: gpu.bwd_gqa(q, k, v, o, lse, do, out=out, workspace=ws),
        "bwd_dropout": lambda out, ws=None: gpu.bwd_dropout(q, k, v, o, lse, do, 0.1, 1, out=out,
                                                            workspace=ws),
    }
    good = lambda: tuple(_t((B, H, N, d)) for _ in range(3))  # noqa: E731
    for name, call in calls.items():
        for pos in range(3):
            for bad, what in _bad_variants((B, H, N, d), "bf16"):
                out = list(good())
                out[pos] = bad
                with pytest.raises(ValueError):
                    call(tuple(out))
        with pytest.raises(ValueError):
            call(good()[:2])
        with pytest.raises(ValueError):  # a workspace in host memory
            call(good(), ws=_t((1 << 16,), "f32", "cpu"))
    lens = _t((B,), "i32")
    for bad, what in _bad_variants((B, H, N, d), "bf16"):
        with pytest.raises(ValueError):
            gpu.bwd_varlen(q, k, v, o, lse, do, lens, lens, out=(bad, _t((B, H, N, d)),
                                                                 _t((B, H, N, d))))


def test_decode_outputs_rejected(gpu):
    B, H, N, d = 2, 4, 256, 64
    q = _t((B, H, 1, d))
    k, v = _t((B, H, N, d)), _t((B, H, N, d))
    for call in (lambda out: gpu.decode(q, k, v, out=out),
                 lambda out: gpu.decode_gqa(q, k[:, :2].contiguous(), v[:, :2].contiguous(),
                                            out=out)):
        for bad, what in _bad_variants((B, H, 1, d), "bf16"):
            with pytest.raises(ValueError):
                call((bad, _t((B, H, 1), "f32")))
        for bad, what in _bad_variants((B, H, 1), "f32"):
            with pytest.raises(ValueError):
                call((_t((B, H, 1, d)), bad))
