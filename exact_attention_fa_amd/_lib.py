"""ctypes binding of libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: torch provides device memory and the current HIP stream, and every
step of the computation runs in the library's kernels. There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM", 4: "FA_ERR_ALIGN",
          5: "FA_ERR_CAUSAL", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_SCALE", 8: "FA_ERR_ARG",
          9: "FA_ERR_HIP"}

# Every entry point include/fa.h declares: name -> (restype, argtypes)
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_U64, _U32, _I64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64
SIGNATURES = {
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_preprocess": (_I, [_P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _P]),
    "fa_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_num_splits": (_I, [_I, _I, _I, _I]),
    "fa_decode_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "fa_decode": (_I, [_P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_decode_noalloc": (_I, [_P] * 5 + [_I] * 5 + [_F, _I, _I, _P]),
    "fa_fwd_dv": (_I, [_P] * 5 + [_I] * 6 + [_F, _I, _P]),
    "fa_bwd_dv": (_I, [_P] * 10 + [_Z] + [_I] * 6 + [_F, _I, _P]),
    "fa_fwd_gqa": (_I, [_P] * 5 + [_I] * 6 + [_F, _I, _P]),
    "fa_bwd_gqa": (_I, [_P] * 10 + [_Z] + [_I] * 6 + [_F, _I, _P]),
    "fa_bwd_gqa_workspace_bytes": (_Z, [_I] * 6),
    "fa_fwd_bias": (_I, [_P] * 6 + [_I64] * 3 + [_I] * 5 + [_F, _I, _P]),
    "fa_bwd_bias": (_I, [_P] * 10 + [_I64] * 3 + [_P, _Z] + [_I] * 5 + [_F, _I, _P]),
    "fa_fwd_fp8_workspace_bytes": (_Z, [_I] * 5),
    "fa_fwd_fp8": (_I, [_P] * 5 + [_I] * 5 + [_F, _I, _I, _U64, _P, _Z, _P]),
    "fa_fwd_dropout": (_I, [_P] * 5 + [_I] * 5 + [_F, _I, _F, _U64, _U32, _P]),
    "fa_bwd_dropout": (_I, [_P] * 10 + [_Z] + [_I] * 5 + [_F, _I, _F, _U64, _U32, _P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_ext": (_I, [_P] * 7 + [_I] * 6 + [_F, _I, _F, _U64, _U32, _P]),
    "fa_bwd_ext_workspace_bytes": (_Z, [_I] * 6),
    "fa_bwd_ext": (_I, [_P] * 12 + [_Z] + [_I] * 6 + [_F, _I, _F, _U64, _U32, _P]),
    "fa_bwd_varlen": (_I, [_P] * 12 + [_Z, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_gqa_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "fa_decode_gqa_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "fa_decode_gqa": (_I, [_P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_paged_num_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "fa_decode_paged_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _I, _I, _I, _F,
                             _I, _P]),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m exact_attention_fa_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise FaError(fn, status)


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, name: str, shape, dtype) -> None:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(ws, nbytes: int, device):
    """A caller's workspace: a contiguous tensor on the GPU of at least nbytes bytes (the library
    checks the size again); None allocates one."""
    import torch
    if ws is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws


def _outs(out, specs):
    """Validate caller-supplied outputs: out is a tuple matched against specs, a list of
    (name, shape, dtype)."""
    if len(out) != len(specs):
        raise ValueError(f"out must hold {len(specs)} tensors")
    for t, (name, shape, dtype) in zip(out, specs):
        _need(t, name, shape, dtype)
    return out


def _scale(scale, d: int) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None):
    """O and LSE of exact attention. q [B,H,Nq,d], k/v [B,H,Nk,d] bf16 -> (o bf16, lse fp32)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, d), torch.bfloat16)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", (B, H, Nq, d), torch.bfloat16)
        _need(lse, "lse", (B, H, Nq), torch.float32)
    st = load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_fwd", st)
    return o, lse


def bwd_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, Nq, Nk, d))


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
        workspace=None, out=None):
    """Gradients (dq, dk, dv) of exact attention by recomputation from the stored LSE."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, H, Nk, d)), (v, "v", (B, H, Nk, d)),
                      (o, "o", (B, H, Nq, d)), (dout, "dout", (B, H, Nq, d))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    nbytes = bwd_workspace_bytes(B, H, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _outs(out, [("dq", tuple(q.shape), torch.bfloat16),
                                 ("dk", tuple(k.shape), torch.bfloat16),
                                 ("dv", tuple(v.shape), torch.bfloat16)])
    st = load().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       B, H, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_bwd", st)
    return dq, dk, dv


def bwd_phase(phase: str, q, k, v, o, lse, dout, dq, dk, dv, workspace, causal: bool = False,
              scale: float | None = None) -> None:
    """Run one backward phase ("preprocess", "dkdv" or "dq") into preallocated outputs."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, H, Nk, d)), (v, "v", (B, H, Nk, d)),
                      (o, "o", (B, H, Nq, d)), (dout, "dout", (B, H, Nq, d)),
                      (dq, "dq", (B, H, Nq, d)), (dk, "dk", (B, H, Nk, d)),
                      (dv, "dv", (B, H, Nk, d))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    lib = load()
    if workspace is None:
        raise ValueError("bwd_phase needs the workspace shared by the three phases")
    workspace = _workspace(workspace, 0, q.device)
    ws, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    sc, ca, st = _scale(scale, d), int(bool(causal)), _stream(q)
    if phase == "preprocess":
        r = lib.fa_bwd_preprocess(o.data_ptr(), lse.data_ptr(), dout.data_ptr(), ws, wsb, B, H,
                                  Nq, Nk, d, st)
    elif phase == "dkdv":
        r = lib.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                            dk.data_ptr(), dv.data_ptr(), ws, wsb, B, H, Nq, Nk, d, sc, ca, st)
    elif phase == "dq":
        r = lib.fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                          dq.data_ptr(), ws, wsb, B, H, Nq, Nk, d, sc, ca, st)
    else:
        raise ValueError(phase)
    _check("fa_bwd_" + phase, r)


def decode_num_splits(B: int, H: int, Nk: int, d: int) -> int:
    return int(load().fa_decode_num_splits(B, H, Nk, d))


def decode_workspace_bytes(B: int, H: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, Nk, d, num_splits))


def decode(q, k, v, scale: float | None = None, num_splits: int = 0, workspace=None, out=None):
    """One decode step: q [B,H,1,d] against k/v [B,H,Nk,d] -> (o [B,H,1,d] bf16, lse [B,H,1])."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, d), torch.bfloat16)
    nbytes = decode_workspace_bytes(B, H, Nk, d, num_splits)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = _outs(out, [("o", (B, H, Nq, d), torch.bfloat16),
                             ("lse", (B, H, Nq), torch.float32)])
    st = load().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          B, H, Nq, Nk, d, _scale(scale, d), 0, int(num_splits), _stream(q))
    _check("fa_decode", st)
    return o, lse


DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20  # FA_DECODE_NOALLOC_SCRATCH_BYTES of fa.h


def decode_noalloc(q, k, v, scale: float | None = None, num_splits: int = 0, out=None):
    """decode() with the split partials in the library's own device array instead of a
    workspace: the library allocates nothing (pass out=(o, lse) to allocate nothing here either).
    Calls that may overlap in time on one GPU race on that array."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, d), torch.bfloat16)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = _outs(out, [("o", (B, H, Nq, d), torch.bfloat16),
                             ("lse", (B, H, Nq), torch.float32)])
    st = load().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, H, Nq, Nk, d, _scale(scale, d), 0,
                                  int(num_splits), _stream(q))
    _check("fa_decode_noalloc", st)
    return o, lse


def decode_gqa_num_splits(B: int, H: int, H_kv: int, Nk: int, d: int) -> int:
    return int(load().fa_decode_gqa_num_splits(B, H, H_kv, Nk, d))


def decode_gqa_workspace_bytes(B: int, H: int, H_kv: int, Nk: int, d: int,
                               num_splits: int = 0) -> int:
    return int(load().fa_decode_gqa_workspace_bytes(B, H, H_kv, Nk, d, num_splits))


def decode_gqa(q, k, v, scale: float | None = None, num_splits: int = 0, workspace=None,
               out=None):
    """One decode step with grouped query heads: q [B,H,1,d] against k/v [B,H_kv,Nk,d]
    -> (o [B,H,1,d] bf16, lse [B,H,1] fp32)."""
    import torch
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    _need(q, "q", (B, H, 1, d), torch.bfloat16)
    _need(k, "k", (B, H_kv, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H_kv, Nk, d), torch.bfloat16)
    nbytes = decode_gqa_workspace_bytes(B, H, H_kv, Nk, d, num_splits)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
    else:
        o, lse = _outs(out, [("o", (B, H, 1, d), torch.bfloat16),
                             ("lse", (B, H, 1), torch.float32)])
    st = load().fa_decode_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), B, H, H_kv, Nk, d,
                              _scale(scale, d), int(num_splits), _stream(q))
    _check("fa_decode_gqa", st)
    return o, lse


def decode_paged_num_splits(B: int, H: int, H_kv: int, max_blocks: int, block_size: int,
                            d: int) -> int:
    return int(load().fa_decode_paged_num_splits(B, H, H_kv, max_blocks, block_size, d))


def decode_paged_workspace_bytes(B: int, H: int, H_kv: int, max_blocks: int, block_size: int,
                                 d: int, num_splits: int = 0) -> int:
    return int(load().fa_decode_paged_workspace_bytes(B, H, H_kv, max_blocks, block_size, d,
                                                      num_splits))


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale: float | None = None,
                 num_splits: int = 0, workspace=None, out=None):
    """One decode step over a paged KV cache with grouped query heads.

    q [B,H,d] bf16; k_cache/v_cache [num_blocks,H_kv,block_size,d] bf16; block_table
    [B,max_blocks] int32; seq_lens [B] int32 -> (o [B,H,d] bf16, lse [B,H] fp32)."""
    import torch
    B, H, d = q.shape
    num_blocks, H_kv, block_size = k_cache.shape[:3]
    max_blocks = block_table.shape[1]
    _need(q, "q", (B, H, d), torch.bfloat16)
    _need(k_cache, "k_cache", (num_blocks, H_kv, block_size, d), torch.bfloat16)
    _need(v_cache, "v_cache", (num_blocks, H_kv, block_size, d), torch.bfloat16)
    _need(block_table, "block_table", (B, max_blocks), torch.int32)
    _need(seq_lens, "seq_lens", (B,), torch.int32)
    nbytes = decode_paged_workspace_bytes(B, H, H_kv, max_blocks, block_size, d, num_splits)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", (B, H, d), torch.bfloat16)
        _need(lse, "lse", (B, H), torch.float32)
    st = load().fa_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                block_table.data_ptr(), seq_lens.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), B, H, H_kv, d,
                                block_size, num_blocks, max_blocks, _scale(scale, d),
                                int(num_splits), _stream(q))
    _check("fa_decode_paged", st)
    return o, lse


def _lens(t, name: str, B: int) -> None:
    import torch
    _need(t, name, (B,), torch.int32)


def fwd_varlen(q, k, v, seq_lens_q, seq_lens_k, causal: bool = False,
               scale: float | None = None, out=None):
    """Forward over a batch of different-length sequences in the padded [B,H,N,d] layout
    (seq_lens_q/seq_lens_k: int32 [B] on the GPU) -> (o, lse); padding rows get o = 0,
    lse = -inf."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, d), torch.bfloat16)
    _lens(seq_lens_q, "seq_lens_q", B)
    _lens(seq_lens_k, "seq_lens_k", B)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", (B, H, Nq, d), torch.bfloat16)
        _need(lse, "lse", (B, H, Nq), torch.float32)
    st = load().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), seq_lens_q.data_ptr(), seq_lens_k.data_ptr(), B, H,
                              Nq, Nk, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_fwd_varlen", st)
    return o, lse


def bwd_varlen(q, k, v, o, lse, dout, seq_lens_q, seq_lens_k, causal: bool = False,
               scale: float | None = None, workspace=None, out=None):
    """Gradients (dq, dk, dv) for fwd_varlen; padding rows and keys get zero gradients."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, H, Nk, d)), (v, "v", (B, H, Nk, d)),
                      (o, "o", (B, H, Nq, d)), (dout, "dout", (B, H, Nq, d))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    _lens(seq_lens_q, "seq_lens_q", B)
    _lens(seq_lens_k, "seq_lens_k", B)
    nbytes = bwd_workspace_bytes(B, H, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _outs(out, [("dq", tuple(q.shape), torch.bfloat16),
                                 ("dk", tuple(k.shape), torch.bfloat16),
                                 ("dv", tuple(v.shape), torch.bfloat16)])
    st = load().fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), seq_lens_q.data_ptr(), seq_lens_k.data_ptr(),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              B, H, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_bwd_varlen", st)
    return dq, dk, dv


def fwd_dropout(q, k, v, p_drop: float, seed: int, offset: int = 0, causal: bool = False,
                scale: float | None = None, out=None):
    """Forward with dropout on P (mask regenerated from (seed, offset), never stored):
    o = (P * Z / (1 - p_drop)) V; lse as for fwd."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, d), torch.bfloat16)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", (B, H, Nq, d), torch.bfloat16)
        _need(lse, "lse", (B, H, Nq), torch.float32)
    st = load().fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), B, H, Nq, Nk, d, _scale(scale, d),
                               int(bool(causal)), float(p_drop), int(seed) & (2**64 - 1),
                               int(offset) & (2**32 - 1), _stream(q))
    _check("fa_fwd_dropout", st)
    return o, lse


def bwd_dropout(q, k, v, o, lse, dout, p_drop: float, seed: int, offset: int = 0,
                causal: bool = False, scale: float | None = None, workspace=None, out=None):
    """Gradients (dq, dk, dv) of fwd_dropout with the same (p_drop, seed, offset)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, H, Nk, d)), (v, "v", (B, H, Nk, d)),
                      (o, "o", (B, H, Nq, d)), (dout, "dout", (B, H, Nq, d))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    nbytes = bwd_workspace_bytes(B, H, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _outs(out, [("dq", tuple(q.shape), torch.bfloat16),
                                 ("dk", tuple(k.shape), torch.bfloat16),
                                 ("dv", tuple(v.shape), torch.bfloat16)])
    st = load().fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), B, H, Nq, Nk, d,
                               _scale(scale, d), int(bool(causal)), float(p_drop),
                               int(seed) & (2**64 - 1), int(offset) & (2**32 - 1), _stream(q))
    _check("fa_bwd_dropout", st)
    return dq, dk, dv


def fwd_fp8_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_fwd_fp8_workspace_bytes(B, H, Nq, Nk, d))


def fwd_fp8(q, k, v, causal: bool = False, incoherent: bool = True, seed: int = 0,
            scale: float | None = None, workspace=None, out=None):
    """FP8 forward with incoherent processing: bf16 q, k, v -> (o bf16, lse fp32, workspace).
    The workspace (uint8, device) holds the FP8 codes and scales afterwards (layout in fa.h)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, d), torch.bfloat16)
    nbytes = fwd_fp8_workspace_bytes(B, H, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", (B, H, Nq, d), torch.bfloat16)
        _need(lse, "lse", (B, H, Nq), torch.float32)
    st = load().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           lse.data_ptr(), B, H, Nq, Nk, d, _scale(scale, d), int(bool(causal)),
                           int(bool(incoherent)), int(seed) & (2**64 - 1), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), _stream(q))
    _check("fa_fwd_fp8", st)
    return o, lse, workspace


def fp8_workspace_views(workspace, B: int, H: int, Nq: int, Nk: int, d: int) -> dict:
    """Views of the FP8 codes and scales inside a workspace written by fwd_fp8 (layout of fa.h):
    q8 [B,H,Nq,d], k8 [B,H,Nk,d], v8t [B,H,d,Nkp] uint8; sq, sk, vpart, sv fp32."""
    import torch
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    nq32, nk64 = (Nq + 31) // 32, (Nk + 63) // 64
    sizes = [("q8", B * H * Nq * d, (B, H, Nq, d), torch.uint8),
             ("k8", B * H * Nk * d, (B, H, Nk, d), torch.uint8),
             ("v8t", B * H * d * nk64 * 64, (B, H, d, nk64 * 64), torch.uint8),
             ("sq", B * H * nq32 * 4, (B, H, nq32), torch.float32),
             ("sk", B * H * nk64 * 4, (B, H, nk64), torch.float32),
             ("vpart", B * H * nk64 * 4, (B, H, nk64), torch.float32),
             ("sv", B * H * 4, (B, H), torch.float32)]
    out, off = {}, 0
    for name, nbytes, shape, dt in sizes:
        out[name] = workspace[off:off + nbytes].view(dt).view(shape)
        off += al(nbytes)
    return out


def _bias_strides(bias, B: int, H: int, Nq: int, Nk: int):
    """Element strides (b, h, q) of a bf16 bias broadcastable to [B, H, Nq, Nk] whose last
    dimension is contiguous; size-1 (or missing) leading dimensions broadcast (stride 0)."""
    import torch
    if bias.dtype != torch.bfloat16:
        raise FaError(f"bias: dtype {bias.dtype}, expected torch.bfloat16")
    while bias.dim() < 4:
        bias = bias.unsqueeze(0)
    shape = tuple(bias.shape)
    want = (B, H, Nq, Nk)
    for i, (s_, w) in enumerate(zip(shape, want)):
        if s_ not in (1, w) or (i == 3 and s_ != w):
            raise FaError(f"bias: shape {shape} does not broadcast to {want}")
    st = [0 if shape[i] == 1 else bias.stride(i) for i in range(3)]
    if bias.stride(3) != 1 or any(x % 8 for x in st) or bias.data_ptr() % 16:
        # the library reads 16-byte rows: re-lay the bias out with rows padded to 8 elements
        # (a copy; callers who keep their bias in this layout pass it through unchanged)
        nk8 = (Nk + 7) // 8 * 8
        padded = torch.zeros(shape[:3] + (nk8,), dtype=bias.dtype, device=bias.device)
        padded[..., :Nk] = bias
        bias = padded[..., :Nk]
        st = [0 if shape[i] == 1 else bias.stride(i) for i in range(3)]
    return bias, st


def fwd_bias(q, k, v, bias, causal: bool = False, scale: float | None = None, out=None):
    """Forward with an additive bf16 bias on the scores (broadcastable to [B,H,Nq,Nk], -inf
    entries mask) -> (o, lse)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, d), torch.bfloat16)
    bias, (sb, sh, sq) = _bias_strides(bias, B, H, Nq, Nk)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = _outs(out, [("o", (B, H, Nq, d), torch.bfloat16),
                             ("lse", (B, H, Nq), torch.float32)])
    st = load().fa_fwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            bias.data_ptr(), sb, sh, sq, B, H, Nq, Nk, d, _scale(scale, d),
                            int(bool(causal)), _stream(q))
    _check("fa_fwd_bias", st)
    return o, lse


def bwd_bias(q, k, v, o, lse, dout, bias, causal: bool = False, scale: float | None = None,
             workspace=None, out=None):
    """Gradients (dq, dk, dv) of fwd_bias (the bias is a constant)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, H, Nk, d)), (v, "v", (B, H, Nk, d)),
                      (o, "o", (B, H, Nq, d)), (dout, "dout", (B, H, Nq, d))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    bias, (sb, sh, sq) = _bias_strides(bias, B, H, Nq, Nk)
    nbytes = bwd_workspace_bytes(B, H, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _outs(out, [("dq", tuple(q.shape), torch.bfloat16),
                                 ("dk", tuple(k.shape), torch.bfloat16),
                                 ("dv", tuple(v.shape), torch.bfloat16)])
    st = load().fa_bwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), bias.data_ptr(), sb, sh, sq, workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), B, H, Nq, Nk, d,
                            _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_bwd_bias", st)
    return dq, dk, dv


def fwd_dv(q, k, v, causal: bool = False, scale: float | None = None, out=None):
    """Forward with V of its own head dimension: q, k [.., d], v [B,H,Nk,d_v] -> o [.., d_v]."""
    import torch
    B, H, Nq, d = q.shape
    Nk, dv_ = k.shape[2], v.shape[3]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, H, Nk, d), torch.bfloat16)
    _need(v, "v", (B, H, Nk, dv_), torch.bfloat16)
    if out is None:
        o = torch.empty((B, H, Nq, dv_), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = _outs(out, [("o", (B, H, Nq, dv_), torch.bfloat16),
                             ("lse", (B, H, Nq), torch.float32)])
    st = load().fa_fwd_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, Nq, Nk, d, dv_, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_fwd_dv", st)
    return o, lse


def bwd_dv(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
           workspace=None, out=None):
    """Gradients (dq, dk, dv) of fwd_dv."""
    import torch
    B, H, Nq, d = q.shape
    Nk, dv_ = k.shape[2], v.shape[3]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, H, Nk, d)),
                      (v, "v", (B, H, Nk, dv_)), (o, "o", (B, H, Nq, dv_)),
                      (dout, "dout", (B, H, Nq, dv_))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    nbytes = bwd_workspace_bytes(B, H, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _outs(out, [("dq", tuple(q.shape), torch.bfloat16),
                                 ("dk", tuple(k.shape), torch.bfloat16),
                                 ("dv", tuple(v.shape), torch.bfloat16)])
    st = load().fa_bwd_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          B, H, Nq, Nk, d, dv_, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_bwd_dv", st)
    return dq, dk, dv


def fwd_gqa(q, k, v, causal: bool = False, scale: float | None = None, out=None):
    """Forward with grouped query heads: q [B,H,Nq,d], k/v [B,H_kv,Nk,d] (H a multiple of H_kv;
    query head h reads K/V head h // (H // H_kv)) -> (o [B,H,Nq,d] bf16, lse [B,H,Nq] fp32)."""
    import torch
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, Hkv, Nk, d), torch.bfloat16)
    _need(v, "v", (B, Hkv, Nk, d), torch.bfloat16)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", (B, H, Nq, d), torch.bfloat16)
        _need(lse, "lse", (B, H, Nq), torch.float32)
    st = load().fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           B, H, Hkv, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_fwd_gqa", st)
    return o, lse


def bwd_gqa_workspace_bytes(B: int, H: int, H_kv: int, Nq: int, Nk: int, d: int) -> int:
    """Workspace bytes of bwd_gqa (more than bwd's when the dK/dV pass keeps partial rows)."""
    return int(load().fa_bwd_gqa_workspace_bytes(B, H, H_kv, Nq, Nk, d))


def bwd_gqa(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
            workspace=None, out=None):
    """Gradients (dq, dk, dv) of fwd_gqa; dk, dv [B,H_kv,Nk,d] sum over each group's query
    heads."""
    import torch
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, Hkv, Nk, d)),
                      (v, "v", (B, Hkv, Nk, d)), (o, "o", (B, H, Nq, d)),
                      (dout, "dout", (B, H, Nq, d))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    nbytes = bwd_gqa_workspace_bytes(B, H, Hkv, Nq, Nk, d)
    workspace = _workspace(workspace, nbytes, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _outs(out, [("dq", tuple(q.shape), torch.bfloat16),
                                 ("dk", tuple(k.shape), torch.bfloat16),
                                 ("dv", tuple(v.shape), torch.bfloat16)])
    st = load().fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           B, H, Hkv, Nq, Nk, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _check("fa_bwd_gqa", st)
    return dq, dk, dv


def fwd_ext(q, k, v, seq_lens_q=None, seq_lens_k=None, p_drop: float = 0.0, seed: int = 0,
            offset: int = 0, causal: bool = False, scale: float | None = None, out=None):
    """Forward with any subset of per-sequence lengths (int32 [B] on the GPU, both or neither),
    grouped K/V heads (k/v [B,H_kv,Nk,d]) and dropout on P (p_drop > 0) -> (o, lse)."""
    import torch
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _need(q, "q", (B, H, Nq, d), torch.bfloat16)
    _need(k, "k", (B, Hkv, Nk, d), torch.bfloat16)
    _need(v, "v", (B, Hkv, Nk, d), torch.bfloat16)
    if (seq_lens_q is None) != (seq_lens_k is None):
        raise ValueError("give both seq_lens_q and seq_lens_k, or neither")
    if seq_lens_q is not None:
        _lens(seq_lens_q, "seq_lens_q", B)
        _lens(seq_lens_k, "seq_lens_k", B)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = _outs(out, [("o", (B, H, Nq, d), torch.bfloat16),
                             ("lse", (B, H, Nq), torch.float32)])
    lq = seq_lens_q.data_ptr() if seq_lens_q is not None else None
    lk = seq_lens_k.data_ptr() if seq_lens_k is not None else None
    st = load().fa_fwd_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           lq, lk, B, H, Hkv, Nq, Nk, d, _scale(scale, d), int(bool(causal)),
                           float(p_drop), int(seed) & (2**64 - 1), int(offset) & (2**32 - 1),
                           _stream(q))
    _check("fa_fwd_ext", st)
    return o, lse


def bwd_ext_workspace_bytes(B: int, H: int, H_kv: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_bwd_ext_workspace_bytes(B, H, H_kv, Nq, Nk, d))


def bwd_ext(q, k, v, o, lse, dout, seq_lens_q=None, seq_lens_k=None, p_drop: float = 0.0,
            seed: int = 0, offset: int = 0, causal: bool = False, scale: float | None = None,
            workspace=None, out=None):
    """Gradients (dq, dk, dv) of fwd_ext with the same options; dk, dv [B,H_kv,Nk,d] sum over
    each group's query heads; padding rows and keys get zero gradients."""
    import torch
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    for t, n, shp in ((q, "q", (B, H, Nq, d)), (k, "k", (B, Hkv, Nk, d)),
                      (v, "v", (B, Hkv, Nk, d)), (o, "o", (B, H, Nq, d)),
                      (dout, "dout", (B, H, Nq, d))):
        _need(t, n, shp, torch.bfloat16)
    _need(lse, "lse", (B, H, Nq), torch.float32)
    if (seq_lens_q is None) != (seq_lens_k is None):
        raise ValueError("give both seq_lens_q and seq_lens_k, or neither")
    if seq_lens_q is not None:
        _lens(seq_lens_q, "seq_lens_q", B)
        _lens(seq_lens_k, "seq_lens_k", B)
    workspace = _workspace(workspace, bwd_ext_workspace_bytes(B, H, Hkv, Nq, Nk, d), q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _outs(out, [("dq", tuple(q.shape), torch.bfloat16),
                                 ("dk", tuple(k.shape), torch.bfloat16),
                                 ("dv", tuple(v.shape), torch.bfloat16)])
    lq = seq_lens_q.data_ptr() if seq_lens_q is not None else None
    lk = seq_lens_k.data_ptr() if seq_lens_k is not None else None
    st = load().fa_bwd_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), lq, lk,
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           B, H, Hkv, Nq, Nk, d, _scale(scale, d), int(bool(causal)),
                           float(p_drop), int(seed) & (2**64 - 1), int(offset) & (2**32 - 1),
                           _stream(q))
    _check("fa_bwd_ext", st)
    return dq, dk, dv
