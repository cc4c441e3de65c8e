"""Python binding of libfa.so, the gfx950 exact-attention library (C ABI in include/fa.h).

Argument marshalling only: every step of the attention path runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no fallback: if the library is
missing or a call is unsupported, these functions raise.

    fa_forward(q, k, v, o, lse, scale, causal, seqlens)            # C-ABI names, caller-owned outputs
    fa_backward(q, k, v, o, do, lse, dq, dk, dv, scale, causal, seqlens, workspace)
    fa_backward_workspace_size(B, H, N, d, dtype)
    fa_forward_block_sparse(q, k, v, o, lse, scale, causal, seqlens, block_mask)
    fa_forward_dropout(q, k, v, o, lse, scale, causal, seqlens, p, seed, offset)
    fa_backward_dropout(q, k, v, o, do, lse, dq, dk, dv, scale, causal, seqlens, p, seed, offset, workspace)
    fa_dropout_mask(B, H, N, p, seed, offset, keep)
    fa_forward_kv_outer(q, k, v, o, lse, scale, lds_bytes, workspace)    # the pages' schedule (IO measurement)
    fa_forward_kv_outer_workspace_size(B, H, N, d)
    fa_forward_fp8(q8, k8, v8, descale_q, descale_k, descale_v, o, lse, scale, causal, seqlens)
    fa_backward_block_sparse(q, k, v, o, do, lse, dq, dk, dv, scale, causal, seqlens, block_mask, workspace)
    fa_backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale, causal, seqlens)   # library-held workspace
    forward(q, k, v, ...) -> (o, lse)                               # allocating conveniences
    backward(q, k, v, o, do, lse, ...) -> (dq, dk, dv)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK = 0
FA_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "FA_OK", 1: "FA_ERR_INVALID_ARGUMENT", 2: "FA_ERR_UNSUPPORTED", 3: "FA_ERR_MISALIGNED",
          4: "FA_ERR_WORKSPACE", 5: "FA_ERR_HIP"}
EXPORTS = ("fa_forward", "fa_backward", "fa_backward_workspace_size", "fa_backward_prepare", "fa_backward_dkdv",
           "fa_backward_dq", "fa_backward_dq_prepare", "fa_forward_block_sparse", "fa_backward_block_sparse", "fa_forward_dropout",
           "fa_backward_dropout", "fa_dropout_mask", "fa_forward_kv_outer", "fa_forward_kv_outer_workspace_size",
           "fa_forward_fp8", "fa_backward_noalloc", "fa_status_string", "fa_last_error")
NOALLOC_WORKSPACE_BYTES = 8 * 1024 * 1024  # FA_NOALLOC_WORKSPACE_BYTES
MASK_BLOCK = 128  # FA_MASK_BLOCK: rows and columns of one block of the block-sparse mask

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libfa.so once and declare the C signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run exact_io_aware_66_amd/build.py (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
    lib.fa_forward.restype = i
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_prepare.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
    lib.fa_backward_prepare.restype = i
    lib.fa_backward_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
    lib.fa_backward_dkdv.restype = i
    lib.fa_backward_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
    lib.fa_backward_dq.restype = i
    lib.fa_backward_dq_prepare.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
    lib.fa_backward_dq_prepare.restype = i
    lib.fa_forward_block_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, i, vp]
    lib.fa_forward_block_sparse.restype = i
    lib.fa_backward_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, i, vp, sz, vp]
    lib.fa_backward_block_sparse.restype = i
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    lib.fa_forward_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, u64, u32, i, vp]
    lib.fa_forward_dropout.restype = i
    lib.fa_backward_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, u64, u32, i, vp, sz,
                                        vp]
    lib.fa_backward_dropout.restype = i
    lib.fa_dropout_mask.argtypes = [i, i, i, f, u64, u32, vp, vp]
    lib.fa_dropout_mask.restype = i
    lib.fa_forward_kv_outer.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, sz, i, vp, sz, vp]
    lib.fa_forward_kv_outer.restype = i
    lib.fa_forward_kv_outer_workspace_size.argtypes = [i, i, i, i]
    lib.fa_forward_kv_outer_workspace_size.restype = sz
    lib.fa_forward_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, f, i, vp, vp]
    lib.fa_forward_fp8.restype = i
    lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
    lib.fa_backward_noalloc.restype = i
    lib.fa_backward_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_backward_workspace_size.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != FA_OK:
        lib = load()
        raise FAError(status, (lib.fa_last_error() or b"").decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dims(q):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    return tuple(int(x) for x in q.shape)


def _dtype_code(t):
    if t.dtype not in FA_DTYPE:
        raise FAError(2, f"dtype {t.dtype} is not supported (float32 or bfloat16 only)")
    return FA_DTYPE[t.dtype]


def _same(ref, *ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if t.device != ref.device:
            raise ValueError("tensors must be on one device")


# The C ABI takes raw pointers and cannot see sizes, so these checks are the only place where a
# tensor of the wrong shape or element type is caught before a kernel reads or writes past it.
def _like(ref, **named):
    """Every named tensor has ref's shape and element type (the [B, H, N, d] operands)."""
    for name, t in named.items():
        if t is None:
            raise ValueError(f"{name} is required")
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
        if t.dtype != ref.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {ref.dtype}")


def _lse(lse, B, H, N):
    """The row statistic: float32 [B, H, N]."""
    if lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        got = None if lse is None else (lse.dtype, tuple(lse.shape))
        raise ValueError(f"lse must be float32 of shape {(B, H, N)} (got {got})")


def _workspace(ws):
    """Workspace bytes: a uint8 tensor (the library checks the size itself)."""
    if ws is None:
        return 0
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError(f"workspace must be a 1-D uint8 tensor (got {ws.dtype}, {ws.dim()}-D)")
    return ws.numel()


def _seqlens(seqlens, B, device):
    if seqlens is None:
        return None
    if not (seqlens.is_cuda and seqlens.dtype == torch.int32 and seqlens.numel() == B and seqlens.is_contiguous()):
        raise ValueError("seqlens must be a contiguous int32 device tensor with B entries")
    if seqlens.device != device:
        raise ValueError("seqlens must be on the tensors' device")
    return seqlens


def _block_mask(block_mask, B, H, N, device):
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    if not (block_mask.is_cuda and block_mask.dtype == torch.uint8 and block_mask.is_contiguous()
            and tuple(block_mask.shape) == (B, H, nb, nb)):
        raise ValueError(f"block_mask must be a contiguous uint8 device tensor of shape [B, H, {nb}, {nb}]")
    if block_mask.device != device:
        raise ValueError("block_mask must be on the tensors' device")
    return block_mask


def fa_backward_workspace_size(B: int, H: int, N: int, d: int, dtype) -> int:
    code = FA_DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(load().fa_backward_workspace_size(B, H, N, d, code))


def fa_forward(q, k, v, o, lse, scale: float, causal: bool = False, seqlens=None, stream=None) -> None:
    """C-ABI fa_forward on caller-owned tensors (o: like q; lse: float32 [B, H, N])."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, lse)
    _like(q, k=k, v=v, o=o)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    _check(lib.fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
                          _ptr(seqlens), _dtype_code(q), _stream(stream)))


def fa_backward(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False, seqlens=None, workspace=None,
                stream=None) -> None:
    """C-ABI fa_backward on caller-owned tensors; `workspace` is a uint8 device tensor."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, do, lse, dq, dk, dv, workspace)
    _like(q, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    nbytes = _workspace(workspace)
    _check(lib.fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                           B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens), _dtype_code(q),
                           _ptr(workspace), nbytes, _stream(stream)))


def fa_backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False, seqlens=None,
                        stream=None) -> None:
    """C-ABI fa_backward_noalloc: fa_backward with the library's own static workspace (nothing allocated;
    calls that overlap in time on one GPU race)."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, do, lse, dq, dk, dv)
    _like(q, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    _check(lib.fa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                   _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens),
                                   _dtype_code(q), _stream(stream)))


def fa_forward_block_sparse(q, k, v, o, lse, scale: float, causal: bool, seqlens, block_mask, stream=None) -> None:
    """C-ABI fa_forward_block_sparse: block_mask is uint8 [B, H, ceil(N/128), ceil(N/128)] on the device."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, lse)
    _like(q, k=k, v=v, o=o)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    block_mask = _block_mask(block_mask, B, H, N, q.device)
    _check(lib.fa_forward_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                       int(bool(causal)), _ptr(seqlens), _ptr(block_mask), _dtype_code(q),
                                       _stream(stream)))


def fa_backward_block_sparse(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, seqlens, block_mask,
                             workspace, stream=None) -> None:
    """C-ABI fa_backward_block_sparse (same block mask as the forward)."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, do, lse, dq, dk, dv, workspace)
    _like(q, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    block_mask = _block_mask(block_mask, B, H, N, q.device)
    nbytes = _workspace(workspace)
    _check(lib.fa_backward_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                        _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens),
                                        _ptr(block_mask), _dtype_code(q), _ptr(workspace), nbytes, _stream(stream)))


def fa_forward_dropout(q, k, v, o, lse, scale: float, causal: bool, seqlens, p: float, seed: int, offset: int,
                       stream=None) -> None:
    """C-ABI fa_forward_dropout: dropout probability p, Philox seed (64-bit) and offset (32-bit)."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, lse)
    _like(q, k=k, v=v, o=o)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    _check(lib.fa_forward_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                  int(bool(causal)), _ptr(seqlens), float(p), int(seed), int(offset), _dtype_code(q),
                                  _stream(stream)))


def fa_backward_dropout(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, seqlens, p: float, seed: int,
                        offset: int, workspace, stream=None) -> None:
    """C-ABI fa_backward_dropout (same p, seed and offset as the forward)."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, do, lse, dq, dk, dv, workspace)
    _like(q, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    nbytes = _workspace(workspace)
    _check(lib.fa_backward_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                   B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens), float(p), int(seed),
                                   int(offset), _dtype_code(q), _ptr(workspace), nbytes, _stream(stream)))


def fa_dropout_mask(B: int, H: int, N: int, p: float, seed: int, offset: int, keep, stream=None) -> None:
    """C-ABI fa_dropout_mask into `keep`, a contiguous uint8 device tensor [B, H, N, N] (1 = kept)."""
    lib = load()
    if not (keep.is_cuda and keep.dtype == torch.uint8 and keep.is_contiguous() and tuple(keep.shape) == (B, H, N, N)):
        raise ValueError("keep must be a contiguous uint8 device tensor [B, H, N, N]")
    _check(lib.fa_dropout_mask(B, H, N, float(p), int(seed), int(offset), _ptr(keep), _stream(stream)))


def fa_forward_kv_outer_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_forward_kv_outer_workspace_size(B, H, N, d))


def fa_forward_kv_outer(q, k, v, o, lse, scale: float, lds_bytes: int, workspace, stream=None) -> None:
    """C-ABI fa_forward_kv_outer: the pages' K/V-outer schedule with an LDS budget of lds_bytes (bf16)."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, lse, workspace)
    _like(q, k=k, v=v, o=o)
    _lse(lse, B, H, N)
    nbytes = _workspace(workspace)
    _check(lib.fa_forward_kv_outer(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                   int(lds_bytes), _dtype_code(q), _ptr(workspace), nbytes, _stream(stream)))


def fa_forward_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, o, lse, scale: float,
                   causal: bool = False, seqlens=None, stream=None) -> None:
    """C-ABI fa_forward_fp8: q8, k8, v8 torch.float8_e4m3fn [B, H, N, 128]; o bfloat16; lse float32."""
    lib = load()
    B, H, N, d = _dims(q8)
    _same(q8, k8, v8, o, lse)
    for t in (q8, k8, v8):
        if t.dtype != torch.float8_e4m3fn:
            raise FAError(2, f"FP8 inputs must be torch.float8_e4m3fn (got {t.dtype})")
    _like(q8, k8=k8, v8=v8)
    if o.dtype != torch.bfloat16 or tuple(o.shape) != tuple(q8.shape):
        raise ValueError(f"o must be bfloat16 of shape {tuple(q8.shape)}")
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q8.device)
    _check(lib.fa_forward_fp8(_ptr(q8), _ptr(k8), _ptr(v8), float(descale_q), float(descale_k), float(descale_v),
                              _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens),
                              _stream(stream)))


def fa_backward_prepare(o, do, lse, workspace, stream=None) -> None:
    """Stage 1 of fa_backward: D = rowsum(dO * O) into the workspace (bf16: also LSE log2 e)."""
    lib = load()
    B, H, N, d = _dims(o)
    _same(o, do, lse, workspace)
    _like(o, do=do)
    _lse(lse, B, H, N)
    nbytes = _workspace(workspace)
    _check(lib.fa_backward_prepare(_ptr(o), _ptr(do), _ptr(lse), B, H, N, d, _dtype_code(o), _ptr(workspace),
                                   nbytes, _stream(stream)))


def fa_backward_dkdv(q, k, v, do, lse, dk, dv, scale: float, causal: bool = False, seqlens=None,
                     workspace=None, stream=None) -> None:
    """Stage 2 of fa_backward: the recompute pass over query blocks per key block (dK, dV)."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, do, lse, dk, dv, workspace)
    _like(q, k=k, v=v, do=do, dk=dk, dv=dv)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    nbytes = _workspace(workspace)
    _check(lib.fa_backward_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dk), _ptr(dv),
                                B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens), _dtype_code(q),
                                _ptr(workspace), nbytes, _stream(stream)))


def fa_backward_dq_prepare(q, k, v, o, do, lse, dq, scale: float, causal: bool = False, seqlens=None,
                           workspace=None, stream=None) -> None:
    """fa_backward_prepare and fa_backward_dq in one call: writes dq and the workspace's row statistics."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, o, do, lse, dq, workspace)
    _like(q, k=k, v=v, o=o, do=do, dq=dq)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    nbytes = _workspace(workspace)
    _check(lib.fa_backward_dq_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                      B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens), _dtype_code(q),
                                      _ptr(workspace), nbytes, _stream(stream)))


def fa_backward_dq(q, k, v, do, lse, dq, scale: float, causal: bool = False, seqlens=None, workspace=None,
                   stream=None) -> None:
    """Stage 3 of fa_backward: the recompute pass over key blocks per query block (dQ)."""
    lib = load()
    B, H, N, d = _dims(q)
    _same(q, k, v, do, lse, dq, workspace)
    _like(q, k=k, v=v, do=do, dq=dq)
    _lse(lse, B, H, N)
    seqlens = _seqlens(seqlens, B, q.device)
    nbytes = _workspace(workspace)
    _check(lib.fa_backward_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dq),
                              B, H, N, d, float(scale), int(bool(causal)), _ptr(seqlens), _dtype_code(q),
                              _ptr(workspace), nbytes, _stream(stream)))


def _default_scale(d: int) -> float:
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def forward(q, k, v, scale: float | None = None, causal: bool = False, seqlens=None, stream=None, block_mask=None,
            dropout=None):
    """Allocate O and LSE and run fa_forward (fa_forward_block_sparse with a block mask, fa_forward_dropout
    with dropout=(p, seed, offset)); returns (o, lse)."""
    B, H, N, d = _dims(q)
    scale = _default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if dropout is not None:
        fa_forward_dropout(q, k, v, o, lse, scale, causal, seqlens, *dropout, stream=stream)
    elif block_mask is None:
        fa_forward(q, k, v, o, lse, scale, causal, seqlens, stream)
    else:
        fa_forward_block_sparse(q, k, v, o, lse, scale, causal, seqlens, block_mask, stream)
    return o, lse


def backward(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False, seqlens=None, stream=None,
             workspace=None, block_mask=None, dropout=None):
    """Allocate dQ, dK, dV (and the workspace unless given) and run fa_backward (fa_backward_block_sparse
    with a block mask); returns (dq, dk, dv)."""
    B, H, N, d = _dims(q)
    scale = _default_scale(d) if scale is None else scale
    if workspace is None:
        workspace = torch.empty(fa_backward_workspace_size(B, H, N, d, q.dtype), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if dropout is not None:
        fa_backward_dropout(q, k, v, o, do, lse, dq, dk, dv, scale, causal, seqlens, *dropout, workspace, stream=stream)
    elif block_mask is None:
        fa_backward(q, k, v, o, do, lse, dq, dk, dv, scale, causal, seqlens, workspace, stream)
    else:
        fa_backward_block_sparse(q, k, v, o, do, lse, dq, dk, dv, scale, causal, seqlens, block_mask, workspace,
                                 stream)
    return dq, dk, dv
