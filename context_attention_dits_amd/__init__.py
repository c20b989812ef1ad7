"""One rank's share of context-parallel attention on an MI355X, from Python.

Thin binding over the C-ABI in include/cp_attn.h. Functions carry the C
names and only marshal arguments: torch tensors supply device pointers,
shapes and strides, ``torch.cuda.current_stream()`` supplies the stream, and
every step runs in the library's HIP kernels. Tensors must live on the GPU;
the binding refuses host tensors rather than hand their addresses to a kernel.

Layouts: Q/K/V/out ``[B, S, H, D]`` with the last axis contiguous, LSE
``[B, H, Sq]`` float32 contiguous. Q/K/V are bfloat16 or float32; out and LSE
are float32.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

from . import _lib
from ._lib import (CP_BF16, CP_BLOCK_ACCUMULATE, CP_ERR_HIP, CP_ERR_INVALID_ARG,  # noqa: F401
                   CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_F32, CP_OK, CP_REGROUP_HEAD_TO_SEQ,
                   CP_REGROUP_SEQ_TO_HEAD, CP_RING_ANYTHING, CP_RING_SEPARATE_MERGE, STATUS_NAMES)

__all__ = [
    "CpAttnError", "load", "cp_abi_version", "cp_last_error", "cp_attn_set_fwd_waves", "cp_attn_block_fwd",
    "cp_lse_merge",
    "cp_ring_attention", "cp_ring_attention_workspace_size", "cp_ulysses_regroup",
]


class CpAttnError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def load():
    return _lib.load()


def _torch():
    import torch
    return torch


def _stream(stream) -> ctypes.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, func: str):
    if status != _lib.CP_OK:
        raise CpAttnError(status, func, _lib.load().cp_last_error().decode())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float32:
        return CP_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _gpu(name: str, t, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _bshd(name: str, t):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, S, H, D] (got shape {tuple(t.shape)})")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the D axis must be unit-stride")
    return t


def _strides(t):
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _f32(name, t):
    torch = _torch()
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")


def _lse_shape(name, t, B, H, Sq):
    _f32(name, t)
    if tuple(t.shape) != (B, H, Sq) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 [B, H, Sq] = {(B, H, Sq)} tensor")


def cp_abi_version() -> int:
    return _lib.load().cp_abi_version()


def cp_last_error() -> str:
    return _lib.load().cp_last_error().decode()


def cp_attn_set_fwd_waves(waves: int) -> int:
    """Workgroup shape of the bfloat16 block kernel (0 auto, 4 or 8); returns the previous one."""
    prev = _lib.load().cp_attn_set_fwd_waves(int(waves))
    if prev < 0:
        raise ValueError(f"cp_attn_set_fwd_waves: waves must be 0, 4 or 8, got {waves}")
    return prev


def cp_attn_block_fwd(q, k, v, out, lse, scale: Optional[float] = None, flags: int = 0, stream=None):
    """Partial attention of q against one K/V block into (out, lse); see cp_attn_block_fwd in the header."""
    lib = _lib.load()
    dev = _gpu("q", _bshd("q", q)).device
    _gpu("k", _bshd("k", k), dev); _gpu("v", _bshd("v", v), dev)
    _gpu("out", _bshd("out", out), dev); _gpu("lse", lse, dev)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if tuple(k.shape) != (B, Skv, H, D) or tuple(v.shape) != (B, Skv, H, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if tuple(out.shape) != (B, Sq, H, D):
        raise ValueError("out must be [B, Sq, H, D]")
    _f32("out", out)
    _lse_shape("lse", lse, B, H, Sq)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.cp_attn_block_fwd(q.data_ptr(), _strides(q), k.data_ptr(), v.data_ptr(), _strides(k),
                               _dtype_code(q), B, H, D, Sq, Skv, scale, flags, out.data_ptr(),
                               _strides(out), lse.data_ptr(), _stream(stream))
    _check(st, "cp_attn_block_fwd")


def cp_lse_merge(out_acc, lse_acc, out_blk, lse_blk, stream=None):
    """(out_acc, lse_acc) <- merge with (out_blk, lse_blk), in place; see cp_lse_merge."""
    lib = _lib.load()
    dev = _gpu("out_acc", _bshd("out_acc", out_acc)).device
    _gpu("out_blk", _bshd("out_blk", out_blk), dev); _gpu("lse_acc", lse_acc, dev); _gpu("lse_blk", lse_blk, dev)
    B, Sq, H, D = out_acc.shape
    if tuple(out_blk.shape) != (B, Sq, H, D):
        raise ValueError("out_blk shape differs from out_acc")
    _f32("out_acc", out_acc); _f32("out_blk", out_blk)
    _lse_shape("lse_acc", lse_acc, B, H, Sq); _lse_shape("lse_blk", lse_blk, B, H, Sq)
    st = lib.cp_lse_merge(out_acc.data_ptr(), lse_acc.data_ptr(), out_blk.data_ptr(), lse_blk.data_ptr(),
                          _strides(out_acc), _strides(out_blk), B, H, Sq, D, _stream(stream))
    _check(st, "cp_lse_merge")


def cp_ring_attention_workspace_size(B: int, H: int, Sq: int, D: int, flags: int = 0) -> int:
    return int(_lib.load().cp_ring_attention_workspace_size(B, H, Sq, D, flags))


def cp_ring_attention(q, k_blocks: Sequence, v_blocks: Sequence, out, lse, scale: Optional[float] = None,
                      flags: int = 0, workspace=None, stream=None):
    """One rank's ring share over resident K/V blocks into (out, lse); see cp_ring_attention.

    ``k_blocks[i]``/``v_blocks[i]`` are ``[B, L_i, H, D]`` views sharing one stride triple
    (e.g. slices of one buffer, or of a padded ``[P, B, Lmax, H, D]`` gather).
    """
    lib = _lib.load()
    dev = _gpu("q", _bshd("q", q)).device
    _gpu("out", _bshd("out", out), dev); _gpu("lse", lse, dev)
    B, Sq, H, D = q.shape
    P = len(k_blocks)
    if P < 1 or len(v_blocks) != P:
        raise ValueError("need as many v_blocks as k_blocks (>= 1)")
    stride0 = None
    for i, (kb, vb) in enumerate(zip(k_blocks, v_blocks)):
        _gpu(f"k_blocks[{i}]", _bshd("k block", kb), dev); _gpu(f"v_blocks[{i}]", _bshd("v block", vb), dev)
        L = kb.shape[1]
        if tuple(kb.shape) != (B, L, H, D) or tuple(vb.shape) != (B, L, H, D):
            raise ValueError(f"block {i}: shapes {tuple(kb.shape)}/{tuple(vb.shape)} do not match q")
        if kb.dtype != q.dtype or vb.dtype != q.dtype:
            raise TypeError("q and every K/V block must share a dtype")
        s = (kb.stride(0), kb.stride(1), kb.stride(2))
        if stride0 is None:
            stride0 = s
        if s != stride0 or (vb.stride(0), vb.stride(1), vb.stride(2)) != stride0:
            raise ValueError("every K/V block must share one stride triple")
    if tuple(out.shape) != (B, Sq, H, D):
        raise ValueError("out must be [B, Sq, H, D]")
    _f32("out", out)
    _lse_shape("lse", lse, B, H, Sq)
    kptr = (ctypes.c_void_p * P)(*[kb.data_ptr() for kb in k_blocks])
    vptr = (ctypes.c_void_p * P)(*[vb.data_ptr() for vb in v_blocks])
    lens = (ctypes.c_int * P)(*[int(kb.shape[1]) for kb in k_blocks])
    kvs = (ctypes.c_int64 * 3)(*stride0)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _gpu("workspace", workspace, dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.cp_ring_attention(q.data_ptr(), _strides(q), kptr, vptr, kvs, lens, P, _dtype_code(q), B, H,
                               D, Sq, scale, flags, out.data_ptr(), _strides(out), lse.data_ptr(), ws_ptr,
                               ws_bytes, _stream(stream))
    _check(st, "cp_ring_attention")


def cp_ulysses_regroup(inp, out, degree: int, direction: int = CP_REGROUP_SEQ_TO_HEAD, stream=None):
    """Ulysses head/token regroup (loopback all-to-all permutation); see cp_ulysses_regroup.

    SEQ_TO_HEAD: inp [B, S_local, H, D] -> out [B, P*S_local, H/P, D];
    HEAD_TO_SEQ: inp [B, P*S_local, H/P, D] -> out [B, S_local, H, D]. Both contiguous.
    """
    lib = _lib.load()
    dev = _gpu("inp", inp).device
    _gpu("out", out, dev)
    if inp.dtype != out.dtype:
        raise TypeError("inp and out must share a dtype")
    if not (inp.is_contiguous() and out.is_contiguous()) or inp.dim() != 4 or out.dim() != 4:
        raise ValueError("regroup tensors must be contiguous [B, S, H, D]")
    seq = inp if direction == CP_REGROUP_SEQ_TO_HEAD else out
    head = out if direction == CP_REGROUP_SEQ_TO_HEAD else inp
    B, S_l, H, D = seq.shape
    if degree < 1 or H % degree:
        raise ValueError(f"H={H} must be divisible by degree={degree}")
    if tuple(head.shape) != (B, degree * S_l, H // degree, D):
        raise ValueError(f"head-sharded side must be {(B, degree * S_l, H // degree, D)}, got {tuple(head.shape)}")
    st = lib.cp_ulysses_regroup(inp.data_ptr(), out.data_ptr(), inp.element_size(), B, S_l, H, D, degree,
                                direction, _stream(stream))
    _check(st, "cp_ulysses_regroup")


# ------------------------------------------------------- allocating helpers ---

def ring_attention(q, k_blocks, v_blocks, scale: Optional[float] = None, ring_anything: Optional[bool] = None,
                   separate_merge: bool = False, stream=None) -> Tuple:
    """Allocate (out, lse) and run cp_ring_attention; returns (out, lse)."""
    torch = _torch()
    B, Sq, H, D = q.shape
    out = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    lens = [kb.shape[1] for kb in k_blocks]
    if ring_anything is None:
        ring_anything = len(set(lens)) > 1 or 0 in lens
    flags = (CP_RING_ANYTHING if ring_anything else 0) | (CP_RING_SEPARATE_MERGE if separate_merge else 0)
    ws = None
    nbytes = cp_ring_attention_workspace_size(B, H, Sq, D, flags)
    if nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    cp_ring_attention(q, k_blocks, v_blocks, out, lse, scale=scale, flags=flags, workspace=ws, stream=stream)
    return out, lse
