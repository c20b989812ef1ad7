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
from ._lib import (CP_BF16, CP_BLOCK_ACCUMULATE, CP_BLOCK_PACKED_V, CP_BWD_ACCUMULATE_DQ,  # noqa: F401
                   CP_ERR_HIP, CP_ERR_INVALID_ARG, CP_ERR_ORDER, CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_F32,
                   CP_FWD_EIGHT_WAVES, CP_FWD_FOUR_WAVES, CP_OK, CP_ONE_LAUNCH_IN_TURN, CP_ONE_LAUNCH_PARALLEL,
                   CP_REGROUP_HEAD_TO_SEQ, CP_REGROUP_SEQ_TO_HEAD, CP_RING_ANYTHING, CP_RING_PACKED_V,
                   CP_RING_SEPARATE_MERGE, STATUS_NAMES)

__all__ = [
    "CpAttnError", "load", "cp_abi_version", "cp_last_error", "wave_flags", "cp_attn_fwd_waves",
    "cp_ring_attention_one_launch", "cp_ring_attention_check", "cp_attn_block_fwd",
    "cp_lse_merge", "PackedV", "cp_attn_packed_v_bytes", "cp_attn_pack_v", "pack_v", "cp_ulysses_regroup_pack_v",
    "cp_ring_attention", "cp_ring_attention_workspace_size", "cp_ulysses_regroup", "cp_ulysses_regroup_multi",
    "cp_ulysses_pack_heads", "cp_ulysses_concat_seq", "split_counts",
    "cp_attn_bwd_workspace_size", "cp_attn_bwd_prep", "cp_attn_block_bwd", "cp_ring_attention_bwd",
    "ring_attention", "ring_attention_bwd",
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


def wave_flags(waves: int) -> int:
    """CP_FWD_FOUR_WAVES / CP_FWD_EIGHT_WAVES for a forced workgroup shape (4 or 8); 0 chooses per launch."""
    if waves not in (0, 4, 8):
        raise ValueError(f"waves must be 0, 4 or 8, got {waves}")
    return {0: 0, 4: CP_FWD_FOUR_WAVES, 8: CP_FWD_EIGHT_WAVES}[waves]


class PackedV:
    """V of one bfloat16 block as written by cp_attn_pack_v: ``data`` is the packed device buffer,
    ``shape`` the [B, Skv, H, D] shape of the V it holds (the layout is the kernel's own)."""

    def __init__(self, data, shape):
        self.data, self.shape = data, tuple(int(x) for x in shape)
        self.dtype = _torch().bfloat16
        self.device = data.device
        self.is_cuda = data.is_cuda

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def cp_attn_packed_v_bytes(B: int, H: int, D: int, Skv: int) -> int:
    return int(_lib.load().cp_attn_packed_v_bytes(B, H, D, Skv))


def cp_attn_pack_v(v, packed, stream=None) -> PackedV:
    """Write bfloat16 V [B, Skv, H, D] into the device buffer ``packed`` (any dtype, contiguous, at
    least cp_attn_packed_v_bytes bytes); returns it as a PackedV. See cp_attn_pack_v in the header."""
    torch = _torch()
    lib = _lib.load()
    dev = _gpu("v", _bshd("v", v)).device
    _gpu("packed", packed, dev)
    if v.dtype != torch.bfloat16:
        raise TypeError("cp_attn_pack_v: v must be bfloat16")
    if not packed.is_contiguous():
        raise ValueError("cp_attn_pack_v: packed must be contiguous")
    B, Skv, H, D = v.shape
    st = lib.cp_attn_pack_v(v.data_ptr(), _strides(v), B, H, D, Skv, packed.data_ptr(),
                            packed.numel() * packed.element_size(), _stream(stream))
    _check(st, "cp_attn_pack_v")
    return PackedV(packed, (B, Skv, H, D))


def cp_ulysses_regroup_pack_v(inp, packed, degree: int, stream=None) -> PackedV:
    """Regroup bfloat16 V [B, S_local, H, D] (contiguous) for the Ulysses degree and pack it, in one
    pass, into ``packed``; returns the PackedV of the [B, degree*S_local, H/degree, D] tensor that
    cp_ulysses_regroup would have produced. See cp_ulysses_regroup_pack_v in the header."""
    torch = _torch()
    lib = _lib.load()
    dev = _gpu("in", _bshd("in", inp)).device
    _gpu("packed", packed, dev)
    if inp.dtype != torch.bfloat16 or not inp.is_contiguous():
        raise ValueError("cp_ulysses_regroup_pack_v: in must be a contiguous bfloat16 tensor")
    if not packed.is_contiguous():
        raise ValueError("cp_ulysses_regroup_pack_v: packed must be contiguous")
    B, S_l, H, D = inp.shape
    st = lib.cp_ulysses_regroup_pack_v(inp.data_ptr(), B, S_l, H, D, int(degree), packed.data_ptr(),
                                       packed.numel() * packed.element_size(), _stream(stream))
    _check(st, "cp_ulysses_regroup_pack_v")
    return PackedV(packed, (B, int(degree) * S_l, H // int(degree), D))


def _v_operand(name, v, dev):
    """(is_packed, v) for a V argument that is a [B, S, H, D] tensor or a PackedV."""
    if isinstance(v, PackedV):
        _gpu(name, v.data, dev)
        if not v.data.is_contiguous():
            raise ValueError(f"{name}: the packed buffer must be contiguous")
        B, S, H, D = v.shape
        need = cp_attn_packed_v_bytes(B, H, D, S)
        if v.data.numel() * v.data.element_size() < need:
            raise ValueError(f"{name}: packed buffer of {need} bytes needed for V of shape {v.shape}")
        return True, v
    return False, _gpu(name, _bshd(name, v), dev)


def cp_attn_fwd_waves(B: int, H: int, D: int, Sq: int, waves: int = 0) -> int:
    """Workgroup shape (4, or 8 for the ping-pong kernel) of the bfloat16 block kernel at these sizes
    (``waves`` forces one, as the call's flags would); 0 for sizes it does not run. Packed V
    (cp_attn_pack_v) pays off in the 8-wave shape."""
    return int(_lib.load().cp_attn_fwd_waves(B, H, D, Sq, wave_flags(waves)))


def cp_ring_attention_one_launch(dtype: int, B: int, H: int, D: int, Sq: int, block_lens, waves: int = 0) -> int:
    """How cp_ring_attention with packed V and a workspace runs these blocks: 0 one launch per block,
    or one launch: CP_ONE_LAUNCH_IN_TURN or CP_ONE_LAUNCH_PARALLEL."""
    lens = (ctypes.c_int * len(block_lens))(*[int(x) for x in block_lens])
    return int(_lib.load().cp_ring_attention_one_launch(dtype, B, H, D, Sq, lens, len(block_lens),
                                                        wave_flags(waves)))


def cp_ring_attention_check(workspace, stream=None):
    """Raise CpAttnError (CP_ERR_ORDER) if a merge wait of the last parallel-partials ring launch on
    this workspace gave up; waits for the stream."""
    lib = _lib.load()
    _gpu("workspace", workspace)
    st = lib.cp_ring_attention_check(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _check(st, "cp_ring_attention_check")


def cp_attn_block_fwd(q, k, v, out, lse, scale: Optional[float] = None, flags: int = 0, stream=None,
                      waves: int = 0):
    """Partial attention of q against one K/V block into (out, lse); see cp_attn_block_fwd in the header.
    ``v`` may be a PackedV (from cp_attn_pack_v), which sets CP_BLOCK_PACKED_V; ``waves`` (4 or 8)
    forces the workgroup shape (CP_FWD_FOUR_WAVES / CP_FWD_EIGHT_WAVES)."""
    lib = _lib.load()
    flags |= wave_flags(waves)
    dev = _gpu("q", _bshd("q", q)).device
    _gpu("k", _bshd("k", k), dev)
    packed, v = _v_operand("v", v, dev)
    _gpu("out", _bshd("out", out), dev); _gpu("lse", lse, dev)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if tuple(k.shape) != (B, Skv, H, D) or tuple(v.shape) != (B, Skv, H, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if packed:
        flags |= CP_BLOCK_PACKED_V
    elif flags & CP_BLOCK_PACKED_V:
        raise ValueError("CP_BLOCK_PACKED_V needs v from cp_attn_pack_v")
    elif k.stride() != v.stride():
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


def _block_list(q, k_blocks, v_blocks, dev, dtype=None, what="K/V", allow_packed=False):
    """Check a list of [B, L_i, H, D] block pairs against q; returns (P, lens, shared stride triple).
    With allow_packed the V blocks may all be PackedV (their strides are then not compared)."""
    B, _, H, D = q.shape
    P = len(k_blocks)
    if P < 1 or len(v_blocks) != P:
        raise ValueError(f"need as many {what} blocks of each kind (>= 1)")
    n_packed = sum(isinstance(vb, PackedV) for vb in v_blocks)
    if n_packed and (not allow_packed or n_packed != P):
        raise ValueError("V blocks must be all packed (cp_attn_pack_v) or all unpacked"
                         if allow_packed else f"{what}: packed V blocks are not accepted here")
    stride0 = None
    for i, (kb, vb) in enumerate(zip(k_blocks, v_blocks)):
        _gpu(f"{what} block {i}", _bshd(f"{what} block", kb), dev)
        _v_operand(f"{what} block {i}", vb, dev)
        L = kb.shape[1]
        if tuple(kb.shape) != (B, L, H, D) or tuple(vb.shape) != (B, L, H, D):
            raise ValueError(f"{what} block {i}: shapes {tuple(kb.shape)}/{tuple(vb.shape)} do not match q")
        want = q.dtype if dtype is None else dtype
        if kb.dtype != want or vb.dtype != want:
            raise TypeError(f"every {what} block must have dtype {want}")
        s = (kb.stride(0), kb.stride(1), kb.stride(2))
        if stride0 is None:
            stride0 = s
        if s != stride0 or (not n_packed and (vb.stride(0), vb.stride(1), vb.stride(2)) != stride0):
            raise ValueError(f"every {what} block must share one stride triple")
    lens = (ctypes.c_int * P)(*[int(kb.shape[1]) for kb in k_blocks])
    return P, lens, stride0


def _workspace(workspace, dev):
    if workspace is None:
        return None, 0
    _gpu("workspace", workspace, dev)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def cp_ring_attention_workspace_size(B: int, H: int, Sq: int, D: int, flags: int = 0) -> int:
    return int(_lib.load().cp_ring_attention_workspace_size(B, H, Sq, D, flags))


def cp_ring_attention(q, k_blocks: Sequence, v_blocks: Sequence, out, lse, scale: Optional[float] = None,
                      flags: int = 0, workspace=None, stream=None, waves: int = 0):
    """One rank's ring share over resident K/V blocks into (out, lse); see cp_ring_attention.

    ``k_blocks[i]``/``v_blocks[i]`` are ``[B, L_i, H, D]`` views sharing one stride triple
    (e.g. slices of one buffer, or of a padded ``[P, B, Lmax, H, D]`` gather). The V blocks may
    instead all be PackedV (cp_attn_pack_v), which sets CP_RING_PACKED_V. ``waves`` (4 or 8)
    forces the workgroup shape.
    """
    lib = _lib.load()
    flags |= wave_flags(waves)
    dev = _gpu("q", _bshd("q", q)).device
    _gpu("out", _bshd("out", out), dev); _gpu("lse", lse, dev)
    B, Sq, H, D = q.shape
    P, lens, stride0 = _block_list(q, k_blocks, v_blocks, dev, allow_packed=True)
    if isinstance(v_blocks[0], PackedV):
        flags |= CP_RING_PACKED_V
    elif flags & CP_RING_PACKED_V:
        raise ValueError("CP_RING_PACKED_V needs V blocks from cp_attn_pack_v")
    if tuple(out.shape) != (B, Sq, H, D):
        raise ValueError("out must be [B, Sq, H, D]")
    _f32("out", out)
    _lse_shape("lse", lse, B, H, Sq)
    kptr = (ctypes.c_void_p * P)(*[kb.data_ptr() for kb in k_blocks])
    vptr = (ctypes.c_void_p * P)(*[vb.data_ptr() for vb in v_blocks])
    kvs = (ctypes.c_int64 * 3)(*stride0)
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.cp_ring_attention(q.data_ptr(), _strides(q), kptr, vptr, kvs, lens, P, _dtype_code(q), B, H,
                               D, Sq, scale, flags, out.data_ptr(), _strides(out), lse.data_ptr(), ws_ptr,
                               ws_bytes, _stream(stream))
    _check(st, "cp_ring_attention")


def _regroup_shapes(inp, out, degree: int, direction: int, dev):
    _gpu("inp", inp, dev)
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
    return B, S_l, H, D


def cp_ulysses_regroup(inp, out, degree: int, direction: int = CP_REGROUP_SEQ_TO_HEAD, stream=None):
    """Ulysses head/token regroup (loopback all-to-all permutation); see cp_ulysses_regroup.

    SEQ_TO_HEAD: inp [B, S_local, H, D] -> out [B, P*S_local, H/P, D];
    HEAD_TO_SEQ: inp [B, P*S_local, H/P, D] -> out [B, S_local, H, D]. Both contiguous.
    """
    lib = _lib.load()
    dev = _gpu("inp", inp).device
    B, S_l, H, D = _regroup_shapes(inp, out, degree, direction, dev)
    st = lib.cp_ulysses_regroup(inp.data_ptr(), out.data_ptr(), inp.element_size(), B, S_l, H, D, degree,
                                direction, _stream(stream))
    _check(st, "cp_ulysses_regroup")


def cp_ulysses_regroup_multi(inputs: Sequence, outputs: Sequence, degree: int,
                             direction: int = CP_REGROUP_SEQ_TO_HEAD, stream=None):
    """cp_ulysses_regroup of several tensors of one shape and dtype (Q, K and V) in one launch."""
    lib = _lib.load()
    if len(inputs) != len(outputs) or not 1 <= len(inputs) <= 8:
        raise ValueError("inputs and outputs must be equally long lists of 1..8 tensors")
    dev = _gpu("inputs[0]", inputs[0]).device
    shapes = {_regroup_shapes(i, o, degree, direction, dev) for i, o in zip(inputs, outputs)}
    if len(shapes) != 1 or len({t.dtype for t in inputs}) != 1:
        raise ValueError("every tensor must have the same shape and dtype")
    B, S_l, H, D = shapes.pop()
    n = len(inputs)
    ip = (ctypes.c_void_p * n)(*[t.data_ptr() for t in inputs])
    op = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outputs])
    st = lib.cp_ulysses_regroup_multi(ip, op, n, inputs[0].element_size(), B, S_l, H, D, degree, direction,
                                      _stream(stream))
    _check(st, "cp_ulysses_regroup_multi")


def split_counts(n: int, parts: int):
    """Uneven split sizes: the first n % parts parts get one more (e.g. 4481 over 4: 1121, 1120, 1120, 1120)."""
    if parts < 1 or n < 0:
        raise ValueError("need n >= 0 and parts >= 1")
    return [n // parts + (1 if i < n % parts else 0) for i in range(parts)]


def _counts(name, counts):
    counts = [int(c) for c in counts]
    if not counts or any(c < 0 for c in counts):
        raise ValueError(f"{name} must be a non-empty list of non-negative counts")
    return (ctypes.c_int * len(counts))(*counts), counts


def cp_ulysses_pack_heads(inp, out, head_counts: Sequence[int], direction: int = CP_REGROUP_SEQ_TO_HEAD,
                          stream=None):
    """Ulysses Anything: [B, S_r, H, D] <-> pieces [B, S_r, H_g, D] back to back (1-D ``out`` or ``inp``).

    SEQ_TO_HEAD: ``inp`` is the contiguous tensor, ``out`` a flat buffer of the same size;
    HEAD_TO_SEQ: the reverse. See cp_ulysses_pack_heads in the header.
    """
    lib = _lib.load()
    dev = _gpu("inp", inp).device
    _gpu("out", out, dev)
    arr, counts = _counts("head_counts", head_counts)
    tensor = inp if direction == CP_REGROUP_SEQ_TO_HEAD else out
    pieces = out if direction == CP_REGROUP_SEQ_TO_HEAD else inp
    if inp.dtype != out.dtype or not (inp.is_contiguous() and out.is_contiguous()) or tensor.dim() != 4:
        raise ValueError("tensors must share a dtype, be contiguous, and the tensor side must be [B, S_r, H, D]")
    B, S_r, H, D = tensor.shape
    if sum(counts) != H or pieces.numel() != tensor.numel():
        raise ValueError(f"head_counts must sum to H={H} and the pieces buffer must hold {tensor.numel()} elements")
    st = lib.cp_ulysses_pack_heads(inp.data_ptr(), out.data_ptr(), inp.element_size(), B, S_r, D, len(counts), arr,
                                   direction, _stream(stream))
    _check(st, "cp_ulysses_pack_heads")


def cp_ulysses_concat_seq(inp, out, seq_counts: Sequence[int], direction: int = CP_REGROUP_SEQ_TO_HEAD,
                          stream=None):
    """Ulysses Anything: pieces [B, S_r, H_g, D] back to back (flat) <-> [B, sum S_r, H_g, D].

    SEQ_TO_HEAD: ``inp`` is the flat pieces buffer, ``out`` the tensor; HEAD_TO_SEQ: the reverse.
    See cp_ulysses_concat_seq in the header.
    """
    lib = _lib.load()
    dev = _gpu("inp", inp).device
    _gpu("out", out, dev)
    arr, counts = _counts("seq_counts", seq_counts)
    tensor = out if direction == CP_REGROUP_SEQ_TO_HEAD else inp
    pieces = inp if direction == CP_REGROUP_SEQ_TO_HEAD else out
    if inp.dtype != out.dtype or not (inp.is_contiguous() and out.is_contiguous()) or tensor.dim() != 4:
        raise ValueError("tensors must share a dtype, be contiguous, and the tensor side must be [B, S, H_g, D]")
    B, S, Hg, D = tensor.shape
    if sum(counts) != S or pieces.numel() != tensor.numel():
        raise ValueError(f"seq_counts must sum to S={S} and the pieces buffer must hold {tensor.numel()} elements")
    st = lib.cp_ulysses_concat_seq(inp.data_ptr(), out.data_ptr(), inp.element_size(), B, Hg, D, len(counts), arr,
                                   direction, _stream(stream))
    _check(st, "cp_ulysses_concat_seq")


def cp_attn_bwd_workspace_size(B: int, H: int, Sq: int, D: int) -> int:
    return int(_lib.load().cp_attn_bwd_workspace_size(B, H, Sq, D))


def cp_attn_bwd_prep(out, dout, workspace, dtype: int = CP_BF16, stream=None):
    """Fill the backward workspace (dO in bfloat16 and D = rowsum(dO * O)); see cp_attn_bwd_prep."""
    lib = _lib.load()
    dev = _gpu("out", _bshd("out", out)).device
    _gpu("dout", _bshd("dout", dout), dev)
    B, Sq, H, D = out.shape
    if tuple(dout.shape) != (B, Sq, H, D):
        raise ValueError("dout must match out")
    _f32("out", out); _f32("dout", dout)
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    st = lib.cp_attn_bwd_prep(out.data_ptr(), _strides(out), dout.data_ptr(), _strides(dout), dtype, B, H, Sq, D,
                              ws_ptr, ws_bytes, _stream(stream))
    _check(st, "cp_attn_bwd_prep")


def cp_attn_block_bwd(q, k, v, lse, workspace, dq, dk, dv, scale: Optional[float] = None, flags: int = 0,
                      stream=None):
    """Gradients of one K/V block (dq overwritten or, with CP_BWD_ACCUMULATE_DQ, added to); see the header."""
    lib = _lib.load()
    dev = _gpu("q", _bshd("q", q)).device
    B, Sq, H, D = q.shape
    _, lens, kvs = _block_list(q, [k], [v], dev)
    _, _, dkvs = _block_list(q, [dk], [dv], dev, dtype=_torch().float32, what="dK/dV")
    if dk.shape[1] != k.shape[1]:
        raise ValueError("dk/dv must match k/v")
    _gpu("dq", _bshd("dq", dq), dev); _gpu("lse", lse, dev)
    if tuple(dq.shape) != (B, Sq, H, D):
        raise ValueError("dq must be [B, Sq, H, D]")
    _f32("dq", dq)
    _lse_shape("lse", lse, B, H, Sq)
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.cp_attn_block_bwd(q.data_ptr(), _strides(q), k.data_ptr(), v.data_ptr(), (ctypes.c_int64 * 3)(*kvs),
                               _dtype_code(q), B, H, D, Sq, lens[0], scale, flags, lse.data_ptr(), ws_ptr, ws_bytes,
                               dq.data_ptr(), _strides(dq), dk.data_ptr(), dv.data_ptr(),
                               (ctypes.c_int64 * 3)(*dkvs), _stream(stream))
    _check(st, "cp_attn_block_bwd")


def cp_ring_attention_bwd(q, k_blocks: Sequence, v_blocks: Sequence, out, lse, dout, dq, dk_blocks: Sequence,
                          dv_blocks: Sequence, scale: Optional[float] = None, flags: int = 0, workspace=None,
                          stream=None):
    """Backward of cp_ring_attention for one rank: dq and per-block dk, dv; see cp_ring_attention_bwd."""
    lib = _lib.load()
    dev = _gpu("q", _bshd("q", q)).device
    B, Sq, H, D = q.shape
    P, lens, kvs = _block_list(q, k_blocks, v_blocks, dev)
    P2, lens2, dkvs = _block_list(q, dk_blocks, dv_blocks, dev, dtype=_torch().float32, what="dK/dV")
    if P2 != P or list(lens2) != list(lens):
        raise ValueError("dk/dv blocks must match the K/V blocks")
    for name, t in (("out", out), ("dout", dout), ("dq", dq)):
        _gpu(name, _bshd(name, t), dev)
        _f32(name, t)
        if tuple(t.shape) != (B, Sq, H, D):
            raise ValueError(f"{name} must be [B, Sq, H, D]")
    _gpu("lse", lse, dev)
    _lse_shape("lse", lse, B, H, Sq)
    kptr = (ctypes.c_void_p * P)(*[t.data_ptr() for t in k_blocks])
    vptr = (ctypes.c_void_p * P)(*[t.data_ptr() for t in v_blocks])
    dkptr = (ctypes.c_void_p * P)(*[t.data_ptr() for t in dk_blocks])
    dvptr = (ctypes.c_void_p * P)(*[t.data_ptr() for t in dv_blocks])
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.cp_ring_attention_bwd(q.data_ptr(), _strides(q), kptr, vptr, (ctypes.c_int64 * 3)(*kvs), lens, P,
                                   _dtype_code(q), B, H, D, Sq, scale, flags, out.data_ptr(), _strides(out),
                                   dout.data_ptr(), _strides(dout), lse.data_ptr(), dq.data_ptr(), _strides(dq),
                                   dkptr, dvptr, (ctypes.c_int64 * 3)(*dkvs), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "cp_ring_attention_bwd")


# ------------------------------------------------------- allocating helpers ---

def pack_v(v, stream=None) -> PackedV:
    """Allocate the packed buffer and run cp_attn_pack_v on bfloat16 V [B, Skv, H, D]."""
    torch = _torch()
    B, Skv, H, D = v.shape
    nbytes = cp_attn_packed_v_bytes(B, H, D, Skv)
    buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=v.device)
    return cp_attn_pack_v(v, buf, stream=stream)


def ring_attention(q, k_blocks, v_blocks, scale: Optional[float] = None, ring_anything: Optional[bool] = None,
                   separate_merge: bool = False, stream=None, waves: int = 0) -> Tuple:
    """Allocate (out, lse) and run cp_ring_attention; returns (out, lse). ``waves`` (4 or 8) forces the
    bf16 block kernel's workgroup shape."""
    torch = _torch()
    B, Sq, H, D = q.shape
    out = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    lens = [kb.shape[1] for kb in k_blocks]
    if ring_anything is None:
        ring_anything = len(set(lens)) > 1 or 0 in lens
    flags = (CP_RING_ANYTHING if ring_anything else 0) | (CP_RING_SEPARATE_MERGE if separate_merge else 0)
    if any(isinstance(vb, PackedV) for vb in v_blocks):
        flags |= CP_RING_PACKED_V  # (the workspace then holds the one-launch ring's flags)
    ws = None
    nbytes = cp_ring_attention_workspace_size(B, H, Sq, D, flags)
    if nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    cp_ring_attention(q, k_blocks, v_blocks, out, lse, scale=scale, flags=flags, workspace=ws, stream=stream,
                      waves=waves)
    return out, lse


def ring_attention_bwd(q, k_blocks, v_blocks, out, lse, dout, scale: Optional[float] = None,
                       ring_anything: Optional[bool] = None, stream=None) -> Tuple:
    """Allocate the gradients and workspace and run cp_ring_attention_bwd; returns (dq, [dk_i], [dv_i]).

    dk_i, dv_i are views of one [B, sum(L_i), H, D] float32 buffer each.
    """
    torch = _torch()
    B, Sq, H, D = q.shape
    dq = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    lens = [kb.shape[1] for kb in k_blocks]
    # one [B, sum(lens), H, D] buffer each, so the blocks share a stride triple
    dk_all = torch.empty((B, sum(lens), H, D), dtype=torch.float32, device=q.device)
    dv_all = torch.empty((B, sum(lens), H, D), dtype=torch.float32, device=q.device)
    offs = [sum(lens[:i]) for i in range(len(lens))]
    dk = [dk_all[:, a:a + L] for a, L in zip(offs, lens)]
    dv = [dv_all[:, a:a + L] for a, L in zip(offs, lens)]
    if ring_anything is None:
        ring_anything = len(set(lens)) > 1 or 0 in lens
    nbytes = cp_attn_bwd_workspace_size(B, H, Sq, D)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    cp_ring_attention_bwd(q, k_blocks, v_blocks, out, lse, dout, dq, dk, dv, scale=scale,
                          flags=CP_RING_ANYTHING if ring_anything else 0, workspace=ws, stream=stream)
    return dq, dk, dv
