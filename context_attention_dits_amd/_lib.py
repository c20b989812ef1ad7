"""ctypes loader for the C-ABI library ``libcpattn.so`` (see include/cp_attn.h).

The library is built in-tree by ``context_attention_dits_amd.build``. There is
no fallback: if it is missing, loading raises, naming the build command.
``CP_ATTN_LIBRARY`` may point at another build of the same sources (e.g. a
tile variant).
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(PKG), "include", "cp_attn.h")
DEFAULT_PATH = os.path.join(PKG, "libcpattn.so")

CP_OK = 0
CP_ERR_INVALID_ARG = 1
CP_ERR_UNSUPPORTED = 2
CP_ERR_WORKSPACE = 3
CP_ERR_HIP = 4
CP_ERR_ORDER = 5
STATUS_NAMES = {0: "CP_OK", 1: "CP_ERR_INVALID_ARG", 2: "CP_ERR_UNSUPPORTED", 3: "CP_ERR_WORKSPACE",
                4: "CP_ERR_HIP", 5: "CP_ERR_ORDER"}
ABI_VERSION = 2

CP_F32 = 0
CP_BF16 = 1

CP_BLOCK_ACCUMULATE = 0x1
CP_BLOCK_PACKED_V = 0x2
CP_RING_ANYTHING = 0x2
CP_RING_SEPARATE_MERGE = 0x4
CP_RING_PACKED_V = 0x8
CP_FWD_FOUR_WAVES = 0x100
CP_FWD_EIGHT_WAVES = 0x200
CP_ONE_LAUNCH_IN_TURN = 1
CP_ONE_LAUNCH_PARALLEL = 2

CP_BWD_ACCUMULATE_DQ = 0x1

CP_REGROUP_SEQ_TO_HEAD = 0
CP_REGROUP_HEAD_TO_SEQ = 1

_vp = ctypes.c_void_p
_i = ctypes.c_int
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "cp_abi_version": (_i, []),
    "cp_last_error": (ctypes.c_char_p, []),
    "cp_attn_fwd_waves": (_i, [_i, _i, _i, _i, ctypes.c_uint]),
    "cp_ring_attention_one_launch": (_i, [_i, _i, _i, _i, _i, ctypes.POINTER(_i), _i, ctypes.c_uint]),
    "cp_ring_attention_check": (_i, [_vp, ctypes.c_size_t, _vp]),
    "cp_ring_attention_noalloc": (_i, [_vp, _i64p, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64p,
                                       ctypes.POINTER(_i), _i, _i, _i, _i, _i, _i, ctypes.c_float, ctypes.c_uint,
                                       _vp, _i64p, _vp, _vp]),
    "cp_attn_block_fwd": (_i, [_vp, _i64p, _vp, _vp, _i64p, _i, _i, _i, _i, _i, _i, ctypes.c_float,
                               ctypes.c_uint, _vp, _i64p, _vp, _vp]),
    "cp_lse_merge": (_i, [_vp, _vp, _vp, _vp, _i64p, _i64p, _i, _i, _i, _i, _vp]),
    "cp_attn_packed_v_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "cp_attn_pack_v": (_i, [_vp, _i64p, _i, _i, _i, _i, _vp, ctypes.c_size_t, _vp]),
    "cp_ulysses_regroup_pack_v": (_i, [_vp, _i, _i, _i, _i, _i, _vp, ctypes.c_size_t, _vp]),
    "cp_ring_attention_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i, ctypes.c_uint]),
    "cp_ring_attention": (_i, [_vp, _i64p, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64p,
                               ctypes.POINTER(_i), _i, _i, _i, _i, _i, _i, ctypes.c_float, ctypes.c_uint,
                               _vp, _i64p, _vp, _vp, ctypes.c_size_t, _vp]),
    "cp_ulysses_regroup": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "cp_ulysses_regroup_multi": (_i, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _i, _i, _i, _i, _i, _i, _i,
                                      _vp]),
    "cp_ulysses_pack_heads": (_i, [_vp, _vp, _i, _i, _i, _i, _i, ctypes.POINTER(_i), _i, _vp]),
    "cp_ulysses_concat_seq": (_i, [_vp, _vp, _i, _i, _i, _i, _i, ctypes.POINTER(_i), _i, _vp]),
    "cp_attn_bwd_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "cp_attn_bwd_prep": (_i, [_vp, _i64p, _vp, _i64p, _i, _i, _i, _i, _i, _vp, ctypes.c_size_t, _vp]),
    "cp_attn_block_bwd": (_i, [_vp, _i64p, _vp, _vp, _i64p, _i, _i, _i, _i, _i, _i, ctypes.c_float,
                               ctypes.c_uint, _vp, _vp, ctypes.c_size_t, _vp, _i64p, _vp, _vp, _i64p, _vp]),
    "cp_ring_attention_bwd": (_i, [_vp, _i64p, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64p,
                                   ctypes.POINTER(_i), _i, _i, _i, _i, _i, _i, ctypes.c_float, ctypes.c_uint,
                                   _vp, _i64p, _vp, _i64p, _vp, _vp, _i64p, ctypes.POINTER(_vp),
                                   ctypes.POINTER(_vp), _i64p, _vp, ctypes.c_size_t, _vp]),
}

_lib = None


def library_path() -> str:
    return os.environ.get("CP_ATTN_LIBRARY") or DEFAULT_PATH


def load() -> ctypes.CDLL:
    """Load (once) and return the library with argument types set."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    try:  # torch's HIP runtime first, so that the library binds to the same one
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not found at {path}. Build it first: "
            "`python -m context_attention_dits_amd.build` (or __graft_entry__.build()).")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.cp_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path}: ABI version {lib.cp_abi_version()}, expected {ABI_VERSION}")
    _lib = lib
    return lib


def declared_symbols(header: str = HEADER):
    """Names of the functions include/cp_attn.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(cp_\w+)\s*\(", text, flags=re.M)))
