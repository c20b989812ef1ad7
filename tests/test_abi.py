"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

The pointers used here are fake host addresses; every call below fails
validation, which happens before anything is enqueued, so none of them is
ever dereferenced.
"""
import ctypes
import os

import pytest

from context_attention_dits_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.library_path()),
                                reason="libcpattn.so not built (python -m context_attention_dits_amd.build)")

FAKE = 0x10000  # 16-byte aligned, never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _lib.declared_symbols()
    assert {"cp_attn_block_fwd", "cp_lse_merge", "cp_ring_attention", "cp_ring_attention_workspace_size",
            "cp_ulysses_regroup", "cp_last_error", "cp_abi_version", "cp_attn_bwd_workspace_size",
            "cp_attn_bwd_prep", "cp_attn_block_bwd", "cp_ring_attention_bwd", "cp_ulysses_pack_heads",
            "cp_ulysses_concat_seq"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.cp_abi_version() == _lib.ABI_VERSION


def test_phase_trace_only_in_the_diagnostic_library(lib):
    """The tile-loop cycle trace (bench.py --phase-trace) and the synthetic ping-pong beside it
    live in their own library; the main one has neither the symbols nor the instrumentation's
    device buffer."""
    from context_attention_dits_amd.build import PHASE_TRACE_LIB
    assert not hasattr(lib, "cp_debug_phase_trace")
    path = os.path.join(os.path.dirname(_lib.DEFAULT_PATH), PHASE_TRACE_LIB)
    if _lib.library_path() != _lib.DEFAULT_PATH or not os.path.exists(path):
        pytest.skip("diagnostic library not built next to the default one")
    diag = ctypes.CDLL(path)
    assert hasattr(diag, "cp_debug_phase_trace")
    diag.cp_debug_phase_trace.argtypes = [ctypes.c_void_p, ctypes.c_long]
    diag.cp_debug_phase_trace.restype = ctypes.c_int
    # argument checks only (no copy is attempted, so no GPU is needed)
    assert diag.cp_debug_phase_trace(None, 8) != 0
    buf = (ctypes.c_ulonglong * 1)()
    assert diag.cp_debug_phase_trace(ctypes.addressof(buf), -1) != 0
    assert diag.cp_debug_phase_trace(ctypes.addressof(buf), 1 << 40) != 0
    # the synthetic ping-pong beside it: argument checks only
    assert not hasattr(lib, "cp_debug_mix_probe")
    diag.cp_debug_mix_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    diag.cp_debug_mix_probe.restype = ctypes.c_int
    cyc, ms = ctypes.c_double(), ctypes.c_double()
    for v, it, a, b in ((8, 100, cyc, ms), (-1, 100, cyc, ms), (0, 1, cyc, ms), (0, 1 << 21, cyc, ms)):
        assert diag.cp_debug_mix_probe(v, it, ctypes.addressof(a), ctypes.addressof(b)) != 0
    assert diag.cp_debug_mix_probe(0, 100, None, ctypes.addressof(ms)) != 0
    assert diag.cp_debug_mix_probe(0, 100, ctypes.addressof(cyc), None) != 0


def _block(lib, dtype=1, B=1, H=2, D=128, Sq=8, Skv=8, scale=0.1, flags=0, q=FAKE, k=FAKE, v=FAKE,
           out=FAKE, lse=FAKE, qs=None, kvs=None, os_=None):
    return lib.cp_attn_block_fwd(q, qs, k, v, kvs, dtype, B, H, D, Sq, Skv, scale, flags, out, os_, lse, None)


def _err(lib):
    return lib.cp_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=7), _lib.CP_ERR_UNSUPPORTED, "dtype"),
    (dict(D=96), _lib.CP_ERR_UNSUPPORTED, "D=96"),
    (dict(D=256), _lib.CP_ERR_UNSUPPORTED, "supported"),
    (dict(B=-1), _lib.CP_ERR_INVALID_ARG, "non-negative"),
    (dict(Skv=-3), _lib.CP_ERR_INVALID_ARG, "non-negative"),
    (dict(scale=0.0), _lib.CP_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), _lib.CP_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("inf")), _lib.CP_ERR_INVALID_ARG, "scale"),
    (dict(flags=0x80), _lib.CP_ERR_INVALID_ARG, "flags"),
    (dict(q=0), _lib.CP_ERR_INVALID_ARG, "non-null"),
    (dict(lse=0), _lib.CP_ERR_INVALID_ARG, "non-null"),
    (dict(k=0), _lib.CP_ERR_INVALID_ARG, "non-null"),
    (dict(q=FAKE + 8), _lib.CP_ERR_UNSUPPORTED, "aligned"),
    (dict(v=FAKE + 2), _lib.CP_ERR_UNSUPPORTED, "aligned"),
])
def test_block_fwd_rejects(lib, kw, status, needle):
    assert _block(lib, **kw) == status
    assert needle in _err(lib)


def test_block_fwd_rejects_bad_strides(lib):
    bad = (ctypes.c_int64 * 3)(8 * 2 * 128, 2 * 128 + 4, 128)  # 4 bf16 = 8 bytes: not 16-B multiple
    assert _block(lib, qs=bad) == _lib.CP_ERR_UNSUPPORTED
    neg = (ctypes.c_int64 * 3)(-1, 256, 128)
    assert _block(lib, kvs=neg) == _lib.CP_ERR_INVALID_ARG
    overlap = (ctypes.c_int64 * 3)(8 * 2 * 128, 2 * 128, 64)  # heads overlap along D=128
    assert _block(lib, os_=overlap) == _lib.CP_ERR_INVALID_ARG


def test_empty_problem_is_a_no_op(lib):
    # B, H or Sq == 0 enqueues nothing, so even null pointers are fine.
    assert _block(lib, Sq=0, q=0, k=0, v=0, out=0, lse=0) == _lib.CP_OK
    assert _block(lib, B=0, q=0, k=0, v=0, out=0, lse=0) == _lib.CP_OK


def _ring(lib, lens, flags=0, dtype=1, ws=None, ws_bytes=0, kptrs=None):
    P = len(lens)
    karr = (ctypes.c_void_p * P)(*(kptrs or [FAKE] * P))
    varr = (ctypes.c_void_p * P)(*([FAKE] * P))
    L = (ctypes.c_int * P)(*lens)
    return lib.cp_ring_attention(FAKE, None, karr, varr, None, L, P, dtype, 1, 2, 128, 8, 0.1, flags, FAKE, None,
                                 FAKE, ws, ws_bytes, None)


def test_ring_rejects_uneven_without_ring_anything(lib):
    assert _ring(lib, [1536, 1536, 1535]) == _lib.CP_ERR_INVALID_ARG
    assert "CP_RING_ANYTHING" in _err(lib)
    assert _ring(lib, [0, 0]) == _lib.CP_ERR_INVALID_ARG
    assert _ring(lib, [4, -1], flags=_lib.CP_RING_ANYTHING) == _lib.CP_ERR_INVALID_ARG


def test_ring_rejects_degree_flags_and_null_blocks(lib):
    assert _ring(lib, []) == _lib.CP_ERR_INVALID_ARG
    assert "ring_degree" in _err(lib)
    assert _ring(lib, [8, 8], flags=0x1000) == _lib.CP_ERR_INVALID_ARG
    assert _ring(lib, [8, 8], kptrs=[FAKE, 0]) == _lib.CP_ERR_INVALID_ARG
    assert "block 1" in _err(lib)


def test_ring_workspace_rules(lib):
    need = lib.cp_ring_attention_workspace_size(1, 2, 8, 128, _lib.CP_RING_SEPARATE_MERGE)
    assert need >= 4 * (1 * 8 * 2 * 128 + 1 * 2 * 8)
    assert lib.cp_ring_attention_workspace_size(1, 2, 8, 128, 0) == 0
    assert _ring(lib, [8, 8], flags=_lib.CP_RING_SEPARATE_MERGE) == _lib.CP_ERR_WORKSPACE
    assert _ring(lib, [8, 8], flags=_lib.CP_RING_SEPARATE_MERGE, ws=FAKE, ws_bytes=need - 1) == _lib.CP_ERR_WORKSPACE
    assert _ring(lib, [8, 8], flags=_lib.CP_RING_SEPARATE_MERGE, ws=FAKE + 16, ws_bytes=need) == _lib.CP_ERR_UNSUPPORTED


def test_merge_rejects(lib):
    f = lib.cp_lse_merge
    assert f(FAKE, FAKE, FAKE + 4096, FAKE + 8192, None, None, 1, 2, 8, 80, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE + 8192, None, None, 1, 2, 8, 128, None) == _lib.CP_ERR_INVALID_ARG
    assert f(0, FAKE, FAKE, FAKE, None, None, 1, 2, 8, 128, None) == _lib.CP_ERR_INVALID_ARG
    assert f(0, 0, 0, 0, None, None, 1, 0, 8, 128, None) == _lib.CP_OK
    # B*Sq*H*D/4 at 2^31 is beyond the kernel's 32-bit indices
    assert f(FAKE, FAKE, FAKE + (1 << 30), FAKE + (1 << 31), None, None, 2, 1 << 10, 1 << 15, 128,
             None) == _lib.CP_ERR_UNSUPPORTED
    assert "2^31" in _err(lib)


def test_regroup_rejects(lib):
    f = lib.cp_ulysses_regroup
    assert f(FAKE, FAKE + (1 << 30), 2, 1, 16, 24, 128, 5, 0, None) == _lib.CP_ERR_INVALID_ARG
    assert "divisible" in _err(lib)
    assert f(FAKE, FAKE + (1 << 30), 3, 1, 16, 24, 128, 2, 0, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(FAKE, FAKE + (1 << 30), 2, 1, 16, 24, 128, 0, 0, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE, FAKE + (1 << 30), 2, 1, 16, 24, 128, 2, 9, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE, FAKE + 64, 2, 1, 16, 24, 128, 2, 0, None) == _lib.CP_ERR_INVALID_ARG  # overlap
    assert "overlap" in _err(lib)
    assert f(0, 0, 2, 0, 16, 24, 128, 2, 0, None) == _lib.CP_OK


def test_regroup_multi_rejects(lib):
    import ctypes
    f = lib.cp_ulysses_regroup_multi
    V = ctypes.c_void_p * 3
    ins, outs = V(FAKE, FAKE + (1 << 28), FAKE + (2 << 28)), V(FAKE + (3 << 28), FAKE + (4 << 28), FAKE + (5 << 28))
    assert f(ins, outs, 0, 2, 1, 16, 24, 128, 2, 0, None) == _lib.CP_ERR_INVALID_ARG
    assert "n_tensors" in _err(lib)
    assert f(ins, outs, 9, 2, 1, 16, 24, 128, 2, 0, None) == _lib.CP_ERR_INVALID_ARG
    assert f(None, outs, 3, 2, 1, 16, 24, 128, 2, 0, None) == _lib.CP_ERR_INVALID_ARG
    assert f(ins, outs, 3, 2, 1, 16, 24, 128, 5, 0, None) == _lib.CP_ERR_INVALID_ARG
    assert "divisible" in _err(lib)
    # an output overlapping another tensor's input, or two outputs overlapping, is refused
    assert f(ins, V(FAKE + (3 << 28), FAKE + 64, FAKE + (5 << 28)), 3, 2, 1, 16, 24, 128, 2, 0,
             None) == _lib.CP_ERR_INVALID_ARG
    assert "overlap" in _err(lib)
    assert f(ins, V(FAKE + (3 << 28), FAKE + (3 << 28) + 64, FAKE + (5 << 28)), 3, 2, 1, 16, 24, 128, 2, 0,
             None) == _lib.CP_ERR_INVALID_ARG
    assert "overlap" in _err(lib)
    # shared inputs are fine; an empty problem enqueues nothing
    assert f(V(0, 0, 0), V(0, 0, 0), 3, 2, 0, 16, 24, 128, 2, 0, None) == _lib.CP_OK


BWD_NEED = 4096 + 256  # bf16 dO [1, 8, 2, 128] and D [1, 2, 8] float32, each padded to 256 bytes


def _block_bwd(lib, dtype=1, B=1, H=2, D=128, Sq=8, Skv=8, scale=0.1, flags=0, q=FAKE, k=FAKE, v=FAKE,
               lse=FAKE, ws=FAKE, ws_bytes=BWD_NEED, dq=FAKE, dk=FAKE, dv=FAKE, qs=None, kvs=None):
    return lib.cp_attn_block_bwd(q, qs, k, v, kvs, dtype, B, H, D, Sq, Skv, scale, flags, lse, ws, ws_bytes,
                                 dq, None, dk, dv, None, None)


def test_bwd_workspace_size(lib):
    assert lib.cp_attn_bwd_workspace_size(1, 2, 8, 128) == BWD_NEED
    assert lib.cp_attn_bwd_workspace_size(1, 24, 4608, 128) == 1 * 4608 * 24 * 128 * 2 + 24 * 4608 * 4
    assert lib.cp_attn_bwd_workspace_size(1, 2, 0, 128) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=0), _lib.CP_ERR_UNSUPPORTED, "CP_BF16"),
    (dict(D=96), _lib.CP_ERR_UNSUPPORTED, "D=96"),
    (dict(flags=0x2), _lib.CP_ERR_INVALID_ARG, "flags"),
    (dict(scale=-1.0), _lib.CP_ERR_INVALID_ARG, "scale"),
    (dict(Skv=-1), _lib.CP_ERR_INVALID_ARG, "non-negative"),
    (dict(q=0), _lib.CP_ERR_INVALID_ARG, "non-null"),
    (dict(dq=0), _lib.CP_ERR_INVALID_ARG, "non-null"),
    (dict(lse=0), _lib.CP_ERR_INVALID_ARG, "non-null"),
    (dict(k=0), _lib.CP_ERR_INVALID_ARG, "non-null"),
    (dict(dv=0), _lib.CP_ERR_INVALID_ARG, "dk and dv"),
    (dict(dk=FAKE + 8), _lib.CP_ERR_INVALID_ARG, "aligned"),
    (dict(ws=0), _lib.CP_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=BWD_NEED - 1), _lib.CP_ERR_WORKSPACE, "workspace"),
    (dict(ws=FAKE + 16), _lib.CP_ERR_UNSUPPORTED, "256-byte"),
    (dict(qs=(ctypes.c_int64 * 3)(1 << 30, (1 << 24) + 8, 128)), _lib.CP_ERR_UNSUPPORTED, "2^24"),
])
def test_block_bwd_rejects(lib, kw, status, needle):
    assert _block_bwd(lib, **kw) == status
    assert needle in _err(lib)


def test_block_bwd_empty_is_a_no_op(lib):
    assert _block_bwd(lib, B=0, q=0, k=0, v=0, lse=0, ws=0, dq=0, dk=0, dv=0) == _lib.CP_OK
    assert _block_bwd(lib, Sq=0, Skv=0, q=0, k=0, v=0, lse=0, ws=0, dq=0, dk=0, dv=0) == _lib.CP_OK


def test_bwd_prep_rejects(lib):
    f = lib.cp_attn_bwd_prep
    assert f(FAKE, None, FAKE, None, 0, 1, 2, 8, 128, FAKE, BWD_NEED, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(0, None, FAKE, None, 1, 1, 2, 8, 128, FAKE, BWD_NEED, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE, None, FAKE + 4, None, 1, 1, 2, 8, 128, FAKE, BWD_NEED, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(FAKE, None, FAKE, None, 1, 1, 2, 8, 128, FAKE, BWD_NEED - 256, None) == _lib.CP_ERR_WORKSPACE
    assert f(0, None, 0, None, 1, 1, 2, 0, 128, 0, 0, None) == _lib.CP_OK


def _ring_bwd(lib, lens, flags=0, dtype=1, ws=FAKE, ws_bytes=BWD_NEED, dkptrs=None, out=FAKE):
    P = len(lens)
    arr = lambda xs: (ctypes.c_void_p * P)(*xs)  # noqa: E731
    L = (ctypes.c_int * P)(*lens)
    return lib.cp_ring_attention_bwd(FAKE, None, arr([FAKE] * P), arr([FAKE] * P), None, L, P, dtype, 1, 2, 128, 8,
                                     0.1, flags, out, None, FAKE, None, FAKE, FAKE, None,
                                     arr(dkptrs or [FAKE] * P), arr([FAKE] * P), None, ws, ws_bytes, None)


def test_ring_bwd_rejects(lib):
    assert _ring_bwd(lib, [8, 7]) == _lib.CP_ERR_INVALID_ARG
    assert "CP_RING_ANYTHING" in _err(lib)
    assert _ring_bwd(lib, []) == _lib.CP_ERR_INVALID_ARG
    assert _ring_bwd(lib, [8, 8], flags=_lib.CP_RING_SEPARATE_MERGE) == _lib.CP_ERR_INVALID_ARG
    assert _ring_bwd(lib, [8, 8], dtype=0) == _lib.CP_ERR_UNSUPPORTED
    assert _ring_bwd(lib, [8, 8], dkptrs=[FAKE, 0]) == _lib.CP_ERR_INVALID_ARG
    assert "block 1" in _err(lib)
    assert _ring_bwd(lib, [8, 8], ws_bytes=16) == _lib.CP_ERR_WORKSPACE
    assert _ring_bwd(lib, [8, 8], out=0) == _lib.CP_ERR_INVALID_ARG
    assert "out and dout" in _err(lib)


def test_uneven_packs_reject(lib):
    counts = (ctypes.c_int * 3)(2, 1, 3)
    big = FAKE + (1 << 30)
    for f in (lib.cp_ulysses_pack_heads, lib.cp_ulysses_concat_seq):
        assert f(FAKE, big, 3, 1, 16, 128, 3, counts, 0, None) == _lib.CP_ERR_UNSUPPORTED  # elem_bytes
        assert f(FAKE, big, 2, 1, 16, 128, 0, counts, 0, None) == _lib.CP_ERR_INVALID_ARG  # degree
        assert f(FAKE, big, 2, 1, 16, 128, 65, counts, 0, None) == _lib.CP_ERR_INVALID_ARG
        assert "1..64" in _err(lib)
        assert f(FAKE, big, 2, 1, 16, 128, 3, None, 0, None) == _lib.CP_ERR_INVALID_ARG  # counts
        assert f(FAKE, big, 2, 1, 16, 128, 3, counts, 5, None) == _lib.CP_ERR_INVALID_ARG  # direction
        neg = (ctypes.c_int * 2)(3, -1)
        assert f(FAKE, big, 2, 1, 16, 128, 2, neg, 0, None) == _lib.CP_ERR_INVALID_ARG
        assert "negative" in _err(lib)
        assert f(FAKE, FAKE + 64, 2, 1, 16, 128, 3, counts, 0, None) == _lib.CP_ERR_INVALID_ARG  # overlap
        assert "overlap" in _err(lib)
        assert f(0, 0, 2, 0, 16, 128, 3, counts, 0, None) == _lib.CP_OK  # empty: nothing enqueued
        huge = (ctypes.c_int * 1)(1 << 20)
        assert f(FAKE, big, 2, 16, 16, 128, 1, huge, 0, None) == _lib.CP_ERR_UNSUPPORTED  # >= 2^32 bytes
        assert "2^32" in _err(lib)


def test_split_counts():
    import context_attention_dits_amd as cp
    assert cp.split_counts(4481, 4) == [1121, 1120, 1120, 1120]
    assert cp.split_counts(24, 5) == [5, 5, 5, 5, 4]
    assert cp.split_counts(2, 3) == [1, 1, 0]


def test_shape_flags(lib):
    """The bf16 workgroup shape is forced per call by a flag; both flags together are refused, and
    the library exports no process-wide setting for it."""
    four, eight = _lib.CP_FWD_FOUR_WAVES, _lib.CP_FWD_EIGHT_WAVES
    assert not hasattr(lib, "cp_attn_set_fwd_waves")
    assert _block(lib, flags=four | eight) == _lib.CP_ERR_INVALID_ARG
    assert "together" in _err(lib)
    assert _ring(lib, [8, 8], flags=four | eight) == _lib.CP_ERR_INVALID_ARG
    # each flag alone passes validation (the call then fails later on the fake pointers' contents
    # only on a GPU; here a zero-sized problem stops it first)
    assert _block(lib, flags=four, B=0) == _lib.CP_OK
    assert _block(lib, flags=eight, B=0) == _lib.CP_OK
    import context_attention_dits_amd as cp
    assert cp.wave_flags(0) == 0 and cp.wave_flags(4) == four and cp.wave_flags(8) == eight
    with pytest.raises(ValueError):
        cp.wave_flags(5)


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    import context_attention_dits_amd as cp
    q = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16)
    out = torch.zeros(1, 8, 2, 128)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError, match="GPU"):
        cp.cp_attn_block_fwd(q, q, q, out, lse)
    with pytest.raises(ValueError, match="GPU"):
        cp.cp_ulysses_regroup(q, q.clone(), 2)


def test_packed_v_size_and_rejects(lib):
    """cp_attn_pack_v and the packed-V flags: every rejection happens on the host."""
    assert lib.cp_attn_packed_v_bytes(1, 24, 128, 2304) == 24 * 36 * 64 * 128 * 2
    assert lib.cp_attn_packed_v_bytes(2, 3, 64, 65) == 2 * 3 * 2 * 64 * 64 * 2  # padded to 64 keys
    assert lib.cp_attn_packed_v_bytes(1, 2, 96, 8) == 0  # unsupported D
    assert lib.cp_attn_packed_v_bytes(1, 2, 128, 0) == 0
    need = lib.cp_attn_packed_v_bytes(1, 2, 128, 8)
    big = FAKE + (1 << 30)
    f = lib.cp_attn_pack_v
    assert f(FAKE, None, 1, 2, 96, 8, big, need, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(FAKE, None, 1, -2, 128, 8, big, need, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE, None, 1, 2, 128, 8, big, need - 1, None) == _lib.CP_ERR_INVALID_ARG
    assert "needed" in _err(lib)
    assert f(0, None, 1, 2, 128, 8, big, need, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE + 8, None, 1, 2, 128, 8, big, need, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(FAKE, None, 1, 2, 128, 8, FAKE + 64, need, None) == _lib.CP_ERR_INVALID_ARG  # overlap
    assert "overlap" in _err(lib)
    bad = (ctypes.c_int64 * 3)(8 * 2 * 128, 2 * 128 + 1, 128)  # row stride not 16-byte aligned
    assert f(FAKE, bad, 1, 2, 128, 8, big, need, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(FAKE, None, 1, 2, 128, 0, 0, 0, None) == _lib.CP_OK  # nothing to pack
    # packed V is bf16 only, on both attention entry points
    assert _block(lib, dtype=0, flags=_lib.CP_BLOCK_PACKED_V) == _lib.CP_ERR_UNSUPPORTED
    assert "packed" in _err(lib)
    assert _block(lib, flags=0x4) == _lib.CP_ERR_INVALID_ARG
    assert _ring(lib, [8, 8], dtype=0, flags=_lib.CP_RING_PACKED_V) == _lib.CP_ERR_UNSUPPORTED
    assert _ring(lib, [8, 8], flags=0x10) == _lib.CP_ERR_INVALID_ARG


def test_regroup_pack_v_rejects(lib):
    f = lib.cp_ulysses_regroup_pack_v
    big = FAKE + (1 << 30)
    need = lib.cp_attn_packed_v_bytes(1, 12, 128, 2 * 16)
    assert f(FAKE, 1, 16, 24, 96, 2, big, need, None) == _lib.CP_ERR_UNSUPPORTED  # D
    assert f(FAKE, 1, 16, 24, 128, 5, big, need, None) == _lib.CP_ERR_INVALID_ARG  # 5 does not divide 24
    assert "divisible" in _err(lib)
    assert f(FAKE, 1, 16, 24, 128, 0, big, need, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE, 1, 16, 24, 128, 2, big, need - 1, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE + 8, 1, 16, 24, 128, 2, big, need, None) == _lib.CP_ERR_UNSUPPORTED
    assert f(FAKE, 1, 16, 24, 128, 2, FAKE + 1024, need, None) == _lib.CP_ERR_INVALID_ARG  # overlap
    assert f(0, 1, 16, 24, 128, 2, big, need, None) == _lib.CP_ERR_INVALID_ARG
    assert f(FAKE, 1, 0, 24, 128, 2, 0, 0, None) == _lib.CP_OK  # nothing to do


def test_fwd_waves_query(lib):
    """The bf16 kernel's workgroup shape for the benchmark shapes, and its knob."""
    def q(B, H, D, Sq, flags=0):
        return lib.cp_attn_fwd_waves(B, H, D, Sq, flags)
    assert q(1, 24, 128, 2304) == 8   # 216 ping-pong workgroups: one round, mostly full
    assert q(1, 12, 128, 4608) == 8
    assert q(1, 24, 128, 8192) == 8
    assert q(2, 24, 128, 1536) == 4   # 288: the second round would be nearly empty
    assert q(1, 12, 128, 2304) == 4   # 108: under half a round
    assert q(1, 24, 64, 8192) == 4    # D = 64 has the 4-wave kernel only
    assert q(0, 24, 128, 2304) == 0 and q(1, 24, 96, 2304) == 0
    eight, four = _lib.CP_FWD_EIGHT_WAVES, _lib.CP_FWD_FOUR_WAVES
    assert q(1, 12, 128, 2304, eight) == 8 and q(1, 24, 64, 8192, eight) == 4
    assert q(1, 24, 128, 2304, four) == 4
    assert q(1, 24, 128, 2304, four | eight) == 0


def test_plain_c_consumer(tmp_path):
    """tests/c/abi_consumer.c, built with gcc as strict C99 against include/cp_attn.h and linked
    to libcpattn.so, runs its size and validation checks (no GPU, no Python in the process)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(_lib.library_path())
    exe = str(tmp_path / "abi_consumer")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(root, "include"),
           os.path.join(root, "tests", "c", "abi_consumer.c"), _lib.library_path(),
           f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_ring_one_launch_workspace_rules(lib):
    """With packed V (bf16, D = 128) the ring can run as one launch, whose error count and
    per-query-tile flags live in the workspace: 256 bytes, then one int per 256-row tile of each
    (b, h), in 256-byte units. Without a workspace the ring still runs, one launch per block; a
    workspace that is too small or misaligned is rejected, and so is one too small or misaligned
    for cp_ring_attention_check."""
    pk = _lib.CP_RING_PACKED_V
    assert lib.cp_ring_attention_workspace_size(1, 24, 2304, 128, pk) == 256 + 1024  # 9 * 24 ints
    assert lib.cp_ring_attention_workspace_size(2, 24, 1536, 128, pk | _lib.CP_RING_ANYTHING) == 256 + 1280
    assert lib.cp_ring_attention_workspace_size(1, 24, 2304, 64, pk) == 0
    assert lib.cp_ring_attention_workspace_size(1, 24, 2304, 128, 0) == 0
    need = lib.cp_ring_attention_workspace_size(1, 2, 8, 128, pk)
    assert need == 512
    assert lib.cp_ring_attention_check(None, need, None) == _lib.CP_ERR_WORKSPACE
    assert lib.cp_ring_attention_check(FAKE, 64, None) == _lib.CP_ERR_WORKSPACE
    assert lib.cp_ring_attention_check(FAKE + 16, need, None) == _lib.CP_ERR_UNSUPPORTED
    assert _ring(lib, [8, 8], flags=pk, ws=FAKE, ws_bytes=need - 4) == _lib.CP_ERR_WORKSPACE
    assert _ring(lib, [8, 8], flags=pk, ws=FAKE + 16, ws_bytes=need) == _lib.CP_ERR_UNSUPPORTED


def test_ring_one_launch_query(lib):
    """Which packed rings run as one launch (bf16, D = 128): 2 to 16 non-empty blocks in parallel
    on grids the per-block launches would run on the 4-wave kernel (one block: split in two), and
    2 to 16 non-empty blocks in turn per workgroup on the 8-wave shape."""
    par, turn = _lib.CP_ONE_LAUNCH_PARALLEL, _lib.CP_ONE_LAUNCH_IN_TURN

    def q(dtype, B, H, D, Sq, lens, flags=0):
        arr = (ctypes.c_int * len(lens))(*lens)
        return lib.cp_ring_attention_one_launch(dtype, B, H, D, Sq, arr, len(lens), flags)
    assert q(1, 2, 24, 128, 1536, [1536, 1536, 1535]) == par   # ring-anything share
    assert q(1, 1, 12, 128, 2304, [2304, 2304]) == par         # USP share
    assert q(1, 1, 24, 128, 2304, [2304, 2304]) == turn        # FLUX ring-2: 8-wave, blocks in turn
    assert q(1, 1, 24, 128, 2304, [2304] * 4) == turn          # 8-wave: up to 16 blocks in turn
    assert q(1, 1, 24, 128, 2304, [2304] * 16 + [0]) == turn
    assert q(1, 1, 24, 128, 2304, [2304] * 17) == 0            # more: one launch per block
    assert q(1, 2, 24, 128, 1536, [1536, 0, 1535]) == par      # empty blocks do not count
    assert q(1, 2, 24, 128, 1536, [1536] * 4) == par           # 4-wave grid: up to 16 blocks in parallel
    assert q(1, 2, 24, 128, 1536, [1536] * 17) == 0
    assert q(1, 2, 24, 128, 1536, [1536, 0, 0]) == par         # one block: two halves in parallel
    assert q(1, 1, 6, 128, 4481, [4481]) == par                # the Ulysses Anything share, split in two
    assert q(1, 1, 12, 128, 4608, [4608]) == 0                 # Ulysses-2: 8-wave per block
    assert q(1, 1, 12, 128, 4608, [4608], _lib.CP_FWD_FOUR_WAVES) == 0
    assert q(1, 1, 6, 128, 4481, [127]) == 0                   # under two tiles: not split
    assert q(0, 2, 24, 128, 1536, [1536, 1536]) == 0           # float32
    assert q(1, 2, 24, 64, 1536, [1536, 1536]) == 0            # D = 64
    assert q(1, 1, 24, 128, 2304, [2304, 2304], _lib.CP_FWD_EIGHT_WAVES) == par
    assert q(1, 1, 12, 128, 2304, [2304, 2304], _lib.CP_FWD_FOUR_WAVES) == 0
    assert q(1, 1, 12, 128, 2304, [2304, 2304], _lib.CP_RING_SEPARATE_MERGE) == 0
