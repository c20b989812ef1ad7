"""cp_ring_attention_noalloc: the ring share with the library's static workspace, no allocation.

Called through the C ABI (ctypes, no binding helper that allocates), checked against
cp_ring_attention with a caller workspace on the same inputs: the same kernels run, so the bits
must agree, and both must match the float64 oracle to the bf16 tolerances. Two calls in a row,
the second with a smaller problem, so the static array's contents left by the first call must be
reset by the second. The shapes run the parallel-partials form (grids the per-block launches
would run on four waves), the one that uses the workspace.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, assert_close, dev, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    import context_attention_dits_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()
    return m


def _noalloc(cp, q, kb, pv, out, lse, scale, flags):
    lib = cp.load()
    P = len(kb)
    B, Sq, H, D = q.shape
    lens = (ctypes.c_int * P)(*[x.shape[1] for x in kb])
    kp = (ctypes.c_void_p * P)(*[x.data_ptr() for x in kb])
    vp = (ctypes.c_void_p * P)(*[x.data.data_ptr() for x in pv])
    kvs = (ctypes.c_int64 * 3)(*kb[0].stride()[:3])
    return lib.cp_ring_attention_noalloc(q.data_ptr(), None, kp, vp, kvs, lens, P, cp.CP_BF16, B, H, D, Sq,
                                         float(scale), flags | cp.CP_RING_PACKED_V, out.data_ptr(), None,
                                         lse.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("first,second", [((2, 3, 700, (300, 0, 257, 64)), (1, 2, 260, (200, 130))),
                                          ((1, 12, 2304, (2304, 2304)), (1, 4, 300, (256, 200)))])
def test_noalloc_matches_workspace_ring(cp, first, second):
    for B, H, Sq, lens in (first, second):
        D = 128
        say("noalloc ring", B, H, Sq, lens)
        assert cp.cp_ring_attention_one_launch(cp.CP_BF16, B, H, D, Sq, lens) == cp.CP_ONE_LAUNCH_PARALLEL
        inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=3100 + Sq + H)
        q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
        offs = workloads.block_offsets(lens)
        kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
        pv = [cp.pack_v(v[:, a:a + L].contiguous()) for a, L in zip(offs, lens)]
        flags = cp.CP_RING_ANYTHING if (len(set(lens)) > 1 or 0 in lens) else 0
        out = torch.full((B, Sq, H, D), float("nan"), device="cuda")
        lse = torch.full((B, H, Sq), float("nan"), device="cuda")
        st = _noalloc(cp, q, kb, pv, out, lse, inp.workload.scale, flags)
        assert st == cp.CP_OK, cp.cp_last_error()
        out_w, lse_w = torch.empty_like(out), torch.empty_like(lse)
        n = cp.cp_ring_attention_workspace_size(B, H, Sq, D, cp.CP_RING_PACKED_V | flags)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        cp.cp_ring_attention(q, kb, pv, out_w, lse_w, scale=inp.workload.scale, flags=flags, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, out_w) and torch.equal(lse, lse_w), "noalloc differs from the workspace ring"
        if B * H * Sq <= 2 * 3 * 1000:
            o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
            assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
            assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])
        else:
            rows = np.arange(0, Sq, 97)
            o_ref, l_ref = oracle.attention(inp.q[:, rows], inp.k, inp.v, inp.workload.scale)
            assert_close("out rows", out.cpu().numpy()[:, rows], o_ref, TOL["bf16"]["o"])
            assert_close("lse rows", lse.cpu().numpy()[:, :, rows], l_ref, TOL["bf16"]["lse"])


def test_noalloc_rejects_beyond_its_scratch(cp):
    """Sizes whose flags exceed the 64 KB static array, and the separate merge, are refused on the
    host (nothing launched)."""
    lib = cp.load()
    lens = (ctypes.c_int * 2)(8, 8)
    kp = (ctypes.c_void_p * 2)(0x10000, 0x10000)
    vp = (ctypes.c_void_p * 2)(0x10000, 0x10000)
    st = lib.cp_ring_attention_noalloc(0x10000, None, kp, vp, None, lens, 2, cp.CP_BF16, 1, 64, 128, 256 * 256,
                                       0.1, cp.CP_RING_PACKED_V, 0x10000, None, 0x10000, None)
    assert st == cp.CP_ERR_WORKSPACE and "static scratch" in cp.cp_last_error()
    st = lib.cp_ring_attention_noalloc(0x10000, None, kp, vp, None, lens, 2, cp.CP_BF16, 1, 2, 128, 8, 0.1,
                                       cp.CP_RING_SEPARATE_MERGE, 0x10000, None, 0x10000, None)
    assert st == cp.CP_ERR_INVALID_ARG
