"""The one-launch ring's bounded merge wait, forced to give up from the host side.

In the parallel-partials form of cp_ring_attention each query tile's merges wait, with a
bounded number of polls, for the previous block's workgroup to publish its partial. A wait
that gives up must never pass for a correct result: it is counted in the workspace, the
tile's out and lse are set to NaN, and cp_ring_attention_check reports CP_ERR_ORDER.

The give-up is forced without touching the GPU's behaviour otherwise: libcpattn_ringwait_test.so
is the same sources built so that every merge, after its real wait for the previous block,
waits 16 polls for a flag value that no workgroup ever publishes (built next to the library by
context_attention_dits_amd.build). Every kernel still ends normally and the merges still run in
block order, so every tile ends as NaN; the test checks the count, the status, the NaN tiles, and
that the normal library's check on the same shapes is CP_OK.
"""
import ctypes
import os

import numpy as np
import pytest

import workloads
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    import context_attention_dits_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()
    return m


@pytest.fixture(scope="module")
def wait_lib(cp):
    from context_attention_dits_amd import _lib
    from context_attention_dits_amd.build import RING_WAIT_TEST_LIB
    path = os.path.join(os.path.dirname(_lib.DEFAULT_PATH), RING_WAIT_TEST_LIB)
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: build with python -m context_attention_dits_amd.build")
    lib = ctypes.CDLL(path)
    for name in ("cp_ring_attention", "cp_ring_attention_check", "cp_ring_attention_workspace_size",
                 "cp_ring_attention_one_launch", "cp_last_error", "cp_abi_version"):
        res, args = _lib._SIGNATURES[name]
        getattr(lib, name).restype = res
        getattr(lib, name).argtypes = args
    assert lib.cp_abi_version() == _lib.ABI_VERSION
    return lib


@pytest.mark.parametrize("B,H,Sq,lens", [(1, 4, 300, (256, 200)), (2, 3, 700, (300, 0, 257, 64))])
def test_forced_give_up_is_reported(cp, wait_lib, B, H, Sq, lens):
    D = 128
    n_blk = sum(1 for L in lens if L)
    arr = (ctypes.c_int * len(lens))(*lens)
    assert wait_lib.cp_ring_attention_one_launch(cp.CP_BF16, B, H, D, Sq, arr, len(lens), 0) == \
        cp.CP_ONE_LAUNCH_PARALLEL
    say("forced ring-wait give-up", B, H, Sq, lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=4242 + Sq)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    pv = [cp.pack_v(v[:, a:a + L].contiguous()) for a, L in zip(offs, lens)]
    flags = cp.CP_RING_PACKED_V | cp.CP_RING_ANYTHING
    nbytes = wait_lib.cp_ring_attention_workspace_size(B, H, Sq, D, flags)
    ws = torch.full((nbytes,), 0x3C, dtype=torch.uint8, device="cuda")
    out = torch.zeros((B, Sq, H, D), device="cuda")
    lse = torch.zeros((B, H, Sq), device="cuda")
    P = len(lens)
    kp = (ctypes.c_void_p * P)(*[x.data_ptr() for x in kb])
    vp = (ctypes.c_void_p * P)(*[x.data.data_ptr() for x in pv])
    kvs = (ctypes.c_int64 * 3)(*kb[0].stride()[:3])
    stream = torch.cuda.current_stream().cuda_stream
    st = wait_lib.cp_ring_attention(q.data_ptr(), None, kp, vp, kvs, arr, P, cp.CP_BF16, B, H, D, Sq,
                                    float(inp.workload.scale), flags, out.data_ptr(), None, lse.data_ptr(),
                                    ws.data_ptr(), nbytes, stream)
    assert st == cp.CP_OK, wait_lib.cp_last_error()
    st = wait_lib.cp_ring_attention_check(ws.data_ptr(), nbytes, stream)
    assert st == cp.CP_ERR_ORDER, st
    msg = wait_lib.cp_last_error().decode()
    say("check:", msg)
    n_tiles = B * H * ((Sq + 255) // 256)
    count = int(ws[:4].view(torch.int32).item())
    assert count == n_tiles * (n_blk - 1), (count, n_tiles, n_blk)
    assert f"{count} merge wait" in msg
    # every merge gave up: every tile's out and lse are NaN, none passes for a result
    assert torch.isnan(out).all().item() and torch.isnan(lse).all().item()

    # the normal library, same inputs and a workspace full of stale values: no give-up, CP_OK
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    ws.fill_(0x3C)
    cp.cp_ring_attention(q, kb, pv, out2, lse2, scale=inp.workload.scale, flags=cp.CP_RING_ANYTHING, workspace=ws)
    cp.cp_ring_attention_check(ws)
    assert int(ws[:4].view(torch.int32).item()) == 0
    assert not torch.isnan(out2).any().item()
    o_ref = np.asarray(out2.cpu().numpy())
    assert np.isfinite(o_ref).all()
