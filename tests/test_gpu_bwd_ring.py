"""GPU parity of the ring backward's two launch plans against the per-block chain.

Where one launch of the dQ or the dK/dV kernel fills its workgroup slots (at
most a quarter of its last round idle), cp_ring_attention_bwd with 2 to 16
non-empty blocks runs the dQ kernel once, each workgroup taking its query tile
through the blocks in turn with dQ summed in registers and written once, and
the dK/dV kernel once over every block's key tiles; elsewhere it runs the
per-block chain, dQ on a second stream. Both are compared here with the
chain built from the public per-block calls (cp_attn_bwd_prep, then
cp_attn_block_bwd per block, dQ added into in place): dK and dV must match
bit for bit, dQ to float32 rounding of the different order of its sum (max
abs difference <= 1e-5 of max |dQ|). The 30-head, 2048-query cases and the
FLUX share take the two launches; the small ones and 17 blocks the chain.
Parity against the float64 oracle for the same calls is in test_gpu_bwd.py.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_dits_amd as m
    m.load()  # raises if the HIP library is missing: no fallback
    return m


CASES = [
    # B, H, D, Sq, block_lens, two launches
    (1, 30, 128, 2048, (2048, 1000, 1), True),   # uneven, a one-key block
    (1, 30, 128, 2048, (0, 2048, 0, 77), True),  # empty blocks skipped
    (1, 30, 64, 2048, (2048,) * 4, True),        # head dim 64
    (1, 24, 128, 2304, (2304, 2304), True),      # the FLUX 1024px ring-2 share
    (1, 2, 128, 200, (256, 200), False),         # small grids: dQ on the second stream
    (2, 3, 64, 130, (64, 1, 129), False),
    (1, 1, 128, 40, (33,) * 17, False),          # more than 16 blocks
]


@pytest.mark.parametrize("B,H,D,Sq,lens,two", CASES)
def test_ring_bwd_equals_per_block_chain(cp, B, H, D, Sq, lens, two):
    say("ring bwd", B, H, D, Sq, lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=6000 + B + H + Sq + sum(lens))
    scale = inp.workload.scale
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, lens)]
    vb = [v[:, o:o + L] for o, L in zip(offs, lens)]
    out, lse = cp.ring_attention(q, kb, vb, scale=scale)
    do = torch.from_numpy(workloads.grad_out((B, Sq, H, D), 61)).cuda()
    dq, dk, dv = cp.ring_attention_bwd(q, kb, vb, out, lse, do, scale=scale)

    # the per-block chain
    ws = torch.empty(cp.cp_attn_bwd_workspace_size(B, H, Sq, D), dtype=torch.uint8, device="cuda")
    cp.cp_attn_bwd_prep(out, do, ws)
    dq_c = torch.empty_like(dq)
    first = True
    dk_c, dv_c = [], []
    for kk, vv in zip(kb, vb):
        dkb = torch.empty(kk.shape, dtype=torch.float32, device="cuda")
        dvb = torch.empty_like(dkb)
        if kk.shape[1] > 0:
            cp.cp_attn_block_bwd(q, kk, vv, lse, ws, dq_c, dkb, dvb, scale=scale,
                                 flags=0 if first else cp.CP_BWD_ACCUMULATE_DQ)
            first = False
        dk_c.append(dkb)
        dv_c.append(dvb)
    torch.cuda.synchronize()
    for i, L in enumerate(lens):
        if L == 0:
            continue
        assert torch.equal(dk[i], dk_c[i]) and torch.equal(dv[i], dv_c[i]), f"block {i}: dK/dV differ"
    d = float((dq - dq_c).abs().max())
    ref = float(dq_c.abs().max())
    say(f"dK, dV bit-equal; max|dQ - chain dQ| = {d:.3e} (max|dQ| {ref:.3e}), "
        f"bit-equal: {torch.equal(dq, dq_c)}")
    assert np.isfinite(d) and d <= 1e-5 * ref, (d, ref)
    if not two:  # the same chain inside the library: the same bits
        assert torch.equal(dq, dq_c)
