"""GPU parity of the float32 ring run as one launch (2 to 4 non-empty blocks).

cp_ring_attention with CP_F32 computes every block's partial in one launch and
merges them in block order inside the workgroup. Each case is compared with the
float64 oracle (max abs error <= 1e-5 on out and LSE) and with the per-block
launches (cp_attn_block_fwd, the first non-empty block written, the others
merged by the accumulating epilogue), which the one launch must match to
float32 rounding. Shapes cover head dims 64 and 128 (64- and 32-key tiles),
ragged query and key tails, blocks of one key, empty blocks, blocks of very
different lengths (groups idle through the longest block's barriers) and five
blocks, which run one launch per block.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, assert_close, dev, say

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
    # B, H, D, Sq, block_lens
    (1, 2, 64, 64, (64, 64, 64, 64)),      # the tiny ring-4 workload's shape
    (2, 3, 64, 50, (130, 1, 64)),          # ragged rows, a one-key block, several tiles
    (1, 2, 128, 33, (40, 100)),            # D = 128: 32-key tiles with a tail
    (1, 1, 128, 17, (0, 70, 0, 31, 5)),    # empty blocks skipped: three partials
    (2, 2, 64, 16, (200, 199, 198, 197)),  # four uneven multi-tile blocks
    (1, 3, 64, 40, (300, 3)),              # one group idles through most barriers
    (1, 2, 64, 20, (10, 10, 10, 10, 10)),  # five blocks: one launch per block
]


@pytest.mark.parametrize("B,H,D,Sq,lens", CASES)
def test_f32_ring_one_launch(cp, B, H, D, Sq, lens):
    say("f32 ring one launch", B, H, D, Sq, lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "f32", seed=4000 + B + H + D + Sq + sum(lens))
    scale = inp.workload.scale
    q, k, v = dev(inp.q, "f32"), dev(inp.k, "f32"), dev(inp.v, "f32")
    offs = workloads.block_offsets(lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, lens)]
    vb = [v[:, o:o + L] for o, L in zip(offs, lens)]
    out, lse = cp.ring_attention(q, kb, vb, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL["f32"]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL["f32"]["lse"])

    # the same ring as one launch per block
    out_b = torch.empty_like(out)
    lse_b = torch.empty_like(lse)
    first = True
    for kk, vv in zip(kb, vb):
        if kk.shape[1] == 0:
            continue
        cp.cp_attn_block_fwd(q, kk, vv, out_b, lse_b, scale=scale,
                             flags=0 if first else cp.CP_BLOCK_ACCUMULATE)
        first = False
    torch.cuda.synchronize()
    d_o = float((out - out_b).abs().max())
    d_l = float((lse - lse_b).abs().max())
    say(f"one launch vs per-block launches: max|d out|={d_o:.3e} max|d lse|={d_l:.3e}, "
        f"bit-identical: {torch.equal(out, out_b) and torch.equal(lse, lse_b)}")
    assert d_o <= 1e-6 and d_l <= 1e-6, (d_o, d_l)


def test_f32_ring_repeat_and_strided_out(cp):
    """Two calls in a row into a strided output view give the same values as a contiguous one."""
    B, H, D, Sq, lens = 1, 2, 64, 48, (64, 30, 64)
    say("f32 ring strided out", lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "f32", seed=77)
    scale = inp.workload.scale
    q, k, v = dev(inp.q, "f32"), dev(inp.k, "f32"), dev(inp.v, "f32")
    offs = workloads.block_offsets(lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, lens)]
    vb = [v[:, o:o + L] for o, L in zip(offs, lens)]
    big = torch.full((B, Sq, H + 1, D), float("nan"), dtype=torch.float32, device="cuda")
    out = big[:, :, 1:]  # a strided view: head stride D, row stride (H + 1) * D
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    for _ in range(2):
        cp.cp_ring_attention(q, kb, vb, out, lse, scale=scale, flags=cp.CP_RING_ANYTHING)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL["f32"]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL["f32"]["lse"])
    assert torch.isnan(big[:, :, 0]).all().item(), "wrote outside the output view"
    o2, l2 = cp.ring_attention(q, kb, vb, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o2, out.contiguous()) and torch.equal(l2, lse)
