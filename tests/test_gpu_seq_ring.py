"""GPU parity of the ring run as one launch with the blocks in turn per workgroup.

With packed V on the 8-wave (ping-pong) shape, cp_ring_attention runs 2 to 16
non-empty blocks as one launch in which each workgroup takes its query tile
through the blocks in order: block 0's partial is written, each later block is
merged into (out, lse) by the same epilogue arithmetic as one launch per block.
So the result must equal the per-block launches bit for bit, and the float64
oracle within the bf16 tolerances (out 1e-2, LSE 1e-3). Small shapes force the
8-wave shape and pass no workspace (with a workspace and a forced 8-wave shape,
the other one-launch form, partials in parallel, is taken); the FLUX ring-2
share takes this path with the library's own shape choice. Cases: ragged query
and key tails, one-key and empty blocks, 5 and 16 blocks, 17 blocks (which run
one launch per block), and strided views of Q, K and the output.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, assert_close, dev, full_ref, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_dits_amd as m
    m.load()  # raises if the HIP library is missing: no fallback
    return m


def _per_block(cp, q, kb, vp, scale, waves=0):
    B, Sq, H, D = q.shape
    out = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    first = True
    for k, v in zip(kb, vp):
        if k.shape[1] == 0:
            continue
        cp.cp_attn_block_fwd(q, k, v, out, lse, scale=scale, flags=0 if first else cp.CP_BLOCK_ACCUMULATE,
                             waves=waves)
        first = False
    return out, lse


CASES = [
    # B, H, D, Sq, block_lens
    (1, 3, 128, 300, (256, 200)),
    (2, 2, 128, 513, (64, 130, 1)),
    (1, 1, 128, 100, (0, 70, 0, 31)),
    (1, 2, 128, 257, (128, 128, 128, 128, 128)),
    (1, 2, 128, 64, (64,) * 16),
    (1, 1, 128, 40, (33,) * 17),
]


@pytest.mark.parametrize("B,H,D,Sq,lens", CASES)
def test_seq_ring_equals_per_block(cp, B, H, D, Sq, lens):
    say("seq ring", B, H, D, Sq, lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=5000 + B + H + Sq + sum(lens))
    scale = inp.workload.scale
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, lens)]
    vp = [cp.pack_v(v[:, o:o + L].contiguous()) for o, L in zip(offs, lens)]
    anything = len(set(lens)) > 1 or 0 in lens
    flags = cp.CP_RING_ANYTHING if anything else 0
    # with a workspace these rings would run their partials in parallel (8 waves forced); without
    # one, as here, the blocks run in turn
    one = cp.cp_ring_attention_one_launch(cp.CP_BF16, B, H, D, Sq, lens, waves=8)
    assert one == (cp.CP_ONE_LAUNCH_PARALLEL if 2 <= sum(1 for L in lens if L) <= 16 else 0), one
    out = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    cp.cp_ring_attention(q, kb, vp, out, lse, scale=scale, flags=flags, waves=8)  # no workspace
    out_b, lse_b = _per_block(cp, q, kb, vp, scale, waves=8)
    torch.cuda.synchronize()
    assert torch.equal(out, out_b) and torch.equal(lse, lse_b), \
        (float((out - out_b).abs().max()), float((lse - lse_b).abs().max()))
    say("one launch equals the per-block launches bit for bit")
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


def test_seq_ring_flux_ring2_share(cp):
    """The FLUX 1024px ring-2 share (216 workgroups) takes this path on the library's own shape
    choice; bit-equal to the per-block launches, and every element against the oracle."""
    w = workloads.by_name("flux1024_ring2_bf16")
    say("seq ring flux ring-2 share")
    inp = workloads.make_inputs(w)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(w.block_lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, w.block_lens)]
    vp = [cp.pack_v(v[:, o:o + L].contiguous()) for o, L in zip(offs, w.block_lens)]
    assert cp.cp_attn_fwd_waves(w.B, w.H, w.D, w.Sq) == 8
    assert cp.cp_ring_attention_one_launch(cp.CP_BF16, w.B, w.H, w.D, w.Sq, w.block_lens) == \
        cp.CP_ONE_LAUNCH_IN_TURN
    out, lse = cp.ring_attention(q, kb, vp, scale=w.scale)
    out_b, lse_b = _per_block(cp, q, kb, vp, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out_b) and torch.equal(lse, lse_b)
    o_ref, l_ref = full_ref(w.name, inp.q, inp.k, inp.v, w.scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


def test_seq_ring_strided_views(cp):
    """Blocks in turn with a strided Q view, K blocks sliced from a NaN-padded all-gather
    buffer [P, B, Lmax, H, D] and an output view inside a larger NaN-filled buffer: the same
    bits as contiguous tensors, nothing written outside the output view, no NaN read."""
    B, H, D, Sq, lens = 2, 3, 128, 300, (256, 130, 64)
    say("seq ring strided views", lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=77)
    scale = inp.workload.scale
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    vp = [cp.pack_v(v[:, o:o + L].contiguous()) for o, L in zip(offs, lens)]
    kb = [k[:, o:o + L] for o, L in zip(offs, lens)]
    Lmax = max(lens)
    kpad = torch.full((len(lens), B, Lmax, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    for i, (o, L) in enumerate(zip(offs, lens)):
        kpad[i, :, :L] = k[:, o:o + L]
    kb_pad = [kpad[i, :, :L] for i, L in enumerate(lens)]
    qbig = torch.zeros((B, Sq, H + 2, D), dtype=torch.bfloat16, device="cuda")
    qbig[:, :, 1:H + 1] = q
    q_view = qbig[:, :, 1:H + 1]
    obig = torch.full((B, Sq, H + 1, D), float("nan"), dtype=torch.float32, device="cuda")
    out_view = obig[:, :, :H]
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    cp.cp_ring_attention(q_view, kb_pad, vp, out_view, lse, scale=scale, flags=cp.CP_RING_ANYTHING, waves=8)
    out_c = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda")
    lse_c = torch.empty_like(lse)
    cp.cp_ring_attention(q, kb, vp, out_c, lse_c, scale=scale, flags=cp.CP_RING_ANYTHING, waves=8)
    torch.cuda.synchronize()
    assert torch.isnan(obig[:, :, H]).all().item(), "wrote outside the output view"
    assert torch.equal(out_view, out_c) and torch.equal(lse, lse_c)
    assert not torch.isnan(out_c).any().item()


@pytest.mark.parametrize("lens", [(128, 128), (129, 128), (128, 129, 128), (128, 64, 129, 1)])
def test_seq_ring_two_tile_blocks_many_seeds(cp, lens):
    """Blocks of two 64-key tiles (128 keys) and of two tiles and one key (129), where the
    pipeline's prologue of one block meets the tail steps of the previous one: 8 heads, six
    seeds, every element against the oracle and bit-equal to one launch per block."""
    B, H, D, Sq = 1, 8, 128, 300
    scale = 1.0 / np.sqrt(D)
    for seed in range(6):
        say("seq ring two-tile blocks", lens, "seed", seed)
        inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=6100 + 37 * seed + sum(lens))
        q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
        offs = workloads.block_offsets(lens)
        kb = [k[:, o:o + L] for o, L in zip(offs, lens)]
        vp = [cp.pack_v(v[:, o:o + L].contiguous()) for o, L in zip(offs, lens)]
        flags = cp.CP_RING_ANYTHING if len(set(lens)) > 1 else 0
        out = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
        cp.cp_ring_attention(q, kb, vp, out, lse, scale=scale, flags=flags, waves=8)
        out_b, lse_b = _per_block(cp, q, kb, vp, scale, waves=8)
        torch.cuda.synchronize()
        assert torch.equal(out, out_b) and torch.equal(lse, lse_b), (seed, lens)
        o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, scale)
        assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
        assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])
