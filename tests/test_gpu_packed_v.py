"""GPU tests of packed V: cp_attn_pack_v's layout, and attention over packed V blocks.

The packed layout is checked element by element against the definition in the
header, rebuilt here with numpy index arithmetic. Attention over packed V feeds
the matrix cores the same operands in the same order as attention over the
unpacked V, so the two must agree bit for bit; at the benchmark's full sizes the
packed ring is also compared with the float64 oracle on every element.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import SHAPES, TOL, assert_close, dev, full_ref, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_dits_amd as m
    m.load()  # raises if the HIP library is missing: no fallback
    return m


def _packed_reference(v_bits):
    """The packed layout of uint16 V [B, Skv, H, D] as the header defines it: per (b, h), tiles
    of 64 keys; fragment f = 4 db + 2 kb + kk2 of 64 lanes x 8 elements; lane l, element e
    holds V[key][32 db + l % 32] with key = 64 t + 32 kb + 16 kk2 + 8 (e // 4) + 4 (l // 32)
    + e % 4, and 0 past Skv."""
    B, Skv, H, D = v_bits.shape
    T = -(-Skv // 64)
    padded = np.zeros((B, H, T * 64, D), dtype=np.uint16)
    padded[:, :, :Skv] = v_bits.transpose(0, 2, 1, 3)
    out = np.empty((B, H, T, D // 32, 2, 2, 64, 8), dtype=np.uint16)
    lane = np.arange(64)[:, None]
    e = np.arange(8)[None, :]
    for db in range(D // 32):
        for kb in range(2):
            for kk2 in range(2):
                key = 32 * kb + 16 * kk2 + 8 * (e // 4) + 4 * (lane // 32) + e % 4  # [64, 8]
                d = 32 * db + lane % 32 + 0 * e
                for t in range(T):
                    out[:, :, t, db, kb, kk2] = padded[:, :, 64 * t + key, d]  # [B, H, 64, 8]
    return out.reshape(-1)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("B,Skv,H,D,strided", [(1, 2304, 3, 128, False), (2, 100, 3, 128, True),
                                                (2, 129, 2, 64, False), (1, 1, 2, 128, False),
                                                (1, 64, 5, 64, True)])
def test_pack_v_layout(cp, B, Skv, H, D, strided):
    say("pack_v layout", B, Skv, H, D, "strided" if strided else "contiguous")
    inp = workloads.make_custom(B, H, D, 1, (Skv,), "bf16", seed=40 + Skv)
    v = dev(inp.v, "bf16")
    if strided:  # a view with gaps between heads and between rows
        big = torch.full((B, Skv, H + 2, D + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
        big[:, :, 1:H + 1, :D] = v
        v = big[:, :, 1:H + 1, :D]
    nbytes = cp.cp_attn_packed_v_bytes(B, H, D, Skv)
    assert nbytes == B * H * (-(-Skv // 64)) * 64 * D * 2
    buf = torch.full((nbytes // 2 + 64,), -1, dtype=torch.int16, device="cuda")  # with a guard tail
    cp.cp_attn_pack_v(v, buf)
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint16)
    want = _packed_reference(_bits(dev(inp.v, "bf16")).reshape(B, Skv, H, D))
    assert np.array_equal(got[:nbytes // 2], want), "packed layout differs from its definition"
    assert np.all(got[nbytes // 2:] == 0xFFFF), "cp_attn_pack_v wrote past its output"


def _block_pair(cp, q, k, v, pv, scale, acc_from=None, waves=0):
    """(out, lse) of one block with unpacked and with packed V; with acc_from, both start from that
    partial and merge the block in."""
    res = []
    for vv in (v, pv):
        if acc_from is None:
            out = torch.empty((q.shape[0], q.shape[1], q.shape[2], q.shape[3]), device="cuda")
            lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), device="cuda")
            flags = 0
        else:
            out, lse = acc_from[0].clone(), acc_from[1].clone()
            flags = cp.CP_BLOCK_ACCUMULATE
        cp.cp_attn_block_fwd(q, k, vv, out, lse, scale=scale, flags=flags, waves=waves)
        res.append((out, lse))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("waves", SHAPES)
@pytest.mark.parametrize("D", [128, 64])
def test_packed_matches_unpacked_bitwise(cp, waves, D):
    """Every pipeline length from one partial tile up, both workgroup shapes, overwrite and merge."""
    B, H, Sq = 1, 4, 300
    for Skv in (1, 63, 64, 100, 128, 129, 192, 257, 1000):
        for seed in range(2):
            say(f"packed vs unpacked waves={waves} D={D} Skv={Skv} seed={seed}")
            inp = workloads.make_custom(B, H, D, Sq, (Skv, 77), "bf16", seed=500 + 7 * Skv + seed)
            q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
            kb, vb = k[:, :Skv], v[:, :Skv]
            pv = cp.pack_v(vb)
            (o0, l0), (o1, l1) = _block_pair(cp, q, kb, vb, pv, inp.workload.scale, waves=waves)
            assert torch.equal(o0, o1) and torch.equal(l0, l1), "overwrite: packed differs"
            # merge the block into a partial over the other 77 keys
            base = cp.ring_attention(q, [k[:, Skv:]], [v[:, Skv:]], scale=inp.workload.scale, waves=waves)
            (o0, l0), (o1, l1) = _block_pair(cp, q, kb, vb, pv, inp.workload.scale, acc_from=base, waves=waves)
            assert torch.equal(o0, o1) and torch.equal(l0, l1), "accumulate: packed differs"
            if Skv in (129, 1000) and seed == 0:
                o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
                assert_close("out", o1.cpu().numpy(), o_ref, TOL["bf16"]["o"])
                assert_close("lse", l1.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


def _edges(n, tile=128):
    e = []
    for t in range(0, n, tile):
        e += [t, t + tile - 1]
    return e[:40] + [n - 1]


@pytest.mark.parametrize("idx", [1, 3, 4])
def test_packed_ring_workload_full_size(cp, idx):
    """The ring share over packed V blocks, as the benchmark runs it: bit-identical to the ring
    over unpacked blocks, and every element within tolerance of the oracle."""
    w = workloads.WORKLOADS[idx]
    say(w.name, "packed V, full size")
    inp = workloads.make_inputs(w)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(w.block_lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, w.block_lens)]
    vb = [v[:, o:o + L] for o, L in zip(offs, w.block_lens)]
    pvb = [cp.pack_v(x) for x in vb]
    out0, lse0 = cp.ring_attention(q, kb, vb, scale=w.scale)
    out1, lse1 = cp.ring_attention(q, kb, pvb, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1), "packed ring differs from unpacked"
    o_ref, l_ref = full_ref(w.name, inp.q, inp.k, inp.v, w.scale)
    assert_close(f"{w.name} out", out1.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close(f"{w.name} lse", lse1.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


def test_packed_rejects(cp):
    """Misuse the binding and the library catch before anything runs."""
    inp = workloads.make_custom(1, 2, 128, 10, (20,), "bf16", seed=3)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    pv = cp.pack_v(v)
    out = torch.empty((1, 10, 2, 128), device="cuda")
    lse = torch.empty((1, 2, 10), device="cuda")
    with pytest.raises(ValueError):  # flag without a packed operand
        cp.cp_attn_block_fwd(q, k, v, out, lse, flags=cp.CP_BLOCK_PACKED_V)
    with pytest.raises(ValueError):  # packed and unpacked blocks mixed
        cp.cp_ring_attention(q, [k, k], [pv, v], out, lse, flags=0)
    small = torch.empty(cp.cp_attn_packed_v_bytes(1, 2, 128, 20) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cp.CpAttnError):  # buffer too small
        cp.cp_attn_pack_v(v, small)
    with pytest.raises(TypeError):
        cp.cp_attn_pack_v(v.float(), small)
    with pytest.raises(ValueError):  # packed V has no backward
        cp.ring_attention_bwd(q, [k], [pv], out, lse, out)
    with pytest.raises(ValueError):  # a PackedV whose buffer is too small for its shape
        cp.cp_attn_block_fwd(q, k, cp.PackedV(pv.data[:-16], pv.shape), out, lse)


@pytest.mark.parametrize("B,S_l,H,D,P", [(1, 2304, 24, 128, 2), (2, 33, 12, 64, 3), (1, 100, 8, 128, 4),
                                         (1, 64, 6, 128, 1)])
def test_regroup_pack_v_is_regroup_then_pack(cp, B, S_l, H, D, P):
    """The fused Ulysses regroup + pack writes the same bytes as the two passes."""
    say("regroup_pack_v", B, S_l, H, D, P)
    inp = workloads.make_custom(B, H, D, 1, (S_l,), "bf16", seed=60 + S_l)
    v = dev(inp.v, "bf16")
    rg = torch.empty((B, P * S_l, H // P, D), dtype=torch.bfloat16, device="cuda")
    cp.cp_ulysses_regroup(v, rg, P, cp.CP_REGROUP_SEQ_TO_HEAD)
    two = cp.pack_v(rg)
    nbytes = cp.cp_attn_packed_v_bytes(B, H // P, D, P * S_l)
    buf = torch.full((nbytes + 256,), 0xAB, dtype=torch.uint8, device="cuda")
    one = cp.cp_ulysses_regroup_pack_v(v, buf, P)
    torch.cuda.synchronize()
    assert one.shape == (B, P * S_l, H // P, D)
    assert torch.equal(buf[:nbytes], two.data[:nbytes]), "fused regroup + pack differs from the two passes"
    assert bool((buf[nbytes:] == 0xAB).all()), "wrote past its output"


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_bench_step_packed_equals_unpacked(cp, idx):
    """The benchmark's step with packed V (its default where the block kernel runs its 8-wave
    shape or the ring runs as one launch) gives the same bits as the step with unpacked V: ring
    shares, the Ulysses share (regroup, then pack), and the ring-anything and USP shares, whose
    packed step is one launch of 8-wave workgroups where the unpacked one runs each block on the
    4-wave kernel (same arithmetic per row, in the same order)."""
    import bench
    w = workloads.WORKLOADS[idx]
    say(w.name, "bench step, packed vs unpacked V")
    res = []
    for packed in (False, True):
        prob = bench.Problem(w, False, packed_v=packed)
        assert prob.packed == packed
        prob.step()
        torch.cuda.synchronize()
        got = [prob.out.clone(), prob.lse.clone()]
        if hasattr(prob, "back"):
            got.append(prob.back.clone())
        res.append(got)
        del prob
    for a, b in zip(*res):
        assert torch.equal(a, b), f"{w.name}: packed step differs from unpacked"


@pytest.mark.parametrize("one_launch", [False, True])
def test_pack_and_ring_replay_in_a_graph(cp, one_launch):
    """Packing V and the ring over packed blocks only enqueue kernels (the one-launch ring's flag
    reset is a kernel too), so they can be captured in a HIP graph; replays (with eager work
    between them, and V changed in place between the second and third) must give exactly the
    eager results."""
    B, H, D, Sq, lens = 1, 4, 128, 300, (256, 200)
    say("graph capture pack_v + packed ring", "one launch" if one_launch else "one launch per block")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=82)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, lens)]
    bufs = [torch.empty(cp.cp_attn_packed_v_bytes(B, H, D, L), dtype=torch.uint8, device="cuda") for L in lens]
    out = torch.empty((B, Sq, H, D), device="cuda")
    lse = torch.empty((B, H, Sq), device="cuda")
    ws = None
    if one_launch:
        n = cp.cp_ring_attention_workspace_size(B, H, Sq, D, cp.CP_RING_PACKED_V)
        assert n > 0
        ws = torch.full((n,), 0x55, dtype=torch.uint8, device="cuda")

    def step():
        pvb = [cp.cp_attn_pack_v(x, buf) for x, buf in zip(vb, bufs)]
        cp.cp_ring_attention(q, kb, pvb, out, lse, scale=inp.workload.scale, flags=cp.CP_RING_ANYTHING,
                             workspace=ws)

    def eager():
        o, l_ = cp.ring_attention(q, kb, vb, scale=inp.workload.scale)
        torch.cuda.synchronize()
        return o, l_

    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        if rep == 2:
            v.mul_(-0.5)  # new V values: the captured pack must pick them up
        want_o, want_l = eager()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        for buf in bufs:
            buf.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l), f"replay {rep} differs from eager"
    say("graph replays of pack + packed ring match the eager unpacked ring bit for bit")


def _ring_pair(cp, q, kb, vb, scale, flags=0, waves=0):
    """(out, lse) of the packed ring as one launch (with a workspace) and as one launch per block; the
    one-launch form's merge order is checked (cp_ring_attention_check) after it."""
    B, Sq, H, D = q.shape
    pvb = [cp.pack_v(x) for x in vb]
    lens = [x.shape[1] for x in kb]
    n = cp.cp_ring_attention_workspace_size(B, H, Sq, D, cp.CP_RING_PACKED_V | flags)
    ws = torch.full((max(n, 1),), 0x7F, dtype=torch.uint8, device="cuda")  # stale flag values
    res = []
    for w in (ws, None):
        out = torch.full((B, Sq, H, D), float("nan"), device="cuda")
        lse = torch.full((B, H, Sq), float("nan"), device="cuda")
        cp.cp_ring_attention(q, kb, pvb, out, lse, scale=scale, flags=flags, workspace=w, waves=waves)
        if w is not None and n > 0 and any(x > 0 for x in lens):
            cp.cp_ring_attention_check(w)  # any form: a call with this workspace leaves its count defined
        res.append((out, lse))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("waves,B,H,Sq,lens", [(8, 1, 4, 300, (256, 200)), (8, 2, 3, 1000, (1536, 1536, 1535)),
                                               (8, 1, 24, 2304, (2304, 2304)), (8, 1, 2, 513, (100, 0, 77, 64)),
                                               (8, 1, 2, 260, (64,) * 4), (0, 1, 12, 2304, (2304, 2304)),
                                               (0, 2, 24, 1536, (1536, 1536, 1535)), (0, 1, 24, 2304, (2304, 2304))])
def test_ring_one_launch_matches_per_block(cp, waves, B, H, Sq, lens):
    """A ring run as one launch gives the same bits as one launch per block, twice on one
    workspace. Rings of 2 or 3 non-empty blocks run every block's partial in parallel (merges
    ordered per query tile through flags) where the 8-wave kernel is forced or the per-block
    launches would run on 4 waves (the USP and ring-anything shares); on the 8-wave shape
    otherwise (the FLUX ring-2 share; 4 or more blocks when forced) each workgroup takes the
    blocks in turn; so every case here with 2 to 16 non-empty blocks is one launch."""
    D = 128
    n_nonempty = sum(1 for L in lens if L > 0)
    one = cp.cp_ring_attention_one_launch(cp.CP_BF16, B, H, D, Sq, lens, waves=waves)
    assert (one != 0) == (2 <= n_nonempty <= 16), one
    parallel = waves == 8 or cp.cp_attn_fwd_waves(B, H, D, Sq) == 4
    assert one == 0 or one == (cp.CP_ONE_LAUNCH_PARALLEL if parallel else cp.CP_ONE_LAUNCH_IN_TURN), one
    say("one-launch ring", "waves", waves, B, H, Sq, lens, {0: "per block", 1: "in turn", 2: "parallel"}[one])
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=700 + len(lens) + Sq)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, lens)]
    flags = cp.CP_RING_ANYTHING if (len(set(lens)) > 1 or 0 in lens) else 0
    for rep in range(2):
        (o1, l1), (o0, l0) = _ring_pair(cp, q, kb, vb, inp.workload.scale, flags, waves=waves)
        assert torch.equal(o1, o0) and torch.equal(l1, l0), f"one launch differs from per-block launches ({rep})"
    if B * H * Sq <= 2 * 3 * 1000:
        o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
        assert_close("out", o1.cpu().numpy(), o_ref, TOL["bf16"]["o"])
        assert_close("lse", l1.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


@pytest.mark.parametrize("B,H,Sq,L", [(1, 6, 4481, 4481), (1, 2, 300, 129), (2, 3, 260, 200), (1, 4, 100, 128)])
def test_ring_one_launch_splits_a_single_block(cp, B, H, Sq, L):
    """A single block on a grid the block kernel would run on 4 waves is split at a 64-key tile
    boundary into two halves computed in parallel and merged by their LSE (the ring's own method,
    one level finer); the result matches the oracle, and one launch per block, to tolerance."""
    D = 128
    assert cp.cp_ring_attention_one_launch(cp.CP_BF16, B, H, D, Sq, [L])
    say("one-launch split", B, H, Sq, L)
    inp = workloads.make_custom(B, H, D, Sq, (L,), "bf16", seed=900 + L + Sq)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    for rep in range(2):
        (o1, l1), (o0, l0) = _ring_pair(cp, q, [k], [v], inp.workload.scale)
        assert_close("split vs per-block out", o1.cpu().numpy(), o0.cpu().numpy(), TOL["bf16"]["o"])
        assert_close("split vs per-block lse", l1.cpu().numpy(), l0.cpu().numpy(), TOL["bf16"]["lse"])
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
    assert_close("out", o1.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close("lse", l1.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


def test_ring_output_beyond_2gib_offsets(cp):
    """The parallel-partials ring addresses out and lse with 32-bit buffer offsets, so a call whose
    output view spans 2 GiB or more must take another launch form. Here batch entry 1 of out lies
    2.25 GiB past batch entry 0 (a view into a 4.5 GiB buffer): the result equals, bit for bit, the
    same call on a compact out (which runs as one parallel-partials launch), and the oracle."""
    B, H, D, Sq, lens = 2, 3, 128, 300, (256, 200)
    assert cp.cp_ring_attention_one_launch(cp.CP_BF16, B, H, D, Sq, lens) == cp.CP_ONE_LAUNCH_PARALLEL
    say("ring with out spanning more than 2 GiB")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=77)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    pv = [cp.pack_v(v[:, a:a + L].contiguous()) for a, L in zip(offs, lens)]
    flags = cp.CP_RING_ANYTHING
    n = cp.cp_ring_attention_workspace_size(B, H, Sq, D, cp.CP_RING_PACKED_V | flags)
    ws = torch.zeros((n,), dtype=torch.uint8, device="cuda")
    out_c = torch.full((B, Sq, H, D), float("nan"), device="cuda")
    lse_c = torch.full((B, H, Sq), float("nan"), device="cuda")
    cp.cp_ring_attention(q, kb, pv, out_c, lse_c, scale=inp.workload.scale, flags=flags, workspace=ws)
    rows = (9 << 30) // (4 * H * D * 4)  # rows per batch entry: 2.25 GiB
    big = torch.empty((B, rows, H, D), device="cuda")
    out_b = big[:, :Sq]
    out_b.fill_(float("nan"))
    lse_b = torch.full((B, H, Sq), float("nan"), device="cuda")
    cp.cp_ring_attention(q, kb, pv, out_b, lse_b, scale=inp.workload.scale, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_b, out_c) and torch.equal(lse_b, lse_c)
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
    assert_close("out", out_b.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close("lse", lse_b.cpu().numpy(), l_ref, TOL["bf16"]["lse"])
    del big, out_b
