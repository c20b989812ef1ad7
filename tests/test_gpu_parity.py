"""GPU parity: the HIP path, called through the C-ABI, against the float64 oracle.

Every case draws seeded inputs from ``workloads``, runs the library on the GPU
and compares element by element with the oracle on the same values. Small
shapes are compared in full (they span several tiles and a ragged tail), and
so are the full-size workloads, in the same launch configuration the benchmark
times: every element of out and LSE against the oracle's full attention
(computed once per workload and head, cached for the session). Tolerances: float32 inputs 1e-5 (out and LSE), bfloat16
inputs 1e-2 (out) and 1e-3 (LSE); the regroup is bit-exact.
"""
import math

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


def _ring_gpu(cp, inp, flags_extra=0, q_dev=None, waves=0):
    w = inp.workload
    q = dev(inp.q, w.dtype) if q_dev is None else q_dev
    k = dev(inp.k, w.dtype)
    v = dev(inp.v, w.dtype)
    offs = workloads.block_offsets(w.block_lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, w.block_lens)]
    vb = [v[:, o:o + L] for o, L in zip(offs, w.block_lens)]
    out, lse = cp.ring_attention(q, kb, vb, scale=w.scale, separate_merge=bool(flags_extra), waves=waves)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check_rows(name, out, lse, q, k, v, scale, rows, dtype):
    """Oracle full attention for the sampled query rows only."""
    o_ref, l_ref = oracle.attention(q[:, rows], k, v, scale)
    assert_close(f"{name} out", out[:, rows], o_ref, TOL[dtype]["o"])
    assert_close(f"{name} lse", lse[:, :, rows], l_ref, TOL[dtype]["lse"])


# ------------------------------------------------------------ small shapes ---

SMALL = [
    # B, H, D, Sq, block_lens, dtype
    (1, 2, 64, 64, (64, 64, 64, 64), "f32"),
    (2, 3, 128, 100, (77, 40), "f32"),
    (2, 3, 128, 200, (300,), "bf16"),
    (1, 4, 128, 257, (128, 128, 1), "bf16"),
    (2, 2, 64, 130, (129, 200), "bf16"),
    (1, 2, 128, 1, (5, 64, 33), "bf16"),
    (1, 3, 64, 70, (3, 1), "f32"),
]


@pytest.mark.parametrize("B,H,D,Sq,lens,dtype", SMALL)
def test_ring_small_full_compare(cp, B, H, D, Sq, lens, dtype):
    say("ring small", B, H, D, Sq, lens, dtype)
    inp = workloads.make_custom(B, H, D, Sq, lens, dtype, seed=1000 + B * 7 + H + D + Sq)
    w = inp.workload
    anything = len(set(lens)) > 1
    q, k, v = dev(inp.q, dtype), dev(inp.k, dtype), dev(inp.v, dtype)
    offs = workloads.block_offsets(lens)
    kb = [k[:, o:o + L] for o, L in zip(offs, lens)]
    vb = [v[:, o:o + L] for o, L in zip(offs, lens)]
    o_ref, l_ref = oracle.ring_attention(inp.q, [inp.k_block(i) for i in range(len(lens))],
                                         [inp.v_block(i) for i in range(len(lens))], w.scale)
    for wv in (SHAPES if dtype == "bf16" else (0,)):
        for sep in (False, True):
            say(f"waves={wv} separate_merge={sep}")
            out, lse = cp.ring_attention(q, kb, vb, scale=w.scale, ring_anything=anything, separate_merge=sep,
                                         waves=wv)
            torch.cuda.synchronize()
            assert_close(f"out sep={sep}", out.cpu().numpy(), o_ref, TOL[dtype]["o"])
            assert_close(f"lse sep={sep}", lse.cpu().numpy(), l_ref, TOL[dtype]["lse"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_fwd_and_accumulate(cp, dtype):
    """One block written, a second merged in by the kernel epilogue, versus oracle partials."""
    B, H, D, Sq, lens = 2, 3, 128, 150, (96, 70)
    say("block+accumulate", dtype)
    inp = workloads.make_custom(B, H, D, Sq, lens, dtype, seed=77)
    q = dev(inp.q, dtype)
    k0, v0 = dev(inp.k_block(0), dtype), dev(inp.v_block(0), dtype)
    k1, v1 = dev(inp.k_block(1), dtype), dev(inp.v_block(1), dtype)
    s = inp.workload.scale
    o0, l0 = oracle.block_attention(inp.q, inp.k_block(0), inp.v_block(0), s)
    o, l = oracle.ring_attention(inp.q, [inp.k_block(0), inp.k_block(1)], [inp.v_block(0), inp.v_block(1)], s)
    for wv in (SHAPES if dtype == "bf16" else (0,)):
        say(f"waves={wv}")
        out = torch.empty(B, Sq, H, D, device="cuda")
        lse = torch.empty(B, H, Sq, device="cuda")
        cp.cp_attn_block_fwd(q, k0, v0, out, lse, scale=s, waves=wv)
        torch.cuda.synchronize()
        assert_close("block0 out", out.cpu().numpy(), o0, TOL[dtype]["o"])
        assert_close("block0 lse", lse.cpu().numpy(), l0, TOL[dtype]["lse"])
        cp.cp_attn_block_fwd(q, k1, v1, out, lse, scale=s, flags=cp.CP_BLOCK_ACCUMULATE, waves=wv)
        torch.cuda.synchronize()
        assert_close("merged out", out.cpu().numpy(), o, TOL[dtype]["o"])
        assert_close("merged lse", lse.cpu().numpy(), l, TOL[dtype]["lse"])


@pytest.mark.parametrize("D,strided", [(128, False), (64, False), (128, True)])
def test_lse_merge_kernel(cp, D, strided):
    say("lse_merge kernel", D, "strided" if strided else "contiguous")
    rng = np.random.default_rng(5 + D)
    B, Sq, H = 2, 37, 5
    oa, ob = rng.standard_normal((B, Sq, H, D)).astype(np.float32), rng.standard_normal((B, Sq, H, D)).astype(np.float32)
    la, lb = (rng.standard_normal((B, H, Sq)) * 4).astype(np.float32), (rng.standard_normal((B, H, Sq)) * 4).astype(np.float32)
    la[0, 1, :5] = -np.inf   # accumulator empty
    lb[1, 2, 3:9] = -np.inf  # block empty
    la[1, 4, 10:12] = -np.inf
    lb[1, 4, 10:12] = -np.inf  # both empty
    oa[1, 10:12, 4] = np.nan  # an empty side's output must not leak
    gla = torch.from_numpy(la).cuda()
    if strided:  # accumulator is every other head of a wider buffer
        wide = torch.full((B, Sq, 2 * H, D), 7.0, device="cuda")
        wide[:, :, ::2] = torch.from_numpy(oa).cuda()
        ga = wide[:, :, ::2]
    else:
        ga = torch.from_numpy(oa).cuda()
    cp.cp_lse_merge(ga, gla, torch.from_numpy(ob).cuda(), torch.from_numpy(lb).cuda())
    torch.cuda.synchronize()
    if strided:
        assert torch.all(wide[:, :, 1::2] == 7.0).item(), "write outside the accumulator view"
    o_ref, l_ref = oracle.lse_merge(np.nan_to_num(oa, nan=0.0), la, ob, lb)
    got_l = gla.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    assert_close("merge lse", got_l[fin], l_ref[fin], 1e-5)
    assert_close("merge out", ga.cpu().numpy(), o_ref, 1e-5)


# ----------------------------------------------------- degenerate / layout ---

def test_ring_anything_nan_padded_gather(cp):
    """K/V blocks as views of a padded [P, B, Lmax, H, D] gather whose pad rows are NaN."""
    B, H, D, Sq, lens = 2, 3, 128, 90, (70, 64, 33)
    say("ring anything padded NaN", lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=91)
    Lmax = max(lens)
    kpad = torch.full((len(lens), B, Lmax, H, D), float("nan"), dtype=torch.bfloat16)
    vpad = torch.full((len(lens), B, Lmax, H, D), float("nan"), dtype=torch.bfloat16)
    for i, L in enumerate(lens):
        kpad[i, :, :L] = torch.from_numpy(inp.k_block(i)).to(torch.bfloat16)
        vpad[i, :, :L] = torch.from_numpy(inp.v_block(i)).to(torch.bfloat16)
    kpad, vpad = kpad.cuda(), vpad.cuda()
    kb = [kpad[i, :, :L] for i, L in enumerate(lens)]
    vb = [vpad[i, :, :L] for i, L in enumerate(lens)]
    q = dev(inp.q, "bf16")
    out, lse = cp.ring_attention(q, kb, vb, scale=inp.workload.scale, ring_anything=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


def test_zero_length_blocks(cp):
    B, H, D, Sq = 1, 2, 128, 40
    say("zero-length blocks")
    inp = workloads.make_custom(B, H, D, Sq, (0, 50, 0, 30), "bf16", seed=12)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    kb = [k[:, 0:0], k[:, 0:50], k[:, 50:50], k[:, 50:80]]
    vb = [v[:, 0:0], v[:, 0:50], v[:, 50:50], v[:, 50:80]]
    out, lse = cp.ring_attention(q, kb, vb, scale=inp.workload.scale, ring_anything=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])
    # every block empty: attention over no keys
    out, lse = cp.ring_attention(q, [k[:, 0:0]] * 2, [v[:, 0:0]] * 2, ring_anything=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item() and torch.all(torch.isneginf(lse)).item()


@pytest.mark.parametrize("dt,packed,lens", [("bf16", True, (64,) * 18), ("bf16", False, (40, 0, 130) * 6 + (7,)),
                                             ("f32", False, (16,) * 20), ("bf16", True, (300,) * 17)])
def test_rings_beyond_sixteen_blocks(cp, dt, packed, lens):
    """Rings longer than the one-launch forms take (16 blocks) run block by block and still equal
    full attention over every block's keys."""
    B, H, D, Sq = 1, 3, 128, 200
    say(f"ring of {len(lens)} blocks, {dt}, packed {packed}")
    inp = workloads.make_custom(B, H, D, Sq, lens, dt, seed=90 + len(lens))
    q, k, v = dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt)
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, lens)]
    if packed:
        vb = [cp.pack_v(x.contiguous()) for x in vb]
    out, lse = cp.ring_attention(q, kb, vb, scale=inp.workload.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL[dt]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL[dt]["lse"])


@pytest.mark.parametrize("waves", SHAPES)
def test_strided_views(cp, waves):
    """Q, K/V and out as non-contiguous views (heads interleaved in wider buffers)."""
    B, H, D, Sq, Skv = 2, 3, 128, 97, 130
    say("strided views, waves", waves)
    inp = workloads.make_custom(B, H, D, Sq, (Skv,), "bf16", seed=33)
    qw = torch.zeros(B, Sq, 2 * H, D, dtype=torch.bfloat16, device="cuda")
    kw = torch.zeros(B, Skv, 2 * H, D, dtype=torch.bfloat16, device="cuda")
    vw = torch.zeros(B, Skv, 2 * H, D, dtype=torch.bfloat16, device="cuda")
    qw[:, :, 1::2] = dev(inp.q, "bf16")
    kw[:, :, 1::2] = dev(inp.k, "bf16")
    vw[:, :, 1::2] = dev(inp.v, "bf16")
    ow = torch.full((B, Sq, H, 2 * D), 7.0, device="cuda")
    out = ow[..., D:]
    lse = torch.empty(B, H, Sq, device="cuda")
    cp.cp_ring_attention(qw[:, :, 1::2], [kw[:, :, 1::2]], [vw[:, :, 1::2]], out, lse,
                         scale=inp.workload.scale, waves=waves)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])
    assert torch.all(ow[..., :D] == 7.0).item(), "write outside the output view"


@pytest.mark.parametrize("waves", SHAPES)
def test_wide_softmax_range(cp, waves):
    """Q scaled by 8: scores spread over a much wider range than N(0,1) gives."""
    B, H, D, Sq, lens = 1, 4, 128, 192, (256, 250)
    say("q*8 stress, waves", waves)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=8, q_scale=8.0)
    out, lse = _ring_gpu(cp, inp, waves=waves)
    o_ref, l_ref = oracle.ring_attention(inp.q, [inp.k_block(0), inp.k_block(1)],
                                         [inp.v_block(0), inp.v_block(1)], inp.workload.scale)
    assert_close("out", out, o_ref, TOL["bf16"]["o"])
    assert_close("lse", lse, l_ref, TOL["bf16"]["lse"])


# ----------------------------------------------------------------- regroup ---

@pytest.mark.parametrize("B,S_l,H,D,P,dt", [(1, 2304, 24, 128, 2, "bf16"), (2, 33, 12, 64, 3, "bf16"),
                                              (1, 50, 8, 128, 4, "f32"), (2, 7, 6, 128, 1, "bf16"),
                                              (1, 5, 6, 4, 2, "bf16")])
def test_regroup_bit_exact(cp, B, S_l, H, D, P, dt):
    say("regroup", B, S_l, H, D, P, dt)
    rng = np.random.default_rng(B * 100 + S_l + H)
    x = rng.standard_normal((B, S_l, H, D)).astype(np.float32)
    if dt == "bf16":
        x = workloads.round_to_bf16(x)
    t = dev(x, dt)
    y = torch.empty(B, P * S_l, H // P, D, dtype=t.dtype, device="cuda")
    cp.cp_ulysses_regroup(t, y, P, cp.CP_REGROUP_SEQ_TO_HEAD)
    back = torch.empty_like(t)
    cp.cp_ulysses_regroup(y, back, P, cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    want = oracle.ulysses_regroup(x, P)
    got = y.float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))
    assert torch.equal(back, t)


@pytest.mark.parametrize("n,B,S_l,H,D,P,dt", [(3, 1, 2304, 24, 128, 2, "bf16"), (2, 2, 33, 12, 64, 3, "f32"),
                                                (8, 1, 17, 6, 128, 3, "bf16"), (1, 1, 9, 4, 4, 2, "bf16")])
def test_regroup_multi_bit_exact(cp, n, B, S_l, H, D, P, dt):
    """n tensors regrouped by one launch: each bit-identical to the oracle's permutation, both ways."""
    say("regroup_multi", n, B, S_l, H, D, P, dt)
    rng = np.random.default_rng(7 * n + S_l)
    xs = [rng.standard_normal((B, S_l, H, D)).astype(np.float32) for _ in range(n)]
    if dt == "bf16":
        xs = [workloads.round_to_bf16(x) for x in xs]
    ts = [dev(x, dt) for x in xs]
    ys = [torch.empty(B, P * S_l, H // P, D, dtype=ts[0].dtype, device="cuda") for _ in range(n)]
    cp.cp_ulysses_regroup_multi(ts, ys, P, cp.CP_REGROUP_SEQ_TO_HEAD)
    backs = [torch.empty_like(t) for t in ts]
    cp.cp_ulysses_regroup_multi(ys, backs, P, cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    for x, y, t, b in zip(xs, ys, ts, backs):
        want = oracle.ulysses_regroup(x, P).astype(np.float32)
        assert np.array_equal(y.float().cpu().numpy().view(np.uint32), want.view(np.uint32))
        assert torch.equal(b, t)


# -------------------------------------------------- the five workloads ---

def _edges(n, tile=128):
    e = []
    for t in range(0, n, tile):
        e += [t, t + tile - 1]
    return e[:40] + [n - 1]


def test_workload_tiny_ring4_f32(cp):
    w = workloads.WORKLOADS[0]
    say(w.name)
    inp = workloads.make_inputs(w)
    out, lse = _ring_gpu(cp, inp)
    o_ref, l_ref = oracle.ring_attention(inp.q, [inp.k_block(i) for i in range(4)],
                                         [inp.v_block(i) for i in range(4)], w.scale)
    assert_close("out", out, o_ref, TOL["f32"]["o"])
    assert_close("lse", lse, l_ref, TOL["f32"]["lse"])


@pytest.mark.parametrize("idx", [1, 3, 4])
def test_workload_ring_full_size(cp, idx):
    """The FLUX ring-2, 32k ring-4 and ring-anything shares at full size, merged in the kernel
    epilogue and by the separate merge kernel: every element against the oracle's full attention
    over all blocks (a full ring equals full attention)."""
    w = workloads.WORKLOADS[idx]
    say(w.name, "full size, every element")
    inp = workloads.make_inputs(w)
    for sep in (False, True):
        out, lse = _ring_gpu(cp, inp, flags_extra=sep)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
        o_ref, l_ref = full_ref(w.name, inp.q, inp.k, inp.v, w.scale)
        assert_close(f"{w.name} sep={sep} out", out, o_ref, TOL[w.dtype]["o"])
        assert_close(f"{w.name} sep={sep} lse", lse, l_ref, TOL[w.dtype]["lse"])


def test_workload_ulysses2(cp):
    w = workloads.WORKLOADS[2]
    say(w.name, "regroup + attention + inverse regroup")
    inp = workloads.make_inputs(w)
    P = w.ulysses_degree
    regrouped = {}
    for name, x in (("q", inp.q), ("k", inp.k), ("v", inp.v)):
        t = dev(x, "bf16")
        y = torch.empty(w.B, P * w.S_local, w.H // P, w.D, dtype=torch.bfloat16, device="cuda")
        cp.cp_ulysses_regroup(t, y, P, cp.CP_REGROUP_SEQ_TO_HEAD)
        regrouped[name] = y
    torch.cuda.synchronize()
    ref = {n: oracle.ulysses_regroup(x, P) for n, x in (("q", inp.q), ("k", inp.k), ("v", inp.v))}
    for n in ref:
        assert np.array_equal(regrouped[n].float().cpu().numpy(), ref[n]), f"regroup of {n} not bit-exact"
    out, lse = cp.ring_attention(regrouped["q"], [regrouped["k"]], [regrouped["v"]], scale=w.scale)
    back = torch.empty(w.B, w.S_local, w.H, w.D, dtype=torch.float32, device="cuda")
    cp.cp_ulysses_regroup(out, back, P, cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    out_np, lse_np = out.cpu().numpy(), lse.cpu().numpy()
    o_ref, l_ref = full_ref(w.name, ref["q"], ref["k"], ref["v"], w.scale)
    assert_close(f"{w.name} out", out_np, o_ref, TOL[w.dtype]["o"])
    assert_close(f"{w.name} lse", lse_np, l_ref, TOL[w.dtype]["lse"])
    assert np.array_equal(back.cpu().numpy(), oracle.ulysses_regroup_inv(out_np, P))


def _usp_gpu(cp, q_local, k_shards, v_shards, P, scale, waves=0):
    """Unified attention share on the GPU: regroup Q and each K/V shard, ring, inverse regroup."""
    def regroup(x):
        t = dev(x, "bf16")
        B, S_l, H, D = t.shape
        y = torch.empty(B, P * S_l, H // P, D, dtype=torch.bfloat16, device="cuda")
        cp.cp_ulysses_regroup(t, y, P, cp.CP_REGROUP_SEQ_TO_HEAD)
        return y
    q = regroup(q_local)
    kb = [regroup(k) for k in k_shards]
    vb = [regroup(v) for v in v_shards]
    out, lse = cp.ring_attention(q, kb, vb, scale=scale, waves=waves)
    B, S_l, H, D = q_local.shape
    back = torch.empty(B, S_l, H, D, dtype=torch.float32, device="cuda")
    cp.cp_ulysses_regroup(out, back, P, cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), back.cpu().numpy(), q.float().cpu().numpy(), \
        [x.float().cpu().numpy() for x in kb], [x.float().cpu().numpy() for x in vb]


@pytest.mark.parametrize("B,S_l,H,D,P,R", [(1, 40, 6, 128, 3, 2), (2, 33, 4, 64, 2, 3), (1, 100, 8, 128, 2, 2)])
def test_usp_small_full_compare(cp, B, S_l, H, D, P, R):
    """Unified attention share (regroup, ring over R blocks, inverse regroup) vs the oracle."""
    say("usp small", B, S_l, H, D, P, R)
    rng = np.random.default_rng(900 + S_l + P + R)
    mk = lambda: workloads.round_to_bf16(rng.standard_normal((B, S_l, H, D), dtype=np.float32))  # noqa: E731
    q, ks, vs = mk(), [mk() for _ in range(R)], [mk() for _ in range(R)]
    scale = 1.0 / math.sqrt(D)
    for wv in SHAPES:
        out, lse, back, *_ = _usp_gpu(cp, q, ks, vs, P, scale, waves=wv)
        o_ref, l_ref = oracle.usp_attention(q, ks, vs, P, scale)
        assert_close(f"usp out (waves={wv})", back, o_ref, TOL["bf16"]["o"])
        assert_close(f"usp lse (waves={wv})", lse, l_ref, TOL["bf16"]["lse"])
        assert np.array_equal(back, oracle.ulysses_regroup_inv(out, P)), "inverse regroup not bit-exact"


def test_workload_usp_u2r2(cp):
    w = workloads.by_name("flux1024_usp_u2r2_bf16")
    say(w.name, "regroups + ring over 2 blocks + inverse regroup, every element")
    inp = workloads.make_inputs(w)
    P, R = w.ulysses_degree, w.ring_degree
    ks = [inp.k_shard(r) for r in range(R)]
    vs = [inp.v_shard(r) for r in range(R)]
    out, lse, back, q_h, kb, vb = _usp_gpu(cp, inp.q, ks, vs, P, w.scale)
    # the GPU's regroups are bit-exact
    assert np.array_equal(q_h, oracle.ulysses_regroup(inp.q, P))
    for r in range(R):
        assert np.array_equal(kb[r], oracle.ulysses_regroup(ks[r], P))
    k_all, v_all = np.concatenate(kb, axis=1), np.concatenate(vb, axis=1)
    o_ref, l_ref = full_ref(w.name, q_h, k_all, v_all, w.scale)
    assert_close(f"{w.name} out", out, o_ref, TOL[w.dtype]["o"])
    assert_close(f"{w.name} lse", lse, l_ref, TOL[w.dtype]["lse"])
    assert np.array_equal(back, oracle.ulysses_regroup_inv(out, P))


# -------------------------------------------------------- Ulysses Anything ---

def _bits(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a.view(np.uint32)


@pytest.mark.parametrize("B,S_r,counts,D,dt", [(1, 1121, (6, 6, 6, 6), 128, "bf16"), (2, 37, (3, 0, 2, 5), 128, "bf16"),
                                               (3, 5, (1, 2), 64, "f32"), (1, 9, (7,), 64, "bf16"),
                                               (2, 3, (1, 1, 1), 4, "bf16")])
def test_pack_heads_bit_exact(cp, B, S_r, counts, D, dt):
    say("pack_heads", B, S_r, counts, D, dt)
    H = sum(counts)
    rng = np.random.default_rng(B * 1000 + S_r + H)
    x = rng.standard_normal((B, S_r, H, D)).astype(np.float32)
    if dt == "bf16":
        x = workloads.round_to_bf16(x)
    t = dev(x, dt)
    buf = torch.empty(t.numel(), dtype=t.dtype, device="cuda")
    cp.cp_ulysses_pack_heads(t, buf, counts, cp.CP_REGROUP_SEQ_TO_HEAD)
    back = torch.full_like(t, float("nan"))
    cp.cp_ulysses_pack_heads(buf, back, counts, cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(buf.float().cpu().numpy()), _bits(oracle.ulysses_pack_heads(x, counts)))
    assert torch.equal(back, t)


@pytest.mark.parametrize("B,counts,Hg,D,dt", [(2, (1121, 1120, 1120, 1120), 6, 128, "bf16"),
                                              (3, (5, 0, 7), 2, 64, "f32"), (1, (4, 3), 3, 128, "bf16"),
                                              (2, (1, 2, 3, 4, 5), 1, 4, "bf16")])
def test_concat_seq_bit_exact(cp, B, counts, Hg, D, dt):
    say("concat_seq", B, counts, Hg, D, dt)
    S = sum(counts)
    rng = np.random.default_rng(B * 7 + S + Hg)
    buf = rng.standard_normal(B * S * Hg * D).astype(np.float32)
    if dt == "bf16":
        buf = workloads.round_to_bf16(buf)
    tb = dev(buf, dt)
    y = torch.empty((B, S, Hg, D), dtype=tb.dtype, device="cuda")
    cp.cp_ulysses_concat_seq(tb, y, counts, cp.CP_REGROUP_SEQ_TO_HEAD)
    back = torch.full_like(tb, float("nan"))
    cp.cp_ulysses_concat_seq(y, back, counts, cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    want = oracle.ulysses_concat_seq(buf, B, counts, Hg, D)
    assert np.array_equal(_bits(y.float().cpu().numpy()), _bits(want))
    assert torch.equal(back, tb)


def _random_layout_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = "f32" if rng.random() < 0.3 else "bf16"
        D = int(rng.choice([8, 64, 128]))
        B = int(rng.integers(1, 4))
        P = int(rng.integers(1, 6))
        S_l = int(rng.integers(1, 300))
        Hg = int(rng.integers(1, 5))
        counts = [int(c) for c in rng.integers(0, 6, size=P)]
        if sum(counts) == 0:
            counts[0] = 1
        out.append((i, dt, D, B, P, S_l, Hg, tuple(counts), int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("case", _random_layout_cases(24, 4242), ids=lambda c: f"r{c[0]}")
def test_random_layouts_bit_exact(cp, case):
    """Seeded random shapes for the three permutations (even regroup, uneven head packs, uneven
    sequence joins), both directions, bit for bit against the oracle's index maps."""
    i, dt, D, B, P, S_l, Hg, counts, seed = case
    say(f"layouts#{i} {dt} D{D} B{B} P{P} S_l{S_l} Hg{Hg} counts{list(counts)}")
    rng = np.random.default_rng(seed)
    # even regroup: [B, S_l, P*Hg, D] <-> [B, P*S_l, Hg, D]
    x = rng.standard_normal((B, S_l, P * Hg, D)).astype(np.float32)
    if dt == "bf16":
        x = workloads.round_to_bf16(x)
    t = dev(x, dt)
    y = torch.empty(B, P * S_l, Hg, D, dtype=t.dtype, device="cuda")
    cp.cp_ulysses_regroup(t, y, P, cp.CP_REGROUP_SEQ_TO_HEAD)
    back = torch.full_like(t, float("nan"))
    cp.cp_ulysses_regroup(y, back, P, cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y.float().cpu().numpy()), _bits(oracle.ulysses_regroup(x, P)))
    assert torch.equal(back, t)
    # uneven head packs: [B, S_l, sum(counts), D] <-> pieces of counts[g] heads
    H = sum(counts)
    x = rng.standard_normal((B, S_l, H, D)).astype(np.float32)
    if dt == "bf16":
        x = workloads.round_to_bf16(x)
    t = dev(x, dt)
    buf = torch.empty(t.numel(), dtype=t.dtype, device="cuda")
    cp.cp_ulysses_pack_heads(t, buf, list(counts), cp.CP_REGROUP_SEQ_TO_HEAD)
    back = torch.full_like(t, float("nan"))
    cp.cp_ulysses_pack_heads(buf, back, list(counts), cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(buf.float().cpu().numpy()), _bits(oracle.ulysses_pack_heads(x, list(counts))))
    assert torch.equal(back, t)
    # uneven sequence joins: pieces of counts[r] tokens <-> [B, sum(counts), Hg, D]
    S = sum(counts)
    flat = rng.standard_normal(B * S * Hg * D).astype(np.float32)
    if dt == "bf16":
        flat = workloads.round_to_bf16(flat)
    tb = dev(flat, dt)
    yy = torch.empty((B, S, Hg, D), dtype=tb.dtype, device="cuda")
    cp.cp_ulysses_concat_seq(tb, yy, list(counts), cp.CP_REGROUP_SEQ_TO_HEAD)
    back = torch.full_like(tb, float("nan"))
    cp.cp_ulysses_concat_seq(yy, back, list(counts), cp.CP_REGROUP_HEAD_TO_SEQ)
    torch.cuda.synchronize()
    want = oracle.ulysses_concat_seq(flat, B, list(counts), Hg, D)
    assert np.array_equal(_bits(yy.float().cpu().numpy()), _bits(want))
    assert torch.equal(back, tb)


def _anything_gpu(cp, q, k, v, seq, heads, scale):
    """Every rank of an uneven Ulysses group on one GPU: the packs and the attention in the
    library, the two exchanges as device copies between the ranks' buffers (test scaffolding)."""
    P = len(seq)
    B, S, H, D = q.shape
    offs = workloads.block_offsets(seq)
    piece = lambda r, g: B * seq[r] * heads[g] * D  # noqa: E731 - elements rank r sends rank g
    views = []
    for x in (q, k, v):
        send = []
        for r in range(P):
            buf = torch.empty(B * seq[r] * H * D, dtype=x.dtype, device="cuda")
            cp.cp_ulysses_pack_heads(x[:, offs[r]:offs[r] + seq[r]].contiguous(), buf, heads)
            send.append(buf)
        per_rank = []
        for g in range(P):
            recv = torch.cat([send[r][sum(piece(r, j) for j in range(g)):][:piece(r, g)] for r in range(P)])
            t = torch.empty((B, S, heads[g], D), dtype=x.dtype, device="cuda")
            cp.cp_ulysses_concat_seq(recv, t, seq, cp.CP_REGROUP_SEQ_TO_HEAD)
            per_rank.append(t)
        views.append(per_rank)
    send2 = []
    for g in range(P):
        if heads[g] == 0:
            send2.append(torch.empty(0, device="cuda"))
            continue
        o, _ = cp.ring_attention(views[0][g], [views[1][g]], [views[2][g]], scale=scale)
        buf = torch.empty(o.numel(), dtype=torch.float32, device="cuda")
        cp.cp_ulysses_concat_seq(o, buf, seq, cp.CP_REGROUP_HEAD_TO_SEQ)
        send2.append(buf)
    outs = []
    for r in range(P):
        got = [send2[g][sum(B * seq[j] * heads[g] * D for j in range(r)):][:B * seq[r] * heads[g] * D]
               for g in range(P)]
        out = torch.empty((B, seq[r], H, D), dtype=torch.float32, device="cuda")
        cp.cp_ulysses_pack_heads(torch.cat(got), out, heads, cp.CP_REGROUP_HEAD_TO_SEQ)
        outs.append(out)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


@pytest.mark.parametrize("B,seq,heads,D", [(2, (40, 39, 39), (2, 2, 1), 128), (1, (70, 69, 69, 69), (3, 2, 2, 2), 64)])
def test_ulysses_anything_all_ranks(cp, B, seq, heads, D):
    """Each rank's output after both exchanges equals full attention on its tokens."""
    say("ulysses anything all ranks", B, seq, heads, D)
    inp = workloads.make_custom(B, sum(heads), D, sum(seq), (sum(seq),), "bf16", seed=61)
    scale = 1.0 / math.sqrt(D)
    outs = _anything_gpu(cp, dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16"), seq, heads, scale)
    want = oracle.ulysses_anything_attention(
        [inp.q[:, a:a + L] for a, L in zip(workloads.block_offsets(seq), seq)],
        [inp.k[:, a:a + L] for a, L in zip(workloads.block_offsets(seq), seq)],
        [inp.v[:, a:a + L] for a, L in zip(workloads.block_offsets(seq), seq)], heads, scale)
    for r in range(len(seq)):
        assert_close(f"rank {r} out", outs[r], want[r], TOL["bf16"]["o"])


def test_workload_ulysses_anything4(cp):
    """Rank 0's share as bench.py runs it: pack of its shards, attention of head group 0 over all
    4481 tokens, unpack of the second exchange's pieces; every element against the oracle."""
    w = workloads.by_name("flux1008_ulysses_anything4_bf16")
    say(w.name)
    import bench
    prob = bench.Problem(w, False)
    prob.step()
    torch.cuda.synchronize()
    inp = prob.inp
    seq, heads = w.seq_counts, w.head_counts
    # the pack of rank 0's own shards is bit-exact
    for x, buf in zip((inp.q, inp.k, inp.v), prob.send):
        want = oracle.ulysses_pack_heads(x[:, :seq[0]], heads)
        assert np.array_equal(_bits(buf.float().cpu().numpy()), _bits(want))
    H0 = heads[0]
    o_ref, l_ref = oracle.attention(inp.q[:, :, :H0], inp.k[:, :, :H0], inp.v[:, :, :H0], w.scale)
    assert_close(f"{w.name} out", prob.out.cpu().numpy(), o_ref, TOL[w.dtype]["o"])
    assert_close(f"{w.name} lse", prob.lse.cpu().numpy(), l_ref, TOL[w.dtype]["lse"])
    # rank 0's final output: full attention on its own tokens, every head, every element
    back = prob.back.cpu().numpy()
    o_ref, _ = oracle.attention(inp.q[:, :seq[0]], inp.k, inp.v, w.scale)
    assert_close(f"{w.name} rank-0 output", back, o_ref, TOL["bf16"]["o"])


# ------------------------------------------------------ short key blocks ---

@pytest.mark.parametrize("waves", SHAPES)
def test_short_blocks_many_seeds(cp, waves):
    """Blocks of one to three 64-key tiles (full and partial), where the pipeline's prologue,
    tail steps and empty-range loads all meet, over several seeds and 8 heads."""
    B, H, D, Sq = 1, 8, 128, 300
    for Skv in (64, 100, 128, 129, 192):
        for seed in range(4):
            inp = workloads.make_custom(B, H, D, Sq, (Skv,), "bf16", seed=900 + 10 * Skv + seed)
            q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
            out = torch.empty((B, Sq, H, D), device="cuda")
            lse = torch.empty((B, H, Sq), device="cuda")
            cp.cp_attn_block_fwd(q, k, v, out, lse, scale=inp.workload.scale, waves=waves)
            torch.cuda.synchronize()
            o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, inp.workload.scale)
            say(f"waves={waves} Skv={Skv} seed={seed}")
            assert_close("out", out.cpu().numpy(), o_ref, TOL["bf16"]["o"])
            assert_close("lse", lse.cpu().numpy(), l_ref, TOL["bf16"]["lse"])


# ---------------------------------------------------- random shapes ---

def _random_cases(n, seed):
    """Seeded shapes spanning the API's combinations: dtype, head dim, batch, heads, ragged query
    counts, 1-5 blocks of equal or uneven (possibly empty) lengths, packed V, the workgroup
    shape, a separate merge and a non-default scale."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = "f32" if rng.random() < 0.25 else "bf16"
        D = int(rng.choice([64, 128, 128]))
        B, H = int(rng.choice([1, 1, 2, 3])), int(rng.integers(1, 5))
        Sq = int(rng.choice([1, 2, 31, 33, 63, 65, 127, 129, 255, 257, int(rng.integers(1, 400))]))
        nb = int(rng.integers(1, 6))
        if rng.random() < 0.5:
            lens = [int(rng.choice([1, 31, 64, 65, 128, 191, int(rng.integers(1, 400))]))] * nb
        else:
            lens = [int(rng.choice([0, 1, 17, 64, 129, int(rng.integers(0, 400))])) for _ in range(nb)]
        if sum(lens) == 0:
            lens[0] = 1
        packed = dt == "bf16" and rng.random() < 0.5
        waves = int(rng.choice([0, 0, 4, 8])) if dt == "bf16" else 0
        sep = bool(rng.random() < 0.2)
        scale = 1.0 / math.sqrt(D) if rng.random() < 0.8 else float(rng.uniform(0.02, 0.2))
        cases.append((i, dt, D, B, H, Sq, tuple(lens), packed, waves, sep, scale, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _random_cases(40, 2026), ids=lambda c: f"r{c[0]}")
def test_random_shapes(cp, case):
    """Every element of out and LSE against the oracle's full attention over the concatenated
    blocks (a full ring equals full attention), on seeded N(0,1) inputs of random shapes."""
    i, dt, D, B, H, Sq, lens, packed, waves, sep, scale, seed = case
    say(f"random#{i} {dt} B{B} H{H} D{D} Sq{Sq} lens{list(lens)} packed{int(packed)} waves{waves} "
        f"sep{int(sep)} scale{scale:.4f}")
    inp = workloads.make_custom(B, H, D, Sq, lens, dt, seed=seed)
    q, k, v = dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt)
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, lens)]
    if packed:
        vb = [cp.pack_v(x.contiguous()) for x in vb]
    out, lse = cp.ring_attention(q, kb, vb, scale=scale, separate_merge=sep, waves=waves)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp.q, inp.k, inp.v, scale)
    assert_close("out", out.cpu().numpy(), o_ref, TOL[dt]["o"])
    assert_close("lse", lse.cpu().numpy(), l_ref, TOL[dt]["lse"])


# ------------------------------------------------------- graph capture ---

def test_ring_and_backward_replay_in_a_graph(cp):
    """cp_ring_attention and cp_ring_attention_bwd only enqueue kernels on the caller's stream,
    so they can be captured into a HIP graph. Replays, with eager work between them, must give
    exactly the eager results (the kernels are deterministic)."""
    B, H, D, Sq, lens = 1, 4, 128, 300, (256, 200)
    say("graph capture ring + backward")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=81)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, lens)]
    do = torch.from_numpy(workloads.grad_out((B, Sq, H, D), 81)).cuda()
    out = torch.empty((B, Sq, H, D), device="cuda")
    lse = torch.empty((B, H, Sq), device="cuda")
    dq = torch.empty_like(out)
    dk_all = torch.empty((B, sum(lens), H, D), device="cuda")
    dv_all = torch.empty_like(dk_all)
    dk = [dk_all[:, a:a + L] for a, L in zip(offs, lens)]
    dv = [dv_all[:, a:a + L] for a, L in zip(offs, lens)]
    ws = torch.empty(cp.cp_attn_bwd_workspace_size(B, H, Sq, D), dtype=torch.uint8, device="cuda")
    flags = cp.CP_RING_ANYTHING

    def step():
        cp.cp_ring_attention(q, kb, vb, out, lse, scale=inp.workload.scale, flags=flags)
        cp.cp_ring_attention_bwd(q, kb, vb, out, lse, do, dq, dk, dv, scale=inp.workload.scale, flags=flags,
                                 workspace=ws)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (out, lse, dq, dk_all, dv_all)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (out, lse, dq, dk_all, dv_all):
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, w in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk_all, dv_all), want):
            assert torch.equal(got, w), f"replay {rep}: {name} differs from the eager run"
    say("graph replays match the eager run bit for bit")


def test_backward_on_another_stream_during_a_capture(cp):
    """While one stream captures a backward whose dQ kernels use the library's second stream, that
    stream belongs to the capture until it ends. An eager backward on another stream meanwhile must
    not join it: it runs on its own stream, completes with the eager results, and the capture still
    replays them."""
    B, H, D, Sq, lens = 1, 4, 128, 300, (256, 200)
    say("eager backward beside a capture")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=83)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, lens)]
    do = torch.from_numpy(workloads.grad_out((B, Sq, H, D), 83)).cuda()
    scale, flags = inp.workload.scale, cp.CP_RING_ANYTHING
    out = torch.empty((B, Sq, H, D), device="cuda")
    lse = torch.empty((B, H, Sq), device="cuda")
    cp.cp_ring_attention(q, kb, vb, out, lse, scale=scale, flags=flags)

    def grads():
        dq = torch.empty_like(out)
        dk_all = torch.empty((B, sum(lens), H, D), device="cuda")
        dv_all = torch.empty_like(dk_all)
        ws = torch.empty(cp.cp_attn_bwd_workspace_size(B, H, Sq, D), dtype=torch.uint8, device="cuda")
        return dq, dk_all, dv_all, ws

    def bwd(g, stream=None):
        dq, dk_all, dv_all, ws = g
        cp.cp_ring_attention_bwd(q, kb, vb, out, lse, do, dq, [dk_all[:, a:a + L] for a, L in zip(offs, lens)],
                                 [dv_all[:, a:a + L] for a, L in zip(offs, lens)], scale=scale, flags=flags,
                                 workspace=ws, stream=stream)

    ref = grads()
    bwd(ref)
    torch.cuda.synchronize()
    cap, eager = grads(), grads()
    cap_stream, other = torch.cuda.Stream(), torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap_stream):  # warm-up on the capture stream
        bwd(cap)
    torch.cuda.current_stream().wait_stream(cap_stream)
    torch.cuda.synchronize()
    for t in eager[:3]:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap_stream, capture_error_mode="relaxed"):
        bwd(cap)  # the second stream joins this capture
        bwd(eager, stream=other.cuda_stream)  # not part of it: runs now, on `other` only
    other.synchronize()
    for name, got, want in zip(("dq", "dk", "dv"), eager[:3], ref[:3]):
        assert torch.equal(got, want), f"eager backward beside the capture: {name} differs"
    for t in cap[:3]:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for name, got, want in zip(("dq", "dk", "dv"), cap[:3], ref[:3]):
        assert torch.equal(got, want), f"captured backward: {name} differs"
    say("eager backward beside the capture and the replay match the eager run")
