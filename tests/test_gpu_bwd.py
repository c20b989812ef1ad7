"""GPU parity of the ring-share backward (bfloat16 Q/K/V, float32 gradients)
against the float64 oracle, through the C-ABI.

The forward results the backward consumes (O and the merged LSE) come from
the oracle, cast to float32, so the comparison isolates the backward kernels.

Tolerance, derived from the kernels' arithmetic (no tolerance for gradients
is fixed elsewhere). With u = 2^-8 the unit roundoff of bfloat16 (8
significant bits) and, per (b, h), P = exp(scale QK^T - LSE), dP = dO V^T,
dS = P (dP - D):
  * dO is rounded to bfloat16 and both dP = dO V^T and D = rowsum(dO O)
    take the rounded dO, so dP_ij - D_i carries at most u (A_ij + a_i) with
    A = |dO| |V|^T and a_i = sum_d |dO_id| |O_id|; dS_ij is rounded to
    bfloat16 (u |dS_ij|). Its error is at most u W_ij with
    W = |dS| + P (A + a).
  * dQ = scale dS K and dK = scale dS^T Q take K and Q exactly (they are
    bfloat16 inputs): |err dQ| <= scale (u + n 2^-24) W |K|, |err dK| <=
    scale (u + n 2^-24) W^T |Q|, the n 2^-24 term bounding float32
    accumulation over n terms.
  * dV = P^T dO with P and dO both rounded: |err dV| <= (2u + n 2^-24) P^T |dO|.
The float32 exponent, the row statistics and the float32 LSE and O inputs
add relative errors near 1e-6 to P and D, far below u; a factor 1.25 on the
bound and an absolute floor of 1e-6 max|ref| cover them. The bound is a
worst case elementwise; the tests also report the typical error, which is
far smaller. It still fails a plausible mistake: one key left out of a
100-query, 120-key case (a CPU emulation of the kernels' rounding sits at
0.6 of the bound at most, the key left out at 5 times it).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U = 2.0 ** -8
EPS32 = 2.0 ** -24


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_dits_amd as m
    m.load()  # raises if the HIP library is missing: no fallback
    return m


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _bounds(q, k_blocks, v_blocks, o, lse, do, scale):
    """Elementwise error bounds (see the module docstring) for dq and each block's dk, dv."""
    B, Sq, H, D = q.shape
    n_total = sum(kb.shape[1] for kb in k_blocks)
    bq = np.zeros(q.shape)
    bks = [np.zeros(kb.shape) for kb in k_blocks]
    bvs = [np.zeros(kb.shape) for kb in k_blocks]
    for b in range(B):
        for h in range(H):
            qh = q[b, :, h].astype(np.float64)
            doh = do[b, :, h].astype(np.float64)
            dlt = np.sum(doh * o[b, :, h], axis=1)
            dlt_abs = np.sum(np.abs(doh) * np.abs(o[b, :, h]), axis=1)
            for i, (kb, vb) in enumerate(zip(k_blocks, v_blocks)):
                if kb.shape[1] == 0:
                    continue
                kh = kb[b, :, h].astype(np.float64)
                vh = vb[b, :, h].astype(np.float64)
                p = np.exp(scale * (qh @ kh.T) - lse[b, h][:, None])
                ds = p * (doh @ vh.T - dlt[:, None])
                w = np.abs(ds) + p * (np.abs(doh) @ np.abs(vh).T + dlt_abs[:, None])
                bq[b, :, h] += scale * (U + n_total * EPS32) * (w @ np.abs(kh))
                bks[i][b, :, h] = scale * (U + Sq * EPS32) * (w.T @ np.abs(qh))
                bvs[i][b, :, h] = (2 * U + Sq * EPS32) * (p.T @ np.abs(doh))
    return bq, bks, bvs


def _compare(name, got, want, bound):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    err = np.abs(got - want)
    if err.size == 0:
        return
    floor = 1e-6 * max(float(np.abs(want).max()), 1e-30)
    tol = 1.25 * bound + floor
    ratio = err / tol
    i = np.unravel_index(int(np.argmax(ratio)), err.shape)
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say(f"{name}: max|err|={err.max():.3e}, worst err/bound={ratio[i]:.3f} at {tuple(int(x) for x in i)} "
        f"(got {got[i]:.6g}, want {want[i]:.6g}), rel Frobenius err {rel:.2e}")
    assert ratio[i] <= 1.0, f"{name}: error {err[i]:.3e} above its bound {tol[i]:.3e} at {i}"


def _run(cp, inp, do, o, lse, scale, q_view=None):
    """cp.ring_attention_bwd on the GPU; returns numpy dq, [dk], [dv]."""
    w = inp.workload
    q = _bf16(inp.q) if q_view is None else q_view
    k = _bf16(inp.k)
    v = _bf16(inp.v)
    offs = workloads.block_offsets(w.block_lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, w.block_lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, w.block_lens)]
    dq, dk, dv = cp.ring_attention_bwd(q, kb, vb, _f32(o), _f32(lse), _f32(do), scale=scale)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), [t.cpu().numpy() for t in dk], [t.cpu().numpy() for t in dv]


def _check_all(name, inp, do, scale, got, heads=None):
    """Oracle forward + backward (optionally on a subset of heads) against the GPU gradients."""
    w = inp.workload
    hs = slice(None) if heads is None else heads
    q = inp.q[:, :, hs]
    kbs = [inp.k_block(i)[:, :, hs] for i in range(len(w.block_lens))]
    vbs = [inp.v_block(i)[:, :, hs] for i in range(len(w.block_lens))]
    dob = do[:, :, hs]
    o, lse = oracle.ring_attention(q, kbs, vbs, scale)
    o32, lse32 = o.astype(np.float32).astype(np.float64), lse.astype(np.float32).astype(np.float64)
    dq_ref, dk_ref, dv_ref = oracle.ring_attention_bwd(q, kbs, vbs, o32, lse32, dob, scale)
    bq, bks, bvs = _bounds(q, kbs, vbs, o32, lse32, dob, scale)
    dq, dk, dv = got
    _compare(f"{name} dq", dq[:, :, hs], dq_ref, bq)
    for i in range(len(kbs)):
        _compare(f"{name} dk[{i}]", dk[i][:, :, hs], dk_ref[i], bks[i])
        _compare(f"{name} dv[{i}]", dv[i][:, :, hs], dv_ref[i], bvs[i])


def _fwd_oracle(inp, scale):
    w = inp.workload
    kbs = [inp.k_block(i) for i in range(len(w.block_lens))]
    vbs = [inp.v_block(i) for i in range(len(w.block_lens))]
    return oracle.ring_attention(inp.q, kbs, vbs, scale)


SMALL = [
    # B, H, D, Sq, block_lens, seed
    (1, 2, 128, 100, (70, 50), 11),        # ragged query and key tiles
    (2, 3, 64, 33, (33, 0, 17), 12),       # ring anything with an empty block, D = 64
    (1, 4, 128, 300, (256, 256), 13),      # several tiles each way
    (1, 2, 64, 257, (129,), 14),           # one block, tails of one row
    (2, 2, 128, 64, (64, 64, 64, 64), 15),  # four equal blocks
]


@pytest.mark.parametrize("B,H,D,Sq,lens,seed", SMALL)
def test_bwd_small_full_compare(cp, B, H, D, Sq, lens, seed):
    say(f"bwd small B={B} H={H} D={D} Sq={Sq} blocks={lens}")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=seed)
    scale = 1.0 / np.sqrt(D)
    do = workloads.grad_out((B, Sq, H, D), seed)
    o, lse = _fwd_oracle(inp, scale)
    got = _run(cp, inp, do, o, lse, scale)
    _check_all(f"bwd B{B} H{H} D{D} Sq{Sq}", inp, do, scale, got)


def _random_bwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        Sq = int(rng.choice([1, 31, 33, 64, 97, 129, int(rng.integers(1, 320))]))
        nb = int(rng.integers(1, 5))
        lens = [int(rng.choice([0, 1, 32, 33, 100, int(rng.integers(0, 320))])) for _ in range(nb)]
        if sum(lens) == 0:
            lens[0] = 7
        q_scale = float(rng.choice([1.0, 1.0, 3.0]))
        cases.append((i, B, H, D, Sq, tuple(lens), q_scale, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _random_bwd_cases(12, 777), ids=lambda c: f"r{c[0]}")
def test_bwd_random_shapes(cp, case):
    """Seeded random shapes (ragged, empty and one-key blocks, D = 64 and 128, some with Q scaled
    by 3) against the oracle's gradients, every element within the derived bound."""
    i, B, H, D, Sq, lens, q_scale, seed = case
    say(f"bwd random#{i} B={B} H={H} D={D} Sq={Sq} blocks={list(lens)} q_scale={q_scale}")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=seed % 100000, q_scale=q_scale)
    scale = 1.0 / np.sqrt(D)
    do = workloads.grad_out((B, Sq, H, D), seed % 100000)
    o, lse = _fwd_oracle(inp, scale)
    got = _run(cp, inp, do, o, lse, scale)
    _check_all(f"bwd random#{i}", inp, do, scale, got)


def test_bwd_peaked_softmax(cp):
    """Q scaled by 4: rows dominated by a few keys (P near 0 and 1)."""
    B, H, D, Sq, lens = 1, 2, 128, 160, (96, 96)
    say("bwd peaked softmax q_scale=4")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=21, q_scale=4.0)
    scale = 1.0 / np.sqrt(D)
    do = workloads.grad_out((B, Sq, H, D), 21)
    o, lse = _fwd_oracle(inp, scale)
    got = _run(cp, inp, do, o, lse, scale)
    _check_all("bwd peaked", inp, do, scale, got)


@pytest.mark.parametrize("D,Sq,lens", [(128, 300, (1,)), (64, 489, (0, 1)), (128, 97, (1, 0, 0))])
def test_bwd_single_key_gradients_vanish(cp, D, Sq, lens):
    """One key in the whole ring: every row's softmax is the constant 1, so O = v and the exact
    dQ and dK are zero (dS = P (dP - D) = dO.v - dO.v). The kernels take dP and D from the same
    bfloat16 dO, so what remains is float32 accumulation order, bounded per row by
    2 D 2^-24 sum_d |dO_id| |v_d| for dS_i; a D computed from a differently rounded dO would
    leave u |dO_i| |v| (128 times more at D = 128)."""
    B, H = 1, 3
    say("bwd single key", D, Sq, lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=41 + D + Sq)
    scale = 1.0 / np.sqrt(D)
    do = workloads.grad_out((B, Sq, H, D), 41)
    o, lse = _fwd_oracle(inp, scale)
    o32, lse32 = o.astype(np.float32), lse.astype(np.float32)
    dq, dks, dvs = _run(cp, inp, do, o32, lse32, scale)
    i = [j for j, L in enumerate(lens) if L == 1][0]
    k1 = inp.k_block(i)[:, 0].astype(np.float64)  # [B, H, D]
    v1 = inp.v_block(i)[:, 0].astype(np.float64)
    dob = do.astype(np.float64)
    b_ds = 2 * D * EPS32 * np.einsum("bshd,bhd->bsh", np.abs(dob), np.abs(v1))  # [B, Sq, H]
    bound_dq = 1.25 * scale * (1 + U) * b_ds[..., None] * np.abs(k1)[:, None] + 1e-7
    bound_dk = 1.25 * scale * (1 + U) * np.einsum("bsh,bshd->bhd", b_ds, np.abs(inp.q.astype(np.float64))) + 1e-7
    say(f"max|dq|={np.abs(dq).max():.3e} (bound {bound_dq.max():.3e}), max|dk|={np.abs(dks[i]).max():.3e} "
        f"(bound {bound_dk.max():.3e})")
    assert np.all(np.abs(dq) <= bound_dq), "dQ of a one-key softmax is not zero to float32 rounding"
    assert np.all(np.abs(dks[i][:, 0]) <= bound_dk), "dK of a one-key softmax is not zero to float32 rounding"
    # dV of the one key is sum_i dO_i (P = 1); the other, empty blocks have no rows
    dv_ref = dob.sum(axis=1)
    _compare("single key dv", dvs[i][:, 0], dv_ref, (2 * U + Sq * EPS32) * np.abs(dob).sum(axis=1))


def test_bwd_block_api_and_strided_views(cp):
    """cp_attn_bwd_prep + cp_attn_block_bwd block by block (dq overwritten, then accumulated), with
    q, out, dout, dq and dk/dv as strided views of larger buffers."""
    B, H, D, Sq, lens = 2, 3, 128, 130, (64, 97)
    say("bwd block API strided")
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=31)
    scale = 0.07
    do = workloads.grad_out((B, Sq, H, D), 31)
    o, lse = _fwd_oracle(inp, scale)
    # q inside a [B, Sq, H + 1, D] buffer; out, dout and dq inside [B, Sq + 3, H, D + 8] buffers
    qbig = torch.zeros((B, Sq, H + 1, D), dtype=torch.bfloat16, device="cuda")
    qbig[:, :, :H] = _bf16(inp.q)
    q = qbig[:, :, :H]

    def padded(x):
        t = torch.full((B, Sq + 3, H, D + 8), float("nan"), dtype=torch.float32, device="cuda")
        if x is not None:
            t[:, :Sq, :, :D] = _f32(x)
        return t[:, :Sq, :, :D]

    out_v, dout_v, dq_v = padded(o), padded(do), padded(None)
    lse_t = _f32(lse)
    ws = torch.empty(cp.cp_attn_bwd_workspace_size(B, H, Sq, D), dtype=torch.uint8, device="cuda")
    cp.cp_attn_bwd_prep(out_v, dout_v, ws)
    k, v = _bf16(inp.k), _bf16(inp.v)
    offs = workloads.block_offsets(lens)
    dks, dvs = [], []
    for i, (a, L) in enumerate(zip(offs, lens)):
        dkbig = torch.full((B, L, H, D + 4), float("nan"), dtype=torch.float32, device="cuda")
        dvbig = torch.full((B, L, H, D + 4), float("nan"), dtype=torch.float32, device="cuda")
        dk, dv = dkbig[..., :D], dvbig[..., :D]
        cp.cp_attn_block_bwd(q, k[:, a:a + L], v[:, a:a + L], lse_t, ws, dq_v, dk, dv, scale=scale,
                             flags=cp.CP_BWD_ACCUMULATE_DQ if i else 0)
        dks.append(dk)
        dvs.append(dv)
    torch.cuda.synchronize()
    got = (dq_v.cpu().numpy(), [t.cpu().numpy() for t in dks], [t.cpu().numpy() for t in dvs])
    _check_all("bwd block API", inp, do, scale, got)


def test_bwd_empty_cases(cp):
    """No keys: dq = 0 (and left alone when accumulating). No queries: dk = dv = 0."""
    B, H, D, Sq = 1, 2, 128, 40
    say("bwd empty cases")
    q = torch.randn((B, Sq, H, D), device="cuda").to(torch.bfloat16)
    o = torch.zeros((B, Sq, H, D), device="cuda")
    do = torch.randn((B, Sq, H, D), device="cuda")
    lse = torch.zeros((B, H, Sq), device="cuda")
    kv0 = torch.empty((B, 0, H, D), dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = cp.ring_attention_bwd(q, [kv0, kv0], [kv0, kv0], o, lse, do, ring_anything=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq).item() == 0 and all(t.numel() == 0 for t in dk + dv)
    # accumulate over an empty block leaves dq as it was
    ws = torch.empty(cp.cp_attn_bwd_workspace_size(B, H, Sq, D), dtype=torch.uint8, device="cuda")
    cp.cp_attn_bwd_prep(o, do, ws)
    dq1 = torch.full((B, Sq, H, D), 3.0, device="cuda")
    e0 = torch.empty((B, 0, H, D), device="cuda")
    cp.cp_attn_block_bwd(q, kv0, kv0, lse, ws, dq1, e0, e0, flags=cp.CP_BWD_ACCUMULATE_DQ)
    cp.cp_attn_block_bwd(q, kv0, kv0, lse, ws, dq, e0, e0)
    torch.cuda.synchronize()
    assert torch.all(dq1 == 3.0).item() and torch.count_nonzero(dq).item() == 0
    # no queries: dk = dv = 0 over 70 keys (outputs pre-filled with NaN must be overwritten)
    q0 = torch.empty((B, 0, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((B, 70, H, D), device="cuda").to(torch.bfloat16)
    dk = torch.full((B, 70, H, D), float("nan"), device="cuda")
    dv = torch.full((B, 70, H, D), float("nan"), device="cuda")
    cp.cp_attn_block_bwd(q0, k, k, torch.empty((B, H, 0), device="cuda"), None,
                         torch.empty((B, 0, H, D), device="cuda"), dk, dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


@pytest.mark.parametrize("idx,heads", [(1, [0, 23]), (3, [0, 13]), (4, [5])])
def test_bwd_workload_full_size_sampled(cp, idx, heads):
    """Full-size workloads (one launch of the whole problem, as the benchmark times it), compared on
    sampled heads. Heads are independent, so the oracle runs on those heads' slices only: their o and
    lse inputs come from the oracle's forward, every other head gets o = 0 and lse = 0 (finite inputs
    whose gradients are not looked at)."""
    w = workloads.WORKLOADS[idx]
    say(f"bwd workload {w.name} heads {heads}")
    inp = workloads.make_inputs(w)
    scale = w.scale
    do = workloads.grad_out((w.B, w.Sq, w.H, w.D), w.seed)
    o = np.zeros((w.B, w.Sq, w.H, w.D))
    lse = np.zeros((w.B, w.H, w.Sq))
    kbs = [inp.k_block(i) for i in range(len(w.block_lens))]
    vbs = [inp.v_block(i) for i in range(len(w.block_lens))]
    for h in heads:
        o_h, l_h = oracle.ring_attention(inp.q[:, :, h:h + 1], [kb[:, :, h:h + 1] for kb in kbs],
                                         [vb[:, :, h:h + 1] for vb in vbs], scale)
        o[:, :, h:h + 1] = o_h
        lse[:, h:h + 1] = l_h
    got = _run(cp, inp, do, o, lse, scale)
    _check_all(f"bwd {w.name}", inp, do, scale, got, heads=heads)


def test_bwd_padded_gather_with_nan_pads(cp):
    """K/V blocks as slices of a padded all-gather [P, B, Lmax, H, D] whose pad rows hold NaN: the
    backward never reads past a block's length."""
    B, H, D, Sq, lens = 2, 2, 128, 90, (64, 63, 50)
    say("bwd padded gather NaN", lens)
    inp = workloads.make_custom(B, H, D, Sq, lens, "bf16", seed=41)
    scale = 1.0 / np.sqrt(D)
    do = workloads.grad_out((B, Sq, H, D), 41)
    o, lse = _fwd_oracle(inp, scale)
    Lmax = max(lens)
    kpad = torch.full((len(lens), B, Lmax, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vpad = torch.full_like(kpad, float("nan"))
    for i, L in enumerate(lens):
        kpad[i, :, :L] = _bf16(inp.k_block(i))
        vpad[i, :, :L] = _bf16(inp.v_block(i))
    kb = [kpad[i, :, :L] for i, L in enumerate(lens)]
    vb = [vpad[i, :, :L] for i, L in enumerate(lens)]
    dq, dk, dv = cp.ring_attention_bwd(_bf16(inp.q), kb, vb, _f32(o), _f32(lse), _f32(do), scale=scale)
    torch.cuda.synchronize()
    got = (dq.cpu().numpy(), [t.cpu().numpy() for t in dk], [t.cpu().numpy() for t in dv])
    _check_all("bwd padded gather", inp, do, scale, got)
