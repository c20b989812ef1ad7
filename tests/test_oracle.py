"""Pins for the CPU oracle: each check fixes the oracle to something other than itself.

Brute force on tiny inputs, a library attention routine, hand-derived golden
values, closed forms and invariants. They are chosen so that a plausible slip
in the oracle -- a dropped scale, a wrong sign, a transposed operand, a merge
that forgets one side's weight, a regroup with swapped indices -- fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
_ENV = {"e": math.e, "log": math.log, "exp": math.exp, "sqrt": math.sqrt,
        "ln3": math.log(3.0), "inf": math.inf}


def _ev(x):
    """Evaluate a golden entry: numbers pass through, strings are closed forms."""
    if isinstance(x, list):
        return [_ev(y) for y in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, _ENV))  # noqa: S307 - fixed local fixture
    return float(x)


def _arr(x):
    return np.array(_ev(x), dtype=np.float64)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------- golden values ---

@pytest.mark.parametrize("case", _golden()["attention"], ids=lambda c: c["name"])
def test_golden_attention(case):
    o, lse = oracle.attention(_arr(case["q"]), _arr(case["k"]), _arr(case["v"]), _ev(case["scale"]))
    np.testing.assert_allclose(o, _arr(case["expected_o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, _arr(case["expected_lse"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", _golden()["merge"], ids=lambda c: c["name"])
def test_golden_merge(case):
    o, lse = oracle.lse_merge(_arr(case["o_a"]), _arr(case["lse_a"]), _arr(case["o_b"]), _arr(case["lse_b"]))
    np.testing.assert_allclose(o, _arr(case["expected_o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, _arr(case["expected_lse"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", _golden()["ring"], ids=lambda c: c["name"])
def test_golden_ring(case):
    q = _arr(case["q"])
    kbs = [_arr(x) for x in case["k_blocks"]]
    vbs = [_arr(x) for x in case["v_blocks"]]
    s = _ev(case["scale"])
    for i, (kb, vb) in enumerate(zip(kbs, vbs)):
        o_i, lse_i = oracle.block_attention(q, kb, vb, s)
        np.testing.assert_allclose(o_i, _arr(case["expected_block_o"][i]), atol=1e-14, rtol=0)
        np.testing.assert_allclose(lse_i, _arr(case["expected_block_lse"][i]), atol=1e-14, rtol=0)
    o, lse = oracle.ring_attention(q, kbs, vbs, s)
    np.testing.assert_allclose(o, _arr(case["expected_o"]), atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, _arr(case["expected_lse"]), atol=1e-14, rtol=0)


@pytest.mark.parametrize("case", _golden()["regroup"], ids=lambda c: c["name"])
def test_golden_regroup(case):
    x = np.array(case["in"], dtype=np.float32)
    want = np.array(case["expected_out"], dtype=np.float32)
    got = oracle.ulysses_regroup(x, case["degree"])
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.ulysses_regroup_inv(want, case["degree"]), x)


# ------------------------------------------------------------- brute force ---

@pytest.mark.parametrize("B,H,D,Sq,Skv,seed", [(1, 2, 4, 3, 7, 0), (2, 3, 5, 4, 6, 1), (1, 1, 8, 1, 1, 2)])
def test_brute_force_agrees(B, H, D, Sq, Skv, seed):
    q, k, v = _rand((B, Sq, H, D), seed), _rand((B, Skv, H, D), seed + 10), _rand((B, Skv, H, D), seed + 20)
    s = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, s)
    ob, lb = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), s)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12, rtol=0)


def test_brute_force_ring_split_3_2_2():
    B, H, D, Sq = 1, 2, 4, 3
    lens = [3, 2, 2]
    q, k, v = _rand((B, Sq, H, D), 3), _rand((B, 7, H, D), 4), _rand((B, 7, H, D), 5)
    s = 0.5
    offs = workloads.block_offsets(lens)
    kbs = [k[:, o:o + L] for o, L in zip(offs, lens)]
    vbs = [v[:, o:o + L] for o, L in zip(offs, lens)]
    o, lse = oracle.ring_attention(q, kbs, vbs, s)
    ob, lb = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), s)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12, rtol=0)


# --------------------------------------------------------- library routine ---

def test_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    B, H, D, Sq, Skv = 2, 3, 16, 37, 53
    q, k, v = _rand((B, Sq, H, D), 7), _rand((B, Skv, H, D), 8), _rand((B, Skv, H, D), 9)
    s = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, s, row_chunk=8)
    # SDPA takes [B, H, S, D]
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s)
    np.testing.assert_allclose(o, ref.numpy().transpose(0, 2, 1, 3), atol=1e-12, rtol=0)
    ref_lse = torch.logsumexp(s * (tq @ tk.transpose(-1, -2)), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12, rtol=0)


# ------------------------------------------------------------ closed forms ---

def test_identical_keys_give_mean_of_v():
    B, H, D, Sq, Skv = 1, 2, 8, 5, 9
    q = _rand((B, Sq, H, D), 11)
    k1 = _rand((B, 1, H, D), 12)
    k = np.repeat(k1, Skv, axis=1)
    v = _rand((B, Skv, H, D), 13)
    s = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, s)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-13)
    dots = np.einsum("bshd,bhd->bhs", q, k1[:, 0])
    np.testing.assert_allclose(lse, s * dots + math.log(Skv), atol=1e-13)


def test_zero_query_gives_mean_and_log_count():
    B, H, D, Sq, Skv = 2, 1, 4, 3, 6
    q = np.zeros((B, Sq, H, D))
    k, v = _rand((B, Skv, H, D), 14), _rand((B, Skv, H, D), 15)
    o, lse = oracle.attention(q, k, v, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(Skv), atol=1e-14)


def test_single_key_returns_its_value():
    B, H, D, Sq = 1, 3, 4, 5
    q, k, v = _rand((B, Sq, H, D), 16), _rand((B, 1, H, D), 17), _rand((B, 1, H, D), 18)
    o, lse = oracle.attention(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * np.einsum("bshd,bhd->bhs", q, k[:, 0]), atol=1e-13)


def test_constant_values_rows_sum_to_one():
    """V = c everywhere gives O = c exactly when the softmax weights sum to 1."""
    B, H, D, Sq, Skv = 1, 2, 6, 7, 11
    q, k = _rand((B, Sq, H, D), 19) * 3, _rand((B, Skv, H, D), 20)
    v = np.full((B, Skv, H, D), 2.5)
    o, _ = oracle.attention(q, k, v, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(o, 2.5, atol=1e-13)


def test_empty_key_set():
    q = _rand((1, 3, 2, 4), 21)
    o, lse = oracle.attention(q, np.zeros((1, 0, 2, 4)), np.zeros((1, 0, 2, 4)), 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# -------------------------------------------------------------- invariants ---

def test_key_shift_moves_only_lse():
    """k_j -> k_j + u adds scale*<q, u> to every score of a row."""
    B, H, D, Sq, Skv = 1, 2, 8, 6, 10
    q, k, v = _rand((B, Sq, H, D), 22), _rand((B, Skv, H, D), 23), _rand((B, Skv, H, D), 24)
    u = _rand((B, 1, H, D), 25)
    s = 1.0 / math.sqrt(D)
    o0, l0 = oracle.attention(q, k, v, s)
    o1, l1 = oracle.attention(q, k + u, v, s)
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1 - l0, s * np.einsum("bshd,bhd->bhs", q, u[:, 0]), atol=1e-12)


def test_key_permutation_invariance_and_query_equivariance():
    B, H, D, Sq, Skv = 2, 2, 4, 5, 9
    q, k, v = _rand((B, Sq, H, D), 26), _rand((B, Skv, H, D), 27), _rand((B, Skv, H, D), 28)
    pk = np.random.default_rng(29).permutation(Skv)
    pq = np.random.default_rng(30).permutation(Sq)
    o0, l0 = oracle.attention(q, k, v, 0.5)
    o1, l1 = oracle.attention(q[:, pq], k[:, pk], v[:, pk], 0.5)
    np.testing.assert_allclose(o1, o0[:, pq], atol=1e-13)
    np.testing.assert_allclose(l1, l0[:, :, pq], atol=1e-13)


def test_heads_and_batches_are_independent():
    """Each (b, h) slice is its own attention problem (no mixing of heads)."""
    B, H, D, Sq, Skv = 2, 3, 4, 4, 6
    q, k, v = _rand((B, Sq, H, D), 31), _rand((B, Skv, H, D), 32), _rand((B, Skv, H, D), 33)
    o, lse = oracle.attention(q, k, v, 0.5)
    for b in range(B):
        for h in range(H):
            ob, lb = oracle.attention(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1], 0.5)
            np.testing.assert_allclose(o[b:b + 1, :, h:h + 1], ob, atol=1e-14)
            np.testing.assert_allclose(lse[b:b + 1, h:h + 1], lb, atol=1e-14)


# ---------------------------------------------------------------- the ring ---

def _split(k, lens):
    offs = workloads.block_offsets(lens)
    return [k[:, o:o + L] for o, L in zip(offs, lens)]


@pytest.mark.parametrize("lens", [[16, 16, 16, 16], [22, 21, 21], [30, 1, 33], [20, 0, 44], [64], [1, 1, 62]])
def test_ring_equals_single_pass(lens):
    B, H, D, Sq = 2, 3, 8, 12
    Skv = sum(lens)
    q, k, v = _rand((B, Sq, H, D), 40), _rand((B, Skv, H, D), 41), _rand((B, Skv, H, D), 42)
    s = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, s)
    orr, lr = oracle.ring_attention(q, _split(k, lens), _split(v, lens), s)
    np.testing.assert_allclose(orr, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lr, lse, atol=1e-12, rtol=0)


def test_ring_block_order_does_not_matter():
    """A real ring starts from the rank's own block; any rotation gives the same result."""
    B, H, D, Sq, lens = 1, 2, 8, 9, [10, 7, 13, 12]
    q, k, v = _rand((B, Sq, H, D), 43), _rand((B, sum(lens), H, D), 44), _rand((B, sum(lens), H, D), 45)
    kb, vb = _split(k, lens), _split(v, lens)
    o0, l0 = oracle.ring_attention(q, kb, vb, 0.4)
    for r in range(1, len(lens)):
        o1, l1 = oracle.ring_attention(q, kb[r:] + kb[:r], vb[r:] + vb[:r], 0.4)
        np.testing.assert_allclose(o1, o0, atol=1e-12)
        np.testing.assert_allclose(l1, l0, atol=1e-12)


def test_ring_anything_split_rule_and_config5_shape():
    assert workloads.split_lengths(4607, 3) == [1536, 1536, 1535]
    assert workloads.split_lengths(4481, 4) == [1121, 1120, 1120, 1120]
    assert workloads.split_lengths(4608, 2) == [2304, 2304]
    w = workloads.by_name("ring_anything3_uneven_bf16")
    assert list(w.block_lens) == workloads.split_lengths(w.Skv, w.ring_degree)


# --------------------------------------------------------------- the merge ---

def _partial(seed, B=2, S=5, H=3, D=4):
    r = np.random.default_rng(seed)
    return r.standard_normal((B, S, H, D)), r.standard_normal((B, H, S)) * 3


def test_merge_commutative_and_associative():
    a, b, c = _partial(50), _partial(51), _partial(52)
    ab = oracle.lse_merge(*a, *b)
    ba = oracle.lse_merge(*b, *a)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-14)
    l = oracle.lse_merge(*ab, *c)
    r = oracle.lse_merge(*a, *oracle.lse_merge(*b, *c))
    np.testing.assert_allclose(l[0], r[0], atol=1e-13)
    np.testing.assert_allclose(l[1], r[1], atol=1e-13)


def test_merge_with_itself_adds_log2():
    o, l = _partial(53)
    mo, ml = oracle.lse_merge(o, l, o, l)
    np.testing.assert_allclose(mo, o, atol=1e-14)
    np.testing.assert_allclose(ml, l + math.log(2.0), atol=1e-14)


def test_merge_with_empty_is_identity_and_empty_pair_stays_empty():
    o, l = _partial(54)
    empty_o, empty_l = np.zeros_like(o), np.full_like(l, -np.inf)
    mo, ml = oracle.lse_merge(o, l, empty_o, empty_l)
    np.testing.assert_array_equal(mo, o)
    np.testing.assert_array_equal(ml, l)
    mo, ml = oracle.lse_merge(empty_o, empty_l, o, l)
    np.testing.assert_array_equal(mo, o)
    np.testing.assert_array_equal(ml, l)
    mo, ml = oracle.lse_merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))


def test_merge_weights_follow_lse_not_position():
    """Hand case with [B, S, H] > 1 to catch a transposed weight layout."""
    B, S, H, D = 1, 2, 3, 1
    o_a = np.zeros((B, S, H, D))
    o_b = np.ones((B, S, H, D))
    lse_a = np.zeros((B, H, S))
    lse_b = np.array([[[0.0, math.log(3)], [math.log(3), 0.0], [-np.inf, math.log(7)]]])
    mo, ml = oracle.lse_merge(o_a, lse_a, o_b, lse_b)
    # weight of b = e^{lse_b} / (1 + e^{lse_b}) per (h, s)
    want = np.array([[[0.5, 0.75, 0.0], [0.75, 0.5, 7 / 8]]])[..., None]
    np.testing.assert_allclose(mo, want, atol=1e-15)
    np.testing.assert_allclose(ml, np.log(1 + np.exp(lse_b)), atol=1e-15)


# ------------------------------------------------------- Ulysses Anything ---

@pytest.mark.parametrize("case", _golden()["ulysses_anything"], ids=lambda c: c["name"])
def test_golden_ulysses_anything(case):
    if case["op"] == "pack_heads":
        x = np.array(case["in"], dtype=np.float64)
        buf = oracle.ulysses_pack_heads(x, case["counts"])
        assert buf.tolist() == case["expected_buf"]
        B, S_r, _, D = x.shape
        assert np.array_equal(oracle.ulysses_unpack_heads(buf, B, S_r, case["counts"], D), x)
    else:
        buf = np.array(case["buf"], dtype=np.float64)
        y = oracle.ulysses_concat_seq(buf, case["B"], case["counts"], case["H_g"], case["D"])
        assert y.tolist() == case["expected_out"]
        assert np.array_equal(oracle.ulysses_split_seq(y, case["counts"]), buf)


@pytest.mark.parametrize("B,S_r,counts,D", [(1, 3, (2, 1, 2), 2), (2, 2, (0, 3, 1), 3), (3, 1, (1,), 2)])
def test_pack_heads_matches_index_loops(B, S_r, counts, D):
    """Pure-Python loops over every element: piece g holds (b, s, head h0_g + j, d) at
    offset B*S_r*D*h0_g + ((b*S_r + s)*H_g + j)*D + d."""
    H = sum(counts)
    x = np.arange(B * S_r * H * D, dtype=np.float64).reshape(B, S_r, H, D)
    buf = oracle.ulysses_pack_heads(x, counts)
    want = [None] * x.size
    h0 = 0
    for Hg in counts:
        for b in range(B):
            for s in range(S_r):
                for j in range(Hg):
                    for d in range(D):
                        want[B * S_r * D * h0 + ((b * S_r + s) * Hg + j) * D + d] = float(x[b, s, h0 + j, d])
        h0 += Hg
    assert buf.tolist() == want


@pytest.mark.parametrize("B,counts,Hg,D", [(1, (3, 2, 2), 2, 2), (2, (1, 0, 3), 1, 3)])
def test_concat_seq_matches_index_loops(B, counts, Hg, D):
    n = B * sum(counts) * Hg * D
    buf = np.arange(n, dtype=np.float64)
    y = oracle.ulysses_concat_seq(buf, B, counts, Hg, D)
    pos = s0 = 0
    for c in counts:
        for b in range(B):
            for s in range(c):
                for h in range(Hg):
                    for d in range(D):
                        assert y[b, s0 + s, h, d] == buf[pos]
                        pos += 1
        s0 += c
    assert pos == n


def test_pack_even_split_is_the_regroup():
    """Equal head groups, one batch: the pieces back to back are the even regroup's tokens chunks."""
    x = _rand((1, 5, 6, 4), 120)
    buf = oracle.ulysses_pack_heads(x, (2, 2, 2))
    np.testing.assert_array_equal(buf.reshape(15, 2, 4), oracle.ulysses_regroup(x, 3)[0])
    np.testing.assert_array_equal(oracle.ulysses_pack_heads(x, (6,)), x.reshape(-1))


@pytest.mark.parametrize("seq,heads,B", [((5, 4, 4), (2, 2, 1), 2), ((3, 3, 3, 2), (2, 1, 1, 2), 1),
                                          ((7, 0), (1, 3), 1)])
def test_ulysses_anything_simulation_is_full_attention(seq, heads, B):
    """All ranks of an uneven Ulysses group, both exchanges simulated: rank outputs concatenated
    over the sequence equal full attention."""
    H, D = sum(heads), 4
    S = sum(seq)
    q, k, v = (_rand((B, S, H, D), sd) for sd in (121, 122, 123))
    offs = np.cumsum((0,) + seq)
    shard = lambda x: [x[:, offs[r]:offs[r + 1]] for r in range(len(seq))]  # noqa: E731
    outs = oracle.ulysses_anything_attention(shard(q), shard(k), shard(v), heads, 0.4)
    want, _ = oracle.attention(q, k, v, 0.4)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), want, atol=1e-12)


# ------------------------------------------------------------- the regroup ---

@pytest.mark.parametrize("B,S_l,H,D,P", [(1, 5, 4, 3, 2), (2, 3, 6, 2, 3), (1, 4, 8, 1, 4), (2, 2, 3, 2, 1)])
def test_regroup_round_trip(B, S_l, H, D, P):
    x = _rand((B, S_l, H, D), 60)
    y = oracle.ulysses_regroup(x, P)
    assert y.shape == (B, P * S_l, H // P, D)
    np.testing.assert_array_equal(oracle.ulysses_regroup_inv(y, P), x)
    if P == 1:
        np.testing.assert_array_equal(y, x)


def test_regroup_index_map_elementwise():
    B, S_l, H, D, P = 2, 3, 6, 2, 3
    x = _rand((B, S_l, H, D), 61)
    y = oracle.ulysses_regroup(x, P)
    Hl = H // P
    for b in range(B):
        for g in range(P):
            for s in range(S_l):
                for h in range(Hl):
                    assert np.array_equal(y[b, g * S_l + s, h], x[b, s, g * Hl + h])


@pytest.mark.parametrize("P", [2, 3])
def test_ulysses_multi_rank_simulation_equals_full_attention(P):
    """Simulate P ranks: regroup, exchange slot g to rank g, attend, regroup back.

    Each rank's final output must equal full attention for its own query
    tokens over all tokens and all heads.
    """
    B, S_l, H, D = 1, 4, 6, 8
    S = P * S_l
    Q, K, V = _rand((B, S, H, D), 62), _rand((B, S, H, D), 63), _rand((B, S, H, D), 64)
    s = 1.0 / math.sqrt(D)
    full_o, _ = oracle.attention(Q, K, V, s)
    shard = lambda X, r: X[:, r * S_l:(r + 1) * S_l]  # noqa: E731
    # first all-to-all: rank r's regrouped chunk g goes to rank g
    sent = {name: [oracle.ulysses_regroup(shard(X, r), P) for r in range(P)] for name, X in (("q", Q), ("k", K), ("v", V))}
    recv = {name: [np.concatenate([sent[name][r][:, g * S_l:(g + 1) * S_l] for r in range(P)], axis=1)
                   for g in range(P)] for name in sent}
    outs = [oracle.attention(recv["q"][g], recv["k"][g], recv["v"][g], s)[0] for g in range(P)]
    Hl = H // P
    for g in range(P):  # each rank now holds every token of head group g
        np.testing.assert_allclose(outs[g], full_o[:, :, g * Hl:(g + 1) * Hl], atol=1e-12)
    # second all-to-all: rank g's token chunk r goes back to rank r
    for r in range(P):
        back = np.concatenate([outs[g][:, r * S_l:(r + 1) * S_l] for g in range(P)], axis=1)
        np.testing.assert_allclose(oracle.ulysses_regroup_inv(back, P), shard(full_o, r), atol=1e-12)


@pytest.mark.parametrize("U,R", [(2, 2), (2, 3), (3, 2)])
def test_usp_multi_rank_simulation_equals_full_attention(U, R):
    """Unified attention on a U x R grid, exchanges simulated.

    The sequence is cut into R ring chunks, each into U Ulysses shards; rank
    (r, u) holds shard u of chunk r. The Ulysses all-to-all inside ring group r
    leaves rank (r, u) with chunk r's tokens for head group u; Ring Attention
    over the R chunks then sees every token; the reverse all-to-all returns each
    rank's tokens with all heads. Every rank must end with full attention rows.
    """
    B, S_l, H, D = 1, 3, 2 * U, 8
    S = U * R * S_l
    Q, K, V = _rand((B, S, H, D), 71), _rand((B, S, H, D), 72), _rand((B, S, H, D), 73)
    s = 1.0 / math.sqrt(D)
    full_o, _ = oracle.attention(Q, K, V, s)
    Hl = H // U
    shard = lambda X, r, u: X[:, (r * U + u) * S_l:(r * U + u + 1) * S_l]  # noqa: E731
    head_sharded = {}  # (name, r, u) -> chunk r's tokens, head group u
    for name, X in (("q", Q), ("k", K), ("v", V)):
        for r in range(R):
            sent = [oracle.ulysses_regroup(shard(X, r, u), U) for u in range(U)]
            for u in range(U):
                head_sharded[(name, r, u)] = np.concatenate(
                    [sent[src][:, u * S_l:(u + 1) * S_l] for src in range(U)], axis=1)
    for u in range(U):
        kb = [head_sharded[("k", r, u)] for r in range(R)]
        vb = [head_sharded[("v", r, u)] for r in range(R)]
        outs = {r: oracle.ring_attention(head_sharded[("q", r, u)], kb, vb, s)[0] for r in range(R)}
        for r in range(R):
            np.testing.assert_allclose(outs[r], full_o[:, r * U * S_l:(r + 1) * U * S_l, u * Hl:(u + 1) * Hl],
                                       atol=1e-12)


def test_usp_share_equals_full_attention_on_exchange_symmetric_data():
    """Pin of ``usp_attention`` (exchanges as loopbacks).

    When, inside every ring chunk, all U shards are the same tokens and all U
    head groups carry the same values, each exchange hands a rank exactly what
    its loopback produces, so one rank's share must equal full attention of the
    whole sequence for that rank's tokens.
    """
    U, R, B, S_l, Hl, D = 2, 3, 1, 3, 2, 8
    H = U * Hl
    s = 1.0 / math.sqrt(D)
    shards = {}
    for name, seed in (("q", 81), ("k", 82), ("v", 83)):
        base = _rand((R, B, S_l, Hl, D), seed)
        shards[name] = [np.concatenate([base[r]] * U, axis=2) for r in range(R)]  # head groups equal
    glob = {n: np.concatenate([x for r in range(R) for x in [shards[n][r]] * U], axis=1) for n in shards}
    full_o, full_l = oracle.attention(glob["q"], glob["k"], glob["v"], s)
    o, lse = oracle.usp_attention(shards["q"][0], shards["k"], shards["v"], U, s)
    np.testing.assert_allclose(o, full_o[:, :S_l], atol=1e-12)
    # LSE is head-sharded: [B, H/U, U*S_l], token chunk g holds this rank's tokens again
    for g in range(U):
        np.testing.assert_allclose(lse[:, :, g * S_l:(g + 1) * S_l], full_l[:, :Hl, :S_l], atol=1e-12)


# ---------------------------------------------------------------- backward ---

def _loss(q, k, v, do, s):
    o, _ = oracle.attention(q, k, v, s)
    return float((o * do).sum())


def test_bwd_matches_central_differences():
    """dL/dq, dL/dk, dL/dv for L = sum(dO * O) against central differences of the forward."""
    B, Sq, Skv, H, D = 1, 3, 4, 2, 3
    q, k, v, do = (_rand(shp, sd) for shp, sd in (((B, Sq, H, D), 91), ((B, Skv, H, D), 92),
                                                  ((B, Skv, H, D), 93), ((B, Sq, H, D), 94)))
    s = 0.7
    o, lse = oracle.attention(q, k, v, s)
    dq, dk, dv = oracle.attention_bwd(q, k, v, o, lse, do, s)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            lp = _loss(**{**args, name: xp}, do=do, s=s)
            lm = _loss(**{**args, name: xm}, do=do, s=s)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=name)


def test_bwd_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    B, Sq, Skv, H, D = 2, 5, 7, 3, 8
    q, k, v, do = (_rand(shp, sd) for shp, sd in (((B, Sq, H, D), 95), ((B, Skv, H, D), 96),
                                                  ((B, Skv, H, D), 97), ((B, Sq, H, D), 98)))
    s = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, s)
    dq, dk, dv = oracle.attention_bwd(q, k, v, o, lse, do, s)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    x = torch.einsum("bqhd,bkhd->bhqk", tq, tk) * s
    to = torch.einsum("bhqk,bkhd->bqhd", torch.softmax(x, dim=-1), tv)
    to.backward(torch.tensor(do, dtype=torch.float64))
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12)


def test_bwd_invariants():
    """Key-shift invariance gives sum_j dK_j = 0; rows of P sum to 1 give
    sum_j dV_j = sum_i dO_i; identical keys make the output independent of q."""
    B, Sq, Skv, H, D = 1, 6, 9, 2, 4
    q, k, v, do = (_rand(shp, sd) for shp, sd in (((B, Sq, H, D), 101), ((B, Skv, H, D), 102),
                                                  ((B, Skv, H, D), 103), ((B, Sq, H, D), 104)))
    s = 0.5
    o, lse = oracle.attention(q, k, v, s)
    dq, dk, dv = oracle.attention_bwd(q, k, v, o, lse, do, s)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)
    k_same = np.broadcast_to(k[:, :1], k.shape).copy()
    o2, lse2 = oracle.attention(q, k_same, v, s)
    dq2, _, _ = oracle.attention_bwd(q, k_same, v, o2, lse2, do, s)
    np.testing.assert_allclose(dq2, 0.0, atol=1e-12)


@pytest.mark.parametrize("lens", [(4, 5), (3, 0, 6), (1, 1, 1, 6)])
def test_ring_bwd_equals_single_pass(lens):
    B, Sq, H, D = 2, 5, 2, 4
    Skv = sum(lens)
    q, k, v, do = (_rand(shp, sd) for shp, sd in (((B, Sq, H, D), 111), ((B, Skv, H, D), 112),
                                                  ((B, Skv, H, D), 113), ((B, Sq, H, D), 114)))
    s = 0.6
    o, lse = oracle.attention(q, k, v, s)
    dq, dk, dv = oracle.attention_bwd(q, k, v, o, lse, do, s)
    offs = workloads.block_offsets(lens)
    kb = [k[:, a:a + L] for a, L in zip(offs, lens)]
    vb = [v[:, a:a + L] for a, L in zip(offs, lens)]
    o_r, lse_r = oracle.ring_attention(q, kb, vb, s)
    dq_r, dks, dvs = oracle.ring_attention_bwd(q, kb, vb, o_r, lse_r, do, s)
    np.testing.assert_allclose(dq_r, dq, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(dks, axis=1), dk, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(dvs, axis=1), dv, atol=1e-12)


# ------------------------------------------------------- the input recipe ---

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(70).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e-39]  # exact ties and a denormal
    ours = workloads.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_workload_inputs_are_seeded_and_bf16_exact():
    w = workloads.by_name("flux1024_ring2_bf16")
    small = workloads.Workload(1, "probe", "bf16", B=1, H=2, D=8, Sq=4, block_lens=(3, 3))
    a, b = workloads.make_inputs(small), workloads.make_inputs(small)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(workloads.round_to_bf16(a.k), a.k)
    assert w.flops == 4 * 1 * 24 * 2304 * 4608 * 128
    u = workloads.by_name("flux1024_ulysses2_bf16")
    assert (u.attn_H, u.Sq, u.Skv) == (12, 4608, 4608)
    usp = workloads.by_name("flux1024_usp_u2r2_bf16")
    assert (usp.attn_H, usp.Sq, usp.Skv, usp.ring_degree) == (12, 2304, 4608, 2)
    assert usp.ulysses_degree * usp.ring_degree * usp.S_local == 4608  # one rank of the 2x2 grid
