"""CPU oracle for one rank's share of context-parallel (Ring / Ulysses) attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package; only the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP path (no kernels,
headers, helpers or constants); the two meet only in the seeded inputs of the
``workloads`` module, which holds none of the method's arithmetic.

Everything here is plain numpy in float64 on exactly the values the GPU sees
(bfloat16 inputs are upcast losslessly). It is written for a reader to check
against the pages by eye: no blocking, fusion or reordering beyond what each
definition states.

Sources (diffusers v0.43.0 documentation pages):
  * "Paralelismo de contexto" (context-parallelism guide, Portuguese),
    sections "Atenção em Anel", "Atenção Ulysses", "Ring Anything Attention";
  * "Paralelismo" (parallelism API reference, Spanish), section
    "ContextParallelConfig", parameters ``ring_degree``, ``convert_to_fp32``,
    ``rotate_method``, ``ring_anything``;
  * "Inferencia distribuida" (distributed-inference guide, Spanish), sections
    "Ring Attention", "Ulysses Attention".

Readings taken where the pages are silent:
  * the merge of per-block partials is the exact log-sum-exp recombination,
    the only merge under which a full ring equals full attention;
  * the softmax scale is 1/sqrt(D) and LSE is the natural log of
    sum_j exp(scale * q.k_j);
  * the Ulysses regroup sends head group g to token slot g (contiguous head
    groups, token chunks concatenated in rank order).

Pins: every function here is checked by the CPU tests against something other
than itself -- a pure-Python brute force, closed forms, a library attention
routine, hand-computed golden values under ``tests/golden/`` and invariants
(ring over any split == single pass, shift/permutation invariance, regroup
round trip, multi-rank Ulysses, Ulysses Anything and Unified simulations); the
uneven packs against a hand-written golden map and pure-Python loops; the backward against
central differences of the forward, a library autograd and its invariants.
No function is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

__all__ = [
    "attention",
    "block_attention",
    "lse_merge",
    "ring_attention",
    "ulysses_regroup",
    "ulysses_regroup_inv",
    "usp_attention",
    "ulysses_pack_heads",
    "ulysses_unpack_heads",
    "ulysses_concat_seq",
    "ulysses_split_seq",
    "ulysses_anything_attention",
    "attention_bwd",
    "ring_attention_bwd",
    "brute_attention",
]

_F64 = np.float64


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              row_chunk: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Full non-causal softmax attention, plus the log-sum-exp of each row.

    Layout is [B, S, H, D] for q (Sq rows), k and v (Skv rows); returns
    O [B, Sq, H, D] and LSE [B, H, Sq], both float64.

    Definition (one (b, h) pair, one query row q_i):
        x_ij  = scale * <q_i, k_j>
        LSE_i = ln sum_j exp(x_ij)
        O_i   = sum_j exp(x_ij - LSE_i) * v_j
    evaluated with the row maximum subtracted before exponentiating, which is
    the same value up to rounding. Each rank of a ring computes exactly this
    between its local Q and one K/V block ("Paralelismo" API reference,
    ContextParallelConfig, ``ring_degree``), and a full ring must reproduce
    it over all tokens ("Paralelismo de contexto", "Atenção em Anel").

    An empty key set (Skv == 0) gives O = 0 and LSE = -inf: the sum over no
    terms is zero, so its log is -inf and it carries no weight in a merge.
    """
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    assert k.shape == (B, Skv, H, D) and v.shape == (B, Skv, H, D), (q.shape, k.shape, v.shape)
    out = np.zeros((B, Sq, H, D), dtype=_F64)
    lse = np.empty((B, H, Sq), dtype=_F64)
    if Skv == 0:
        lse[...] = -np.inf
        return out, lse
    for b in range(B):
        for h in range(H):
            kh = np.asarray(k[b, :, h, :], dtype=_F64)  # [Skv, D]
            vh = np.asarray(v[b, :, h, :], dtype=_F64)
            for r0 in range(0, Sq, row_chunk):
                r1 = min(Sq, r0 + row_chunk)
                qh = np.asarray(q[b, r0:r1, h, :], dtype=_F64)  # [rows, D]
                x = scale * (qh @ kh.T)                       # scores [rows, Skv]
                m = x.max(axis=1, keepdims=True)
                e = np.exp(x - m)
                l = e.sum(axis=1, keepdims=True)
                out[b, r0:r1, h, :] = (e @ vh) / l
                lse[b, h, r0:r1] = (m + np.log(l))[:, 0]
    return out, lse


def block_attention(q: np.ndarray, k_block: np.ndarray, v_block: np.ndarray,
                    scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Partial attention of the local Q against one K/V block.

    Each block yields a partial output and its LSE; ``convert_to_fp32`` keeps
    both in float32 on the GPU so that the merge is stable ("Paralelismo",
    ContextParallelConfig, ``convert_to_fp32``). Here both are float64.
    A Ring Anything block is first cut back to its true length
    ("Paralelismo de contexto", "Ring Anything Attention"); callers pass the
    already-cut block, whose length may be zero.
    """
    return attention(q, k_block, v_block, scale)


def lse_merge(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray,
              lse_b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two partial results of the same queries over disjoint key sets.

    With O in [B, S, H, D] and LSE in [B, H, S]:
        M   = max(LSE_a, LSE_b)
        w_a = exp(LSE_a - M),  w_b = exp(LSE_b - M)
        LSE = M + ln(w_a + w_b)
        O   = (w_a * O_a + w_b * O_b) / (w_a + w_b)
    which is attention over the union of the two key sets. The pages name
    the merged quantities (partial output and LSE, kept in float32) but do
    not print the formula; this is the exact recombination
    ("Paralelismo", ContextParallelConfig, ``convert_to_fp32``).

    A side with LSE = -inf (no keys) gets weight 0. If both are -inf the
    result is O = 0, LSE = -inf.
    """
    lse_a = np.asarray(lse_a, dtype=_F64)
    lse_b = np.asarray(lse_b, dtype=_F64)
    m = np.maximum(lse_a, lse_b)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    w_a = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - m_safe))
    w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))
    tot = w_a + w_b
    with np.errstate(divide="ignore"):
        lse = np.where(both_empty, -np.inf, m_safe + np.log(np.where(both_empty, 1.0, tot)))
    # weights are [B, H, S]; outputs are [B, S, H, D]
    wa = np.transpose(w_a, (0, 2, 1))[..., None]
    wb = np.transpose(w_b, (0, 2, 1))[..., None]
    den = np.transpose(np.where(both_empty, 1.0, tot), (0, 2, 1))[..., None]
    o = (wa * np.asarray(o_a, dtype=_F64) + wb * np.asarray(o_b, dtype=_F64)) / den
    return o, lse


def ring_attention(q: np.ndarray, k_blocks: Sequence[np.ndarray], v_blocks: Sequence[np.ndarray],
                   scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One rank's share of Ring Attention with all K/V blocks resident.

    The rank attends its local Q to each K/V block in turn and folds the
    partials into an accumulator, block 0 first ("Paralelismo de contexto",
    "Atenção em Anel": after a full loop every rank has seen the K/V of all
    tokens; "Paralelismo", ContextParallelConfig, ``rotate_method`` --
    all-gather, so every block is present before the loop).
    """
    assert len(k_blocks) == len(v_blocks) and len(k_blocks) >= 1
    o, lse = block_attention(q, k_blocks[0], v_blocks[0], scale)
    for kb, vb in zip(k_blocks[1:], v_blocks[1:]):
        o_i, lse_i = block_attention(q, kb, vb, scale)
        o, lse = lse_merge(o, lse, o_i, lse_i)
    return o, lse


def ulysses_regroup(x: np.ndarray, degree: int) -> np.ndarray:
    """Sequence-sharded -> head-sharded layout of one rank (all-to-all, loopback).

    x is [B, S_local, H, D]. The first all-to-all leaves each rank with every
    token for a subset of heads ("Paralelismo de contexto", "Atenção Ulysses").
    With the exchange replaced by a loopback, head group g (heads
    g*H/P .. (g+1)*H/P - 1) of this rank's tokens becomes token chunk g:
        out[b, g*S_local + s, h, d] = x[b, s, g*(H/P) + h, d]
    Result: [B, P*S_local, H/P, D]. A pure permutation: bit-exact.
    """
    B, S_l, H, D = x.shape
    assert H % degree == 0
    Hl = H // degree
    return np.ascontiguousarray(
        x.reshape(B, S_l, degree, Hl, D).transpose(0, 2, 1, 3, 4).reshape(B, degree * S_l, Hl, D))


def ulysses_regroup_inv(y: np.ndarray, degree: int) -> np.ndarray:
    """Head-sharded -> sequence-sharded: the second all-to-all, regrouping by token.

    y is [B, P*S_local, H/P, D]; inverse of ``ulysses_regroup``:
        out[b, s, g*(H/P) + h, d] = y[b, g*S_local + s, h, d]
    """
    B, S, Hl, D = y.shape
    assert S % degree == 0
    S_l = S // degree
    return np.ascontiguousarray(
        y.reshape(B, degree, S_l, Hl, D).transpose(0, 2, 1, 3, 4).reshape(B, S_l, degree * Hl, D))


def usp_attention(q: np.ndarray, k_shards: Sequence[np.ndarray], v_shards: Sequence[np.ndarray],
                  degree: int, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One rank's share of Unified (Ulysses x Ring) attention, exchanges as loopbacks.

    "Paralelismo de contexto", "Atenção Unificada": an all-to-all regroups
    heads and tokens, Ring Attention runs on the result, and the all-to-all is
    reversed. q is this rank's [B, S_local, H, D] shard; k_shards[r] and
    v_shards[r] are ring rank r's [B, S_local, H, D] shards, each regrouped the
    same way and forming ring block r. Returns the output in the original
    layout [B, S_local, H, D] and the LSE in the head-sharded layout
    [B, H/P, P*S_local].
    """
    q_h = ulysses_regroup(q, degree)
    kb = [ulysses_regroup(k, degree) for k in k_shards]
    vb = [ulysses_regroup(v, degree) for v in v_shards]
    o_h, lse = ring_attention(q_h, kb, vb, scale)
    return ulysses_regroup_inv(o_h, degree), lse


def ulysses_pack_heads(x: np.ndarray, head_counts: Sequence[int]) -> np.ndarray:
    """Ulysses Anything: one rank's all-to-all buffer ordered by head group.

    "Paralelismo de contexto", "Ulysses Anything Attention" (and the API's
    ``ulysses_anything``): the sequence length and the head count need not
    divide by the degree. x is the rank's [B, S_r, H, D]; head group g is the
    next head_counts[g] heads (sum = H, contiguous, in order) and goes to rank
    g. The first all-to-all sends piece g = x[:, :, heads of g, :] (shape
    [B, S_r, H_g, D], row-major) to rank g; the pieces lie back to back in the
    returned 1-D buffer. A pure permutation.
    """
    B, S_r, H, D = x.shape
    assert sum(head_counts) == H and all(c >= 0 for c in head_counts)
    pieces = []
    h0 = 0
    for c in head_counts:
        pieces.append(np.ascontiguousarray(x[:, :, h0:h0 + c, :]).reshape(-1))
        h0 += c
    return np.concatenate(pieces) if pieces else np.zeros(0, dtype=x.dtype)


def ulysses_unpack_heads(buf: np.ndarray, B: int, S_r: int, head_counts: Sequence[int], D: int) -> np.ndarray:
    """Inverse of ``ulysses_pack_heads``: after the second all-to-all a rank
    holds, from each rank g, its S_r tokens for head group g back to back;
    they are placed at heads g's offset of a [B, S_r, H, D] tensor."""
    H = sum(head_counts)
    out = np.zeros((B, S_r, H, D), dtype=buf.dtype)
    pos = h0 = 0
    for c in head_counts:
        n = B * S_r * c * D
        out[:, :, h0:h0 + c, :] = buf[pos:pos + n].reshape(B, S_r, c, D)
        pos += n
        h0 += c
    assert pos == buf.size
    return out


def ulysses_concat_seq(buf: np.ndarray, B: int, seq_counts: Sequence[int], H_g: int, D: int) -> np.ndarray:
    """The receiving side of the first all-to-all: from each rank r a piece
    [B, S_r, H_g, D] (back to back, rank order) becomes the token range of rank
    r in [B, sum S_r, H_g, D] (every token of this rank's heads)."""
    parts = []
    pos = 0
    for c in seq_counts:
        n = B * c * H_g * D
        parts.append(buf[pos:pos + n].reshape(B, c, H_g, D))
        pos += n
    assert pos == buf.size
    return np.concatenate(parts, axis=1)


def ulysses_split_seq(y: np.ndarray, seq_counts: Sequence[int]) -> np.ndarray:
    """Inverse of ``ulysses_concat_seq``: the sending side of the second
    all-to-all, token range of rank r as piece r ([B, S_r, H_g, D]), back to back."""
    assert sum(seq_counts) == y.shape[1]
    pieces = []
    s0 = 0
    for c in seq_counts:
        pieces.append(np.ascontiguousarray(y[:, s0:s0 + c]).reshape(-1))
        s0 += c
    return np.concatenate(pieces) if pieces else np.zeros(0, dtype=y.dtype)


def ulysses_anything_attention(q_shards: Sequence[np.ndarray], k_shards: Sequence[np.ndarray],
                               v_shards: Sequence[np.ndarray], head_counts: Sequence[int],
                               scale: float) -> List[np.ndarray]:
    """Every rank of an uneven Ulysses group, with both all-to-alls simulated.

    Rank r holds the [B, S_r, H, D] shards of Q, K and V (S_r arbitrary); rank
    g ends up with every token of head group g (head_counts[g] heads), attends
    over the whole sequence, and the second all-to-all returns each rank its
    own tokens with every head. Returns each rank's output [B, S_r, H, D]; the
    concatenation over ranks is full attention on the whole sequence.
    """
    P = len(q_shards)
    assert len(head_counts) == P
    B, _, H, D = q_shards[0].shape
    seq_counts = [x.shape[1] for x in q_shards]

    def exchange(send_bufs, piece_sizes):
        # piece_sizes[r][g]: elements rank r sends to rank g; rank g receives in rank order
        recv = []
        for g in range(P):
            parts = []
            for r in range(P):
                off = sum(piece_sizes[r][:g])
                parts.append(send_bufs[r][off:off + piece_sizes[r][g]])
            recv.append(np.concatenate(parts))
        return recv

    sizes1 = [[B * seq_counts[r] * head_counts[g] * D for g in range(P)] for r in range(P)]
    heads_view = []
    for shards in (q_shards, k_shards, v_shards):
        recv = exchange([ulysses_pack_heads(x, head_counts) for x in shards], sizes1)
        heads_view.append([ulysses_concat_seq(recv[g], B, seq_counts, head_counts[g], D) for g in range(P)])
    outs = [attention(heads_view[0][g], heads_view[1][g], heads_view[2][g], scale)[0] for g in range(P)]
    sizes2 = [[B * seq_counts[r] * head_counts[g] * D for r in range(P)] for g in range(P)]
    recv = exchange([ulysses_split_seq(outs[g], seq_counts) for g in range(P)], sizes2)
    return [ulysses_unpack_heads(recv[r], B, seq_counts[r], head_counts, D) for r in range(P)]


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, o: np.ndarray, lse: np.ndarray,
                  do: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of ``attention`` with respect to q, k and v, given dL/dO.

    The pages run Ring Attention for training as well as inference (only the
    Ring Anything variant is inference-only: "Paralelismo de contexto",
    "Ring Anything Attention"), so the ring's blocks need a backward pass.
    The pages print no formula; this is the derivative of the definition in
    ``attention`` (o and lse are that function's outputs for q, k, v), for one
    (b, h) pair:
        P_ij  = exp(scale * <q_i, k_j> - LSE_i)      (the softmax weights)
        D_i   = sum_d dO_id * O_id
        dV_j  = sum_i P_ij dO_i
        dP_ij = <dO_i, v_j>
        dS_ij = P_ij * (dP_ij - D_i)
        dQ_i  = scale * sum_j dS_ij k_j
        dK_j  = scale * sum_i dS_ij q_i
    All float64; returns dq [B, Sq, H, D], dk and dv [B, Skv, H, D].
    """
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    dq = np.zeros((B, Sq, H, D), dtype=_F64)
    dk = np.zeros((B, Skv, H, D), dtype=_F64)
    dv = np.zeros((B, Skv, H, D), dtype=_F64)
    if Skv == 0 or Sq == 0:
        return dq, dk, dv
    for b in range(B):
        for h in range(H):
            qh = np.asarray(q[b, :, h, :], dtype=_F64)
            kh = np.asarray(k[b, :, h, :], dtype=_F64)
            vh = np.asarray(v[b, :, h, :], dtype=_F64)
            oh = np.asarray(o[b, :, h, :], dtype=_F64)
            doh = np.asarray(do[b, :, h, :], dtype=_F64)
            lh = np.asarray(lse[b, h, :], dtype=_F64)[:, None]
            p = np.exp(scale * (qh @ kh.T) - lh)      # [Sq, Skv]
            d = (doh * oh).sum(axis=1, keepdims=True)  # [Sq, 1]
            dv[b, :, h, :] = p.T @ doh
            ds = p * (doh @ vh.T - d)
            dq[b, :, h, :] = scale * (ds @ kh)
            dk[b, :, h, :] = scale * (ds.T @ qh)
    return dq, dk, dv


def ring_attention_bwd(q: np.ndarray, k_blocks: Sequence[np.ndarray], v_blocks: Sequence[np.ndarray],
                       o: np.ndarray, lse: np.ndarray, do: np.ndarray,
                       scale: float) -> Tuple[np.ndarray, List[np.ndarray], List[np.ndarray]]:
    """Backward of one rank's ring share, block by block.

    o and lse are the merged (full-ring) output and LSE. Block i contributes
    ``attention_bwd`` evaluated with those global o and lse on its own keys:
    the softmax weights of its keys are exp(scale <q, k> - LSE) with the
    global LSE, so the per-block terms add up to the single-pass gradient.
    Returns dq (summed over blocks) and each block's dk, dv.
    """
    dq = np.zeros(q.shape, dtype=_F64)
    dks, dvs = [], []
    for kb, vb in zip(k_blocks, v_blocks):
        dq_i, dk_i, dv_i = attention_bwd(q, kb, vb, o, lse, do, scale)
        dq += dq_i
        dks.append(dk_i)
        dvs.append(dv_i)
    return dq, dks, dvs


def brute_attention(q, k, v, scale: float):
    """Pure-Python attention with math.exp / math.log, for tiny shapes only.

    Same definition as ``attention`` with nothing vectorised and no max
    subtraction (tiny inputs cannot overflow), so it shares no evaluation
    order with the numpy version. Returns nested lists O[b][s][h][d],
    LSE[b][h][s].
    """
    B, Sq, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Skv = len(k[0])
    O = [[[[0.0] * D for _ in range(H)] for _ in range(Sq)] for _ in range(B)]
    L = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                w = []
                for j in range(Skv):
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[b][i][h][d]) * float(k[b][j][h][d])
                    w.append(math.exp(scale * dot))
                tot = sum(w)
                L[b][h][i] = math.log(tot) if Skv else -math.inf
                for d in range(D):
                    acc = 0.0
                    for j in range(Skv):
                        acc += w[j] * float(v[b][j][h][d])
                    O[b][i][h][d] = acc / tot if Skv else 0.0
    return O, L
