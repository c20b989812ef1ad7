"""Seeded synthetic inputs for the ring-block attention path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds shapes, seeds and the rounding of inputs to bfloat16 --
nothing of the attention arithmetic itself, so neither side can borrow the
other's math through it.

Workloads follow the context-parallel pages ("Paralelismo de contexto",
diffusers v0.43.0): FLUX.1-dev at 1024x1024 has 4096 image tokens plus 512
text tokens, 24 heads of dimension 128 (FLUX's attention shape; the pages name
the model, not its internals). Values are i.i.d. N(0, 1) in float32 and, for
bfloat16 workloads, rounded to bfloat16 (round-to-nearest-even) before either
side sees them, so the oracle and the GPU consume bit-identical values.

Seeds: ``numpy.random.default_rng(42 + index)``; 42 is the seed the pages'
example script gives its generator. Draw order: Q_local, then K, then V, each
``standard_normal(shape, dtype=float32)``. The backward's output gradient dO
is drawn by ``grad_out`` from its own generator (seed + 1000), float32 N(0, 1)
and not rounded (the loss gradient arrives in float32). Q_local is drawn directly at its
local shape ``[B, Sq, H, D]`` (one rank's slice); K and V are drawn at
``[B, sum(block_lens), H, D]`` and ring block i is the contiguous token range
``[off_i, off_i + L_i)``. The Ulysses Anything workload draws Q, K and V
for the whole sequence ``[B, Sq, H, D]``; rank r's shard is its token range
(``split_lengths``), head group g its share of the heads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    ``block_lens`` are the ring K/V block lengths (ring_degree entries) as the
    attention sees them. For a Ulysses workload (``ulysses_degree = P > 1``)
    the drawn Q is one rank's sequence shard ``[B, S_local, H, D]`` and K/V
    hold the ring ranks' shards back to back, ``[B, ring_degree * S_local, H,
    D]``; after the local head/token regroup of each shard the attention runs
    with ``H / P`` heads, ``P * S_local`` queries and one block of
    ``P * S_local`` keys per ring rank (ring_degree 1: plain Ulysses; more:
    Unified attention).
    """

    index: int
    name: str
    dtype: str  # "f32" or "bf16"
    B: int
    H: int
    D: int
    Sq: int
    block_lens: tuple
    ulysses_degree: int = 1
    S_local: int = 0  # Ulysses: tokens per rank before the regroup (Ulysses Anything: rank 0's)
    anything: bool = False  # Ulysses Anything: uneven sequence and head splits over the ranks

    @property
    def seed(self) -> int:
        return 42 + self.index

    @property
    def ring_degree(self) -> int:
        return len(self.block_lens)

    @property
    def Skv(self) -> int:
        return int(sum(self.block_lens))

    @property
    def attn_H(self) -> int:
        """Heads seen by the attention kernel (after any Ulysses regroup; rank 0's group)."""
        if self.anything:
            return self.head_counts[0]
        return self.H // self.ulysses_degree

    @property
    def seq_counts(self) -> List[int]:
        """Ulysses Anything: tokens per rank (the whole sequence is Sq)."""
        return split_lengths(self.Sq, self.ulysses_degree)

    @property
    def head_counts(self) -> List[int]:
        """Ulysses Anything: heads per rank's group."""
        return split_lengths(self.H, self.ulysses_degree)

    @property
    def flops(self) -> int:
        """Algorithmic flops of the attention: 4 * B * H * Sq * Skv * D."""
        return 4 * self.B * self.attn_H * self.Sq * self.Skv * self.D

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS: List[Workload] = [
    Workload(0, "tiny_ring4_f32", "f32", B=1, H=2, D=64, Sq=64, block_lens=(64, 64, 64, 64)),
    Workload(1, "flux1024_ring2_bf16", "bf16", B=1, H=24, D=128, Sq=2304, block_lens=(2304, 2304)),
    Workload(2, "flux1024_ulysses2_bf16", "bf16", B=1, H=24, D=128, Sq=4608, block_lens=(4608,),
             ulysses_degree=2, S_local=2304),
    Workload(3, "video32k_ring4_bf16", "bf16", B=1, H=24, D=128, Sq=8192,
             block_lens=(8192, 8192, 8192, 8192)),
    Workload(4, "ring_anything3_uneven_bf16", "bf16", B=2, H=24, D=128, Sq=1536,
             block_lens=(1536, 1536, 1535)),
    # Unified attention, one rank of a 2 (Ulysses) x 2 (ring) grid on the FLUX
    # 1024px sequence: 1152 tokens per rank, 12 heads over 2304 queries after
    # the regroup, two ring blocks of 2304 keys.
    Workload(5, "flux1024_usp_u2r2_bf16", "bf16", B=1, H=24, D=128, Sq=2304, block_lens=(2304, 2304),
             ulysses_degree=2, S_local=1152),
    # Ulysses Anything, rank 0 of 4 on FLUX at 1008x1008: 63*63 image + 512
    # text = 4481 tokens (1121, 1120, 1120, 1120 per rank), 6 heads per rank
    # after the exchange, attention over all 4481 tokens.
    Workload(6, "flux1008_ulysses_anything4_bf16", "bf16", B=1, H=24, D=128, Sq=4481, block_lens=(4481,),
             ulysses_degree=4, S_local=1121, anything=True),
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def split_lengths(total: int, parts: int) -> List[int]:
    """Uneven split rule: the first ``total % parts`` blocks get one extra token.

    The pages only say each rank pads to the longest local length; this rule
    reproduces the 1536/1536/1535 split of a 4607-token sequence over 3 ranks.
    """
    base, extra = divmod(total, parts)
    return [base + (1 if i < extra else 0) for i in range(parts)]


def block_offsets(lens: Sequence[int]) -> List[int]:
    offs, acc = [], 0
    for L in lens:
        offs.append(acc)
        acc += int(L)
    return offs


# ---------------------------------------------------------------- bfloat16 ---

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the workloads are finite normal draws).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


# ------------------------------------------------------------------ inputs ---

@dataclasses.dataclass
class Inputs:
    """float32 arrays holding exactly the values the kernels consume."""

    q: np.ndarray  # [B, Sq, H, D]   (Ulysses: [B, S_local, H, D] before regroup)
    k: np.ndarray  # [B, Skv, H, D]  (Ulysses: [B, ring_degree * S_local, H, D])
    v: np.ndarray
    workload: Workload

    def k_shard(self, r: int) -> np.ndarray:
        """Ulysses: ring rank r's K shard [B, S_local, H, D], before its regroup."""
        S_l = self.workload.S_local
        return self.k[:, r * S_l:(r + 1) * S_l]

    def v_shard(self, r: int) -> np.ndarray:
        S_l = self.workload.S_local
        return self.v[:, r * S_l:(r + 1) * S_l]

    def k_block(self, i: int) -> np.ndarray:
        offs = block_offsets(self.workload.block_lens)
        return self.k[:, offs[i]:offs[i] + self.workload.block_lens[i]]

    def v_block(self, i: int) -> np.ndarray:
        offs = block_offsets(self.workload.block_lens)
        return self.v[:, offs[i]:offs[i] + self.workload.block_lens[i]]


def draw(shape, rng: np.random.Generator, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        x = round_to_bf16(x)
    return x


def make_inputs(w: Workload, q_scale: float = 1.0) -> Inputs:
    """Seeded inputs of workload ``w`` (see the module docstring for the recipe).

    ``q_scale`` multiplies Q before rounding (a stress variant that widens the
    softmax's dynamic range); 1.0 is the standard recipe.
    """
    rng = np.random.default_rng(w.seed)
    if w.anything:
        # every rank's shards: rank r holds tokens [off_r, off_r + S_r) of each
        shp = (w.B, w.Sq, w.H, w.D)
        q = rng.standard_normal(shp, dtype=np.float32)
        k = rng.standard_normal(shp, dtype=np.float32)
        v = rng.standard_normal(shp, dtype=np.float32)
    elif w.ulysses_degree > 1:
        q = rng.standard_normal((w.B, w.S_local, w.H, w.D), dtype=np.float32)
        shp = (w.B, w.ring_degree * w.S_local, w.H, w.D)
        k = rng.standard_normal(shp, dtype=np.float32)
        v = rng.standard_normal(shp, dtype=np.float32)
    else:
        q = rng.standard_normal((w.B, w.Sq, w.H, w.D), dtype=np.float32)
        k = rng.standard_normal((w.B, w.Skv, w.H, w.D), dtype=np.float32)
        v = rng.standard_normal((w.B, w.Skv, w.H, w.D), dtype=np.float32)
    if q_scale != 1.0:
        q = (q * np.float32(q_scale)).astype(np.float32)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return Inputs(q=q, k=k, v=v, workload=w)


def make_custom(B: int, H: int, D: int, Sq: int, block_lens: Sequence[int], dtype: str,
                seed: int, q_scale: float = 1.0) -> Inputs:
    """Inputs for an ad-hoc shape (parity sweeps), same recipe, explicit seed."""
    w = Workload(-1, f"custom_B{B}_H{H}_D{D}_Sq{Sq}_{'-'.join(map(str, block_lens))}_{dtype}",
                 dtype, B=B, H=H, D=D, Sq=Sq, block_lens=tuple(int(x) for x in block_lens))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, D), dtype=np.float32)
    k = rng.standard_normal((B, w.Skv, H, D), dtype=np.float32)
    v = rng.standard_normal((B, w.Skv, H, D), dtype=np.float32)
    if q_scale != 1.0:
        q = (q * np.float32(q_scale)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return Inputs(q=q, k=k, v=v, workload=w)


def grad_out(shape, seed: int) -> np.ndarray:
    """dL/dO for the backward: float32 N(0, 1) of ``shape`` from ``default_rng(seed + 1000)``."""
    return np.random.default_rng(seed + 1000).standard_normal(tuple(shape), dtype=np.float32)


def sample_rows(n_rows: int, n_samples: int, seed: int, must: Optional[Sequence[int]] = None) -> np.ndarray:
    """Sorted, distinct row indices for sampled parity checks at full size.

    Always includes the first and last row and any ``must`` rows (tile edges).
    """
    rng = np.random.default_rng(seed)
    pick = set(int(x) for x in rng.choice(n_rows, size=min(n_samples, n_rows), replace=False))
    pick.update({0, n_rows - 1})
    if must:
        pick.update(int(m) for m in must if 0 <= m < n_rows)
    return np.array(sorted(pick), dtype=np.int64)
