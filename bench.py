#!/usr/bin/env python3
"""Benchmark: one rank's share of ring-block attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: for a ring workload, attention of the local Q
against every K/V block with each float32 partial merged by LSE rescaling
(cp_ring_attention); for the Ulysses workloads, the head/token regroup of Q,
K and V, attention over all tokens for the local heads, and the inverse
regroup of the output (Ulysses Anything: the uneven head-group packs around
the two exchanges, which are outside the step).

bf16 workloads whose block kernel runs its 8-wave shape (cp_attn_fwd_waves)
pass V to the attention kernel packed (cp_attn_pack_v), and the
step includes the packing a rank does itself: a ring rank packs its own V block
(the other ranks' blocks arrive packed by their owners, so they are packed once
at setup, as the peers would have done); a Ulysses rank packs the V it received
(its regrouped V), a pass of its own after the regroup, as it would be after a
real exchange (cp_ulysses_regroup_pack_v, which fuses the two on one GPU, would
skip the send buffer a real all-to-all needs). ``--unpacked-v`` runs the same
step with V as [B, S, H, D].

Prints ONE JSON line on stdout. ``value`` is attention TFLOP/s over the whole
step, counting 4*B*H*Sq*Skv*D flops; ``roofline`` prices the dominant kernel
(block attention) from its per-launch duration measured with HIP events on
the launch stream; ``cpu_baseline`` times the float64 CPU oracle on a bounded
sample of the same workload on this host. ``backward`` times the ring
share's backward (bf16 workloads) on the same inputs, outside the step.

Before the W warm-up steps, untimed steps run for --prewarm-seconds (default
1 s) so that the K timed steps see the clock the GPU holds under sustained
load rather than its ramp; the JSON line reports how many ran.

``--graph`` captures the K timed steps into one HIP graph and times its
replay: for launch-bound workloads (the tiny float32 ring) the host's
enqueue rate, not the GPU, otherwise sets the step time.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-seconds S] [--graph] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "ring-block attention TFLOP/s (fwd+LSE merge) and % of MI355X bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA bf16; fp32 vector ALU
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "flux1024_ulysses2_bf16"
# Block kernels timed in the same run besides the step's own workload (roofline only).
EXTRA_ROOFLINES = ("video32k_ring4_bf16",)
NOMINAL_CLOCK_MHZ = 2400.0  # the clock the dense peaks are quoted at


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-seconds", type=float, default=1.0,
                    help="untimed steps run for this long before the warm-up steps, so that the timed "
                         "steps see the clock the GPU settles at under sustained load (0 disables it)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=[w.name for w in workloads.WORKLOADS])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time for the oracle baseline sample (0 disables it)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps into one HIP graph and time its replay (launch-bound "
                         "workloads: the host no longer enqueues each launch)")
    ap.add_argument("--unpacked-v", action="store_true",
                    help="pass V as [B, S, H, D] instead of packed (bf16 workloads)")
    ap.add_argument("--separate-merge", action="store_true",
                    help="merge partials with the standalone merge kernel instead of the fused epilogue")
    ap.add_argument("--extra", default=",".join(EXTRA_ROOFLINES),
                    help="comma-separated workloads whose block kernel is also timed (roofline_extra); '' for none")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward")
    ap.add_argument("--no-hbm", action="store_true", help="skip the cold-cache HBM kernels")
    ap.add_argument("--phase-trace", action="store_true",
                    help="instead of the benchmark: load the diagnostic library (libcpattn_phase.so) and "
                         "print the core-clock cycles of the block kernel's tile-loop intervals for the "
                         "workload's one-block launch (8-wave shape), and those of a synthetic ping-pong "
                         "with the loop's instruction mix")
    return ap.parse_args()


def clock_beside(run_once, cycles: int = 40_000_000):
    """Shader clock (MHz) while `run_once` keeps the GPU busy: a one-thread kernel that spins for
    `cycles` of the shader clock (torch.cuda._sleep counts s_memtime, the shader-clock counter)
    runs on a second stream (default priority) while the launches repeat on the current one; its
    duration between two HIP events gives the clock. It needs a free compute unit to start on:
    where every unit is busy it starts when one frees, which the long spin makes a few percent
    at most. None if torch lacks the spin kernel."""
    import torch
    if not hasattr(torch.cuda, "_sleep"):
        return None
    side = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    run_once()
    with torch.cuda.stream(side):
        e0.record(side)
        torch.cuda._sleep(cycles)
        e1.record(side)
    t0 = time.perf_counter()
    while not e1.query() and time.perf_counter() - t0 < 10.0:
        for _ in range(4):
            run_once()
    torch.cuda.synchronize()
    return cycles / (e0.elapsed_time(e1) * 1e3)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


class Problem:
    """Device-resident inputs and outputs of one workload, and its step."""

    def __init__(self, w: workloads.Workload, separate_merge: bool, packed_v: bool = True):
        import torch
        import context_attention_dits_amd as cp
        self.cp, self.torch, self.w = cp, torch, w
        inp = workloads.make_inputs(w)
        self.inp = inp
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        to = lambda x: torch.from_numpy(x).to(tdt).cuda()  # noqa: E731
        self.q, self.k, self.v = to(inp.q), to(inp.k), to(inp.v)
        B, D = w.B, w.D
        self.flags = cp.CP_RING_SEPARATE_MERGE if separate_merge else 0
        if len(set(w.block_lens)) > 1:
            self.flags |= cp.CP_RING_ANYTHING
        if w.anything:
            self._setup_anything(tdt)
        elif w.ulysses_degree > 1:
            # This rank regroups its own Q/K/V shard every step; the other ring
            # ranks' blocks arrive already regrouped (they are regrouped once,
            # here, as the peers would have done).
            P, S_l = w.ulysses_degree, w.S_local
            shp = (B, P * S_l, w.H // P, D)
            self.qr = torch.empty(shp, dtype=tdt, device="cuda")
            self.k_own = self.k[:, :S_l].contiguous()
            self.v_own = self.v[:, :S_l].contiguous()
            self.kb = [torch.empty(shp, dtype=tdt, device="cuda") for _ in range(w.ring_degree)]
            self.vb = [torch.empty(shp, dtype=tdt, device="cuda") for _ in range(w.ring_degree)]
            for r in range(1, w.ring_degree):
                cp.cp_ulysses_regroup(self.k[:, r * S_l:(r + 1) * S_l].contiguous(), self.kb[r], P,
                                      cp.CP_REGROUP_SEQ_TO_HEAD)
                cp.cp_ulysses_regroup(self.v[:, r * S_l:(r + 1) * S_l].contiguous(), self.vb[r], P,
                                      cp.CP_REGROUP_SEQ_TO_HEAD)
            # this rank's own block, regrouped once here too (the backward reads it unpacked)
            cp.cp_ulysses_regroup(self.v_own, self.vb[0], P, cp.CP_REGROUP_SEQ_TO_HEAD)
            self.back = torch.empty((B, S_l, w.H, D), dtype=torch.float32, device="cuda")
            self.q_att = self.qr
        else:
            self.q_att = self.q
            offs = workloads.block_offsets(w.block_lens)
            self.kb = [self.k[:, o:o + L] for o, L in zip(offs, w.block_lens)]
            self.vb = [self.v[:, o:o + L] for o, L in zip(offs, w.block_lens)]
        H = w.attn_H
        # V as the attention kernel reads it: block 0 (this rank's own block, or the V it received)
        # is packed in every step, the others once here
        # (where the block kernel runs its 8-wave shape, or the packed ring runs as one launch;
        # the 4-wave kernel on its own gains nothing from it)
        lens = [kb.shape[1] for kb in self.kb]
        self.packed = bool(packed_v and w.dtype == "bf16" and (
            cp.cp_attn_fwd_waves(B, H, D, w.Sq) == 8
            or cp.cp_ring_attention_one_launch(cp.CP_BF16, B, H, D, w.Sq, lens)))
        self.vb_att = list(self.vb)
        if self.packed:
            self.vb_att = [cp.pack_v(x) for x in self.vb]
            torch.cuda.synchronize()
        self.out = torch.empty((B, w.Sq, H, D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B, H, w.Sq), dtype=torch.float32, device="cuda")
        # with packed V the workspace also lets the ring run as one launch
        nbytes = cp.cp_ring_attention_workspace_size(B, H, w.Sq, D,
                                                     self.flags | (cp.CP_RING_PACKED_V if self.packed else 0))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None

    def _setup_anything(self, tdt):
        """Ulysses Anything, rank 0 of the group. The step packs this rank's Q/K/V shards by head
        group (the first exchange's send buffers), attends over every token of its head group and
        unpacks the output pieces of the second exchange into [B, S_0, H, D]. The exchanges are
        outside the step: their receive buffers are filled here, once, with what every rank (this
        one included) sends; with B = 1 a receive buffer is already the [B, S, H_0, D] tensor and
        the send buffer of the second exchange is the output itself, so concat_seq is not needed."""
        torch, cp, w = self.torch, self.cp, self.w
        B, H, D, P = w.B, w.H, w.D, w.ulysses_degree
        assert B == 1
        seq, heads = w.seq_counts, w.head_counts
        offs = workloads.block_offsets(seq)
        self.seq, self.heads = seq, heads
        S0, H0 = seq[0], heads[0]
        own = [x[:, :S0].contiguous() for x in (self.q, self.k, self.v)]
        self.own = own
        self.send = [torch.empty(x.numel(), dtype=tdt, device="cuda") for x in own]
        recv = []
        for x in (self.q, self.k, self.v):  # piece 0 of every rank r, back to back
            pieces = []
            for r in range(P):
                buf = torch.empty(B * seq[r] * H * D, dtype=tdt, device="cuda")
                cp.cp_ulysses_pack_heads(x[:, offs[r]:offs[r] + seq[r]].contiguous(), buf, heads)
                pieces.append(buf[:B * seq[r] * H0 * D])
            recv.append(torch.cat(pieces).view(B, w.Sq, H0, D))
        self.q_att, kfull, vfull = recv
        self.kb, self.vb = [kfull], [vfull]
        # second exchange: from each rank g, rank 0's tokens of head group g (the peers' outputs,
        # computed once here with the library itself)
        hoffs = workloads.block_offsets(heads)
        pieces2 = []
        for g in range(P):
            cols = slice(hoffs[g], hoffs[g] + heads[g])
            q_g = self.q[:, :, cols].contiguous()
            o_g, _ = cp.ring_attention(q_g, [self.k[:, :, cols].contiguous()], [self.v[:, :, cols].contiguous()],
                                       scale=w.scale)
            pieces2.append(o_g[:, :S0].contiguous().view(-1))
        self.recv2 = torch.cat(pieces2)
        self.back = torch.empty((B, S0, H, D), dtype=torch.float32, device="cuda")

    def step(self):
        cp, w = self.cp, self.w
        if w.anything:
            for x, buf in zip(self.own, self.send):
                cp.cp_ulysses_pack_heads(x, buf, self.heads, cp.CP_REGROUP_SEQ_TO_HEAD)
            if self.packed:
                cp.cp_attn_pack_v(self.vb[0], self.vb_att[0].data)
            cp.cp_ring_attention(self.q_att, self.kb, self.vb_att, self.out, self.lse, scale=w.scale,
                                 flags=self.flags, workspace=self.ws)
            cp.cp_ulysses_pack_heads(self.recv2, self.back, self.heads, cp.CP_REGROUP_HEAD_TO_SEQ)
            return
        if w.ulysses_degree > 1:
            # this rank's Q, K and V shards, regrouped by one launch
            cp.cp_ulysses_regroup_multi([self.q, self.k_own, self.v_own], [self.qr, self.kb[0], self.vb[0]],
                                        w.ulysses_degree, cp.CP_REGROUP_SEQ_TO_HEAD)
        if self.packed:
            cp.cp_attn_pack_v(self.vb[0], self.vb_att[0].data)
        cp.cp_ring_attention(self.q_att, self.kb, self.vb_att, self.out, self.lse, scale=w.scale,
                             flags=self.flags, workspace=self.ws)
        if w.ulysses_degree > 1:
            cp.cp_ulysses_regroup(self.out, self.back, w.ulysses_degree, cp.CP_REGROUP_HEAD_TO_SEQ)

    def _timed_passes(self, one_pass, reps: int, graph: bool) -> float:
        """ms for `reps` back-to-back calls of one_pass between two HIP events on the launch
        stream; with graph, the reps are captured as one HIP graph whose replay is timed."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        one_pass()
        torch.cuda.synchronize()
        g = None
        if graph:
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                one_pass()
            stream.wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    one_pass()
            g.replay()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if g is not None:
            g.replay()
        else:
            for _ in range(reps):
                one_pass()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def time_block_kernels(self, reps: int, graph: bool = False):
        """Average duration of one block-attention launch, as the ring issues them.

        Block 0 is written, later blocks are merged in by the kernel epilogue.
        The launches of `reps` ring passes run back to back between two HIP
        events on the stream they are launched on (with graph, captured as one
        HIP graph whose replay is timed); the mean is the region's time over
        the number of launches. Where the step runs the ring as one
        launch (packed V, cp_ring_attention_one_launch), that launch (and the
        flag reset before it) is what is timed, with the flops of all blocks; so
        too for a float32 ring of 2 to 4 non-empty blocks, which always runs as
        one launch.
        """
        cp, w = self.cp, self.w
        blocks = [(i, kb, vb) for i, (kb, vb) in enumerate(zip(self.kb, self.vb_att)) if kb.shape[1] > 0]
        lens = [kb.shape[1] for kb in self.kb]
        f32_one = (w.dtype == "f32" and not self.flags & cp.CP_RING_SEPARATE_MERGE
                   and 2 <= sum(1 for L in lens if L > 0) <= 4)
        if f32_one or (self.packed and self.ws is not None and cp.cp_ring_attention_one_launch(
                cp.CP_BF16, w.B, w.attn_H, w.D, w.Sq, lens)):
            # the step runs the whole ring as one launch (after a flag reset): time that
            def one_pass():
                cp.cp_ring_attention(self.q_att, self.kb, self.vb_att, self.out, self.lse, scale=w.scale,
                                     flags=self.flags, workspace=self.ws)

            ms = self._timed_passes(one_pass, reps, graph)
            self.block_launch = "one launch for all blocks"
            self.block_pass = one_pass
            return ms / reps, w.flops
        self.block_launch = "one launch per block"

        def one_pass():
            for i, kb, vb in blocks:
                cp.cp_attn_block_fwd(self.q_att, kb, vb, self.out, self.lse, scale=w.scale,
                                     flags=cp.CP_BLOCK_ACCUMULATE if i > 0 else 0)

        ms = self._timed_passes(one_pass, reps, graph)
        self.block_pass = one_pass
        flops = sum(4 * w.B * w.attn_H * w.Sq * kb.shape[1] * w.D for _, kb, _ in blocks) / len(blocks)
        return ms / (reps * len(blocks)), flops


    def time_backward(self, reps: int):
        """The ring share's backward (cp_ring_attention_bwd: prep, then the dq and dkv kernels per
        block) on this step's Q/K/V, its merged out/LSE and a seeded dO: mean time of `reps` passes
        run back to back between two HIP events, and the algorithmic flops of one pass,
        10*B*H*Sq*Skv*D (the products S = QK^T, dP = dO V^T, dV, dK and dQ)."""
        torch, cp, w = self.torch, self.cp, self.w
        B, H, D, Sq = w.B, w.attn_H, w.D, w.Sq
        self.step()  # out, lse of the forward
        do = torch.from_numpy(workloads.grad_out((B, Sq, H, D), w.seed)).cuda()
        lens = [kb.shape[1] for kb in self.kb]
        dq = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda")
        dk_all = torch.empty((B, sum(lens), H, D), dtype=torch.float32, device="cuda")
        dv_all = torch.empty_like(dk_all)
        offs = workloads.block_offsets(lens)
        dk = [dk_all[:, a:a + L] for a, L in zip(offs, lens)]
        dv = [dv_all[:, a:a + L] for a, L in zip(offs, lens)]
        ws = torch.empty(cp.cp_attn_bwd_workspace_size(B, H, Sq, D), dtype=torch.uint8, device="cuda")
        flags = cp.CP_RING_ANYTHING if (len(set(lens)) > 1 or 0 in lens) else 0

        def one_pass():
            cp.cp_ring_attention_bwd(self.q_att, self.kb, self.vb, self.out, self.lse, do, dq, dk, dv,
                                     scale=w.scale, flags=flags, workspace=ws)

        stream = torch.cuda.current_stream()
        one_pass()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            one_pass()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, 10 * B * H * Sq * sum(lens) * D


def time_hbm_kernels(reps: int = 5):
    """HBM rate of the bandwidth-bound kernels, cold caches.

    cp_lse_merge on the 32k-token ring-4 share (out [1, 8192, 24, 128] float32,
    in place); the Ulysses-2 share's regroup of its Q, K and V shards
    ([1, 2304, 24, 128] bf16 each -> [1, 4608, 12, 128]) as the step runs it
    (one cp_ulysses_regroup_multi launch) and as three cp_ulysses_regroup
    launches, and back to back over six sets of operands (the rate in a
    pipeline, launch latency hidden); cp_ulysses_regroup SEQ_TO_HEAD of a [1, 16384, 24, 128] bf16
    tensor at degree 2, cp_ulysses_pack_heads of the same tensor into uneven
    head groups (7, 6, 6, 5) and cp_attn_pack_v of it (as one V block of 16384
    keys). Before each timed launch a 512 MiB buffer is read so that neither L2
    nor the 256 MB Infinity Cache holds the operands; bytes are the algorithmic
    ones (every element read once, written once).
    """
    import torch
    import context_attention_dits_amd as cp
    stream = torch.cuda.current_stream()
    # Read, not written: dirty lines left by a writing flush would be written
    # back to HBM during the timed launch and slow it.
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def timed(fn):
        ms = []
        for _ in range(reps + 1):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return sum(ms[1:]) / reps

    out = {}

    def record(name, ms, nb, shape):
        gbs = nb / (ms * 1e-3) / 1e9
        out[name] = {"GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "us": round(ms * 1e3, 2),
                     "bytes": nb, "shape": shape}

    B, Sq, H, D = 1, 8192, 24, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    oa = torch.randn(B, Sq, H, D, device="cuda", generator=g)
    ob = torch.randn(B, Sq, H, D, device="cuda", generator=g)
    la = torch.randn(B, H, Sq, device="cuda", generator=g)
    lb = torch.randn(B, H, Sq, device="cuda", generator=g)
    record("lse_merge", timed(lambda: cp.cp_lse_merge(oa, la, ob, lb)),
           3 * 4 * B * Sq * H * D + 3 * 4 * B * H * Sq, "out [1,8192,24,128] f32 + lse, in place (32k ring-4 share)")
    del oa, ob, la, lb
    # the Ulysses-2 share's own regroup: Q, K, V shards [1, 2304, 24, 128] bf16
    S3, P = 2304, 2
    xs = [torch.randn(1, S3, H, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3)]
    ys = [torch.empty(1, P * S3, H // P, D, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    qkv_bytes = 3 * 2 * 2 * S3 * H * D
    record("ulysses_regroup_qkv", timed(lambda: cp.cp_ulysses_regroup_multi(xs, ys, P, cp.CP_REGROUP_SEQ_TO_HEAD)),
           qkv_bytes, "Q, K, V [1,2304,24,128] bf16 -> [1,4608,12,128], one launch (Ulysses-2 share)")

    def three():
        for x, y in zip(xs, ys):
            cp.cp_ulysses_regroup(x, y, P, cp.CP_REGROUP_SEQ_TO_HEAD)

    record("ulysses_regroup_qkv_3launch", timed(three), qkv_bytes,
           "Q, K, V [1,2304,24,128] bf16 -> [1,4608,12,128], one launch per tensor (Ulysses-2 share)")
    # back to back, as in a pipeline (the launch overlaps the previous kernel), over 6 sets of
    # operands (510 MB, twice the Infinity Cache) so that each launch reads uncached data
    sets = [([torch.randn(1, S3, H, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3)],
             [torch.empty(1, P * S3, H // P, D, dtype=torch.bfloat16, device="cuda") for _ in range(3)])
            for _ in range(6)]
    n_b2b = 60

    def b2b():
        for i in range(n_b2b):
            cp.cp_ulysses_regroup_multi(*sets[i % len(sets)], P, cp.CP_REGROUP_SEQ_TO_HEAD)

    record("ulysses_regroup_qkv_back_to_back", timed(b2b) / n_b2b, qkv_bytes,
           "Q, K, V [1,2304,24,128] bf16 -> [1,4608,12,128], one launch, 60 launches back to back over 6 "
           "operand sets (Ulysses-2 share)")
    del xs, ys, sets
    S_l = 16384
    x = torch.randn(B, S_l, H, D, device="cuda", generator=g).to(torch.bfloat16)
    y = torch.empty(B, P * S_l, H // P, D, dtype=torch.bfloat16, device="cuda")
    big = 2 * 2 * B * S_l * H * D
    record("ulysses_regroup", timed(lambda: cp.cp_ulysses_regroup(x, y, P, cp.CP_REGROUP_SEQ_TO_HEAD)), big,
           "[1,16384,24,128] bf16 -> [1,32768,12,128], degree 2")
    pieces = torch.empty(x.numel(), dtype=torch.bfloat16, device="cuda")
    record("ulysses_pack_heads",
           timed(lambda: cp.cp_ulysses_pack_heads(x, pieces, [7, 6, 6, 5], cp.CP_REGROUP_SEQ_TO_HEAD)), big,
           "[1,16384,24,128] bf16 -> pieces of 7, 6, 6, 5 heads")
    pv = torch.empty(cp.cp_attn_packed_v_bytes(B, H, D, S_l), dtype=torch.uint8, device="cuda")
    record("pack_v", timed(lambda: cp.cp_attn_pack_v(x, pv)), big, "V [1,16384,24,128] bf16 -> packed tiles")
    return out


def cpu_baseline(w: workloads.Workload, inp, target_s: float):
    """Time the float64 oracle on the same workload for about target_s of CPU work.

    Whole heads of the workload (all blocks, merged) are run through the oracle;
    if the full workload takes less than target_s it is repeated, otherwise a
    subset of heads is timed.
    """
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - threadpoolctl is optional
        cores = 1
    if w.anything:  # rank 0's head group over every token
        H0 = w.head_counts[0]
        q = inp.q[:, :, :H0]
        k_blocks, v_blocks = [inp.k[:, :, :H0]], [inp.v[:, :, :H0]]
    elif w.ulysses_degree > 1:
        P = w.ulysses_degree
        q = oracle.ulysses_regroup(inp.q, P)
        k_blocks = [oracle.ulysses_regroup(inp.k_shard(r), P) for r in range(w.ring_degree)]
        v_blocks = [oracle.ulysses_regroup(inp.v_shard(r), P) for r in range(w.ring_degree)]
    else:
        q = inp.q
        offs = workloads.block_offsets(w.block_lens)
        k_blocks = [inp.k[:, o:o + L] for o, L in zip(offs, w.block_lens)]
        v_blocks = [inp.v[:, o:o + L] for o, L in zip(offs, w.block_lens)]
    H = w.attn_H

    def run(h0, h1):
        kb = [x[:, :, h0:h1] for x in k_blocks]
        vb = [x[:, :, h0:h1] for x in v_blocks]
        t = time.perf_counter()
        oracle.ring_attention(q[:, :, h0:h1], kb, vb, w.scale)
        return time.perf_counter() - t

    t1 = run(0, 1)  # one head, to size the sample
    n_heads = int(max(1, min(H, math.floor(target_s / max(t1, 1e-6)))))
    passes, total = 0, 0.0
    while True:
        total += run(0, n_heads)
        passes += 1
        if n_heads < H or total >= 0.8 * target_s:
            break
    flops = 4 * w.B * n_heads * w.Sq * w.Skv * w.D * passes
    what = f"{n_heads} of {H} heads" if n_heads < H else f"all {H} heads x {passes} passes"
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{what}, B={w.B} Sq={w.Sq} Skv={w.Skv} (every block, merged), numpy float64, "
                      f"{total:.1f} s"}


def hbm_traffic(w: workloads.Workload):
    """HBM bytes per block-kernel launch from the committed counter summary.

    profiles/attn_fwd_bf16_traffic.json holds FETCH_SIZE/WRITE_SIZE of one
    launch (scaled by the same counters' reading for a copy of known size)
    together with the SHA-256 of the kernel source they were taken from; the
    figure is reported only while that source is unchanged.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fwd_bf16_traffic.json")
    src = os.path.join(ROOT, "context_attention_dits_amd", "csrc", "attn_fwd_bf16.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(w.name)
    if rec.get("kernel_source_sha256") != sha or not entry:
        return None
    return entry.get("hbm_bytes_per_launch")


def block_roofline(prob, reps: int, graph: bool):
    """The roofline entry of one workload's block kernel: HIP-event time per launch as the step
    launches it, TFLOP/s against the dense peak at the nominal clock, and the shader clock
    measured beside the same launches (clock_beside, a pass of its own after the timed one) with
    the fraction of the peak at that clock."""
    w = prob.w
    k_ms, k_flops = prob.time_block_kernels(reps, graph=graph)
    achieved = k_flops / (k_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    mhz = clock_beside(prob.block_pass)
    return {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(achieved, 2),
            "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": hbm_traffic(w),
            "kernel": "attn_fwd_bf16_kernel" if w.dtype == "bf16" else "attn_fwd_f32_kernel",
            "us_per_launch": round(k_ms * 1e3, 2), "flops_per_launch": k_flops, "launches": prob.block_launch,
            "clock_mhz": None if mhz is None else round(mhz, 1),
            "clock_method": "one-thread s_memtime spin on a second stream beside the same launches",
            "frac_at_clock": None if mhz is None else round(achieved / (peak * mhz / NOMINAL_CLOCK_MHZ), 4)}


PHASE_VALUES = 8  # per wave: [interval parity][work, wait at the barrier], interval count, unused


def phase_trace(prob, warm_seconds: float = 0.5) -> dict:
    """Cycle accounting of the block kernel's ping-pong tile loop (diagnostic library only).

    Every wave of the 8-wave one-block launch reads the core clock (s_memtime) before and after
    each workgroup barrier of its tile loop (the loop's first three barriers left out) and sums,
    per interval parity, the work up to the barrier's waits and the time in them (tile loads, LDS
    accesses, the other waves). Each reading is a scalar memory round trip the wave waits for, so
    the traced launch runs slower than the plain one and both sums include those trips. Group A
    (waves 0-3) runs its softmax in the odd intervals and its matrix-core half in the even ones,
    group B (waves 4-7) the other way round. Medians over the workgroups' waves, in cycles per
    interval, after `warm_seconds` of launches; one traced launch timed with HIP events."""
    import ctypes
    import numpy as np
    import torch
    cp, w = prob.cp, prob.w
    lib = ctypes.CDLL(cp._lib.library_path())
    if not hasattr(lib, "cp_debug_phase_trace"):
        raise SystemExit(f"{cp._lib.library_path()} is not the diagnostic build (no cp_debug_phase_trace)")
    lib.cp_debug_phase_trace.argtypes = [ctypes.c_void_p, ctypes.c_long]
    lib.cp_debug_phase_trace.restype = ctypes.c_int
    if w.dtype != "bf16" or len(prob.kb) != 1 or cp.cp_attn_fwd_waves(w.B, w.attn_H, w.D, w.Sq) != 8:
        raise SystemExit("the phase trace covers the bfloat16 one-block launch on the 8-wave shape")
    n_wg = -(-w.Sq // 256) * w.attn_H * w.B
    if n_wg > 1024:
        raise SystemExit(f"the diagnostic build records 1024 workgroups; this launch has {n_wg}")

    def once():
        cp.cp_attn_block_fwd(prob.q_att, prob.kb[0], prob.vb_att[0], prob.out, prob.lse, scale=w.scale)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_seconds:
        for _ in range(10):
            once()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    once()
    e1.record()
    torch.cuda.synchronize()
    n = n_wg * 8 * PHASE_VALUES
    buf = (ctypes.c_ulonglong * n)()
    st = lib.cp_debug_phase_trace(ctypes.addressof(buf), n)
    if st != 0:
        raise SystemExit(f"cp_debug_phase_trace failed ({st})")
    a = np.frombuffer(buf, dtype=np.uint64).reshape(n_wg, 8, PHASE_VALUES).astype(np.float64)
    count = a[:, :, 4]
    if not (count > 1).all():
        raise SystemExit("some waves recorded no intervals")
    per = a[:, :, :4].reshape(n_wg, 8, 2, 2) / (count[:, :, None, None] / 2)
    kinds = []
    for par, name, a_half, b_half in ((1, "A softmax / B matrix half", "softmax", "matrix half"),
                                      (0, "A matrix half / B softmax", "matrix half", "softmax")):
        x = per[:, :, par, :]
        grp = {}
        for g, ws, half in (("A", slice(0, 4), a_half), ("B", slice(4, 8), b_half)):
            med = np.median(x[:, ws, :].reshape(-1, 2), axis=0)
            grp[g] = {"half": half, "work": round(float(med[0])), "wait": round(float(med[1]))}
        kinds.append({"interval": name, "cycles": round(float(np.median(x.sum(axis=2)))), **grp})
    step = sum(k["cycles"] for k in kinds)
    return {"workload": w.name, "traced_launch_us": round(e0.elapsed_time(e1) * 1e3, 2), "workgroups": n_wg,
            "intervals_per_wave": int(np.median(count)), "cycles_per_step": step,
            "mfma_cycles_per_simd_step": 64 * 32, "intervals": kinds, "synthetic_mix": mix_probe(lib)}


MIX_VARIANTS = ("as_the_loop", "mfma_16x16x32", "fragments_in_registers", "groups_in_phase",
                "fragment_reads_only", "fragment_reads_only_all_waves", "8_reads_one_half_early",
                "16_reads_one_half_early")


def mix_probe(lib, iters: int = 4000) -> dict:
    """The diagnostic library's synthetic ping-pong (cp_debug_mix_probe): the tile loop's interval
    structure and instruction mix on random bf16 with no memory traffic, 8 waves on each of the 256
    compute units. Per variant, the mean core-clock cycles of one interval (one group's matrix half,
    the other's softmax half, one barrier) and the milliseconds of the timed launch of `iters`
    intervals. Variants: as the loop does it; the same flops as twice as many 16x16x32 MFMAs; the
    fragments taken from registers instead of LDS; both groups in the same phase; the matrix
    half's 32 LDS fragment reads alone (no MFMAs, the other group idle); those reads by all 8
    waves in every interval; as the loop with 8 or 16 of a matrix half's fragment reads issued
    during the wave's preceding softmax half (into registers the loop does not have to spare)."""
    import ctypes
    lib.cp_debug_mix_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]
    lib.cp_debug_mix_probe.restype = ctypes.c_int
    res = {}
    for v, name in enumerate(MIX_VARIANTS):
        cyc, ms = ctypes.c_double(), ctypes.c_double()
        st = lib.cp_debug_mix_probe(v, iters, ctypes.byref(cyc), ctypes.byref(ms))
        if st != 0:
            raise SystemExit(f"cp_debug_mix_probe({v}) failed ({st})")
        res[name] = {"cycles_per_interval": round(cyc.value, 1), "ms": round(ms.value, 3)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.phase_trace:
        # the diagnostic build, loaded before anything else loads the library
        from context_attention_dits_amd.build import PHASE_TRACE_LIB
        os.environ["CP_ATTN_LIBRARY"] = os.path.join(ROOT, "context_attention_dits_amd", PHASE_TRACE_LIB)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    w = workloads.by_name(args.workload)
    log(f"[bench] workload {w.name}: B={w.B} H={w.attn_H} D={w.D} Sq={w.Sq} blocks={list(w.block_lens)}")
    prob = Problem(w, args.separate_merge, packed_v=not args.unpacked_v)
    if args.phase_trace:
        print(json.dumps({"phase_trace": phase_trace(prob)}), flush=True)
        return 0

    # A burst of a few milliseconds runs on a GPU that is still changing its clock: the first
    # ~30 ms of steps of the FLUX ring-2 share take ~15% longer than later ones. Untimed steps
    # for prewarm_seconds first, then the warm-up steps, so the timed steps are steady-state.
    prewarm_steps, pw0 = 0, time.perf_counter()
    while time.perf_counter() - pw0 < args.prewarm_seconds:
        for _ in range(10):
            prob.step()
        prewarm_steps += 10
        torch.cuda.synchronize()
    prewarm_s = time.perf_counter() - pw0
    for _ in range(args.warmup):
        prob.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph = None
    if args.graph:
        # the library only enqueues kernels on the caller's stream: capture the K steps as
        # one graph (after a run on the capture stream), replay it once untimed
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            prob.step()
        stream.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                prob.step()
        graph.replay()
        torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            prob.step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    log(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall * 1e6 / args.steps:.1f} us/step)")
    tflops = w.flops / (ms_step * 1e-3) / 1e12

    peak = PEAK_TFLOPS[w.dtype]
    roofline = block_roofline(prob, max(5, min(args.steps, 200)), args.graph)
    log(f"[bench] block kernel: {roofline['us_per_launch']:.1f} us/launch, {roofline['achieved']:.1f} TFLOP/s "
        f"({roofline['frac']:.1%} of {peak}; clock {roofline['clock_mhz']} MHz, "
        f"{roofline['frac_at_clock']} of the peak at that clock)")
    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != w.name]:
        wx = workloads.by_name(name)
        px = Problem(wx, args.separate_merge, packed_v=not args.unpacked_v)
        for _ in range(10):
            px.step()
        torch.cuda.synchronize()
        rx = block_roofline(px, 30, args.graph)
        rx["workload"] = name
        extra[name] = rx
        log(f"[bench] {name} block kernel: {rx['us_per_launch']:.1f} us/launch, {rx['achieved']:.1f} TFLOP/s "
            f"({rx['frac']:.1%} of {PEAK_TFLOPS[wx.dtype]}; clock {rx['clock_mhz']} MHz)")
        del px
        torch.cuda.empty_cache()

    bwd = None
    if w.dtype == "bf16" and not args.no_backward:
        b_ms, b_flops = prob.time_backward(max(5, min(args.steps, 20)))
        b_tf = b_flops / (b_ms * 1e-3) / 1e12
        bwd = {"TFLOP/s": round(b_tf, 2), "frac": round(b_tf / PEAK_TFLOPS["bf16"], 4),
               "ms_per_pass": round(b_ms, 5), "flops_per_pass": b_flops,
               "counting": "10*B*H*Sq*Skv*D (S, dP, dV, dK, dQ products)",
               "kernels": "attn_bwd_prep_kernel, attn_bwd_dq_kernel, attn_bwd_dkv_kernel"}
        log(f"[bench] backward: {b_ms * 1e3:.1f} us/pass, {b_tf:.1f} TFLOP/s ({b_tf / PEAK_TFLOPS['bf16']:.1%} of bf16 peak)")

    hbm = {} if args.no_hbm else time_hbm_kernels()
    for name, r in hbm.items():
        log(f"[bench] {name}: {r['us']:.1f} us, {r['GB/s']:.0f} GB/s ({r['frac']:.1%} of {PEAK_HBM_GBS:.0f}), {r['shape']}")

    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(w, prob.inp, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads ({cpu['sample']})")

    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": {"seconds": round(prewarm_s, 3), "steps": prewarm_steps},
        "launch": "hip graph of the timed steps" if args.graph else "eager",
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) Q/K/V (bf16-rounded), FLUX-like shapes",
        "config": {"workload": w.name, "B": w.B, "H": w.attn_H, "D": w.D, "Sq": w.Sq,
                   "block_lens": list(w.block_lens), "ring_degree": w.ring_degree,
                   "ulysses_degree": w.ulysses_degree,
                   **({"seq_counts": w.seq_counts, "head_counts": w.head_counts} if w.anything else {}),
                   "merge": "separate" if args.separate_merge else "fused",
                   "v_layout": "packed" if prob.packed else "bshd",
                   "pct_of_bf16_peak": round(100 * tflops / PEAK_TFLOPS["bf16"], 2)},
        "roofline": roofline,
        "roofline_extra": extra,
        "cpu_baseline": cpu,
        "hbm_kernels": hbm,
        "backward": bwd,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
