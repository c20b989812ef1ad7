// Internal launch interface between the C-ABI layer (api.hip) and the gfx950
// kernels. Arguments reaching these launchers have been validated already.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// Element strides of a [B, S, H, D] tensor (D is unit-stride).
struct Strides {
  int64_t b, s, h;
};

// Unsigned 32-bit division by a divisor fixed at launch, as a multiply-high,
// an add and two shifts (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994, the round-up multiplier with an extra
// add for the 33-bit case): for l = ceil(log2 d),
//   m = floor(2^32 (2^l - d) / d) + 1,  t = mulhi(n, m),
//   n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0)   for all n < 2^32.
struct FastDiv {
  uint32_t d, m, s1, s2;
  FastDiv() = default;
  explicit FastDiv(uint32_t div) : d(div) {
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < div) ++l;
    m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - div)) / div + 1);
    s1 = l < 1 ? l : 1;
    s2 = l > 1 ? l - 1 : 0;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t t = __umulhi(n, m);
    return (t + ((n - t) >> s1)) >> s2;
  }
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  float* lse;
  Strides qs, kvs, os;
  int B, H, D, Sq, Skv;
  float scale;
  bool accumulate;  // merge into (out, lse) instead of overwriting
  int waves;        // bf16 workgroup shape: 4, 8, or 0 to choose per launch
  bool v_packed;    // bf16: v is the output of launch_pack_v for this block (kvs is K's)
  // bf16 ring calls given a workspace: its count of merge waits that gave up. The
  // parallel-partials launch resets it with its own reset kernel; the other
  // launches set it to 0 from their first workgroup, so that it always
  // describes the last call that used the workspace.
  int* err = nullptr;
};

// V of one bf16 block rewritten in the tile / fragment order that the
// attention kernel reads with v_packed (ceil(Skv / 64) * 64 keys per (b, h),
// zeros past Skv); packed_v_bytes is its size. Keys come in Skv / piece
// pieces: key j of head h is read at (j % piece) * vs.s + ((j / piece) * H
// + h) * vs.h -- piece = Skv for a plain [B, Skv, H, D] tensor; for the
// Ulysses regroup fused in, vs describes the sequence-sharded tensor, H is
// the group's head count and piece = S_local.
int64_t packed_v_bytes(int B, int H, int D, int Skv);
hipError_t launch_pack_v(const void* v, Strides vs, void* packed, int B, int H, int D, int Skv, int piece,
                         hipStream_t stream);

// Backward of one ring block (bf16 inputs): dQ (+)= scale dS K, dK = scale dS^T Q,
// dV = P^T dO with P from the global LSE and dS = P (dO V^T - delta).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout_b;  // dO rounded to bf16, contiguous [B, Sq, H, D]
  const float* lse;    // [B, H, Sq], natural log, full-ring
  const float* delta;  // [B, H, Sq], rowsum(dO * O)
  float* dq;
  float* dk;
  float* dv;
  Strides qs, kvs, dqs, dkvs;
  int B, H, D, Sq, Skv;
  float scale;
  bool accumulate_dq;
  // Stream of the dq kernel (nullptr: the launch stream). The dq and dkv
  // kernels of a block read the same inputs and write disjoint outputs, so
  // they may run concurrently; the caller orders dq_stream against stream.
  hipStream_t dq_stream;
};
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream);

// The backward of 2..kMaxBwdBlocks non-empty blocks of a ring in two
// launches: dQ with every workgroup taking its query tile through the blocks
// in turn (accumulated in registers, written once: a.accumulate_dq must be
// false), and dK, dV of every block in one grid. a.k, a.v, a.dk, a.dv and
// a.Skv are not used; a.kvs / a.dkvs are the blocks' shared strides.
constexpr int kMaxBwdBlocks = 16;
struct BwdBlocks {
  int n;
  const void* const* k;
  const void* const* v;
  float* const* dk;
  float* const* dv;
  const int* len;  // each >= 1
};
hipError_t launch_attn_bwd_ring_bf16(const BwdArgs& a, const BwdBlocks& bb, hipStream_t stream);
// delta = rowsum(dO * O) and dO rounded to bf16 (contiguous [B, Sq, H, D]).
hipError_t launch_attn_bwd_prep(const float* out, Strides os, const float* dout, Strides ds, void* dout_b,
                                float* delta, int B, int H, int Sq, int D, hipStream_t stream);

// Partial attention of Q against one K/V block (Skv >= 1), float32 out + LSE.
hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream);
// Workgroup shape (waves: 4, or 8 for the ping-pong kernel) the bf16 launch uses for a.
int pick_waves(const FwdArgs& a);

// One launch for all the (non-empty) blocks of a ring, bf16, D = 128, packed V: the
// blocks' partials are computed in parallel and merged into (out, lse) in
// block order, each query tile's merges ordered through a flag. ws is caller
// memory, 4-byte aligned: ws[0] counts the merge waits that gave up (their
// tiles are set to NaN), ws[kRingFlagOffset ..] holds ring_flag_count flags;
// both are reset by the launch. a.k, a.v, a.Skv and a.accumulate are not
// used; a.kvs is the blocks' shared stride triple and a.v_packed says whether
// every v[i] is packed.
struct RingBlocks {
  int n;
  const void* const* k;  // K of block i at its first key (kvs strides)
  const void* const* v;  // packed V buffer holding block i
  const int* len;        // keys of block i
  const int* vt0;        // block i's first tile in its packed buffer (0 unless part of a larger block)
  const int* vnt;        // tiles per (b, h) of that buffer
};
int ring_max_blocks();
int64_t ring_flag_count(int B, int H, int Sq);
constexpr int kRingFlagOffset = 64;  // ints before the first flag (256 bytes: the error count, padding)
hipError_t launch_ring_bf16(const FwdArgs& a, const RingBlocks& rb, int* ws, hipStream_t stream);
// One launch for 2..seq_max_blocks() non-empty blocks (bf16, D = 128, packed V,
// 8-wave shape): each workgroup takes its query tile through the blocks in
// turn, block 0 written and later blocks merged in its epilogue (the
// per-block launches' arithmetic in the same order: the same bits). No
// flags; a.k, a.v, a.Skv, a.accumulate unused. seq_max_blocks() is 0 when the
// library is built without it.
int seq_max_blocks();
hipError_t launch_ring_seq_bf16(const FwdArgs& a, const RingBlocks& rb, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream);

// One launch for a ring of 2..kMaxF32RingBlocks non-empty float32 blocks
// (rb.vt0 / rb.vnt unused; a.k, a.v, a.Skv and a.accumulate not used): each
// workgroup computes every block's partial for its query rows and merges them
// in block order into (out, lse), which are overwritten.
constexpr int kMaxF32RingBlocks = 4;
hipError_t launch_ring_f32(const FwdArgs& a, const RingBlocks& rb, hipStream_t stream);

// out = 0, lse = -inf for every (b, s, h): attention over an empty key set.
hipError_t launch_fill_empty(float* out, Strides os, float* lse, int B, int H, int Sq, int D,
                             hipStream_t stream);

// (out_acc, lse_acc) <- (out_acc, lse_acc) (+) (out_blk, lse_blk).
hipError_t launch_lse_merge(float* out_acc, float* lse_acc, const float* out_blk,
                            const float* lse_blk, Strides as, Strides bs, int B, int H, int Sq,
                            int D, hipStream_t stream);

// Largest degree of the uneven Ulysses packs (per-piece tables travel in the kernel arguments).
constexpr int kMaxUlyssesDegree = 64;

// Uneven split of a [B, M, units_per_row] tensor (units of unit_bytes) along
// M (axis 1, seg_units in rows) or along a row (axis 2, seg_units in units)
// into P pieces back to back; to_pieces selects the direction. The caller
// guarantees fewer than 2^31 words and unit_bytes a multiple of 2.
hipError_t launch_pieces(const void* in, void* out, int axis, int64_t B, int64_t M, int64_t unit_bytes,
                         int64_t units_per_row, const int* seg_units, int P, int to_pieces, hipStream_t stream);

// Ulysses regroup bit copy of n (1..kMaxRegroupTensors) tensors of one shape in
// one launch; see cp_ulysses_regroup and cp_ulysses_regroup_multi.
constexpr int kMaxRegroupTensors = 8;
hipError_t launch_regroup(const void* const* in, void* const* out, int n, int elem_bytes, int B, int S_local,
                          int H, int D, int degree, int direction, hipStream_t stream);

}  // namespace cpattn
