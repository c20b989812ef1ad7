/*
 * cp_attn.h -- one rank's share of context-parallel attention on one AMD
 * Instinct MI355X (gfx950): blockwise non-causal softmax attention of a local
 * Q slice against ring K/V blocks, float32 partial outputs with their
 * log-sum-exp (LSE), the LSE merge of partials, and the Ulysses head/token
 * regroup as a local permutation.
 *
 * Sources (diffusers v0.43.0 documentation pages):
 *   [CP]  "Paralelismo de contexto" -- context-parallelism guide;
 *         sections "Atencao em Anel" (Ring Attention), "Atencao Ulysses",
 *         "Ring Anything Attention".
 *   [API] "Paralelismo" -- parallelism API reference; section
 *         "ContextParallelConfig" (ring_degree, ulysses_degree,
 *         convert_to_fp32, rotate_method, ring_anything).
 *
 * Conventions for every entry point:
 *   - Tensors are [B, S, H, D] with the D axis unit-stride. Strides are given
 *     as a host array int64_t[3] = {stride_b, stride_s, stride_h} in elements
 *     of the tensor's own dtype; NULL means contiguous [B, S, H, D].
 *   - LSE tensors are float32 [B, H, Sq], contiguous, natural log.
 *   - Device pointers must be 16-byte aligned and every stride times the
 *     element size must be a multiple of 16 bytes. The K/V sequence stride
 *     must not exceed 2^24 elements.
 *   - The caller allocates and owns every buffer (inputs, outputs and any
 *     workspace). The library keeps no pointer to them after a call returns
 *     and allocates no device memory. What it does own, created on first use
 *     and kept until the process ends: per device, one extra stream and two
 *     events used by the backward (see "Streams" at the backward entry
 *     points), and one process-wide mutex that serialises the backward's
 *     enqueueing of work on them. It holds no other state between calls:
 *     every choice of launch form is made from the call's own arguments.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     work on that stream and never synchronise the host (the one exception
 *     is cp_ring_attention_check, which says so); results are ready once the
 *     stream has reached that point.
 *   - Arguments are validated on the host before anything is enqueued. On
 *     error nothing is launched, a non-zero status is returned and
 *     cp_last_error() describes the problem. CP_ERR_HIP reports a failed
 *     launch.
 *   - Inputs and outputs must not overlap, except where an entry point says
 *     it updates a buffer in place.
 *   - Supported: dtype CP_BF16 or CP_F32 for Q/K/V, head dim D = 64 or 128.
 *     Outputs are always float32: the partial output and LSE are kept in
 *     float32 for a stable merge ([API] convert_to_fp32, default True).
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CP_ATTN_ABI_VERSION 2

typedef enum cp_status {
  CP_OK = 0,
  CP_ERR_INVALID_ARG = 1, /* bad pointer, size, stride or combination */
  CP_ERR_UNSUPPORTED = 2, /* valid request outside the supported set (dtype, D, alignment) */
  CP_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  CP_ERR_HIP = 4,         /* the HIP runtime reported an error at launch */
  CP_ERR_ORDER = 5        /* cp_ring_attention_check: a merge of a one-launch ring ran out of order */
} cp_status_t;

typedef enum cp_dtype { CP_F32 = 0, CP_BF16 = 1 } cp_dtype_t;

/* cp_attn_block_fwd flag: merge this block into (out, lse) instead of overwriting them. */
#define CP_BLOCK_ACCUMULATE 0x1u
/* cp_attn_block_fwd flag: v is this block's V as written by cp_attn_pack_v (CP_BF16 only). */
#define CP_BLOCK_PACKED_V 0x2u
/* cp_ring_attention flag: allow unequal block lengths, zero included ([CP] Ring Anything). */
#define CP_RING_ANYTHING 0x2u
/* cp_ring_attention flag: write each block's partial into the workspace and merge it with
 * a separate cp_lse_merge pass, instead of merging inside the attention kernel. */
#define CP_RING_SEPARATE_MERGE 0x4u
/* cp_ring_attention flag: every v_blocks[i] is block i's V as written by cp_attn_pack_v
 * (CP_BF16 only). */
#define CP_RING_PACKED_V 0x8u

/* cp_attn_block_fwd and cp_ring_attention flags: force the bf16 block kernel's workgroup shape
 * for this call (a property of this implementation, not of the pages): four waves and 128 query
 * rows per workgroup, or eight waves and 256 rows in two ping-pong groups. Without either the
 * shape is chosen per launch from the grid size (cp_attn_fwd_waves); head dim 64 always uses
 * four waves. Results agree to rounding either way. Setting both is CP_ERR_INVALID_ARG. */
#define CP_FWD_FOUR_WAVES 0x100u
#define CP_FWD_EIGHT_WAVES 0x200u

/* cp_attn_block_bwd flag: add this block's dQ to dq instead of overwriting it. */
#define CP_BWD_ACCUMULATE_DQ 0x1u

/* cp_ulysses_regroup directions. */
#define CP_REGROUP_SEQ_TO_HEAD 0 /* first all-to-all: [B, S_local, H, D] -> [B, P*S_local, H/P, D] */
#define CP_REGROUP_HEAD_TO_SEQ 1 /* second all-to-all: [B, P*S_local, H/P, D] -> [B, S_local, H, D] */

/*
 * cp_attn_block_fwd -- partial attention of the local Q against one K/V block.
 *
 * [CP] "Atencao em Anel": each GPU computes attention of its local Q against
 * the K/V block it holds; [API] ring_degree: attention between the local Q
 * and each K/V block passed around the ring; [API] convert_to_fp32: the
 * block's output and LSE are float32.
 *
 * For every (b, h) and query row i (non-causal, no mask):
 *   x_ij   = scale * <q_i, k_j>,  j = 0 .. Skv-1
 *   lse_i  = ln sum_j exp(x_ij)
 *   out_i  = sum_j exp(x_ij - lse_i) * v_j
 *
 *   q    [B, Sq, H, D]  dtype, strides q_strides
 *   k, v [B, Skv, H, D] dtype, shared strides kv_strides (a block of a
 *        larger resident buffer, e.g. a padded all-gather, is passed as a
 *        base pointer plus that buffer's strides; rows >= Skv are never read)
 *   out  [B, Sq, H, D]  float32, strides out_strides
 *   lse  [B, H, Sq]     float32, contiguous
 *   scale  > 0 and finite (the usual choice is 1/sqrt(D))
 *   flags  0, CP_BLOCK_ACCUMULATE, CP_BLOCK_PACKED_V or both. With
 *          CP_BLOCK_ACCUMULATE, (out, lse) must already hold a partial result
 *          of the same queries over other keys; they are updated in place to
 *          the merge of that partial with this block (the cp_lse_merge
 *          formula). With CP_BLOCK_PACKED_V (CP_BF16 only), v is the output
 *          of cp_attn_pack_v for this block's V (same B, H, D, Skv; the
 *          library cannot check its size) and kv_strides describe K only;
 *          the result is bit-identical to passing the unpacked V.
 *
 * Skv == 0 is allowed: without CP_BLOCK_ACCUMULATE it writes out = 0 and
 * lse = -inf (attention over no keys); with it, it leaves (out, lse) as they
 * are. B, H or Sq == 0 enqueues nothing.
 */
cp_status_t cp_attn_block_fwd(const void* q, const int64_t* q_strides,
                              const void* k, const void* v, const int64_t* kv_strides,
                              int dtype, int B, int H, int D, int Sq, int Skv, float scale,
                              unsigned flags, float* out, const int64_t* out_strides, float* lse,
                              void* stream);

/*
 * cp_lse_merge -- (out_acc, lse_acc) <- (out_acc, lse_acc) (+) (out_blk, lse_blk), in place.
 *
 * [API] convert_to_fp32 (partials kept in float32 for the ring's merge) and
 * [CP] "Atencao em Anel" (after a full loop every rank has seen every
 * token's K/V). The pages name the merged quantities but print no formula;
 * this is the exact recombination of two softmax partials over disjoint keys:
 *   M   = max(lse_a, lse_b),  w_a = exp(lse_a - M),  w_b = exp(lse_b - M)
 *   lse = M + ln(w_a + w_b),  out = (w_a*out_a + w_b*out_b) / (w_a + w_b)
 * A side with lse = -inf has weight 0; if both are -inf the result is
 * out = 0, lse = -inf.
 *
 *   out_acc, out_blk [B, Sq, H, D] float32 with strides acc_strides / blk_strides
 *   lse_acc, lse_blk [B, H, Sq]    float32, contiguous
 * out_blk/lse_blk are read only and must not overlap the accumulators.
 * B*Sq*H*D/4 must be below 2^31 (else CP_ERR_UNSUPPORTED).
 */
cp_status_t cp_lse_merge(float* out_acc, float* lse_acc, const float* out_blk, const float* lse_blk,
                         const int64_t* acc_strides, const int64_t* blk_strides,
                         int B, int H, int Sq, int D, void* stream);

/*
 * cp_ring_attention_workspace_size -- bytes of workspace cp_ring_attention
 * uses for these sizes and flags. With CP_RING_SEPARATE_MERGE: one float32
 * partial output [B, Sq, H, D] and its LSE (required). Otherwise, with
 * CP_RING_PACKED_V and D = 128: 256 bytes (a count of merge waits that gave
 * up, see cp_ring_attention_check) plus one int per 256-row query tile of
 * each (b, h), rounded up to 256 bytes (optional: with it, bf16 rings of
 * 2..16 non-empty blocks, or one block of two or more key tiles, on grids
 * the per-block launches would run on four waves run as one launch; without
 * it, as one launch per block or with the blocks in turn). Else 0.
 */
size_t cp_ring_attention_workspace_size(int B, int H, int Sq, int D, unsigned flags);

/*
 * cp_ring_attention -- one rank's share of Ring Attention, all K/V blocks resident.
 *
 * [CP] "Atencao em Anel" and [API] ring_degree / rotate_method: the local Q
 * attends to each of the ring_degree K/V blocks in turn (block 0 first) and
 * the float32 partials are merged by LSE rescaling; with all blocks present
 * after an all-gather (the only rotate method the pages support) the loop
 * runs locally. The result equals attention of Q over the concatenation of
 * all blocks.
 *
 *   k_blocks, v_blocks  host arrays of ring_degree device pointers; block i
 *                       is [B, block_len[i], H, D] with the shared kv_strides
 *   block_len           host array of ring_degree lengths
 *   ring_degree         >= 1
 *   flags               CP_RING_ANYTHING: lengths may differ and may be 0
 *                       ([CP] "Ring Anything Attention": each padded block
 *                       is cut back to its true length; pad rows are never
 *                       read). Without it every length must be equal and
 *                       >= 1 (plain ring attention needs the sequence to
 *                       divide evenly by ring_degree).
 *                       CP_RING_SEPARATE_MERGE: see above; needs workspace.
 *                       CP_RING_PACKED_V: v_blocks[i] is the output of
 *                       cp_attn_pack_v for block i (as CP_BLOCK_PACKED_V).
 *   out, lse            as cp_attn_block_fwd; overwritten.
 *   workspace           device buffer of workspace_bytes, 256-byte aligned,
 *                       at least cp_ring_attention_workspace_size(); may be
 *                       NULL unless CP_RING_SEPARATE_MERGE is set.
 *   flags also takes CP_FWD_FOUR_WAVES or CP_FWD_EIGHT_WAVES.
 * One launch for the whole ring (packed V with a workspace, bf16, D = 128,
 * 2 to 16 non-empty blocks, and a grid the per-block launches would run on
 * the 4-wave kernel; cp_ring_attention_one_launch says whether a call
 * qualifies, CP_ONE_LAUNCH_PARALLEL): the partials of all blocks are
 * computed in parallel, and each query tile's merges still run in block
 * order through the same epilogue arithmetic (ordered by per-tile flags in
 * the workspace with agent-scope acquire/release; cp_ring_attention_check
 * reports a wait that gave up), so the result is the same, bit for bit, as
 * one launch per block. A single non-empty block of at least 128 keys on such
 * a grid is split at a 64-key tile boundary into two halves run the same way
 * (two partials merged by their LSE: equal to one pass up to rounding). Calls
 * that share a workspace must not overlap.
 * Otherwise, with packed V on the 8-wave shape (cp_attn_fwd_waves), 2 to 16
 * non-empty blocks run as one launch without workspace in which each
 * workgroup takes its query tile through the blocks in order, writing block
 * 0's partial and merging the others in its epilogue: the same bits as one
 * launch per block.
 * CP_F32 with 2 to 4 non-empty blocks (and no CP_RING_SEPARATE_MERGE) also
 * runs as one launch, without workspace: each workgroup computes every
 * block's partial for its query rows and merges them in block order with the
 * same LSE arithmetic as the per-block launches.
 * If every block is empty the result is out = 0, lse = -inf.
 */
cp_status_t cp_ring_attention(const void* q, const int64_t* q_strides,
                              const void* const* k_blocks, const void* const* v_blocks,
                              const int64_t* kv_strides, const int* block_len, int ring_degree,
                              int dtype, int B, int H, int D, int Sq, float scale, unsigned flags,
                              float* out, const int64_t* out_strides, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * cp_attn_packed_v_bytes, cp_attn_pack_v -- V of one K/V block, rewritten in
 * the order the bf16 attention kernel's PV products read it.
 *
 * Not an operation of the pages: a layout change of the V operand of the
 * block attention above ([CP] "Atencao em Anel"), so that the kernel loads V
 * tiles straight into on-chip memory instead of transposing them on every
 * compute unit. In a ring, a rank would pack its own V block once and every
 * other rank would receive it packed; a block that is read by several
 * launches is packed once.
 *
 *   v       [B, Skv, H, D] bf16, strides v_strides (NULL = contiguous),
 *           16-byte aligned rows
 *   packed  device buffer of packed_bytes >= cp_attn_packed_v_bytes(B, H, D,
 *           Skv) = B * H * ceil(Skv / 64) * 64 * D * 2 bytes, 16-byte aligned,
 *           not overlapping v. Layout (the kernel's, opaque to callers): per
 *           (b, h) in (b, h) order, ceil(Skv / 64) tiles of 64 keys, each D/8
 *           fragments of 1 KB; fragment 4 db + 2 kb + kk2 of tile t holds, for
 *           lane l (l32 = l % 32, hi = l / 32) and element e < 8 (16 bytes per
 *           lane), V[b, key, h, 32 db + l32] with key = 64 t + 32 kb + 16 kk2
 *           + 8 (e / 4) + 4 hi + e % 4; keys >= Skv are 0.
 * D must be 64 or 128 (cp_attn_packed_v_bytes returns 0 otherwise);
 * B*H*ceil(Skv/64) must be below 2^31. Sizes of 0 enqueue nothing.
 */
size_t cp_attn_packed_v_bytes(int B, int H, int D, int Skv);
cp_status_t cp_attn_pack_v(const void* v, const int64_t* v_strides, int B, int H, int D, int Skv,
                           void* packed, size_t packed_bytes, void* stream);

/*
 * cp_ulysses_regroup_pack_v -- the Ulysses regroup of V and its packing in one pass.
 *
 * Writes into `packed` exactly what cp_ulysses_regroup(in, tmp, 2, B, S_local,
 * H, D, degree, CP_REGROUP_SEQ_TO_HEAD) followed by cp_attn_pack_v(tmp, NULL,
 * B, H / degree, D, degree * S_local, packed, ...) would, without the
 * intermediate tensor: [CP] "Atencao Ulysses" -- after the first all-to-all a
 * rank holds V of every token for its head group, which its attention then
 * reads. This fuses the loopback regroup (which stands in for the send buffer
 * of that exchange) with the packing, so it is for one-GPU use; across GPUs
 * the receiver packs what arrives with cp_attn_pack_v.
 * in is the sequence-sharded V [B, S_local, H, D] bf16, contiguous,
 * 16-byte aligned; degree >= 1 divides H; packed holds at least
 * cp_attn_packed_v_bytes(B, H / degree, D, degree * S_local) bytes, 16-byte
 * aligned, not overlapping in. D must be 64 or 128.
 */
cp_status_t cp_ulysses_regroup_pack_v(const void* in, int B, int S_local, int H, int D, int degree,
                                      void* packed, size_t packed_bytes, void* stream);

/* How cp_ring_attention, given these sizes, block lengths and flags with packed V
 * (CP_RING_PACKED_V) and a workspace of cp_ring_attention_workspace_size bytes, runs the ring:
 * 0 one launch per block, CP_ONE_LAUNCH_IN_TURN one launch with the blocks in turn per
 * workgroup, CP_ONE_LAUNCH_PARALLEL one launch with the blocks' partials in parallel (the form
 * whose merges wait on other workgroups; see cp_ring_attention_check). A caller that packs V
 * only for speed can use this and cp_attn_fwd_waves to decide whether to. */
#define CP_ONE_LAUNCH_IN_TURN 1
#define CP_ONE_LAUNCH_PARALLEL 2
int cp_ring_attention_one_launch(int dtype, int B, int H, int D, int Sq, const int* block_len, int ring_degree,
                                 unsigned flags);

/*
 * cp_ring_attention_check -- whether every merge of the last cp_ring_attention call that used
 * this workspace (packed V, bf16, D = 128) ran in order.
 *
 * In the parallel-partials form (CP_ONE_LAUNCH_PARALLEL) a merge waits, with a bounded number
 * of polls, for the previous block's workgroup to publish its partial. A wait
 * that gives up is counted in the workspace, and the query tile's out and lse are set to NaN
 * instead of merged, so a wrong result is never silent. This call waits for `stream` (it
 * synchronises the host with it), reads the count and returns CP_OK when it is 0, CP_ERR_ORDER
 * otherwise. Every cp_ring_attention call that is given such a workspace and runs a bf16 kernel
 * resets the count (the other forms have no waits and leave it 0).
 */
cp_status_t cp_ring_attention_check(const void* workspace, size_t workspace_bytes, void* stream);

/*
 * cp_ulysses_regroup -- the Ulysses all-to-all's local permutation, loopback.
 *
 * [CP] "Atencao Ulysses": the first all-to-all leaves each GPU with every
 * token for a subset of heads; the second regroups the results by token.
 * With the exchange replaced by a loopback, head group g (heads g*H/P ..
 * (g+1)*H/P - 1) of this rank's S_local tokens becomes token chunk g:
 *   SEQ_TO_HEAD: out[b, g*S_local + s, h, d] = in[b, s, g*(H/P) + h, d]
 *   HEAD_TO_SEQ: out[b, s, g*(H/P) + h, d] = in[b, g*S_local + s, h, d]
 * A bit copy: elem_bytes is 2 (bf16/fp16) or 4 (float32); contiguous tensors.
 * S_local and H always describe the sequence-sharded side [B, S_local, H, D];
 * degree is the Ulysses degree P >= 1 and must divide H ([CP]: the number of
 * heads must be divisible by ulysses_degree). in and out must not overlap.
 */
cp_status_t cp_ulysses_regroup(const void* in, void* out, int elem_bytes, int B, int S_local, int H,
                               int D, int degree, int direction, void* stream);

/*
 * cp_ulysses_regroup_multi -- cp_ulysses_regroup of n_tensors tensors of the
 * same shape in one launch.
 *
 * [CP] "Atencao Ulysses": the first all-to-all moves the query, key and value
 * projections together, so a rank regroups three tensors of one shape at a
 * time; one launch pays the start-up and drain of a bandwidth-bound pass once
 * instead of per tensor. in and out are host arrays of n_tensors (1..8)
 * device pointers; tensor i is regrouped from in[i] into out[i] exactly as
 * cp_ulysses_regroup would (same arguments and layouts). No output may
 * overlap any input or another output; inputs may coincide.
 */
cp_status_t cp_ulysses_regroup_multi(const void* const* in, void* const* out, int n_tensors, int elem_bytes, int B,
                                     int S_local, int H, int D, int degree, int direction, void* stream);

/*
 * Ulysses Anything: the packs around an all-to-all whose splits are uneven.
 *
 * [CP] "Ulysses Anything Attention" and [API] ulysses_anything: the sequence
 * length and the head count need not divide by ulysses_degree (FLUX at
 * 1008x1008, 4481 tokens over 4 GPUs). Rank r holds S_r tokens of every head;
 * head group g (head_counts[g] consecutive heads) goes to rank g. Around the
 * exchange (which is not part of this library) a rank runs:
 *   first all-to-all:  cp_ulysses_pack_heads  SEQ_TO_HEAD, exchange,
 *                      cp_ulysses_concat_seq  SEQ_TO_HEAD
 *   second all-to-all: cp_ulysses_concat_seq  HEAD_TO_SEQ, exchange,
 *                      cp_ulysses_pack_heads  HEAD_TO_SEQ
 * Both are bit-exact permutations of elem_bytes-sized elements (2 or 4).
 * Pieces lie back to back, each row-major, in rank order. degree is 1..64;
 * counts may hold zeros. Tensors must stay below 2^32 bytes; in and out
 * must not overlap. Zero-sized problems enqueue nothing.
 */

/*
 * cp_ulysses_pack_heads -- [B, S_r, H, D] <-> pieces [B, S_r, head_counts[g], D],
 * H = sum of head_counts.
 *   SEQ_TO_HEAD: in = the tensor, out = the pieces (the first exchange's send buffer)
 *   HEAD_TO_SEQ: in = the pieces (the second exchange's receive buffer, from
 *                rank g the tokens of this rank for head group g), out = the tensor
 */
cp_status_t cp_ulysses_pack_heads(const void* in, void* out, int elem_bytes, int B, int S_r, int D, int degree,
                                  const int* head_counts, int direction, void* stream);

/*
 * cp_ulysses_concat_seq -- pieces [B, seq_counts[r], H_g, D] <-> [B, S, H_g, D],
 * S = sum of seq_counts (every token of this rank's head group).
 *   SEQ_TO_HEAD: in = the pieces (the first exchange's receive buffer, rank r's
 *                tokens from rank r), out = the tensor
 *   HEAD_TO_SEQ: in = the tensor (this rank's output), out = the pieces (the
 *                second exchange's send buffer)
 * With B = 1 the two layouts coincide and the call is a plain copy.
 */
cp_status_t cp_ulysses_concat_seq(const void* in, void* out, int elem_bytes, int B, int H_g, int D, int degree,
                                  const int* seq_counts, int direction, void* stream);

/*
 * Backward of the ring share (bfloat16 Q/K/V, float32 gradients).
 *
 * [CP] the variants table that opens the page and the note under "Ring
 * Anything Attention" restrict only Ring Anything to inference; [API] the
 * introduction of "Paralelismo" names training as well as inference. So ring
 * attention's blocks also run backward. With O and LSE the merged forward
 * results over all blocks (cp_ring_attention's out and lse) and dO the loss
 * gradient with respect to O, for every (b, h):
 *   P_ij  = exp(scale <q_i, k_j> - lse_i)        (global softmax weights)
 *   D_i   = sum_d dO_id O_id
 *   dS_ij = P_ij (<dO_i, v_j> - D_i)
 *   dV_j  = sum_i P_ij dO_i
 *   dK_j  = scale sum_i dS_ij q_i
 *   dQ_i  = scale sum_j dS_ij k_j                (sum over every block's keys)
 * the derivative of softmax attention; per block, j runs over that block's
 * keys. The MFMA operands dO and P, dS are rounded to bfloat16, D_i, the
 * exponent and every accumulation are float32; D_i is summed from the same
 * bfloat16 dO the products use, so dP - D is exact for that dO (with one key,
 * P = 1 and O = v give dS = 0, as they should).
 *
 * Workspace (caller-owned, 256-byte aligned): dO rounded to bfloat16
 * ([B, Sq, H, D], contiguous) and D ([B, H, Sq] float32), written by
 * cp_attn_bwd_prep and read by cp_attn_block_bwd.
 *
 * Streams: where one launch of the dQ kernel or of the dK/dV kernel alone
 * would leave a quarter or more of the GPU's last round of workgroup slots
 * idle, cp_attn_block_bwd and cp_ring_attention_bwd run the dQ kernels on a
 * second stream that the library creates once per device (non-blocking,
 * default priority; never while the caller's stream is capturing a graph),
 * forked from the caller's stream by an event and joined back before the
 * call returns. The caller sees one stream-ordered operation on its stream,
 * also under graph capture; calls on one device from several host threads
 * are serialised while they enqueue. Under capture the second stream joins
 * the capturing graph until that capture ends; meanwhile a call whose stream
 * is not part of that same capture runs all its kernels on its own stream.
 */

/* Bytes of backward workspace for these sizes (0 if any size is <= 0). */
size_t cp_attn_bwd_workspace_size(int B, int H, int Sq, int D);

/*
 * cp_attn_bwd_prep -- fill the workspace from O and dO (once per backward,
 * before the blocks).
 *   out, dout  [B, Sq, H, D] float32, strides out_strides / dout_strides
 *   dtype      CP_BF16 (the dtype of the Q/K/V the blocks will use)
 * B*Sq*H*D/8 must be below 2^31. B, H or Sq == 0 enqueues nothing.
 */
cp_status_t cp_attn_bwd_prep(const float* out, const int64_t* out_strides, const float* dout,
                             const int64_t* dout_strides, int dtype, int B, int H, int Sq, int D,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * cp_attn_block_bwd -- gradients of one K/V block.
 *   q      [B, Sq, H, D] bfloat16, strides q_strides
 *   k, v   [B, Skv, H, D] bfloat16, shared strides kv_strides
 *   lse    [B, H, Sq] float32: the merged LSE over all blocks (not this
 *          block's own)
 *   workspace  as filled by cp_attn_bwd_prep for the same B, H, Sq, D
 *   dq     [B, Sq, H, D] float32, strides dq_strides: overwritten with this
 *          block's dQ, or, with CP_BWD_ACCUMULATE_DQ, added to in place
 *   dk, dv [B, Skv, H, D] float32, shared strides dkv_strides: overwritten
 * The sequence strides of q and k/v, and H*D, must not exceed 2^24 elements.
 * Skv == 0 writes dq = 0 (or leaves it with CP_BWD_ACCUMULATE_DQ); Sq == 0
 * writes dk = dv = 0 and needs no workspace (it may be NULL); B or H == 0
 * enqueues nothing. dtype CP_F32 is CP_ERR_UNSUPPORTED.
 */
cp_status_t cp_attn_block_bwd(const void* q, const int64_t* q_strides, const void* k, const void* v,
                              const int64_t* kv_strides, int dtype, int B, int H, int D, int Sq, int Skv,
                              float scale, unsigned flags, const float* lse, const void* workspace,
                              size_t workspace_bytes, float* dq, const int64_t* dq_strides, float* dk, float* dv,
                              const int64_t* dkv_strides, void* stream);

/*
 * cp_ring_attention_bwd -- backward of cp_ring_attention for one rank: the
 * prep, then every block in ring order; dQ is summed over the blocks.
 *   q, k_blocks, v_blocks, kv_strides, block_len, ring_degree, dtype, B, H,
 *   D, Sq, scale, flags (0 or CP_RING_ANYTHING)  as cp_ring_attention
 *   out, lse   the forward's merged output and LSE
 *   dout       [B, Sq, H, D] float32, strides dout_strides
 *   dq         [B, Sq, H, D] float32, overwritten
 *   dk_blocks, dv_blocks  ring_degree pointers to [B, block_len[i], H, D]
 *              float32 outputs (shared strides dkv_strides), overwritten;
 *              entries of empty blocks are not used
 *   workspace  cp_attn_bwd_workspace_size(B, H, Sq, D) bytes
 * If every block is empty, dq = 0.
 * Launch plan: where neither kernel's grid would leave a quarter of its last
 * round of workgroup slots idle (see "Streams" above), 2 to 16 non-empty
 * blocks run as two launches: dQ with every workgroup taking its query tile
 * through the blocks in turn (summed in registers, written once; equal to
 * the per-block chain up to float32 rounding of the sum's order), and dK, dV
 * of every block in one grid (the same bits as per block). Otherwise the
 * blocks run one after the other, dQ added into in place.
 */
cp_status_t cp_ring_attention_bwd(const void* q, const int64_t* q_strides, const void* const* k_blocks,
                                  const void* const* v_blocks, const int64_t* kv_strides, const int* block_len,
                                  int ring_degree, int dtype, int B, int H, int D, int Sq, float scale,
                                  unsigned flags, const float* out, const int64_t* out_strides, const float* dout,
                                  const int64_t* dout_strides, const float* lse, float* dq,
                                  const int64_t* dq_strides, float* const* dk_blocks, float* const* dv_blocks,
                                  const int64_t* dkv_strides, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* The workgroup shape (4 or 8 waves, see CP_FWD_FOUR_WAVES) the bfloat16 block kernel will use
 * for these sizes and flags (only the two shape flags matter); 0 if B, H or Sq is not positive,
 * D is not 64 or 128, or both shape flags are set. V packed by cp_attn_pack_v speeds up the
 * 8-wave shape only (the 4-wave kernel reads V at the same speed either way), so a caller that
 * has to pack V itself can skip it when this returns 4. */
int cp_attn_fwd_waves(int B, int H, int D, int Sq, unsigned flags);

/*
 * cp_ring_attention_noalloc -- cp_ring_attention without a workspace argument and without
 * allocating anything, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, layouts and results as cp_ring_attention, except that the workspace of the
 * parallel-partials form (256 bytes plus one int per 256-row query tile of each (b, h)) lives
 * in a static device array of 64 KB that the library holds on every GPU it runs on until the
 * process ends: packed-V calls with B * H * ceil(Sq / 256) above 16320 are CP_ERR_WORKSPACE, and
 * CP_RING_SEPARATE_MERGE (whose partial buffer is as large as out) is CP_ERR_INVALID_ARG. The call allocates and frees nothing; its first call on a device looks up
 * that device's copy of the array. Every call on one GPU shares that array and each parallel-
 * partials launch resets it first, so calls that overlap in time on one GPU (on different
 * streams) race and must not be issued; calls in one stream are fine.
 */
cp_status_t cp_ring_attention_noalloc(const void* q, const int64_t* q_strides, const void* const* k_blocks,
                                      const void* const* v_blocks, const int64_t* kv_strides, const int* block_len,
                                      int ring_degree, int dtype, int B, int H, int D, int Sq, float scale,
                                      unsigned flags, float* out, const int64_t* out_strides, float* lse,
                                      void* stream);

/* Message for the last non-CP_OK status returned on the calling thread ("" if none). */
const char* cp_last_error(void);

/* CP_ATTN_ABI_VERSION of the loaded library. */
int cp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
