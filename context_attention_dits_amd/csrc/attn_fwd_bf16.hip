// Partial attention of a local Q slice against one K/V block, bf16 inputs,
// float32 output + LSE, on gfx950 matrix cores.
//
// What it computes ("Paralelismo de contexto", section "Atencao em Anel";
// "Paralelismo", ContextParallelConfig, ring_degree / convert_to_fp32): for
// each (b, h) and query row i, lse_i = ln sum_j exp(scale <q_i, k_j>) and
// out_i = sum_j exp(scale <q_i, k_j> - lse_i) v_j, both float32. With the
// accumulate flag the block result is merged into (out, lse) in the epilogue
// by the exact LSE recombination instead of being stored on its own.
//
// Design (per workgroup: NW waves, each owning QB x 32 query rows of one
// (b, h); the K/V block is streamed through LDS in tiles of 64 keys):
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_f32_32x32x16_bf16: the A operand is a K fragment read from LDS,
//     the B operand is the wave's Q held in registers for the whole block. In
//     the 32x32 accumulator layout lane l holds query (l % 32) and 16 keys, so
//     the row statistics of the online softmax are lane-local plus one swap of
//     the two 32-lane halves (v_permlane32_swap).
//   * The output is accumulated transposed too, O^T += V^T . P^T: the B
//     operand P^T is the softmax'd score registers converted to bf16 in place
//     (no data movement), with the contraction over keys taken in the order
//     the accumulator layout holds them. Each lane's O registers belong to its
//     own query row, so rescaling needs no cross-lane traffic.
//   * K and V tiles go from global memory straight into LDS (buffer loads
//     with the LDS flag: lane i of a load fills bytes 16i..16i+15 of a 1 KB
//     LDS block), so staging costs no registers and no LDS-store
//     instructions. K is laid out per MFMA fragment: each (32-key block,
//     16-dim step) pair is one contiguous 1 KB block in exactly the lane
//     order of the A operand, read back with one conflict-free ds_read_b128
//     at an immediate offset. V stays row-major (one key per row) with its
//     16-byte chunks XOR-swizzled by row; V^T fragments are read from it with
//     ds_read_b64_tr_b16, which transposes 4 keys x 16 dims across each
//     16-lane group; the swizzle spreads the 8 rows one read touches over
//     all LDS banks.
//   * Lazy rescaling: the running row maximum is only raised (and O and the
//     row sum rescaled) when a tile's maximum exceeds it by more than 2^8 in
//     probability, so most tiles skip the rescale; exponentials stay <= 2^8.
//     Row sums are accumulated in float32 from the unrounded probabilities
//     (summing the bf16-rounded ones would cost up to 2^-9 relative in LSE
//     when a few keys dominate a row).
//   * The exponent uses base 2 with scale*log2(e) folded into one FMA.
//   * Two workgroup shapes, picked per launch:
//     - 4 waves (128 query rows, two workgroups per CU): two LDS stages, one
//       barrier per tile; each wave computes the next tile's scores on the
//       matrix cores interleaved with the current tile's exponentials, then
//       the PV product with V^T read by transposing LDS reads.
//     - 8 waves (256 rows, one workgroup per CU, half the K/V traffic per
//       row) in ping-pong: two groups of four waves, one wave of each group
//       per SIMD, run one half-step apart. Each step is a softmax half
//       (vector ALUs, plus the tile loads and a share of the V transposition)
//       and a matrix-core half (PV and next scores, LDS reads and MFMAs
//       only), separated by workgroup barriers, so each SIMD overlaps one
//       wave's softmax with the other wave's MFMAs. Three LDS stages of K,
//       raw V and V^T in fragment order (read with ds_read_b128).
//   * Packed V (PACKED): V may arrive already rewritten by pack_v_kernel
//     into the LDS image of its V^T fragments; tiles are then loaded with
//     contiguous 1 KB DMA loads and need no transposition (the ping-pong
//     kernel keeps no raw V stages). Same operands, same order: the results
//     are bit-identical to unpacked V.
//   * One launch for a ring (RING, ping-pong shape, packed V): workgroups
//     are block-major, each computes one block's partial for one query tile,
//     and the epilogues of a tile merge into (out, lse) in block order, each
//     waiting for a per-tile flag that the previous block's workgroup sets
//     after its stores. Same epilogue arithmetic in the same order as one
//     launch per block, so the same bits.
//   * Workgroups are remapped so that consecutive query tiles of one head run
//     on the same XCD (each XCD has its own L2) and share its K/V reads.
//   * Keys beyond Skv are never read: the buffer descriptor's range ends at
//     key Skv, so their LDS rows are zeros, and their scores are set to -inf.
//     Query rows beyond Sq are computed on zeros and not stored.
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

#ifndef CP_FWD_QB
#define CP_FWD_QB 1  // 32-query blocks per wave (the 8-wave shape needs 1: other values run 4 waves only)
#endif
#ifndef CP_FWD_NW
#define CP_FWD_NW 0  // default workgroup shape for D = 128: 4, 8 (ping-pong), or 0 to choose per launch
#endif
#ifndef CP_FWD_WPE
#define CP_FWD_WPE 2  // minimum waves per SIMD the register budget must allow
#endif
#ifndef CP_FWD_SCHED
#define CP_FWD_SCHED 7  // VALU ops scheduled between consecutive score MFMAs (0: no hints)
#endif
#ifndef CP_FWD_SCHED_PV
#define CP_FWD_SCHED_PV 1  // pipeline the transposing V reads ahead of the PV MFMAs
#endif
#ifndef CP_RING_ACQREL
#define CP_RING_ACQREL 0  // 1: order the one-launch ring's merges with agent-scope acquire/release (measured slower)
#endif
#ifndef CP_RING_SPIN_LIMIT
#define CP_RING_SPIN_LIMIT (1 << 22)  // one-launch ring: polls before a merge wait gives up
#endif
#ifndef CP_RING_TEST_NEVER_READY
#define CP_RING_TEST_NEVER_READY 0  // test builds only: after its real wait, every merge waits for a flag no workgroup sets
#endif
#ifndef CP_FWD_SEQ
#define CP_FWD_SEQ 1  // rings of 2+ blocks on the 8-wave shape: one launch, blocks in turn per workgroup
#endif
#ifndef CP_FWD_PHASE_TRACE
#define CP_FWD_PHASE_TRACE 0  // diagnostic builds only: cycle sums of the one-block launch's tile-loop intervals
#endif
#ifndef CP_FWD_LAZY
#define CP_FWD_LAZY 8.0f  // rescale threshold on the row maximum, log2 units
#endif

namespace cpattn {
#if CP_FWD_PHASE_TRACE
// Diagnostic builds: for each of the first kPhaseWg workgroups of a one-block launch and each
// wave, core-clock cycles of the tile loop's barrier intervals (the first three left out),
// summed by interval parity: [parity][work, wait at the barrier (tile loads, LDS accesses and
// the other waves)], then the number of intervals summed. Each launch overwrites the entries of
// the workgroups it runs.
constexpr int kPhaseWg = 1024, kPhaseVals = 8;
__device__ unsigned long long g_phase[kPhaseWg * 8 * kPhaseVals];
#endif
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Word 3 of a raw (unswizzled, untyped) buffer descriptor on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;

// Cache-policy operand of buffer loads: sc0 makes a load miss the CU's L1
// (it is served by the XCD's L2).
constexpr int kMissL1 = 1;

// One launch over several ring blocks: at most this many (more run as one launch each).
constexpr int kMaxRingBlocks = 16;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* out;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t kv_sb, kv_ss, kv_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, H, Sq, Skv;
  int n_qt;  // query tiles per (b, h)
  int n_wg;  // total workgroups (ring launch: query tiles, i.e. workgroups per block)
  float c;   // scale * log2(e)
  // Ring launch only: workgroup i works on block i / u8 (u8 = n_wg rounded up
  // to a multiple of 8, so that a query tile has the same XCD in every block);
  // flags[tile] = index of the last block merged into (out, lse) for that tile;
  // *err counts the merge waits that gave up (their query tiles are set to NaN).
  int n_blk, u8, spin_limit;
  int* flags;
  int* err;  // also for the other forms: zeroed by workgroup 0 when not null
  const uint16_t* kblk[kMaxRingBlocks];
  const uint16_t* vblk[kMaxRingBlocks];
  int lblk[kMaxRingBlocks];
  // packed V of block i: vblk[i] points at its first tile within (b, h) = 0
  // of a buffer with vnt[i] tiles per (b, h) (a block may be a tile-aligned
  // part of a larger packed block)
  int vnt[kMaxRingBlocks];
};

// Maximum that propagates NaN (IEEE maximum): unlike fmaxf it needs no
// quieting of its operands first, so a row maximum costs only v_maximum3 ops.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Both 32-lane halves of a wave64 end up with max/sum over the pair (l, l^32).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Index of the XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15; }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16 bytes per lane from global memory at base + voff into LDS at
// lds + 16 * lane, through a raw buffer descriptor covering [base, base +
// nbytes): lanes whose offset falls outside that range read nothing and
// write zeros. base, nbytes and lds must be wave-uniform.
__device__ __forceinline__ void buffer_to_lds16(const void* base, int nbytes, int voff, char* lds) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// Map the hardware workgroup id (dispatched round-robin over 8 XCDs) to a
// logical tile id so that each XCD receives one contiguous range of tiles.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, loc = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
}

template <int D, int QB, int NW>
struct Cfg {
  static constexpr int BN = 64;                   // keys per tile
  static constexpr int BM = NW * QB * 32;         // query rows per workgroup
  static constexpr int NT = NW * 64;              // threads per workgroup
  static constexpr int KB = BN / 32;              // 32-key blocks per tile
  static constexpr int KK = D / 16;               // 16-dim MFMA steps of QK^T
  static constexpr int K_BYTES = KB * KK * 1024;  // one 1 KB block per (kb, kk)
  static constexpr int VROW = D * 2;              // bytes per V row (one key)
  static constexpr int V_BYTES = BN * VROW;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int V_RPI = 1024 / VROW;       // V rows per 1 KB direct load
  static constexpr int V_LPR = VROW / 16;         // lanes per V row
  static constexpr bool PINGPONG = (NW == 8);     // two wave groups half a step apart
  static constexpr int NBUF = PINGPONG ? 3 : 2;   // LDS buffers per operand
  static constexpr int K_PER_WAVE = KB * KK / NW;
  static constexpr int V_PER_WAVE = (BN / V_RPI) / NW;
  static_assert(D == 64 || D == 128, "head dim");
  static_assert((KB * KK) % NW == 0 && (BN / V_RPI) % NW == 0, "load split");
  static_assert(KK % K_PER_WAVE == 0, "a wave's K blocks share one key block");
};

// XOR applied to a V row's 16-byte chunk index: the 8 rows that one
// transposing read touches (4 consecutive keys, and the same 4 keys + 4)
// cover every bank exactly twice.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 128) {
    return (r & 3) << 2;
  } else {
    return ((r >> 1) & 1) << 2;
  }
}

// A no-op hook for the memory-traffic slots of a compute phase.
struct Nothing {
  template <typename... A>
  __device__ __forceinline__ void operator()(A...) const {}
};

template <int D, int QB, int NW, bool ACC, bool PACKED, bool RING, bool SEQ = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                               amdgpu_waves_per_eu(CP_FWD_WPE)))
attn_fwd_bf16_kernel(Params p) {
  using C = Cfg<D, QB, NW>;
  // PACKED: p.v is V already in the tile / fragment order that the PV
  // products read (pack_v_kernel), so V tiles need no transposition here.
  // Separate arrays per buffer, so the compiler can tell the buffers being
  // read from the ones the next tiles are being loaded into.
  // vbuf*: raw V tiles (4 waves: V tiles as loaded, raw or packed; ping-pong:
  // raw V awaiting transposition, none when PACKED).
  constexpr int RAW_V = (C::PINGPONG && PACKED) ? 16 : C::V_BYTES;
  __shared__ __attribute__((aligned(1024))) char kbuf0[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[RAW_V];
  __shared__ __attribute__((aligned(1024))) char vbuf1[RAW_V];
  // ping-pong only: third stage, and V^T in MFMA fragment order (three stages)
  __shared__ __attribute__((aligned(1024))) char kbuf2[C::NBUF > 2 ? C::K_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char vbuf2[C::NBUF > 2 ? RAW_V : 16];
  __shared__ __attribute__((aligned(1024))) char vtb0[C::NBUF > 2 ? C::V_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char vtb1[C::NBUF > 2 ? C::V_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char vtb2[C::NBUF > 2 ? C::V_BYTES : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // RING: this workgroup's block (uniform) and query tile; padding workgroups
  // (tiles n_wg .. u8-1 of a block) exit at once.
  int blk = 0, tile;
  if constexpr (RING) {
    blk = blockIdx.x / p.u8;
    tile = xcd_remap(blockIdx.x - blk * p.u8, p.u8);
    if (tile >= p.n_wg) return;
  } else {
    tile = xcd_remap(blockIdx.x, p.n_wg);
  }
  int qt = tile % p.n_qt;
  int bh = tile / p.n_qt;
  int h = bh % p.H, b = bh / p.H;
  int qrow0 = qt * C::BM + wave * (QB * 32);
  if constexpr (!RING) {
    // a ring call's workspace error count: this form has no merge waits
    if (p.err != nullptr && blockIdx.x == 0 && tid == 0) *p.err = 0;
  }

  // SEQ: the workgroup takes its query tile through every block in turn
  // (block 0 written, later blocks merged by the epilogue); the next block's
  // first loads wait for the other wave group only where they would land in
  // an LDS stage it may still be reading (see the prologue). Each lane keeps its row's LSE (as
  // stored) in a register; the output it merges is what the same lane wrote.
  // Q is loaded again for every block, as by one launch per block.
  float lse_keep[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lse_keep[qb] = 0.f;
  // (The block loop is a backward jump that only the SEQ instantiation has,
  // so the other shapes compile exactly as without it.)
  int sblk = 0;
  int seq_prev_stage = -1;  // SEQ: LDS stage of the previous block's last tile
seq_next_block:
  if constexpr (SEQ) blk = sblk;

  // Kernel arguments used inside the tile loop, pinned in SGPRs: reloading
  // them from the argument segment there would make the next LDS wait also
  // wait for that scalar load.
  int skv = (RING || SEQ) ? p.lblk[blk] : p.Skv;
  float csc = p.c;
  asm volatile("" : "+s"(skv), "+s"(csc));
  const int n_tiles = (skv + C::BN - 1) / C::BN;

  const uint16_t* kblock = (RING || SEQ) ? p.kblk[blk] : p.k;
  const uint16_t* vblock = (RING || SEQ) ? p.vblk[blk] : p.v;
  const uint16_t* kbase = kblock + b * p.kv_sb + h * p.kv_sh;
  // packed V: n_tiles contiguous tiles of V_BYTES per (b, h), (b, h) in order
  // (RING: this block's tiles within its buffer's (b, h) row of vnt tiles)
  const int64_t v_tile0 = (int64_t)bh * ((RING || SEQ) ? p.vnt[blk] : n_tiles);
  const uint16_t* vbase = PACKED ? vblock + v_tile0 * (C::V_BYTES / 2) : vblock + b * p.kv_sb + h * p.kv_sh;

  // ---- Q (B operand of S^T = K Q^T): lane holds query l32, dims kk*16 + hi*8 .. +7
  bf16x8 qf[QB][C::KK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + l32;
    const uint16_t* qp = p.q + b * p.q_sb + (int64_t)row * p.q_ss + h * p.q_sh + hi * 8;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      if (row < p.Sq) {
        qf[qb][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
      } else {
        qf[qb][kk] = bf16x8{};
      }
    }
  }

  // ---- global -> LDS (this wave's share of a tile's 1 KB blocks) through
  // buffer loads: a scalar descriptor based at the tile's first key whose
  // range ends at key Skv, plus a per-lane byte offset that is the same for
  // every tile. Keys past Skv fall outside the range, are never read and
  // arrive in LDS as zeros.
  const int64_t row_bytes = p.kv_ss * 2;
  const int lw = wave;
  int k_voff;  // K block m = (kb, kk): key kb*32 + l32, 16-byte chunk 2*kk + hi
  {
    const int kb = (lw * C::K_PER_WAVE) / C::KK;
    k_voff = (int)((kb * 32 + l32) * row_bytes) + hi * 16;
  }
  int v_voff[C::V_PER_WAVE];  // V rows m*V_RPI + lane/V_LPR, swizzled chunks
#pragma unroll
  for (int i = 0; i < C::V_PER_WAVE; ++i) {
    const int r = (lw * C::V_PER_WAVE + i) * C::V_RPI + lane / C::V_LPR;
    v_voff[i] = (int)(r * row_bytes) + (((lane % C::V_LPR) ^ vswz<D>(r)) << 4);
  }
  // Source of tile t: a base pointer at its first key and the byte range up
  // to key Skv. Tiles past the end get an empty range (nothing is read; the
  // unused buffer they target receives zeros), so the pipeline can issue
  // loads unconditionally.
  auto tile_range = [&](int t, const uint16_t* head, const uint16_t*& base, int& nbytes) {
    base = head + (int64_t)(min(t, n_tiles - 1) * C::BN) * p.kv_ss;
    const int64_t avail = (int64_t)(skv - t * C::BN) * row_bytes;  // <= 0 past the end
    nbytes = (int)max((int64_t)0, min(avail, (int64_t)0x7fffffff));
  };
  auto issue_k = [&](int t, char* Ks) {
    const uint16_t* base;
    int nbytes;
    tile_range(t, kbase, base, nbytes);
#pragma unroll
    for (int i = 0; i < C::K_PER_WAVE; ++i) {
      const int m = lw * C::K_PER_WAVE + i;  // K block = (kb, kk); the wave's blocks share kb
      const int kk = m % C::KK;
      buffer_to_lds16(base, nbytes, k_voff + kk * 32, Ks + m * 1024);
    }
  };
  auto issue_v = [&](int t, char* Vs) {
    const uint16_t* base;
    int nbytes;
    if constexpr (PACKED) {
      // a packed tile is one contiguous V_BYTES block, its 1 KB fragments in
      // LDS order; past the last tile the range is empty
      base = vbase + (int64_t)min(t, n_tiles - 1) * (C::V_BYTES / 2);
      nbytes = t < n_tiles ? C::V_BYTES : 0;
    } else {
      tile_range(t, vbase, base, nbytes);
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_WAVE; ++i) {
      const int m = lw * C::V_PER_WAVE + i;
      buffer_to_lds16(base, nbytes, PACKED ? m * 1024 + lane * 16 : v_voff[i], Vs + m * 1024);
    }
  };

  // Per-lane byte offset of the transposed V reads (see vswz): within a
  // 16-lane group lane i supplies the address of key (i/4), dims 4*(i%4)..+3.
  int vlane;
  {
    const int i16 = lane & 15, jq = i16 >> 2, q = i16 & 3, blk = (lane >> 4) & 1;
    const int sw = (D == 128) ? jq : (jq >> 1);
    vlane = (4 * hi + jq) * C::VROW + (sw << 6) + ((blk * 2 + (q >> 1)) << 4) + ((q & 1) << 3);
  }

  f32x16 o[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[qb][db] = f32x16{};
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  // S^T = K Q^T for one 64-key tile held in LDS.
  auto scores = [&](const char* Ks, f32x16 (&s)[QB][C::KB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) s[qb][kb] = f32x16{};
    const char* kfrag = Ks + lane * 16;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kfrag + (kb * C::KK + kk) * 1024);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][kk], s[qb][kb], 0, 0, 0);
      }
    }
  };

  // Probabilities of the tile whose PV product is pending, as the bf16 B
  // operand of O^T += V^T P^T (key order as the score accumulators hold it).
  bf16x8 pf[QB][C::KB][2];

  // Softmax of tile j: tail mask, row maxima and lazy rescale, exponentials
  // into pf and the row sums. Fused form: the scores of tile j+1 (from k_read
  // into s_next) run on the matrix cores interleaved with the exponentials on
  // the vector ALUs. On entry s_cur holds tile j's scores.
  auto half_a = [&](auto last_tag, auto fuse_tag, int j, f32x16 (&s_cur)[QB][C::KB],
                    f32x16 (&s_next)[QB][C::KB], const char* k_read, auto pre, auto post) {
    constexpr bool LAST = decltype(last_tag)::value;  // the final tile: mask, no next tile
    constexpr bool FUSE = decltype(fuse_tag)::value && !LAST;  // next tile's scores computed here
    pre();  // memory traffic first, so its latency hides behind the arithmetic

    // tail mask: keys >= Skv get -inf (only the last tile can have them)
    if constexpr (LAST) {
      const int key0 = j * C::BN;
      if (key0 + C::BN > skv) {
        // This lane holds keys key0 + 4*hi + (kb*32 + 8*(r/4) + r%4).
        const int lim = skv - key0 - 4 * hi;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s_cur[qb][kb][r] = -INFINITY;
      }
    }

    // row maxima of tile j; raise the running maximum only when a row's
    // maximum grows by more than 2^CP_FWD_LAZY (then O and l are rescaled)
    float alpha[QB];
    bool rescale = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // two independent chains of maxima (half the dependent latency)
      float mx0 = s_cur[qb][0][0], mx1 = s_cur[qb][0][1];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) {
          mx0 = vmax(mx0, s_cur[qb][kb][r]);
          mx1 = vmax(mx1, s_cur[qb][kb][r + 1]);
        }
      const float mt = half_max(vmax(mx0, mx1)) * csc;
      const bool need = __builtin_amdgcn_ballot_w64(mt > m_run[qb] + CP_FWD_LAZY) != 0;
      const float m_new = need ? fmaxf(m_run[qb], mt) : m_run[qb];
      alpha[qb] = fast_exp2(m_run[qb] - m_new);  // 1 when the maximum is kept
      rescale |= need;
      m_run[qb] = m_new;
    }
    if (rescale) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_run[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[qb][db] *= alpha[qb];
      }
    }

    if constexpr (FUSE) scores(k_read, s_next);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mneg = -m_run[qb];
      // float32 sums of the unrounded probabilities (LSE needs them), in four
      // independent partial sums so that the adds do not form one dependent chain
      float ls[4];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          post((qb * C::KB + kb) * 2 + kk2);  // hook between groups of 8 exponentials
          bf16x8 t;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float e = fast_exp2(fmaf(s_cur[qb][kb][kk2 * 8 + jj], csc, mneg));
            if (kb == 0 && kk2 == 0 && jj < 4) {
              ls[jj] = e;
            } else {
              ls[jj & 3] += e;
            }
            t[jj] = (__bf16)e;
          }
          pf[qb][kb][kk2] = t;
        }
      l_run[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
    if constexpr (!decltype(fuse_tag)::value) {
      // Split form: pin the probabilities and row sums here, so the compiler
      // cannot sink their arithmetic past the barrier into the MFMA half.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        asm volatile("" : "+v"(l_run[qb]));
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          asm volatile("" : "+v"(pf[qb][kb][0]));
          asm volatile("" : "+v"(pf[qb][kb][1]));
        }
      }
    }
#if CP_FWD_SCHED
    if constexpr (FUSE) {
    // 16*QB score MFMAs, their 16 fragment reads and ~112*QB VALU ops:
    // keep two reads ahead and spread the VALU work between the MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < C::KB * C::KK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, CP_FWD_SCHED, 0);
    }
    }
#endif
  };

  // Second half: O^T += V^T P^T with the V tile in v_read (V^T fragments via
  // transposing LDS reads).
  auto half_b = [&](const char* v_read) {
    if constexpr (PACKED) {
      // V^T fragments as packed: one ds_read_b128 each (fragment order below)
      const char* vfrag = v_read + lane * 16;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int kk2 = 0; kk2 < 2; ++kk2) {
            const int f = (db * C::KB + kb) * 2 + kk2;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(vfrag + f * 1024);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kb][kk2], o[qb][db], 0, 0, 0);
          }
#if CP_FWD_SCHED_PV
      // keep four fragments ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < (D / 32) * C::KB * 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#endif
      return;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const char* vb = v_read + (vlane ^ (db << 6));
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const char* a0 = vb + (kb * 32 + kk2 * 16) * C::VROW;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * C::VROW));
          const bf16x8 a = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                                   __builtin_bit_cast(bf16x4, hi4), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kb][kk2], o[qb][db], 0, 0, 0);
        }
    }
#if CP_FWD_SCHED_PV
    // keep four V^T fragments (eight transposing reads) ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < (D / 32) * C::KB * 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#endif
  };

  // Ping-pong only: V^T of one tile in MFMA fragment order. Fragment
  // f = (db * KB + kb) * 2 + kk2 is the A operand of O^T += V^T P^T for dims
  // db*32.. and keys kb*32 + kk2*16..; lane l's 16 bytes sit at f*1024 + l*16,
  // so it is read back with one conflict-free ds_read_b128.
  constexpr int N_VFRAG = (D / 32) * C::KB * 2;
  // Transpose this wave's share of the fragments of a raw V tile (row-major,
  // swizzled, as loaded) into vt: two transposing reads (read_vt) and one
  // write (write_vt) each.
  static_assert(N_VFRAG % NW == 0, "fragment split");
  constexpr int VT_PER_WAVE = N_VFRAG / NW > 0 ? N_VFRAG / NW : 1;
  auto read_vt = [&](const char* v_raw, i16x8 (&frag)[VT_PER_WAVE]) {
#pragma unroll
    for (int i = 0; i < N_VFRAG / NW; ++i) {
      const int f = wave * (N_VFRAG / NW) + i;
      const int db = f / (2 * C::KB), kb = (f / 2) % C::KB, kk2 = f % 2;
      const char* a0 = v_raw + (vlane ^ (db << 6)) + (kb * 32 + kk2 * 16) * C::VROW;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * C::VROW));
      frag[i] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto write_vt = [&](char* vt, const i16x8 (&frag)[VT_PER_WAVE]) {
#pragma unroll
    for (int i = 0; i < N_VFRAG / NW; ++i) {
      const int f = wave * (N_VFRAG / NW) + i;
      *reinterpret_cast<i16x8*>(vt + f * 1024 + lane * 16) = frag[i];
    }
  };

  // Matrix-core half of a ping-pong step: O^T += V_j^T P_j^T from vt_read and,
  // unless tile j is the last, the scores of tile j+1 from k_read into s_next.
  // Only LDS reads and MFMAs: the vector ALU work of the step is in half_a.
  auto half_m = [&](auto last_tag, f32x16 (&s_next)[QB][C::KB], const char* k_read, const char* vt_read) {
    constexpr bool LAST = decltype(last_tag)::value;
    // Scores first: the next softmax half waits on them, not on the PV
    // products, which finish on the matrix cores behind it.
    if constexpr (!LAST) scores(k_read, s_next);
    const char* vfrag = vt_read + lane * 16;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const int f = (db * C::KB + kb) * 2 + kk2;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vfrag + f * 1024);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kb][kk2], o[qb][db], 0, 0, 0);
        }
#if CP_FWD_SCHED_PV
    // Keep the LDS reads ahead of the MFMAs: eight reads up front, then two
    // per MFMA, then one, until the reads run out.
    constexpr int n_mfma = QB * ((D / 32) * C::KB * 2 + (LAST ? 0 : C::KB * C::KK));
    constexpr int n_rd = (D / 32) * C::KB * 2 + (LAST ? 0 : C::KB * C::KK);
    constexpr int pre = n_rd < 8 ? n_rd : 8;
    constexpr int two = (n_rd - pre) / 2 < n_mfma ? (n_rd - pre) / 2 : n_mfma;
    constexpr int one = n_rd - pre - 2 * two;
    __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);
#pragma unroll
    for (int i = 0; i < n_mfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < two) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (i < two + one) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#endif
  };

  // Workgroup barrier after this wave's LDS reads have completed and all but
  // its `pending` most recent global->LDS loads have landed (loads complete in
  // issue order). The memory clobbers keep the compiler from moving LDS
  // accesses across it.
#if CP_FWD_PHASE_TRACE
  // The core clock (s_memtime, waited for in the same statement: each reading is a scalar
  // memory round trip that the wave waits for, which the cycle counts include), read before and
  // after each barrier's waits; sums (see g_phase) of the work up to the wait, and of the wait for
  // tile loads and LDS accesses plus the barrier wait. 32-bit: differences of the counter's low
  // word, and sums over a launch, stay far below 2^32.
  constexpr bool TRACE = !RING && !SEQ;
  auto clock_now = [] {
    unsigned long long t;
    asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t));
    return (uint32_t)t;
  };
  uint32_t ph_prev = TRACE ? clock_now() : 0;
  uint32_t ph_sum[2][2] = {{0, 0}, {0, 0}};
  int ph_i = 0;
#endif
  auto sync = [&](auto pending_tag) {
    constexpr int PENDING = decltype(pending_tag)::value;  // 63: no wait on loads
    static_assert(PENDING >= 0 && PENDING < 64, "vmcnt field");
#if CP_FWD_PHASE_TRACE
    uint32_t t1 = 0;
    if constexpr (TRACE) t1 = clock_now();
#endif
    // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4] (7 = no wait), lgkmcnt[11:8]
    __builtin_amdgcn_s_waitcnt(0x0070 | (PENDING & 15) | ((PENDING >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#if CP_FWD_PHASE_TRACE
    if constexpr (TRACE) {
      const uint32_t t2 = clock_now();
      if (ph_i >= 3) {
        ph_sum[ph_i & 1][0] += t1 - ph_prev;
        ph_sum[ph_i & 1][1] += t2 - t1;
      }
      ph_prev = t2;
      ++ph_i;
    }
#endif
  };
  using Pend0 = std::integral_constant<int, 0>;
  using PendAll = std::integral_constant<int, 63>;
  using Mid = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;

  using Fused = std::integral_constant<bool, true>;
  using Split = std::integral_constant<bool, false>;

  f32x16 sa[QB][C::KB];
  int j = 0;
  if constexpr (!C::PINGPONG) {
    // prologue: K_0, V_0, K_1 loaded; scores of tile 0. K_j lives in
    // kbuf(j % 2) and V_j in vbuf(j % 2).
    issue_k(0, kbuf0);
    issue_v(0, vbuf0);
    issue_k(1, kbuf1);
    sync(Pend0{});
    scores(kbuf0, sa);
    sync(Pend0{});  // every wave is done with K_0 before K_2 overwrites it
    f32x16 sb[QB][C::KB];
    // One step over tile j: loads of K_{j+2} and V_{j+1} are issued, then
    // the fused softmax / next scores and the PV product run, then one
    // barrier. The score registers swap roles each tile, so the loop runs two
    // tiles at a time; the final tile is masked.
    auto step = [&](auto last_tag, int jj, f32x16 (&s_cur)[QB][C::KB], f32x16 (&s_next)[QB][C::KB],
                    const char* k_read, char* k_write, const char* v_read, char* v_write) {
      constexpr bool LAST = decltype(last_tag)::value;
      if constexpr (!LAST) {
        issue_k(jj + 2, k_write);
        issue_v(jj + 1, v_write);
      }
      half_a(last_tag, Fused{}, jj, s_cur, s_next, k_read, Nothing{}, Nothing{});
      half_b(v_read);
      if constexpr (!LAST) sync(Pend0{});
    };
    for (; j + 2 < n_tiles; j += 2) {
      step(Mid{}, j, sa, sb, kbuf1, kbuf0, vbuf0, vbuf1);
      step(Mid{}, j + 1, sb, sa, kbuf0, kbuf1, vbuf1, vbuf0);
    }
    if (j + 2 == n_tiles) {
      step(Mid{}, j, sa, sb, kbuf1, kbuf0, vbuf0, vbuf1);
      step(Last{}, j + 1, sb, sa, kbuf0, kbuf1, vbuf1, vbuf0);
    } else {
      step(Last{}, j, sa, sb, kbuf1, kbuf0, vbuf0, vbuf1);
    }
  } else {
    // Ping-pong: waves [0, NW/2) (group A) and [NW/2, NW) (group B) share
    // the SIMDs pairwise (wave w and w + NW/2 on one SIMD) and run the same
    // program one interval apart, so that on each SIMD one wave's softmax
    // (vector ALUs) runs while the other wave's matrix-core half (LDS reads
    // and MFMAs only) runs. Intervals end with a workgroup barrier. Group A
    // runs the softmax of tile j in interval 2j and its MFMA half (PV of tile
    // j, scores of tile j+1) in 2j+1; group B one interval later.
    // Three LDS stages of K, raw V and V^T: tile t lives in stage t % 3.
    // During its softmax of tile j every wave issues its share of K_{j+2} and
    // raw V_{j+3} and transposes its share of raw V_{j+1} into V_{j+1}^T.
    // The buffers it writes were last read in interval 2j-1 or earlier; the
    // tiles it loads are first read in interval 2j+3 (K) and 2j+4 (V). Group
    // A waits for its loads one softmax later (all but the newest, at the end
    // of interval 2j+2); group B, which issues in 2j+1, waits for all of its
    // loads at the end of its MFMA half in 2j+2. Every barrier waits for the
    // wave's LDS accesses, so a transposed tile is complete one interval
    // after the second group wrote its share.
    // With packed V there is no raw V and no transposition: V_{j+1}^T is
    // loaded straight into its stage during the softmax of tile j, with
    // K_{j+2}. Its stage last held V_{j-2}^T, read in interval 2j-2 at the
    // latest, and it is first read in interval 2j+3, after the same waits as
    // K_{j+2}.
    using PendL = std::integral_constant<int, C::K_PER_WAVE + C::V_PER_WAVE>;
    const bool grp_b = wave >= NW / 2;
    char* const kb3[3] = {kbuf0, kbuf1, kbuf2};
    char* const vb3[3] = {vbuf0, vbuf1, vbuf2};
    char* const vt3[3] = {vtb0, vtb1, vtb2};
    // prologue: K_0, K_1 and raw V_0..V_2 loaded, V_0^T built (packed: K_0,
    // K_1 and V_0^T loaded), scores of tile 0
    // SEQ, later blocks: the other wave group may still be in the previous
    // block's last MFMA half, which reads only that block's last V^T stage
    // (no scores, so no K stage): the K loads go at once, V_0's only after a
    // workgroup barrier when it lands in that stage.
    issue_k(0, kbuf0);
    issue_k(1, kbuf1);
    if constexpr (PACKED) {
      if constexpr (SEQ) {
        if (seq_prev_stage == 0) __syncthreads();
      }
      issue_v(0, vtb0);
      sync(Pend0{});
      scores(kbuf0, sa);
    } else {
      issue_v(0, vbuf0);
      issue_v(1, vbuf1);
      issue_v(2, vbuf2);
      sync(Pend0{});
      scores(kbuf0, sa);
      i16x8 fr[VT_PER_WAVE];
      read_vt(vbuf0, fr);
      write_vt(vtb0, fr);
    }
    if (grp_b) sync(Pend0{});  // group B idles in interval 0
    // one tile; c = j % 3, known at compile time in the unrolled loop
    auto step = [&](auto last_tag, auto c_tag, int jj) {
      constexpr bool LAST = decltype(last_tag)::value;
      constexpr int c = decltype(c_tag)::value;
      const char* k_read = kb3[(c + 1) % 3];
      const char* vt_read = vt3[c];
      if constexpr (!LAST) {
        if constexpr (PACKED) {
          half_a(
              last_tag, Split{}, jj, sa, sa, k_read,
              [&] {
                issue_k(jj + 2, kb3[(c + 2) % 3]);
                issue_v(jj + 1, vt3[(c + 1) % 3]);
              },
              Nothing{});
        } else {
          i16x8 fr[VT_PER_WAVE];
          half_a(
              last_tag, Split{}, jj, sa, sa, k_read,
              [&] {
                issue_k(jj + 2, kb3[(c + 2) % 3]);
                issue_v(jj + 3, vb3[c]);
                read_vt(vb3[(c + 1) % 3], fr);
              },
              [&](int g) {
                if (g == 0) write_vt(vt3[(c + 1) % 3], fr);
              });
        }
        if (grp_b) sync(PendAll{});
        else sync(PendL{});
        half_m(last_tag, sa, k_read, vt_read);
        if (grp_b) sync(Pend0{});
        else sync(PendAll{});
      } else {
        // The last barrier ends interval 2n-2: group A passes it after its
        // last softmax, group B after its last MFMA half but one.
        half_a(last_tag, Split{}, jj, sa, sa, k_read, Nothing{}, Nothing{});
        if (!grp_b) sync(Pend0{});
        half_m(last_tag, sa, k_read, vt_read);
      }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    for (; j + 3 < n_tiles; j += 3) {
      step(Mid{}, C0{}, j);
      step(Mid{}, C1{}, j + 1);
      step(Mid{}, C2{}, j + 2);
    }
    if (j + 3 == n_tiles) {
      step(Mid{}, C0{}, j);
      step(Mid{}, C1{}, j + 1);
      step(Last{}, C2{}, j + 2);
    } else if (j + 2 == n_tiles) {
      step(Mid{}, C0{}, j);
      step(Last{}, C1{}, j + 1);
    } else {
      step(Last{}, C0{}, j);
    }
  }

#if CP_FWD_PHASE_TRACE
  if constexpr (TRACE) {
    if (blockIdx.x < kPhaseWg && lane == 0) {
      unsigned long long* d = g_phase + (blockIdx.x * 8 + wave) * kPhaseVals;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = ph_sum[i / 2][i % 2];
      d[4] = (unsigned long long)(ph_i > 3 ? ph_i - 3 : 0);
    }
  }
#endif

  // ---- epilogue: normalise, LSE, optional merge into the accumulator
  // RING: block 0 writes, later blocks merge, each after the previous block's
  // workgroup for the same query tile has published its (out, lse): that
  // workgroup's stores have completed (reached its XCD's L2) before it sets
  // flags[tile] = 16 * blk + (its XCD), and this workgroup waits for
  // 16 * (blk - 1) + x. The merge reads out and lse past its CU's L1, from the
  // L2, which holds what the publisher wrote only if x is this workgroup's
  // own XCD: workgroups whose index differs by a multiple of 8 run on one
  // XCD, which the launch arranges, and the flag checks it (a flag from
  // another XCD counts as a failed wait). No cache is written back or
  // invalidated. (CP_RING_ACQREL=1 builds order the merges with agent-scope
  // acquire/release instead, which is slower.) The wait cannot deadlock: the
  // awaited workgroup has the same index modulo u8 and a lower index, and it
  // waits only on lower ones itself. It is bounded all the same: a wait that
  // gives up counts itself in *err and sets the tile's out and lse to NaN
  // instead of merging, then publishes as usual, so no later block waits on
  // it in vain and the result cannot pass for a correct one.
  bool acc = ACC || (SEQ && sblk > 0);
  bool gave_up = false;
  if constexpr (RING) {
    acc = blk > 0;
    if (acc) {
      __shared__ int s_gave_up;
      if (threadIdx.x == 0) {
        auto poll = [&] {
          return CP_RING_ACQREL ? __hip_atomic_load(p.flags + tile, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)
                                : __hip_atomic_load(p.flags + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        int n = 0, f = -1;
        bool ready;
        while (!(ready = (f = poll()) >= 0 && (f >> 4) == blk - 1) && ++n < p.spin_limit) __builtin_amdgcn_s_sleep(1);
        if (!CP_RING_ACQREL && ready && (f & 15) != xcc_id()) ready = false;  // not this XCD's L2
        if (CP_RING_TEST_NEVER_READY && ready) {
          // test builds: then a second, short wait for a value no workgroup publishes
          n = 0;
          while (!(ready = poll() == 16 * (blk + 1000)) && ++n < 16) __builtin_amdgcn_s_sleep(1);
        }
        s_gave_up = !ready;
        if (!ready) __hip_atomic_fetch_add(p.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      gave_up = s_gave_up != 0;
    }
  }
  // accesses to out and lse. RING: through a buffer descriptor with 32-bit
  // offsets (fewer address registers than 64-bit pointers).
  const __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc(p.out, (short)0, 0x7fffffff, kBufferFlags);
  const __amdgpu_buffer_rsrc_t lrsrc =
      __builtin_amdgcn_make_buffer_rsrc(p.lse, (short)0, 0x7fffffff, kBufferFlags);
  constexpr int kMergeLoad = CP_RING_ACQREL ? 0 : kMissL1;  // RING: past any stale L1 copy
  auto o_load = [&](const float* ptr) -> f32x4 {
    if constexpr (RING) {
      return __builtin_amdgcn_raw_buffer_load_b128(orsrc, (int)((ptr - p.out) * 4), 0, kMergeLoad);
    } else {
      return *reinterpret_cast<const f32x4*>(ptr);
    }
  };
  auto o_store = [&](float* ptr, f32x4 v) {
    if constexpr (RING) {
      __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, (int)((ptr - p.out) * 4), 0, 0);
    } else {
      *reinterpret_cast<f32x4*>(ptr) = v;
    }
  };
  auto l_load = [&](const float* ptr) -> float {
    if constexpr (RING) {
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrsrc, (int)((ptr - p.lse) * 4), 0,
                                                                            kMergeLoad));
    } else {
      return *ptr;
    }
  };
  auto l_store = [&](float* ptr, float v) { *ptr = v; };
  // In the accumulator layout a lane holds one row and 16 of the 32 columns
  // of each 32-column block, so its stores cover a 128-byte line of out in
  // 32-byte pieces. STAGE (the parallel-partials ring): the values (merged,
  // where merging, in that layout) go through a per-wave LDS area instead,
  // from which lane L takes row L/8 (+8, +16, +24) and columns 4(L%8)..+3 of
  // the block, so that eight lanes store one whole line. Chunk c of staged
  // row r sits at c ^ (r % 8), spreading the banks. SR rows are staged per
  // pass, as the LDS left by the tile stages allows. The area is the wave's
  // own, and a wave's LDS accesses complete in order: no barrier. There the
  // merges' pieces reached memory separately (more bytes written than out
  // holds) and whole lines run faster; the one-block launches run slightly
  // slower staged, and in the blocks-in-turn form the staging inside the
  // block loop makes the compiler schedule the tile loop for fewer registers
  // (its LDS reads no longer run ahead). Same values either way.
  constexpr bool STAGE = RING;
  constexpr int SR = (C::PINGPONG && PACKED) ? 32 : 16;
  __shared__ __attribute__((aligned(1024))) char ostage[STAGE ? NW * SR * 128 : 16];
  f32x4* const stg = reinterpret_cast<f32x4*>(ostage) + (STAGE ? wave * SR * 8 : 0);
  const int sr = lane >> 3, sc = lane & 7;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + l32;
    const float lt = half_sum(l_run[qb]);
    const float lse2 = m_run[qb] + fast_log2(lt);  // log2 units
    // this lane's row: out = fa * out_old + fb * o, with no old part when fa < 0
    float fa = -1.f, fb = 1.0f / lt, lse_out = lse2 * kLn2;
    float* const lrow = p.lse + ((int64_t)b * p.H + h) * p.Sq + row;
    float* const orow = p.out + b * p.o_sb + (int64_t)row * p.o_ss + h * p.o_sh + 4 * hi;
    if (RING && gave_up) {
      // the previous block's partial for this tile was not seen: no merge
      fb = NAN;
      lse_out = NAN;
    } else if (acc && row < p.Sq) {
      const float la2 = (SEQ ? lse_keep[qb] : l_load(lrow)) * kLog2e;
      const float M = fmaxf(la2, lse2);
      const float wa = fast_exp2(la2 - M);  // 0 when the accumulator is empty (-inf)
      const float wb = fast_exp2(lse2 - M);
      const float tot = wa + wb;
      if (wa > 0.f) fa = wa / tot;
      fb *= wb / tot;
      lse_out = (M + fast_log2(tot)) * kLn2;
    }
    if (row < p.Sq) {
      if constexpr (SEQ) lse_keep[qb] = lse_out;
      if (hi == 0) l_store(lrow, lse_out);
    }
    // the lane's value for columns db*32 + 8g + 4hi .. +3 of its row
    auto value = [&](int db, int g) -> f32x4 {
      const f32x4 ob = {o[qb][db][4 * g], o[qb][db][4 * g + 1], o[qb][db][4 * g + 2], o[qb][db][4 * g + 3]};
      f32x4 v = fb * ob;
      if (fa >= 0.f) {
        const f32x4 a = o_load(orow + db * 32 + 8 * g);
        v = f32x4{__builtin_fmaf(fa, a[0], v[0]), __builtin_fmaf(fa, a[1], v[1]), __builtin_fmaf(fa, a[2], v[2]),
                  __builtin_fmaf(fa, a[3], v[3])};
      }
      return v;
    };
    if constexpr (!STAGE) {
      if (row < p.Sq) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) o_store(orow + db * 32 + 8 * g, value(db, g));
      }
    } else {
#pragma unroll
      for (int pp = 0; pp < 32 / SR; ++pp) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          if (SR == 32 || l32 / SR == pp) {
            const int rl = l32 % SR;
#pragma unroll
            for (int g = 0; g < 4; ++g) stg[rl * 8 + ((2 * g + hi) ^ (rl & 7))] = value(db, g);
          }
          f32x4 v[SR / 8];
#pragma unroll
          for (int i = 0; i < SR / 8; ++i) v[i] = stg[(sr + 8 * i) * 8 + (sc ^ sr)];
          // read here, all at once, not inside the row checks below
          if constexpr (SR == 32) {
            asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
          } else {
            asm volatile("" : "+v"(v[0]), "+v"(v[1]));
          }
#pragma unroll
          for (int i = 0; i < SR / 8; ++i) {
            const int grow = qrow0 + qb * 32 + pp * SR + sr + 8 * i;
            if (grow < p.Sq)
              o_store(p.out + b * p.o_sb + (int64_t)grow * p.o_ss + h * p.o_sh + db * 32 + 4 * sc, v[i]);
          }
        }
      }
    }
  }
  if constexpr (RING) {
    // publish: every wave's stores have completed, then the flag (release:
    // those stores become visible to an acquiring reader first)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt: no wait
    __syncthreads();
    if (threadIdx.x == 0) {
      const int f = 16 * blk + xcc_id();
      if (CP_RING_ACQREL)
        __hip_atomic_store(p.flags + tile, f, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_store(p.flags + tile, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (SEQ) {
    seq_prev_stage = (n_tiles - 1) % 3;
    if (++sblk < p.n_blk) goto seq_next_block;
  }
}

template <int D, int NW, bool ACC, bool PACKED>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  constexpr int QB = CP_FWD_QB;
  using C = Cfg<D, QB, NW>;
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.out = a.out;
  p.lse = a.lse;
  p.q_sb = a.qs.b; p.q_ss = a.qs.s; p.q_sh = a.qs.h;
  p.kv_sb = a.kvs.b; p.kv_ss = a.kvs.s; p.kv_sh = a.kvs.h;
  p.o_sb = a.os.b; p.o_ss = a.os.s; p.o_sh = a.os.h;
  p.B = a.B; p.H = a.H; p.Sq = a.Sq; p.Skv = a.Skv;
  p.n_qt = (a.Sq + C::BM - 1) / C::BM;
  const int64_t n_wg = (int64_t)p.n_qt * a.H * a.B;
  if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.n_wg = (int)n_wg;
  p.c = a.scale * kLog2e;
  p.err = a.err;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, QB, NW, ACC, PACKED, false>), dim3(p.n_wg), dim3(C::NT), 0, stream,
                     p);
  return hipGetLastError();
}

// Reset of the ring launch's workspace: the error count to 0, every flag to -1.
__global__ void __launch_bounds__(256) fill_flags_kernel(int* err, int* flags, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) flags[i] = -1;
  if (i == 0) *err = 0;
}

// One launch for a ring of blocks (ping-pong shape, D = 128): n_blk * u8
// workgroups, block-major; see the kernel's epilogue for the ordering of the
// merges. ws: the error count, then (at int 64) n_wg flags, reset here by a
// fill kernel (no memset, so the pair can be captured in a graph).
template <bool PACKED>
hipError_t launch_ring_128(const FwdArgs& a, const RingBlocks& rb, int* ws, hipStream_t stream) {
  int* const err = ws;
  int* const flags = ws + kRingFlagOffset;
  constexpr int QB = CP_FWD_QB;
  using C = Cfg<128, QB, 8>;
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = nullptr;
  p.v = nullptr;
  p.out = a.out;
  p.lse = a.lse;
  p.q_sb = a.qs.b; p.q_ss = a.qs.s; p.q_sh = a.qs.h;
  p.kv_sb = a.kvs.b; p.kv_ss = a.kvs.s; p.kv_sh = a.kvs.h;
  p.o_sb = a.os.b; p.o_ss = a.os.s; p.o_sh = a.os.h;
  p.B = a.B; p.H = a.H; p.Sq = a.Sq; p.Skv = 0;
  p.n_qt = (a.Sq + C::BM - 1) / C::BM;
  const int64_t n_wg = (int64_t)p.n_qt * a.H * a.B;
  const int64_t u8 = (n_wg + 7) / 8 * 8;
  if (rb.n < 1 || rb.n > kMaxRingBlocks || u8 * rb.n > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.n_wg = (int)n_wg;
  p.u8 = (int)u8;
  p.n_blk = rb.n;
  p.spin_limit = CP_RING_SPIN_LIMIT;
  p.flags = flags;
  p.err = err;
  p.c = a.scale * kLog2e;
  for (int i = 0; i < kMaxRingBlocks; ++i) {
    p.kblk[i] = i < rb.n ? static_cast<const uint16_t*>(rb.k[i]) : nullptr;
    p.vblk[i] = i < rb.n ? static_cast<const uint16_t*>(rb.v[i]) + (int64_t)rb.vt0[i] * (C::V_BYTES / 2) : nullptr;
    p.lblk[i] = i < rb.n ? rb.len[i] : 0;
    p.vnt[i] = i < rb.n ? rb.vnt[i] : 0;
  }
  if (a.accumulate) return hipErrorInvalidValue;  // the ring launch writes block 0
  hipLaunchKernelGGL(fill_flags_kernel, dim3((unsigned)((n_wg + 255) / 256)), dim3(256), 0, stream, err, flags,
                     (int)n_wg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, QB, 8, false, PACKED, true>), dim3((unsigned)(u8 * rb.n)),
                     dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

// One launch for a ring of blocks on the ping-pong shape, blocks in turn
// within each workgroup (SEQ): the per-block launches' grid, block 0 written
// and later blocks merged in the epilogue, in block order, by the workgroup
// that owns the query tile. No flags and no workspace.
hipError_t launch_seq_128(const FwdArgs& a, const RingBlocks& rb, hipStream_t stream) {
  constexpr int QB = CP_FWD_QB;
  using C = Cfg<128, QB, 8>;
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = nullptr;
  p.v = nullptr;
  p.out = a.out;
  p.lse = a.lse;
  p.q_sb = a.qs.b; p.q_ss = a.qs.s; p.q_sh = a.qs.h;
  p.kv_sb = a.kvs.b; p.kv_ss = a.kvs.s; p.kv_sh = a.kvs.h;
  p.o_sb = a.os.b; p.o_ss = a.os.s; p.o_sh = a.os.h;
  p.B = a.B; p.H = a.H; p.Sq = a.Sq; p.Skv = 0;
  p.n_qt = (a.Sq + C::BM - 1) / C::BM;
  const int64_t n_wg = (int64_t)p.n_qt * a.H * a.B;
  if (rb.n < 1 || rb.n > kMaxRingBlocks || n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.accumulate || !a.v_packed) return hipErrorInvalidValue;
  p.n_wg = (int)n_wg;
  p.u8 = 0;
  p.n_blk = rb.n;
  p.spin_limit = 0;
  p.flags = nullptr;
  p.err = a.err;
  p.c = a.scale * kLog2e;
  for (int i = 0; i < kMaxRingBlocks; ++i) {
    const bool in = i < rb.n;
    if (in && rb.len[i] < 1) return hipErrorInvalidValue;
    p.kblk[i] = in ? static_cast<const uint16_t*>(rb.k[i]) : nullptr;
    p.vblk[i] = in ? static_cast<const uint16_t*>(rb.v[i]) + (int64_t)rb.vt0[i] * (C::V_BYTES / 2) : nullptr;
    p.lblk[i] = in ? rb.len[i] : 0;
    p.vnt[i] = in ? rb.vnt[i] : 0;
  }
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, QB, 8, false, true, false, true>), dim3((unsigned)n_wg),
                     dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_dw(const FwdArgs& a, hipStream_t stream) {
  if (a.v_packed)
    return a.accumulate ? launch_d<D, NW, true, true>(a, stream) : launch_d<D, NW, false, true>(a, stream);
  return a.accumulate ? launch_d<D, NW, true, false>(a, stream) : launch_d<D, NW, false, false>(a, stream);
}

// V of one block in the order the PV products read it, for the kernel above
// with PACKED: per (b, h), in (b, h) order, ceil(Skv / 64) tiles of 64 keys,
// each D * 128 bytes: fragment f = (db * 2 + kb) * 2 + kk2 (db: 32 dims, kb:
// 32 keys, kk2: 16 keys) is 1 KB in which lane l (l32 = l % 32, hi = l / 32)
// has 8 values, element e being V[key][d] for d = 32 db + l32 and
// key = 64 t + 32 kb + 16 kk2 + 8 (e / 4) + 4 hi + e % 4 -- the key order in
// which the score accumulators hold the probabilities. Keys >= Skv are zero.
// One workgroup per tile: the tile goes through LDS as rows (padded by 16
// bytes, so that the two 32-lane halves of a gather, 4 keys apart, fall on
// different banks), then each thread gathers whole 16-byte lanes.
// Key `key` of head h is read at v + b sb + s ss + (g hg + h) sh with
// g = key / piece, s = key % piece: piece = Skv for a plain V; for the
// Ulysses regroup fused in, V is the regrouped [B, P * S_local, H / P, D]
// read from the sequence-sharded [B, S_local, H, D] (piece = S_local, hg = H / P).
template <int D>
__global__ void __launch_bounds__(256) pack_v_kernel(const uint16_t* __restrict__ v, int64_t sb, int64_t ss,
                                                     int64_t sh, uint16_t* __restrict__ out, int H, int Skv,
                                                     int n_tiles, uint32_t piece, int hg) {
  constexpr int RS = D + 8;            // LDS row stride, elements
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int NF = (D / 32) * 4;     // fragments per tile
  constexpr int NLD = 64 * CPR / 256;  // 16-byte loads per thread
  constexpr int NST = NF * 64 / 256;   // 16-byte stores per thread
  __shared__ __attribute__((aligned(16))) uint16_t rows[64 * RS];
  const int wg = blockIdx.x;
  const int t = wg % n_tiles, bh = wg / n_tiles;
  const int h = bh % H, b = bh / H;
  const uint16_t* src = v + b * sb + h * sh;
  // every load in flight before the first LDS store
  uint4 x[NLD];
#pragma unroll
  for (int it = 0; it < NLD; ++it) {
    const int i = threadIdx.x + it * 256;
    const int key = t * 64 + i / CPR;
    // rows past Skv load the last row (no branch around the load) and are zeroed
    const uint32_t kc = (uint32_t)min(key, Skv - 1);
    const uint32_t g = kc / piece, sk = kc - g * piece;
    const uint4 y = *reinterpret_cast<const uint4*>(src + (int64_t)sk * ss + (int64_t)(g * hg) * sh + (i % CPR) * 8);
    const bool in = key < Skv;
    x[it] = make_uint4(in ? y.x : 0u, in ? y.y : 0u, in ? y.z : 0u, in ? y.w : 0u);
  }
#pragma unroll
  for (int it = 0; it < NLD; ++it) {
    const int i = threadIdx.x + it * 256;
    *reinterpret_cast<uint4*>(rows + (i / CPR) * RS + (i % CPR) * 8) = x[it];
  }
  __syncthreads();
  uint16_t* dst = out + ((int64_t)bh * n_tiles + t) * (NF * 512);
#pragma unroll
  for (int it = 0; it < NST; ++it) {
    const int i = threadIdx.x + it * 256;
    const int f = i / 64, l = i % 64;
    const int db = f / 4, kb = (f / 2) % 2, kk2 = f % 2;
    const int d = db * 32 + (l & 31), k0 = kb * 32 + kk2 * 16 + 4 * (l >> 5);
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = rows[(k0 + 8 * (j >> 2) + (j & 3)) * RS + d];
    uint4 y;
    y.x = e[0] | ((uint32_t)e[1] << 16);
    y.y = e[2] | ((uint32_t)e[3] << 16);
    y.z = e[4] | ((uint32_t)e[5] << 16);
    y.w = e[6] | ((uint32_t)e[7] << 16);
    *reinterpret_cast<uint4*>(dst + i * 8) = y;
  }
}

}  // namespace

int64_t packed_v_bytes(int B, int H, int D, int Skv) {
  return (int64_t)B * H * ((Skv + 63) / 64) * 64 * D * 2;
}

hipError_t launch_pack_v(const void* v, Strides vs, void* packed, int B, int H, int D, int Skv, int piece,
                         hipStream_t stream) {
  const int n_tiles = (Skv + 63) / 64;
  const int64_t n_wg = (int64_t)B * H * n_tiles;
  if (n_wg == 0) return hipSuccess;
  if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
  const uint16_t* src = static_cast<const uint16_t*>(v);
  uint16_t* dst = static_cast<uint16_t*>(packed);
  if (piece <= 0 || Skv % piece) return hipErrorInvalidValue;
  if (D == 128)
    hipLaunchKernelGGL(pack_v_kernel<128>, dim3((int)n_wg), dim3(256), 0, stream, src, vs.b, vs.s, vs.h, dst, H,
                       Skv, n_tiles, (uint32_t)piece, H);
  else if (D == 64)
    hipLaunchKernelGGL(pack_v_kernel<64>, dim3((int)n_wg), dim3(256), 0, stream, src, vs.b, vs.s, vs.h, dst, H,
                       Skv, n_tiles, (uint32_t)piece, H);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Workgroup shape for one launch. The ping-pong kernel (8 waves, 256 query
// rows, one workgroup per CU) is the faster one per workgroup; the 4-wave
// kernel (128 rows, two workgroups per CU) spreads a small grid, or a nearly
// empty last round of workgroups, over twice as many CUs, and a workgroup
// alone on a CU runs at full speed. So: ping-pong unless its grid is under
// four rounds of 256 workgroups and its last (or only) round is less than
// half full.
int pick_waves(const FwdArgs& a) {
  if (a.D != 128 || CP_FWD_QB != 1) return 4;
  if (a.waves != 0) return a.waves;
  if (CP_FWD_NW != 0) return CP_FWD_NW;
  const int64_t n_wg8 = (int64_t)((a.Sq + 255) / 256) * a.H * a.B;
  const int64_t rounds = (n_wg8 + 255) / 256, last = n_wg8 - (rounds - 1) * 256;
  return (rounds < 4 && last < 128) ? 4 : 8;
}

template <int D>
hipError_t launch_dn(const FwdArgs& a, hipStream_t stream) {
  if constexpr (D == 128 && CP_FWD_QB == 1) {
    if (pick_waves(a) == 8) return launch_dw<D, 8>(a, stream);
  }
  return launch_dw<D, 4>(a, stream);
}

// The merges of the ring launch read past the L1, so no stale copy of a tile
// can be hit however many blocks merge into it.
int ring_max_blocks() { return CP_FWD_QB != 1 ? 0 : kMaxRingBlocks; }

int seq_max_blocks() { return (CP_FWD_SEQ && CP_FWD_QB == 1) ? kMaxRingBlocks : 0; }

hipError_t launch_ring_seq_bf16(const FwdArgs& a, const RingBlocks& rb, hipStream_t stream) {
  if constexpr (CP_FWD_SEQ && CP_FWD_QB == 1) {
    if (a.D != 128 || !a.v_packed) return hipErrorInvalidValue;
    return launch_seq_128(a, rb, stream);
  }
  return hipErrorInvalidValue;
}

int64_t ring_flag_count(int B, int H, int Sq) { return (int64_t)((Sq + 255) / 256) * H * B; }


hipError_t launch_ring_bf16(const FwdArgs& a, const RingBlocks& rb, int* ws, hipStream_t stream) {
  if constexpr (CP_FWD_QB == 1) {
    // packed V only: with V transposed in the kernel the ring variant spills heavily
    if (a.D != 128 || !a.v_packed) return hipErrorInvalidValue;
    return launch_ring_128<true>(a, rb, ws, stream);
  }
  return hipErrorInvalidValue;
}

#if CP_FWD_PHASE_TRACE
// Diagnostic builds only (not part of the C ABI header): copy the first n values of g_phase.
extern "C" int cp_debug_phase_trace(unsigned long long* host, long n) {
  const long total = (long)kPhaseWg * 8 * kPhaseVals;
  if (host == nullptr || n < 0 || n > total) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase), (size_t)n * 8, 0, hipMemcpyDeviceToHost);
}
#endif

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch_dn<128>(a, stream);
  if (a.D == 64) return launch_dn<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
