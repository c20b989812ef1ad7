// Backward of one ring block, bf16 inputs, float32 gradients, on gfx950
// matrix cores.
//
// What it computes: ring attention serves training as well as inference
// ("Paralelismo", introduction; "Paralelismo de contexto", the variants table
// and the note under "Ring Anything Attention" restrict only Ring Anything to
// inference). With O and LSE the merged (full-ring)
// forward results and dO the gradient of the loss with respect to O, block i
// of a rank's ring contributes, for each (b, h):
//   P_ij  = exp(scale <q_i, k_j> - LSE_i)      (global softmax weights)
//   D_i   = sum_d dO_id O_id                    (bwd_prep)
//   dV_j  = sum_i P_ij dO_i                     (dkv kernel)
//   dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dK_j  = scale sum_i dS_ij q_i               (dkv kernel)
//   dQ_i += scale sum_j dS_ij k_j               (dq kernel, summed over blocks)
// the derivative of softmax attention; summed over the blocks these are the
// single-pass gradients.
//
// Design (reusing the forward's layouts, see attn_fwd_bf16.hip):
//   * bwd_prep: one 16- or 8-lane group per (b, s, h) row writes dO rounded
//     to bf16, the MFMA operand of both kernels, and computes D_i from that
//     rounded dO (so that dP - D is exact for the dO the products use).
//   * dq kernel, one lane per query as in the forward: S^T = K Q^T and
//     dP^T = V dO^T on v_mfma_f32_32x32x16_bf16 with Q and dO in registers,
//     K and V fragments from LDS; P^T and dS^T stay in the accumulator
//     registers (the row statistics LSE_i and D_i are per lane), and
//     dQ^T += K^T dS^T takes K^T from transposing LDS reads of a row-major
//     copy of the K tile and dS^T as bf16 in the accumulator's key order.
//     The next tile's S and dP run on the matrix cores while the vector ALUs
//     turn the current tile into dS (three LDS stages).
//   * dkv kernel, one lane per key: the same with the roles of queries and
//     keys exchanged: S = Q K^T and dP = dO V^T with K^T, V^T in registers and
//     Q, dO fragments from LDS; the accumulator rows are queries, so LSE_i and
//     D_i come per register from a small LDS table; dV^T += dO^T P and
//     dK^T += Q^T dS take dO^T and Q^T from transposing reads of row-major
//     copies.
//   * Tiles of 32 rows (keys for dq, queries for dkv) go from global memory
//     straight into LDS with buffer loads (descriptor ranges end at the valid
//     rows, so padding rows arrive as zeros), one barrier per tile. Padding queries have Q = dO = 0 and contribute nothing; padding
//     keys have their scores set to -inf in the dq kernel and their dK, dV
//     rows are not stored by the dkv kernel.
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

#ifndef CP_BWD_DKV_WPE
#define CP_BWD_DKV_WPE 2  // waves per SIMD the dkv kernel's register budget must allow (1 or 2)
#endif

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufferFlags = 0x00020000;  // word 3 of a raw buffer descriptor (gfx9 family)
constexpr int NW = 4;                     // waves per workgroup
constexpr int TR = 32;                    // rows per streamed tile

// 16 bytes per lane into LDS at lds + 16 * lane from base + voff, through a
// buffer descriptor covering [base, base + nbytes) (out-of-range lanes write
// zeros). base, nbytes and lds must be wave-uniform.
__device__ __forceinline__ void buffer_to_lds16(const void* base, int nbytes, int voff, char* lds) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 0);
}
// Same with 4 bytes per lane (lds + 4 * lane).
__device__ __forceinline__ void buffer_to_lds4(const void* base, int nbytes, int voff, char* lds) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 4, voff, 0, 0, 0);
}

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, loc = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
}

template <int D>
struct TileCfg {
  static constexpr int KK = D / 16;             // 16-dim MFMA steps
  static constexpr int ROW = D * 2;             // bytes per bf16 row
  static constexpr int BYTES = TR * ROW;        // one 32-row tile
  static constexpr int RPI = 1024 / ROW;        // rows per 1 KB load
  static constexpr int LPR = ROW / 16;          // lanes per row
  static constexpr int FRAG_LOADS = KK;         // 1 KB loads of a fragment-order tile
  static constexpr int ROW_LOADS = TR / RPI;    // 1 KB loads of a row-major tile
};

// XOR applied to a row's 16-byte chunk index in the row-major tiles (as in the
// forward's V tile): the rows one transposing read touches cover all banks.
template <int D>
__device__ __forceinline__ int row_swz(int r) {
  if constexpr (D == 128) {
    return (r & 3) << 2;
  } else {
    return ((r >> 1) & 1) << 2;
  }
}

// Per-lane byte offset of transposing reads (see row_swz): within a 16-lane
// group lane i supplies the address of row (i/4), dims 4*(i%4)..+3. The read
// at tile + (tr_lane ^ (db << 6)) + step*16*ROW yields the A operand
// [32 dims of block db] x [16 rows of step] in the accumulator's row order.
template <int D>
__device__ __forceinline__ int tr_lane_offset(int lane) {
  const int hi = lane >> 5;
  const int i16 = lane & 15, jq = i16 >> 2, q = i16 & 3, blk = (lane >> 4) & 1;
  const int sw = (D == 128) ? jq : (jq >> 1);
  return (4 * hi + jq) * TileCfg<D>::ROW + (sw << 6) + ((blk * 2 + (q >> 1)) << 4) + ((q & 1) << 3);
}

template <int D>
__device__ __forceinline__ bf16x8 tr_read(const char* tile, int tr_lane, int db, int step) {
  const char* a0 = tile + (tr_lane ^ (db << 6)) + step * 16 * TileCfg<D>::ROW;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
  const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * TileCfg<D>::ROW));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi4), 0, 1, 2, 3, 4,
                                 5, 6, 7);
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dob;   // dO in bf16, contiguous [B, Sq, H, D]
  const float* lse;      // [B, H, Sq]
  const float* delta;    // [B, H, Sq]
  float* dq;
  float* dk;
  float* dv;
  int64_t q_sb, q_ss, q_sh;
  int64_t kv_sb, kv_ss, kv_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dkv_sb, dkv_ss, dkv_sh;
  int B, H, Sq, Skv;
  int n_t;   // row tiles (of NW * 32) per (b, h)
  int n_wg;
  float c;   // scale * log2(e)
  float scale;
  // MULTI launches (all of a ring's non-empty blocks at once; the single-block
  // fields k, v, dk, dv, Skv unused): block i's K, V, dK, dV at its first key
  // (shared strides) and its length; dkv: wg0[i] = first workgroup of block i
  // in the remapped order, wg0[n_blk] = n_wg.
  int n_blk;
  const uint16_t* kblk[kMaxBwdBlocks];
  const uint16_t* vblk[kMaxBwdBlocks];
  float* dkblk[kMaxBwdBlocks];
  float* dvblk[kMaxBwdBlocks];
  int lblk[kMaxBwdBlocks];
  int wg0[kMaxBwdBlocks + 1];
};

// Global -> LDS loads of one 32-row tile starting at row r0 of a [rows, D]
// bf16 matrix (row stride rs elements, valid rows r_end), this wave's share:
// fragment order (1 KB block kk: row l%32, dims 16kk + 8(l/32)..+7) and/or
// row-major with swizzled chunks.
template <int D>
struct TileLoader {
  using T = TileCfg<D>;
  int frag_voff;            // lane's offset within a fragment block, minus the kk part
  int row_voff[(T::ROW_LOADS + NW - 1) / NW];
  int wave;
  __device__ void init(int wave_, int lane, int64_t row_bytes) {
    wave = wave_;
    frag_voff = (int)((lane & 31) * row_bytes) + (lane >> 5) * 16;
#pragma unroll
    for (int i = 0; i < (T::ROW_LOADS + NW - 1) / NW; ++i) {
      const int blk = wave + i * NW;
      const int r = blk * T::RPI + lane / T::LPR;
      row_voff[i] = (int)(r * row_bytes) + (((lane % T::LPR) ^ row_swz<D>(r)) << 4);
    }
  }
  // fragment-order tile: KK blocks split over the waves
  __device__ void frag(const uint16_t* base, int nbytes, char* lds) const {
#pragma unroll
    for (int i = 0; i < (T::KK + NW - 1) / NW; ++i) {
      const int kk = wave + i * NW;
      if (kk < T::KK) buffer_to_lds16(base, nbytes, frag_voff + kk * 32, lds + kk * 1024);
    }
  }
  __device__ void rows(const uint16_t* base, int nbytes, char* lds) const {
#pragma unroll
    for (int i = 0; i < (T::ROW_LOADS + NW - 1) / NW; ++i) {
      const int blk = wave + i * NW;
      if (blk < T::ROW_LOADS) buffer_to_lds16(base, nbytes, row_voff[i], lds + blk * 1024);
    }
  }
};

__device__ __forceinline__ int range_bytes(int rows_left, int64_t row_bytes) {
  const int64_t n = (int64_t)rows_left * row_bytes;
  return (int)(n < 0 ? 0 : (n > 0x7fffffff ? 0x7fffffff : n));
}

// ---------------------------------------------------------------- dQ kernel
//
// Software-pipelined over 32-key tiles: while the vector ALUs turn tile t's
// scores into dS_t, the matrix cores compute tile t+1's S and dP; then
// dQ += K_t^T dS_t. Three LDS stages: in iteration t the waves read tile t+1's
// fragments and tile t's row-major K, while tile t+2 is being loaded.

template <int D, bool ACC, bool MULTI = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2)))
attn_bwd_dq_kernel(BwdParams p) {
  using T = TileCfg<D>;
  __shared__ __attribute__((aligned(1024))) char kf0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char kf1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char kf2[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char vf0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char vf1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char vf2[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char kr0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char kr1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char kr2[T::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, p.n_wg);
  const int qt = tile % p.n_t, bh = tile / p.n_t;
  const int h = bh % p.H, b = bh / p.H;
  const int row = qt * (NW * 32) + wave * 32 + l32;  // this lane's query
  const bool valid = row < p.Sq;

  bf16x8 qf[T::KK], df[T::KK];
  {
    const uint16_t* qp = p.q + b * p.q_sb + (int64_t)row * p.q_ss + h * p.q_sh + hi * 8;
    const uint16_t* dp = p.dob + (((int64_t)b * p.Sq + row) * p.H + h) * D + hi * 8;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      qf[kk] = valid ? *reinterpret_cast<const bf16x8*>(qp + kk * 16) : bf16x8{};
      df[kk] = valid ? *reinterpret_cast<const bf16x8*>(dp + kk * 16) : bf16x8{};
    }
  }
  const int64_t stat = ((int64_t)b * p.H + h) * p.Sq + row;
  const float lse2 = valid ? p.lse[stat] * kLog2e : 0.f;
  const float dlt = valid ? p.delta[stat] : 0.f;

  const int64_t row_bytes = p.kv_ss * 2;
  TileLoader<D> ld;
  ld.init(wave, lane, row_bytes);
  const int tr_lane = tr_lane_offset<D>(lane);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  // MULTI: the blocks in turn, dQ accumulated in registers across them and
  // written once; a workgroup barrier before each later block's first loads
  // (the other waves may still read the previous block's last stages). The
  // loop is a backward jump only that instantiation has.
  int sblk = 0;
dq_next_block:
  if constexpr (MULTI) {
    if (sblk > 0) __syncthreads();
  }
  const int skv = MULTI ? p.lblk[sblk] : p.Skv;
  const uint16_t* kbase = (MULTI ? p.kblk[sblk] : p.k) + b * p.kv_sb + h * p.kv_sh;
  const uint16_t* vbase = (MULTI ? p.vblk[sblk] : p.v) + b * p.kv_sb + h * p.kv_sh;
  const int n_tiles = (skv + TR - 1) / TR;

  auto issue = [&](int t, char* kf, char* vf, char* kr) {
    const int64_t off = (int64_t)t * TR * p.kv_ss;
    const int nb = range_bytes(skv - t * TR, row_bytes);
    ld.frag(kbase + off, nb, kf);
    ld.frag(vbase + off, nb, vf);
    ld.rows(kbase + off, nb, kr);
  };
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // S^T = K Q^T and dP^T = V dO^T of one tile (16 MFMAs), fragments from LDS.
  auto scores = [&](const char* kf, const char* vf, f32x16& s, f32x16& dpt) {
    s = f32x16{};
    dpt = f32x16{};
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kf + kk * 1024 + lane * 16);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
      const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(vf + kk * 1024 + lane * 16);
      dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, df[kk], dpt, 0, 0, 0);
    }
  };
  // dS^T of tile t as bf16 B operands; this lane holds keys t*32 + 8*(r/4) +
  // 4*hi + r%4, and only the last tile can hold keys past Skv (P = 0 there).
  auto softmax = [&](auto last_tag, int t, const f32x16& s, const f32x16& dpt, bf16x8 (&dsb)[2]) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int lim = skv - t * TR - 4 * hi;
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = kk2 * 8 + jj;
        float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -lse2));
        if constexpr (LAST) pr = (8 * (r >> 2) + (r & 3) < lim) ? pr : 0.f;
        dsb[kk2][jj] = (__bf16)(pr * (dpt[r] - dlt));
      }
    }
  };
  // dQ^T += K^T dS^T for one tile (8 MFMAs), K^T from transposing reads.
  auto dq_update = [&](const char* kr, const bf16x8 (&dsb)[2]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(kr, tr_lane, db, kk2), dsb[kk2], acc[db], 0, 0, 0);
  };

  f32x16 s_cur, d_cur, s_nxt, d_nxt;
  // One iteration: tile t's softmax interleaved with tile t+1's scores, then
  // tile t's dQ update. Stage c holds tile t, stage n tile t+1, stage f is
  // free (tile t+2 goes there).
  auto iter = [&](int t, const char* kr_c, const char* kf_n, const char* vf_n, const char* kr_n, char* kf_f,
                  char* vf_f, char* kr_f) {
    sync();  // tile t+1 has landed; every wave is done with the free stage
    if (t + 2 < n_tiles) issue(t + 2, kf_f, vf_f, kr_f);
    bf16x8 dsb[2];
    if (t + 1 < n_tiles) {
      scores(kf_n, vf_n, s_nxt, d_nxt);
      softmax(std::false_type{}, t, s_cur, d_cur, dsb);
      // 16 MFMAs with their 16 fragment reads, ~80 VALU ops between them
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    } else {
      softmax(std::true_type{}, t, s_cur, d_cur, dsb);
    }
    dq_update(kr_c, dsb);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    s_cur = s_nxt;
    d_cur = d_nxt;
    (void)kr_n;
  };

  if (n_tiles > 0) {  // no keys: dQ = 0
    issue(0, kf0, vf0, kr0);
    if (n_tiles > 1) issue(1, kf1, vf1, kr1);
    __builtin_amdgcn_s_waitcnt(0);  // tiles 0 and 1 in LDS
    __syncthreads();
    scores(kf0, vf0, s_cur, d_cur);
  }
  int t = 0;
  for (; t + 3 <= n_tiles; t += 3) {
    iter(t, kr0, kf1, vf1, kr1, kf2, vf2, kr2);
    iter(t + 1, kr1, kf2, vf2, kr2, kf0, vf0, kr0);
    iter(t + 2, kr2, kf0, vf0, kr0, kf1, vf1, kr1);
  }
  if (t < n_tiles) iter(t, kr0, kf1, vf1, kr1, kf2, vf2, kr2);
  if (t + 1 < n_tiles) iter(t + 1, kr1, kf2, vf2, kr2, kf0, vf0, kr0);
  if constexpr (MULTI) {
    if (++sblk < p.n_blk) goto dq_next_block;
  }

  if (valid) {
    float* out = p.dq + b * p.dq_sb + (int64_t)row * p.dq_ss + h * p.dq_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4* dst = reinterpret_cast<f32x4*>(out + db * 32 + 8 * g + 4 * hi);
        const f32x4 val = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        if constexpr (ACC) {
          *dst = *dst + val * p.scale;
        } else {
          *dst = val * p.scale;
        }
      }
  }
}


// --------------------------------------------------------------- dKV kernel

template <int D, bool MULTI = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(CP_BWD_DKV_WPE)))
attn_bwd_dkv_kernel(BwdParams p) {
  using T = TileCfg<D>;
  __shared__ __attribute__((aligned(1024))) char qf0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char qf1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char df0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char df1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char qr0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char qr1[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char dr0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char dr1[T::BYTES];
  __shared__ __attribute__((aligned(256))) char st0[512];  // LSE (bytes 0..255) and D (256..511) of 32 queries
  __shared__ __attribute__((aligned(256))) char st1[512];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  // MULTI: one grid over every block's key tiles (block-major after the XCD
  // remap, so a block's tiles of one head stay on one XCD); the workgroup's
  // block is found in the wg0 table.
  int tile = xcd_remap(blockIdx.x, p.n_wg);
  int blk = 0;
  if constexpr (MULTI) {
    while (blk + 1 < p.n_blk && tile >= p.wg0[blk + 1]) ++blk;
    tile -= p.wg0[blk];
  }
  const int skv = MULTI ? p.lblk[blk] : p.Skv;
  const int n_t = MULTI ? (skv + NW * 32 - 1) / (NW * 32) : p.n_t;
  const int kt = tile % n_t, bh = tile / n_t;
  const int h = bh % p.H, b = bh / p.H;
  const int key = kt * (NW * 32) + wave * 32 + l32;  // this lane's key
  const bool valid = key < skv;

  // K^T and V^T as B operands: lane holds key l32, dims 16kk + 8hi..+7
  bf16x8 kt_[T::KK], vt_[T::KK];
  {
    const uint16_t* kp = (MULTI ? p.kblk[blk] : p.k) + b * p.kv_sb + (int64_t)key * p.kv_ss + h * p.kv_sh + hi * 8;
    const uint16_t* vp = (MULTI ? p.vblk[blk] : p.v) + b * p.kv_sb + (int64_t)key * p.kv_ss + h * p.kv_sh + hi * 8;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      kt_[kk] = valid ? *reinterpret_cast<const bf16x8*>(kp + kk * 16) : bf16x8{};
      vt_[kk] = valid ? *reinterpret_cast<const bf16x8*>(vp + kk * 16) : bf16x8{};
    }
  }

  const int64_t q_row_bytes = p.q_ss * 2;
  const int64_t d_row_bytes = (int64_t)p.H * D * 2;
  const uint16_t* qbase = p.q + b * p.q_sb + h * p.q_sh;
  const uint16_t* dbase = p.dob + ((int64_t)b * p.Sq * p.H + h) * D;
  const float* lbase = p.lse + ((int64_t)b * p.H + h) * p.Sq;
  const float* dlbase = p.delta + ((int64_t)b * p.H + h) * p.Sq;
  TileLoader<D> lq, ldo;
  lq.init(wave, lane, q_row_bytes);
  ldo.init(wave, lane, d_row_bytes);
  const int tr_lane = tr_lane_offset<D>(lane);
  const int n_tiles = (p.Sq + TR - 1) / TR;

  auto issue = [&](int t, char* qf, char* df, char* qr, char* dr, char* st) {
    const int rows_left = p.Sq - t * TR;
    lq.frag(qbase + (int64_t)t * TR * p.q_ss, range_bytes(rows_left, q_row_bytes), qf);
    lq.rows(qbase + (int64_t)t * TR * p.q_ss, range_bytes(rows_left, q_row_bytes), qr);
    ldo.frag(dbase + (int64_t)t * TR * p.H * D, range_bytes(rows_left, d_row_bytes), df);
    ldo.rows(dbase + (int64_t)t * TR * p.H * D, range_bytes(rows_left, d_row_bytes), dr);
    if (wave == 0) {  // 32 LSE and 32 D values (what lanes 32..63 fetch is not used)
      buffer_to_lds4(lbase + t * TR, range_bytes(rows_left, 4), lane * 4, st);
      buffer_to_lds4(dlbase + t * TR, range_bytes(rows_left, 4), lane * 4, st + 256);
    }
  };
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  f32x16 dva[D / 32], dka[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dva[db] = f32x16{};
    dka[db] = f32x16{};
  }

  auto step = [&](const char* qf, const char* df, const char* qr, const char* dr, const char* st) {
    // S and dP interleaved: each fragment read is consumed at once, which
    // keeps the register count within two waves per SIMD.
    f32x16 s = f32x16{}, dpm = f32x16{};
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qf + kk * 1024 + lane * 16);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kt_[kk], s, 0, 0, 0);
      const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(df + kk * 1024 + lane * 16);
      dpm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, vt_[kk], dpm, 0, 0, 0);
    }
    // Register r holds query 8*(r/4) + 4*hi + r%4 of the tile; its LSE and D
    // are 4 consecutive floats per group of 4 registers.
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + (8 * g + 4 * hi) * 4);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + 256 + (8 * g + 4 * hi) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -l4[e] * kLog2e));
        pb[r >> 3][r & 7] = (__bf16)pr;
        dsb[r >> 3][r & 7] = (__bf16)(pr * (dpm[r] - d4[e]));
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(dr, tr_lane, db, kk2), pb[kk2], dva[db], 0, 0, 0);
        dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(qr, tr_lane, db, kk2), dsb[kk2], dka[db], 0, 0, 0);
      }
  };

  issue(0, qf0, df0, qr0, dr0, st0);
  sync();
  int t = 0;
  for (; t + 2 <= n_tiles; t += 2) {
    issue(t + 1, qf1, df1, qr1, dr1, st1);
    step(qf0, df0, qr0, dr0, st0);
    sync();
    if (t + 2 < n_tiles) issue(t + 2, qf0, df0, qr0, dr0, st0);
    step(qf1, df1, qr1, dr1, st1);
    sync();
  }
  if (t < n_tiles) step(qf0, df0, qr0, dr0, st0);

  if (valid) {
    float* kout = (MULTI ? p.dkblk[blk] : p.dk) + b * p.dkv_sb + (int64_t)key * p.dkv_ss + h * p.dkv_sh;
    float* vout = (MULTI ? p.dvblk[blk] : p.dv) + b * p.dkv_sb + (int64_t)key * p.dkv_ss + h * p.dkv_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hi;
        const f32x4 kv = {dka[db][4 * g], dka[db][4 * g + 1], dka[db][4 * g + 2], dka[db][4 * g + 3]};
        const f32x4 vv = {dva[db][4 * g], dva[db][4 * g + 1], dva[db][4 * g + 2], dva[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(kout + d0) = kv * p.scale;
        *reinterpret_cast<f32x4*>(vout + d0) = vv;
      }
  }
}

// ------------------------------------------------------------------ prep

// dO rounded to bf16 (contiguous [B, Sq, H, D]) and D_i = sum_d dO_id O_id of that rounded dO.
// G = D / 8 lanes per (b, s, h) row, 8 elements each.
template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_prep_kernel(const float* __restrict__ out, Strides os, const float* __restrict__ dout, Strides ds,
                     uint16_t* __restrict__ dob, float* __restrict__ delta, int H, int Sq, int n_rows) {
  constexpr int G = D / 8;
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const int row = tid / G;  // (b * Sq + s) * H + h
  const int c = tid % G;
  const bool ok = row < n_rows;
  float acc = 0.f;
  if (ok) {
    const int bs = row / H, h = row - bs * H;
    const int b = bs / Sq, s = bs - b * Sq;
    const float* op = out + b * os.b + (int64_t)s * os.s + h * os.h + c * 8;
    const float* dp = dout + b * ds.b + (int64_t)s * ds.s + h * ds.h + c * 8;
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(op), o1 = *reinterpret_cast<const f32x4*>(op + 4);
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(dp), d1 = *reinterpret_cast<const f32x4*>(dp + 4);
    // D from dO as rounded for the products (dP = dO V^T takes the bfloat16 dO): then
    // dP - D is the exact difference for that dO, and cancels where it should (one key:
    // P = 1, O = v, dS = 0) instead of leaving dO's rounding error times |dO| |v|.
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = (__bf16)d0[e];
      w[4 + e] = (__bf16)d1[e];
      acc = fmaf(o0[e], (float)w[e], acc);
      acc = fmaf(o1[e], (float)w[4 + e], acc);
    }
    *reinterpret_cast<bf16x8*>(dob + (int64_t)row * D + c * 8) = w;
  }
  // sum over the G lanes of the row (aligned groups of G lanes in one wave)
#pragma unroll
  for (int m = 1; m < G; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (ok && c == 0) {
    const int bs = row / H, h = row - bs * H;
    const int b = bs / Sq, s = bs - b * Sq;
    delta[((int64_t)b * H + h) * Sq + s] = acc;
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dob = static_cast<const uint16_t*>(a.dout_b);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.q_sb = a.qs.b; p.q_ss = a.qs.s; p.q_sh = a.qs.h;
  p.kv_sb = a.kvs.b; p.kv_ss = a.kvs.s; p.kv_sh = a.kvs.h;
  p.dq_sb = a.dqs.b; p.dq_ss = a.dqs.s; p.dq_sh = a.dqs.h;
  p.dkv_sb = a.dkvs.b; p.dkv_ss = a.dkvs.s; p.dkv_sh = a.dkvs.h;
  p.B = a.B; p.H = a.H; p.Sq = a.Sq; p.Skv = a.Skv;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  // dQ
  p.n_t = (a.Sq + NW * 32 - 1) / (NW * 32);
  int64_t n = (int64_t)p.n_t * a.H * a.B;
  if (n > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.n_wg = (int)n;
  if (p.n_wg > 0) {  // no queries: no dQ
    hipStream_t sq = a.dq_stream ? a.dq_stream : stream;
    if (a.accumulate_dq) {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<D, true>), dim3(p.n_wg), dim3(NW * 64), 0, sq, p);
    } else {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<D, false>), dim3(p.n_wg), dim3(NW * 64), 0, sq, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dK, dV
  p.n_t = (a.Skv + NW * 32 - 1) / (NW * 32);
  n = (int64_t)p.n_t * a.H * a.B;
  if (n > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.n_wg = (int)n;
  if (p.n_wg == 0) return hipSuccess;  // no keys: no dK, dV
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<D>), dim3(p.n_wg), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_ring_d(const BwdArgs& a, const BwdBlocks& bb, hipStream_t stream) {
  if (bb.n < 1 || bb.n > kMaxBwdBlocks || a.accumulate_dq) return hipErrorInvalidValue;
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = nullptr;
  p.v = nullptr;
  p.dob = static_cast<const uint16_t*>(a.dout_b);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = a.dq;
  p.dk = nullptr;
  p.dv = nullptr;
  p.q_sb = a.qs.b; p.q_ss = a.qs.s; p.q_sh = a.qs.h;
  p.kv_sb = a.kvs.b; p.kv_ss = a.kvs.s; p.kv_sh = a.kvs.h;
  p.dq_sb = a.dqs.b; p.dq_ss = a.dqs.s; p.dq_sh = a.dqs.h;
  p.dkv_sb = a.dkvs.b; p.dkv_ss = a.dkvs.s; p.dkv_sh = a.dkvs.h;
  p.B = a.B; p.H = a.H; p.Sq = a.Sq; p.Skv = 0;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.n_blk = bb.n;
  int64_t tot = 0;
  for (int i = 0; i < kMaxBwdBlocks; ++i) {
    const bool in = i < bb.n;
    if (in && bb.len[i] < 1) return hipErrorInvalidValue;
    p.kblk[i] = in ? static_cast<const uint16_t*>(bb.k[i]) : nullptr;
    p.vblk[i] = in ? static_cast<const uint16_t*>(bb.v[i]) : nullptr;
    p.dkblk[i] = in ? bb.dk[i] : nullptr;
    p.dvblk[i] = in ? bb.dv[i] : nullptr;
    p.lblk[i] = in ? bb.len[i] : 0;
    p.wg0[i] = (int)tot;
    if (in) tot += (int64_t)((bb.len[i] + NW * 32 - 1) / (NW * 32)) * a.H * a.B;
    if (tot > 0x7fffffff) return hipErrorInvalidConfiguration;
  }
  p.wg0[kMaxBwdBlocks] = (int)tot;
  // dQ: one launch, the blocks in turn
  p.n_t = (a.Sq + NW * 32 - 1) / (NW * 32);
  const int64_t n = (int64_t)p.n_t * a.H * a.B;
  if (n > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.n_wg = (int)n;
  if (p.n_wg > 0) {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, false, true>), dim3(p.n_wg), dim3(NW * 64), 0,
                       a.dq_stream ? a.dq_stream : stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dK, dV: one grid over every block's key tiles
  p.n_t = 0;
  p.n_wg = (int)tot;
  if (p.n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, true>), dim3(p.n_wg), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_ring_bf16(const BwdArgs& a, const BwdBlocks& bb, hipStream_t stream) {
  if (a.D == 128) return launch_bwd_ring_d<128>(a, bb, stream);
  if (a.D == 64) return launch_bwd_ring_d<64>(a, bb, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd_prep(const float* out, Strides os, const float* dout, Strides ds, void* dout_b,
                                float* delta, int B, int H, int Sq, int D, hipStream_t stream) {
  const int64_t n_rows = (int64_t)B * Sq * H;
  if (n_rows == 0) return hipSuccess;
  const int64_t threads = n_rows * (D / 8);
  if (threads > 0x7fffffff) return hipErrorInvalidConfiguration;
  const unsigned g = (unsigned)((threads + 255) / 256);
  if (D == 128) {
    hipLaunchKernelGGL(attn_bwd_prep_kernel<128>, dim3(g), dim3(256), 0, stream, out, os, dout, ds,
                       static_cast<uint16_t*>(dout_b), delta, H, Sq, (int)n_rows);
  } else if (D == 64) {
    hipLaunchKernelGGL(attn_bwd_prep_kernel<64>, dim3(g), dim3(256), 0, stream, out, os, dout, ds,
                       static_cast<uint16_t*>(dout_b), delta, H, Sq, (int)n_rows);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch_bwd_d<128>(a, stream);
  if (a.D == 64) return launch_bwd_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
