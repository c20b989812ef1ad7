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
// (b, h); the K/V block is streamed through LDS in tiles of BN keys):
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_f32_32x32x16_bf16: the A operand is a K tile read from LDS, the
//     B operand is the wave's Q held in registers for the whole block. In the
//     32x32 accumulator layout lane l holds query (l % 32) and 16 keys, so the
//     row statistics of the online softmax are lane-local plus one swap of
//     the two 32-lane halves (v_permlane32_swap).
//   * The output is accumulated transposed too, O^T += V^T . P^T: the B
//     operand P^T is exactly the softmax'd score registers converted to bf16
//     (no data movement); the contraction order over keys is permuted to
//     match and the V^T tile is stored in LDS in that permuted key order.
//     Each lane's O registers all belong to its own query row, so the
//     rescale by exp(m_old - m_new) needs no cross-lane traffic.
//   * V is transposed while it is written to LDS (four keys x eight dims per
//     thread, 8-byte LDS stores), so every MFMA operand read is one 16-byte
//     LDS load. Rows are XOR-swizzled in 16-byte units so the 16-byte reads
//     of 8 (or 16) consecutive lanes land in distinct banks.
//   * Two LDS stages: tile j+1 is fetched from global memory into registers
//     while tile j is computed, then stored to the other stage; one barrier
//     per tile.
//   * The exponent uses base 2 with scale*log2(e) folded into one FMA.
//   * Workgroups are remapped so that consecutive query tiles of one head run
//     on the same XCD (each XCD has its own L2) and share its K/V reads.
//   * Keys beyond Skv are never read (zero-filled in LDS) and get score
//     -inf; query rows beyond Sq are computed on zeros and not stored.
#include <stdint.h>

#include "kernels.h"

#ifndef CP_FWD_QB
#define CP_FWD_QB 1  // 32-query blocks per wave
#endif
#ifndef CP_FWD_BN
#define CP_FWD_BN 64  // keys per LDS tile
#endif
#ifndef CP_FWD_NW
#define CP_FWD_NW 4  // waves per workgroup
#endif
#ifndef CP_FWD_WPE
#define CP_FWD_WPE 2  // minimum waves per SIMD the register budget must allow
#endif

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
  int n_wg;  // total workgroups
  float c;   // scale * log2(e)
};

// 16-byte-unit XOR swizzle for a row of NCH 16-byte chunks. For NCH >= 16
// any 16 consecutive rows map one chunk index to 16 distinct chunks; for
// NCH == 8 any 8 consecutive rows, and each parity class of 16 consecutive
// rows, map to 8 distinct chunks.
template <int NCH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (NCH >= 16) {
    return r & (NCH - 1);
  } else {
    return (r ^ (r >> 3)) & (NCH - 1);
  }
}

// Both 32-lane halves of a wave64 end up with max/sum over the pair (l, l^32).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Map the hardware workgroup id (dispatched round-robin over 8 XCDs) to a
// logical tile id so that each XCD receives one contiguous range of tiles.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, loc = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
}

template <int D, int QB, int BN, int NW>
struct Cfg {
  static constexpr int BM = NW * QB * 32;    // query rows per workgroup
  static constexpr int NT = NW * 64;         // threads per workgroup
  static constexpr int DCH = D / 8;          // 16-byte chunks per K row
  static constexpr int KROW = D * 2;         // bytes per K row in LDS
  static constexpr int K_BYTES = BN * KROW;  // K tile
  static constexpr int KCH = BN / 8;         // 16-byte chunks per V^T row
  static constexpr int VROW = BN * 2;        // bytes per V^T row (one head dim)
  static constexpr int V_BYTES = D * VROW;   // V^T tile
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int KL = BN * DCH / NT;             // K chunks per thread
  static constexpr int VL = (BN / 4) * (D / 8) / NT;   // (4 keys x 8 dims) V tasks per thread
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert((BN * DCH) % NT == 0 && ((BN / 4) * (D / 8)) % NT == 0, "staging split");
  static_assert(KL >= 1 && VL >= 1, "staging split");
};

template <int D, int QB, int BN, int NW, bool ACC>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                               amdgpu_waves_per_eu(D == 64 ? 1 : CP_FWD_WPE)))
attn_fwd_bf16_kernel(Params p) {
  using C = Cfg<D, QB, BN, NW>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, p.n_wg);
  const int qt = tile % p.n_qt;
  const int bh = tile / p.n_qt;
  const int h = bh % p.H, b = bh / p.H;
  const int qrow0 = qt * C::BM + wave * (QB * 32);

  const uint16_t* kbase = p.k + b * p.kv_sb + h * p.kv_sh;
  const uint16_t* vbase = p.v + b * p.kv_sb + h * p.kv_sh;

  // ---- Q (B operand of S^T = K Q^T): lane holds query l32, dims kk*16 + hi*8 .. +7
  bf16x8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + l32;
    const uint16_t* qp = p.q + b * p.q_sb + (int64_t)row * p.q_ss + h * p.q_sh + hi * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (row < p.Sq) {
        qf[qb][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
      } else {
        qf[qb][kk] = bf16x8{};
      }
    }
  }

  // ---- global -> register staging of one K/V tile
  u32x4 kreg[C::KL];
  u32x4 vreg[C::VL][4];
  auto gload = [&](int key0) {
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
      const int cid = tid + i * C::NT;
      const int n = cid / C::DCH, c = cid % C::DCH;
      const int key = key0 + n;
      kreg[i] = (key < p.Skv)
                    ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * p.kv_ss + c * 8)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < C::VL; ++i) {
      const int task = tid + i * C::NT;
      const int dq = task % (D / 8), kq = task / (D / 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + kq * 4 + e;
        vreg[i][e] = (key < p.Skv)
                         ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * p.kv_ss + dq * 8)
                         : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // ---- register -> LDS: K row-major (swizzled); V transposed, keys in MFMA order
  auto swrite = [&](int stage) {
    char* Ks = smem + stage * C::STAGE;
    char* Vs = Ks + C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
      const int cid = tid + i * C::NT;
      const int n = cid / C::DCH, c = cid % C::DCH;
      *reinterpret_cast<u32x4*>(Ks + n * C::KROW + ((c ^ swz<C::DCH>(n)) << 4)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VL; ++i) {
      const int task = tid + i * C::NT;
      const int dq = task % (D / 8), kq = task / (D / 8);
      // Within each 16-key group the keys are stored in the order
      // 0-3, 8-11, 4-7, 12-15: the key order of the P^T registers.
      const int quad = kq & 3;
      const int pos = (quad == 1) ? 2 : (quad == 2) ? 1 : quad;
      const int p0 = (kq >> 2) * 16 + pos * 4;
      const int ch = p0 >> 3, off = (p0 & 7) * 2;
      const u32x4 v0 = vreg[i][0], v1 = vreg[i][1], v2 = vreg[i][2], v3 = vreg[i][3];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int de = dq * 8 + 2 * w, dodd = de + 1;
        const u32x2 even = {(v0[w] & 0xffffu) | (v1[w] << 16), (v2[w] & 0xffffu) | (v3[w] << 16)};
        const u32x2 odd = {(v0[w] >> 16) | (v1[w] & 0xffff0000u), (v2[w] >> 16) | (v3[w] & 0xffff0000u)};
        *reinterpret_cast<u32x2*>(Vs + de * C::VROW + ((ch ^ swz<C::KCH>(de)) << 4) + off) = even;
        *reinterpret_cast<u32x2*>(Vs + dodd * C::VROW + ((ch ^ swz<C::KCH>(dodd)) << 4) + off) = odd;
      }
    }
  };

  f32x16 o[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[qb][db] = f32x16{};
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const int n_tiles = (p.Skv + BN - 1) / BN;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int key0 = j * BN;
    const bool has_next = (j + 1) < n_tiles;
    if (has_next) gload(key0 + BN);

    const char* Ks = smem + (j & 1) * C::STAGE;
    const char* Vs = Ks + C::K_BYTES;

    // ---- S^T = K Q^T for BN keys x (QB*32) queries
    f32x16 s[QB][BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      const int n = kb * 32 + l32;
      const char* krow = Ks + n * C::KROW;
      const int sw = swz<C::DCH>(n);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((kk * 2 + hi) ^ sw) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][kk], s[qb][kb], 0, 0, 0);
      }
    }

    // ---- tail mask: keys >= Skv get -inf (only the last tile can have them)
    if (key0 + BN > p.Skv) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= p.Skv) s[qb][kb][r] = -INFINITY;
          }
    }

    // ---- online softmax (base 2), P^T in bf16
    bf16x8 pf[QB][BN / 32][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = half_max(mx);
      const float m_new = fmaxf(m_run[qb], mx * p.c);
      const float alpha = fast_exp2(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(s[qb][kb][r], p.c, -m_new));
          s[qb][kb][r] = e;
          ls += e;
        }
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          bf16x8 t;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) t[jj] = (__bf16)s[qb][kb][kk2 * 8 + jj];
          pf[qb][kb][kk2] = t;
        }
      }
      l_run[qb] = l_run[qb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[qb][db] *= alpha;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + l32;
      const char* vrow = Vs + d * C::VROW;
      const int sw = swz<C::KCH>(d);
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(vrow + (((kb * 4 + kk2 * 2 + hi) ^ sw) << 4));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kb][kk2], o[qb][db], 0, 0, 0);
        }
    }

    if (has_next) swrite((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, LSE, optional merge into the accumulator
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + l32;
    const float lt = half_sum(l_run[qb]);
    const float lse2 = m_run[qb] + fast_log2(lt);  // log2 units
    const float inv = 1.0f / lt;
    if (row < p.Sq) {
      float* orow = p.out + b * p.o_sb + (int64_t)row * p.o_ss + h * p.o_sh;
      float* lrow = p.lse + ((int64_t)b * p.H + h) * p.Sq + row;
      if constexpr (ACC) {
        const float la2 = *lrow * kLog2e;
        const float M = fmaxf(la2, lse2);
        const float wa = fast_exp2(la2 - M);  // 0 when the accumulator is empty (-inf)
        const float wb = fast_exp2(lse2 - M);
        const float tot = wa + wb;
        const float fa = wa / tot, fb = (wb / tot) * inv;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4* dst = reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi);
            const f32x4 ob = {o[qb][db][4 * g], o[qb][db][4 * g + 1], o[qb][db][4 * g + 2],
                              o[qb][db][4 * g + 3]};
            const f32x4 oa = *dst;
            *dst = (wa > 0.f) ? (fa * oa + fb * ob) : (fb * ob);
          }
        if (hi == 0) *lrow = (M + fast_log2(tot)) * kLn2;
      } else {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 ob = {o[qb][db][4 * g], o[qb][db][4 * g + 1], o[qb][db][4 * g + 2],
                              o[qb][db][4 * g + 3]};
            *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = ob * inv;
          }
        if (hi == 0) *lrow = lse2 * kLn2;
      }
    }
  }
}

template <int D, bool ACC>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  // D = 64 uses 128-key tiles so that every thread has a (4 keys x 8 dims) V task.
  constexpr int QB = CP_FWD_QB, NW = CP_FWD_NW, BN = (D == 64) ? 128 : CP_FWD_BN;
  using C = Cfg<D, QB, BN, NW>;
  Params p;
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
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, QB, BN, NW, ACC>), dim3(p.n_wg), dim3(C::NT), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.accumulate ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  if (a.D == 64) return a.accumulate ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
