// Partial attention of a local Q slice against one K/V block with float32
// inputs, float32 output + LSE (same definition as the bf16 kernel:
// "Paralelismo de contexto", "Atencao em Anel"; "Paralelismo",
// ContextParallelConfig, convert_to_fp32).
//
// The float32 path keeps every product and sum in float32 on the vector ALUs
// so that it stays within float32 rounding of the exact result. It serves
// small float32 problems; large workloads use the bf16 matrix-core kernel.
//
// Layout: a workgroup of 128 threads owns 16 query rows of one (b, h); each
// row is split over a group of 8 consecutive lanes, each holding an eighth of
// D of the query and of the output accumulator. K/V are staged through LDS in
// tiles of 64 keys (zero-filled past Skv) and read back as float4 vectors.
// Scores of a tile are partial dot products per lane plus three exchanges
// within the group (lane ^ 1, ^ 2, ^ 4), after which all eight lanes hold the
// same scores, maxima and sums. The work per lane, which sets the latency of
// these small problems, is an eighth of the row's.
//
// A ring of 2 to 4 non-empty blocks can run as one launch (ring kernel
// below): a workgroup holds one 128-thread group per block for the same 16
// query rows, each group computes its block's partial (unnormalised output,
// row maximum and sum) in its own LDS tiles, and the partials are merged in
// block order by the LSE recombination of the per-block epilogue, in
// registers and LDS instead of through (out, lse) in memory. At the small
// sizes this path serves, one launch instead of one per block is what the
// time is made of.
#include <stdint.h>

#include "kernels.h"

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRows = 16;   // query rows per workgroup
constexpr int kTile = 64;   // keys per LDS tile
constexpr int kThreads = 128;
constexpr int kLanesPerRow = 8;

struct Params {
  const float* q;
  const float* k;
  const float* v;
  float* out;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t kv_sb, kv_ss, kv_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, H, Sq, Skv, n_qt;
  float c;  // scale * log2(e)
};

// K and V rows key0 .. key0 + TILE - 1 of one (b, h) into LDS (zeros past
// skv), as float4 words spread over NT threads.
template <int D, int TILE, int NT>
__device__ __forceinline__ void stage_tile(const float* kbase, const float* vbase, int64_t ss, int key0,
                                           int skv, int t, float (*Ks)[D], float (*Vs)[D]) {
#pragma unroll
  for (int it = 0; it < TILE * (D / 4) / NT; ++it) {
    const int idx = t + it * NT;
    const int n = idx / (D / 4), c4 = idx % (D / 4);
    const int key = key0 + n;
    f32x4 kx{}, vx{};
    if (key < skv) {
      kx = *reinterpret_cast<const f32x4*>(kbase + (int64_t)key * ss + c4 * 4);
      vx = *reinterpret_cast<const f32x4*>(vbase + (int64_t)key * ss + c4 * 4);
    }
    *reinterpret_cast<f32x4*>(&Ks[n][c4 * 4]) = kx;
    *reinterpret_cast<f32x4*>(&Vs[n][c4 * 4]) = vx;
  }
}

// Online-softmax update of one query row (this lane's eighth of D: qv, o)
// with the TILE keys staged in Ks/Vs: scores (keys >= skv masked to -inf),
// running maximum m (log2 units) and sum l, output rescaled and accumulated.
template <int D, int TILE>
__device__ __forceinline__ void tile_update(const float (&qv)[D / kLanesPerRow], const float (*Ks)[D],
                                            const float (*Vs)[D], int part, int key0, int skv, float c,
                                            float (&o)[D / kLanesPerRow], float& m, float& l) {
  constexpr int DQ = D / kLanesPerRow;
  float sc[TILE];
  float mt = -INFINITY;
#pragma unroll
  for (int j = 0; j < TILE; ++j) {
    float part_sum = 0.f;
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f32x4 kx = *reinterpret_cast<const f32x4*>(&Ks[j][part * DQ + i]);
      part_sum = fmaf(qv[i], kx[0], part_sum);
      part_sum = fmaf(qv[i + 1], kx[1], part_sum);
      part_sum = fmaf(qv[i + 2], kx[2], part_sum);
      part_sum = fmaf(qv[i + 3], kx[3], part_sum);
    }
    // the group's eight partial sums, added pairwise: the same value in every lane
    const float s01 = part_sum + __shfl_xor(part_sum, 1);
    const float s03 = s01 + __shfl_xor(s01, 2);
    const float full = s03 + __shfl_xor(s03, 4);
    sc[j] = (key0 + j < skv) ? full * c : -INFINITY;
    mt = fmaxf(mt, sc[j]);
  }
  const float m_new = fmaxf(m, mt);
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  m = m_new;
  l *= alpha;
#pragma unroll
  for (int i = 0; i < DQ; ++i) o[i] *= alpha;
#pragma unroll
  for (int j = 0; j < TILE; ++j) {
    const float pj = __builtin_amdgcn_exp2f(sc[j] - m_new);
    l += pj;
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f32x4 vx = *reinterpret_cast<const f32x4*>(&Vs[j][part * DQ + i]);
      o[i] = fmaf(pj, vx[0], o[i]);
      o[i + 1] = fmaf(pj, vx[1], o[i + 1]);
      o[i + 2] = fmaf(pj, vx[2], o[i + 2]);
      o[i + 3] = fmaf(pj, vx[3], o[i + 3]);
    }
  }
}

template <int D, bool ACC>
__global__ void __launch_bounds__(kThreads) attn_fwd_f32_kernel(Params p) {
  constexpr int DQ = D / kLanesPerRow;  // dims per lane
  __shared__ __attribute__((aligned(16))) float Ks[kTile][D];
  __shared__ __attribute__((aligned(16))) float Vs[kTile][D];

  const int tid = threadIdx.x;
  const int qi = tid / kLanesPerRow, part = tid % kLanesPerRow;
  const int qt = blockIdx.x % p.n_qt;
  const int bh = blockIdx.x / p.n_qt;
  const int h = bh % p.H, b = bh / p.H;
  const int row = qt * kRows + qi;

  float qv[DQ], o[DQ];
  {
    const float* qp = p.q + b * p.q_sb + (int64_t)row * p.q_ss + h * p.q_sh + part * DQ;
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f32x4 x = (row < p.Sq) ? *reinterpret_cast<const f32x4*>(qp + i) : f32x4{};
      qv[i] = x[0]; qv[i + 1] = x[1]; qv[i + 2] = x[2]; qv[i + 3] = x[3];
    }
  }
#pragma unroll
  for (int i = 0; i < DQ; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const float* kbase = p.k + b * p.kv_sb + h * p.kv_sh;
  const float* vbase = p.v + b * p.kv_sb + h * p.kv_sh;

  for (int key0 = 0; key0 < p.Skv; key0 += kTile) {
    __syncthreads();
    stage_tile<D, kTile, kThreads>(kbase, vbase, p.kv_ss, key0, p.Skv, tid, Ks, Vs);
    __syncthreads();
    tile_update<D, kTile>(qv, Ks, Vs, part, key0, p.Skv, p.c, o, m, l);
  }

  if (row >= p.Sq) return;
  const float lse2 = m + __builtin_amdgcn_logf(l);
  const float inv = 1.0f / l;
  float* orow = p.out + b * p.o_sb + (int64_t)row * p.o_ss + h * p.o_sh + part * DQ;
  float* lrow = p.lse + ((int64_t)b * p.H + h) * p.Sq + row;
  if constexpr (ACC) {
    const float la2 = *lrow * kLog2e;
    const float M = fmaxf(la2, lse2);
    const float wa = __builtin_amdgcn_exp2f(la2 - M);
    const float wb = __builtin_amdgcn_exp2f(lse2 - M);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = (wb / tot) * inv;
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      f32x4* dst = reinterpret_cast<f32x4*>(orow + i);
      const f32x4 ob = {o[i], o[i + 1], o[i + 2], o[i + 3]};
      const f32x4 oa = *dst;
      *dst = (wa > 0.f) ? (fa * oa + fb * ob) : (fb * ob);
    }
    // every lane of the group read lse above; only lane 0 writes it, after
    // the group's reads (they come first in program order within the wave)
    if (part == 0) *lrow = (M + __builtin_amdgcn_logf(tot)) * kLn2;
  } else {
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f32x4 ob = {o[i], o[i + 1], o[i + 2], o[i + 3]};
      *reinterpret_cast<f32x4*>(orow + i) = ob * inv;
    }
    if (part == 0) *lrow = lse2 * kLn2;
  }
}

// (acc_o, acc_lse) <- (acc_o, acc_lse) (+) block partial, the arithmetic of the
// accumulating epilogue above: acc_o is a normalised output, acc_lse a natural
// log (as stored in lse), o the block's unnormalised output with inv = 1 / its
// row sum and lse2 its LSE in log2 units.
template <int DQ>
__device__ __forceinline__ void merge_partial(float (&acc_o)[DQ], float& acc_lse, const float (&o)[DQ], float lse2,
                                              float inv) {
  const float la2 = acc_lse * kLog2e;
  const float M = fmaxf(la2, lse2);
  const float wa = __builtin_amdgcn_exp2f(la2 - M);
  const float wb = __builtin_amdgcn_exp2f(lse2 - M);
  const float tot = wa + wb;
  const float fa = wa / tot, fb = (wb / tot) * inv;
#pragma unroll
  for (int i = 0; i < DQ; i += 4) {
    const f32x4 ob = {o[i], o[i + 1], o[i + 2], o[i + 3]};
    const f32x4 oa = {acc_o[i], acc_o[i + 1], acc_o[i + 2], acc_o[i + 3]};
    const f32x4 r = (wa > 0.f) ? (fa * oa + fb * ob) : (fb * ob);
    acc_o[i] = r[0]; acc_o[i + 1] = r[1]; acc_o[i + 2] = r[2]; acc_o[i + 3] = r[3];
  }
  acc_lse = (M + __builtin_amdgcn_logf(tot)) * kLn2;
}

struct RingParams {
  const float* q;
  float* out;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t kv_sb, kv_ss, kv_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, H, Sq, n_qt;
  int n_iter;  // tiles of the longest block: every group runs this many barrier pairs
  float c;     // scale * log2(e)
  const float* k[kMaxF32RingBlocks];
  const float* v[kMaxF32RingBlocks];
  int len[kMaxF32RingBlocks];
};

// One launch over G = 2..4 non-empty ring blocks. Group g (threads 128 g ..
// 128 g + 127, two whole waves) computes block g's partial for the
// workgroup's 16 query rows with tiles of TILE keys in its own LDS; all
// groups pass the same barriers (n_iter pairs; a group whose block has run
// out of tiles idles through them). The partials meet in LDS and group 0
// merges them in block order, as the per-block launches would through
// (out, lse).
template <int D, int G>
__global__ void __launch_bounds__(kThreads * G) attn_fwd_f32_ring_kernel(RingParams p) {
  constexpr int DQ = D / kLanesPerRow;
  constexpr int TILE = D == 64 ? 64 : 32;  // 32 KB of K + V tiles per group
  static_assert(kRows * D + 2 * kRows <= TILE * D, "a group's partial fits in its K tile");
  __shared__ __attribute__((aligned(16))) float Ks[G][TILE][D];
  __shared__ __attribute__((aligned(16))) float Vs[G][TILE][D];

  const int grp = threadIdx.x / kThreads;  // uniform within a wave
  const int t = threadIdx.x % kThreads;
  const int qi = t / kLanesPerRow, part = t % kLanesPerRow;
  const int qt = blockIdx.x % p.n_qt;
  const int bh = blockIdx.x / p.n_qt;
  const int h = bh % p.H, b = bh / p.H;
  const int row = qt * kRows + qi;

  float qv[DQ], o[DQ];
  {
    const float* qp = p.q + b * p.q_sb + (int64_t)row * p.q_ss + h * p.q_sh + part * DQ;
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f32x4 x = (row < p.Sq) ? *reinterpret_cast<const f32x4*>(qp + i) : f32x4{};
      qv[i] = x[0]; qv[i + 1] = x[1]; qv[i + 2] = x[2]; qv[i + 3] = x[3];
    }
  }
#pragma unroll
  for (int i = 0; i < DQ; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int skv = p.len[grp];
  const float* kbase = p.k[grp] + b * p.kv_sb + h * p.kv_sh;
  const float* vbase = p.v[grp] + b * p.kv_sb + h * p.kv_sh;
  for (int it = 0; it < p.n_iter; ++it) {
    const int key0 = it * TILE;
    __syncthreads();
    if (key0 < skv) stage_tile<D, TILE, kThreads>(kbase, vbase, p.kv_ss, key0, skv, t, Ks[grp], Vs[grp]);
    __syncthreads();
    if (key0 < skv) tile_update<D, TILE>(qv, Ks[grp], Vs[grp], part, key0, skv, p.c, o, m, l);
  }

  // every group's partial into the (now free) K tile of its group:
  // [kRows][D] unnormalised output, then kRows LSEs (log2 units), kRows 1/sum
  const float lse2 = m + __builtin_amdgcn_logf(l);
  const float inv = 1.0f / l;
  __syncthreads();
  float* slot = &Ks[grp][0][0];
#pragma unroll
  for (int i = 0; i < DQ; i += 4)
    *reinterpret_cast<f32x4*>(slot + qi * D + part * DQ + i) = f32x4{o[i], o[i + 1], o[i + 2], o[i + 3]};
  if (part == 0) {
    slot[kRows * D + qi] = lse2;
    slot[kRows * D + kRows + qi] = inv;
  }
  __syncthreads();
  if (grp != 0 || row >= p.Sq) return;

  float acc_o[DQ];
#pragma unroll
  for (int i = 0; i < DQ; i += 4) {
    const f32x4 r = f32x4{o[i], o[i + 1], o[i + 2], o[i + 3]} * inv;
    acc_o[i] = r[0]; acc_o[i + 1] = r[1]; acc_o[i + 2] = r[2]; acc_o[i + 3] = r[3];
  }
  float acc_lse = lse2 * kLn2;
#pragma unroll
  for (int g = 1; g < G; ++g) {
    const float* sg = &Ks[g][0][0];
    float og[DQ];
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(sg + qi * D + part * DQ + i);
      og[i] = x[0]; og[i + 1] = x[1]; og[i + 2] = x[2]; og[i + 3] = x[3];
    }
    merge_partial<DQ>(acc_o, acc_lse, og, sg[kRows * D + qi], sg[kRows * D + kRows + qi]);
  }
  float* orow = p.out + b * p.o_sb + (int64_t)row * p.o_ss + h * p.o_sh + part * DQ;
#pragma unroll
  for (int i = 0; i < DQ; i += 4)
    *reinterpret_cast<f32x4*>(orow + i) = f32x4{acc_o[i], acc_o[i + 1], acc_o[i + 2], acc_o[i + 3]};
  if (part == 0) p.lse[((int64_t)b * p.H + h) * p.Sq + row] = acc_lse;
}

template <int D, int G>
hipError_t launch_ring_dg(const RingParams& p, int64_t n_wg, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_f32_ring_kernel<D, G>), dim3((unsigned)n_wg), dim3(kThreads * G), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ring_d(const RingParams& p, int G, int64_t n_wg, hipStream_t stream) {
  if (G == 2) return launch_ring_dg<D, 2>(p, n_wg, stream);
  if (G == 3) return launch_ring_dg<D, 3>(p, n_wg, stream);
  if (G == 4) return launch_ring_dg<D, 4>(p, n_wg, stream);
  return hipErrorInvalidValue;
}

template <int D, bool ACC>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.out = a.out;
  p.lse = a.lse;
  p.q_sb = a.qs.b; p.q_ss = a.qs.s; p.q_sh = a.qs.h;
  p.kv_sb = a.kvs.b; p.kv_ss = a.kvs.s; p.kv_sh = a.kvs.h;
  p.o_sb = a.os.b; p.o_ss = a.os.s; p.o_sh = a.os.h;
  p.B = a.B; p.H = a.H; p.Sq = a.Sq; p.Skv = a.Skv;
  p.n_qt = (a.Sq + kRows - 1) / kRows;
  p.c = a.scale * kLog2e;
  const int64_t n_wg = (int64_t)p.n_qt * a.H * a.B;
  if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, ACC>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ring_f32(const FwdArgs& a, const RingBlocks& rb, hipStream_t stream) {
  if (rb.n < 2 || rb.n > kMaxF32RingBlocks || (a.D != 64 && a.D != 128)) return hipErrorInvalidValue;
  RingParams p;
  p.q = static_cast<const float*>(a.q);
  p.out = a.out;
  p.lse = a.lse;
  p.q_sb = a.qs.b; p.q_ss = a.qs.s; p.q_sh = a.qs.h;
  p.kv_sb = a.kvs.b; p.kv_ss = a.kvs.s; p.kv_sh = a.kvs.h;
  p.o_sb = a.os.b; p.o_ss = a.os.s; p.o_sh = a.os.h;
  p.B = a.B; p.H = a.H; p.Sq = a.Sq;
  p.n_qt = (a.Sq + kRows - 1) / kRows;
  p.c = a.scale * kLog2e;
  const int tile = a.D == 64 ? 64 : 32;
  int longest = 0;
  for (int i = 0; i < kMaxF32RingBlocks; ++i) {
    const bool in = i < rb.n;
    if (in && rb.len[i] < 1) return hipErrorInvalidValue;
    p.k[i] = in ? static_cast<const float*>(rb.k[i]) : nullptr;
    p.v[i] = in ? static_cast<const float*>(rb.v[i]) : nullptr;
    p.len[i] = in ? rb.len[i] : 0;
    if (in && rb.len[i] > longest) longest = rb.len[i];
  }
  p.n_iter = (longest + tile - 1) / tile;
  const int64_t n_wg = (int64_t)p.n_qt * a.H * a.B;
  if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (n_wg == 0) return hipSuccess;
  return a.D == 64 ? launch_ring_d<64>(p, rb.n, n_wg, stream) : launch_ring_d<128>(p, rb.n, n_wg, stream);
}

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.accumulate ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  if (a.D == 64) return a.accumulate ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
