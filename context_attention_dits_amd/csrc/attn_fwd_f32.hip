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
#pragma unroll
    for (int it = 0; it < kTile * (D / 4) / kThreads; ++it) {
      const int idx = tid + it * kThreads;
      const int n = idx / (D / 4), c4 = idx % (D / 4);
      const int key = key0 + n;
      f32x4 kx{}, vx{};
      if (key < p.Skv) {
        kx = *reinterpret_cast<const f32x4*>(kbase + (int64_t)key * p.kv_ss + c4 * 4);
        vx = *reinterpret_cast<const f32x4*>(vbase + (int64_t)key * p.kv_ss + c4 * 4);
      }
      *reinterpret_cast<f32x4*>(&Ks[n][c4 * 4]) = kx;
      *reinterpret_cast<f32x4*>(&Vs[n][c4 * 4]) = vx;
    }
    __syncthreads();

    float sc[kTile];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
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
      sc[j] = (key0 + j < p.Skv) ? full * p.c : -INFINITY;
      mt = fmaxf(mt, sc[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
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

hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.accumulate ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  if (a.D == 64) return a.accumulate ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
