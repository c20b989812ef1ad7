// Partial attention of a local Q slice against one K/V block with float32
// inputs, float32 output + LSE (same definition as the bf16 kernel:
// "Paralelismo de contexto", "Atencao em Anel"; "Paralelismo",
// ContextParallelConfig, convert_to_fp32).
//
// The float32 path keeps every product and sum in float32 on the vector ALUs
// so that it stays within float32 rounding of the exact result. It serves
// small float32 problems; large workloads use the bf16 matrix-core kernel.
//
// Layout: a workgroup of 128 threads owns 64 query rows of one (b, h); each
// row is split over a thread pair, each thread holding half of D of the
// query and of the output accumulator. K/V are staged through LDS in tiles of
// 32 keys (zero-filled past Skv). Scores of a tile are formed by a partial
// dot product per thread plus one exchange with the partner lane; both
// partners then hold identical scores, maxima and sums.
#include <stdint.h>

#include "kernels.h"

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRows = 64;   // query rows per workgroup
constexpr int kTile = 32;   // keys per LDS tile
constexpr int kThreads = 128;

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
  constexpr int DH = D / 2;
  __shared__ __attribute__((aligned(16))) float Ks[kTile][D];
  __shared__ __attribute__((aligned(16))) float Vs[kTile][D];

  const int tid = threadIdx.x;
  const int qi = tid >> 1, half = tid & 1;
  const int qt = blockIdx.x % p.n_qt;
  const int bh = blockIdx.x / p.n_qt;
  const int h = bh % p.H, b = bh / p.H;
  const int row = qt * kRows + qi;

  float qv[DH], o[DH];
  {
    const float* qp = p.q + b * p.q_sb + (int64_t)row * p.q_ss + h * p.q_sh + half * DH;
#pragma unroll
    for (int i = 0; i < DH; i += 4) {
      const f32x4 x = (row < p.Sq) ? *reinterpret_cast<const f32x4*>(qp + i) : f32x4{};
      qv[i] = x[0]; qv[i + 1] = x[1]; qv[i + 2] = x[2]; qv[i + 3] = x[3];
    }
  }
#pragma unroll
  for (int i = 0; i < DH; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const float* kbase = p.k + b * p.kv_sb + h * p.kv_sh;
  const float* vbase = p.v + b * p.kv_sb + h * p.kv_sh;

  for (int key0 = 0; key0 < p.Skv; key0 += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * (D / 4); idx += kThreads) {
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
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < DH; ++i) part = fmaf(qv[i], Ks[j][half * DH + i], part);
      const float full = part + __shfl_xor(part, 1);
      sc[j] = (key0 + j < p.Skv) ? full * p.c : -INFINITY;
      mt = fmaxf(mt, sc[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DH; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float pj = __builtin_amdgcn_exp2f(sc[j] - m_new);
      l += pj;
#pragma unroll
      for (int i = 0; i < DH; ++i) o[i] = fmaf(pj, Vs[j][half * DH + i], o[i]);
    }
  }

  if (row >= p.Sq) return;
  const float lse2 = m + __builtin_amdgcn_logf(l);
  const float inv = 1.0f / l;
  float* orow = p.out + b * p.o_sb + (int64_t)row * p.o_ss + h * p.o_sh + half * DH;
  float* lrow = p.lse + ((int64_t)b * p.H + h) * p.Sq + row;
  if constexpr (ACC) {
    const float la2 = *lrow * kLog2e;
    const float M = fmaxf(la2, lse2);
    const float wa = __builtin_amdgcn_exp2f(la2 - M);
    const float wb = __builtin_amdgcn_exp2f(lse2 - M);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = (wb / tot) * inv;
#pragma unroll
    for (int i = 0; i < DH; i += 4) {
      f32x4* dst = reinterpret_cast<f32x4*>(orow + i);
      const f32x4 ob = {o[i], o[i + 1], o[i + 2], o[i + 3]};
      const f32x4 oa = *dst;
      *dst = (wa > 0.f) ? (fa * oa + fb * ob) : (fb * ob);
    }
    if (half == 0) *lrow = (M + __builtin_amdgcn_logf(tot)) * kLn2;
  } else {
#pragma unroll
    for (int i = 0; i < DH; i += 4) {
      const f32x4 ob = {o[i], o[i + 1], o[i + 2], o[i + 3]};
      *reinterpret_cast<f32x4*>(orow + i) = ob * inv;
    }
    if (half == 0) *lrow = lse2 * kLn2;
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
