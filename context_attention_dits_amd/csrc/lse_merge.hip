// LSE merge of two float32 attention partials, in place into the accumulator,
// and the fill for attention over an empty key set.
//
// The pages keep each block's partial output and LSE in float32 for a stable
// ring merge ("Paralelismo", ContextParallelConfig, convert_to_fp32) and
// require the full ring to see every token's K/V ("Paralelismo de contexto",
// "Atencao em Anel"); the exact recombination of two softmax partials over
// disjoint key sets is
//   M = max(lse_a, lse_b), w = exp(lse - M), lse = M + ln(w_a + w_b),
//   out = (w_a out_a + w_b out_b) / (w_a + w_b).
//
// Memory-bound: each float4 of out_acc is read, combined with the matching
// float4 of out_blk and written back; the weights are recomputed per float4
// from the two LSE values of its row (4 bytes each, served from cache). The
// D/4 threads of one row sit in one wavefront, so the row's LSE is read by
// all of them before the row's first thread overwrites it.
#include <stdint.h>

#include "kernels.h"

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// One wave per workgroup: on MI355X the 32k ring-4 share's merge (304 MB,
// operands not cached) runs at 76% of 8 TB/s so, 73% with 256 threads.
constexpr int kThreads = 64;

// One float4 of out_acc per thread, consecutive threads on consecutive
// float4 of a row; 32-bit index math with multiply-shift divisions (the host
// checks B*Sq*H*D/4 < 2^31).
// On MI355X this plain shape streams faster than batching several float4 per
// thread or non-temporal accesses.
template <int D>
__global__ void __launch_bounds__(kThreads)
lse_merge_kernel(float* __restrict__ oa, float* __restrict__ la, const float* __restrict__ ob,
                 const float* __restrict__ lb, Strides as, Strides bs, FastDiv div_h, FastDiv div_sq,
                 int n_vec) {
  constexpr int V = D / 4;  // float4 per row
  const int id = blockIdx.x * kThreads + threadIdx.x;
  if (id >= n_vec) return;
  const int H = (int)div_h.d, Sq = (int)div_sq.d;
  const int row = id / V;  // (b * Sq + s) * H + h
  const int c4 = id % V;
  const int bs_row = (int)div_h.div((uint32_t)row);
  const int h = row - bs_row * H;
  const int b = (int)div_sq.div((uint32_t)bs_row);
  const int s = bs_row - b * Sq;
  const int64_t li = ((int64_t)b * H + h) * Sq + s;
  f32x4* pa = reinterpret_cast<f32x4*>(oa + b * as.b + (int64_t)s * as.s + h * as.h + c4 * 4);
  const f32x4 va = *pa;
  const f32x4 vb = *reinterpret_cast<const f32x4*>(ob + b * bs.b + (int64_t)s * bs.s + h * bs.h + c4 * 4);
  const float a2 = la[li] * kLog2e;
  const float b2 = lb[li] * kLog2e;
  const float M = fmaxf(a2, b2);
  f32x4 r = f32x4{};
  float lse = -INFINITY;
  if (M != -INFINITY) {  // else both partials are over no keys
    const float wa = __builtin_amdgcn_exp2f(a2 - M);
    const float wb = __builtin_amdgcn_exp2f(b2 - M);
    const float tot = wa + wb;
    const float inv = 1.0f / tot;
    // A side with weight 0 contributes nothing, whatever its (unused) output holds.
    const f32x4 ra = (wa > 0.f) ? va * (wa * inv) : f32x4{};
    const f32x4 rb = (wb > 0.f) ? vb * (wb * inv) : f32x4{};
    r = ra + rb;
    lse = (M + __builtin_amdgcn_logf(tot)) * kLn2;
  }
  *pa = r;
  if (c4 == 0) la[li] = lse;
}

template <int D>
__global__ void __launch_bounds__(kThreads)
fill_empty_kernel(float* __restrict__ out, Strides os, float* __restrict__ lse, int H, int Sq,
                  int64_t n_vec) {
  constexpr int V = D / 4;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= n_vec) return;
  const int64_t row = id / V;
  const int c4 = (int)(id % V);
  const int h = (int)(row % H);
  const int64_t bs_row = row / H;
  const int s = (int)(bs_row % Sq);
  const int b = (int)(bs_row / Sq);
  *reinterpret_cast<f32x4*>(out + b * os.b + (int64_t)s * os.s + h * os.h + c4 * 4) = f32x4{};
  if (c4 == 0) lse[((int64_t)b * H + h) * Sq + s] = -INFINITY;
}

int64_t grid_for(int64_t n) { return (n + kThreads - 1) / kThreads; }

}  // namespace

hipError_t launch_lse_merge(float* out_acc, float* lse_acc, const float* out_blk,
                            const float* lse_blk, Strides as, Strides bs, int B, int H, int Sq,
                            int D, hipStream_t stream) {
  const int64_t n_vec = (int64_t)B * Sq * H * (D / 4);
  if (n_vec == 0) return hipSuccess;
  if (n_vec > 0x7fffffff) return hipErrorInvalidConfiguration;  // 32-bit indices
  const int64_t g = grid_for(n_vec);
  if (D == 128) {
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3((unsigned)g), dim3(kThreads), 0, stream, out_acc,
                       lse_acc, out_blk, lse_blk, as, bs, FastDiv((uint32_t)H), FastDiv((uint32_t)Sq),
                       (int)n_vec);
  } else if (D == 64) {
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3((unsigned)g), dim3(kThreads), 0, stream, out_acc,
                       lse_acc, out_blk, lse_blk, as, bs, FastDiv((uint32_t)H), FastDiv((uint32_t)Sq),
                       (int)n_vec);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fill_empty(float* out, Strides os, float* lse, int B, int H, int Sq, int D,
                             hipStream_t stream) {
  const int64_t n_vec = (int64_t)B * Sq * H * (D / 4);
  const int64_t g = grid_for(n_vec);
  if (g > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (D == 128) {
    hipLaunchKernelGGL(fill_empty_kernel<128>, dim3((unsigned)g), dim3(kThreads), 0, stream, out, os,
                       lse, H, Sq, n_vec);
  } else if (D == 64) {
    hipLaunchKernelGGL(fill_empty_kernel<64>, dim3((unsigned)g), dim3(kThreads), 0, stream, out, os,
                       lse, H, Sq, n_vec);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
