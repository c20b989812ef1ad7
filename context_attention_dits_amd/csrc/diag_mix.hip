// Diagnostic (built only into the diagnostic library, not into libcpattn.so): a synthetic
// ping-pong with the block kernel's tile-loop instruction mix and none of its memory traffic,
// to compare the kernel's traced intervals with what the hardware sustains for that mix.
//
// 8 waves per workgroup, one workgroup per CU (its LDS request), 256 workgroups. In interval i
// the waves of one group (waves 0-3 or 4-7, alternating) run a matrix half: 32 fragment reads
// of 1 KB from LDS (ds_read_b128), 16 score and 16 PV MFMAs 32x32x16 bf16 on random data; the
// other group a softmax half over 32 values per lane (maxima, FMA, exp2, sums, bf16
// conversion); then a workgroup barrier. Variants: 0 as described; 1 the same flops as twice as
// many 16x16x32 MFMAs; 2 fragments taken from registers instead of LDS; 3 both groups in the
// same phase instead of ping-pong; 4 the matrix half's 32 fragment reads alone (all issued
// before their results are used, no MFMAs; the other group idles); 5 as 4 with all 8 waves
// reading in every interval; 6 and 7 as 0 with the first 8 or 16 of a matrix half's fragment
// reads issued by the wave during its preceding softmax half, into registers it keeps for them.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWgs = 256, kThreads = 512, kFrags = 32;

template <int VARIANT>
__global__ void __launch_bounds__(kThreads) mix_kernel(const bf16x8* __restrict__ src, float* __restrict__ out,
                                                       int iters, unsigned long long* __restrict__ ticks) {
  __shared__ __attribute__((aligned(1024))) bf16x8 frag[kFrags * 64];  // 32 KB
  __shared__ char pad[100 * 1024];                                     // one workgroup per CU
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16x8* mine = src + (size_t)blockIdx.x * (kFrags * 64);
  for (int i = tid; i < kFrags * 64; i += kThreads) frag[i] = mine[i];
  bf16x8 q[4], pf[4];
  for (int i = 0; i < 4; ++i) {
    q[i] = mine[(tid * 4 + i) % (kFrags * 64)];
    pf[i] = mine[(tid * 4 + i + 1) % (kFrags * 64)];
  }
  float x[32];
  for (int i = 0; i < 32; ++i) x[i] = (float)mine[(tid * 7 + i) % (kFrags * 64)][i & 7];
  __syncthreads();
  const int grp = (VARIANT == 3 || VARIANT == 5) ? 0 : (wave >> 2);
  u32x4 rd = {0u, 0u, 0u, 0u};
  f32x16 o32[4] = {}, s32[2] = {};
  f32x4 o16[16] = {}, s16[8] = {};
  constexpr int R = VARIANT == 6 ? 8 : VARIANT == 7 ? 16 : 0;  // fragments read one half early
  bf16x8 early[R > 0 ? R : 1];
  for (int i = 0; i < (R > 0 ? R : 1); ++i) early[i] = q[i & 3];
  float m = 0.f, l = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if (VARIANT == 4 || VARIANT == 5) {
      if (VARIANT == 5 || ((it + grp) & 1) == 0) {
        const int rot = (it & 7) * 64;  // the addresses move a little from one interval to the next
        bf16x8 r[kFrags];
#pragma unroll
        for (int f = 0; f < kFrags; ++f) r[f] = frag[((f * 64 + rot) & (kFrags * 64 - 1)) + lane];
#pragma unroll
        for (int f = 0; f < kFrags; ++f) rd ^= __builtin_bit_cast(u32x4, r[f]);
      }
    } else if (((it + grp) & 1) == 0) {
      if (VARIANT == 1) {
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const bf16x8 a = frag[f * 64 + lane];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s16[(f & 3) * 2 + qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q[(f + qb) & 3], s16[(f & 3) * 2 + qb], 0, 0, 0);
        }
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const bf16x8 a = frag[(16 + f) * 64 + lane];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o16[(f >> 1) * 2 + qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[(f + qb) & 3], o16[(f >> 1) * 2 + qb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const bf16x8 a = VARIANT == 2 ? q[(f + 1) & 3] : f < R ? early[f < R ? f : 0] : frag[f * 64 + lane];
          s32[f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[f & 3], s32[f & 1], 0, 0, 0);
        }
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const bf16x8 a = VARIANT == 2 ? q[(f + 2) & 3]
                           : 16 + f < R ? early[16 + f < R ? 16 + f : 0] : frag[(16 + f) * 64 + lane];
          o32[f >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[f & 3], o32[f >> 2], 0, 0, 0);
        }
      }
    } else {
      const int rot = (it & 7) * 64;
#pragma unroll
      for (int f = 0; f < R; ++f) early[f] = frag[((f * 64 + rot) & (kFrags * 64 - 1)) + lane];
      float mx0 = x[0], mx1 = x[1];
#pragma unroll
      for (int i = 2; i < 32; i += 2) {
        mx0 = __builtin_elementwise_maximum(mx0, x[i]);
        mx1 = __builtin_elementwise_maximum(mx1, x[i + 1]);
      }
      m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(mx0, mx1) * 0.125f);
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x8 t;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x[g * 8 + jj], 0.125f, -m));
          ls[jj & 3] += e;
          t[jj] = (__bf16)e;
        }
        pf[g] = t;
      }
      l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = VARIANT == 1 ? s16[i >> 2][i & 3] : s32[i >> 4][i & 15];
    }
    __syncthreads();
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float sink = l + m + (float)(rd[0] ^ rd[1] ^ rd[2] ^ rd[3]);
  for (int i = 0; i < (R > 0 ? R : 1); ++i) sink += (float)early[i][i & 7];
  for (int i = 0; i < 16; ++i) sink += VARIANT == 1 ? o16[i][0] + o16[i][3] : o32[i >> 2][i & 15] + o32[3][i];
  pad[tid] = (char)sink;
  __syncthreads();
  out[(size_t)blockIdx.x * kThreads + tid] = sink + pad[(tid * 7) & (kThreads - 1)];
  if (lane == 0) ticks[blockIdx.x * 8 + wave] = t1 - t0;
}

}  // namespace

// Runs variant `variant` (0-7, see above) for `iters` intervals after one untimed launch and
// returns the mean core-clock cycles per interval (s_memtime, every wave) and the timed
// launch's milliseconds. Allocates and frees its own device buffers; blocks until done.
extern "C" int cp_debug_mix_probe(int variant, int iters, double* cycles_per_interval, double* ms) {
  if (variant < 0 || variant > 7 || iters < 2 || iters > (1 << 20) || !cycles_per_interval || !ms)
    return (int)hipErrorInvalidValue;
  const size_t n_src = (size_t)kWgs * kFrags * 64;
  bf16x8* src = nullptr;
  float* out = nullptr;
  unsigned long long* ticks = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&src, n_src * sizeof(bf16x8));
  if (e == hipSuccess) e = hipMalloc(&out, (size_t)kWgs * kThreads * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&ticks, (size_t)kWgs * 8 * sizeof(unsigned long long));
  bf16x8* host = (bf16x8*)malloc(n_src * sizeof(bf16x8));
  unsigned long long* hticks = (unsigned long long*)malloc((size_t)kWgs * 8 * sizeof(unsigned long long));
  if (e == hipSuccess && (!host || !hticks)) e = hipErrorOutOfMemory;
  if (e == hipSuccess) {
    uint32_t s = 777u;  // random bf16 in [-2, 2]
    for (size_t i = 0; i < n_src; ++i)
      for (int k = 0; k < 8; ++k) {
        s = s * 1664525u + 1013904223u;
        host[i][k] = (__bf16)((float)((int)(s >> 9) % 2001 - 1000) * 0.002f);
      }
    e = hipMemcpy(src, host, n_src * sizeof(bf16x8), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  float t_ms = 0.f;
  for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
    e = hipEventRecord(e0, 0);
    if (e != hipSuccess) break;
    switch (variant) {
      case 0: hipLaunchKernelGGL(mix_kernel<0>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
      case 1: hipLaunchKernelGGL(mix_kernel<1>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
      case 2: hipLaunchKernelGGL(mix_kernel<2>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
      case 3: hipLaunchKernelGGL(mix_kernel<3>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
      case 4: hipLaunchKernelGGL(mix_kernel<4>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
      case 5: hipLaunchKernelGGL(mix_kernel<5>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
      case 6: hipLaunchKernelGGL(mix_kernel<6>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
      default: hipLaunchKernelGGL(mix_kernel<7>, dim3(kWgs), dim3(kThreads), 0, 0, src, out, iters, ticks); break;
    }
    e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&t_ms, e0, e1);
  }
  if (e == hipSuccess)
    e = hipMemcpy(hticks, ticks, (size_t)kWgs * 8 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    double sum = 0;
    for (int i = 0; i < kWgs * 8; ++i) sum += (double)hticks[i];
    *cycles_per_interval = sum / (kWgs * 8) / iters;
    *ms = t_ms;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(src);
  (void)hipFree(out);
  (void)hipFree(ticks);
  free(host);
  free(hticks);
  return (int)e;
}
