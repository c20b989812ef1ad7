// Ulysses head/token regroup: the local permutation of the all-to-all with
// the exchange replaced by a loopback ("Paralelismo de contexto", section
// "Atencao Ulysses": the first all-to-all leaves each GPU with every token of
// a subset of heads, the second regroups the results by token).
//
//   SEQ_TO_HEAD: out[b, g*S_local + s, h, d] = in[b, s, g*(H/P) + h, d]
//   HEAD_TO_SEQ: out[b, s, g*(H/P) + h, d] = in[b, g*S_local + s, h, d]
//
// For every (b, s, g) both sides hold the same (H/P)*D elements contiguously,
// so the permutation is a copy of B*S_local*P contiguous chunks. Each thread
// moves W-byte words (16 when the chunk size and pointers allow) with
// consecutive threads on consecutive words, several words per thread to keep
// enough bytes in flight. Bit-exact for any element type.
#include <stdint.h>

#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;

template <int W>
struct Word;
template <>
struct Word<16> {
  typedef uint32_t type __attribute__((ext_vector_type(4)));
};
template <>
struct Word<8> {
  typedef uint32_t type __attribute__((ext_vector_type(2)));
};
template <>
struct Word<4> {
  typedef uint32_t type;
};
template <>
struct Word<2> {
  typedef uint16_t type;
};

template <int W>
__global__ void __launch_bounds__(kThreads)
regroup_kernel(const char* __restrict__ in, char* __restrict__ out, int S_local, int P,
               int64_t chunk_words, int64_t src_row_words, int64_t n_words, int direction) {
  using T = typename Word<W>::type;
  const T* src = reinterpret_cast<const T*>(in);
  T* dst = reinterpret_cast<T*>(out);
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kPerThread) + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t id = base + (int64_t)i * kThreads;
    if (id >= n_words) return;
    const int64_t cid = id / chunk_words;
    const int64_t w = id - cid * chunk_words;
    // cid enumerates (b, s, g) with g fastest: the sequence-sharded side's order.
    const int g = (int)(cid % P);
    const int64_t bs = cid / P;
    const int s = (int)(bs % S_local);
    const int64_t b = bs / S_local;
    const int64_t seq_off = bs * src_row_words + (int64_t)g * chunk_words + w;  // [b, s, g*Hl..]
    const int64_t head_off = ((b * P + g) * S_local + s) * chunk_words + w;      // [b, g*S_l + s, ..]
    if (direction == 0) {
      dst[head_off] = src[seq_off];
    } else {
      dst[seq_off] = src[head_off];
    }
  }
}

template <int W>
hipError_t launch_w(const void* in, void* out, int64_t chunk_bytes, int B, int S_local, int P,
                    int direction, hipStream_t stream) {
  const int64_t chunk_words = chunk_bytes / W;
  const int64_t n_words = chunk_words * P * S_local * B;
  const int64_t per_block = (int64_t)kThreads * kPerThread;
  const int64_t g = (n_words + per_block - 1) / per_block;
  if (g > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(regroup_kernel<W>, dim3((unsigned)g), dim3(kThreads), 0, stream,
                     static_cast<const char*>(in), static_cast<char*>(out), S_local, P, chunk_words,
                     chunk_words * P, n_words, direction);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_regroup(const void* in, void* out, int elem_bytes, int B, int S_local, int H,
                          int D, int degree, int direction, hipStream_t stream) {
  const int64_t chunk_bytes = (int64_t)(H / degree) * D * elem_bytes;
  const uintptr_t align = reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out) |
                          static_cast<uintptr_t>(chunk_bytes);
  if ((align & 15) == 0) return launch_w<16>(in, out, chunk_bytes, B, S_local, degree, direction, stream);
  if ((align & 7) == 0) return launch_w<8>(in, out, chunk_bytes, B, S_local, degree, direction, stream);
  if ((align & 3) == 0) return launch_w<4>(in, out, chunk_bytes, B, S_local, degree, direction, stream);
  return launch_w<2>(in, out, chunk_bytes, B, S_local, degree, direction, stream);
}

}  // namespace cpattn
