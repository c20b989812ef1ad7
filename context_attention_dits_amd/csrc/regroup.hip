// Ulysses head/token regroup: the local permutation of the all-to-all with
// the exchange replaced by a loopback ("Paralelismo de contexto", section
// "Atencao Ulysses": the first all-to-all leaves each GPU with every token of
// a subset of heads, the second regroups the results by token). Below it, the
// packs around an all-to-all with uneven splits (section "Ulysses Anything
// Attention": sequence length and head count need not divide by the degree).
//
//   SEQ_TO_HEAD: out[b, g*S_local + s, h, d] = in[b, s, g*(H/P) + h, d]
//   HEAD_TO_SEQ: out[b, s, g*(H/P) + h, d] = in[b, g*S_local + s, h, d]
//
// For every (b, s, g) both sides hold the same (H/P)*D elements contiguously,
// so the permutation is a copy of B*S_local*P contiguous chunks, moved in
// W-byte words (16 when the chunk size and pointers allow). Bit-exact for any
// element type.
#include <stdint.h>

#include "kernels.h"

namespace cpattn {
namespace {

// One wave per workgroup: measured on MI355X (back-to-back launches, operands
// not cached), a copy of 85 MB moves at 5.4 TB/s with 64-thread workgroups,
// 5.0 with 128, 256 or 1024 (302 MB: 6.0 vs 5.8-5.9).
constexpr int kThreads = 64;
constexpr int kMaxPieces = kMaxUlyssesDegree;

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

// One W-byte word per thread, consecutive threads on consecutive words of the
// sequence-sharded side; I is the index type (32-bit, with multiply-shift
// divisions, unless the tensor has 2^31 words or more). On MI355X this plain
// shape streams faster than moving several words per thread (2 or 4 words per
// thread, grid-strided or in runs: 4-15% slower at 85 MB) or non-temporal
// accesses, and at the rate of a plain copy of the same bytes.
template <int W, typename I>
struct RegroupDiv;
template <int W>
struct RegroupDiv<W, uint32_t> {  // divisors as multiply-shift
  FastDiv chunk, p, s_local;
  __device__ __forceinline__ uint32_t by_chunk(uint32_t n) const { return chunk.div(n); }
  __device__ __forceinline__ uint32_t by_p(uint32_t n) const { return p.div(n); }
  __device__ __forceinline__ uint32_t by_s(uint32_t n) const { return s_local.div(n); }
};
template <int W>
struct RegroupDiv<W, int64_t> {  // plain 64-bit division for tensors of 2^31 words or more
  int64_t chunk, p, s_local;
  __device__ __forceinline__ int64_t by_chunk(int64_t n) const { return n / chunk; }
  __device__ __forceinline__ int64_t by_p(int64_t n) const { return n / p; }
  __device__ __forceinline__ int64_t by_s(int64_t n) const { return n / s_local; }
};

// Up to kMaxRegroupTensors tensors of one shape regrouped by one launch (the
// Ulysses exchange moves Q, K and V together): blockIdx.y picks the tensor.
struct RegroupPtrs {
  const char* in[kMaxRegroupTensors];
  char* out[kMaxRegroupTensors];
};

template <int W, typename I>
__global__ void __launch_bounds__(kThreads)
regroup_kernel(RegroupPtrs ptrs, RegroupDiv<W, I> dv, I S_local, I P, I chunk_words, I n_words, int direction) {
  using T = typename Word<W>::type;
  const T* src = reinterpret_cast<const T*>(ptrs.in[blockIdx.y]);
  T* dst = reinterpret_cast<T*>(ptrs.out[blockIdx.y]);
  const I id = (I)blockIdx.x * kThreads + (I)threadIdx.x;
  if (id >= n_words) return;
  const I cid = dv.by_chunk(id);  // (b, s, g), g fastest: the sequence-sharded order
  const I w = id - cid * chunk_words;
  const I bs = dv.by_p(cid);
  const I g = cid - bs * P;
  const I b = dv.by_s(bs);
  const I s = bs - b * S_local;
  const int64_t head_off = (((int64_t)b * P + g) * S_local + s) * chunk_words + w;  // [b, g*S_l + s, ..]
  if (direction == 0) {
    dst[head_off] = src[id];
  } else {
    dst[id] = src[head_off];
  }
}

template <int W>
hipError_t launch_w(const RegroupPtrs& ptrs, int n, int64_t chunk_bytes, int B, int S_local, int P,
                    int direction, hipStream_t stream) {
  const int64_t chunk_words = chunk_bytes / W;
  const int64_t n_words = chunk_words * P * S_local * B;
  if (n_words == 0 || n == 0) return hipSuccess;
  const int64_t g = (n_words + kThreads - 1) / kThreads;
  if (g > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (n_words <= 0x7fffffff) {
    RegroupDiv<W, uint32_t> dv{FastDiv((uint32_t)chunk_words), FastDiv((uint32_t)P), FastDiv((uint32_t)S_local)};
    hipLaunchKernelGGL((regroup_kernel<W, uint32_t>), dim3((unsigned)g, (unsigned)n), dim3(kThreads), 0, stream,
                       ptrs, dv, (uint32_t)S_local, (uint32_t)P, (uint32_t)chunk_words, (uint32_t)n_words,
                       direction);
  } else {
    RegroupDiv<W, int64_t> dv{chunk_words, (int64_t)P, (int64_t)S_local};
    hipLaunchKernelGGL((regroup_kernel<W, int64_t>), dim3((unsigned)g, (unsigned)n), dim3(kThreads), 0, stream,
                       ptrs, dv, (int64_t)S_local, (int64_t)P, chunk_words, n_words, direction);
  }
  return hipGetLastError();
}

// ---- uneven splits (Ulysses Anything)
//
// A tensor of B x M x N words is split along M (AXIS 1) or N (AXIS 2) into
// segments; piece g, the segment's words in the tensor's order ([B, n_g, N]
// or [B, M, n_g]), sits at word base_g of a buffer of pieces back to back.
// Workgroups along y take one piece each, so every per-piece quantity is
// uniform (scalar loads from the kernel arguments); a thread moves one word,
// contiguous on the pieces side and in runs of n_g (or n_g*N) words on the
// tensor side.
struct PieceTable {
  uint32_t base[kMaxPieces];   // first word of piece g in the pieces buffer
  uint32_t off[kMaxPieces];    // first row (AXIS 1) or column (AXIS 2) of piece g in the tensor
  uint32_t words[kMaxPieces];  // words in piece g
  FastDiv div[kMaxPieces];     // AXIS 1: n_g * N words per batch entry; AXIS 2: n_g words per row
};

template <int W, int AXIS>
__global__ void __launch_bounds__(kThreads)
pieces_kernel(const char* __restrict__ in, char* __restrict__ out, PieceTable t, uint32_t M, uint32_t N,
              int to_pieces) {
  using T = typename Word<W>::type;
  const int g = blockIdx.y;
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;  // word within piece g
  if (i >= t.words[g]) return;
  uint32_t tensor_word;
  if constexpr (AXIS == 1) {
    const uint32_t b = t.div[g].div(i);  // batch entry; the rest is a run of n_g * N words
    tensor_word = (b * M + t.off[g]) * N + (i - b * t.div[g].d);
  } else {
    const uint32_t row = t.div[g].div(i);  // (b, m); the rest is a column within the piece
    tensor_word = row * N + t.off[g] + (i - row * t.div[g].d);
  }
  const uint32_t piece_word = t.base[g] + i;
  const T* src = reinterpret_cast<const T*>(in);
  T* dst = reinterpret_cast<T*>(out);
  if (to_pieces) {
    dst[piece_word] = src[tensor_word];
  } else {
    dst[tensor_word] = src[piece_word];
  }
}

template <int W>
hipError_t launch_pieces_w(const void* in, void* out, int axis, int64_t B, int64_t M, int64_t N,
                           const int* seg_words, int P, int to_pieces, hipStream_t stream) {
  // seg_words[g]: segment width along the split axis, in rows (AXIS 1) or words (AXIS 2)
  PieceTable t;
  uint64_t base = 0, off = 0, max_words = 0;
  for (int g = 0; g < P; ++g) {
    const uint64_t n = (uint64_t)seg_words[g];
    const uint64_t per = axis == 1 ? n * (uint64_t)N : n;  // words per batch entry or per row
    const uint64_t words = axis == 1 ? per * (uint64_t)B : per * (uint64_t)(B * M);
    t.base[g] = (uint32_t)base;
    t.off[g] = (uint32_t)off;
    t.words[g] = (uint32_t)words;
    t.div[g] = FastDiv(per > 0 ? (uint32_t)per : 1u);
    base += words;
    off += n;
    if (words > max_words) max_words = words;
  }
  if (max_words == 0) return hipSuccess;
  const unsigned gx = (unsigned)((max_words + kThreads - 1) / kThreads);
  const char* src = static_cast<const char*>(in);
  char* dst = static_cast<char*>(out);
  if (axis == 1) {
    hipLaunchKernelGGL((pieces_kernel<W, 1>), dim3(gx, P), dim3(kThreads), 0, stream, src, dst, t,
                       (uint32_t)M, (uint32_t)N, to_pieces);
  } else {
    hipLaunchKernelGGL((pieces_kernel<W, 2>), dim3(gx, P), dim3(kThreads), 0, stream, src, dst, t,
                       (uint32_t)M, (uint32_t)N, to_pieces);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pieces(const void* in, void* out, int axis, int64_t B, int64_t M, int64_t unit_bytes,
                         int64_t units_per_row, const int* seg_units, int P, int to_pieces, hipStream_t stream) {
  // The tensor is [B, M, units_per_row] units of unit_bytes; AXIS 1 splits M
  // (seg_units in rows), AXIS 2 splits the units of a row.
  const uintptr_t align = reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out) |
                          static_cast<uintptr_t>(unit_bytes);
  const int W = (align & 15) == 0 ? 16 : (align & 7) == 0 ? 8 : (align & 3) == 0 ? 4 : 2;
  const int64_t wpu = unit_bytes / W;  // words per unit
  int seg[kMaxPieces];
  for (int g = 0; g < P; ++g) seg[g] = axis == 1 ? seg_units[g] : (int)(seg_units[g] * wpu);
  const int64_t N = units_per_row * wpu;
  switch (W) {
    case 16: return launch_pieces_w<16>(in, out, axis, B, M, N, seg, P, to_pieces, stream);
    case 8: return launch_pieces_w<8>(in, out, axis, B, M, N, seg, P, to_pieces, stream);
    case 4: return launch_pieces_w<4>(in, out, axis, B, M, N, seg, P, to_pieces, stream);
    default: return launch_pieces_w<2>(in, out, axis, B, M, N, seg, P, to_pieces, stream);
  }
}

hipError_t launch_regroup(const void* const* in, void* const* out, int n, int elem_bytes, int B, int S_local,
                          int H, int D, int degree, int direction, hipStream_t stream) {
  if (n < 1 || n > kMaxRegroupTensors) return hipErrorInvalidValue;
  const int64_t chunk_bytes = (int64_t)(H / degree) * D * elem_bytes;
  RegroupPtrs ptrs{};
  uintptr_t align = static_cast<uintptr_t>(chunk_bytes);
  for (int i = 0; i < n; ++i) {
    ptrs.in[i] = static_cast<const char*>(in[i]);
    ptrs.out[i] = static_cast<char*>(out[i]);
    align |= reinterpret_cast<uintptr_t>(in[i]) | reinterpret_cast<uintptr_t>(out[i]);
  }
  if ((align & 15) == 0) return launch_w<16>(ptrs, n, chunk_bytes, B, S_local, degree, direction, stream);
  if ((align & 7) == 0) return launch_w<8>(ptrs, n, chunk_bytes, B, S_local, degree, direction, stream);
  if ((align & 3) == 0) return launch_w<4>(ptrs, n, chunk_bytes, B, S_local, degree, direction, stream);
  return launch_w<2>(ptrs, n, chunk_bytes, B, S_local, degree, direction, stream);
}

}  // namespace cpattn
