// C-ABI of the library: host-side validation, launch selection and the ring
// loop. Every check runs before anything is enqueued, so a failing call
// launches nothing. See include/cp_attn.h for the contract of each entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "cp_attn.h"
#include "kernels.h"

#ifndef CP_BWD_MULTI
#define CP_BWD_MULTI 1  // ring backward: dQ over all blocks in one launch, dK/dV of all blocks in one grid
#endif
#ifndef CP_BWD_SIDE_STREAM
#define CP_BWD_SIDE_STREAM 1  // backward: dq kernels on a second stream, concurrent with dkv (0: one stream)
#endif

namespace {

using cpattn::Strides;

thread_local std::string g_err;

cp_status_t fail(cp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

cp_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CP_OK;
  return fail(CP_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

const char* kSupported = "supported: dtype CP_F32 (0) or CP_BF16 (1), head dim D = 64 or 128";

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Resolve a host stride triple (NULL = contiguous [B, S, H, D]).
Strides resolve(const int64_t* s, int S, int H, int D) {
  if (s == nullptr) return Strides{(int64_t)S * H * D, (int64_t)H * D, (int64_t)D};
  return Strides{s[0], s[1], s[2]};
}

cp_status_t check_strides(const char* name, Strides st, int elem_bytes, int S, int H, int D) {
  if (st.b < 0 || st.s < 0 || st.h < 0)
    return fail(CP_ERR_INVALID_ARG, "%s: strides must be non-negative (got b=%lld s=%lld h=%lld)",
                name, (long long)st.b, (long long)st.s, (long long)st.h);
  if ((st.b * elem_bytes) % 16 || (st.s * elem_bytes) % 16 || (st.h * elem_bytes) % 16)
    return fail(CP_ERR_UNSUPPORTED,
                "%s: every stride times the element size must be a multiple of 16 bytes", name);
  // Rows of one head must not overlap each other along D.
  if (H > 1 && st.h < D)
    return fail(CP_ERR_INVALID_ARG, "%s: head stride %lld smaller than D=%d", name, (long long)st.h, D);
  if (S > 1 && st.s < D)
    return fail(CP_ERR_INVALID_ARG, "%s: sequence stride %lld smaller than D=%d", name,
                (long long)st.s, D);
  return CP_OK;
}

int elem_size(int dtype) { return dtype == CP_BF16 ? 2 : 4; }

// Arguments common to block attention and the ring; K/V lengths checked by callers.
cp_status_t check_common(const void* q, Strides qs, Strides kvs, int dtype, int B, int H, int D,
                         int Sq, float scale, const float* out, Strides os, const float* lse) {
  if (dtype != CP_F32 && dtype != CP_BF16)
    return fail(CP_ERR_UNSUPPORTED, "dtype %d is not supported; %s", dtype, kSupported);
  if (D != 64 && D != 128)
    return fail(CP_ERR_UNSUPPORTED, "head dim D=%d is not supported; %s", D, kSupported);
  if (B < 0 || H < 0 || Sq < 0)
    return fail(CP_ERR_INVALID_ARG, "sizes must be non-negative (B=%d H=%d Sq=%d)", B, H, Sq);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(CP_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  if (B == 0 || H == 0 || Sq == 0) return CP_OK;
  if (q == nullptr || out == nullptr || lse == nullptr)
    return fail(CP_ERR_INVALID_ARG, "q, out and lse must be non-null");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return fail(CP_ERR_UNSUPPORTED, "q and out must be 16-byte aligned, lse 4-byte aligned");
  const int es = elem_size(dtype);
  cp_status_t st;
  if ((st = check_strides("q", qs, es, Sq, H, D)) != CP_OK) return st;
  if ((st = check_strides("k/v", kvs, es, 2, H, D)) != CP_OK) return st;
  // K/V tiles are fetched through buffer descriptors with 32-bit offsets.
  if (kvs.s > (int64_t(1) << 24))
    return fail(CP_ERR_UNSUPPORTED, "k/v: sequence stride %lld exceeds 2^24 elements", (long long)kvs.s);
  if ((st = check_strides("out", os, 4, Sq, H, D)) != CP_OK) return st;
  return CP_OK;
}

cp_status_t check_kv(const void* k, const void* v, int Skv) {
  if (Skv < 0) return fail(CP_ERR_INVALID_ARG, "K/V length must be non-negative (got %d)", Skv);
  if (Skv == 0) return CP_OK;
  if (k == nullptr || v == nullptr) return fail(CP_ERR_INVALID_ARG, "k and v must be non-null");
  if (!aligned(k, 16) || !aligned(v, 16))
    return fail(CP_ERR_UNSUPPORTED, "k and v must be 16-byte aligned");
  return CP_OK;
}

// One validated block: launches the attention (overwrite or accumulate) or the empty fill.
cp_status_t run_block(const void* q, Strides qs, const void* k, const void* v, Strides kvs, int dtype,
                      int B, int H, int D, int Sq, int Skv, float scale, bool accumulate, bool v_packed,
                      int waves, float* out, Strides os, float* lse, hipStream_t stream, int* err = nullptr) {
  if (Skv == 0) {
    if (accumulate) return CP_OK;
    return hip_status(cpattn::launch_fill_empty(out, os, lse, B, H, Sq, D, stream), "fill_empty");
  }
  cpattn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.qs = qs; a.kvs = kvs; a.os = os;
  a.B = B; a.H = H; a.D = D; a.Sq = Sq; a.Skv = Skv;
  a.scale = scale;
  a.accumulate = accumulate;
  a.waves = waves;
  a.v_packed = v_packed;
  a.err = err;
  if (dtype == CP_BF16) return hip_status(cpattn::launch_attn_fwd_bf16(a, stream), "attn_fwd_bf16");
  return hip_status(cpattn::launch_attn_fwd_f32(a, stream), "attn_fwd_f32");
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr unsigned kWaveFlags = CP_FWD_FOUR_WAVES | CP_FWD_EIGHT_WAVES;

// The workgroup shape a call's flags force (4 or 8), or 0 to choose per launch.
int forced_waves(unsigned flags) {
  return (flags & CP_FWD_FOUR_WAVES) ? 4 : (flags & CP_FWD_EIGHT_WAVES) ? 8 : 0;
}

// Does a packed-V ring with a workspace run as one launch? When the blocks'
// own launches would use the 4-wave kernel (a grid too small, or with a
// nearly empty last round, for the ping-pong one) and there are 2 .. the
// kernel's maximum non-empty blocks: then the one launch runs every block's
// partial in parallel on ping-pong workgroups. A single block of at least two
// 64-key tiles is split at a tile boundary into two halves that run the same
// way (the ring's own method, one level finer: two partials merged by their
// LSE). Bigger grids keep one launch per block, which measured as fast or
// faster. (The output's byte offsets must also fit the kernel's 32-bit buffer
// offsets; checked by the caller through o_end.)
bool one_launch_ring(int dtype, int B, int H, int D, int Sq, const int* block_len, int ring_degree, int waves) {
  if (dtype != CP_BF16 || D != 128 || B <= 0 || H <= 0 || Sq <= 0) return false;
  if (cpattn::ring_max_blocks() < 2) return false;  // library built without the 8-wave shape
  if (waves == 4) return false;
  cpattn::FwdArgs a{};
  a.B = B; a.H = H; a.D = D; a.Sq = Sq;
  a.waves = waves;
  if (waves == 0 && cpattn::pick_waves(a) == 8) return false;
  int n = 0, only = 0;
  for (int i = 0; i < ring_degree; ++i)
    if (block_len[i] > 0) {
      ++n;
      only = block_len[i];
    }
  if (n == 1) return only >= 128;
  return n >= 2 && n <= cpattn::ring_max_blocks();
}

// Whether cp_ring_attention with packed V runs the blocks in turn within one
// launch of the 8-wave kernel (the grid the per-block launches would run on
// the 8-wave shape, 2 .. seq_max_blocks() non-empty blocks): saves the fixed
// cost of every launch after the first (on the FLUX ring-2 share ~12-17 us of
// a ~66 us launch).
bool seq_ring(int dtype, int B, int H, int D, int Sq, const int* block_len, int ring_degree, int waves) {
  if (dtype != CP_BF16 || D != 128 || B <= 0 || H <= 0 || Sq <= 0) return false;
  if (waves == 4) return false;
  cpattn::FwdArgs a{};
  a.B = B; a.H = H; a.D = D; a.Sq = Sq;
  a.waves = waves;
  if (cpattn::pick_waves(a) != 8) return false;
  int n = 0;
  for (int i = 0; i < ring_degree; ++i) n += block_len[i] > 0;
  return n >= 2 && n <= cpattn::seq_max_blocks();
}

size_t partial_bytes(int B, int H, int Sq, int D) {
  return align_up((size_t)B * Sq * H * D * sizeof(float), 256) + align_up((size_t)B * H * Sq * sizeof(float), 256);
}

}  // namespace

extern "C" {

int cp_abi_version(void) { return CP_ATTN_ABI_VERSION; }

const char* cp_last_error(void) { return g_err.c_str(); }

int cp_attn_fwd_waves(int B, int H, int D, int Sq, unsigned flags) {
  if (B <= 0 || H <= 0 || Sq <= 0 || (D != 64 && D != 128)) return 0;
  if ((flags & kWaveFlags) == kWaveFlags) return 0;
  cpattn::FwdArgs a{};
  a.B = B; a.H = H; a.D = D; a.Sq = Sq;
  a.waves = forced_waves(flags);
  return cpattn::pick_waves(a);
}

int cp_ring_attention_one_launch(int dtype, int B, int H, int D, int Sq, const int* block_len, int ring_degree,
                                 unsigned flags) {
  if (block_len == nullptr || ring_degree < 1) return 0;
  if ((flags & kWaveFlags) == kWaveFlags || (flags & CP_RING_SEPARATE_MERGE)) return 0;
  for (int i = 0; i < ring_degree; ++i)
    if (block_len[i] < 0) return 0;
  const int waves = forced_waves(flags);
  if (one_launch_ring(dtype, B, H, D, Sq, block_len, ring_degree, waves)) return CP_ONE_LAUNCH_PARALLEL;
  if (seq_ring(dtype, B, H, D, Sq, block_len, ring_degree, waves)) return CP_ONE_LAUNCH_IN_TURN;
  return 0;
}

cp_status_t cp_attn_block_fwd(const void* q, const int64_t* q_strides, const void* k, const void* v,
                              const int64_t* kv_strides, int dtype, int B, int H, int D, int Sq,
                              int Skv, float scale, unsigned flags, float* out,
                              const int64_t* out_strides, float* lse, void* stream) {
  if (flags & ~(CP_BLOCK_ACCUMULATE | CP_BLOCK_PACKED_V | kWaveFlags))
    return fail(CP_ERR_INVALID_ARG, "cp_attn_block_fwd: unknown flags 0x%x", flags);
  if ((flags & kWaveFlags) == kWaveFlags)
    return fail(CP_ERR_INVALID_ARG, "cp_attn_block_fwd: CP_FWD_FOUR_WAVES and CP_FWD_EIGHT_WAVES together");
  const bool packed = (flags & CP_BLOCK_PACKED_V) != 0;
  if (packed && dtype != CP_BF16)
    return fail(CP_ERR_UNSUPPORTED, "cp_attn_block_fwd: packed V is for CP_BF16 only");
  const Strides qs = resolve(q_strides, Sq, H, D);
  const Strides kvs = resolve(kv_strides, Skv, H, D);
  const Strides os = resolve(out_strides, Sq, H, D);
  cp_status_t st = check_common(q, qs, kvs, dtype, B, H, D, Sq, scale, out, os, lse);
  if (st != CP_OK) return st;
  if (B == 0 || H == 0 || Sq == 0) return CP_OK;
  if ((st = check_kv(k, v, Skv)) != CP_OK) return st;
  return run_block(q, qs, k, v, kvs, dtype, B, H, D, Sq, Skv, scale, (flags & CP_BLOCK_ACCUMULATE) != 0,
                   packed, forced_waves(flags), out, os, lse, static_cast<hipStream_t>(stream));
}

cp_status_t cp_lse_merge(float* out_acc, float* lse_acc, const float* out_blk, const float* lse_blk,
                         const int64_t* acc_strides, const int64_t* blk_strides, int B, int H, int Sq,
                         int D, void* stream) {
  if (D != 64 && D != 128)
    return fail(CP_ERR_UNSUPPORTED, "cp_lse_merge: head dim D=%d is not supported (D = 64 or 128)", D);
  if (B < 0 || H < 0 || Sq < 0)
    return fail(CP_ERR_INVALID_ARG, "cp_lse_merge: sizes must be non-negative");
  if (B == 0 || H == 0 || Sq == 0) return CP_OK;
  if (!out_acc || !lse_acc || !out_blk || !lse_blk)
    return fail(CP_ERR_INVALID_ARG, "cp_lse_merge: pointers must be non-null");
  if (!aligned(out_acc, 16) || !aligned(out_blk, 16) || !aligned(lse_acc, 4) || !aligned(lse_blk, 4))
    return fail(CP_ERR_UNSUPPORTED, "cp_lse_merge: outputs must be 16-byte aligned, LSE 4-byte");
  if (out_acc == out_blk || lse_acc == lse_blk)
    return fail(CP_ERR_INVALID_ARG, "cp_lse_merge: accumulator and block must be distinct buffers");
  if ((int64_t)B * Sq * H * (D / 4) > 0x7fffffff)
    return fail(CP_ERR_UNSUPPORTED, "cp_lse_merge: B*Sq*H*D/4 must be below 2^31");
  const Strides as = resolve(acc_strides, Sq, H, D);
  const Strides bs = resolve(blk_strides, Sq, H, D);
  cp_status_t st;
  if ((st = check_strides("out_acc", as, 4, Sq, H, D)) != CP_OK) return st;
  if ((st = check_strides("out_blk", bs, 4, Sq, H, D)) != CP_OK) return st;
  return hip_status(cpattn::launch_lse_merge(out_acc, lse_acc, out_blk, lse_blk, as, bs, B, H, Sq, D,
                                             static_cast<hipStream_t>(stream)),
                    "lse_merge");
}

size_t cp_attn_packed_v_bytes(int B, int H, int D, int Skv) {
  if (B < 0 || H < 0 || Skv < 0 || (D != 64 && D != 128)) return 0;
  return (size_t)cpattn::packed_v_bytes(B, H, D, Skv);
}

cp_status_t cp_attn_pack_v(const void* v, const int64_t* v_strides, int B, int H, int D, int Skv,
                           void* packed, size_t packed_bytes, void* stream) {
  if (D != 64 && D != 128)
    return fail(CP_ERR_UNSUPPORTED, "cp_attn_pack_v: head dim D=%d is not supported (D = 64 or 128)", D);
  if (B < 0 || H < 0 || Skv < 0)
    return fail(CP_ERR_INVALID_ARG, "cp_attn_pack_v: sizes must be non-negative (B=%d H=%d Skv=%d)", B, H,
                Skv);
  if (B == 0 || H == 0 || Skv == 0) return CP_OK;
  const size_t need = (size_t)cpattn::packed_v_bytes(B, H, D, Skv);
  if (v == nullptr || packed == nullptr)
    return fail(CP_ERR_INVALID_ARG, "cp_attn_pack_v: v and packed must be non-null");
  if (packed_bytes < need)
    return fail(CP_ERR_INVALID_ARG, "cp_attn_pack_v: packed buffer of %zu bytes needed, %zu given", need,
                packed_bytes);
  if (!aligned(v, 16) || !aligned(packed, 16))
    return fail(CP_ERR_UNSUPPORTED, "cp_attn_pack_v: v and packed must be 16-byte aligned");
  const Strides vs = resolve(v_strides, Skv, H, D);
  cp_status_t st;
  if ((st = check_strides("v", vs, 2, Skv, H, D)) != CP_OK) return st;
  if ((int64_t)B * H * ((Skv + 63) / 64) > 0x7fffffff)
    return fail(CP_ERR_UNSUPPORTED, "cp_attn_pack_v: B*H*ceil(Skv/64) must be below 2^31");
  const char* src = static_cast<const char*>(v);
  const char* dst = static_cast<const char*>(packed);
  const int64_t v_end = ((B - 1) * vs.b + (int64_t)(Skv - 1) * vs.s + (H - 1) * vs.h + D) * 2;
  if (dst < src + v_end && src < dst + need)
    return fail(CP_ERR_INVALID_ARG, "cp_attn_pack_v: v and packed overlap");
  return hip_status(cpattn::launch_pack_v(v, vs, packed, B, H, D, Skv, Skv, static_cast<hipStream_t>(stream)),
                    "pack_v");
}

cp_status_t cp_ulysses_regroup_pack_v(const void* in, int B, int S_local, int H, int D, int degree,
                                      void* packed, size_t packed_bytes, void* stream) {
  const char* fn = "cp_ulysses_regroup_pack_v";
  if (D != 64 && D != 128) return fail(CP_ERR_UNSUPPORTED, "%s: head dim D=%d is not supported (D = 64 or 128)", fn, D);
  if (B < 0 || S_local < 0 || H < 0) return fail(CP_ERR_INVALID_ARG, "%s: sizes must be non-negative", fn);
  if (degree < 1) return fail(CP_ERR_INVALID_ARG, "%s: degree must be >= 1 (got %d)", fn, degree);
  if (H % degree != 0)
    return fail(CP_ERR_INVALID_ARG, "%s: the number of heads H=%d must be divisible by the Ulysses degree %d", fn,
                H, degree);
  if ((int64_t)degree * S_local > 0x7fffffff) return fail(CP_ERR_UNSUPPORTED, "%s: degree*S_local too large", fn);
  const int Hg = H / degree, S = degree * S_local;
  if (B == 0 || S == 0 || Hg == 0) return CP_OK;
  const size_t need = (size_t)cpattn::packed_v_bytes(B, Hg, D, S);
  if (in == nullptr || packed == nullptr) return fail(CP_ERR_INVALID_ARG, "%s: pointers must be non-null", fn);
  if (packed_bytes < need)
    return fail(CP_ERR_INVALID_ARG, "%s: packed buffer of %zu bytes needed, %zu given", fn, need, packed_bytes);
  if (!aligned(in, 16) || !aligned(packed, 16))
    return fail(CP_ERR_UNSUPPORTED, "%s: in and packed must be 16-byte aligned", fn);
  if ((int64_t)B * Hg * ((S + 63) / 64) > 0x7fffffff)
    return fail(CP_ERR_UNSUPPORTED, "%s: B*(H/degree)*ceil(degree*S_local/64) must be below 2^31", fn);
  const size_t in_bytes = (size_t)B * S_local * H * D * 2;
  const char* a = static_cast<const char*>(in);
  const char* b = static_cast<const char*>(packed);
  if (b < a + in_bytes && a < b + need) return fail(CP_ERR_INVALID_ARG, "%s: in and packed overlap", fn);
  const Strides is{(int64_t)S_local * H * D, (int64_t)H * D, (int64_t)D};
  return hip_status(cpattn::launch_pack_v(in, is, packed, B, Hg, D, S, S_local, static_cast<hipStream_t>(stream)),
                    "ulysses_regroup_pack_v");
}

size_t cp_ring_attention_workspace_size(int B, int H, int Sq, int D, unsigned flags) {
  if (B <= 0 || H <= 0 || Sq <= 0 || D <= 0) return 0;
  if (flags & CP_RING_SEPARATE_MERGE) return partial_bytes(B, H, Sq, D);
  if (D == 128 && (flags & CP_RING_PACKED_V))
    return align_up((size_t)(cpattn::kRingFlagOffset + cpattn::ring_flag_count(B, H, Sq)) * sizeof(int), 256);
  return 0;
}

cp_status_t cp_ring_attention(const void* q, const int64_t* q_strides, const void* const* k_blocks,
                              const void* const* v_blocks, const int64_t* kv_strides,
                              const int* block_len, int ring_degree, int dtype, int B, int H, int D,
                              int Sq, float scale, unsigned flags, float* out,
                              const int64_t* out_strides, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (flags & ~(CP_RING_ANYTHING | CP_RING_SEPARATE_MERGE | CP_RING_PACKED_V | kWaveFlags))
    return fail(CP_ERR_INVALID_ARG, "cp_ring_attention: unknown flags 0x%x", flags);
  if ((flags & kWaveFlags) == kWaveFlags)
    return fail(CP_ERR_INVALID_ARG, "cp_ring_attention: CP_FWD_FOUR_WAVES and CP_FWD_EIGHT_WAVES together");
  const int waves = forced_waves(flags);
  const bool packed = (flags & CP_RING_PACKED_V) != 0;
  if (packed && dtype != CP_BF16)
    return fail(CP_ERR_UNSUPPORTED, "cp_ring_attention: packed V is for CP_BF16 only");
  if (ring_degree < 1)
    return fail(CP_ERR_INVALID_ARG, "cp_ring_attention: ring_degree must be >= 1 (got %d)", ring_degree);
  if (!k_blocks || !v_blocks || !block_len)
    return fail(CP_ERR_INVALID_ARG, "cp_ring_attention: block arrays must be non-null");
  const bool anything = (flags & CP_RING_ANYTHING) != 0;
  int64_t total = 0;
  for (int i = 0; i < ring_degree; ++i) {
    if (block_len[i] < 0)
      return fail(CP_ERR_INVALID_ARG, "cp_ring_attention: block %d has negative length %d", i, block_len[i]);
    if (!anything && block_len[i] != block_len[0])
      return fail(CP_ERR_INVALID_ARG,
                  "cp_ring_attention: block lengths differ (block 0: %d, block %d: %d); plain ring "
                  "attention needs the sequence to divide evenly by ring_degree -- pass "
                  "CP_RING_ANYTHING for uneven blocks",
                  block_len[0], i, block_len[i]);
    total += block_len[i];
  }
  if (!anything && block_len[0] == 0)
    return fail(CP_ERR_INVALID_ARG, "cp_ring_attention: empty blocks need CP_RING_ANYTHING");
  const Strides qs = resolve(q_strides, Sq, H, D);
  const Strides kvs = resolve(kv_strides, total > 0x7fffffff ? 0 : (int)total, H, D);
  const Strides os = resolve(out_strides, Sq, H, D);
  cp_status_t st = check_common(q, qs, kvs, dtype, B, H, D, Sq, scale, out, os, lse);
  if (st != CP_OK) return st;
  for (int i = 0; i < ring_degree; ++i)
    if ((st = check_kv(k_blocks[i], v_blocks[i], block_len[i])) != CP_OK)
      return fail(st, "cp_ring_attention: block %d: %s", i, g_err.c_str());
  const bool separate = (flags & CP_RING_SEPARATE_MERGE) != 0;
  float* ws_out = nullptr;
  float* ws_lse = nullptr;
  int* ws_flags = nullptr;  // one launch for all blocks (see cp_ring_attention_workspace_size)
  if (!separate && workspace != nullptr && B > 0 && H > 0 && Sq > 0 && D == 128 && packed) {
    const size_t need = cp_ring_attention_workspace_size(B, H, Sq, D, flags);
    if (workspace_bytes < need)
      return fail(CP_ERR_WORKSPACE, "cp_ring_attention: workspace of %zu bytes needed, %zu given", need,
                  workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(CP_ERR_UNSUPPORTED, "cp_ring_attention: workspace must be 256-byte aligned");
    ws_flags = static_cast<int*>(workspace);
  }
  if (separate && B > 0 && H > 0 && Sq > 0) {
    const size_t need = partial_bytes(B, H, Sq, D);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(CP_ERR_WORKSPACE, "cp_ring_attention: workspace of %zu bytes needed, %zu given", need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(CP_ERR_UNSUPPORTED, "cp_ring_attention: workspace must be 256-byte aligned");
    ws_out = static_cast<float*>(workspace);
    ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      align_up((size_t)B * Sq * H * D * sizeof(float), 256));
  }
  if (B == 0 || H == 0 || Sq == 0) return CP_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ws_flags != nullptr && packed && one_launch_ring(dtype, B, H, D, Sq, block_len, ring_degree, waves)) {
    const void* kb[16];
    const void* vb[16];
    int len[16], vt0[16], vnt[16];
    int n = 0;
    for (int i = 0; i < ring_degree; ++i) {
      if (block_len[i] == 0) continue;
      kb[n] = k_blocks[i];
      vb[n] = v_blocks[i];
      len[n] = block_len[i];
      vt0[n] = 0;
      vnt[n] = (block_len[i] + 63) / 64;
      ++n;
    }
    if (n == 1) {  // two halves of the one block, split at a 64-key tile boundary
      const int L = len[0], L0 = ((L + 1) / 2 + 63) / 64 * 64;
      kb[1] = static_cast<const char*>(kb[0]) + (int64_t)L0 * kvs.s * 2;
      vb[1] = vb[0];
      len[0] = L0;
      len[1] = L - L0;
      vt0[1] = L0 / 64;
      vnt[1] = vnt[0];
      n = 2;
    }
    const int64_t o_end = ((int64_t)(B - 1) * os.b + (int64_t)(Sq - 1) * os.s + (int64_t)(H - 1) * os.h + D) * 4;
    if (o_end < 0x7fffffff) {
      cpattn::FwdArgs a;
      a.q = q; a.k = nullptr; a.v = nullptr; a.out = out; a.lse = lse;
      a.qs = qs; a.kvs = kvs; a.os = os;
      a.B = B; a.H = H; a.D = D; a.Sq = Sq; a.Skv = 0;
      a.scale = scale;
      a.accumulate = false;
      a.waves = 8;
      a.v_packed = packed;
      const cpattn::RingBlocks rb{n, kb, vb, len, vt0, vnt};
      return hip_status(cpattn::launch_ring_bf16(a, rb, ws_flags, s), "attn_fwd_bf16 (ring)");
    }
  }
  if (packed && !separate && seq_ring(dtype, B, H, D, Sq, block_len, ring_degree, waves)) {
    const void* kb[16];
    const void* vb[16];
    int len[16], vt0[16], vnt[16];
    int n = 0;
    for (int i = 0; i < ring_degree && n < 16; ++i) {
      if (block_len[i] == 0) continue;
      kb[n] = k_blocks[i];
      vb[n] = v_blocks[i];
      len[n] = block_len[i];
      vt0[n] = 0;
      vnt[n] = (block_len[i] + 63) / 64;
      ++n;
    }
    cpattn::FwdArgs a;
    a.q = q; a.k = nullptr; a.v = nullptr; a.out = out; a.lse = lse;
    a.qs = qs; a.kvs = kvs; a.os = os;
    a.B = B; a.H = H; a.D = D; a.Sq = Sq; a.Skv = 0;
    a.scale = scale;
    a.accumulate = false;
    a.waves = 8;
    a.v_packed = true;
    a.err = ws_flags;
    const cpattn::RingBlocks rb{n, kb, vb, len, vt0, vnt};
    return hip_status(cpattn::launch_ring_seq_bf16(a, rb, s), "attn_fwd_bf16 (blocks in turn)");
  }
  if (dtype == CP_F32 && !separate) {
    // 2..4 non-empty float32 blocks: one launch computes and merges them all
    const void* kb[cpattn::kMaxF32RingBlocks];
    const void* vb[cpattn::kMaxF32RingBlocks];
    int len[cpattn::kMaxF32RingBlocks];
    int n = 0;
    for (int i = 0; i < ring_degree && n <= cpattn::kMaxF32RingBlocks; ++i) {
      if (block_len[i] == 0) continue;
      if (n < cpattn::kMaxF32RingBlocks) {
        kb[n] = k_blocks[i];
        vb[n] = v_blocks[i];
        len[n] = block_len[i];
      }
      ++n;
    }
    if (n >= 2 && n <= cpattn::kMaxF32RingBlocks) {
      cpattn::FwdArgs a;
      a.q = q; a.k = nullptr; a.v = nullptr; a.out = out; a.lse = lse;
      a.qs = qs; a.kvs = kvs; a.os = os;
      a.B = B; a.H = H; a.D = D; a.Sq = Sq; a.Skv = 0;
      a.scale = scale;
      a.accumulate = false;
      a.waves = 0;
      a.v_packed = false;
      const cpattn::RingBlocks rb{n, kb, vb, len, nullptr, nullptr};
      return hip_status(cpattn::launch_ring_f32(a, rb, s), "attn_fwd_f32 (ring)");
    }
  }
  const Strides ws_s = resolve(nullptr, Sq, H, D);
  bool have = false;  // does (out, lse) hold a partial yet?
  for (int i = 0; i < ring_degree; ++i) {
    if (block_len[i] == 0) continue;  // a block over no keys has weight 0 in the merge
    if (!have) {
      st = run_block(q, qs, k_blocks[i], v_blocks[i], kvs, dtype, B, H, D, Sq, block_len[i], scale, false,
                     packed, waves, out, os, lse, s, ws_flags);
      have = true;
    } else if (separate) {
      st = run_block(q, qs, k_blocks[i], v_blocks[i], kvs, dtype, B, H, D, Sq, block_len[i], scale, false,
                     packed, waves, ws_out, ws_s, ws_lse, s);
      if (st == CP_OK)
        st = hip_status(cpattn::launch_lse_merge(out, lse, ws_out, ws_lse, os, ws_s, B, H, Sq, D, s),
                        "lse_merge");
    } else {
      st = run_block(q, qs, k_blocks[i], v_blocks[i], kvs, dtype, B, H, D, Sq, block_len[i], scale, true,
                     packed, waves, out, os, lse, s);
    }
    if (st != CP_OK) return st;
  }
  if (!have) return hip_status(cpattn::launch_fill_empty(out, os, lse, B, H, Sq, D, s), "fill_empty");
  return CP_OK;
}

cp_status_t cp_ring_attention_check(const void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "cp_ring_attention_check";
  if (workspace == nullptr || workspace_bytes < (size_t)cpattn::kRingFlagOffset * sizeof(int))
    return fail(CP_ERR_WORKSPACE, "%s: a ring workspace of at least %zu bytes is needed", fn,
                (size_t)cpattn::kRingFlagOffset * sizeof(int));
  if (!aligned(workspace, 256)) return fail(CP_ERR_UNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int gave_up = 0;
  cp_status_t st = hip_status(hipMemcpyAsync(&gave_up, workspace, sizeof(int), hipMemcpyDeviceToHost, s), fn);
  if (st != CP_OK) return st;
  if ((st = hip_status(hipStreamSynchronize(s), fn)) != CP_OK) return st;
  if (gave_up != 0)
    return fail(CP_ERR_ORDER,
                "%s: %d merge wait(s) of the last parallel-partials ring launch gave up; the query tiles "
                "concerned hold NaN",
                fn, gave_up);
  return CP_OK;
}

size_t cp_attn_bwd_workspace_size(int B, int H, int Sq, int D) {
  if (B <= 0 || H <= 0 || Sq <= 0 || D <= 0) return 0;
  return align_up((size_t)B * Sq * H * D * 2, 256) + align_up((size_t)B * H * Sq * sizeof(float), 256);
}

}  // extern "C"

namespace {

// The two parts of the backward workspace: dO in bf16 and delta.
struct BwdWorkspace {
  void* dout_b;
  float* delta;
};

cp_status_t bwd_workspace(const char* fn, void* workspace, size_t bytes, int B, int H, int Sq, int D,
                          BwdWorkspace* w) {
  const size_t need = cp_attn_bwd_workspace_size(B, H, Sq, D);
  if (workspace == nullptr || bytes < need)
    return fail(CP_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace == nullptr ? (size_t)0 : bytes);
  if (!aligned(workspace, 256)) return fail(CP_ERR_UNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
  w->dout_b = workspace;
  w->delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up((size_t)B * Sq * H * D * 2, 256));
  return CP_OK;
}

cp_status_t check_bwd_common(const char* fn, int dtype, int B, int H, int D, int Sq, float scale) {
  if (dtype != CP_BF16)
    return fail(CP_ERR_UNSUPPORTED, "%s: the backward supports dtype CP_BF16 (1) only (got %d)", fn, dtype);
  if (D != 64 && D != 128)
    return fail(CP_ERR_UNSUPPORTED, "%s: head dim D=%d is not supported (D = 64 or 128)", fn, D);
  if (B < 0 || H < 0 || Sq < 0) return fail(CP_ERR_INVALID_ARG, "%s: sizes must be non-negative", fn);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(CP_ERR_INVALID_ARG, "%s: scale must be finite and > 0 (got %g)", fn, (double)scale);
  return CP_OK;
}

// A second stream per device for the backward's dq kernels, which then run
// concurrently with the dkv kernels on the caller's stream (each kind alone
// leaves workgroup slots idle on the FLUX-sized shares). Created on first use
// outside graph capture (non-blocking, default priority) and kept for the
// life of the process. A call forks it from the caller's stream with an event
// and joins it back with another before returning, so the caller sees one
// stream-ordered operation, also when capturing a graph (the side stream then
// joins the capture through the fork event). The fork-join sequence is
// enqueued under a lock, since the events are shared per device.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;  // creation failed once: run single-stream from then on
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// Whether the backward's dq and dkv kernels should share the GPU. Each kind
// runs 4-wave workgroups, two per CU. Measured on MI355X, running them
// concurrently pays when a kernel alone would leave a quarter or more of its
// last round of workgroup slots idle (ring-anything share: 1018 -> 855 us per
// pass; USP share 430 -> 343 us), and costs where every round is full (32k
// ring-4 share: 10.56 -> 11.38 ms, the two kernels' workgroups then compete
// for each XCD's L2) or nearly so (FLUX ring-2 and Ulysses-2 shares: within
// 2%). n_dq, n_dkv: workgroups of one launch of each kernel.
bool bwd_concurrent(int64_t n_dq, int64_t n_dkv) {
  if (!CP_BWD_SIDE_STREAM) return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return false;
  }
  const int64_t slots = 2 * (int64_t)cus;
  auto idle_quarter = [&](int64_t n) {
    if (n <= 0) return false;
    const int64_t cap = (n + slots - 1) / slots * slots;
    return 4 * (cap - n) >= cap;
  };
  return idle_quarter(n_dq) || idle_quarter(n_dkv);
}

// Under g_side_mu: the device's side stream forked from s, or nullptr to run
// everything on s (no device id, s belongs to another device than the
// current one, creation failed, first use while s is being captured, or the
// side stream is part of a graph capture that s is not).
hipStream_t side_fork(hipStream_t s) {
  if (!CP_BWD_SIDE_STREAM) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev) {
      (void)hipGetLastError();
      return nullptr;
    }
  }
  SideStream& ss = g_side[dev];
  if (ss.failed) return nullptr;
  if (ss.s == nullptr) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      ss.failed = true;
      (void)hipGetLastError();
      return nullptr;
    }
  }
  // The side stream joins a graph capture through the fork event and stays
  // in it until that capture ends. While it is part of a capture that s does
  // not belong to (another thread's), this call runs on s alone.
  hipStreamCaptureStatus side_cs = hipStreamCaptureStatusNone;
  unsigned long long side_id = 0;
  if (hipStreamGetCaptureInfo(ss.s, &side_cs, &side_id) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (side_cs != hipStreamCaptureStatusNone) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    if (hipStreamGetCaptureInfo(s, &cs, &id) != hipSuccess || cs != hipStreamCaptureStatusActive || id != side_id) {
      (void)hipGetLastError();
      return nullptr;
    }
  }
  if (hipEventRecord(ss.fork, s) != hipSuccess) return nullptr;
  if (hipStreamWaitEvent(ss.s, ss.fork, 0) != hipSuccess) return nullptr;
  return ss.s;
}

// Under g_side_mu: s waits for everything enqueued on the side stream.
hipError_t side_join(hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  SideStream& ss = g_side[dev];
  if ((e = hipEventRecord(ss.join, ss.s)) != hipSuccess) return e;
  return hipStreamWaitEvent(s, ss.join, 0);
}

// Arguments of one block's backward once the common checks passed.
cp_status_t run_block_bwd(const void* q, Strides qs, const void* k, const void* v, Strides kvs, int B, int H,
                          int D, int Sq, int Skv, float scale, bool accumulate_dq, const float* lse,
                          const BwdWorkspace& w, float* dq, Strides dqs, float* dk, float* dv, Strides dkvs,
                          hipStream_t stream, hipStream_t dq_stream = nullptr) {
  if (Skv == 0 && accumulate_dq) return CP_OK;  // no keys: nothing to add
  cpattn::BwdArgs a;
  a.q = q; a.k = k; a.v = v;
  a.dout_b = w.dout_b; a.lse = lse; a.delta = w.delta;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.qs = qs; a.kvs = kvs; a.dqs = dqs; a.dkvs = dkvs;
  a.B = B; a.H = H; a.D = D; a.Sq = Sq; a.Skv = Skv;
  a.scale = scale;
  a.accumulate_dq = accumulate_dq;
  a.dq_stream = dq_stream;
  return hip_status(cpattn::launch_attn_bwd_bf16(a, stream), "attn_bwd_bf16");
}

// Q side (when Sq > 0) and the stride limits of the tile loads: row offsets
// within a 32-row tile are 32-bit, so sequence strides (and H*D, the row
// stride of the bf16 dO copy) stay at most 2^24 elements.
cp_status_t check_bwd_tensors(const char* fn, int Sq, int H, int D, const void* q, Strides qs, Strides kvs,
                              const float* lse, const float* dq, Strides dqs, Strides dkvs) {
  cp_status_t st;
  if ((st = check_strides("k/v", kvs, 2, 2, H, D)) != CP_OK) return st;
  if ((st = check_strides("dk/dv", dkvs, 4, 2, H, D)) != CP_OK) return st;
  if (qs.s > (int64_t(1) << 24) || kvs.s > (int64_t(1) << 24) || (int64_t)H * D > (int64_t(1) << 24))
    return fail(CP_ERR_UNSUPPORTED, "%s: q and k/v sequence strides and H*D must not exceed 2^24 elements", fn);
  if (Sq == 0) return CP_OK;
  if (!q || !dq || !lse) return fail(CP_ERR_INVALID_ARG, "%s: q, dq and lse must be non-null", fn);
  if (!aligned(q, 16) || !aligned(dq, 16) || !aligned(lse, 4))
    return fail(CP_ERR_UNSUPPORTED, "%s: q and dq must be 16-byte aligned, lse 4-byte aligned", fn);
  // q rows are fetched in tiles through a byte range that ends at row Sq, so
  // a row must not extend past the next one's start even when Sq == 1.
  if ((st = check_strides("q", qs, 2, 2, H, D)) != CP_OK) return st;
  if ((st = check_strides("dq", dqs, 4, Sq, H, D)) != CP_OK) return st;
  return CP_OK;
}

}  // namespace

extern "C" {

cp_status_t cp_attn_bwd_prep(const float* out, const int64_t* out_strides, const float* dout,
                             const int64_t* dout_strides, int dtype, int B, int H, int Sq, int D,
                             void* workspace, size_t workspace_bytes, void* stream) {
  cp_status_t st = check_bwd_common("cp_attn_bwd_prep", dtype, B, H, D, Sq, 1.f);
  if (st != CP_OK) return st;
  if (B == 0 || H == 0 || Sq == 0) return CP_OK;
  if (!out || !dout) return fail(CP_ERR_INVALID_ARG, "cp_attn_bwd_prep: out and dout must be non-null");
  if (!aligned(out, 16) || !aligned(dout, 16))
    return fail(CP_ERR_UNSUPPORTED, "cp_attn_bwd_prep: out and dout must be 16-byte aligned");
  if ((int64_t)B * Sq * H * (D / 8) > 0x7fffffff)
    return fail(CP_ERR_UNSUPPORTED, "cp_attn_bwd_prep: B*Sq*H*D/8 must be below 2^31");
  const Strides os = resolve(out_strides, Sq, H, D);
  const Strides ds = resolve(dout_strides, Sq, H, D);
  if ((st = check_strides("out", os, 4, Sq, H, D)) != CP_OK) return st;
  if ((st = check_strides("dout", ds, 4, Sq, H, D)) != CP_OK) return st;
  BwdWorkspace w;
  if ((st = bwd_workspace("cp_attn_bwd_prep", workspace, workspace_bytes, B, H, Sq, D, &w)) != CP_OK) return st;
  return hip_status(cpattn::launch_attn_bwd_prep(out, os, dout, ds, w.dout_b, w.delta, B, H, Sq, D,
                                                 static_cast<hipStream_t>(stream)),
                    "attn_bwd_prep");
}

cp_status_t cp_attn_block_bwd(const void* q, const int64_t* q_strides, const void* k, const void* v,
                              const int64_t* kv_strides, int dtype, int B, int H, int D, int Sq, int Skv,
                              float scale, unsigned flags, const float* lse, const void* workspace,
                              size_t workspace_bytes, float* dq, const int64_t* dq_strides, float* dk, float* dv,
                              const int64_t* dkv_strides, void* stream) {
  const char* fn = "cp_attn_block_bwd";
  if (flags & ~CP_BWD_ACCUMULATE_DQ) return fail(CP_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
  cp_status_t st = check_bwd_common(fn, dtype, B, H, D, Sq, scale);
  if (st != CP_OK) return st;
  if (Skv < 0) return fail(CP_ERR_INVALID_ARG, "%s: K/V length must be non-negative (got %d)", fn, Skv);
  if (B == 0 || H == 0 || (Sq == 0 && Skv == 0)) return CP_OK;
  const Strides qs = resolve(q_strides, Sq, H, D);
  const Strides kvs = resolve(kv_strides, Skv, H, D);
  const Strides dqs = resolve(dq_strides, Sq, H, D);
  const Strides dkvs = resolve(dkv_strides, Skv, H, D);
  if ((st = check_bwd_tensors(fn, Sq, H, D, q, qs, kvs, lse, dq, dqs, dkvs)) != CP_OK) return st;
  if ((st = check_kv(k, v, Skv)) != CP_OK) return st;
  if (Skv > 0 && (!dk || !dv || !aligned(dk, 16) || !aligned(dv, 16)))
    return fail(CP_ERR_INVALID_ARG, "%s: dk and dv must be non-null and 16-byte aligned", fn);
  BwdWorkspace w{nullptr, nullptr};  // with no queries the kernels read no dO and no delta
  if (Sq > 0 && (st = bwd_workspace(fn, const_cast<void*>(workspace), workspace_bytes, B, H, Sq, D, &w)) != CP_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Sq == 0 || Skv == 0)  // one kernel at most
    return run_block_bwd(q, qs, k, v, kvs, B, H, D, Sq, Skv, scale, (flags & CP_BWD_ACCUMULATE_DQ) != 0, lse, w,
                         dq, dqs, dk, dv, dkvs, s);
  std::lock_guard<std::mutex> lock(g_side_mu);
  const int64_t bh = (int64_t)B * H;
  hipStream_t side = bwd_concurrent(bh * ((Sq + 127) / 128), bh * ((Skv + 127) / 128)) ? side_fork(s) : nullptr;
  st = run_block_bwd(q, qs, k, v, kvs, B, H, D, Sq, Skv, scale, (flags & CP_BWD_ACCUMULATE_DQ) != 0, lse, w, dq,
                     dqs, dk, dv, dkvs, s, side);
  if (side != nullptr) {
    const cp_status_t sj = hip_status(side_join(s), "attn_bwd_bf16 (join)");
    if (st == CP_OK) st = sj;
  }
  return st;
}

cp_status_t cp_ring_attention_bwd(const void* q, const int64_t* q_strides, const void* const* k_blocks,
                                  const void* const* v_blocks, const int64_t* kv_strides, const int* block_len,
                                  int ring_degree, int dtype, int B, int H, int D, int Sq, float scale,
                                  unsigned flags, const float* out, const int64_t* out_strides, const float* dout,
                                  const int64_t* dout_strides, const float* lse, float* dq,
                                  const int64_t* dq_strides, float* const* dk_blocks, float* const* dv_blocks,
                                  const int64_t* dkv_strides, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  const char* fn = "cp_ring_attention_bwd";
  if (flags & ~CP_RING_ANYTHING) return fail(CP_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
  if (ring_degree < 1) return fail(CP_ERR_INVALID_ARG, "%s: ring_degree must be >= 1 (got %d)", fn, ring_degree);
  if (!k_blocks || !v_blocks || !block_len || !dk_blocks || !dv_blocks)
    return fail(CP_ERR_INVALID_ARG, "%s: block arrays must be non-null", fn);
  const bool anything = (flags & CP_RING_ANYTHING) != 0;
  int64_t total = 0;
  for (int i = 0; i < ring_degree; ++i) {
    if (block_len[i] < 0)
      return fail(CP_ERR_INVALID_ARG, "%s: block %d has negative length %d", fn, i, block_len[i]);
    if (!anything && block_len[i] != block_len[0])
      return fail(CP_ERR_INVALID_ARG, "%s: block lengths differ (block 0: %d, block %d: %d); pass "
                  "CP_RING_ANYTHING for uneven blocks", fn, block_len[0], i, block_len[i]);
    total += block_len[i];
  }
  if (!anything && block_len[0] == 0) return fail(CP_ERR_INVALID_ARG, "%s: empty blocks need CP_RING_ANYTHING", fn);
  cp_status_t st = check_bwd_common(fn, dtype, B, H, D, Sq, scale);
  if (st != CP_OK) return st;
  if (B == 0 || H == 0) return CP_OK;
  const int tot = total > 0x7fffffff ? 0 : (int)total;
  const Strides qs = resolve(q_strides, Sq, H, D);
  const Strides kvs = resolve(kv_strides, tot, H, D);
  const Strides dqs = resolve(dq_strides, Sq, H, D);
  const Strides dkvs = resolve(dkv_strides, tot, H, D);
  if ((st = check_bwd_tensors(fn, Sq, H, D, q, qs, kvs, lse, dq, dqs, dkvs)) != CP_OK) return st;
  for (int i = 0; i < ring_degree; ++i) {
    if ((st = check_kv(k_blocks[i], v_blocks[i], block_len[i])) != CP_OK)
      return fail(st, "%s: block %d: %s", fn, i, g_err.c_str());
    if (block_len[i] > 0 && (!dk_blocks[i] || !dv_blocks[i] || !aligned(dk_blocks[i], 16) ||
                             !aligned(dv_blocks[i], 16)))
      return fail(CP_ERR_INVALID_ARG, "%s: block %d: dk and dv must be non-null and 16-byte aligned", fn, i);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  BwdWorkspace w{nullptr, nullptr};
  if (Sq > 0) {
    if ((st = bwd_workspace(fn, workspace, workspace_bytes, B, H, Sq, D, &w)) != CP_OK) return st;
    if (!out || !dout || !aligned(out, 16) || !aligned(dout, 16))
      return fail(CP_ERR_INVALID_ARG, "%s: out and dout must be non-null and 16-byte aligned", fn);
    const Strides os = resolve(out_strides, Sq, H, D);
    const Strides ds = resolve(dout_strides, Sq, H, D);
    if ((st = check_strides("out", os, 4, Sq, H, D)) != CP_OK) return st;
    if ((st = check_strides("dout", ds, 4, Sq, H, D)) != CP_OK) return st;
    if ((int64_t)B * Sq * H * (D / 8) > 0x7fffffff)
      return fail(CP_ERR_UNSUPPORTED, "%s: B*Sq*H*D/8 must be below 2^31", fn);
    if ((st = hip_status(cpattn::launch_attn_bwd_prep(out, os, dout, ds, w.dout_b, w.delta, B, H, Sq, D, s),
                         "attn_bwd_prep")) != CP_OK)
      return st;
  }  // with no queries every dK, dV is zero (the dkv kernel still writes them) and no workspace is read
  bool have_dq = false;
  {
    // dq kernels (a chain: each block adds into dQ) on the side stream, dkv
    // kernels on s; with no queries only the dkv kernels run
    std::lock_guard<std::mutex> lock(g_side_mu);
    int longest = 0, n_nonempty = 0;
    for (int i = 0; i < ring_degree; ++i) {
      longest = block_len[i] > longest ? block_len[i] : longest;
      n_nonempty += block_len[i] > 0;
    }
    // Where one launch of either kernel fills its slots (no second stream), the
    // whole ring runs as two launches (dQ through the blocks in turn, dK/dV of
    // all blocks in one grid): FLUX ring-2 share 635 -> 608 us per pass, 32k
    // ring-4 10.77 -> 10.65 ms. With the second stream the per-block pairs
    // overlap better (USP share 346 us per block pair vs 384 as two launches:
    // the long dQ workgroups hold their slots and push part of the dK/dV grid
    // into a second round).
    const int64_t bh = (int64_t)B * H;
    const bool conc = Sq > 0 && bwd_concurrent(bh * ((Sq + 127) / 128), bh * ((longest + 127) / 128));
    const bool multi =
        CP_BWD_MULTI && !conc && Sq > 0 && n_nonempty >= 2 && n_nonempty <= cpattn::kMaxBwdBlocks;
    hipStream_t side = conc ? side_fork(s) : nullptr;
    if (multi) {
      const void* kb[cpattn::kMaxBwdBlocks];
      const void* vb[cpattn::kMaxBwdBlocks];
      float* dkb[cpattn::kMaxBwdBlocks];
      float* dvb[cpattn::kMaxBwdBlocks];
      int len[cpattn::kMaxBwdBlocks];
      int n = 0;
      for (int i = 0; i < ring_degree; ++i) {
        if (block_len[i] == 0) continue;
        kb[n] = k_blocks[i];
        vb[n] = v_blocks[i];
        dkb[n] = dk_blocks[i];
        dvb[n] = dv_blocks[i];
        len[n] = block_len[i];
        ++n;
      }
      cpattn::BwdArgs a;
      a.q = q; a.k = nullptr; a.v = nullptr;
      a.dout_b = w.dout_b; a.lse = lse; a.delta = w.delta;
      a.dq = dq; a.dk = nullptr; a.dv = nullptr;
      a.qs = qs; a.kvs = kvs; a.dqs = dqs; a.dkvs = dkvs;
      a.B = B; a.H = H; a.D = D; a.Sq = Sq; a.Skv = 0;
      a.scale = scale;
      a.accumulate_dq = false;
      a.dq_stream = side;
      const cpattn::BwdBlocks bb{n, kb, vb, dkb, dvb, len};
      st = hip_status(cpattn::launch_attn_bwd_ring_bf16(a, bb, s), "attn_bwd_bf16 (ring)");
      have_dq = true;
    }
    for (int i = 0; i < ring_degree && st == CP_OK && !multi; ++i) {
      if (block_len[i] == 0) continue;
      st = run_block_bwd(q, qs, k_blocks[i], v_blocks[i], kvs, B, H, D, Sq, block_len[i], scale, have_dq, lse, w,
                         dq, dqs, dk_blocks[i], dv_blocks[i], dkvs, s, side);
      have_dq = true;
    }
    if (side != nullptr) {
      const cp_status_t sj = hip_status(side_join(s), "attn_bwd_bf16 (join)");
      if (st == CP_OK) st = sj;
    }
    if (st != CP_OK) return st;
  }
  if (!have_dq && Sq > 0)  // every block empty: dQ = 0 (the dq kernel over no keys writes zeros)
    return run_block_bwd(q, qs, nullptr, nullptr, kvs, B, H, D, Sq, 0, scale, false, lse, w, dq, dqs, nullptr,
                         nullptr, dkvs, s);
  return CP_OK;
}

}  // extern "C"

namespace {

// Checks and launch shared by cp_ulysses_regroup (one tensor) and cp_ulysses_regroup_multi.
cp_status_t regroup_impl(const char* fn, const void* const* in, void* const* out, int n_tensors, int elem_bytes,
                         int B, int S_local, int H, int D, int degree, int direction, void* stream) {
  if (elem_bytes != 2 && elem_bytes != 4)
    return fail(CP_ERR_UNSUPPORTED, "%s: elem_bytes must be 2 or 4 (got %d)", fn, elem_bytes);
  if (B < 0 || S_local < 0 || H < 0 || D < 0) return fail(CP_ERR_INVALID_ARG, "%s: sizes must be non-negative", fn);
  if (degree < 1) return fail(CP_ERR_INVALID_ARG, "%s: degree must be >= 1 (got %d)", fn, degree);
  if (H % degree != 0)
    return fail(CP_ERR_INVALID_ARG, "%s: the number of heads H=%d must be divisible by the Ulysses degree %d", fn,
                H, degree);
  if (direction != CP_REGROUP_SEQ_TO_HEAD && direction != CP_REGROUP_HEAD_TO_SEQ)
    return fail(CP_ERR_INVALID_ARG, "%s: unknown direction %d", fn, direction);
  const int64_t bytes = (int64_t)B * S_local * H * D * elem_bytes;
  if (bytes == 0) return CP_OK;
  auto overlap = [bytes](const void* x, const void* y) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes;
  };
  for (int i = 0; i < n_tensors; ++i) {
    if (!in[i] || !out[i]) return fail(CP_ERR_INVALID_ARG, "%s: pointers must be non-null", fn);
    if (!aligned(in[i], elem_bytes) || !aligned(out[i], elem_bytes))
      return fail(CP_ERR_UNSUPPORTED, "%s: pointers must be aligned to elem_bytes", fn);
    for (int j = 0; j < n_tensors; ++j) {
      if (overlap(in[j], out[i])) return fail(CP_ERR_INVALID_ARG, "%s: in and out overlap", fn);
      if (j != i && overlap(out[j], out[i])) return fail(CP_ERR_INVALID_ARG, "%s: outputs %d and %d overlap", fn, j, i);
    }
  }
  return hip_status(cpattn::launch_regroup(in, out, n_tensors, elem_bytes, B, S_local, H, D, degree, direction,
                                           static_cast<hipStream_t>(stream)),
                    "ulysses_regroup");
}

}  // namespace

extern "C" {

cp_status_t cp_ulysses_regroup(const void* in, void* out, int elem_bytes, int B, int S_local, int H,
                               int D, int degree, int direction, void* stream) {
  return regroup_impl("cp_ulysses_regroup", &in, &out, 1, elem_bytes, B, S_local, H, D, degree, direction, stream);
}

cp_status_t cp_ulysses_regroup_multi(const void* const* in, void* const* out, int n_tensors, int elem_bytes, int B,
                                     int S_local, int H, int D, int degree, int direction, void* stream) {
  const char* fn = "cp_ulysses_regroup_multi";
  if (n_tensors < 1 || n_tensors > cpattn::kMaxRegroupTensors)
    return fail(CP_ERR_INVALID_ARG, "%s: n_tensors must be in 1..%d (got %d)", fn, cpattn::kMaxRegroupTensors,
                n_tensors);
  if (!in || !out) return fail(CP_ERR_INVALID_ARG, "%s: pointer arrays must be non-null", fn);
  return regroup_impl(fn, in, out, n_tensors, elem_bytes, B, S_local, H, D, degree, direction, stream);
}

}  // extern "C"
namespace {

// Shared checks of the uneven packs; *total receives the sum of counts.
cp_status_t check_pieces(const char* fn, const void* in, void* out, int elem_bytes, int B, int other, int D,
                         int degree, const int* counts, int direction, int64_t* total) {
  if (elem_bytes != 2 && elem_bytes != 4)
    return fail(CP_ERR_UNSUPPORTED, "%s: elem_bytes must be 2 or 4 (got %d)", fn, elem_bytes);
  if (B < 0 || other < 0 || D < 0) return fail(CP_ERR_INVALID_ARG, "%s: sizes must be non-negative", fn);
  if (degree < 1 || degree > cpattn::kMaxUlyssesDegree)
    return fail(CP_ERR_INVALID_ARG, "%s: degree must be in 1..%d (got %d)", fn, cpattn::kMaxUlyssesDegree,
                degree);
  if (!counts) return fail(CP_ERR_INVALID_ARG, "%s: counts must be non-null", fn);
  if (direction != CP_REGROUP_SEQ_TO_HEAD && direction != CP_REGROUP_HEAD_TO_SEQ)
    return fail(CP_ERR_INVALID_ARG, "%s: unknown direction %d", fn, direction);
  int64_t t = 0;
  for (int g = 0; g < degree; ++g) {
    if (counts[g] < 0) return fail(CP_ERR_INVALID_ARG, "%s: counts[%d] = %d is negative", fn, g, counts[g]);
    t += counts[g];
  }
  *total = t;
  const int64_t bytes = (int64_t)B * other * t * D * elem_bytes;
  if (bytes == 0) return CP_OK;
  if (bytes >= (int64_t(1) << 32))
    return fail(CP_ERR_UNSUPPORTED, "%s: tensors of 2^32 bytes or more are not supported", fn);
  if (!in || !out) return fail(CP_ERR_INVALID_ARG, "%s: pointers must be non-null", fn);
  const uintptr_t a = reinterpret_cast<uintptr_t>(in), b = reinterpret_cast<uintptr_t>(out);
  if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes)
    return fail(CP_ERR_INVALID_ARG, "%s: in and out overlap", fn);
  if (!aligned(in, elem_bytes) || !aligned(out, elem_bytes))
    return fail(CP_ERR_UNSUPPORTED, "%s: pointers must be aligned to elem_bytes", fn);
  return CP_OK;
}

}  // namespace

extern "C" {

cp_status_t cp_ulysses_pack_heads(const void* in, void* out, int elem_bytes, int B, int S_r, int D, int degree,
                                  const int* head_counts, int direction, void* stream) {
  int64_t H = 0;
  cp_status_t st = check_pieces("cp_ulysses_pack_heads", in, out, elem_bytes, B, S_r, D, degree, head_counts,
                                direction, &H);
  if (st != CP_OK || (int64_t)B * S_r * H * D == 0) return st;
  // [B*S_r, H heads] rows split by head: axis 2 with one unit per head
  return hip_status(cpattn::launch_pieces(in, out, 2, 1, (int64_t)B * S_r, (int64_t)D * elem_bytes, H,
                                          head_counts, degree, direction == CP_REGROUP_SEQ_TO_HEAD,
                                          static_cast<hipStream_t>(stream)),
                    "ulysses_pack_heads");
}

cp_status_t cp_ulysses_concat_seq(const void* in, void* out, int elem_bytes, int B, int H_g, int D, int degree,
                                  const int* seq_counts, int direction, void* stream) {
  int64_t S = 0;
  cp_status_t st = check_pieces("cp_ulysses_concat_seq", in, out, elem_bytes, B, H_g, D, degree, seq_counts,
                                direction, &S);
  if (st != CP_OK || (int64_t)B * S * H_g * D == 0) return st;
  // [B, S tokens, one token's H_g*D elements] split by token: axis 1
  return hip_status(cpattn::launch_pieces(in, out, 1, B, S, (int64_t)H_g * D * elem_bytes, 1, seq_counts, degree,
                                          direction == CP_REGROUP_HEAD_TO_SEQ, static_cast<hipStream_t>(stream)),
                    "ulysses_concat_seq");
}

}  // extern "C"

// ---- cp_ring_attention_noalloc: the ring with a library-owned static workspace
namespace {

// Device memory the no-allocation ring uses in place of a caller's workspace: the
// parallel-partials form's error count and per-tile flags. One copy per GPU, for the life of
// the process; every call on a GPU shares it.
constexpr size_t kScratchBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device (with that device
// current). In host code the array's own name is not a device address.
cp_status_t scratch_address(const char* fn, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(CP_ERR_UNSUPPORTED, "%s: device %d is beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, fn);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CP_OK;
}

}  // namespace

extern "C" {

cp_status_t cp_ring_attention_noalloc(const void* q, const int64_t* q_strides, const void* const* k_blocks,
                                      const void* const* v_blocks, const int64_t* kv_strides, const int* block_len,
                                      int ring_degree, int dtype, int B, int H, int D, int Sq, float scale,
                                      unsigned flags, float* out, const int64_t* out_strides, float* lse,
                                      void* stream) {
  const char* fn = "cp_ring_attention_noalloc";
  if (flags & CP_RING_SEPARATE_MERGE)
    return fail(CP_ERR_INVALID_ARG, "%s: CP_RING_SEPARATE_MERGE needs a caller workspace (use cp_ring_attention)", fn);
  const size_t need = cp_ring_attention_workspace_size(B, H, Sq, D, flags);
  if (need > kScratchBytes)
    return fail(CP_ERR_WORKSPACE,
                "%s: these sizes need %zu bytes of workspace, more than the %zu-byte static scratch "
                "(B*H*ceil(Sq/256) must stay at most %zu); use cp_ring_attention with a workspace",
                fn, need, kScratchBytes, (kScratchBytes - 256) / sizeof(int));
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (need > 0) {
    cp_status_t st = scratch_address(fn, &ws);
    if (st != CP_OK) return st;
    ws_bytes = kScratchBytes;
  }
  return cp_ring_attention(q, q_strides, k_blocks, v_blocks, kv_strides, block_len, ring_degree, dtype, B, H, D,
                           Sq, scale, flags, out, out_strides, lse, ws, ws_bytes, stream);
}

}  // extern "C"
