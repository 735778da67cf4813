// pa_api.cpp -- the C ABI of libpa.so: argument checks, dispatch to the launchers, host-side
// validators and the thread-local error message.  No exception crosses the ABI.

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <algorithm>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

static_assert(pa::kSharedRunColumns == PA_SHARED_RUN_COLUMNS, "run columns of the kernels");

namespace {
thread_local std::string g_error;
}  // namespace

int pa::set_error_v(int code, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_error = buf;
  return code;
}

int pa::set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = set_error_v(code, fmt, ap);
  va_end(ap);
  return r;
}

int pa::clear_error() {
  g_error.clear();
  return PA_OK;
}

namespace {

__attribute__((format(printf, 2, 3))) int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = pa::set_error_v(code, fmt, ap);
  va_end(ap);
  return r;
}

int ok() { return pa::clear_error(); }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(int d) { return d == PA_F32 || d == PA_BF16 || d == PA_FP8_E4M3; }
int elem_bytes(int d) { return d == PA_F32 ? 4 : (d == PA_BF16 ? 2 : 1); }

// Shapes the kernels are built for.
int check_shape(int D, int bs, int kv_dtype) {
  if (D != 64 && D != 128) return fail(PA_ENOTSUP, "head_dim %d not supported (64 or 128)", D);
  if (bs != 16 && bs != 32) return fail(PA_ENOTSUP, "block_size %d not supported (16 or 32)", bs);
  if (!valid_dtype(kv_dtype)) return fail(PA_EINVAL, "unknown kv dtype %d", kv_dtype);
  if (kv_dtype == PA_F32 && D == 128 && bs == 32)
    return fail(PA_ENOTSUP, "f32 cache with head_dim 128 and block_size 32 not supported");
  return PA_OK;
}

int check_heads(int Hq, int Hkv) {
  if (Hq < 1 || Hkv < 1) return fail(PA_EINVAL, "head counts must be positive (Hq %d, Hkv %d)", Hq, Hkv);
  if (Hq % Hkv) return fail(PA_EINVAL, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PA_ENOTSUP, "query heads per kv head %d not supported (1, 2, 4, 8, 16)", G);
  if (Hkv > 65535) return fail(PA_ENOTSUP, "Hkv %d too large", Hkv);
  return PA_OK;
}

int check_attn_dtypes(int q_dtype, int kv_dtype) {
  if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype))
    return fail(PA_EINVAL, "unknown dtype (q %d, kv %d)", q_dtype, kv_dtype);
  const bool okc = (q_dtype == PA_F32 && kv_dtype == PA_F32) ||
                   (q_dtype == PA_BF16 && kv_dtype == PA_BF16) ||
                   (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3);
  if (!okc) return fail(PA_ENOTSUP, "dtype combination q %d / kv %d not supported", q_dtype, kv_dtype);
  return PA_OK;
}

int check_scales(int kv_dtype, float k_scale, float v_scale) {
  if (kv_dtype != PA_FP8_E4M3) return PA_OK;
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PA_EINVAL, "fp8 scales must be finite and positive (k %g, v %g)", k_scale, v_scale);
  return PA_OK;
}

}  // namespace

int pa::device_compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

extern "C" {

const char* pa_last_error(void) { return g_error.c_str(); }

const char* pa_build_info(void) { return "libpa 0.1 (paged attention), kernels for gfx950"; }

int pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t T, int64_t NB, int Hkv, int D,
                         int block_size, pa_dtype src_dtype, pa_dtype kv_dtype, float k_scale,
                         float v_scale, void* stream) {
  if (T < 0 || NB < 1 || Hkv < 1) return fail(PA_EINVAL, "bad sizes (T %lld, NB %lld, Hkv %d)", (long long)T, (long long)NB, Hkv);
  if (int r = check_shape(D, block_size, kv_dtype)) return r;
  if (!valid_dtype(src_dtype) || src_dtype == PA_FP8_E4M3)
    return fail(PA_EINVAL, "source dtype %d must be f32 or bf16", (int)src_dtype);
  const bool okc = (kv_dtype == src_dtype) || kv_dtype == PA_FP8_E4M3;
  if (!okc) return fail(PA_ENOTSUP, "storing dtype %d rows in a dtype %d cache not supported", (int)src_dtype, (int)kv_dtype);
  if (int r = check_scales(kv_dtype, k_scale, v_scale)) return r;
  if (T > 0x7fffffff) return fail(PA_ENOTSUP, "T %lld too large for one call", (long long)T);
  if (T == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return fail(PA_EINVAL, "null pointer argument");
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15)
    return fail(PA_EINVAL, "k, v and the caches must be 16-byte aligned");
  return hip_status(pa::launch_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, T, NB, Hkv, D,
                                                 block_size, src_dtype, kv_dtype, k_scale, v_scale,
                                                 (hipStream_t)stream),
                    "reshape_and_cache launch");
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int64_t N, int64_t NB,
                   int Hkv, int D, int block_size, pa_dtype kv_dtype, void* stream) {
  if (N < 0 || NB < 1 || Hkv < 1) return fail(PA_EINVAL, "bad sizes (N %lld, NB %lld, Hkv %d)", (long long)N, (long long)NB, Hkv);
  if (int r = check_shape(D, block_size, kv_dtype)) return r;
  if (N > 0x7fffffff) return fail(PA_ENOTSUP, "N %lld too large for one call", (long long)N);
  if (N == 0) return ok();
  if (!k_cache || !v_cache || !pairs) return fail(PA_EINVAL, "null pointer argument");
  const int64_t frame_bytes = (int64_t)Hkv * block_size * D * elem_bytes(kv_dtype);
  return hip_status(pa::launch_copy_blocks(k_cache, v_cache, pairs, N, NB, frame_bytes, (hipStream_t)stream),
                    "copy_blocks launch");
}

size_t pa_decode_workspace_bytes(int B, int Hq, int D, int block_size, pa_dtype kv_dtype,
                                 int max_context_len) {
  if (B <= 0 || Hq <= 0 || D <= 0 || block_size <= 0 || max_context_len <= 0) return 0;
  return pa::decode_workspace_bytes(B, Hq, D, block_size, kv_dtype, max_context_len);
}

int pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
              int B, int Hq, int Hkv, int D, int block_size, int64_t NB, float scale,
              pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
              int max_context_len, void* workspace, size_t workspace_bytes, unsigned flags,
                 void* stream) {
  if (B < 0 || NB < 1 || max_blocks_per_seq < 1)
    return fail(PA_EINVAL, "bad sizes (B %d, NB %lld, max_blocks_per_seq %d)", B, (long long)NB, max_blocks_per_seq);
  if (B > 65535) return fail(PA_ENOTSUP, "batch %d too large for one call (max 65535)", B);
  if (int r = check_heads(Hq, Hkv)) return r;
  if (int r = check_shape(D, block_size, kv_dtype)) return r;
  if (int r = check_attn_dtypes(q_dtype, kv_dtype)) return r;
  if (int r = check_scales(kv_dtype, k_scale, v_scale)) return r;
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale must be finite");
  if (flags & ~(unsigned)PA_DECODE_SHARED_FRAMES) return fail(PA_EINVAL, "unknown decode flags 0x%x", flags);
  if (B == 0) return ok();
  if (max_context_len < 1) return fail(PA_EINVAL, "max_context_len %d must be positive", max_context_len);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_EINVAL, "null pointer argument");
  const size_t need = pa::decode_workspace_bytes(B, Hq, D, block_size, kv_dtype, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ENOSPC, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && ((uintptr_t)workspace & 255u))
    return fail(PA_EINVAL, "workspace must be 256-byte aligned");
  pa::DecodeParams p{out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     B, Hq, Hkv, D, block_size, NB, scale, (int)kv_dtype, k_scale, v_scale,
                     max_context_len, need > 0 ? workspace : nullptr,
                     (flags & PA_DECODE_SHARED_FRAMES) != 0};
  return hip_status(pa::launch_decode(p, (hipStream_t)stream), "decode launch");
}

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int B, int Hq, int Hkv, int D, int block_size,
                      int64_t NB, float scale, pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale,
                      float v_scale, int max_context_len, unsigned flags, void* stream) {
  // The same checks as pa_decode_ex (a null workspace of size 0 passes them only when the call
  // needs none), then the library's own device scratch instead of a caller's workspace.
  size_t need = 0;
  if (B > 0 && max_context_len > 0 && D > 0 && block_size > 0 && Hq > 0)
    need = pa::decode_workspace_bytes(B, Hq, D, block_size, kv_dtype, max_context_len);
  if (need > pa::kDecodeScratchBytes)
    return fail(PA_ENOSPC, "pa_decode_noalloc: this device needs %zu bytes of scratch, the "
                "library holds %zu per GPU (use pa_decode with a workspace)", need,
                pa::kDecodeScratchBytes);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = pa::decode_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "pa_decode_noalloc scratch address");
  }
  return pa_decode_ex(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, B,
                      Hq, Hkv, D, block_size, NB, scale, q_dtype, kv_dtype, k_scale, v_scale,
                      max_context_len, scratch, need > 0 ? pa::kDecodeScratchBytes : 0, flags,
                      stream);
}

size_t pa_decode_shared_workspace_bytes(int B, int Hq, int D, int block_size, pa_dtype kv_dtype,
                                        int max_context_len) {
  if (B <= 0 || Hq <= 0 || D <= 0 || block_size <= 0 || max_context_len <= 0) return 0;
  return pa::decode_shared_workspace_bytes(D);
}

int pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                     int B, int Hq, int Hkv, int D, int block_size, int64_t NB, float scale,
                     pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                     int max_context_len, const int32_t* shared_blocks, const int32_t* run_size,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || NB < 1 || max_blocks_per_seq < 1)
    return fail(PA_EINVAL, "bad sizes (B %d, NB %lld, max_blocks_per_seq %d)", B, (long long)NB, max_blocks_per_seq);
  if (B > 65535) return fail(PA_ENOTSUP, "batch %d too large for one call (max 65535)", B);
  if (int r = check_heads(Hq, Hkv)) return r;
  if (int r = check_shape(D, block_size, kv_dtype)) return r;
  if (int r = check_attn_dtypes(q_dtype, kv_dtype)) return r;
  if (int r = check_scales(kv_dtype, k_scale, v_scale)) return r;
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale must be finite");
  if (B == 0) return ok();
  if (max_context_len < 1) return fail(PA_EINVAL, "max_context_len %d must be positive", max_context_len);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !shared_blocks || !run_size)
    return fail(PA_EINVAL, "null pointer argument");
  const size_t need = pa::decode_shared_workspace_bytes(D);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ENOSPC, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && ((uintptr_t)workspace & 255u))
    return fail(PA_EINVAL, "workspace must be 256-byte aligned");
  pa::DecodeParams p{out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     B, Hq, Hkv, D, block_size, NB, scale, (int)kv_dtype, k_scale, v_scale,
                     max_context_len, need > 0 ? workspace : nullptr, true, run_size, shared_blocks};
  return hip_status(pa::launch_decode(p, (hipStream_t)stream), "decode_shared launch");
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
              int B, int Hq, int Hkv, int D, int block_size, int64_t NB, float scale,
              pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
              int max_context_len, void* workspace, size_t workspace_bytes, void* stream) {
  return pa_decode_ex(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, B,
                      Hq, Hkv, D, block_size, NB, scale, q_dtype, kv_dtype, k_scale, v_scale,
                      max_context_len, workspace, workspace_bytes, 0u, stream);
}

size_t pa_prefill_chunk_workspace_bytes(int num_chunks, int64_t total_q, int max_chunk_len,
                                        int max_context_len, int Hq, int Hkv, int D,
                                        int block_size, pa_dtype kv_dtype) {
  (void)block_size;
  if (num_chunks <= 0 || total_q <= 0 || max_chunk_len <= 0 || max_context_len <= 0 || Hq <= 0 ||
      Hkv <= 0 || D <= 0 || Hq % Hkv)
    return 0;
  return pa::prefill_workspace_bytes(num_chunks, total_q, max_chunk_len, max_context_len, Hq, Hkv, D, (int)kv_dtype);
}

int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* query_start_loc, const int32_t* context_lens, int num_chunks,
                     int64_t total_q, int max_chunk_len, int max_context_len, int Hq, int Hkv,
                     int D, int block_size, int64_t NB, float scale, pa_dtype q_dtype,
                     pa_dtype kv_dtype, float k_scale, float v_scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (num_chunks < 0 || total_q < 0 || NB < 1 || max_blocks_per_seq < 1)
    return fail(PA_EINVAL, "bad sizes (num_chunks %d, total_q %lld, NB %lld)", num_chunks, (long long)total_q, (long long)NB);
  if (int r = check_heads(Hq, Hkv)) return r;
  if (int r = check_shape(D, block_size, kv_dtype)) return r;
  if (int r = check_attn_dtypes(q_dtype, kv_dtype)) return r;
  if (int r = check_scales(kv_dtype, k_scale, v_scale)) return r;
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale must be finite");
  if (num_chunks == 0 || total_q == 0) return ok();
  if (max_chunk_len < 1 || max_context_len < max_chunk_len)
    return fail(PA_EINVAL, "need 1 <= max_chunk_len (%d) <= max_context_len (%d)", max_chunk_len, max_context_len);
  if (total_q > 0x7fffffff) return fail(PA_ENOTSUP, "total_q %lld too large", (long long)total_q);
  if ((long long)num_chunks * Hkv > 65535) return fail(PA_ENOTSUP, "num_chunks * Hkv too large (max 65535)");
  if (total_q * Hq > 4LL * 0x7fffffff) return fail(PA_ENOTSUP, "total_q * Hq too large");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens)
    return fail(PA_EINVAL, "null pointer argument");
  const size_t need = pa::prefill_workspace_bytes(num_chunks, total_q, max_chunk_len, max_context_len, Hq, Hkv, D, (int)kv_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ENOSPC, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && ((uintptr_t)workspace & 255u))
    return fail(PA_EINVAL, "workspace must be 256-byte aligned");
  pa::PrefillParams p{out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, query_start_loc,
                      context_lens, num_chunks, total_q, max_chunk_len, max_context_len, Hq, Hkv,
                      D, block_size, NB, scale, (int)kv_dtype, k_scale, v_scale,
                      need > 0 ? workspace : nullptr, 0};
  return hip_status(pa::launch_prefill(p, (hipStream_t)stream), "prefill_chunk launch");
}

// Size and shape checks shared by the mixed-batch calls.
static int check_mixed(int num_decodes, int num_chunks, int64_t total_q, int max_chunk_len,
                       int max_context_len, int Hq, int Hkv, int D, int block_size,
                       pa_dtype kv_dtype) {
  if (num_decodes < 0 || num_chunks < 0 || total_q < num_decodes)
    return fail(PA_EINVAL, "bad sizes (num_decodes %d, num_chunks %d, total_q %lld)", num_decodes,
                num_chunks, (long long)total_q);
  if (num_decodes > 65535) return fail(PA_ENOTSUP, "%d decodes too many for one call (max 65535)", num_decodes);
  if (int r = check_heads(Hq, Hkv)) return r;
  if (int r = check_shape(D, block_size, kv_dtype)) return r;
  if (max_context_len < 1) return fail(PA_EINVAL, "max_context_len %d must be positive", max_context_len);
  if (num_chunks > 0 && total_q > num_decodes &&
      (max_chunk_len < 1 || max_context_len < max_chunk_len))
    return fail(PA_EINVAL, "need 1 <= max_chunk_len (%d) <= max_context_len (%d)", max_chunk_len, max_context_len);
  if (total_q > 0x7fffffff) return fail(PA_ENOTSUP, "total_q %lld too large", (long long)total_q);
  if ((long long)num_chunks * Hkv > 65535) return fail(PA_ENOTSUP, "num_chunks * Hkv too large (max 65535)");
  if (total_q * Hq > 4LL * 0x7fffffff) return fail(PA_ENOTSUP, "total_q * Hq too large");
  return PA_OK;
}

static pa::MixedParams mixed_params(int num_decodes, int num_chunks, int64_t total_q,
                                    int max_chunk_len, int max_context_len, int64_t decode_tokens,
                                    int Hq, int Hkv, int D, int block_size, pa_dtype kv_dtype) {
  pa::MixedParams p{};
  p.num_decodes = num_decodes;
  p.num_chunks = num_chunks;
  p.total_q = total_q;
  p.max_chunk_len = max_chunk_len;
  p.max_context_len = max_context_len;
  p.decode_tokens = decode_tokens;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.bs = block_size;
  p.kv_dtype = (int)kv_dtype;
  return p;
}

size_t pa_mixed_workspace_bytes(int num_decodes, int num_chunks, int64_t total_q,
                                int max_chunk_len, int max_context_len, int Hq, int Hkv, int D,
                                int block_size, pa_dtype kv_dtype) {
  if (check_mixed(num_decodes, num_chunks, total_q, max_chunk_len, max_context_len, Hq, Hkv, D,
                  block_size, kv_dtype) != PA_OK)
    return 0;
  return pa::mixed_workspace_bytes(num_decodes, num_chunks, total_q, max_chunk_len,
                                   max_context_len, Hq, Hkv, D, (int)kv_dtype);
}

static int mixed_mode(unsigned flags) {
  return (flags & PA_MIXED_SPLIT) ? pa::MIXED_SPLIT
                                  : ((flags & PA_MIXED_SEPARATE) ? pa::MIXED_SEPARATE : pa::MIXED_AUTO);
}

int pa_mixed_prefill_units(int num_decodes, int num_chunks, int64_t total_q, int max_chunk_len,
                           int max_context_len, int64_t decode_tokens, int Hq, int Hkv, int D,
                           int block_size, pa_dtype kv_dtype, unsigned flags) {
  if (check_mixed(num_decodes, num_chunks, total_q, max_chunk_len, max_context_len, Hq, Hkv, D,
                  block_size, kv_dtype) != PA_OK)
    return -1;
  if ((flags & PA_MIXED_SPLIT) && (flags & PA_MIXED_SEPARATE)) return -1;
  pa::MixedParams p = mixed_params(num_decodes, num_chunks, total_q, max_chunk_len, max_context_len,
                                   decode_tokens, Hq, Hkv, D, block_size, kv_dtype);
  p.mode = mixed_mode(flags);
  return pa::mixed_prefill_workgroups(p);
}

int pa_mixed_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* query_start_loc, const int32_t* context_lens,
                       int num_decodes, int num_chunks, int64_t total_q, int max_chunk_len,
                       int max_context_len, int64_t decode_tokens, int Hq, int Hkv, int D,
                       int block_size, int64_t NB, float scale, pa_dtype q_dtype,
                       pa_dtype kv_dtype, float k_scale, float v_scale, void* workspace,
                       size_t workspace_bytes, unsigned flags, void* stream) {
  if (NB < 1 || max_blocks_per_seq < 1)
    return fail(PA_EINVAL, "bad sizes (NB %lld, max_blocks_per_seq %d)", (long long)NB, max_blocks_per_seq);
  if (int r = check_mixed(num_decodes, num_chunks, total_q, max_chunk_len, max_context_len, Hq,
                          Hkv, D, block_size, kv_dtype))
    return r;
  if (int r = check_attn_dtypes(q_dtype, kv_dtype)) return r;
  if (int r = check_scales(kv_dtype, k_scale, v_scale)) return r;
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale must be finite");
  if (flags & ~(unsigned)(PA_DECODE_SHARED_FRAMES | PA_MIXED_SPLIT | PA_MIXED_SEPARATE))
    return fail(PA_EINVAL, "unknown flags 0x%x", flags);
  if ((flags & PA_MIXED_SPLIT) && (flags & PA_MIXED_SEPARATE))
    return fail(PA_EINVAL, "PA_MIXED_SPLIT and PA_MIXED_SEPARATE exclude each other");
  if (num_decodes == 0 && (num_chunks == 0 || total_q == 0)) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens ||
      (num_chunks > 0 && !query_start_loc))
    return fail(PA_EINVAL, "null pointer argument");
  const size_t need = pa::mixed_workspace_bytes(num_decodes, num_chunks, total_q, max_chunk_len,
                                                max_context_len, Hq, Hkv, D, (int)kv_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ENOSPC, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && ((uintptr_t)workspace & 255u))
    return fail(PA_EINVAL, "workspace must be 256-byte aligned");
  pa::MixedParams p = mixed_params(num_decodes, num_chunks, total_q, max_chunk_len,
                                   max_context_len, decode_tokens, Hq, Hkv, D, block_size, kv_dtype);
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.query_start_loc = query_start_loc;
  p.context_lens = context_lens;
  p.NB = NB;
  p.scale = scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.workspace = need > 0 ? workspace : nullptr;
  p.shared_frames = (flags & PA_DECODE_SHARED_FRAMES) != 0;
  p.mode = mixed_mode(flags);
  return hip_status(pa::launch_mixed(p, (hipStream_t)stream), "mixed_attention launch");
}

// ----------------------------------------------------------------------------- validators

int pa_validate_decode_indices(const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int B, int block_size, int64_t NB,
                               int max_context_len) {
  if (B < 0 || max_blocks_per_seq < 1 || block_size < 1 || NB < 1) return fail(PA_EINVAL, "bad sizes");
  if (B > 0 && (!block_tables || !context_lens)) return fail(PA_EINVAL, "null pointer argument");
  const long long cap = std::min<long long>(max_context_len, (long long)max_blocks_per_seq * block_size);
  for (int b = 0; b < B; ++b) {
    const int L = context_lens[b];
    if (L < 1 || L > cap)
      return fail(PA_ERANGE, "context_lens[%d] = %d outside [1, %lld]", b, L, cap);
    const int nblk = (L + block_size - 1) / block_size;
    for (int i = 0; i < nblk; ++i) {
      const int32_t f = block_tables[(size_t)b * max_blocks_per_seq + i];
      if (f < 0 || f >= NB)
        return fail(PA_ERANGE, "block_tables[%d][%d] = %d outside [0, %lld)", b, i, f, (long long)NB);
    }
  }
  return ok();
}

int pa_validate_slots(const int64_t* slot_mapping, int64_t T, int64_t NB, int block_size) {
  if (T < 0 || NB < 1 || block_size < 1) return fail(PA_EINVAL, "bad sizes");
  if (T > 0 && !slot_mapping) return fail(PA_EINVAL, "null pointer argument");
  const int64_t nslots = NB * block_size;
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)T);
  for (int64_t i = 0; i < T; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;
    if (s >= nslots)
      return fail(PA_ERANGE, "slot_mapping[%lld] = %lld outside [0, %lld)", (long long)i, (long long)s, (long long)nslots);
    if (!seen.insert(s).second)
      return fail(PA_EINVAL, "slot %lld written twice (slot_mapping[%lld])", (long long)s, (long long)i);
  }
  return ok();
}

int pa_validate_copy_pairs(const int64_t* pairs, int64_t N, int64_t NB) {
  if (N < 0 || NB < 1) return fail(PA_EINVAL, "bad sizes");
  if (N > 0 && !pairs) return fail(PA_EINVAL, "null pointer argument");
  std::unordered_set<int64_t> src, dst;
  for (int64_t i = 0; i < N; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= NB || d < 0 || d >= NB)
      return fail(PA_ERANGE, "pair %lld (%lld -> %lld) outside [0, %lld)", (long long)i, (long long)s, (long long)d, (long long)NB);
    src.insert(s);
    if (!dst.insert(d).second) return fail(PA_EINVAL, "destination %lld repeated (pair %lld)", (long long)d, (long long)i);
  }
  for (int64_t d : dst)
    if (src.count(d)) return fail(PA_EINVAL, "frame %lld is both a source and a destination", (long long)d);
  return ok();
}

// Chunk rules for sequences [first, first + n) of a batch whose chunk rows start at row0
// (messages name the batch's own indices).
static int check_chunks(const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* query_start_loc, const int32_t* context_lens, int first,
                        int n, int32_t row0, int block_size, int64_t NB, int max_chunk_len,
                        int max_context_len) {
  if (n > 0 && query_start_loc[first] != row0)
    return fail(PA_EINVAL, "query_start_loc[%d] = %d, must be %d", first, query_start_loc[first], row0);
  const long long cap = std::min<long long>(max_context_len, (long long)max_blocks_per_seq * block_size);
  for (int c = first; c < first + n; ++c) {
    const int C = query_start_loc[c + 1] - query_start_loc[c];
    const int L = context_lens[c];
    if (C < 0) return fail(PA_EINVAL, "query_start_loc decreases at %d", c);
    if (C > max_chunk_len) return fail(PA_ERANGE, "chunk %d has %d rows > max_chunk_len %d", c, C, max_chunk_len);
    if (L < 1 || L > cap) return fail(PA_ERANGE, "context_lens[%d] = %d outside [1, %lld]", c, L, cap);
    if (C > L) return fail(PA_ERANGE, "chunk %d has %d rows but context length %d", c, C, L);
    const int nblk = (L + block_size - 1) / block_size;
    for (int i = 0; i < nblk; ++i) {
      const int32_t f = block_tables[(size_t)c * max_blocks_per_seq + i];
      if (f < 0 || f >= NB)
        return fail(PA_ERANGE, "block_tables[%d][%d] = %d outside [0, %lld)", c, i, f, (long long)NB);
    }
  }
  return ok();
}

int pa_validate_chunk_indices(const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* query_start_loc, const int32_t* context_lens,
                              int num_chunks, int block_size, int64_t NB, int max_chunk_len,
                              int max_context_len) {
  if (num_chunks < 0 || max_blocks_per_seq < 1 || block_size < 1 || NB < 1) return fail(PA_EINVAL, "bad sizes");
  if (num_chunks > 0 && (!block_tables || !query_start_loc || !context_lens))
    return fail(PA_EINVAL, "null pointer argument");
  return check_chunks(block_tables, max_blocks_per_seq, query_start_loc, context_lens, 0,
                      num_chunks, 0, block_size, NB, max_chunk_len, max_context_len);
}

int pa_validate_mixed_indices(const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* query_start_loc, const int32_t* context_lens,
                              int num_decodes, int num_chunks, int block_size, int64_t NB,
                              int max_chunk_len, int max_context_len) {
  if (num_decodes < 0 || num_chunks < 0 || max_blocks_per_seq < 1 || block_size < 1 || NB < 1)
    return fail(PA_EINVAL, "bad sizes");
  if (num_decodes + num_chunks == 0) return PA_OK;  // nothing to check, and nothing is read
  if (!block_tables || !query_start_loc || !context_lens)
    return fail(PA_EINVAL, "null pointer argument");
  for (int b = 0; b <= num_decodes; ++b)
    if (query_start_loc[b] != b)
      return fail(PA_EINVAL, "query_start_loc[%d] = %d, a decode row must be %d", b, query_start_loc[b], b);
  if (int r = pa_validate_decode_indices(block_tables, max_blocks_per_seq, context_lens,
                                         num_decodes, block_size, NB, max_context_len))
    return r;
  return check_chunks(block_tables, max_blocks_per_seq, query_start_loc, context_lens,
                      num_decodes, num_chunks, num_decodes, block_size, NB, max_chunk_len,
                      max_context_len);
}

int pa_find_shared_prefixes(const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens, int B, int block_size, int max_run,
                            int32_t* shared_blocks, int32_t* run_size, int* num_runs) {
  if (B < 0 || max_blocks_per_seq < 1 || block_size < 1 || max_run < 1 ||
      max_run > PA_SHARED_RUN_COLUMNS)
    return fail(PA_EINVAL, "bad sizes (B %d, max_blocks_per_seq %d, block_size %d, max_run %d)",
                B, max_blocks_per_seq, block_size, max_run);
  if (!num_runs || (B > 0 && (!block_tables || !context_lens || !shared_blocks || !run_size)))
    return fail(PA_EINVAL, "null pointer argument");
  // full blocks before the token at position L - 1 (the one a decode step has just written)
  auto full = [&](int b) {
    const int L = context_lens[b];
    return L >= 1 ? std::min((L - 1) / block_size, max_blocks_per_seq) : 0;
  };
  auto row = [&](int b) { return block_tables + (size_t)b * max_blocks_per_seq; };
  int runs = 0;
  for (int b = 0; b < B;) {
    // the longest stretch from b of at most max_run sequences that share at least one full block
    int e = b + 1, P = full(b);
    while (e < B && e - b < max_run && P >= 1) {
      int f = 0;
      const int lim = std::min(P, full(e));
      while (f < lim && row(e)[f] == row(b)[f]) ++f;
      if (f < 1) break;
      P = f;
      ++e;
    }
    if (e - b >= 2 && P >= 1 && row(b)[0] >= 0) {
      for (int m = b; m < e; ++m) {
        shared_blocks[m] = P;
        run_size[m] = m == b ? e - b : 0;
      }
      ++runs;
    } else {
      e = b + 1;
      shared_blocks[b] = 0;
      run_size[b] = 1;
    }
    b = e;
  }
  *num_runs = runs;
  return ok();
}

int pa_validate_shared_prefixes(const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int B, int block_size,
                                const int32_t* shared_blocks, const int32_t* run_size, int G) {
  if (B < 0 || max_blocks_per_seq < 1 || block_size < 1 || G < 1 || G > 16)
    return fail(PA_EINVAL, "bad sizes");
  if (B == 0) return ok();
  if (!block_tables || !context_lens || !shared_blocks || !run_size)
    return fail(PA_EINVAL, "null pointer argument");
  for (int b = 0; b < B;) {
    const int s = run_size[b];
    if (s < 1) return fail(PA_EINVAL, "run_size[%d] = %d: sequence %d starts no run and is in none", b, s, b);
    if (b + s > B) return fail(PA_ERANGE, "run at %d of %d sequences runs past the batch", b, s);
    if ((long long)s * G > PA_SHARED_RUN_COLUMNS)
      return fail(PA_ERANGE, "run at %d has %d sequences: %d x %d query heads exceed %d columns", b,
                  s, s, G, PA_SHARED_RUN_COLUMNS);
    const int P = shared_blocks[b];
    if (s == 1 && P != 0) return fail(PA_EINVAL, "shared_blocks[%d] = %d for a run of one", b, P);
    if (P < 0 || P > max_blocks_per_seq) return fail(PA_ERANGE, "shared_blocks[%d] = %d", b, P);
    for (int m = b; m < b + s; ++m) {
      if (m > b && run_size[m] != 0)
        return fail(PA_EINVAL, "run_size[%d] = %d inside the run that starts at %d", m, run_size[m], b);
      if (shared_blocks[m] != P)
        return fail(PA_EINVAL, "shared_blocks[%d] = %d differs from its run's %d", m, shared_blocks[m], P);
      if ((long long)P * block_size >= context_lens[m])
        return fail(PA_EINVAL, "sequence %d: %d shared blocks leave no frame of its own among its %d tokens", m, P, context_lens[m]);
      for (int f = 0; f < P; ++f)
        if (block_tables[(size_t)m * max_blocks_per_seq + f] != block_tables[(size_t)b * max_blocks_per_seq + f])
          return fail(PA_EINVAL, "block_tables[%d][%d] differs from the shared frame of its run", m, f);
    }
    b += s;
  }
  return ok();
}

}  // extern "C"
