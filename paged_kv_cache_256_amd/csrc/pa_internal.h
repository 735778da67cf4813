// pa_internal.h -- host-side launchers behind the C ABI (no validation here; pa_api.cpp checks
// every scalar argument before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum DType { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int B, Hq, Hkv, D, bs;
  int64_t NB;
  float scale;
  int kv_dtype;  // DType; q/out are f32 for an f32 cache, bf16 otherwise
  float k_scale, v_scale;
  int max_context_len;
  void* workspace;
  bool shared_frames;  // frames referenced by several sequences: keep them cacheable
  // runs of consecutive sequences that share their first block-table entries (pa_decode_shared;
  // null for pa_decode): run_size[b] >= 1 starts a run of run_size[b] sequences, 0 marks a
  // sequence inside one; shared_blocks[b] is the shared entries of b's run
  const int32_t* run_size = nullptr;
  const int32_t* shared_blocks = nullptr;
};

struct PrefillParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int num_chunks;
  int64_t total_q;
  int max_chunk_len, max_context_len;
  int Hq, Hkv, D, bs;
  int64_t NB;
  float scale;
  int kv_dtype;
  float k_scale, v_scale;
  void* workspace;
  int64_t row_base;  // rows [0, row_base) of q / out belong to others; partials start there
};

// A mixed batch: sequences [0, num_decodes) are decodes (one query row each, row b), sequences
// [num_decodes, num_decodes + num_chunks) are prefill chunks; block_tables, query_start_loc and
// context_lens cover the whole batch.
struct MixedParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int num_decodes, num_chunks;
  int64_t total_q;
  int max_chunk_len, max_context_len;
  int64_t decode_tokens;  // sum of the decodes' context lengths (<= 0: unknown)
  int Hq, Hkv, D, bs;
  int64_t NB;
  float scale;
  int kv_dtype;
  float k_scale, v_scale;
  void* workspace;
  bool shared_frames;
  int mode;  // MixedMode
};

enum MixedMode { MIXED_AUTO = 0, MIXED_SPLIT = 1, MIXED_SEPARATE = 2 };

// The calling thread's error message (pa_last_error): set_error formats it and returns `code`,
// clear_error empties it and returns PA_OK.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int set_error_v(int code, const char* fmt, va_list ap);
int clear_error();

// Compute units of the current device (cached per device; 256 when no device is visible).
int device_compute_units();

size_t decode_workspace_bytes(int B, int Hq, int D, int bs, int kv_dtype, int max_context_len);
// Score columns of one run of sequences that share frames (one matrix-core tile).
constexpr int kSharedRunColumns = 16;
// Workspace of a decode over runs of sequences that share frames (more wavefronts per CU).
size_t decode_shared_workspace_bytes(int D);
// The allocation-free decode's device scratch: kDecodeScratchBytes per GPU, in a file-scope
// device array; decode_scratch() returns the current device's copy (its address is looked up
// on the first call per device).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
hipError_t decode_scratch(void** out);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// The decode plan (wavefront starts) of W wavefronts, computed by one workgroup.
hipError_t launch_decode_plan(const int32_t* context_lens, int32_t* plan, int B, int Hkv, int bs,
                              int cap, int W, hipStream_t stream);

size_t prefill_workspace_bytes(int num_chunks, int64_t total_q, int max_chunk_len,
                               int max_context_len, int Hq, int Hkv, int D, int kv_dtype);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

size_t mixed_workspace_bytes(int num_decodes, int num_chunks, int64_t total_q, int max_chunk_len,
                             int max_context_len, int Hq, int Hkv, int D, int kv_dtype);
// Workgroups a mixed launch gives to prefill tiles (the rest run the decode stream).
int mixed_prefill_workgroups(const MixedParams& p);
hipError_t launch_mixed(const MixedParams& p, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slots, int64_t T, int64_t NB, int Hkv, int D,
                                    int bs, int src_dtype, int kv_dtype, float k_scale,
                                    float v_scale, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int64_t N,
                              int64_t NB, int64_t frame_bytes, hipStream_t stream);

}  // namespace pa
