/*
 * pa.h -- paged attention on AMD Instinct MI355X (gfx950): the C ABI of libpa.so.
 *
 * The operations follow the pages that describe PagedAttention:
 *  - "Inside vLLM v0.7: How PagedAttention & Chunked Prefill Scaled 10x Token Serving"
 *    (bicarait.com), "Architectural Blueprint 2" (fixed-size blocks of 16 or 32 tokens,
 *    a block table from logical block index to physical frame, frames shared by
 *    pointer) and "Architectural Blueprint 3" (512-token prefill chunks run in the same
 *    iteration as decodes).
 *  - "Inside vLLM Architecture" (codebumble.net), "Architectural Anatomy" (the kernel
 *    gathers non-contiguous K/V while computing QK^T), "The Block Table Mapping
 *    Subsystem" (a position splits into logical block = pos / block_size and offset =
 *    pos % block_size), "CUDA Shared Memory Optimization" (coalesced per-block fetches,
 *    partial softmax results merged by a final normalised reduction), and its FAQ
 *    (PagedAttention is exact attention; only addressing changes).
 *  - "High-Throughput LLM Serving with vLLM & PagedAttention" (infoisland), section 2
 *    (branches share prompt blocks; copy-on-write when they diverge) and section 4
 *    (an fp8 KV cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every data pointer is a device pointer (memory of the current HIP device)
 *   except in the pa_validate_* functions, which read host memory only.  The caller
 *   owns all memory.  The library allocates nothing and keeps no state besides the
 *   thread-local error message.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   call enqueues its kernels on that stream and returns without synchronising.
 * Errors.  Each call returns PA_OK or a negative status; pa_last_error() then holds a
 *   message.  Scalar arguments (sizes, dtypes, null pointers, workspace size) are always
 *   checked before anything is launched.  The contents of index arrays (block tables,
 *   context lengths, slots, copy pairs) live on the device and are NOT read by the
 *   entry points; check them with the pa_validate_* functions on a host copy.  The
 *   kernels never access memory outside the buffers the arguments describe, even for
 *   invalid indices: a frame id outside [0, NB) is skipped, a context length is clamped
 *   to [0, min(max_context_len, max_blocks_per_seq * block_size)], a slot outside
 *   [0, NB * block_size) is skipped.  Results for such inputs are unspecified.
 * Shapes.  Hq query heads share Hkv KV heads in groups of G = Hq / Hkv: query head h
 *   reads KV head h / G.  Supported: D (head_dim) in {64, 128}, block_size in {16, 32},
 *   G in {1, 2, 4, 8, 16}, and (q, kv, out) dtypes (f32, f32, f32), (bf16, bf16, bf16),
 *   (bf16, fp8, bf16); an f32 cache with D = 128 and block_size = 32 is not supported.
 *   Accumulation is fp32; outputs are rounded to nearest even.
 *
 * KV cache layout
 * ---------------
 * k_cache and v_cache each hold NB frames; frame f holds Hkv tiles, the tile of KV head
 * g starting at element (f * Hkv + g) * block_size * D.  A tile holds the block_size
 * tokens of the frame for one head; token slot o (0 <= o < block_size) of frame f is
 * slot number f * block_size + o.  Inside a tile, with b = bytes per element, the
 * value of slot o and head-dim index d sits at byte
 *   K:  h = o / 16, kl = o % 16, j = d / (D/4), t = d % (D/4)
 *       byte = 1024 * (h * (D*b/64) + (t*b) / 16) + 16 * (16*j + kl) + (t*b) % 16
 *   V:  h = o / 16, j = (o % 16) / 4, i = o % 4, c = d / 16, dl = d % 16,
 *       u = h * (D/16) + c, Q = 4 / b
 *       byte = 1024 * (u / Q) + 16 * (16*j + dl) + (4 * (u % Q) + i) * b
 * i.e. a tile is a sequence of 1 KiB pieces, each 64 lanes x 16 bytes, and each lane's
 * 16 bytes are exactly what one lane of a 64-wide wavefront feeds a matrix-core
 * instruction: every gather of a tile is a run of fully contiguous 1 KiB loads.
 * fp8 values are OCP e4m3fn codes; a stored code c means value(c) * scale with the
 * per-tensor k_scale (v_scale) of the cache.  Write the caches only through
 * pa_reshape_and_cache (and copy frames with pa_copy_blocks).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

enum {
  PA_OK = 0,
  PA_EINVAL = -1,  /* null pointer, bad size, or an index array that fails validation */
  PA_ERANGE = -2,  /* a value outside its allowed range (validators) */
  PA_ENOTSUP = -3, /* a shape or dtype combination the library does not implement */
  PA_EHIP = -4,    /* a HIP runtime call or kernel launch failed */
  PA_ENOSPC = -5   /* the workspace is smaller than the *_workspace_bytes result */
};

/* Score columns of one run of pa_decode_shared: a run of s sequences needs s * G of them
 * (G = Hq / Hkv query heads per KV head). */
#define PA_SHARED_RUN_COLUMNS 16

/* Message describing the last failure on the calling thread ("" after success). */
const char* pa_last_error(void);

/* Library version and the GPU architecture its kernels are built for. */
const char* pa_build_info(void);

/*
 * pa_reshape_and_cache -- store this step's new K and V rows in their cache slots.
 * Defined by the block-table mapping (codebumble.net, "The Block Table Mapping
 * Subsystem"): token i goes to frame slot_mapping[i] / block_size at offset
 * slot_mapping[i] % block_size, for every KV head.
 *   k, v          [T, Hkv, D] rows in src_dtype (f32 or bf16), contiguous, 16-byte aligned
 *                 (as are the caches; PA_EINVAL otherwise).
 *   k_cache, v_cache  caches in kv_dtype, layout above, written in place.
 *   slot_mapping  int64 [T]; a negative slot skips the token (padding).  Two tokens must
 *                 not name the same slot in one call (the later write is unspecified).
 *   kv_dtype      f32 from f32 and bf16 from bf16 store the bits unchanged; fp8 from
 *                 bf16 stores e4m3fn(RNE, saturating to +-448)(fp32(x) / scale), with
 *                 scale = k_scale for K and v_scale for V (NaN stays NaN).
 */
int pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t T, int64_t NB, int Hkv, int D,
                         int block_size, pa_dtype src_dtype, pa_dtype kv_dtype, float k_scale,
                         float v_scale, void* stream);

/*
 * pa_copy_blocks -- copy-on-write support (infoisland, section 2): for every pair
 * (src, dst) of `pairs` (int64 [N][2]) frame dst of both caches becomes a bit copy of
 * frame src (all Hkv tiles).  Destinations must be distinct and none may be a source;
 * the copies then do not depend on their order.  A pair with an index outside [0, NB)
 * is skipped.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int64_t N, int64_t NB,
                   int Hkv, int D, int block_size, pa_dtype kv_dtype, void* stream);

/*
 * Bytes of device workspace pa_decode needs (0 only for invalid arguments).  The size follows
 * head_dim and the device's compute-unit count, not the batch: it holds the plan of the launch
 * and two partial-result slots per persistent wavefront.  max_context_len bounds every
 * context_lens entry.
 */
size_t pa_decode_workspace_bytes(int B, int Hq, int D, int block_size, pa_dtype kv_dtype,
                                 int max_context_len);

/*
 * pa_decode -- one decode step of paged attention (codebumble.net, "Architectural
 * Anatomy" and FAQ; bicarait.com, "Architectural Blueprint 2"):
 *   out[b, h, :] = sum_t softmax_t(scale * q[b, h, :] . K_b[t, h/G, :]) V_b[t, h/G, :]
 * over t < context_lens[b], where K_b[t] and V_b[t] are read from frame
 * block_tables[b, t / block_size], slot t % block_size, dequantised for fp8.
 *   out, q        [B, Hq, D] in q_dtype (out has the q dtype), contiguous.
 *   block_tables  int32 [B, max_blocks_per_seq]; entries past ceil(L/block_size) unused.
 *   context_lens  int32 [B], each in [1, max_context_len]; the count includes the token
 *                 written this step (write it with pa_reshape_and_cache first, on the
 *                 same stream).
 *   max_context_len  host-side bound on the lengths.
 *   workspace     device scratch of at least pa_decode_workspace_bytes(...) bytes, 256-byte
 *                 aligned (hipMalloc'd memory is).  Nothing in it is read before this call
 *                 writes it; concurrent calls must not share one.
 * The batch's (sequence, kv head, frame) work is split into equal contiguous ranges over a
 * set of persistent wavefronts (three per compute unit, fewer when the host-known bound
 * B Hkv ceil(max_context_len / block_size) leaves too little work for them, so the launch
 * depends on B, Hkv, block_size and max_context_len only); a sequence cut by a range boundary
 * is merged from partial results by a second (reduce) kernel, exactly up to fp32 rounding
 * ("CUDA Shared Memory Optimization": a final normalised reduction).  The merge order is fixed,
 * so equal inputs give equal output bits.  A small batch -- ceil(max_context_len / block_size)
 * at most 28 and B Hkv at most the wavefront count above -- launches one wavefront per
 * (sequence, kv head) instead, each writing its output directly, and no reduce kernel.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
              int B, int Hq, int Hkv, int D, int block_size, int64_t NB, float scale,
              pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
              int max_context_len, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_ex -- pa_decode with flags (pa_decode is pa_decode_ex with flags 0):
 *   PA_DECODE_SHARED_FRAMES  some frames appear in the block tables of several sequences of
 *     the batch (copy-on-write branches of one prompt, cached prefixes; bicarait.com,
 *     "Architectural Blueprint 2"; infoisland, section 2).  K/V tiles are then read with loads
 *     that keep them in the caches, so the sequences after the first find shared frames there;
 *     without the flag tiles are read once each and bypass cache retention.  The flag changes
 *     only where data is cached: results are bit-identical either way.
 * Unknown flag bits are PA_EINVAL.
 */
enum { PA_DECODE_SHARED_FRAMES = 1 };
int pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                 int B, int Hq, int Hkv, int D, int block_size, int64_t NB, float scale,
                 pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                 int max_context_len, void* workspace, size_t workspace_bytes, unsigned flags,
                 void* stream);

/*
 * pa_decode_noalloc -- pa_decode_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It allocates nothing: the decode's plan and partial results go to a
 * scratch array of 16 MiB that the library holds on every GPU it runs on, from the first call
 * on that GPU until the process ends.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (on different streams, or from different threads without
 * ordering) race and must not be issued; calls ordered on one stream are fine.  The array keeps
 * the last call's contents; nothing in it is read before the call writes it.  Arguments,
 * results (bit-identical to pa_decode_ex with the same arguments) and errors are pa_decode_ex's;
 * PA_ENOSPC when this device's launch would need more scratch than the array holds
 * (pa_decode_workspace_bytes above 16 MiB, i.e. more than ~320 compute units at head_dim 128).
 */
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int B, int Hq, int Hkv, int D, int block_size,
                      int64_t NB, float scale, pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale,
                      float v_scale, int max_context_len, unsigned flags, void* stream);

/*
 * pa_decode_shared -- pa_decode for a batch in which runs of consecutive sequences share the
 * first frames of their block tables: the branches of one prompt in parallel sampling or beam
 * search, which reference the prompt's frames instead of copying them (bicarait.com,
 * "Architectural Blueprint 2" and "Physical Memory Sharing"; infoisland, section 2).  The result
 * is pa_decode's (to fp32 rounding); the shared frames are read once per run instead of once per
 * sequence.  A run's members put their G query heads side by side in the PA_SHARED_RUN_COLUMNS
 * (16) columns of the matrix-core score tile (at G = 8 a plain decode leaves half of them
 * empty): the run streams the shared frames once for all members, then each member's own frames
 * with the other members' columns masked, with one online softmax per column.
 *   Arguments shared with pa_decode have its meaning, except the workspace: at least
 *   pa_decode_shared_workspace_bytes(...) bytes (the launch runs more wavefronts than
 *   pa_decode's), 256-byte aligned.
 *   run_size       int32 [B], device: run_size[b] = s >= 1 starts a run of the sequences
 *                  [b, b + s); 0 marks a sequence inside a run.  Every sequence is in one run;
 *                  s * G <= PA_SHARED_RUN_COLUMNS (G = Hq / Hkv).
 *   shared_blocks  int32 [B], device: the block-table entries the members of b's run share (the
 *                  same for all members; 0 for a run of one).  The members' first
 *                  shared_blocks[b] entries are equal, and shared_blocks[b] * block_size <
 *                  context_lens[b] (the frame of the token written this step is never shared).
 * Runs of one sequence with no shared block make this pa_decode_ex with PA_DECODE_SHARED_FRAMES.
 * The run arrays are trusted on the device (invalid ones give unspecified results, never an
 * access outside the buffers); check them with pa_validate_shared_prefixes on host copies.
 */
size_t pa_decode_shared_workspace_bytes(int B, int Hq, int D, int block_size, pa_dtype kv_dtype,
                                        int max_context_len);
int pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                     int B, int Hq, int Hkv, int D, int block_size, int64_t NB, float scale,
                     pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                     int max_context_len, const int32_t* shared_blocks, const int32_t* run_size,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_find_shared_prefixes -- host-only: runs for pa_decode_shared, found in host copies of a
 * batch's block tables and context lengths.  From each sequence on, the longest stretch of at most
 * max_run (1 .. PA_SHARED_RUN_COLUMNS; PA_SHARED_RUN_COLUMNS / G for pa_decode_shared)
 * consecutive sequences whose tables agree on at
 * least their first entry becomes a run; its shared blocks are the leading entries all members
 * agree on, limited to the blocks before each member's last token.  Sequences that join no such
 * stretch are runs of one.  Outputs: shared_blocks and run_size (int32 [B] each), and
 * *num_runs, the runs of two or more.  A block manager knows the same from its reference counts;
 * this scan is for callers without one.
 */
int pa_find_shared_prefixes(const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens, int B, int block_size, int max_run,
                            int32_t* shared_blocks, int32_t* run_size, int* num_runs);

/* Bytes of device workspace pa_prefill_chunk needs for these bounds (0 is a valid answer:
 * then workspace may be NULL).  The arguments are the ones pa_prefill_chunk receives. */
size_t pa_prefill_chunk_workspace_bytes(int num_chunks, int64_t total_q, int max_chunk_len,
                                        int max_context_len, int Hq, int Hkv, int D,
                                        int block_size, pa_dtype kv_dtype);

/*
 * pa_prefill_chunk -- causal attention of prefill chunks over their paged context
 * (bicarait.com, "Architectural Blueprint 3"; infoisland, section 5).  Chunk c owns the
 * query rows r in [query_start_loc[c], query_start_loc[c+1]) (C_c rows); its sequence has
 * L_c = context_lens[c] tokens including the chunk, so row i of the chunk sits at
 * position L_c - C_c + i and attends keys 0 .. L_c - C_c + i (inclusive) through
 * block_tables[c]:
 *   out[r, h, :] = sum_{t <= pos} softmax_t(scale * q[r, h, :] . K[t, h/G, :]) V[t, h/G, :].
 *   out, q           [total_q, Hq, D] in q_dtype, contiguous; total_q = query_start_loc[num_chunks].
 *   query_start_loc  int32 [num_chunks + 1], non-decreasing, starting at 0.
 *   context_lens     int32 [num_chunks], C_c <= L_c <= max_context_len.
 *   max_chunk_len    host-side bound on C_c; sizes the grid together with max_context_len.
 *   workspace        at least pa_prefill_chunk_workspace_bytes(...) bytes, 256-byte aligned.
 * The chunk's own K/V must already be in the cache (pa_reshape_and_cache on the same
 * stream).
 */
int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* query_start_loc, const int32_t* context_lens, int num_chunks,
                     int64_t total_q, int max_chunk_len, int max_context_len, int Hq, int Hkv,
                     int D, int block_size, int64_t NB, float scale, pa_dtype q_dtype,
                     pa_dtype kv_dtype, float k_scale, float v_scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace pa_mixed_attention needs for these bounds (0 is a valid answer:
 * then workspace may be NULL).  It holds the decode plan and partials (sized, as for
 * pa_decode, by the device's compute units) and the chunk rows' split partials.
 */
size_t pa_mixed_workspace_bytes(int num_decodes, int num_chunks, int64_t total_q,
                                int max_chunk_len, int max_context_len, int Hq, int Hkv, int D,
                                int block_size, pa_dtype kv_dtype);

/*
 * pa_mixed_attention -- one step of a mixed batch in one attention kernel: prefill chunks
 * paired with the ongoing decodes in the same GPU iteration (bicarait.com, "Architectural
 * Blueprint 3"; infoisland, section 5).  The batch has num_decodes + num_chunks sequences,
 * decodes first:
 *   sequence b < num_decodes      a decode: query row b (query_start_loc[b] = b); out[b] is
 *                                 pa_decode's result for q[b], block_tables[b], context_lens[b].
 *   sequence s = num_decodes + c  chunk c: rows [query_start_loc[s], query_start_loc[s+1]);
 *                                 out rows are pa_prefill_chunk's result for that chunk.
 *   out, q           [total_q, Hq, D] in q_dtype, contiguous;
 *                    total_q = query_start_loc[num_decodes + num_chunks].
 *   block_tables     int32 [num_decodes + num_chunks, max_blocks_per_seq].
 *   query_start_loc  int32 [num_decodes + num_chunks + 1], query_start_loc[b] = b for
 *                    b <= num_decodes, non-decreasing after.
 *   context_lens     int32 [num_decodes + num_chunks], each in [1, max_context_len]; a
 *                    chunk's length is at least its row count.
 *   max_chunk_len    host-side bound on the chunks' row counts (ignored when num_chunks = 0).
 *   decode_tokens    the sum of the decodes' context lengths as the host knows it (a block
 *                    manager does), or <= 0 if unknown.  It only decides how many compute
 *                    units take each half; the results do not depend on it.
 *   flags            PA_DECODE_SHARED_FRAMES as for pa_decode_ex (decode loads only);
 *                    PA_MIXED_SPLIT or PA_MIXED_SEPARATE force the mode (below) instead of
 *                    the host's choice (for tuning and tests; results agree either way).
 *   workspace        at least pa_mixed_workspace_bytes(...) bytes, 256-byte aligned;
 *                    concurrent calls must not share one.
 * Every K/V the step attends (the chunks' own rows and the decodes' new tokens) must already be
 * in the cache (pa_reshape_and_cache on the same stream).  Outputs match pa_decode and
 * pa_prefill_chunk to fp32 rounding (the context splits differ); equal inputs and decode_tokens
 * give equal output bits.  Argument errors are those of the two calls.  The kernels read
 * query_start_loc only for the chunks; pa_validate_mixed_indices checks the whole batch on the
 * host.
 * Modes, picked on the host from the sizes and decode_tokens:
 *   split     one persistent attention kernel with one workgroup per compute unit: some run
 *             prefill tiles while the others stream the decodes, so the matrix cores and HBM
 *             work at once; then one kernel merges the split partials of both halves (above
 *             1024 decodes a one-workgroup plan kernel runs first).
 *   separate  the pa_prefill_chunk kernels on the chunks, then the pa_decode kernels.
 * The split is taken when the decodes' bytes are small next to the chunks' matrix work, where it
 * is predicted to be faster.
 */
enum { PA_MIXED_SPLIT = 2, PA_MIXED_SEPARATE = 4 };
int pa_mixed_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* query_start_loc, const int32_t* context_lens,
                       int num_decodes, int num_chunks, int64_t total_q, int max_chunk_len,
                       int max_context_len, int64_t decode_tokens, int Hq, int Hkv, int D,
                       int block_size, int64_t NB, float scale, pa_dtype q_dtype,
                       pa_dtype kv_dtype, float k_scale, float v_scale, void* workspace,
                       size_t workspace_bytes, unsigned flags, void* stream);

/*
 * How a pa_mixed_attention call with these arguments (and flags) uses the device: the number of
 * workgroups (one per compute unit) that run prefill tiles while the others stream the decodes
 * from the start (split mode).  The device's compute-unit count means the separate mode (or
 * chunks only), 0 means decodes only.  -1 on invalid arguments.
 */
int pa_mixed_prefill_units(int num_decodes, int num_chunks, int64_t total_q, int max_chunk_len,
                           int max_context_len, int64_t decode_tokens, int Hq, int Hkv, int D,
                           int block_size, pa_dtype kv_dtype, unsigned flags);

/*
 * Host-side validators (no GPU needed).  Each returns PA_OK or PA_EINVAL/PA_ERANGE with
 * pa_last_error() naming the first offending entry.
 *  pa_validate_decode_indices: 1 <= context_lens[b] <= min(max_context_len,
 *    max_blocks_per_seq * block_size) and 0 <= block_tables[b, i] < NB for every
 *    i < ceil(context_lens[b] / block_size).
 *  pa_validate_slots: every slot is negative (skip) or in [0, NB * block_size), and no
 *    non-negative slot repeats.
 *  pa_validate_copy_pairs: every index in [0, NB), destinations distinct, no destination
 *    is also a source.
 *  pa_validate_chunk_indices: query_start_loc starts at 0 and does not decrease, every
 *    chunk length is at most max_chunk_len and at most its context length, context
 *    lengths are in [1, max_context_len], and the table entries the context covers are
 *    in [0, NB).
 *  pa_validate_mixed_indices: the decode rules for sequences [0, num_decodes), with
 *    query_start_loc[b] = b for b <= num_decodes, and the chunk rules (query rows counted
 *    from query_start_loc[num_decodes]) for the num_chunks sequences after them.
 */
int pa_validate_decode_indices(const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int B, int block_size, int64_t NB,
                               int max_context_len);
int pa_validate_slots(const int64_t* slot_mapping, int64_t T, int64_t NB, int block_size);
int pa_validate_copy_pairs(const int64_t* pairs, int64_t N, int64_t NB);
int pa_validate_chunk_indices(const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* query_start_loc, const int32_t* context_lens,
                              int num_chunks, int block_size, int64_t NB, int max_chunk_len,
                              int max_context_len);
int pa_validate_mixed_indices(const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* query_start_loc, const int32_t* context_lens,
                              int num_decodes, int num_chunks, int block_size, int64_t NB,
                              int max_chunk_len, int max_context_len);
/*  pa_validate_shared_prefixes: run_size and shared_blocks cut the batch into runs as
 *    pa_decode_shared requires (every sequence in one run of at most PA_SHARED_RUN_COLUMNS / G
 *    sequences, equal
 *    shared blocks within a run, 0 for runs of one, equal shared table entries, context lengths
 *    above the shared blocks' tokens). */
int pa_validate_shared_prefixes(const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int B, int block_size,
                                const int32_t* shared_blocks, const int32_t* run_size, int G);

/*
 * Host-side block manager (no GPU involved): the bookkeeping that produces the block tables,
 * slot mappings and copy-on-write pairs the calls above consume.  It follows
 * codebumble.net, "The Block Table Mapping Subsystem" (a global free list; a position splits
 * into logical block = pos / block_size and offset = pos % block_size; a frame is taken from
 * the free list when a token starts a block), bicarait.com, "Architectural Blueprint 2" and
 * infoisland, section 2 (branches of one prompt reference the same frames; a frame is copied
 * only when a branch writes into it while others still reference it).
 *   Frames: 0 .. num_frames-1, initially all free in increasing order; allocation takes the
 *     head of the free list, a frame whose last reference is dropped goes to its tail.
 *   Sequences are named by caller-chosen int64 ids.  A handle is not thread safe: callers
 *     serialise calls on one handle.  Every mutating call either succeeds completely or
 *     changes nothing (PA_ENOSPC when the free list is too short, PA_EINVAL for unknown or
 *     duplicate ids).
 */
typedef struct pa_block_manager pa_block_manager;

/* Create a manager of num_frames frames of block_size tokens; *out receives the handle. */
int pa_bm_create(int64_t num_frames, int block_size, pa_block_manager** out);
/* Destroy a handle (NULL is allowed). */
void pa_bm_destroy(pa_block_manager* bm);

/*
 * Append one token to each listed sequence, in list order (an id listed k times gets k
 * tokens; an unknown id starts a new sequence).  slots[i] (int64 [n]) receives the cache slot
 * frame * block_size + offset of entry i's token.  When a token goes into a frame other
 * sequences still reference, the writer first moves to a fresh frame: the pair (old, new) is
 * appended to copy_pairs (int64 [n][2], room for n pairs) and *num_copies counts them.  Apply
 * the copies (pa_copy_blocks) before writing the tokens (pa_reshape_and_cache).
 */
int pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, int64_t n, int64_t* slots,
                 int64_t* copy_pairs, int64_t* num_copies);
/*
 * Prefix caching (codebumble.net, "CUDA Shared Memory Optimization": a prefix tree of token
 * blocks lets a prompt reuse the blocks an earlier prompt computed).  Start sequence `seq` (a new
 * id) with the n prompt tokens `tokens` (int32 ids).  The prompt's leading full blocks that match
 * a registered block chain -- same token ids, block by block, from the first block on -- are
 * referenced instead of allocated; *num_cached receives their token count (a multiple of
 * block_size: their K/V are already in the cache and need no prefill).  The other blocks are
 * allocated; the full ones are registered for later prompts.  slots (int64 [n]) receives every
 * token's slot.  A registered frame that is released stays matchable while it waits in the
 * free list and is dropped from the tree when allocation reuses it.
 */
int pa_bm_append_prompt(pa_block_manager* bm, int64_t seq, const int32_t* tokens, int64_t n,
                        int64_t* slots, int64_t* num_cached);
/* The child (a new id) references every frame of the parent and has its length. */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
/* Drop a sequence; frames no other sequence references return to the free list. */
int pa_bm_free(pa_block_manager* bm, int64_t seq);
/* Queries: free frames, a sequence's token count, a frame's reference count, and the free
 * list in allocation order (capacity entries of room; *count receives the length). */
int pa_bm_num_free(const pa_block_manager* bm, int64_t* out);
int pa_bm_seq_len(const pa_block_manager* bm, int64_t seq, int64_t* out);
int pa_bm_ref_count(const pa_block_manager* bm, int64_t frame, int32_t* out);
int pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int64_t capacity, int64_t* count);
/*
 * Block tables and context lengths of n sequences for pa_decode / pa_prefill_chunk:
 * tables (int32 [n][max_blocks_per_seq], entries past a sequence's blocks are -1) and
 * context_lens (int32 [n], tokens written so far).  PA_ERANGE if a sequence has more blocks.
 */
int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int64_t n,
                       int32_t* tables, int max_blocks_per_seq, int32_t* context_lens);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
