// pa_prefill.hip -- causal attention of prefill chunks over their paged context (gfx950).
//
// What is computed (bicarait.com, "Architectural Blueprint 3"; infoisland, section 5): a long
// prompt is processed in chunks (512 tokens in the pages' example) that run in the same step
// as decodes.  Row i of a chunk of C rows in a sequence of L tokens sits at position
// L - C + i and attends keys 0 .. L - C + i through the sequence's block table.
//
// The work is a dense contraction, so it runs on the matrix cores:
//  * A workgroup (8 wavefronts, one workgroup per compute unit) owns TQ chunk rows x the G
//    heads of one kv head: each wavefront holds NT tiles of 16 query rows (row = token x head,
//    so GQA heads of one token share every K/V fragment) as the columns of S^T = K Q^T.
//  * K/V tiles are staged through a ring of four LDS buffers, 64 keys per stage (32 for f32):
//    each wavefront copies its share of a later stage straight from global memory into LDS with
//    LDS-DMA loads while the wavefronts compute, and every wavefront then reads the same tile
//    from LDS, so one fetch from L2/HBM serves 8 x NT x 16 query rows.  One meeting point per
//    stage; the copies of the next two stages stay in flight across it.  The block ids come in
//    windows of 64 frames (one vector load, a window ahead) and are turned into tile indices once
//    per window, so issuing a stage's copies costs a few scalar instructions per block and never
//    waits for memory.  fp8 stages are widened to bf16 once, in LDS, by the whole workgroup.
//  * Online softmax per query row (causal mask on the diagonal stages), O^T += V^T P^T with
//    16x16x32 products over pairs of 16-key groups; each pair also issues its part of the next
//    stage's score MFMAs, so the matrix cores work beside the exponentials.
//  * Tiles that read the same key range are dealt to one XCD, so the range is read into one L2.
//  * The context is split into KS-key ranges across workgroups so that a single chunk fills
//    the GPU; rows covered by one range are written directly, the others as unnormalised
//    partials merged by prefill_reduce_kernel (log-sum-exp rule).

#include "pa_prefill_impl.h"

namespace pa {

using namespace pre;

namespace {

constexpr int kXcds = 8;  // accelerator complex dies of an MI355X

template <int KIND, int D, int BS, int NT>
__global__ __launch_bounds__(kPWaves * 64, 1) void prefill_chunk_kernel(
    void* __restrict__ out, const void* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, int mbps, int Hq, int Hkv, int G,
    long long NB, long long total_q, long long row_base, int nsplit, int nq, int nz, int KS,
    int max_ctx, float qk_scale, float v_scale) {
  constexpr int S = prefill_stage_bytes<KIND, D, BS>();
  constexpr int SW = prefill_widened_bytes<KIND, D, BS>();
  __shared__ __attribute__((aligned(1024))) char ring0[S], ring1[S], ring2[S], ring3[S];
  __shared__ __attribute__((aligned(1024))) char wide0[SW], wide1[SW];
  // One workgroup per (key range x, query tile y, chunk and kv head z).  Workgroups reach the
  // 8 XCDs round-robin by id; when the (x, z) groups -- tiles that read the same keys -- come in
  // multiples of 8, every tile of a group is dealt to one XCD, so its keys are read into one L2.
  const int id = blockIdx.x, groups = nsplit * nz;
  int x, y, z;
  if (groups % kXcds == 0) {
    const int k = id % kXcds, slot = id / kXcds;
    const int grp = k + kXcds * (slot / nq);
    y = slot % nq;
    x = grp % nsplit;
    z = grp / nsplit;
  } else {
    x = id % nsplit;
    y = (id / nsplit) % nq;
    z = id / (nsplit * nq);
  }
  prefill_tile<KIND, D, BS, NT>(ring0, ring1, ring2, ring3, wide0, wide1, x, y, z / Hkv, z % Hkv,
                                row_base, out, q, k_cache, v_cache, block_tables, qsl, context_lens,
                                ws_ml, ws_o, mbps, Hq, Hkv, G, NB, total_q, nsplit, KS, max_ctx,
                                qk_scale, v_scale);
}

template <int KIND, int D>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens, int num_chunks,
    long long total_q, long long row_base, int Hq, int nsplit, int KS, int cap, float v_scale) {
  prefill_reduce_wave<KIND, D>((long long)blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63,
                               row_base, out, ws_ml, ws_o, qsl, context_lens, num_chunks, total_q, Hq,
                               nsplit, KS, cap, v_scale);
}

template <int KIND, int D, int BS>
hipError_t launch_prefill_typed(const PrefillParams& p, hipStream_t stream) {
  constexpr int NT = tiles_per_wave(KIND);
  const Split sp = choose_split(p.num_chunks, p.max_chunk_len, p.max_context_len, p.Hq, p.Hkv, KIND,
                                device_compute_units());
  const int G = p.Hq / p.Hkv;
  const int TQ = kPWaves * NT * 16 / G;
  float* ws_ml = (float*)p.workspace;
  const long long rows = p.total_q - p.row_base;  // rows of the chunks
  float* ws_o = ws_ml ? ws_ml + partial_ml_floats(rows * p.Hq, sp.nsplit) : nullptr;
  const float qk_scale = p.scale * (KIND == KFP8 ? p.k_scale : 1.0f) * kLog2e;
  const float v_scale = KIND == KFP8 ? p.v_scale : 1.0f;
  const int nq = (p.max_chunk_len + TQ - 1) / TQ, nz = p.num_chunks * p.Hkv;
  const long long nwg = (long long)sp.nsplit * nq * nz;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_chunk_kernel<KIND, D, BS, NT>), dim3((unsigned)nwg), dim3(kPWaves * 64), 0,
                     stream, p.out, p.q, (const char*)p.k_cache, (const char*)p.v_cache,
                     p.block_tables, p.query_start_loc, p.context_lens, ws_ml, ws_o,
                     p.max_blocks_per_seq, p.Hq, p.Hkv, G, (long long)p.NB,
                     (long long)p.total_q, (long long)p.row_base, sp.nsplit, nq, nz, sp.KS,
                     p.max_context_len, qk_scale, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.nsplit <= 1) return e;
  const int cap = p.max_context_len < p.max_blocks_per_seq * BS ? p.max_context_len
                                                                 : p.max_blocks_per_seq * BS;
  const long long pairs = rows * p.Hq;
  hipLaunchKernelGGL((prefill_reduce_kernel<KIND, D>), dim3((unsigned)((pairs + 7) / 8)), dim3(256), 0,
                     stream, p.out, ws_ml, ws_o, p.query_start_loc, p.context_lens, p.num_chunks,
                     (long long)p.total_q, (long long)p.row_base, p.Hq, sp.nsplit, sp.KS, cap,
                     v_scale);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_prefill_kind(const PrefillParams& p, hipStream_t s) {
  if (p.D == 64 && p.bs == 16) return launch_prefill_typed<KIND, 64, 16>(p, s);
  if (p.D == 64 && p.bs == 32) return launch_prefill_typed<KIND, 64, 32>(p, s);
  if (p.D == 128 && p.bs == 16) return launch_prefill_typed<KIND, 128, 16>(p, s);
  if constexpr (KIND != KF32) {
    if (p.D == 128 && p.bs == 32) return launch_prefill_typed<KIND, 128, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_workspace_bytes(int num_chunks, int64_t total_q, int max_chunk_len,
                               int max_context_len, int Hq, int Hkv, int D, int kv_dtype) {
  const int kind = kv_dtype == DT_F32 ? KF32 : (kv_dtype == DT_BF16 ? KBF16 : KFP8);
  const Split sp = choose_split(num_chunks, max_chunk_len, max_context_len, Hq, Hkv, kind,
                                device_compute_units());
  if (sp.nsplit <= 1) return 0;
  return partial_bytes(total_q * Hq, sp.nsplit, D);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.num_chunks == 0 || p.total_q == 0) return hipSuccess;
  switch (p.kv_dtype) {
    case DT_F32: return launch_prefill_kind<KF32>(p, stream);
    case DT_BF16: return launch_prefill_kind<KBF16>(p, stream);
    case DT_FP8: return launch_prefill_kind<KFP8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
