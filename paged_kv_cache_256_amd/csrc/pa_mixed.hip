// pa_mixed.hip -- one launch for a mixed batch (gfx950): the prefill chunks and the decodes of a
// step run side by side in a single persistent kernel.
//
// What is computed (bicarait.com, "Architectural Blueprint 3"; infoisland, section 5): each
// iteration pairs a prefill chunk (512 tokens in the pages' example) with the ongoing
// single-token decodes.  The results are those of pa_prefill_chunk on the chunks and pa_decode on
// the decodes; only the way the two share the GPU differs.
//
// The halves load the chip differently: a chunk is a dense contraction held back by the matrix
// cores and LDS (its K/V mostly come from L2), a decode streams each frame of its context once
// and is held back by HBM.  When the decodes' bytes are small next to the chunk's matrix work,
// one persistent kernel runs both halves at once ("split"): one 8-wavefront workgroup per compute
// unit, the first P running prefill tiles (the tile body of pa_prefill_chunk) while the other
// CUs - P put their wavefronts on the decode stream (the stream body of pa_decode over
// (CUs - P) x 8 wavefronts), and a second small kernel merges the split partials of both.
// Otherwise the call runs the chunks and then the decodes with the kernels of pa_prefill_chunk
// and pa_decode ("separate").
//
// Measured on MI355X, the split pays only in a narrow range: a compute unit streams at most
// ~45 GB/s (8 wavefronts' loads in flight), so the decode half needs many CUs to reach the HBM
// rate, and the chunk runs ~1.4x slower per CU while the decode stream holds HBM (its K/V
// fetches wait behind the stream).  Starting the decode stream on the CUs whose prefill tiles end
// early (one kernel, prefill then decode in every workgroup) was slower than two launches for
// the same reason.  The host predicts both modes with these rates -- the caller's count of the
// decodes' context tokens feeds the decode term -- and takes the split only when it wins by a
// margin.  The count moves the choice only, never the results.
//
// Prefill tiles that share a key range are dealt to workgroups of one XCD (workgroups go to the
// 8 XCDs round-robin by id), so that range is read into one L2 only.

#include <algorithm>

#include "pa_decode_impl.h"
#include "pa_prefill_impl.h"

namespace pa {

using namespace dec;
using namespace pre;

namespace {

constexpr int kXcds = 8;

// Rates of the two bodies on MI355X (measured): the prefill tiles' matrix work per compute
// unit, its slowdown while the decode stream holds HBM, the decode stream's bytes per compute
// unit (8 wavefronts) and the rate at which HBM serves the whole decode stream.
constexpr double kPrefillFlopsPerCu = 2.9e12;  // bf16 / fp8 operands; f32 runs at a quarter
constexpr double kPrefillContention = 1.4;
constexpr double kDecodeBytesPerCu = 45e9;
constexpr double kDecodeHbmBytes = 5.7e12;
constexpr double kSeparateGapSec = 10e-6;  // launch gaps of the separate kernels
constexpr double kSplitMargin = 0.97;       // the split must beat the separate kernels by 3%

struct MixedArgs {
  void* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  // decodes: sequences [0, B) of the batch
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t* plan;
  float* d_ml;
  float* d_o;
  int B, dcap;
  bool inline_plan;
  // chunks: sequences [B, B + nc) of the batch, seen from their own first entry
  const int32_t* tables_c;
  const int32_t* qsl_c;
  const int32_t* lens_c;
  float* p_ml;
  float* p_o;
  int nc, QT, tiles, nsplit, KS, max_ctx;
  long long total_q, row_base;
  // shared
  int P, xcd_deal, mbps, Hq, Hkv, G;
  long long NB;
  float qk_scale, v_scale;
};

template <int KIND, int D, int BS, bool NTL>
__global__ __launch_bounds__(kPWaves * 64, 1) void mixed_kernel(MixedArgs a) {
  constexpr int NT = tiles_per_wave(KIND);
  constexpr int F = step_frames<KIND, D, BS>();
  constexpr int S = prefill_stage_bytes<KIND, D, BS>();
  constexpr int SW = prefill_widened_bytes<KIND, D, BS>();
  __shared__ __attribute__((aligned(1024))) char ring0[S], ring1[S], ring2[S], ring3[S];
  __shared__ __attribute__((aligned(1024))) char wide0[SW], wide1[SW];
  const int wg = blockIdx.x;
  if (wg < a.P) {
    // tiles are ordered key range (x, chunk, kv head) first, query tile last; with P a multiple
    // of 8, XCD k receives the contiguous tiles [k P / 8, (k + 1) P / 8) of every round
    const int rank = a.xcd_deal ? (wg % kXcds) * (a.P / kXcds) + wg / kXcds : wg;
    const int ncg = a.nc * a.Hkv;
    for (int t = rank; t < a.tiles; t += a.P) {
      const int grp = t / a.QT, qt = t - grp * a.QT;
      const int x = grp / ncg, cg = grp - x * ncg;
      prefill_tile<KIND, D, BS, NT>(ring0, ring1, ring2, ring3, wide0, wide1, x, qt, cg / a.Hkv, cg % a.Hkv, a.row_base, a.out,
                                    a.q, a.k_cache, a.v_cache, a.tables_c, a.qsl_c, a.lens_c,
                                    a.p_ml, a.p_o, a.mbps, a.Hq, a.Hkv, a.G, a.NB, a.total_q,
                                    a.nsplit, a.KS, a.max_ctx, a.qk_scale, a.v_scale);
      __syncthreads();  // the next tile refills the LDS ring
    }
    return;
  }
  // decode workgroups: XCD k takes the k-th eighth of the decode ranges (as in pa_decode), when
  // the prefill and decode workgroup counts keep the round-robin aligned
  const int nd = (int)gridDim.x - a.P, rd = wg - a.P;
  const int r = (a.P % kXcds == 0 && nd % kXcds == 0) ? (rd % kXcds) * (nd / kXcds) + rd / kXcds : rd;
  decode_stream_wave<KIND, D, BS, F, NTL>(
      r * kPWaves + uniform(threadIdx.x >> 6), nd * kPWaves, a.out,
      a.q, a.k_cache, a.v_cache, a.block_tables, a.context_lens, a.plan, a.inline_plan, a.d_ml,
      a.d_o, a.B, a.mbps, a.Hq, a.Hkv, a.G, a.NB, a.dcap, a.qk_scale, a.v_scale);
}

struct MergeArgs {
  void* out;
  const float* d_ml;
  const float* d_o;
  const int32_t* plan;
  int dblocks, Wd;
  const float* p_ml;
  const float* p_o;
  const int32_t* qsl_c;
  const int32_t* lens_c;
  int nc, nsplit, KS, pcap;
  long long total_q, row_base;
  int Hq, Hkv, G;
  float v_scale;
};

// Workgroups [0, dblocks) merge decode runs (one wavefront per wavefront-range boundary), the
// rest merge chunk rows whose keys span several ranges (one wavefront per (row, head)).
template <int KIND, int D>
__global__ __launch_bounds__(256) void mixed_merge_kernel(MergeArgs m) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < m.dblocks) {
    const int k = blockIdx.x * 4 + wave;
    if (k < m.Wd - 1)
      decode_reduce_wave<KIND, D>(k, lane, m.out, m.d_ml, m.d_o, m.plan, m.Hq, m.Hkv, m.G, m.Wd,
                                  m.v_scale);
    return;
  }
  prefill_reduce_wave<KIND, D>((long long)(blockIdx.x - m.dblocks) * 4 + wave, lane, m.row_base,
                               m.out, m.p_ml, m.p_o, m.qsl_c, m.lens_c, m.nc, m.total_q, m.Hq,
                               m.nsplit, m.KS, m.pcap, m.v_scale);
}

int kind_of(int kv_dtype) { return kv_dtype == DT_F32 ? KF32 : (kv_dtype == DT_BF16 ? KBF16 : KFP8); }

int elem_bytes_of(int kv_dtype) { return kv_dtype == DT_F32 ? 4 : (kv_dtype == DT_BF16 ? 2 : 1); }

struct Roles {
  int P;          // split: workgroups running prefill tiles (the rest stream the decodes)
  bool separate;  // the pa_prefill_chunk kernels, then the pa_decode kernels
  Split sp;
};

// Chunk rows of the batch (the rows after the decodes' one row each).
long long chunk_rows(const MixedParams& p) { return p.total_q - p.num_decodes; }

Roles choose_roles(const MixedParams& p, int cus) {
  const int kind = kind_of(p.kv_dtype);
  const bool has_c = p.num_chunks > 0 && chunk_rows(p) > 0;
  if (!has_c) return Roles{0, true, Split{1, 64}};
  const Split full = choose_split(p.num_chunks, p.max_chunk_len, p.max_context_len, p.Hq, p.Hkv, kind, cus);
  if (p.num_decodes == 0 || cus < 2) return Roles{cus, true, full};
  const int G = p.Hq / p.Hkv;
  const int NT = tiles_per_wave(kind);
  const int TQ = kPWaves * NT * 16 / G;
  const long long base_tiles = (long long)p.num_chunks * ((p.max_chunk_len + TQ - 1) / TQ) * p.Hkv;
  const double stage_flops = (double)kPWaves * NT * 16 * 32 * 4 * p.D;
  const double prate = kPrefillFlopsPerCu / (kind == KF32 ? 4.0 : 1.0);
  // chunk time on P compute units (rounds of tiles x stages per tile)
  auto chunk_time = [&](int P, const Split& sp) {
    const long long tiles = base_tiles * sp.nsplit;
    const long long rounds = (tiles + P - 1) / P;
    const int keys = sp.KS < p.max_context_len ? sp.KS : p.max_context_len;
    return rounds * ((keys + 31) / 32) * stage_flops / prate;
  };
  const long long dtok = p.decode_tokens > 0 ? p.decode_tokens
                                             : (long long)p.num_decodes * p.max_context_len / 2;
  const double dbytes = (double)dtok * p.Hkv * p.D * 2.0 * elem_bytes_of(p.kv_dtype);
  auto decode_time = [&](int n) { return dbytes / std::min(kDecodeHbmBytes, n * kDecodeBytesPerCu); };
  const double t_separate = chunk_time(cus, full) + decode_time(cus) + kSeparateGapSec;
  Roles split{0, false, full};
  double t_split = 1e300;
  const int step = cus >= 4 * kXcds ? kXcds : 1;
  for (int P = step; P <= cus - step; P += step) {
    const Split sp = choose_split(p.num_chunks, p.max_chunk_len, p.max_context_len, p.Hq, p.Hkv, kind, P);
    const double t = std::max(kPrefillContention * chunk_time(P, sp), decode_time(cus - P));
    if (t < t_split) {
      t_split = t;
      split = Roles{P, false, sp};
    }
  }
  const Roles separate{cus, true, full};
  if (p.mode == MIXED_SEPARATE || split.P == 0) return separate;
  if (p.mode == MIXED_SPLIT) return split;
  return t_split < kSplitMargin * t_separate ? split : separate;
}

// Workspace: the decode plan and partials sized for every wavefront of the chip, then the chunk
// partials sized for the largest context split a launch can choose (the one for all CUs).
struct MixedLayout {
  size_t dec_bytes, pre_bytes;
  int nsplit_max;
};

MixedLayout mixed_layout(int num_decodes, int num_chunks, long long crows, int max_chunk_len,
                         int max_context_len, int Hq, int Hkv, int D, int kv_dtype) {
  MixedLayout l{0, 0, 1};
  if (num_decodes > 0) {
    const Layout d = layout(D, device_compute_units() * kPWaves);
    l.dec_bytes = d.plan_bytes + d.ml_bytes + (d.o_bytes + 255) / 256 * 256;
  }
  if (num_chunks > 0 && crows > 0) {
    l.nsplit_max = choose_split(num_chunks, max_chunk_len, max_context_len, Hq, Hkv,
                                kind_of(kv_dtype), device_compute_units()).nsplit;
    if (l.nsplit_max > 1) l.pre_bytes = partial_bytes(crows * Hq, l.nsplit_max, D);
  }
  return l;
}

// The separate mode: the chunks with the pa_prefill_chunk kernels (chunk rows after the decode
// rows), then the decodes with the pa_decode kernels, on the caller's stream.
hipError_t launch_separate(const MixedParams& p, const MixedLayout& ml, hipStream_t stream) {
  char* ws = (char*)p.workspace;
  if (p.num_chunks > 0 && chunk_rows(p) > 0) {
    PrefillParams pp{p.out, p.q, p.k_cache, p.v_cache,
                     p.block_tables + (size_t)p.num_decodes * p.max_blocks_per_seq,
                     p.max_blocks_per_seq, p.query_start_loc + p.num_decodes,
                     p.context_lens + p.num_decodes, p.num_chunks, p.total_q, p.max_chunk_len,
                     p.max_context_len, p.Hq, p.Hkv, p.D, p.bs, p.NB, p.scale, p.kv_dtype,
                     p.k_scale, p.v_scale, ml.pre_bytes > 0 ? ws + ml.dec_bytes : nullptr,
                     p.num_decodes};
    const hipError_t e = launch_prefill(pp, stream);
    if (e != hipSuccess) return e;
  }
  if (p.num_decodes == 0) return hipSuccess;
  DecodeParams dp{p.out, p.q, p.k_cache, p.v_cache, p.block_tables, p.max_blocks_per_seq,
                  p.context_lens, p.num_decodes, p.Hq, p.Hkv, p.D, p.bs, p.NB, p.scale,
                  p.kv_dtype, p.k_scale, p.v_scale, p.max_context_len, ws, p.shared_frames};
  return launch_decode(dp, stream);
}

template <int KIND, int D, int BS>
hipError_t launch_mixed_typed(const MixedParams& p, hipStream_t stream) {
  const int cus = device_compute_units();
  const MixedLayout ml = mixed_layout(p.num_decodes, p.num_chunks, chunk_rows(p), p.max_chunk_len,
                                      p.max_context_len, p.Hq, p.Hkv, p.D, p.kv_dtype);
  const Roles roles = choose_roles(p, cus);
  if (roles.separate) return launch_separate(p, ml, stream);
  const bool has_c = roles.P > 0;
  const bool has_d = p.num_decodes > 0;
  const int grid = cus;
  const int Wd = (grid - roles.P) * kPWaves;
  const Layout dl = layout(D, cus * kPWaves);
  char* ws = (char*)p.workspace;

  MixedArgs a{};
  a.out = p.out;
  a.q = p.q;
  a.k_cache = (const char*)p.k_cache;
  a.v_cache = (const char*)p.v_cache;
  a.block_tables = p.block_tables;
  a.context_lens = p.context_lens;
  a.plan = has_d ? (int32_t*)ws : nullptr;
  a.d_ml = has_d ? (float*)(ws + dl.plan_bytes) : nullptr;
  a.d_o = has_d ? (float*)(ws + dl.plan_bytes + dl.ml_bytes) : nullptr;
  a.B = p.num_decodes;
  a.dcap = p.max_context_len < p.max_blocks_per_seq * BS ? p.max_context_len : p.max_blocks_per_seq * BS;
  a.inline_plan = p.num_decodes <= kInlinePlanMax;
  a.tables_c = p.block_tables + (size_t)p.num_decodes * p.max_blocks_per_seq;
  a.qsl_c = p.query_start_loc + p.num_decodes;
  a.lens_c = p.context_lens + p.num_decodes;
  const long long crows = chunk_rows(p);
  const bool psplit = has_c && roles.sp.nsplit > 1;
  a.p_ml = psplit ? (float*)(ws + ml.dec_bytes) : nullptr;
  a.p_o = psplit ? a.p_ml + partial_ml_floats(crows * p.Hq, roles.sp.nsplit) : nullptr;
  a.nc = p.num_chunks;
  const int G = p.Hq / p.Hkv;
  const int TQ = kPWaves * tiles_per_wave(KIND) * 16 / G;
  a.QT = (p.max_chunk_len + TQ - 1) / TQ;
  a.tiles = has_c ? p.num_chunks * a.QT * p.Hkv * roles.sp.nsplit : 0;
  a.nsplit = roles.sp.nsplit;
  a.KS = roles.sp.KS;
  a.max_ctx = p.max_context_len;
  a.total_q = p.total_q;
  a.row_base = p.num_decodes;
  a.P = roles.P;
  a.xcd_deal = roles.P % kXcds == 0 ? 1 : 0;
  a.mbps = p.max_blocks_per_seq;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = G;
  a.NB = p.NB;
  a.qk_scale = p.scale * (KIND == KFP8 ? p.k_scale : 1.0f) * kLog2e;
  a.v_scale = KIND == KFP8 ? p.v_scale : 1.0f;

  hipError_t e;
  if (has_d && !a.inline_plan) {
    e = launch_decode_plan(p.context_lens, a.plan, p.num_decodes, p.Hkv, BS, a.dcap, Wd, stream);
    if (e != hipSuccess) return e;
  }
  auto kernel = p.shared_frames ? mixed_kernel<KIND, D, BS, false> : mixed_kernel<KIND, D, BS, true>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kPWaves * 64), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  MergeArgs m{};
  m.out = p.out;
  m.d_ml = a.d_ml;
  m.d_o = a.d_o;
  m.plan = a.plan;
  m.Wd = Wd;
  m.dblocks = Wd > 1 ? (Wd - 1 + 3) / 4 : 0;
  m.p_ml = a.p_ml;
  m.p_o = a.p_o;
  m.qsl_c = a.qsl_c;
  m.lens_c = a.lens_c;
  m.nc = p.num_chunks;
  m.nsplit = roles.sp.nsplit;
  m.KS = roles.sp.KS;
  m.pcap = a.dcap;
  m.total_q = p.total_q;
  m.row_base = p.num_decodes;
  m.Hq = p.Hq;
  m.Hkv = p.Hkv;
  m.G = G;
  m.v_scale = a.v_scale;
  const long long pblocks = psplit ? (crows * p.Hq + 7) / 8 : 0;
  const long long blocks = m.dblocks + pblocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mixed_merge_kernel<KIND, D>), dim3((unsigned)blocks), dim3(256), 0, stream, m);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_mixed_kind(const MixedParams& p, hipStream_t s) {
  if (p.D == 64 && p.bs == 16) return launch_mixed_typed<KIND, 64, 16>(p, s);
  if (p.D == 64 && p.bs == 32) return launch_mixed_typed<KIND, 64, 32>(p, s);
  if (p.D == 128 && p.bs == 16) return launch_mixed_typed<KIND, 128, 16>(p, s);
  if constexpr (KIND != KF32) {
    if (p.D == 128 && p.bs == 32) return launch_mixed_typed<KIND, 128, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t mixed_workspace_bytes(int num_decodes, int num_chunks, int64_t total_q, int max_chunk_len,
                             int max_context_len, int Hq, int Hkv, int D, int kv_dtype) {
  const MixedLayout l = mixed_layout(num_decodes, num_chunks, total_q - num_decodes, max_chunk_len,
                                     max_context_len, Hq, Hkv, D, kv_dtype);
  return l.dec_bytes + l.pre_bytes;
}

int mixed_prefill_workgroups(const MixedParams& p) { return choose_roles(p, device_compute_units()).P; }

hipError_t launch_mixed(const MixedParams& p, hipStream_t stream) {
  if (p.num_decodes == 0 && (p.num_chunks == 0 || chunk_rows(p) == 0)) return hipSuccess;
  switch (p.kv_dtype) {
    case DT_F32: return launch_mixed_kind<KF32>(p, stream);
    case DT_BF16: return launch_mixed_kind<KBF16>(p, stream);
    case DT_FP8: return launch_mixed_kind<KFP8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
