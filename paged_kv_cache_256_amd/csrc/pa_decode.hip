// pa_decode.hip -- paged-attention decode for gfx950: stream and reduce kernels (plus a plan
// kernel for batches above 1024 sequences).
//
// What is computed (codebumble.net, "Architectural Anatomy" and its FAQ; bicarait.com,
// "Architectural Blueprint 2"): for sequence b and query head h, exact softmax attention of
// q[b, h] over the context_lens[b] keys and values that block_tables[b] scatters over physical
// frames.  The page's kernel gathers the frames during QK^T and lets different warps score
// different blocks before a final normalised reduction ("CUDA Shared Memory Optimization").
//
// Work decomposition (split-K over the whole batch, stream style).  All (sequence b, kv head g)
// runs of the batch are laid end to end, b-major, each costing u[b] = nblk[b] + R units: R units
// for the fixed cost of starting a run (fetching its query, block ids and first tiles) and one
// unit per frame:
//     X(b, g) = Hkv * cum[b] + g * u[b],   cum[b] = sum_{b' < b} u[b'],
// and the W persistent wavefronts of the launch split the F = Hkv * cum[B] units into W equal
// contiguous ranges [floor(F w / W), floor(F (w+1) / W)).  Every wavefront therefore does the same
// work whatever the mix of context lengths: no idle workgroups for short sequences, no tail of
// long ones, and no wavefront stuck with many more run starts than the others.  Each wavefront
// finds where its range starts with a scan over the batch's lengths (done inside the wavefront
// for up to 1024 sequences, by a one-workgroup plan kernel above that).  A wavefront whose range
// starts inside a run's R units starts at the run's first frame; one whose range ends inside them
// leaves the run to the next.  A run that lies inside one wavefront's range is finished there and
// written to `out`; a run cut by range boundaries leaves an unnormalised partial (max, sum,
// accumulator) in one of the two partial slots of each wavefront it touches, and the reduce
// kernel merges them with the log-sum-exp rule.  (pa_decode_shared lays its runs out in blocks of
// consecutive sequences and inside a block head by head, so that the runs of one prompt stream
// its shared frames at the same time; the split and the merge are the same.)  A small batch whose
// runs all fit one wavefront's share by the host-known bound launches run-aligned instead:
// wavefront w takes run (w / Hkv, w mod Hkv) whole (X of its own run, from one wave-wide sum), so
// nothing is cut and no reduce kernel runs.
//
// Inside a wavefront: the frame ids of up to 64 blocks come in with one vector load (one id per
// lane) and are broadcast with readlane; each step gathers F frames' K and V tiles straight into
// registers (the tile layout puts every lane's matrix-core fragment in one 16-byte load, so a
// tile is NL fully contiguous 1 KiB loads), double-buffered so that one step is in flight while
// the other is computed.  The pipeline does not drain between chunks of 64 frames or between
// runs: the next chunk's ids and query are fetched during the current chunk, whose last two
// load steps already gather the next chunk's first two.  Tiles are read with non-temporal loads:
// each is used once (unless the caller flags frames shared between sequences).  The ranges are
// dealt to the XCDs in contiguous eighths, so neighbouring runs share an L2.  The G
// query heads of the group are the 16 columns of a 16x16 MFMA (GQA: the group shares every K/V
// fragment; unused columns hold zero queries): S^T = K Q^T, an online softmax in the log2 domain
// with the running max reduced across the 4 lanes holding a row, O^T += V^T P^T.  fp8 tiles are
// widened to bf16 in registers; the K scale is folded into the score scale, the V scale into the
// output.


#include <algorithm>

#include "pa_decode_impl.h"

#include <mutex>

namespace pa {

// Device memory of the allocation-free decode entry point: a file-scope array each GPU holds
// for the life of the process.  Host code never uses the array's name as an address (on the
// host it is only a stand-in); the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

using namespace dec;

namespace {

constexpr int kXcds = 8;  // accelerator complex dies of an MI355X

// The same plan for any batch size, in one workgroup: thread t owns the contiguous sequences
// [t*per, (t+1)*per); a block-wide scan of the per-thread unit counts gives every thread its
// offset; each wavefront start is then located by a binary search over the 1024 per-thread
// offsets (in LDS) and a walk over at most `per` sequences, one thread per wavefront.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t* __restrict__ context_lens,
                                                           int32_t* __restrict__ plan, int B,
                                                           int Hkv, int BS, int cap, int W,
                                                           Runs runs) {
  // (runs.size null: every sequence is a run of its own)
  auto units_of = [&](int b) {
    return run_units(runs.size ? run_frames<true>(context_lens, b, B, cap, BS, runs)
                               : run_frames<false>(context_lens, b, B, cap, BS, runs));
  };
  __shared__ int32_t wsum[16];
  __shared__ int32_t tex[1024];  // units before thread t's first sequence
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int per = (B + 1023) / 1024;
  const int b0 = min(B, t * per), b1 = min(B, b0 + per);
  int mine = 0;
  for (int b = b0; b < b1; ++b) mine += units_of(b);
  int incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int k = 0; k < 16; ++k) {
    const int v = wsum[k];
    if (k < wv) before += v;
    total += v;
  }
  tex[t] = before + incl - mine;
  if (t == 0) plan[0] = total;
  __syncthreads();
  const long long F = (long long)Hkv * total;
  const long long q = F / W;
  const unsigned r = (unsigned)(F % W);
  for (int w = t; w < W; w += 1024) {
    const long long aw = q * w + (long long)(r * (unsigned)w / (unsigned)W);  // floor(F w / W)
    const int ap = (int)(aw / max(Hkv, 1));
    int lo = 0, hi = 1023;  // last thread whose first offset is <= ap (it holds unit aw)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tex[mid] <= ap) lo = mid; else hi = mid - 1;
    }
    int cc = tex[lo];
    int b = min(B, lo * per);
    const int bend = min(B, b + per);
    int su = 0;
    int4 st;
    if (runs.size) {
      // runs of sequences that share frames: (block lo, head g, run) order, the block being
      // this thread's sequences (grouped_block(B) of them)
      const int Ut = (lo < 1023 ? tex[lo + 1] : total) - cc;
      const int rem = (int)(aw - (long long)Hkv * cc);
      const int off = Ut > 0 ? rem % Ut : 0;
      int c2 = 0;
      for (; b < bend; ++b) {
        su = units_of(b);
        if (off < c2 + su) break;
        c2 += su;
      }
      st.x = b;
      st.y = Ut > 0 ? rem / Ut : 0;
      st.z = off - c2;
      st.w = su;
    } else {
      for (; b < bend; ++b) {
        su = units_of(b);
        if (ap < cc + su) break;
        cc += su;
      }
      const int off = (int)(aw - (long long)Hkv * cc);
      st.x = b;
      st.y = su > 0 ? off / su : 0;
      st.z = su > 0 ? off % su : 0;
      st.w = su;
    }
    ((int4*)(plan + 4))[w] = st;
  }
}

// (GROUPED runs hold more per lane -- the members' columns, their chunk bounds -- and take up to
// 512 registers: the launch of 3 wavefronts per CU has at most one workgroup on a CU anyway)
template <int KIND, int D, int BS, int F, bool NT, bool GROUPED>
__global__ __launch_bounds__(kWaves * 64, GROUPED ? 1 : kWgPerCu) void decode_stream_kernel(
    void* __restrict__ out, const void* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t* __restrict__ plan, bool inline_plan,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, int B, int mbps, int Hq, int Hkv, int G,
    long long NB, int cap, float qk_scale, float v_scale, Runs runs, bool aligned) {
  // Workgroups reach the 8 XCDs round-robin by id.  XCD k (workgroups k, k + 8, ...) takes the
  // k-th eighth of the ranges, so that runs next to each other in the batch -- branches that share
  // frames -- stream through the same L2.
  const int nwg = gridDim.x;
  const int r = nwg % kXcds == 0 ? (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds
                                 : blockIdx.x;
  decode_stream_wave<KIND, D, BS, F, NT, GROUPED>(
      r * kWaves + uniform(threadIdx.x >> 6), gridDim.x * kWaves, out, q, k_cache,
      v_cache, block_tables, context_lens, plan, inline_plan, ws_ml, ws_o, B, mbps, Hq, Hkv, G,
      NB, cap, qk_scale, v_scale, runs, aligned);
}

template <int KIND, int D, bool GROUPED, bool WIDE>
__global__ __launch_bounds__(64) void decode_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ plan, int Hq, int Hkv, int G, int W, float v_scale, Runs runs,
    int B) {
  // Boundaries in XCD-contiguous blocks: XCD x (workgroups x, x + 8, ...) takes the x-th block of
  // consecutive boundaries.  The wavefronts that merge one heavily cut run by column slices are
  // consecutive boundaries; on one XCD they read each partial row's cache lines into one L2
  // instead of eight.
  const int n = gridDim.x, q = n / kXcds, r = n % kXcds, x = blockIdx.x % kXcds;
  const int k = x * q + min(x, r) + blockIdx.x / kXcds;
  decode_reduce_wave<KIND, D, GROUPED, WIDE>(k, threadIdx.x, out, ws_ml, ws_o, plan, Hq, Hkv, G,
                                             W, v_scale, runs, B, blockIdx.y);
}

// Wavefronts of a launch: the full stream (3 per CU) unless the batch holds too few units for it.
// The host knows an upper bound of the units, B Hkv (ceil(cap / BS) + kRestart); each wavefront
// gets at least kMinUnitsPerWave of it, so a small batch is not cut into one-frame pieces that
// each pay the whole latency chain (plan, ids, tiles, partial, merge).
#ifndef PA_MIN_UNITS_PER_WAVE
#define PA_MIN_UNITS_PER_WAVE 16
#endif
constexpr long long kMinUnitsPerWave = PA_MIN_UNITS_PER_WAVE;

// A batch whose runs all fit in a wavefront's minimum share, by the host-known bound (at most
// kAlignedMaxUnits units: 28 frames), and that holds no more runs than the stream has
// wavefronts, launches one wavefront per run instead (run-aligned): every run is then whole in
// one wavefront, which writes its output directly, and no merge is launched.  A longer chain of
// frames per wavefront costs less than the partials and the merge launch.
constexpr int kAlignedMaxUnits = 2 * kMinUnitsPerWave;

inline bool run_aligned(int B, int Hkv, int cap, int BS) {
  return (long long)B * Hkv <= stream_waves() && (cap + BS - 1) / BS + kRestart <= kAlignedMaxUnits;
}

inline int launch_waves(int B, int Hkv, int cap, int BS) {
  const long long units = (long long)B * Hkv * ((cap + BS - 1) / BS + kRestart);
  const long long want = (units + kMinUnitsPerWave - 1) / kMinUnitsPerWave;
  const long long w = (want + kWaves - 1) / kWaves * kWaves;
  const int full = stream_waves();
  return w >= full ? full : (int)(w > kWaves ? w : kWaves);
}

// Runs of sequences that share frames (pa_decode_shared) launch 4 wavefronts per CU, one per
// SIMD with up to 512 registers each: measured on the 70B-shape fp8 copy-on-write batch (128 runs
// of two branches), 93.4 us against 104.5 us at 3 per CU; two more frames per pipeline step
// instead made it 117 us.  The L2 / MALL hits on the shared frames leave that stream short of
// loads in flight rather than of HBM bandwidth, and the extra wavefronts add them.
constexpr int kGroupedWavesPerCu = 4;

inline int grouped_waves() { return device_compute_units() * kGroupedWavesPerCu / kWaves * kWaves; }

template <int KIND, int D, int BS>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  constexpr int F = step_frames<KIND, D, BS>();
  const int cap = p.max_context_len < p.max_blocks_per_seq * BS ? p.max_context_len
                                                                 : p.max_blocks_per_seq * BS;
  const bool aligned = !p.run_size && run_aligned(p.B, p.Hkv, cap, BS);
  const int Ws = aligned ? (p.B * p.Hkv + kWaves - 1) / kWaves * kWaves
                         : launch_waves(p.B, p.Hkv, cap, BS);
  const Layout l = layout(D, p.run_size ? std::min(Ws / kStreamWavesPerCu * kGroupedWavesPerCu,
                                                   grouped_waves())
                                        : Ws);  // within the workspace's size
  int32_t* plan = (int32_t*)p.workspace;
  float* ws_ml = (float*)((char*)p.workspace + l.plan_bytes);
  float* ws_o = (float*)((char*)p.workspace + l.plan_bytes + l.ml_bytes);
  const int G = p.Hq / p.Hkv;
  const float qk_scale = p.scale * (KIND == KFP8 ? p.k_scale : 1.0f) * kLog2e;
  const float v_scale = KIND == KFP8 ? p.v_scale : 1.0f;
  const bool inline_plan = p.B <= kInlinePlanMax;
  const Runs runs{p.run_size, p.shared_blocks};
  const bool grouped = p.run_size != nullptr;
  hipError_t e;
  if (!inline_plan && !aligned) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, p.context_lens, plan,
                       p.B, p.Hkv, BS, cap, l.W, runs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // runs of sequences that share frames (pa_decode_shared) keep their tiles cacheable too
  auto stream_kernel = grouped ? decode_stream_kernel<KIND, D, BS, F, false, true>
                       : p.shared_frames ? decode_stream_kernel<KIND, D, BS, F, false, false>
                                         : decode_stream_kernel<KIND, D, BS, F, true, false>;
  hipLaunchKernelGGL(stream_kernel, dim3(l.W / kWaves), dim3(kWaves * 64), 0, stream, p.out, p.q, (const char*)p.k_cache, (const char*)p.v_cache,
                     p.block_tables, p.context_lens, plan, inline_plan, ws_ml, ws_o, p.B,
                     p.max_blocks_per_seq, p.Hq, p.Hkv, G, (long long)p.NB, cap, qk_scale, v_scale,
                     runs, aligned);
  e = hipGetLastError();
  if (e != hipSuccess || aligned) return e;
  // few runs against the wavefronts (a few long sequences): each run is cut into many pieces,
  // and the wide merge spreads them over more wavefronts and loads
  const bool wide = !grouped && (long long)l.W >= 16LL * p.B * p.Hkv;
  auto reduce_kernel = grouped ? decode_reduce_kernel<KIND, D, true, false>
                       : wide  ? decode_reduce_kernel<KIND, D, false, true>
                               : decode_reduce_kernel<KIND, D, false, false>;
  // (a grouped launch's merge has two wavefronts per boundary: they split the columns)
  hipLaunchKernelGGL(reduce_kernel, dim3(l.W - 1, grouped ? 2 : 1), dim3(64), 0, stream, p.out, ws_ml,
                     ws_o, plan, p.Hq, p.Hkv, G, l.W, v_scale, runs, p.B);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const DecodeParams& p, hipStream_t s) {
  if (p.D == 64 && p.bs == 16) return launch_typed<KIND, 64, 16>(p, s);
  if (p.D == 64 && p.bs == 32) return launch_typed<KIND, 64, 32>(p, s);
  if (p.D == 128 && p.bs == 16) return launch_typed<KIND, 128, 16>(p, s);
  if constexpr (KIND != KF32) {
    if (p.D == 128 && p.bs == 32) return launch_typed<KIND, 128, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t decode_workspace_bytes(int /*B*/, int /*Hq*/, int D, int /*bs*/, int /*kv_dtype*/,
                              int /*max_context_len*/) {
  const Layout l = layout(D, stream_waves());
  return l.plan_bytes + l.ml_bytes + l.o_bytes;
}

size_t decode_shared_workspace_bytes(int D) {
  const Layout l = layout(D, grouped_waves());
  return l.plan_bytes + l.ml_bytes + l.o_bytes;
}

hipError_t launch_decode_plan(const int32_t* context_lens, int32_t* plan, int B, int Hkv, int bs,
                              int cap, int W, hipStream_t stream) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, context_lens, plan, B, Hkv,
                     bs, cap, W, Runs{});
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  switch (p.kv_dtype) {
    case DT_F32: return launch_kind<KF32>(p, stream);
    case DT_BF16: return launch_kind<KBF16>(p, stream);
    case DT_FP8: return launch_kind<KFP8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa