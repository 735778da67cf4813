// pa_decode.hip -- paged-attention decode for gfx950: plan, stream and reduce kernels.
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
// unit per 4 KiB-class frame:
//     X(b, g) = Hkv * cum[b] + g * u[b],   cum[b] = sum_{b' < b} u[b'],
// and the W persistent wavefronts of the launch split the units into W equal contiguous ranges.
// Every wavefront therefore does the same work whatever the mix of context lengths: no idle
// workgroups for short sequences, no tail of long ones, and no wavefront stuck with many more
// run starts than the others.  A wavefront whose range starts inside a run's R units starts at
// the run's first frame; one whose range ends inside them leaves the run to the next.  A run that
// lies inside one wavefront's range is finished there and written to `out`; a run cut by a range
// boundary leaves an unnormalised partial (max, sum, accumulator) in one of the two partial slots
// of each wavefront it touches, and decode_reduce_kernel merges them with the log-sum-exp rule.
//
// Inside a wavefront: the frame ids of up to 64 blocks come in with one vector load (one id per
// lane) and are broadcast with readlane; each step gathers F frames' K and V tiles straight into
// registers (the tile layout puts every lane's matrix-core fragment in one 16-byte load, so a
// tile is NL fully contiguous 1 KiB loads), double-buffered so that one step is in flight while
// the other is computed.  Tiles are read with non-temporal loads: each is used once.  The G
// query heads of the group are the 16 columns of a 16x16 MFMA (GQA: the group shares every K/V
// fragment; unused columns hold zero queries): S^T = K Q^T, an online softmax in the log2 domain
// with the running max reduced across the 4 lanes holding a row, O^T += V^T P^T.  fp8 tiles are
// widened to bf16 in registers; the K scale is folded into the score scale, the V scale into the
// output.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;    // wavefronts per workgroup (each an independent worker)
constexpr int kWgPerCu = 2;  // persistent workgroups per compute unit (2 waves per SIMD)
constexpr int kIds = 64;     // block ids fetched per vector load

// Cost units of a (sequence, kv head) run of nblk frames: one per frame plus kRestart for the
// run's fixed start-up cost (about two memory latencies, i.e. roughly two frames of a
// wavefront's streaming time).
#ifndef PA_DECODE_RESTART_UNITS
#define PA_DECODE_RESTART_UNITS 2
#endif
constexpr int kRestart = PA_DECODE_RESTART_UNITS;
__host__ __device__ inline int run_units(int nblk) { return nblk > 0 ? nblk + kRestart : 0; }

// Tile loads bypass cache retention by default (each tile is read once per step).
#ifndef PA_DECODE_NONTEMPORAL
#define PA_DECODE_NONTEMPORAL 1
#endif
__device__ inline u32x4 load_tile16(const u32x4* p) {
#if PA_DECODE_NONTEMPORAL
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Frames per pipeline step: two when a tile is 4 KiB or less (double-buffered K+V of two frames
// = 128 VGPRs), one for larger tiles.
template <int KIND, int D, int BS>
constexpr int step_frames() { return KvOps<KIND, D, BS>::NL <= 4 ? 2 : 1; }

template <int KIND>
struct QType {
  static constexpr int bytes = KIND == KF32 ? 4 : 2;
};

// Plan: cum[0..B] (cost units before each sequence, per kv head) and the start (b, g, unit) of
// every wavefront.  One workgroup; thread t owns the contiguous sequences [t*per, (t+1)*per).  A
// block-wide scan of the per-thread unit counts gives every sequence its offset; then each
// wavefront start a_w is located by a binary search over the 1024 per-thread offsets (in LDS) and
// a walk over at most `per` sequences, one thread per wavefront.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t* __restrict__ context_lens,
                                                           int32_t* __restrict__ plan, int B,
                                                           int Hkv, int BS, int cap, int W) {
  int32_t* cum = plan;
  int32_t* start = plan + B + 1;
  __shared__ int32_t wsum[16];
  __shared__ int32_t tex[1024];  // units before thread t's first sequence
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int per = (B + 1023) / 1024;
  const int b0 = min(B, t * per), b1 = min(B, b0 + per);
  int mine = 0;
  for (int b = b0; b < b1; ++b) mine += run_units((max(0, min(context_lens[b], cap)) + BS - 1) / BS);
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
  const int ex = before + incl - mine;
  tex[t] = ex;
  int c = ex;
  for (int b = b0; b < b1; ++b) {
    cum[b] = c;
    c += run_units((max(0, min(context_lens[b], cap)) + BS - 1) / BS);
  }
  if (t == 1023) cum[B] = total;
  __syncthreads();
  const long long F = (long long)Hkv * total;
  if (F <= 0) return;
  const long long q = F / W;
  const unsigned r = (unsigned)(F % W);
  for (int w = t; w < W; w += 1024) {
    const long long aw = q * w + (long long)(r * (unsigned)w / (unsigned)W);  // floor(F w / W)
    const int ap = (int)(aw / Hkv);
    int lo = 0, hi = 1023;  // last thread whose first offset is <= ap (it holds unit aw)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tex[mid] <= ap) lo = mid; else hi = mid - 1;
    }
    int cc = tex[lo];
    int b = min(B, lo * per);
    const int bend = min(B, b + per);
    int su = 0;
    for (; b < bend; ++b) {
      su = run_units((max(0, min(context_lens[b], cap)) + BS - 1) / BS);
      if (ap < cc + su) break;
      cc += su;
    }
    const int off = (int)(aw - (long long)Hkv * cc);
    start[3 * w] = b;
    start[3 * w + 1] = su > 0 ? off / su : 0;
    start[3 * w + 2] = su > 0 ? off % su : 0;
  }
}

__device__ inline long long range_begin(long long F, int w, int W) { return F * w / W; }

template <int KIND, int D, int BS, int F>
__global__ __launch_bounds__(kWaves * 64, kWgPerCu) void decode_stream_kernel(
    void* __restrict__ out, const void* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ plan,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, int B, int mbps, int Hq, int Hkv, int G,
    long long NB, int cap, float qk_scale, float v_scale) {
  using Ops = KvOps<KIND, D, BS>;
  constexpr int NL = Ops::NL, KG = Ops::KG, NS = Ops::NS, NC = Ops::NC, QW = Ops::QW;
  constexpr int NGS = F * KG;  // 16-key groups per step
  constexpr int QB = QType<KIND>::bytes;
  constexpr size_t TILE = Ops::TILE;

  const int W = gridDim.x * kWaves;
  const int w = blockIdx.x * kWaves + uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, j = lane >> 4, n = lane & 15;

  const int32_t* cum = plan;
  const int32_t* start = plan + B + 1;
  const long long Ftot = (long long)Hkv * cum[B];
  const long long a = range_begin(Ftot, w, W), e = range_begin(Ftot, w + 1, W);
  if (a >= e) return;
  int b = start[3 * w], g = start[3 * w + 1], u = start[3 * w + 2];  // u: unit within the run

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[NC];
  uint32_t qw[QW];

  // frame ids of the current chunk (one per lane) and the lane stride of their loads: 1 for a
  // live frame, 0 for a dead one (past the chunk, or an invalid id), which then reads the same
  // 16 bytes of frame 0 in every lane -- the load stays unconditional but moves no tile
  int vfid = 0, vstride = 0;
  uint64_t live_mask = 0;
  int L = 0, cblk = 0;  // context length and first block of the current chunk

  auto load_step = [&](u32x4 (&kt)[F][NL], u32x4 (&vt)[F][NL], int s) {
    // keep a step's loads together and in order: the in-order load counter then lets the
    // compute of the previous step wait for exactly its own data
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = min(s * F + f, 63);
      const int fr = __builtin_amdgcn_readlane(vfid, i);
      const int ls = lane * __builtin_amdgcn_readlane(vstride, i);
      const u32x4* kp = (const u32x4*)(k_cache + ((size_t)fr * Hkv + g) * TILE) + ls;
      const u32x4* vp = (const u32x4*)(v_cache + ((size_t)fr * Hkv + g) * TILE) + ls;
#pragma unroll
      for (int r = 0; r < NL; ++r) kt[f][r] = load_tile16(kp + r * 64);
#pragma unroll
      for (int r = 0; r < NL; ++r) vt[f][r] = load_tile16(vp + r * 64);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Consume step s of the current chunk.  No loads in here: the only branch between a step's
  // loads and this use is the loop back-edge, so the next step's loads stay in flight.
  auto compute_step = [&](u32x4 (&kt)[F][NL], u32x4 (&vt)[F][NL], int s) {
    f32x4 sc[NGS];
    float mx = -INFINITY;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = s * F + f;
      const bool live = i < 64 && ((live_mask >> i) & 1ull);
      const int valid = live ? L - (cblk + i) * BS : 0;  // keys of this frame inside the context
#pragma unroll
      for (int h = 0; h < KG; ++h) {
        f32x4 sv = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) sv = Ops::qk(sv, Ops::kop(kt[f], h, sl), Ops::qop(qw, sl));
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float v = (16 * h + 4 * j + ii < valid) ? sv[ii] * qk_scale : -INFINITY;
          sc[f * KG + h][ii] = v;
          mx = fmaxf(mx, v);
        }
      }
      if (valid < BS) {
        // dead frame, or the last frame of the context: clear V of the slots outside it so that
        // whatever they hold (weighted by probability 0) cannot reach the accumulator
#pragma unroll
        for (int h = 0; h < KG; ++h) {
          const int keep = min(4, max(0, valid - (16 * h + 4 * j)));
#pragma unroll
          for (int c = 0; c < NC; ++c) Ops::zero_quad(vt[f], h, c, keep);
        }
      }
    }
    mx = wave_max_over_j(mx);
    const float mnew = fmaxf(m, mx);
    if (mnew == -INFINITY) return;  // nothing live yet
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] *= alpha;
    typename Ops::PFrag pf[NGS];
#pragma unroll
    for (int gi = 0; gi < NGS; ++gi) {
      f32x4 p;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) p[ii] = __builtin_amdgcn_exp2f(sc[gi][ii] - mnew);
      pf[gi] = Ops::pfrag(p, lsum);
    }
#pragma unroll
    for (int pp = 0; pp < NGS / 2; ++pp) {
      const int ga = 2 * pp, gb = 2 * pp + 1;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        acc[c] = Ops::pv2(acc[c], Ops::vop(vt[ga / KG], ga % KG, c), Ops::vop(vt[gb / KG], gb % KG, c),
                          pf[ga], pf[gb]);
    }
    if constexpr (NGS % 2) {
      constexpr int gl = NGS - 1;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = Ops::pv(acc[c], Ops::vop(vt[gl / KG], gl % KG, c), pf[gl]);
    }
  };

  u32x4 kA[F][NL], vA[F][NL], kB[F][NL], vB[F][NL];
  long long x = a;
  while (x < e && b < B) {
    L = max(0, min(context_lens[b], cap));
    const int nblk = (L + BS - 1) / BS;
    const int units = (int)min((long long)(run_units(nblk) - u), e - x);  // of this run, here
    // frames of the run inside this wavefront's range (its first kRestart units hold none)
    const int f0 = max(0, u - kRestart), f1 = min(nblk, u + units - kRestart);
    const int n_here = f1 - f0;
    if (n_here > 0) {
      const long long s0 = x - u;  // first unit of this (b, g) run
      const bool complete = f0 == 0 && f1 == nblk;
      const int blk = f0;
      // query fragment of row n: dims (D/4)*j .. of head g*G + n (zero if n >= G)
      {
        const bool qv = n < G;
        const size_t row = (size_t)b * Hq + (size_t)g * G + (qv ? n : 0);
        const u32x4* src = (const u32x4*)((const char*)q + (row * D + (size_t)(D / 4) * j) * QB);
#pragma unroll
        for (int i = 0; i < QW / 4; ++i) {
          u32x4 v4 = src[i];
          if (!qv) v4 = (u32x4){0u, 0u, 0u, 0u};
          qw[4 * i] = v4[0]; qw[4 * i + 1] = v4[1]; qw[4 * i + 2] = v4[2]; qw[4 * i + 3] = v4[3];
        }
      }
      m = -INFINITY;
      lsum = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};

      for (int c0 = 0; c0 < n_here; c0 += kIds) {
        const int cn = min(kIds, n_here - c0);
        cblk = blk + c0;
        const int f_raw = block_tables[(size_t)b * mbps + min(cblk + lane, nblk - 1)];
        const bool ok = lane < cn && f_raw >= 0 && (long long)f_raw < NB;
        live_mask = __ballot(ok);
        vfid = ok ? f_raw : 0;
        vstride = ok ? 1 : 0;
        const int nsteps = (cn + F - 1) / F;
        load_step(kA, vA, 0);
        load_step(kB, vB, 1);
        for (int s = 0; s < nsteps; s += 2) {
          compute_step(kA, vA, s);
          load_step(kA, vA, s + 2);
          compute_step(kB, vB, s + 1);
          load_step(kB, vB, s + 3);
        }
      }

      const float lrow = wave_sum_over_j(lsum);
      if (n < G) {
        if (complete) {
          const float inv = v_scale / lrow;
          const size_t o = ((size_t)b * Hq + (size_t)g * G + n) * D + 4 * j;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if constexpr (KIND == KF32) {
              *(f32x4*)((float*)out + o + 16 * c) = acc[c] * inv;
            } else {
              u32x2 pk;
              pk[0] = pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv);
              pk[1] = pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv);
              *(u32x2*)((__bf16*)out + o + 16 * c) = pk;
            }
          }
        } else {
          const size_t row = ((size_t)w * 2 + (s0 > a ? 1 : 0)) * 16 + n;
#pragma unroll
          for (int c = 0; c < NC; ++c) *(f32x4*)(ws_o + row * D + 16 * c + 4 * j) = acc[c];
          if (j == 0) {
            ws_ml[2 * row] = m;
            ws_ml[2 * row + 1] = lrow;
          }
        }
      }
    }
    x += units > 0 ? units : 0;
    u = 0;
    if (++g == Hkv) {
      g = 0;
      ++b;
    }
  }
}

// Merge the partials of every (b, g) run that crosses a wavefront boundary:
// out = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w, M = max_w m_w.
// The wavefronts holding the run are w0..w1; wavefront w keeps it in slot 1 if the run began
// after the start of w's range (then it is w's last run), else in slot 0.
template <int KIND>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ plan, int B, int Hq, int Hkv, int G, int D, int W,
    float v_scale) {
  // One workgroup per (b, g); runs finished inside one stream wavefront exit at once.
  constexpr int kPer = 8;   // outputs per thread: G * D <= 16 * 128 = 8 * 256
  constexpr int kBatch = 4; // partials whose loads are issued together
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int32_t* cum = plan;
  const int c0 = cum[b], c1 = cum[b + 1], cB = cum[B];
  const long long F = (long long)Hkv * cB;
  const int su = c1 - c0;  // units of each kv head's run of sequence b
  const int nblk = su - kRestart;
  if (su <= 0 || nblk <= 0 || F <= 0) return;
  const long long s0 = (long long)Hkv * c0 + (long long)g * su;  // first unit of the run
  const long long x0 = s0 + kRestart, x1 = s0 + su - 1;           // its first and last frame
  // wavefront holding unit x: the largest w with floor(F w / W) <= x
  const int w0 = (int)(((x0 + 1) * W + F - 1) / F - 1);
  const int w1 = (int)(((x1 + 1) * W + F - 1) / F - 1);
  if (w0 == w1) return;  // finished inside one wavefront
  const long long q = F / W;
  const unsigned r = (unsigned)(F % W);
  const int nout = G * D;
  float M[kPer], num[kPer], den[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    M[k] = -INFINITY;
    num[k] = 0.f;
    den[k] = 0.f;
  }
  // partials in wavefront order (a fixed merge order: the result does not depend on timing),
  // kBatch at a time with all their loads in flight together
  for (int wb = w0; wb <= w1; wb += kBatch) {
    int row0[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int w = wb + i;
      row0[i] = -1;
      if (w <= w1) {
        const long long aw = q * w + (long long)(r * (unsigned)w / (unsigned)W);
        const long long aw1 = q * (w + 1) + (long long)(r * (unsigned)(w + 1) / (unsigned)W);
        if (aw < aw1) row0[i] = (w * 2 + (s0 > aw ? 1 : 0)) * 16;
      }
    }
    float mw[kBatch][kPer], lw[kBatch][kPer], ow[kBatch][kPer];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int idx = t + 256 * k;
        const int rr = idx / D;
        const bool ok = row0[i] >= 0 && idx < nout;
        const size_t prow = (size_t)(ok ? row0[i] + rr : 0);
        mw[i][k] = ok ? ws_ml[2 * prow] : -INFINITY;
        lw[i][k] = ok ? ws_ml[2 * prow + 1] : 0.f;
        ow[i][k] = ok ? ws_o[prow * D + (idx - rr * D)] : 0.f;
      }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        if (mw[i][k] == -INFINITY) continue;
        if (mw[i][k] > M[k]) {
          const float sc = __builtin_amdgcn_exp2f(M[k] - mw[i][k]);
          num[k] *= sc;
          den[k] *= sc;
          M[k] = mw[i][k];
        }
        const float e = __builtin_amdgcn_exp2f(mw[i][k] - M[k]);
        num[k] += e * ow[i][k];
        den[k] += e * lw[i][k];
      }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = t + 256 * k;
    if (idx >= nout) break;
    const int rr = idx / D, d = idx - rr * D;
    const float o = num[k] / den[k] * v_scale;
    const size_t oi = ((size_t)b * Hq + (size_t)g * G + rr) * D + d;
    if constexpr (KIND == KF32) {
      ((float*)out)[oi] = o;
    } else {
      ((__bf16*)out)[oi] = (__bf16)o;
    }
  }
}

struct Layout {
  int W;
  size_t plan_bytes, ml_bytes, o_bytes;
};

Layout layout(int B, int D) {
  Layout l;
  l.W = device_compute_units() * kWgPerCu * kWaves;
  l.plan_bytes = (((size_t)(B + 1) + 3 * (size_t)l.W) * sizeof(int32_t) + 255) / 256 * 256;
  l.ml_bytes = (((size_t)l.W * 2 * 16 * 2) * sizeof(float) + 255) / 256 * 256;
  l.o_bytes = (size_t)l.W * 2 * 16 * D * sizeof(float);
  return l;
}

template <int KIND, int D, int BS>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  constexpr int F = step_frames<KIND, D, BS>();
  const Layout l = layout(p.B, D);
  int32_t* plan = (int32_t*)p.workspace;
  float* ws_ml = (float*)((char*)p.workspace + l.plan_bytes);
  float* ws_o = (float*)((char*)p.workspace + l.plan_bytes + l.ml_bytes);
  const int G = p.Hq / p.Hkv;
  const int cap = p.max_context_len < p.max_blocks_per_seq * BS ? p.max_context_len
                                                                 : p.max_blocks_per_seq * BS;
  const float qk_scale = p.scale * (KIND == KFP8 ? p.k_scale : 1.0f) * kLog2e;
  const float v_scale = KIND == KFP8 ? p.v_scale : 1.0f;
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, p.context_lens, plan, p.B,
                     p.Hkv, BS, cap, l.W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_stream_kernel<KIND, D, BS, F>), dim3(l.W / kWaves), dim3(kWaves * 64),
                     0, stream, p.out, p.q, (const char*)p.k_cache, (const char*)p.v_cache,
                     p.block_tables, p.context_lens, plan, ws_ml, ws_o, p.B, p.max_blocks_per_seq,
                     p.Hq, p.Hkv, G, (long long)p.NB, cap, qk_scale, v_scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<KIND>), dim3(p.Hkv, p.B), dim3(256), 0, stream, p.out,
                     ws_ml, ws_o, plan, p.B, p.Hq, p.Hkv, G, D, l.W, v_scale);
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

size_t decode_workspace_bytes(int B, int /*Hq*/, int D, int /*bs*/, int /*kv_dtype*/,
                              int /*max_context_len*/) {
  const Layout l = layout(B, D);
  return l.plan_bytes + l.ml_bytes + l.o_bytes;
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
