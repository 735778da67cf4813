// pa_decode.hip -- paged-attention decode for gfx950: plan, stream and reduce kernels.
//
// What is computed (codebumble.net, "Architectural Anatomy" and its FAQ; bicarait.com,
// "Architectural Blueprint 2"): for sequence b and query head h, exact softmax attention of
// q[b, h] over the context_lens[b] keys and values that block_tables[b] scatters over physical
// frames.  The page's kernel gathers the frames during QK^T and lets different warps score
// different blocks before a final normalised reduction ("CUDA Shared Memory Optimization").
//
// Work decomposition (split-K over the whole batch, stream style).  All (sequence b, kv head g,
// logical block) frames of the batch form one sequence ordered by b, then g, then block:
//     x(b, g, blk) = Hkv * cum[b] + g * nblk[b] + blk,   cum[b] = sum_{b' < b} nblk[b'],
// and the W persistent wavefronts of the launch split it into W equal contiguous ranges.  Every
// wavefront therefore streams the same number of tiles whatever the mix of context lengths (no
// idle workgroups for short sequences, no tail of long ones).  A (b, g) run that lies inside one
// wavefront's range is finished there and written to `out`; a run cut by a range boundary
// leaves an unnormalised partial (max, sum, accumulator) in one of the two partial slots of each
// wavefront it touches, and decode_reduce_kernel merges them with the log-sum-exp rule.
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

// Frames per pipeline step: two when a tile is 4 KiB or less (double-buffered K+V of two frames
// = 128 VGPRs), one for larger tiles.
template <int KIND, int D, int BS>
constexpr int step_frames() { return KvOps<KIND, D, BS>::NL <= 4 ? 2 : 1; }

template <int KIND>
struct QType {
  static constexpr int bytes = KIND == KF32 ? 4 : 2;
};

// Plan: cum[0..B] (blocks before each sequence) and the start (b, g, blk) of every wavefront.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t* __restrict__ context_lens,
                                                           int32_t* __restrict__ plan, int B,
                                                           int Hkv, int BS, int cap, int W) {
  int32_t* cum = plan;
  int32_t* start = plan + B + 1;
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  const int t = threadIdx.x;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    const int b = base + t;
    int v = 0;
    if (b < B) {
      const int L = max(0, min(context_lens[b], cap));
      v = (L + BS - 1) / BS;
    }
    part[t] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = t >= off ? part[t - off] : 0;
      __syncthreads();
      part[t] += add;
      __syncthreads();
    }
    if (b < B) cum[b] = carry + part[t] - v;
    __syncthreads();
    if (t == 1023) carry += part[1023];
    __syncthreads();
  }
  if (t == 0) cum[B] = carry;
  __threadfence();
  __syncthreads();
  const long long F = (long long)Hkv * carry;
  for (int w = t; w < W; w += 1024) {
    const long long a = F * w / W;
    int b = 0, g = 0, blk = 0;
    if (a < F) {
      const long long ap = a / Hkv;
      int lo = 0, hi = B - 1;  // last b with cum[b] <= ap: the sequence holding frame a
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cum[mid] <= ap) lo = mid; else hi = mid - 1;
      }
      b = lo;
      const int nb = cum[b + 1] - cum[b];
      const long long r = a - (long long)Hkv * cum[b];
      g = (int)(r / nb);
      blk = (int)(r % nb);
    }
    start[3 * w] = b;
    start[3 * w + 1] = g;
    start[3 * w + 2] = blk;
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
  int b = start[3 * w], g = start[3 * w + 1], blk = start[3 * w + 2];

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
      for (int r = 0; r < NL; ++r) kt[f][r] = __builtin_nontemporal_load(kp + r * 64);
#pragma unroll
      for (int r = 0; r < NL; ++r) vt[f][r] = __builtin_nontemporal_load(vp + r * 64);
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
    const int n_here = (int)min((long long)(nblk - blk), e - x);
    if (n_here > 0) {
      const long long s0 = x - blk;  // first frame of this (b, g) run
      const bool complete = blk == 0 && n_here == nblk;
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
    x += n_here > 0 ? n_here : 0;
    blk = 0;
    if (++g == Hkv) {
      g = 0;
      ++b;
    }
  }
}

// Merge the partials of every (b, g) run that crosses a wavefront boundary:
// out = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w, M = max_w m_w.
template <int KIND>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ plan, int B, int Hq, int Hkv, int G, int D, int W,
    float v_scale) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int32_t* cum = plan;
  const long long F = (long long)Hkv * cum[B];
  const int nblk = cum[b + 1] - cum[b];
  if (nblk <= 0 || F <= 0) return;
  const long long s0 = (long long)Hkv * cum[b] + (long long)g * nblk;
  const long long s1 = s0 + nblk;
  // wavefront holding frame x: the largest w with floor(F w / W) <= x
  const int w0 = (int)(((s0 + 1) * W + F - 1) / F - 1);
  const int w1 = (int)((s1 * W + F - 1) / F - 1);
  if (w0 == w1) return;  // finished inside one wavefront
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int r = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int w = w0; w <= w1; ++w) {
      const long long aw = range_begin(F, w, W);
      if (aw >= range_begin(F, w + 1, W)) continue;
      M = fmaxf(M, ws_ml[2 * (((size_t)w * 2 + (s0 > aw ? 1 : 0)) * 16 + r)]);
    }
    float num = 0.f, den = 0.f;
    for (int w = w0; w <= w1; ++w) {
      const long long aw = range_begin(F, w, W);
      if (aw >= range_begin(F, w + 1, W)) continue;
      const size_t row = ((size_t)w * 2 + (s0 > aw ? 1 : 0)) * 16 + r;
      const float mw = ws_ml[2 * row];
      if (mw == -INFINITY) continue;
      const float sc = __builtin_amdgcn_exp2f(mw - M);
      num += sc * ws_o[row * D + d];
      den += sc * ws_ml[2 * row + 1];
    }
    const float o = num / den * v_scale;
    const size_t oi = ((size_t)b * Hq + (size_t)g * G + r) * D + d;
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
