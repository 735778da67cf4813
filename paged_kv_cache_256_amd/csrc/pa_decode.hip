// pa_decode.hip -- paged-attention decode for gfx950: a partition kernel and a reduce kernel.
//
// What is computed (codebumble.net, "Architectural Anatomy" and its FAQ; bicarait.com,
// "Architectural Blueprint 2"): for sequence b and query head h, exact softmax attention of
// q[b, h] over the context_lens[b] keys and values that block_tables[b] scatters over
// physical frames.  The page's kernel gathers the frames during QK^T, stages tiles close to
// the compute units and lets different warps score different blocks before a final
// normalised reduction ("CUDA Shared Memory Optimization").  Here:
//
//  * One workgroup of WAVES wavefronts owns a partition of PB = WAVES * MAXF consecutive
//    logical blocks of one (sequence, kv head).  Wavefront w takes blocks w, w + WAVES, ...
//    and gathers each (frame, head) K and V tile straight into registers with NL contiguous
//    1 KiB loads (the tile layout puts every lane's MFMA fragment in one 16-byte load), one
//    step of F frames ahead of the frames it is computing.  The block table is read with
//    scalar loads; all address arithmetic is scalar.
//  * The G query heads of the group are the 16 columns of a 16x16 MFMA (GQA: the group
//    shares every K/V tile; unused columns are zero queries).  S^T = K Q^T, an online
//    softmax in the log2 domain with the running max reduced across the 4 lanes holding a
//    row, and O^T += V^T P^T on the matrix cores.  fp8 tiles are widened to bf16 in
//    registers; the K scale is folded into the score scale and the V scale into the output.
//  * The wavefronts of a workgroup merge their (max, sum, accumulator) in LDS.  A sequence
//    that fits one partition writes its output directly; longer ones write unnormalised
//    partials (split-K over the context) that decode_reduce_kernel merges with the
//    log-sum-exp rule.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxF = 8;  // frames per wavefront per partition

// Frames per pipeline step: two when a tile is 4 KiB or less (double-buffered K+V of two
// frames = 128 VGPRs), one for larger tiles.
template <int KIND, int D, int BS>
constexpr int step_frames() { return KvOps<KIND, D, BS>::NL <= 4 ? 2 : 1; }

template <int KIND>
struct QType {
  static constexpr int bytes = KIND == KF32 ? 4 : 2;
};

template <int KIND, int D, int BS, int WAVES, int MAXF, int F>
__global__ __launch_bounds__(WAVES * 64, 2) void decode_partition_kernel(
    void* __restrict__ out, const void* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, float* __restrict__ ws_ml,
    float* __restrict__ ws_o, int mbps, int Hq, int Hkv, int G, long long NB, int max_parts,
    int max_ctx, float qk_scale, float v_scale) {
  using Ops = KvOps<KIND, D, BS>;
  constexpr int NL = Ops::NL, KG = Ops::KG, NS = Ops::NS, NC = Ops::NC, QW = Ops::QW;
  constexpr int PB = WAVES * MAXF;
  constexpr int STEPS = MAXF / F;
  static_assert(MAXF % F == 0, "steps must tile the frames of a wavefront");
  constexpr int QB = QType<KIND>::bytes;

  __shared__ float sm_o[WAVES][16][D + 4];
  __shared__ float sm_m[WAVES][16];
  __shared__ float sm_l[WAVES][16];

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int w = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, j = lane >> 4, n = lane & 15;

  const int cap = min(max_ctx, mbps * BS);
  const int L = max(0, min(context_lens[b], cap));
  const int nblk = (L + BS - 1) / BS;
  const int blk0 = part * PB;
  if (blk0 >= nblk) return;
  const int nb_part = min(PB, nblk - blk0);
  const int nparts = (nblk + PB - 1) / PB;
  const int cnt = nb_part > w ? (nb_part - w + WAVES - 1) / WAVES : 0;

  // Query fragment of row n: dims (D/4)*j .. (D/4)*(j+1) of head g*G + n (zero if n >= G).
  uint32_t qw[QW];
  {
    const bool qv = n < G;
    const size_t row = (size_t)b * Hq + (size_t)g * G + (qv ? n : 0);
    const u32x4* src = (const u32x4*)((const char*)q + (row * D + (size_t)(D / 4) * j) * QB);
#pragma unroll
    for (int i = 0; i < QW / 4; ++i) {
      u32x4 x = src[i];
      if (!qv) x = (u32x4){0u, 0u, 0u, 0u};
      qw[4 * i] = x[0]; qw[4 * i + 1] = x[1]; qw[4 * i + 2] = x[2]; qw[4 * i + 3] = x[3];
    }
  }

  // Frame ids of this wavefront's blocks (scalar loads); invalid entries are skipped.
  int fid[MAXF];
#pragma unroll
  for (int i = 0; i < MAXF; ++i) {
    int f = -1;
    if (i < cnt) f = block_tables[(size_t)b * mbps + blk0 + w + i * WAVES];
    fid[i] = uniform((f >= 0 && (long long)f < NB) ? f : -1);
  }

  const size_t tile_stride = (size_t)Ops::TILE;
  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  u32x4 kA[F][NL], vA[F][NL], kB[F][NL], vB[F][NL];

  auto load_step = [&](u32x4 (&kt)[F][NL], u32x4 (&vt)[F][NL], int s) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = s * F + f;
      if (i < cnt && fid[i] >= 0) {
        const size_t off = ((size_t)fid[i] * Hkv + g) * tile_stride;
        const u32x4* kp = (const u32x4*)(k_cache + off) + lane;
        const u32x4* vp = (const u32x4*)(v_cache + off) + lane;
#pragma unroll
        for (int r = 0; r < NL; ++r) kt[f][r] = kp[r * 64];
#pragma unroll
        for (int r = 0; r < NL; ++r) vt[f][r] = vp[r * 64];
      }
    }
  };

  auto compute_step = [&](u32x4 (&kt)[F][NL], u32x4 (&vt)[F][NL], int s) {
    f32x4 sc[F][KG];
    float mx = -INFINITY;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = s * F + f;
      const bool live = i < cnt && fid[i] >= 0;
      const int valid = L - (blk0 + w + i * WAVES) * BS;  // keys of this frame inside the context
#pragma unroll
      for (int h = 0; h < KG; ++h) {
        f32x4 a = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (live) {
#pragma unroll
          for (int sl = 0; sl < NS; ++sl) a = Ops::qk(a, Ops::kop(kt[f], h, sl), Ops::qop(qw, sl));
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int key = 16 * h + 4 * j + ii;
          const float v = (live && key < valid) ? a[ii] * qk_scale : -INFINITY;
          sc[f][h][ii] = v;
          mx = fmaxf(mx, v);
        }
      }
      if (live && valid < BS) {
        // last frame of the context: clear V of the slots past it, so that whatever they
        // hold (weighted by probability 0) cannot reach the accumulator
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
    if (mnew == -INFINITY) return;  // nothing live in this step
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] *= alpha;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = s * F + f;
      if (!(i < cnt && fid[i] >= 0)) continue;
#pragma unroll
      for (int h = 0; h < KG; ++h) {
        f32x4 p;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) p[ii] = __builtin_amdgcn_exp2f(sc[f][h][ii] - mnew);
        const auto pf = Ops::pfrag(p, lsum);
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = Ops::pv(acc[c], Ops::vop(vt[f], h, c), pf);
      }
    }
  };

  load_step(kA, vA, 0);
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (s * F >= cnt) break;
    if ((s & 1) == 0) {
      if (s + 1 < STEPS) load_step(kB, vB, s + 1);
      compute_step(kA, vA, s);
    } else {
      if (s + 1 < STEPS) load_step(kA, vA, s + 1);
      compute_step(kB, vB, s);
    }
  }

  // Merge the wavefronts of the workgroup.
  const float lrow = wave_sum_over_j(lsum);
  if (n < G) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sm_o[w][n][16 * c + 4 * j + ii] = acc[c][ii];
    if (j == 0) {
      sm_m[w][n] = m;
      sm_l[w][n] = lrow;
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += WAVES * 64) {
    const int r = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2) M = fmaxf(M, sm_m[w2][r]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2) {
      const float mw = sm_m[w2][r];
      if (mw == -INFINITY) continue;
      const float e = __builtin_amdgcn_exp2f(mw - M);
      num += e * sm_o[w2][r][d];
      den += e * sm_l[w2][r];
    }
    const size_t h = (size_t)g * G + r;
    if (nparts == 1) {
      const float o = num / den * v_scale;
      if constexpr (KIND == KF32) {
        ((float*)out)[((size_t)b * Hq + h) * D + d] = o;
      } else {
        ((__bf16*)out)[((size_t)b * Hq + h) * D + d] = (__bf16)o;
      }
    } else {
      const size_t pi = ((size_t)b * Hq + h) * max_parts + part;
      ws_o[pi * D + d] = num;
      if (d == 0) {
        ws_ml[2 * pi] = M;
        ws_ml[2 * pi + 1] = den;
      }
    }
  }
}

// Merge the partitions of every sequence longer than one partition:
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
template <int KIND>
__global__ __launch_bounds__(128) void decode_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, int Hq, int D, int max_parts, int part_tokens,
    int cap, float v_scale) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = max(0, min(context_lens[b], cap));
  const int nparts = (L + part_tokens - 1) / part_tokens;
  if (nparts <= 1) return;
  const size_t base = ((size_t)b * Hq + h) * max_parts;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ws_ml[2 * (base + p)]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int p = 0; p < nparts; ++p) {
      const float mp = ws_ml[2 * (base + p)];
      if (mp == -INFINITY) continue;
      const float e = __builtin_amdgcn_exp2f(mp - M);
      num += e * ws_o[(base + p) * D + d];
      den += e * ws_ml[2 * (base + p) + 1];
    }
    const float o = num / den * v_scale;
    if constexpr (KIND == KF32) {
      ((float*)out)[((size_t)b * Hq + h) * D + d] = o;
    } else {
      ((__bf16*)out)[((size_t)b * Hq + h) * D + d] = (__bf16)o;
    }
  }
}

template <int KIND, int D, int BS>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  constexpr int PB = kWaves * kMaxF;
  const int nblk_max = (p.max_context_len + BS - 1) / BS;
  const int max_parts = (nblk_max + PB - 1) / PB;
  float* ws_ml = (float*)p.workspace;
  float* ws_o = ws_ml ? ws_ml + (size_t)2 * p.B * p.Hq * max_parts : nullptr;
  const int G = p.Hq / p.Hkv;
  const float qk_scale = p.scale * (KIND == KFP8 ? p.k_scale : 1.0f) * kLog2e;
  const float v_scale = KIND == KFP8 ? p.v_scale : 1.0f;
  dim3 grid(max_parts, p.Hkv, p.B);
  hipLaunchKernelGGL((decode_partition_kernel<KIND, D, BS, kWaves, kMaxF, step_frames<KIND, D, BS>()>), grid,
                     dim3(kWaves * 64), 0, stream, p.out, p.q, (const char*)p.k_cache,
                     (const char*)p.v_cache, p.block_tables, p.context_lens, ws_ml, ws_o,
                     p.max_blocks_per_seq, p.Hq, p.Hkv, G, (long long)p.NB, max_parts,
                     p.max_context_len, qk_scale, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_parts <= 1) return e;
  const int cap = p.max_context_len < p.max_blocks_per_seq * BS ? p.max_context_len
                                                                 : p.max_blocks_per_seq * BS;
  hipLaunchKernelGGL((decode_reduce_kernel<KIND>), dim3(p.Hq, p.B), dim3(D), 0, stream, p.out,
                     ws_ml, ws_o, p.context_lens, p.Hq, D, max_parts, PB * BS, cap, v_scale);
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

int decode_partition_tokens(int bs, int /*kv_dtype*/) { return kWaves * kMaxF * bs; }

size_t decode_workspace_bytes(int B, int Hq, int D, int bs, int kv_dtype, int max_context_len) {
  const int pt = decode_partition_tokens(bs, kv_dtype);
  const size_t max_parts = ((size_t)max_context_len + pt - 1) / pt;
  if (max_parts <= 1) return 0;
  return (size_t)B * Hq * max_parts * (2 + (size_t)D) * sizeof(float);
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
