// pa_prefill_impl.h -- the prefill-chunk tile and split-merge bodies shared by the prefill
// kernels and the mixed-batch kernel.  The work they do is described at the top of
// pa_prefill.hip.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace pre {

constexpr int kPWaves = 8;      // wavefronts per workgroup (one workgroup per compute unit)
constexpr float kLazy = 8.f;    // log2-domain slack before the running shift moves

// 16-row query tiles per wavefront (f32 operands take twice the registers).
constexpr int tiles_per_wave(int kind) { return kind == KF32 ? 1 : 2; }

template <int KIND>
struct PQ {
  static constexpr int bytes = KIND == KF32 ? 4 : 2;
};

// N consecutive LDS-DMA copies (global_load_lds_dwordx4) of 1 KiB blocks: block i is read at
// sbase + 1024 i and lands at lds + 1024 i, each lane's 16 bytes at the lane's offset voff in the
// block (voff = 16 lane).  sbase is wavefront-uniform (the instruction's scalar base); the
// instruction's immediate offset moves the global and the LDS address together, so one M0 and
// one base serve the N blocks.  Issued as assembly so that the compiler does not make unrelated
// LDS reads wait for the copies (the pipeline below waits for them itself); the kernels that use
// it leave M0 to it.
template <int N>
__device__ inline void lds_dma16_run(const char* sbase, uint32_t voff, uint32_t lds_addr) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 blocks");
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr);
  if constexpr (N == 1) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
                 "s"(sbase), "s"(base)
                 : "memory");
  } else if constexpr (N == 2) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024" ::"v"(voff), "s"(sbase), "s"(base)
                 : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:3072" ::"v"(voff), "s"(sbase), "s"(base)
                 : "memory");
  }
}

// The 32-bit LDS address of a pointer into a __shared__ buffer.
__device__ inline uint32_t lds_address(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// P^T fragment of four probabilities for the prefill tile.  bf16 / fp8 kinds: rounded to bf16
// for the matrix core, and the row sum taken over the fp32 values before rounding (four
// additions, no unpacking); the normalisation then differs from the rounded weights by a
// relative error of about 2^-9 / sqrt(keys), far below the bf16 output's own rounding.
template <int KIND, class Ops>
__device__ inline typename Ops::PFrag prefill_pfrag(f32x4 p, float& lsum) {
  if constexpr (KIND == KF32) {
    return Ops::pfrag(p, lsum);
  } else {
    u32x2 pp;
    pp[0] = pack_bf16x2(p[0], p[1]);
    pp[1] = pack_bf16x2(p[2], p[3]);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    return pp;
  }
}

// Keys per pipeline stage: 64 (32 for f32, whose tiles are twice as large: a ring of four 64-key
// stages would not fit LDS).  64-key stages halve the per-stage costs (the meeting point, the
// rescale decision, the masks) against 32-key ones: 3-10% faster on bf16 / fp8 chunks.
constexpr int stage_keys(int kind) { return kind == KF32 ? 32 : 64; }

// Bytes of K and V per stage in LDS.
template <int KIND, int D, int BS>
constexpr int prefill_stage_bytes() {
  return (stage_keys(KIND) / BS) * 2 * KvOps<KIND, D, BS>::TILE;
}

// fp8 stages are widened once to bf16 in LDS (two buffers of this size): the bytes of one
// widened stage, or a token size for the other kinds, which read their stages directly.
template <int KIND, int D, int BS>
constexpr int prefill_widened_bytes() {
  return KIND == KFP8 ? prefill_stage_bytes<KBF16, D, BS>() : 16;
}

// One workgroup's tile: context range x (keys [x KS, (x+1) KS)), query tile qt of chunk c, kv
// head g.  Rows are absolute rows of q / out; partials are indexed from row_base.  ring0..3 are
// the LDS stage buffers (prefill_stage_bytes each); wide0 / wide1 the widened fp8 stages
// (prefill_widened_bytes each).
template <int KIND, int D, int BS, int NT>
__device__ __forceinline__ void prefill_tile(
    char* ring0, char* ring1, char* ring2, char* ring3, char* wide0, char* wide1, int x, int qt,
    int c, int g,
    long long row_base, void* __restrict__ out, const void* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, int mbps, int Hq, int Hkv, int G,
    long long NB, long long total_q, int nsplit, int KS, int max_ctx, float qk_scale,
    float v_scale) {
  // fp8 tiles are staged as they are stored and widened once per stage into a bf16 copy (the
  // widening is exact), which the matrix-core code then reads like a bf16 cache's tiles: every
  // wavefront of the workgroup shares one conversion instead of repeating it in registers.
  constexpr bool WIDEN = KIND == KFP8;
  using Ops = KvOps<WIDEN ? KBF16 : KIND, D, BS>;  // operands as the matrix cores read them
  using OpsS = KvOps<KIND, D, BS>;                  // tiles as they are stored and staged
  constexpr int NL = Ops::NL, KG = Ops::KG, NS = Ops::NS, NC = Ops::NC, QW = Ops::QW;
  constexpr int TILE = Ops::TILE;
  constexpr int NLS = OpsS::NL, TILE_S = OpsS::TILE;
  constexpr int SK = stage_keys(KIND);   // keys per stage
  constexpr int SF = SK / BS;            // frames per stage
  constexpr int NG = SF * KG;            // 16-key groups per stage
  constexpr int STAGE = SF * 2 * TILE_S; // bytes of K and V per staged stage
  static_assert(NG % 2 == 0, "a stage is pairs of 16-key groups");
  static_assert(!WIDEN || (TILE == 2 * TILE_S && NL == 2 * NLS), "fp8 widens to twice the bytes");
  constexpr int QB = PQ<KIND>::bytes;

  static_assert(STAGE == prefill_stage_bytes<KIND, D, BS>(), "stage size");

  const int w = uniform(threadIdx.x >> 6) & (kPWaves - 1);  // (the mask tells the compiler w < 8)
  const int lane = threadIdx.x & 63, j = lane >> 4, n = lane & 15;

  const int r0 = qsl[c];
  const int C = qsl[c + 1] - r0;
  const int cap = min(max_ctx, mbps * BS);
  const int L = min(context_lens[c], cap);
  if (r0 < 0 || (long long)qsl[c + 1] > total_q || C <= 0 || C > L) return;
  const int TQ = kPWaves * NT * 16 / G;
  const int t0 = qt * TQ;
  if (t0 >= C) return;
  const int pos0 = L - C;
  const int tq_end = min(t0 + TQ, C);
  const int kbeg = x * KS;
  const int kend = min(kbeg + KS, pos0 + tq_end);
  if (kbeg >= kend) return;

  // Query fragments and positions of this wavefront's NT tiles.  A negative score scale is
  // moved into the query's sign bits (exact), so the scores scale by qk_abs >= 0 and a row's
  // maximum can be taken on the unscaled products.
  // (a zero scale is replaced by 1e-30: every product is then far below half an ulp of the
  // row shift, so each probability is still exactly 1, and -inf * qk_abs stays -inf)
  const float qk_abs = fmaxf(fabsf(qk_scale), 1e-30f);
  const uint32_t qsign = qk_scale < 0.f ? (KIND == KF32 ? 0x80000000u : 0x80008000u) : 0u;
  uint32_t qw[NT][QW];
  int rpos[NT];
  // The largest key every row of this wavefront's tiles may see: keys past it (past a tile's
  // first row, whose position is the tile's smallest, or at or past kend) need the mask.  A tile
  // past the chunk counts as position -1.
  int lim = kend - 1;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int qrow = (w * NT + t) * 16 + n;
    const int tok = t0 + qrow / G;
    const bool ok = tok < C;
    rpos[t] = ok ? pos0 + tok : -1;
    {
      const int tok0 = t0 + (w * NT + t) * 16 / G;
      lim = min(lim, tok0 < C ? pos0 + tok0 : -1);
    }
    const size_t row = (size_t)(r0 + (ok ? tok : 0)) * Hq + (size_t)g * G + qrow % G;
    const u32x4* src = (const u32x4*)((const char*)q + (row * D + (size_t)(D / 4) * j) * QB);
#pragma unroll
    for (int i = 0; i < QW / 4; ++i) {
      u32x4 v = src[i];
      if (!ok) v = (u32x4){0u, 0u, 0u, 0u};
      v ^= (u32x4){qsign, qsign, qsign, qsign};
      qw[t][4 * i] = v[0]; qw[t][4 * i + 1] = v[1]; qw[t][4 * i + 2] = v[2]; qw[t][4 * i + 3] = v[3];
    }
  }

  // m: each row's running shift; mth = m + kLazy (the bound a stage's scores are tested
  // against) and nm = -m (0 while m = -inf: the exponentials' offset) change only with m
  float m[NT], mth[NT], nm[NT], lsum[NT];
  f32x4 acc[NT][NC];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m[t] = -INFINITY;
    mth[t] = -INFINITY;
    nm[t] = 0.f;
    lsum[t] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) acc[t][cc] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  const int nst = (kend - kbeg + SK - 1) / SK;
  // the stage whose keys reach past kend (the last, unless the range is whole stages), or -1
  const int tail_st = (kend - kbeg) % SK ? nst - 1 : -1;
  const size_t trow = (size_t)c * mbps;

  // Staging of a stage: its K and V tiles are NBLK blocks of 1 KiB in the cache's tile
  // layout (a block holds one 16-byte fragment per lane), stored in LDS as [frame][K, V][block].
  // Wavefront w copies the BPW consecutive blocks w BPW, ..., all of one K or V tile, straight
  // from global memory into the stage's LDS buffer with LDS-DMA loads (lane l's 16 bytes land at
  // the block's base + 16 l): no register or LDS store of the wavefront carries them, and the
  // copy of a later stage runs while this one is computed.
  constexpr int NBLK = STAGE / 1024;
  constexpr int BPW = (NBLK + kPWaves - 1) / kPWaves;  // blocks per wavefront and stage
  static_assert(NBLK % kPWaves == 0 || NBLK < kPWaves, "stage blocks must split over waves");
  static_assert(NLS % BPW == 0, "a wavefront's blocks lie in one tile");
  static_assert(64 % SF == 0, "a stage's frames lie in one window of 64 block ids");
  // Block ids come in windows of 64 frames, one per lane, fetched one window ahead with a single
  // vector load: lane l of window wi loads the table entry of frame kbeg / BS + 64 wi + l (the
  // index clamped to the range's last frame, so the load needs no branch).  When a window
  // becomes current, its lanes turn their entries into tile indices f Hkv + g, or -1 for frames
  // past the range and ids outside the pool, in vector code once for its 64 frames; a stage then
  // only reads its frames' indices with readlane.  The one wait on a window's load lands a window
  // after the load was issued, and the next window is requested after the copies of the stage
  // that starts a window.  (The scalar unit is shared by the CU's eight wavefronts: the per-stage
  // copy issue is kept to a few scalar instructions per block.)
  const int F0 = kbeg / BS;
  const int Flast = (kend - 1) / BS;  // last frame of the range
  const int lane16 = lane * 16;       // byte offset of a lane's 16 bytes in a 1 KiB block
  const int nb32 = NB < 0x7fffffffLL ? (int)NB : 0x7fffffff;  // every valid id is below it
  auto load_window = [&](int wi) { return block_tables[trow + min(F0 + 64 * wi + lane, Flast)]; };
  auto tiles_of = [&](int raw, int wi) {
    const int fi = F0 + 64 * wi + lane;
    return (fi * BS < kend && raw >= 0 && raw < nb32) ? raw * Hkv + g : -1;
  };
  int win = 0;  // window held in tix_cur
  int tix_cur = tiles_of(load_window(0), 0);
  int raw_nxt = load_window(1);
  auto dma = [&](char* buf, int st) {
    const int wi = (st * SF) >> 6;
    const bool next = wi != win;  // wavefront-uniform; stages are copied in order
    if (next) {
      // (the empty statement keeps this a branch: as a select, the conversion would read
      // raw_nxt, a load the compiler cannot see completed, at every stage and wait there)
      asm volatile("");
      tix_cur = tiles_of(raw_nxt, wi);
      win = wi;
    }
    const int blk = w * BPW;  // (wavefront-uniform)
    if (NBLK >= kPWaves || blk < NBLK) {
      const int fl = blk / (2 * NLS), kind = (blk / NLS) & 1, r = blk % NLS;
      const int t = __builtin_amdgcn_readlane(tix_cur, (st * SF + fl) & 63);
      // frames past the range and invalid ids copy blocks of tile 0 instead (never used):
      // every stage issues the same copies, so the wait counts below hold
      const char* base = kind ? v_cache : k_cache;
      lds_dma16_run<BPW>(base + (size_t)(uint32_t)max(t, 0) * TILE_S + r * 1024, lane16,
                         lds_address(buf) + blk * 1024);
    }
    if (next) {
      // the window after the new one, requested after this stage's copies
      __builtin_amdgcn_sched_barrier(0);
      raw_nxt = load_window(wi + 1);
    }
  };
  // Wait until this wavefront's copies of every stage but the newest have landed in LDS, then
  // meet the other wavefronts (after which their copies have landed too).  Written as assembly:
  // the compiler's barrier would also wait for the newest stage's copies.
  auto sync_stage = [&]() {
    if (NBLK >= kPWaves || w < NBLK) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(BPW) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };

  // Scores of frames [f_lo, f_hi) of a stage (K from its LDS buffer).
  auto qk = [&](const char* sb, f32x4 (&s)[NT][NG], int f_lo, int f_hi) {
#pragma unroll
    for (int fl = f_lo; fl < f_hi; ++fl) {
      u32x4 kt[NL];
#pragma unroll
      for (int r = 0; r < NL; ++r)
        kt[r] = *((const u32x4*)(sb + 2 * fl * TILE + r * 1024) + lane);
#pragma unroll
      for (int h = 0; h < KG; ++h) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          f32x4 a = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sl = 0; sl < NS; ++sl) a = Ops::qk(a, Ops::kop(kt, h, sl), Ops::qop(qw[t], sl));
          s[t][fl * KG + h] = a;
        }
      }
    }
  };

  // Softmax and P.V of stage st (V from its LDS buffer).  `overlap(pp)` issues the score MFMAs
  // of part pp of the next stage next to the exponentials and P.V products of pair pp, so that
  // the matrix cores and the vector ALUs work side by side.
  auto finish = [&](int st, const char* sb, f32x4 (&s)[NT][NG], auto&& overlap) {
    const int key0 = kbeg + SK * st;
    // Online softmax per query row with a lazily moved shift: m[t] only moves (and the
    // accumulators are rescaled) when a row's stage maximum exceeds it by more than kLazy in
    // the log2 domain; otherwise the probabilities exp2(s - m) of the stage may exceed 1 (by at
    // most 2^kLazy), which changes neither the normalised result nor the fp32 accumulation.
    // One wavefront-uniform rescale decision per stage keeps the accumulators in place.  The
    // causal / range mask is applied only on stages that reach past a row's position or the
    // range end.
    if (key0 + SK - 1 > lim) {  // (wavefront-uniform; true from some stage on)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int key = key0 + 16 * gi + 4 * j + ii;
            s[t][gi][ii] = (key < kend && key <= rpos[t]) ? s[t][gi][ii] : -INFINITY;
          }
    }
    // A row's stage maximum exceeds m + kLazy exactly when the maximum over one of its lanes'
    // keys does (scaling by qk_abs > 0 keeps the order), so the decision is taken on each lane's
    // own maximum, and the maxima are reduced across the row's lanes only on the stages where the
    // shift moves.
    float lmx[NT];
    bool grow = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) mx = fmaxf(mx, s[t][gi][ii]);
      lmx[t] = mx;
      grow = grow || mx * qk_abs > mth[t];  // (-inf * qk_abs is -inf: never grows)
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float mx = wave_max_over_j(lmx[t]);
        mx = mx == -INFINITY ? -INFINITY : mx * qk_abs;  // scores scale by qk_abs >= 0
        const float mnew = fmaxf(m[t], mx);
        const float alpha = m[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[t] - mnew);
        m[t] = mnew;
        mth[t] = mnew + kLazy;
        nm[t] = mnew == -INFINITY ? 0.f : -mnew;
        lsum[t] *= alpha;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) acc[t][cc] *= alpha;
      }
    }
    // Per pair of 16-key groups: the score products of the next stage's frames that the pair's
    // index selects (`overlap`), the pair's exponentials, and its P.V products.  The compiler
    // interleaves the score products with the exponentials (and the P.V products of a pair with
    // the next pair's work); splitting the stage into pairs keeps the registers in flight to
    // about one pair's worth (the whole stage as one block spills).
    const bool tail = st == tail_st;  // (key0 + SK > kend)
    // P * V over pairs of 16-key groups (one 16x16x32 product each); with 16-key frames the two
    // groups are two frames, with 32-key frames the two halves of one
#pragma unroll
    for (int pp = 0; pp < NG / 2; ++pp) {
      overlap(pp);
      typename Ops::PFrag pf[NT][2];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 p;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            // a masked score is -inf and qk_abs > 0: its probability is exactly 0
            p[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * pp + h][ii], qk_abs, nm[t]));
          }
          pf[t][h] = prefill_pfrag<KIND, Ops>(p, lsum[t]);
        }
      }
      constexpr int FPP = KG == 1 ? 2 : 1;  // frames per pair
      u32x4 vt[FPP][NL];
#pragma unroll
      for (int fl = 0; fl < FPP; ++fl)
#pragma unroll
        for (int r = 0; r < NL; ++r)
          vt[fl][r] = *((const u32x4*)(sb + (2 * (pp * FPP + fl) + 1) * TILE + r * 1024) + lane);
      if (tail) {
        // keys past the range end may be unwritten slots: clear their values
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gi = 2 * pp + h;
          const int keep = min(4, max(0, kend - (key0 + 16 * gi + 4 * j)));
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) Ops::zero_quad(vt[h / KG], h % KG, cc, keep);
        }
      }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const auto va = Ops::vop(vt[0], 0, cc);
        const auto vb = Ops::vop(vt[1 / KG], 1 % KG, cc);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][cc] = Ops::pv2(acc[t][cc], va, vb, pf[t][0], pf[t][1]);
      }
    }
  };

  // Software pipeline over a ring of four LDS stage buffers: while the softmax and P.V of stage
  // st run on the vector ALUs, the score MFMAs of stage st + 1 are already issued and the copies
  // of stages st + 2 and st + 3 are in flight.  Stage st + 3 goes into the buffer of stage st - 1,
  // which every wavefront finished reading before the previous meeting point.
  //
  // fp8: a staged stage is widened into the bf16 buffer wide[st % 2] by all wavefronts together
  // (wavefront w takes blocks w, w + 8, ...).  A lane's 16 bytes of fp8 block r of a K or V tile
  // widen, in order, to its 16 bytes of bf16 blocks 2r and 2r + 1 of the same tile in the bf16
  // layout.  Stage st + 1 is widened at the start of stage st: its copies landed before the
  // previous meeting point, and the buffer it overwrites held stage st - 1, which every wavefront
  // finished reading before that meeting point.  A second meeting point then publishes it.
  auto widen = [&](const char* staged, char* wide) {
    if constexpr (WIDEN) {
      constexpr int WPW = (NBLK + kPWaves - 1) / kPWaves;  // blocks per wavefront
#pragma unroll
      for (int k = 0; k < WPW; ++k) {
        const int blk = w + k * kPWaves;
        if (NBLK < kPWaves && blk >= NBLK) break;  // wavefront-uniform
        const int fl = blk / (2 * NLS), kind = (blk / NLS) & 1, r = blk % NLS;
        const u32x4 x8 = *((const u32x4*)(staged + blk * 1024) + lane);
        const u32x2 a = fp8x4_to_bf16x4(x8[0]), b = fp8x4_to_bf16x4(x8[1]);
        const u32x2 c2 = fp8x4_to_bf16x4(x8[2]), d2 = fp8x4_to_bf16x4(x8[3]);
        char* dst = wide + (2 * fl + kind) * TILE + 2 * r * 1024;
        *((u32x4*)dst + lane) = (u32x4){a[0], a[1], b[0], b[1]};
        *((u32x4*)(dst + 1024) + lane) = (u32x4){c2[0], c2[1], d2[0], d2[1]};
      }
    }
  };
  auto publish = [&]() {
    if constexpr (WIDEN) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  dma(ring0, 0);
  dma(ring1, 1);
  dma(ring2, 2);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  f32x4 sa[NT][NG], sz[NT][NG];
  widen(ring0, wide0);
  publish();
  qk(WIDEN ? wide0 : ring0, sa, 0, SF);
  // one stage: copy stage st + 3 into the buffer stage st - 1 used, finish stage st (its scores
  // in s_cur) while the scores of stage st + 1 go into s_nxt, meet
  auto stage = [&](int st, const char* cur, const char* nxt, char* free_buf, f32x4 (&s_cur)[NT][NG],
                   f32x4 (&s_nxt)[NT][NG]) {
    dma(free_buf, st + 3);
    if constexpr (WIDEN) {
      char* wcur = (st & 1) ? wide1 : wide0;
      char* wnxt = (st & 1) ? wide0 : wide1;
      widen(nxt, wnxt);
      publish();
      cur = wcur;
      nxt = wnxt;
    }
    // (past the last stage the next-stage scores read a buffer already written and are never
    // used: issuing them unconditionally keeps them in the exponentials' block)
    // the next stage's frames scored while pair pp of this stage is finished
    constexpr int FQ = 2 * SF / NG;
    auto next_scores = [&](int pp) { qk(nxt, s_nxt, pp * FQ, (pp + 1) * FQ); };
    finish(st, cur, s_cur, next_scores);
    sync_stage();
  };
  for (int st = 0; st < nst; st += 4) {
    stage(st, ring0, ring1, ring3, sa, sz);
    if (st + 1 >= nst) break;
    stage(st + 1, ring1, ring2, ring0, sz, sa);
    if (st + 2 >= nst) break;
    stage(st + 2, ring2, ring3, ring1, sa, sz);
    if (st + 3 >= nst) break;
    stage(st + 3, ring3, ring0, ring2, sz, sa);
  }
  // copies of stages past the last are still in flight: let them land before the buffers are
  // reused or the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Results: direct output for rows covered by a single key range, partials otherwise.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lrow = wave_sum_over_j(lsum[t]);
    if (rpos[t] < kbeg) continue;  // no key of this range is visible to the row
    const int qrow = (w * NT + t) * 16 + n;
    const size_t r = (size_t)r0 + (rpos[t] - pos0);
    const size_t h = (size_t)g * G + qrow % G;
    const int nsp = min(nsplit, rpos[t] / KS + 1);
    if (nsp == 1) {
      const float inv = v_scale / lrow;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const size_t o = (r * Hq + h) * D + 16 * cc + 4 * j;
        if constexpr (KIND == KF32) {
          *(f32x4*)((float*)out + o) = acc[t][cc] * inv;
        } else {
          u32x2 pk;
          pk[0] = pack_bf16x2(acc[t][cc][0] * inv, acc[t][cc][1] * inv);
          pk[1] = pack_bf16x2(acc[t][cc][2] * inv, acc[t][cc][3] * inv);
          *(u32x2*)((__bf16*)out + o) = pk;
        }
      }
    } else {
      const size_t pi = ((r - row_base) * Hq + h) * nsplit + x;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) *(f32x4*)(ws_o + pi * D + 16 * cc + 4 * j) = acc[t][cc];
      if (j == 0) {
        ws_ml[2 * pi] = m[t];
        ws_ml[2 * pi + 1] = lrow;
      }
    }
  }
}

// Merge the context splits of every (row, head) whose keys span more than one split:
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.  Each half of a wavefront
// takes one (row, head) pair (wavefront wv: pairs 2 wv and 2 wv + 1), so that every pair of a
// chunk is in flight at once; lane l of the half merges head-dim elements [l NV, (l+1) NV)
// with 16- (or 8-) byte loads.  kBatch partials of a pair are loaded before any is used.
template <int KIND, int D>
__device__ __forceinline__ void prefill_reduce_wave(
    long long wv, int lane, long long row_base, void* __restrict__ out, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_o, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ context_lens, int num_chunks, long long total_q, int Hq, int nsplit,
    int KS, int cap, float v_scale) {
  constexpr int NV = D / 32;   // outputs per lane (4 or 2)
  constexpr int kBatch = 4;    // partials held in registers at once
  typedef float fv __attribute__((ext_vector_type(NV)));
  const long long pair = 2 * wv + (lane >> 5);
  const int l = lane & 31;
  if (pair >= (total_q - row_base) * Hq) return;
  const long long r = row_base + pair / Hq;
  const int h = (int)(pair % Hq);
  int lo = 0, hi = num_chunks - 1;  // last chunk c with qsl[c] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (qsl[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int c = lo;
  const int C = qsl[c + 1] - qsl[c];
  const int L = min(context_lens[c], cap);
  if (r < qsl[c] || r >= qsl[c + 1] || C <= 0 || C > L) return;
  const int pos = L - C + (int)(r - qsl[c]);
  const int nsp = min(nsplit, pos / KS + 1);
  if (nsp <= 1) return;
  const size_t base = (size_t)pair * nsplit;
  float M = -INFINITY, den = 0.f;
  fv num = (fv)0.f;
  for (int p0 = 0; p0 < nsp; p0 += kBatch) {
    float mp[kBatch], lp[kBatch];
    fv op[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const bool has = p0 + i < nsp;
      const size_t q = base + (has ? p0 + i : 0);
      mp[i] = has ? ws_ml[2 * q] : -INFINITY;
      lp[i] = has ? ws_ml[2 * q + 1] : 0.f;
      op[i] = has ? *(const fv*)(ws_o + q * D + l * NV) : (fv)0.f;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (mp[i] == -INFINITY) continue;
      if (mp[i] > M) {
        const float sc = __builtin_amdgcn_exp2f(M - mp[i]);
        den *= sc;
        num *= sc;
        M = mp[i];
      }
      const float e = __builtin_amdgcn_exp2f(mp[i] - M);
      den += e * lp[i];
      num += e * op[i];
    }
  }
  const size_t o = ((size_t)r * Hq + h) * D + l * NV;
  const fv x = num / den * v_scale;
  if constexpr (KIND == KF32) {
    *(fv*)((float*)out + o) = x;
  } else {
#pragma unroll
    for (int v = 0; v < NV; v += 2) *(uint32_t*)((__bf16*)out + o + v) = pack_bf16x2(x[v], x[v + 1]);
  }
}

struct Split {
  int nsplit, KS;
};

// Split partials of `pairs` (row, head) pairs over nsplit ranges: the (max, sum) pairs, then the
// accumulator rows from a 16-byte boundary.
inline size_t partial_ml_floats(long long pairs, int nsplit) {
  return ((size_t)2 * pairs * nsplit + 3) / 4 * 4;
}
inline size_t partial_bytes(long long pairs, int nsplit, int D) {
  return (partial_ml_floats(pairs, nsplit) + (size_t)pairs * nsplit * D) * sizeof(float);
}

// Context split of a launch that aims for `target` workgroups: nsplit key ranges of KS keys
// (a multiple of 64, at least 256 keys per range unless the context is shorter).
inline Split choose_split(int num_chunks, int max_chunk_len, int max_ctx, int Hq, int Hkv, int kind,
                          int target) {
  const int G = Hq / Hkv;
  const int TQ = kPWaves * tiles_per_wave(kind) * 16 / G;
  const long long tiles = (long long)num_chunks * ((max_chunk_len + TQ - 1) / TQ) * Hkv;
  int want = (int)((target + tiles - 1) / (tiles > 0 ? tiles : 1));
  const int most = (max_ctx + 255) / 256;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int KS = (max_ctx + want - 1) / want;
  KS = ((KS + 63) / 64) * 64;
  if (KS < 64) KS = 64;
  return Split{(max_ctx + KS - 1) / KS, KS};
}

}  // namespace pre
}  // namespace pa
