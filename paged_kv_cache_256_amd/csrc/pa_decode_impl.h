// pa_decode_impl.h -- the decode stream and merge bodies shared by the decode kernels and the
// mixed-batch kernel (one wavefront's work each; the kernels only map hardware ids onto them).
// The decomposition they implement is described at the top of pa_decode.hip.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

#include <type_traits>

namespace pa {
namespace dec {

constexpr int kWaves = 4;    // wavefronts per workgroup (each an independent worker)
constexpr int kWgPerCu = 2;  // register budget: two workgroups per CU (256 VGPRs a wavefront)
constexpr int kIds = 64;     // block ids fetched per vector load

// Wavefronts of a decode launch per compute unit.  Measured on MI355X over the 8B / 70B shapes,
// bf16 and fp8: 3 per CU (192 four-wavefront workgroups on 256 CUs, 24 per XCD) streams 4-6%
// faster than 8 per CU; with 8 per CU some 64 MB of tile loads are in flight, far past what HBM
// needs to stay busy, and the excess only queues.  Launches whose workgroups do not spread evenly
// over the CUs (5 or 6 per CU) are 10-15% slower.
constexpr int kStreamWavesPerCu = 3;

inline int stream_waves() {
  const int w = device_compute_units() * kStreamWavesPerCu / kWaves * kWaves;
  return w > kWaves ? w : kWaves;
}

// Cost units of a (sequence, kv head) run of nblk frames: one per frame plus kRestart for the
// run's fixed start-up cost (its query, block ids and first tiles arrive a few memory latencies
// after the run starts, about four frames of a wavefront's streaming time at 3 wavefronts per CU;
// 3 to 6 measure alike and 1.5% faster than 2 over four 70B-shape batches).
constexpr int kRestart = 4;

// log2-domain slack before a run's running shift moves (its accumulators are then rescaled)
constexpr float kLazyShift = 8.f;
__host__ __device__ inline int run_units(int nblk) { return nblk > 0 ? nblk + kRestart : 0; }

// Tile loads: non-temporal (not retained in the caches) when every frame is read once per call;
// ordinary loads when frames are shared between sequences of the batch (copy-on-write branches,
// cached prefixes), so that the sequences after the first find them in L2 / the MALL.
template <bool NONTEMPORAL>
__device__ inline u32x4 load_tile16(const u32x4* p) {
  if constexpr (NONTEMPORAL) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

// Frames per pipeline step: two when a tile is 4 KiB or less (double-buffered K+V of two frames
// = 128 VGPRs), one for larger tiles.
template <int KIND, int D, int BS>
constexpr int step_frames() { return KvOps<KIND, D, BS>::NL <= 4 ? 2 : 1; }

template <int KIND>
struct QType {
  static constexpr int bytes = KIND == KF32 ? 4 : 2;
};

// The plan of a launch: plan[0] = U, the cost units of one kv head summed over the batch (the
// launch holds F = Hkv * U units), then from plan[4] one int4 per wavefront w: the run (b, g)
// holding unit a_w = floor(F w / W), the unit u of that run at which a_w falls, and the run's
// unit count su.

// Start of wavefront w found inside the wavefront itself (batches of at most kInlinePlanMax
// sequences): lane l sums the units of sequences [l*per, (l+1)*per), a wave-wide scan gives every
// lane its offset, a ballot finds the lane holding unit a_w / Hkv and a walk over its (at most 16)
// sequences finds the run.
constexpr int kInlinePlanMax = 1024;

struct Start {
  int b, g, u, su;
  long long F;
};

// Runs of a batch whose sequences share the first frames of their block tables (the GROUPED
// variant of the bodies below; branches of one prompt).  size[b] >= 1 starts a run of the
// consecutive sequences [b, b + size[b]); size[b] = 0 marks a sequence inside a run.  The members
// of a run share their first shared[b] block-table entries (0 for a run of one), and their G
// query heads each take G of the 16 columns of the score tile: the run streams the shared frames
// once for all members, then each member's own frames with the other members' columns masked.
struct Runs {
  const int32_t* size;
  const int32_t* shared;
};

__host__ __device__ inline int blocks_of(const int32_t* __restrict__ context_lens, int b, int cap,
                                         int BS) {
  return (max(0, min(context_lens[b], cap)) + BS - 1) / BS;
}

// Frames of the run that sequence b leads: its blocks, plus every other member's blocks after the
// shared ones (0 if b is inside another run).
template <bool GROUPED>
__device__ inline int run_frames(const int32_t* __restrict__ context_lens, int b, int B, int cap,
                                 int BS, Runs runs) {
  const int nb = blocks_of(context_lens, b, cap, BS);
  if constexpr (!GROUPED) {
    return nb;
  } else {
    const int sz = runs.size[b];
    if (sz <= 0) return 0;
    const int P = runs.shared[b];
    int n = nb;
    for (int mm = 1; mm < sz && b + mm < B; ++mm) n += blocks_of(context_lens, b + mm, cap, BS) - P;
    return n;
  }
}

// GROUPED order: the runs are taken in blocks of grouped_block(B) consecutive sequences, and
// inside a block head by head: (block, g, run).  The runs of one block -- branches of one prompt
// when the batch holds a prompt's branches next to each other -- then sit next to each other for
// each kv head, so the wavefronts that stream them at the same time read the same shared frames
// (an L2 hit for all but the first).  The block is a lane's sequences in the in-wavefront plan
// and a thread's in the plan kernel.
__host__ __device__ inline int grouped_block(int B) {
  return B <= kInlinePlanMax ? max(8, (B + 63) / 64) : (B + 1023) / 1024;
}

template <bool GROUPED = false>
__device__ inline Start wave_plan(const int32_t* __restrict__ context_lens, int B, int Hkv, int BS,
                                  int cap, int W, int w, int lane, Runs runs = Runs{}) {
  constexpr int kPer = kInlinePlanMax / 64;
  const int per = GROUPED ? grouped_block(B) : (B + 63) / 64;
  int un[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int bb = lane * per + i;
    un[i] = (i < per && bb < B) ? run_units(run_frames<GROUPED>(context_lens, bb, B, cap, BS, runs))
                                : 0;
    mine += un[i];
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  const int U = __builtin_amdgcn_readlane(incl, 63);
  const int ex = incl - mine;
  Start st;
  st.F = (long long)Hkv * U;
  const long long aw = st.F * w / W;
  const int ap = (int)(aw / Hkv);
  // lanes whose first offset is <= ap form a prefix; the last of them holds unit ap
  const int k = __popcll(__ballot(ex <= ap)) - 1;
  int cc = __builtin_amdgcn_readlane(ex, k);
  int bb = k * per, su = 0;
  if constexpr (GROUPED) {
    // (block k, head g, run): unit aw lies Hkv ex_k + g U_k + (the block's runs before it) in
    const int Uk = __builtin_amdgcn_readlane(mine, k);  // > 0: lane k holds unit ap
    const int rem = (int)(aw - (long long)Hkv * cc);
    const int off = Uk > 0 ? rem % Uk : 0;
    int c2 = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (i < per && bb < B) {
        su = __builtin_amdgcn_readlane(un[i], k);
        if (off < c2 + su) break;
        c2 += su;
        ++bb;
      }
    }
    st.b = bb;
    st.g = Uk > 0 ? rem / Uk : 0;
    st.u = off - c2;
    st.su = su;
    return st;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (i < per && bb < B) {
      su = __builtin_amdgcn_readlane(un[i], k);
      if (ap < cc + su) break;
      cc += su;
      ++bb;
    }
  }
  const int off = (int)(aw - (long long)Hkv * cc);
  st.b = bb;
  st.g = su > 0 ? off / su : 0;
  st.u = su > 0 ? off % su : 0;
  st.su = su;
  return st;
}

__device__ inline long long range_begin(long long F, int w, int W) { return F * w / W; }

// The work of wavefront w out of the W wavefronts that split the batch.  (GROUPED: the units are
// the runs of `runs` instead of single sequences.)
template <int KIND, int D, int BS, int F, bool NT, bool GROUPED = false>
__device__ __forceinline__ void decode_stream_wave(
    int w, int W, void* __restrict__ out, const void* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t* __restrict__ plan, bool inline_plan,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, int B, int mbps, int Hq, int Hkv, int G,
    long long NB, int cap, float qk_scale, float v_scale, Runs runs = Runs{},
    bool aligned = false) {
  using Ops = KvOps<KIND, D, BS>;
  constexpr int NL = Ops::NL, KG = Ops::KG, NS = Ops::NS, NC = Ops::NC, QW = Ops::QW;
  constexpr int NGS = F * KG;  // 16-key groups per step
  constexpr int QB = QType<KIND>::bytes;
  constexpr size_t TILE = Ops::TILE;

  const int lane = threadIdx.x & 63, j = lane >> 4, n = lane & 15;

  long long a, e;  // the wavefront's units [a, e)
  int b, g, u;  // u: unit within the run
  if (aligned) {
    // one run per wavefront: run (b, g) = (w / Hkv, w % Hkv), whole; its first unit is Hkv times
    // the units of the sequences before b, plus g runs of b
    b = w / Hkv;
    g = w - b * Hkv;
    u = 0;
    if (b >= B) return;
    int pre = 0;
    for (int bb = lane; bb < b; bb += 64) pre += run_units(blocks_of(context_lens, bb, cap, BS));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pre += __shfl_xor(pre, off);
    const int su = run_units(blocks_of(context_lens, b, cap, BS));
    a = (long long)Hkv * uniform(pre) + (long long)g * su;
    e = a + su;
  } else {
    long long Ftot;
    if (inline_plan) {
      const Start st = wave_plan<GROUPED>(context_lens, B, Hkv, BS, cap, W, w, lane, runs);
      Ftot = st.F;
      b = st.b;
      g = st.g;
      u = st.u;
      if (lane == 0) {
        ((int4*)(plan + 4))[w] = make_int4(st.b, st.g, st.u, st.su);
        if (w == 0) plan[0] = (int)(Ftot / Hkv);
      }
    } else {
      Ftot = (long long)Hkv * plan[0];
      const int4 st = ((const int4*)(plan + 4))[w];
      b = uniform(st.x);
      g = uniform(st.y);
      u = uniform(st.z);
    }
    a = range_begin(Ftot, w, W);
    e = range_begin(Ftot, w + 1, W);
  }
  if (a >= e) return;

  // Scores scale by qk_abs >= 0; a negative scale goes into the query's sign bits (exact).  (A zero
  // scale is replaced by 1e-30: every product is then far below half an ulp of the shift, so each
  // probability is exactly 1, and -inf * qk_abs stays -inf.)
  const float qk_abs = fmaxf(fabsf(qk_scale), 1e-30f);
  const uint32_t qsign = qk_scale < 0.f ? (KIND == KF32 ? 0x80000000u : 0x80008000u) : 0u;
  // m: the running shift of the scaled scores (lazily moved); mth = m + kLazyShift, and nm = -m
  // (0 while m = -inf), the exponentials' offset, change only with m
  float m = -INFINITY, mth = -INFINITY, nm = 0.f, lsum = 0.f;
  f32x4 acc[NC];
  uint32_t qw[QW];

  // frame ids of the current chunk (one per lane) and the lane stride of their loads: 1 for a
  // live frame, 0 for a dead one (past the chunk, or an invalid id), which then reads the same
  // 16 bytes of frame 0 in every lane -- the load stays unconditional but moves no tile
  int vfid = 0, vstride = 0;
  uint64_t live_mask = 0;
  int L = 0, cblk = 0;  // context length and first block of the current chunk
  int col0 = 0, col1 = 16;  // GROUPED: score columns (member heads) the current chunk is for

  // Gather step s of a chunk whose frame ids (one per lane) and lane strides are fid / fstride,
  // for kv head gg.
  auto load_step = [&](u32x4 (&kt)[F][NL], u32x4 (&vt)[F][NL], int s, int fid, int fstride, int gg) {
    // keep a step's loads together and in order: the in-order load counter then lets the
    // compute of the previous step wait for exactly its own data
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = min(s * F + f, 63);
      const int fr = __builtin_amdgcn_readlane(fid, i);
      // the tile's address is wavefront-uniform and a lane's offset is 16 lane or 0: the loads
      // take the tile address as their scalar base
      const uint32_t off = __builtin_amdgcn_readlane(fstride, i) ? 16u * (uint32_t)lane : 0u;
      const char* kb = k_cache + ((size_t)fr * Hkv + gg) * TILE + off;
      const char* vb = v_cache + ((size_t)fr * Hkv + gg) * TILE + off;
#pragma unroll
      for (int r = 0; r < NL; ++r) kt[f][r] = load_tile16<NT>((const u32x4*)(kb + r * 1024));
#pragma unroll
      for (int r = 0; r < NL; ++r) vt[f][r] = load_tile16<NT>((const u32x4*)(vb + r * 1024));
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Consume step s of the current chunk.  No loads in here: the only branch between a step's
  // loads and this use is the loop back-edge, so the next step's loads stay in flight.
  // Online softmax with a lazily moved shift: the accumulators are rescaled only when a step's
  // scaled scores exceed m + kLazyShift (log2 domain); otherwise the step's probabilities
  // exp2(s - m) may exceed 1 by at most 2^kLazyShift, which changes neither the normalised result
  // nor the fp32 accumulation.  A row's step maximum exceeds the bound exactly when one of its
  // lanes' does (scaling by qk_abs > 0 keeps the order), so each lane tests its own maximum and
  // the row maxima are reduced across lanes only on the steps where the shift moves.  Keys are
  // masked only in frames that need it (the context's last frame, dead frames, and member
  // columns of a grouped run).
  auto compute_step = [&](u32x4 (&kt)[F][NL], u32x4 (&vt)[F][NL], int s) {
    f32x4 sc[NGS];
    float lmx = -INFINITY;
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
        sc[f * KG + h] = sv;
      }
      const bool cols = GROUPED && (col0 > 0 || col1 < 16);  // (wavefront-uniform)
      if (valid < BS || cols) {
#pragma unroll
        for (int h = 0; h < KG; ++h)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            bool keep = 16 * h + 4 * j + ii < valid;
            if constexpr (GROUPED) keep = keep && n >= col0 && n < col1;
            sc[f * KG + h][ii] = keep ? sc[f * KG + h][ii] : -INFINITY;
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
#pragma unroll
      for (int h = 0; h < KG; ++h)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) lmx = fmaxf(lmx, sc[f * KG + h][ii]);
    }
    if (__builtin_amdgcn_ballot_w64(lmx * qk_abs > mth)) {  // (-inf * qk_abs is -inf: no move)
      float mx = wave_max_over_j(lmx);
      mx = mx == -INFINITY ? -INFINITY : mx * qk_abs;
      const float mnew = fmaxf(m, mx);
      // a row (GROUPED: a member's column) that has seen no key keeps m = -inf, shifts by 0 and
      // gets probabilities exp2(-inf) = 0
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      mth = mnew + kLazyShift;
      nm = mnew == -INFINITY ? 0.f : -mnew;
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] *= alpha;
    }
    typename Ops::PFrag pf[NGS];
#pragma unroll
    for (int gi = 0; gi < NGS; ++gi) {
      f32x4 p;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) p[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[gi][ii], qk_abs, nm));
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

  // The wavefront's frames are visited as chunks of up to kIds consecutive frames of one run
  // piece (the frames of a (sequence, kv head) run that lie in this wavefront's range).  The tile
  // pipeline runs on across chunk and run boundaries: while a chunk is computed, the block ids
  // and the query of the next chunk are fetched, and the chunk's last two load steps gather the
  // next chunk's first two steps (in place of loads past the chunk), so the wavefront keeps two
  // steps of tiles in flight from its first frame to its last.
  struct Piece {
    int b, g, L, nblk, f0, n, slot;
    int sz, P;  // GROUPED: members of the run and their shared blocks
    bool complete;
  };
  long long x = a;  // first unit of the next run to look at
  int rb = b, rg = g, ru = u;
  const int gblk = grouped_block(B);  // (GROUPED order)
  // The next run piece with frames in [x, e), or false past the end of the range.
  auto find_piece = [&](Piece& pc) -> bool {
    while (x < e && rb < B) {
      const int Lr = max(0, min(context_lens[rb], cap));
      const int nb = GROUPED ? run_frames<GROUPED>(context_lens, rb, B, cap, BS, runs)
                             : (Lr + BS - 1) / BS;
      const int units = (int)min((long long)(run_units(nb) - ru), e - x);
      // frames of the run inside this wavefront's range (its first kRestart units hold none)
      const int f0 = max(0, ru - kRestart), f1 = min(nb, ru + units - kRestart);
      const long long s0 = x - ru;  // first unit of this (b, g) run
      const int pb = rb, pg = rg;
      x += units > 0 ? units : 0;
      ru = 0;
      if constexpr (GROUPED) {
        // the block's next run for this head, else its first run for the next head, else the
        // next block
        const int blk0 = pb / gblk * gblk, blk1 = min(B, blk0 + gblk);
        if (++rb == blk1) {
          if (++rg == Hkv) {
            rg = 0;
          } else {
            rb = blk0;
          }
        }
      } else {
        if (++rg == Hkv) {
          rg = 0;
          ++rb;
        }
      }
      if (f1 > f0) {
        pc.b = pb;
        pc.g = pg;
        pc.L = Lr;
        pc.nblk = nb;
        pc.f0 = f0;
        pc.n = f1 - f0;
        pc.complete = f0 == 0 && f1 == nb;
        pc.slot = s0 > a ? 1 : 0;
        if constexpr (GROUPED) {
          pc.sz = runs.size[pb];
          pc.P = runs.shared[pb];
        }
        return true;
      }
    }
    return false;
  };
  // Raw block id of lane `lane` of chunk c0 of piece pc (clamped to the run's last block).
  auto chunk_id = [&](const Piece& pc, int c0) {
    return block_tables[(size_t)pc.b * mbps + min(pc.f0 + c0 + lane, pc.nblk - 1)];
  };
  // GROUPED: a chunk is up to kIds frames of one table row -- the shared frames (read from the
  // first member's row, for every member's columns) or one member's own frames (its columns).
  struct Chunk {
    int row, blk0, len, L, col0, col1;
  };
  auto chunk_of = [&](const Piece& pc, int c0) {
    Chunk ch;
    const int x = pc.f0 + c0;  // frame of the run
    int end;
    if (x < pc.P) {
      ch.row = pc.b;
      ch.blk0 = x;
      end = pc.P;
      ch.L = pc.L;
      ch.col0 = 0;
      ch.col1 = 16;
    } else {
      int cum = pc.P, mm = 0, nbm = 0;
      for (; mm < pc.sz && pc.b + mm < B; ++mm) {
        nbm = blocks_of(context_lens, pc.b + mm, cap, BS);
        if (x < cum + nbm - pc.P) break;
        cum += nbm - pc.P;
      }
      mm = min(mm, min(pc.sz, B - pc.b) - 1);
      ch.row = pc.b + mm;
      ch.blk0 = pc.P + (x - cum);
      end = cum + nbm - pc.P;
      ch.L = max(0, min(context_lens[pc.b + mm], cap));
      ch.col0 = mm * G;
      ch.col1 = (mm + 1) * G;
    }
    ch.len = max(1, min(kIds, min(pc.n - c0, end - x)));
    return ch;
  };
  auto chunk_id_of = [&](const Chunk& ch) {
    return block_tables[(size_t)ch.row * mbps + max(0, min(ch.blk0 + min(lane, ch.len - 1), mbps - 1))];
  };
  // query fragment of row n: dims (D/4)*j .. of head g*G + n (zero if n >= G); GROUPED: column n
  // is head n % G of member n / G
  auto load_q = [&](uint32_t (&dst)[QW], const Piece& pc) {
    const bool qv = GROUPED ? n < pc.sz * G && pc.b + n / G < B : n < G;
    const size_t row = GROUPED ? (size_t)(pc.b + (qv ? n / G : 0)) * Hq + (size_t)pc.g * G + (qv ? n % G : 0)
                               : (size_t)pc.b * Hq + (size_t)pc.g * G + (qv ? n : 0);
    const u32x4* src = (const u32x4*)((const char*)q + (row * D + (size_t)(D / 4) * j) * QB);
#pragma unroll
    for (int i = 0; i < QW / 4; ++i) {
      u32x4 v4 = src[i];
      if (!qv) v4 = (u32x4){0u, 0u, 0u, 0u};
      v4 ^= (u32x4){qsign, qsign, qsign, qsign};
      dst[4 * i] = v4[0]; dst[4 * i + 1] = v4[1]; dst[4 * i + 2] = v4[2]; dst[4 * i + 3] = v4[3];
    }
  };
  // ids of a chunk: live lanes (inside the chunk, valid id) load their frame, dead ones read the
  // same 16 bytes of frame 0 (stride 0)
  auto resolve = [&](int f_raw, int cn, bool any, int& fid, int& fstride, uint64_t& mask) {
    const bool ok = any && lane < cn && f_raw >= 0 && (long long)f_raw < NB;
    mask = __ballot(ok);
    fid = ok ? f_raw : 0;
    fstride = ok ? 1 : 0;
  };
  auto finalize = [&](const Piece& pc) {
    const float lrow = wave_sum_over_j(lsum);
    const bool nrow = GROUPED ? n < pc.sz * G && pc.b + n / G < B : n < G;
    if (nrow) {
      if (pc.complete) {
        const float inv = v_scale / lrow;
        const size_t o = GROUPED ? ((size_t)(pc.b + n / G) * Hq + (size_t)pc.g * G + n % G) * D + 4 * j
                                 : ((size_t)pc.b * Hq + (size_t)pc.g * G + n) * D + 4 * j;
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
        const size_t row = ((size_t)w * 2 + pc.slot) * 16 + n;
#pragma unroll
        for (int c = 0; c < NC; ++c) *(f32x4*)(ws_o + row * D + 16 * c + 4 * j) = acc[c];
        if (j == 0) {
          ws_ml[2 * row] = m;
          ws_ml[2 * row + 1] = lrow;
        }
      }
    }
  };

  Piece pc;
  if (!find_piece(pc)) return;
  int c0 = 0;  // first frame of the current chunk within its piece
  Chunk cc{}, cx{};  // GROUPED: the current and the next chunk
  if constexpr (GROUPED) {
    cc = chunk_of(pc, 0);
    L = cc.L;
    cblk = cc.blk0;
    col0 = cc.col0;
    col1 = cc.col1;
    resolve(chunk_id_of(cc), cc.len, true, vfid, vstride, live_mask);
  } else {
    L = pc.L;
    cblk = pc.f0;
    resolve(chunk_id(pc, 0), min(kIds, pc.n), true, vfid, vstride, live_mask);
  }
  load_q(qw, pc);
  m = -INFINITY;
  mth = -INFINITY;
  nm = 0.f;
  lsum = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  u32x4 kA[F][NL], vA[F][NL], kB[F][NL], vB[F][NL];
  load_step(kA, vA, 0, vfid, vstride, pc.g);
  load_step(kB, vB, 1, vfid, vstride, pc.g);
  // the next chunk's query is prefetched unless its fragment is large (f32 with D = 128: a second
  // copy would not fit the register budget)
  constexpr bool kPrefetchQ = QW <= 16;
  uint32_t qn[QW];
  for (;;) {
    // the next chunk: the rest of this piece, or the next piece
    Piece pn = pc;
    int c0n = c0 + (GROUPED ? cc.len : kIds);
    bool more = c0n < pc.n;
    if (!more) {
      c0n = 0;
      more = find_piece(pn);
    }
    // its raw ids and query, fetched now and used at the end of this chunk
    int f_raw_n = 0;
    if constexpr (GROUPED) {
      if (more) {
        cx = chunk_of(pn, c0n);
        f_raw_n = chunk_id_of(cx);
      }
    } else {
      if (more) f_raw_n = chunk_id(pn, c0n);
    }
    if constexpr (kPrefetchQ) load_q(qn, pn);
    const int cnn = more ? (GROUPED ? cx.len : min(kIds, pn.n - c0n)) : 0;
    const int cn = GROUPED ? cc.len : min(kIds, pc.n - c0);
    const int np = (cn + 2 * F - 1) / (2 * F) * 2;  // steps of the chunk, an even count
    int vfid_n = 0, vstride_n = 0;
    uint64_t live_n = 0;
    // load step s2 of this chunk, or step s2 - np of the next one
    auto load_next = [&](u32x4 (&kt)[F][NL], u32x4 (&vt)[F][NL], int s2) {
      const bool nx = s2 >= np;
      load_step(kt, vt, nx ? s2 - np : s2, nx ? vfid_n : vfid, nx ? vstride_n : vstride,
                nx ? pn.g : pc.g);
    };
    for (int s = 0; s < np; s += 2) {
      compute_step(kA, vA, s);
      if (s + 2 >= np) resolve(f_raw_n, cnn, more, vfid_n, vstride_n, live_n);
      load_next(kA, vA, s + 2);
      compute_step(kB, vB, s + 1);
      load_next(kB, vB, s + 3);
    }
    if (c0 + cn >= pc.n) finalize(pc);
    if (!more) break;
    const bool fresh = c0n == 0;
    pc = pn;
    c0 = c0n;
    if constexpr (GROUPED) {
      cc = cx;
      L = cc.L;
      cblk = cc.blk0;
      col0 = cc.col0;
      col1 = cc.col1;
    } else {
      L = pc.L;
      cblk = pc.f0 + c0;
    }
    vfid = vfid_n;
    vstride = vstride_n;
    live_mask = live_n;
    if constexpr (kPrefetchQ) {
#pragma unroll
      for (int i = 0; i < QW; ++i) qw[i] = qn[i];
    } else {
      load_q(qw, pc);
    }
    if (fresh) {
      m = -INFINITY;
      mth = -INFINITY;
      nm = 0.f;
      lsum = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }
  // the loads of the last two steps (past the range) land before the wavefront ends
}

// Merge the partials of the runs cut by wavefront range boundaries:
// out = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w, M = max_w m_w (the final normalised
// reduction of codebumble.net, "CUDA Shared Memory Optimization").  There is one wavefront per
// boundary k (between the ranges of wavefronts k and k + 1); it looks at the run holding unit
// a_{k+1}.  Every boundary w0 <= k < w1 that cuts a run sees that same run, where w0 and w1 are
// the wavefronts holding the run's first and last frames; the run's partials are those of
// wavefronts w0..w1 (any with an empty range hold none).  The merge is spread over those
// boundary wavefronts by output columns: the first S of them (S a power of two, at most
// w1 - w0 and at most D / 4) each merge a slice of D / S columns for every partial.  A run cut
// once is merged by one wavefront; a run cut into ~100 pieces (one long sequence over the whole
// GPU) by up to 32 (D = 128), each reading only its slice of the partials.  Wavefront w keeps a run in
// partial slot 1 if the run began after the start of w's range (it is then w's last run), else
// in slot 0.
// Lanes: a slice's G x (D/S) outputs are held by groups of LPG lanes (row rr, QPL quads of
// columns per lane); the 64 / LPG groups of the wavefront take the partials in turn (partial p by
// group p mod groups), each with its own running (max, sum, accumulator) and 16, 8 or 4 of its
// partials loaded at once (one, two or more quads per lane), and the groups are
// combined by the same rule with lane swaps at the end.  The merge order depends only on the
// sizes, so equal inputs give equal bits.  (GROUPED: a run's rows are its members' heads, row r
// being head r % G of member r / G.)
// WIDE (launches whose runs are few against the wavefronts, i.e. a few long sequences): slices
// down to one quad per row (S at most D / 4), and groups with more than 4 partials load 8 or 16
// of them at once.  Other launches keep S at most D / 8 and batches of 4, a smaller kernel.
template <int KIND, int D, bool GROUPED = false, bool WIDE = false>
__device__ __forceinline__ void decode_reduce_wave(
    int k, int lane, void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ plan, int Hq, int Hkv, int G, int W, float v_scale,
    Runs runs = Runs{}, int B = 0, int sub = 0) {
  // partials per group in flight together when a lane holds more than two quads of a row (8
  // took ~330 registers and made the merge of the 70B-shape batch 6.8 us instead of 4.6 us);
  // lanes with one or two quads keep 16 or 8 in flight
  constexpr int kBatch = 4;
  constexpr int NV = D / 16;  // quads per lane at most (G = 16, one slice)
  const int U = plan[0];
  const int4 st = ((const int4*)(plan + 4))[k + 1];
  const long long F = (long long)Hkv * U;
  const long long a1 = F * (k + 1) / W;
  const int u = st.z, su = st.w;
  if (a1 >= F || u <= kRestart) return;  // no frames of this run before the boundary
  const long long s0 = a1 - u;            // first unit of the run
  const long long x0 = s0 + kRestart, x1 = s0 + su - 1;
  // wavefront holding unit x: the largest w with floor(F w / W) <= x
  const int w0 = (int)(((x0 + 1) * W + F - 1) / F - 1);
  const int w1 = (int)(((x1 + 1) * W + F - 1) / F - 1);
  const int cuts = w1 - w0;  // boundaries cutting the run's frames, k among them
  // A grouped run's partials hold 16 rows: each boundary then has kParts wavefronts (sub), which
  // split its columns, so a run cut once is merged by two wavefronts.
  constexpr int kParts = GROUPED ? 2 : 1;
  int S = 1;
  while (2 * S <= cuts && 2 * S * kParts <= (WIDE ? D / 4 : D / 8)) S *= 2;
  if (k - w0 >= S) return;
  const int sl = (k - w0) * kParts + sub;  // this wavefront's slice of the run's columns
  S *= kParts;
  const int b = st.x, g = st.y;
  // rows of the run, and a power of two at least that many for the lane layout (a grouped run
  // lays out all 16 rows of its partials: its row count, a load that depends on the plan, then
  // only decides which rows are stored, and the partials' loads need not wait for it; rows past
  // the run, never written, are merged in their own lanes and dropped)
  const int rows = GROUPED ? min(runs.size[b] * G, min(16, (B - b) * G)) : G;
  const int Gr = GROUPED ? 16 : G;
  const int cq = D / (4 * S);                  // quads of a slice row
  const int lpr = cq < 64 / Gr ? cq : 64 / Gr; // lanes per row in a group
  const int qpl = cq / lpr;                    // quads per lane
  const int lpg = Gr * lpr;                    // lanes per group
  const int groups = 64 / lpg;
  const int grp = lane / lpg, rr = (lane % lpg) / lpr, ql = lane % lpr;
  const int col = sl * (D / S) + ql * qpl * 4;  // first output column of the lane
  float M = -INFINITY, den = 0.f;
  f32x4 num[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) num[v] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const long long aw0 = F * w0 / W;
  const bool dense = F >= W;  // no empty ranges: every wavefront w0..w1 holds a partial
  // the group's partials, QPL quads each, BATCH of them loaded before any is used
  auto merge = [&](auto qpl_c, auto batch_c) {
    constexpr int QPL = decltype(qpl_c)::value, BATCH = decltype(batch_c)::value;
    for (int wb = w0 + grp; wb <= w1; wb += BATCH * groups) {
      f32x4 ob[BATCH][QPL];
      float mb[BATCH], lb[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int w = wb + i * groups;
        bool has = w <= w1;
        if (!dense && has) has = F * w / W < F * (w + 1) / W;
        const int slot = (w == w0 && s0 > aw0) ? 1 : 0;
        const size_t prow = ((size_t)w * 2 + slot) * 16 + rr;
        const f32x4* src = (const f32x4*)(ws_o + prow * D + col);
#pragma unroll
        for (int v = 0; v < QPL; ++v) ob[i][v] = (has && v < qpl) ? src[v] : (f32x4){0.f, 0.f, 0.f, 0.f};
        mb[i] = has ? ws_ml[2 * prow] : -INFINITY;
        lb[i] = has ? ws_ml[2 * prow + 1] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if (mb[i] == -INFINITY) continue;
        if (mb[i] > M) {
          const float sc = __builtin_amdgcn_exp2f(M - mb[i]);
          den *= sc;
#pragma unroll
          for (int v = 0; v < QPL; ++v) num[v] *= sc;
          M = mb[i];
        }
        const float ew = __builtin_amdgcn_exp2f(mb[i] - M);
        den += ew * lb[i];
#pragma unroll
        for (int v = 0; v < QPL; ++v) num[v] += ew * ob[i][v];
      }
    }
  };
  // (the batch size sets only how many loads are in flight: partials are merged in the same
  // order, so every choice gives the same bits)
  if constexpr (WIDE) {
    const int per_group = (w1 - w0 + groups) / groups;  // partials of a group, at most
    if (qpl == 1 && per_group > 8) {
      merge(std::integral_constant<int, 1>{}, std::integral_constant<int, 16>{});
    } else if (qpl <= 2 && per_group > kBatch) {
      merge(std::integral_constant<int, 2>{}, std::integral_constant<int, 8>{});
    } else {
      merge(std::integral_constant<int, NV>{}, std::integral_constant<int, kBatch>{});
    }
  } else {
    for (int wb = w0 + grp; wb <= w1; wb += kBatch * groups) {
      f32x4 ob[kBatch][NV];
      float mb[kBatch], lb[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int w = wb + i * groups;
        bool has = w <= w1;
        if (!dense && has) has = F * w / W < F * (w + 1) / W;
        const int slot = (w == w0 && s0 > aw0) ? 1 : 0;
        const size_t prow = ((size_t)w * 2 + slot) * 16 + rr;
        const f32x4* src = (const f32x4*)(ws_o + prow * D + col);
#pragma unroll
        for (int v = 0; v < NV; ++v) ob[i][v] = (has && v < qpl) ? src[v] : (f32x4){0.f, 0.f, 0.f, 0.f};
        mb[i] = has ? ws_ml[2 * prow] : -INFINITY;
        lb[i] = has ? ws_ml[2 * prow + 1] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (mb[i] == -INFINITY) continue;
        if (mb[i] > M) {
          const float sc = __builtin_amdgcn_exp2f(M - mb[i]);
          den *= sc;
#pragma unroll
          for (int v = 0; v < NV; ++v) num[v] *= sc;
          M = mb[i];
        }
        const float ew = __builtin_amdgcn_exp2f(mb[i] - M);
        den += ew * lb[i];
#pragma unroll
        for (int v = 0; v < NV; ++v) num[v] += ew * ob[i][v];
      }
    }
  }
  // combine the groups: after the swap at distance d, each lane holds the merge of its group
  // and the group d lanes away (lanes of one row and columns line up across groups)
  for (int d = lpg; d < 64; d *= 2) {
    const float M2 = __shfl_xor(M, d), den2 = __shfl_xor(den, d);
    const float Mn = fmaxf(M, M2);
    const float s1 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    const float s2 = M2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M2 - Mn);
    den = den * s1 + den2 * s2;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      f32x4 o2;
#pragma unroll
      for (int e = 0; e < 4; ++e) o2[e] = __shfl_xor(num[v][e], d);
      num[v] = num[v] * s1 + o2 * s2;
    }
    M = Mn;
  }
  if (grp != 0) return;
  if (GROUPED && rr >= rows) return;
  const float inv = v_scale / den;
  const size_t o = GROUPED ? ((size_t)(b + rr / G) * Hq + (size_t)g * G + rr % G) * D + col
                           : ((size_t)b * Hq + (size_t)g * G + rr) * D + col;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    if (v >= qpl) break;
    if constexpr (KIND == KF32) {
      *(f32x4*)((float*)out + o + 4 * v) = num[v] * inv;
    } else {
      u32x2 pk;
      pk[0] = pack_bf16x2(num[v][0] * inv, num[v][1] * inv);
      pk[1] = pack_bf16x2(num[v][2] * inv, num[v][3] * inv);
      *(u32x2*)((__bf16*)out + o + 4 * v) = pk;
    }
  }
}

// Workspace: the plan (4 ints, then an int4 per wavefront), then the two partial slots of every
// wavefront (max and sum per row, then the 16 x D accumulator rows).
struct Layout {
  int W;
  size_t plan_bytes, ml_bytes, o_bytes;
};

// Workspace of a launch of up to W wavefronts.
inline Layout layout(int D, int W) {
  Layout l;
  l.W = W;
  l.plan_bytes = ((4 + 4 * (size_t)l.W) * sizeof(int32_t) + 255) / 256 * 256;
  l.ml_bytes = (((size_t)l.W * 2 * 16 * 2) * sizeof(float) + 255) / 256 * 256;
  l.o_bytes = (size_t)l.W * 2 * 16 * D * sizeof(float);
  return l;
}

}  // namespace dec
}  // namespace pa
