// pa_device.h -- device-side building blocks shared by the paged-attention kernels (gfx950).
//
// Cache tiles are stored in "operand order" (the layout written out in include/pa.h): a
// (frame, kv-head) tile is a run of 1 KiB pieces, 64 lanes x 16 bytes, and the 16 bytes lane
// l loads from piece r are exactly the operand fragment that lane feeds a matrix-core
// instruction.  A wavefront gathers a tile with NL fully contiguous 1 KiB loads and never
// shuffles data between lanes.
//
// Scores are computed transposed, S^T = K * Q^T, so that keys are the 16 rows of the MFMA
// output and the query rows (GQA heads, or tokens x heads in a prefill chunk) its 16 columns.
// The 16x16 accumulator leaves lane (j = l/16, n = l%16) with the scores of query row n for
// keys 4j..4j+3 -- the exact B-operand fragment of the P*V product O^T = V^T * P^T, which
// therefore needs no transpose either.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Kind { KF32 = 0, KBF16 = 1, KFP8 = 2 };

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------------- tile layout

// Byte offset of (token slot o, head-dim index d) inside a K tile with element size b.
__host__ __device__ constexpr uint32_t k_tile_byte(int o, int d, int D, int b) {
  return 1024u * (uint32_t)((o / 16) * (D * b / 64) + ((d % (D / 4)) * b) / 16) +
         16u * (uint32_t)(16 * (d / (D / 4)) + (o % 16)) + (uint32_t)(((d % (D / 4)) * b) % 16);
}

// Byte offset of (token slot o, head-dim index d) inside a V tile with element size b.
__host__ __device__ constexpr uint32_t v_tile_byte(int o, int d, int D, int b) {
  return 1024u * (uint32_t)(((o / 16) * (D / 16) + d / 16) / (4 / b)) +
         16u * (uint32_t)(16 * ((o % 16) / 4) + (d % 16)) +
         (uint32_t)((4 * (((o / 16) * (D / 16) + d / 16) % (4 / b)) + (o % 4)) * b);
}

// ------------------------------------------------------------------------- conversions

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  // a two-wide fptrunc is one v_cvt_pk_bf16_f32 (round to nearest even) on gfx950
  const bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four e4m3fn codes (one dword, byte k = element k) -> four bf16 (two dwords).  Every e4m3fn
// value has at most 4 significant bits and an exponent inside bf16's range, so the conversion is
// exact.  gfx950's scaled conversion turns two codes into a bf16 pair in one instruction; with a
// scale of 1 it equals widening to fp32 and keeping the high halves, bit for bit over all 65,536
// code pairs (NaNs included; checked on the hardware).
__device__ inline u32x2 fp8x4_to_bf16x4(uint32_t w) {
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// fp32 -> e4m3fn code, round to nearest even, saturating to +-448, NaN -> 0x7f | sign.
// Integer arithmetic on the fp32 bits: with E = max(exponent, -6) the value is rounded to a
// multiple of 2^(E-3), n = round(value / 2^(E-3)) in [0, 16], and code = (E + 6) * 8 + n
// (n = 16 carries into the exponent field by itself; E = -6 covers the subnormal codes).
__device__ inline uint32_t f32_to_e4m3fn(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;  // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |y| >= 448 (and inf): saturate
  const int ebits = (int)(a >> 23);
  const uint32_t sig = (a & 0x7fffffu) | (ebits ? 0x800000u : 0u);
  const int e = (ebits ? ebits : 1) - 127;
  const int E = e > -6 ? e : -6;
  const int shift = 20 + E - e;  // >= 20
  uint32_t n = 0;
  if (shift < 32) {
    n = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (n & 1u))) ++n;
  }
  return sign | (uint32_t)((E + 6) * 8 + (int)n);
}

// ------------------------------------------------------------------------- matrix cores

__device__ inline f32x4 mfma_x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mfma_x16_bf16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ inline f32x4 mfma_x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------------- operand traits
//
// KvOps<KIND, D, BS> describes one (frame, head) tile held in registers as NL u32x4 loads:
//   kop(t, h, s)   A fragment of S^T for key group h (16 keys) and contraction slice s
//   vop(t, h, c)   A fragment of O^T = V^T P^T for key group h and head-dim tile c (16 dims)
//   qk(acc, kop, qop) / pv(acc, vop, p) the matching matrix-core steps
// The query operand is kept as the D/4 head-dim values of row n at dims (D/4)*j .. +D/4.

template <int KIND, int D, int BS>
struct KvOps;

template <int D, int BS>
struct KvOps<KBF16, D, BS> {
  static constexpr int EB = 2;
  static constexpr int TILE = BS * D * EB;
  static constexpr int NL = TILE / 1024;
  static constexpr int KG = BS / 16;
  static constexpr int NS = D / 32;   // 16x16x32 slices over the head dim
  static constexpr int NC = D / 16;   // 16-wide head-dim tiles
  static constexpr int QW = D / 8;    // dwords of the query fragment (D/4 bf16)
  static constexpr int KLPG = D * EB / 64;
  typedef u32x4 KOp;
  __device__ static KOp kop(const u32x4* t, int h, int s) { return t[h * KLPG + s]; }
  __device__ static u32x2 vop(const u32x4* t, int h, int c) {
    const int u = h * NC + c;
    const u32x4 x = t[u >> 1];
    u32x2 r;
    r[0] = (u & 1) ? x[2] : x[0];
    r[1] = (u & 1) ? x[3] : x[1];
    return r;
  }
  __device__ static u32x4 qop(const uint32_t* qw, int s) {
    u32x4 r;
    r[0] = qw[4 * s]; r[1] = qw[4 * s + 1]; r[2] = qw[4 * s + 2]; r[3] = qw[4 * s + 3];
    return r;
  }
  __device__ static f32x4 qk(f32x4 acc, KOp k, u32x4 q) { return mfma_x32_bf16(k, q, acc); }
  // P^T fragment: the probabilities rounded to bf16; the row sum uses the rounded values so
  // that the normalisation matches the weights the matrix core actually applies.
  typedef u32x2 PFrag;
  __device__ static PFrag pfrag(f32x4 p, float& lsum) {
    u32x2 pp;
    pp[0] = pack_bf16x2(p[0], p[1]);
    pp[1] = pack_bf16x2(p[2], p[3]);
    lsum += (bf16_lo(pp[0]) + bf16_hi(pp[0])) + (bf16_lo(pp[1]) + bf16_hi(pp[1]));
    return pp;
  }
  __device__ static f32x4 pv(f32x4 acc, u32x2 v, PFrag p) { return mfma_x16_bf16(v, p, acc); }
  // Two 16-key groups in one 16x16x32 step: elements 0-3 of each lane are group a's keys,
  // elements 4-7 group b's, identically in the V^T and P^T fragments.
  __device__ static f32x4 pv2(f32x4 acc, u32x2 va, u32x2 vb, PFrag pa, PFrag pb) {
    u32x4 a, b;
    a[0] = va[0]; a[1] = va[1]; a[2] = vb[0]; a[3] = vb[1];
    b[0] = pa[0]; b[1] = pa[1]; b[2] = pb[0]; b[3] = pb[1];
    return mfma_x32_bf16(a, b, acc);
  }
  __device__ static void zero_quad(u32x4* t, int h, int c, int keep) {
    // zero the elements for keys 4j+i with i >= keep of quad (h, c)
    const int u = h * NC + c;
    u32x4& x = t[u >> 1];
    const int w0 = (u & 1) ? 2 : 0;
    const uint32_t m0 = keep >= 2 ? 0xffffffffu : (keep == 1 ? 0x0000ffffu : 0u);
    const uint32_t m1 = keep >= 4 ? 0xffffffffu : (keep == 3 ? 0x0000ffffu : 0u);
    x[w0] &= m0;
    x[w0 + 1] &= m1;
  }
};

template <int D, int BS>
struct KvOps<KFP8, D, BS> {
  static constexpr int EB = 1;
  static constexpr int TILE = BS * D * EB;
  static constexpr int NL = TILE / 1024;
  static constexpr int KG = BS / 16;
  static constexpr int NS = D / 32;
  static constexpr int NC = D / 16;
  static constexpr int QW = D / 8;
  static constexpr int KLPG = D * EB / 64;
  typedef u32x4 KOp;
  __device__ static KOp kop(const u32x4* t, int h, int s) {
    const u32x4 x = t[h * KLPG + (s >> 1)];
    const u32x2 a = fp8x4_to_bf16x4((s & 1) ? x[2] : x[0]);
    const u32x2 b = fp8x4_to_bf16x4((s & 1) ? x[3] : x[1]);
    u32x4 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
  }
  __device__ static u32x2 vop(const u32x4* t, int h, int c) {
    const int u = h * NC + c;
    return fp8x4_to_bf16x4(t[u >> 2][u & 3]);
  }
  __device__ static u32x4 qop(const uint32_t* qw, int s) {
    u32x4 r;
    r[0] = qw[4 * s]; r[1] = qw[4 * s + 1]; r[2] = qw[4 * s + 2]; r[3] = qw[4 * s + 3];
    return r;
  }
  __device__ static f32x4 qk(f32x4 acc, KOp k, u32x4 q) { return mfma_x32_bf16(k, q, acc); }
  typedef u32x2 PFrag;
  __device__ static PFrag pfrag(f32x4 p, float& lsum) { return KvOps<KBF16, D, BS>::pfrag(p, lsum); }
  __device__ static f32x4 pv(f32x4 acc, u32x2 v, PFrag p) { return mfma_x16_bf16(v, p, acc); }
  __device__ static f32x4 pv2(f32x4 acc, u32x2 va, u32x2 vb, PFrag pa, PFrag pb) {
    return KvOps<KBF16, D, BS>::pv2(acc, va, vb, pa, pb);
  }
  __device__ static void zero_quad(u32x4* t, int h, int c, int keep) {
    const int u = h * NC + c;
    const uint32_t m = keep >= 4 ? 0xffffffffu : ((1u << (8 * keep)) - 1u);
    t[u >> 2][u & 3] &= m;
  }
};

template <int D, int BS>
struct KvOps<KF32, D, BS> {
  static constexpr int EB = 4;
  static constexpr int TILE = BS * D * EB;
  static constexpr int NL = TILE / 1024;
  static constexpr int KG = BS / 16;
  static constexpr int NS = D / 4;   // 16x16x4 slices, one value per lane
  static constexpr int NC = D / 16;
  static constexpr int QW = D / 4;   // dwords of the query fragment (D/4 floats)
  static constexpr int KLPG = D * EB / 64;
  typedef float KOp;
  __device__ static KOp kop(const u32x4* t, int h, int s) {
    return __uint_as_float(t[h * KLPG + (s >> 2)][s & 3]);
  }
  __device__ static u32x4 vop(const u32x4* t, int h, int c) { return t[h * NC + c]; }
  __device__ static float qop(const uint32_t* qw, int s) { return __uint_as_float(qw[s]); }
  __device__ static f32x4 qk(f32x4 acc, KOp k, float q) { return mfma_x4_f32(k, q, acc); }
  typedef f32x4 PFrag;
  __device__ static PFrag pfrag(f32x4 p, float& lsum) {
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    return p;
  }
  __device__ static f32x4 pv(f32x4 acc, u32x4 v, PFrag p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma_x4_f32(__uint_as_float(v[i]), p[i], acc);
    return acc;
  }
  __device__ static f32x4 pv2(f32x4 acc, u32x4 va, u32x4 vb, PFrag pa, PFrag pb) {
    return pv(pv(acc, va, pa), vb, pb);
  }
  __device__ static void zero_quad(u32x4* t, int h, int c, int keep) {
    u32x4& x = t[h * NC + c];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i >= keep) x[i] = 0u;
  }
};

// ------------------------------------------------------------------------- wave helpers

// Lanes n, n+16, n+32, n+48 hold the same query row: reduce across them.  The gfx950 row
// swaps exchange 16-lane rows 1<->0 and 3<->2 (then 32-lane halves) between two registers, so
// after each swap one of the pair holds the partner lanes' values -- all in the VALU, with no
// LDS round trip.
__device__ inline float wave_max_over_j(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float wave_sum_over_j(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace pa
