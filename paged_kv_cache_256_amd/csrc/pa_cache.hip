// pa_cache.hip -- cache writes (reshape_and_cache) and frame copies (copy_blocks) for gfx950.
//
// reshape_and_cache follows the block-table mapping of codebumble.net ("The Block Table
// Mapping Subsystem"): a token's slot names its frame (slot / block_size) and its offset in
// the frame (slot % block_size).  Each workgroup stores one token: every KV head's D values
// go to their places in the (frame, head) tile of the operand-order layout (16-byte stores for
// K, element stores into consecutive 16-byte lines for V).  An fp8 cache stores e4m3fn(fp32(x) / scale), rounded to nearest
// even with saturation.
//
// copy_blocks implements the copy half of copy-on-write (infoisland, section 2): a frame
// shared by several sequences is duplicated before one of them writes into it.

#include "pa_device.h"
#include "pa_internal.h"

#include <type_traits>

namespace pa {

namespace {

// One workgroup per token.  K: thread t takes one 16-byte piece of the token's K row in the
// tile layout (EPC = 16 / element-bytes consecutive head-dim values of one KV head, contiguous
// in the K tile since a lane's fragment holds consecutive head-dim values of one key) and stores
// it with one 16-byte store.  V: a V fragment holds consecutive keys, so the token's value for
// head-dim index d lands in the 16-byte line of column d; thread t takes the elements t, t + 256,
// ... of the token's V row, so that the lanes of a wavefront store into consecutive lines (a few
// cache lines per store instruction rather than one line per lane).
constexpr int kCacheThreads = 256;  // threads of a cache-write workgroup

template <int SRC, int KV, int D, int BS>
__global__ __launch_bounds__(kCacheThreads) void reshape_and_cache_kernel(
    const void* __restrict__ k, const void* __restrict__ v, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int64_t* __restrict__ slots, long long NB, int Hkv,
    float k_scale, float v_scale) {
  constexpr int EB = KV == KF32 ? 4 : (KV == KBF16 ? 2 : 1);
  constexpr int TILE = BS * D * EB;
  constexpr int EPC = 16 / EB;  // elements per 16-byte piece
  static_assert((D / 4) % EPC == 0, "a piece must not cross a fragment");
  constexpr int SB = SRC == KF32 ? 4 : 2;  // bytes of a source element
  typedef uint32_t SrcPiece __attribute__((ext_vector_type(EPC * SB / 4)));
  typedef std::conditional_t<SB == 4, uint32_t, uint16_t> SrcElem;
  const long long i = blockIdx.x;
  const int t = threadIdx.x;
  // The source rows do not depend on the slot: the first K piece and V element of each thread
  // are loaded before the slot is known, so the loads overlap instead of forming a chain.
  const int npc = Hkv * (D / EPC), nel = Hkv * D;
  const SrcElem* vrow = (const SrcElem*)v + (size_t)i * nel;
  constexpr int kVB = 4;  // V elements of a thread loaded together (t + kCacheThreads u)
  SrcPiece k0 = {};
  SrcElem vb[kVB];
  if (t < npc) k0 = *(const SrcPiece*)((const char*)k + ((size_t)i * nel + (size_t)t * EPC) * SB);
#pragma unroll
  for (int u = 0; u < kVB; ++u) vb[u] = t + kCacheThreads * u < nel ? vrow[t + kCacheThreads * u] : 0;
  const long long s = slots[i];
  if (s < 0 || s >= NB * BS) return;
  const long long f = s / BS;
  const int o = (int)(s % BS);
  for (int pc = t; pc < npc; pc += kCacheThreads) {
    const int g = pc / (D / EPC), d0 = (pc % (D / EPC)) * EPC;
    if (pc != t) k0 = *(const SrcPiece*)((const char*)k + (((size_t)i * Hkv + g) * D + d0) * SB);
    const char* ks = (const char*)&k0;
    u32x4 kp;
    uint8_t* kb = (uint8_t*)&kp;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if constexpr (KV == KF32) {
        ((uint32_t*)kb)[e] = ((const uint32_t*)ks)[e];
      } else if constexpr (KV == KBF16) {
        ((uint16_t*)kb)[e] = ((const uint16_t*)ks)[e];
      } else {
        const float xk = SRC == KF32 ? ((const float*)ks)[e]
                                     : __uint_as_float((uint32_t)((const uint16_t*)ks)[e] << 16);
        kb[e] = (uint8_t)f32_to_e4m3fn(__fdiv_rn(xk, k_scale));
      }
    }
    *(u32x4*)(k_cache + ((size_t)f * Hkv + g) * TILE + k_tile_byte(o, d0, D, EB)) = kp;
  }
  for (int e0 = 0; e0 < nel; e0 += kCacheThreads * kVB) {
    if (e0 > 0) {
#pragma unroll
      for (int u = 0; u < kVB; ++u) {
        const int e = e0 + t + kCacheThreads * u;
        vb[u] = e < nel ? vrow[e] : 0;
      }
    }
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const int e = e0 + t + kCacheThreads * u;
      if (e >= nel) break;
      const int g = e / D, d = e % D;
      char* vdst = v_cache + ((size_t)f * Hkv + g) * TILE + v_tile_byte(o, d, D, EB);
      if constexpr (KV == KF32) {
        *(uint32_t*)vdst = vb[u];
      } else if constexpr (KV == KBF16) {
        *(uint16_t*)vdst = vb[u];
      } else {
        const float xv = SRC == KF32 ? __uint_as_float((uint32_t)vb[u])
                                     : __uint_as_float((uint32_t)vb[u] << 16);
        *(uint8_t*)vdst = (uint8_t)f32_to_e4m3fn(__fdiv_rn(xv, v_scale));
      }
    }
  }
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_cache,
                                                          char* __restrict__ v_cache,
                                                          const int64_t* __restrict__ pairs,
                                                          long long NB, long long frame_bytes) {
  const long long p = blockIdx.x;
  const long long src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= NB || dst < 0 || dst >= NB) return;
  char* base = blockIdx.y ? v_cache : k_cache;
  const u32x4* s = (const u32x4*)(base + src * frame_bytes);
  u32x4* d = (u32x4*)(base + dst * frame_bytes);
  const long long n16 = frame_bytes / 16;
  // up to kBatch pieces of each thread in flight before any is stored (a frame of the 70B-shape
  // cache is 2,048 pieces: 8 per thread, one memory latency instead of eight); the copy of a
  // pair reads only its source frame and writes only its destination, which no pair reads
  constexpr int kBatch = 8;
  for (long long t0 = threadIdx.x; t0 < n16; t0 += (long long)blockDim.x * kBatch) {
    u32x4 buf[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const long long t = t0 + (long long)u * blockDim.x;
      if (t < n16) buf[u] = s[t];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const long long t = t0 + (long long)u * blockDim.x;
      if (t < n16) d[t] = buf[u];
    }
  }
}

template <int SRC, int KV, int D, int BS>
hipError_t launch_reshape_typed(const void* k, const void* v, void* kc, void* vc,
                                const int64_t* slots, int64_t T, int64_t NB, int Hkv,
                                float ks, float vs, hipStream_t stream) {
  hipLaunchKernelGGL((reshape_and_cache_kernel<SRC, KV, D, BS>), dim3((unsigned)T), dim3(kCacheThreads), 0,
                     stream, k, v, (char*)kc, (char*)vc, slots, (long long)NB, Hkv, ks, vs);
  return hipGetLastError();
}

template <int SRC, int KV>
hipError_t launch_reshape_kind(const void* k, const void* v, void* kc, void* vc,
                               const int64_t* slots, int64_t T, int64_t NB, int Hkv, int D,
                               int bs, float ks, float vs, hipStream_t s) {
  if (D == 64 && bs == 16) return launch_reshape_typed<SRC, KV, 64, 16>(k, v, kc, vc, slots, T, NB, Hkv, ks, vs, s);
  if (D == 64 && bs == 32) return launch_reshape_typed<SRC, KV, 64, 32>(k, v, kc, vc, slots, T, NB, Hkv, ks, vs, s);
  if (D == 128 && bs == 16) return launch_reshape_typed<SRC, KV, 128, 16>(k, v, kc, vc, slots, T, NB, Hkv, ks, vs, s);
  if (D == 128 && bs == 32) return launch_reshape_typed<SRC, KV, 128, 32>(k, v, kc, vc, slots, T, NB, Hkv, ks, vs, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slots, int64_t T, int64_t NB, int Hkv, int D,
                                    int bs, int src_dtype, int kv_dtype, float k_scale,
                                    float v_scale, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (src_dtype == DT_F32 && kv_dtype == DT_F32)
    return launch_reshape_kind<KF32, KF32>(k, v, k_cache, v_cache, slots, T, NB, Hkv, D, bs, k_scale, v_scale, stream);
  if (src_dtype == DT_BF16 && kv_dtype == DT_BF16)
    return launch_reshape_kind<KBF16, KBF16>(k, v, k_cache, v_cache, slots, T, NB, Hkv, D, bs, k_scale, v_scale, stream);
  if (src_dtype == DT_BF16 && kv_dtype == DT_FP8)
    return launch_reshape_kind<KBF16, KFP8>(k, v, k_cache, v_cache, slots, T, NB, Hkv, D, bs, k_scale, v_scale, stream);
  if (src_dtype == DT_F32 && kv_dtype == DT_FP8)
    return launch_reshape_kind<KF32, KFP8>(k, v, k_cache, v_cache, slots, T, NB, Hkv, D, bs, k_scale, v_scale, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int64_t N,
                              int64_t NB, int64_t frame_bytes, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)N, 2), dim3(256), 0, stream,
                     (char*)k_cache, (char*)v_cache, pairs, (long long)NB,
                     (long long)frame_bytes);
  return hipGetLastError();
}

}  // namespace pa
