// pa_cache.hip -- cache writes (reshape_and_cache) and frame copies (copy_blocks) for gfx950.
//
// reshape_and_cache follows the block-table mapping of codebumble.net ("The Block Table
// Mapping Subsystem"): a token's slot names its frame (slot / block_size) and its offset in
// the frame (slot % block_size).  Each workgroup stores one token: every KV head's D values
// go to their places in the (frame, head) tile of the operand-order layout (16-byte stores for
// K, element stores for V).  An fp8 cache stores e4m3fn(fp32(x) / scale), rounded to nearest
// even with saturation.
//
// copy_blocks implements the copy half of copy-on-write (infoisland, section 2): a frame
// shared by several sequences is duplicated before one of them writes into it.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// One workgroup per token.  Thread t takes one 16-byte piece of the token's K row in the tile
// layout (EPC = 16 / element-bytes consecutive head-dim values of one KV head, contiguous in the
// K tile since a lane's fragment holds consecutive head-dim values of one key) and stores it
// with one 16-byte store; the same head-dim values of V sit in EPC different fragments of the
// V tile (there a fragment holds consecutive keys) and are stored one by one.
template <int SRC, int KV, int D, int BS>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const void* __restrict__ k, const void* __restrict__ v, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int64_t* __restrict__ slots, long long NB, int Hkv,
    float k_scale, float v_scale) {
  constexpr int EB = KV == KF32 ? 4 : (KV == KBF16 ? 2 : 1);
  constexpr int TILE = BS * D * EB;
  constexpr int EPC = 16 / EB;  // elements per 16-byte piece
  static_assert((D / 4) % EPC == 0, "a piece must not cross a fragment");
  constexpr int SB = SRC == KF32 ? 4 : 2;  // bytes of a source element
  typedef uint32_t SrcPiece __attribute__((ext_vector_type(EPC * SB / 4)));
  const long long i = blockIdx.x;
  // The source rows do not depend on the slot: the first piece of each thread is loaded before
  // the slot is known, so the two loads overlap instead of forming a chain.
  const int npc = Hkv * (D / EPC);
  SrcPiece k0 = {}, v0 = {};
  if ((int)threadIdx.x < npc) {
    const size_t src0 = ((size_t)i * Hkv * D + (size_t)threadIdx.x * EPC) * SB;
    k0 = *(const SrcPiece*)((const char*)k + src0);
    v0 = *(const SrcPiece*)((const char*)v + src0);
  }
  const long long s = slots[i];
  if (s < 0 || s >= NB * BS) return;
  const long long f = s / BS;
  const int o = (int)(s % BS);
  for (int pc = threadIdx.x; pc < npc; pc += blockDim.x) {
    const int g = pc / (D / EPC), d0 = (pc % (D / EPC)) * EPC;
    const size_t src = ((size_t)i * Hkv + g) * D + d0;
    if (pc != (int)threadIdx.x) {
      k0 = *(const SrcPiece*)((const char*)k + src * SB);
      v0 = *(const SrcPiece*)((const char*)v + src * SB);
    }
    const char* ks = (const char*)&k0;
    const char* vs = (const char*)&v0;
    const size_t tile = ((size_t)f * Hkv + g) * TILE;
    u32x4 kp;
    uint8_t* kb = (uint8_t*)&kp;
    char* vd = v_cache + tile;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      char* vdst = vd + v_tile_byte(o, d0 + e, D, EB);
      if constexpr (KV == KF32) {
        ((uint32_t*)kb)[e] = ((const uint32_t*)ks)[e];
        *(uint32_t*)vdst = ((const uint32_t*)vs)[e];
      } else if constexpr (KV == KBF16) {
        ((uint16_t*)kb)[e] = ((const uint16_t*)ks)[e];
        *(uint16_t*)vdst = ((const uint16_t*)vs)[e];
      } else {
        float xk, xv;
        if constexpr (SRC == KF32) {
          xk = ((const float*)ks)[e];
          xv = ((const float*)vs)[e];
        } else {
          xk = __uint_as_float((uint32_t)((const uint16_t*)ks)[e] << 16);
          xv = __uint_as_float((uint32_t)((const uint16_t*)vs)[e] << 16);
        }
        kb[e] = (uint8_t)f32_to_e4m3fn(__fdiv_rn(xk, k_scale));
        *(uint8_t*)vdst = (uint8_t)f32_to_e4m3fn(__fdiv_rn(xv, v_scale));
      }
    }
    *(u32x4*)(k_cache + tile + k_tile_byte(o, d0, D, EB)) = kp;
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
  hipLaunchKernelGGL((reshape_and_cache_kernel<SRC, KV, D, BS>), dim3((unsigned)T), dim3(256), 0,
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
