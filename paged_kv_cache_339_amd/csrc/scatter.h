// Storing one new token's key and value rows into the slot the block
// manager reserved for it ("What is PagedAttention" (tecyfy), How it works:
// blocks handed out as a sequence grows).  Shared by the reshape_and_cache
// kernel and the fused append-and-plan kernel of a decode step.
#pragma once

#include "device_common.h"

namespace pkv {

// k_cache[slot / B][h][slot % B][:] = k[i][h][:] (and v) for every KV head h,
// moved in 16-byte pieces: the caller's thread takes pieces first,
// first + stride, ... (stride = the threads given to the token, which may
// span several workgroups).  A slot outside [0, num_slots) stores nothing.  The slot and every key/value load
// of a thread (up to kScatterAhead pieces of each) are in flight together,
// so a token costs one memory round trip, not one per piece.
constexpr int kScatterAhead = 8;

__device__ __forceinline__ void scatter_token(const char* __restrict__ k, const char* __restrict__ v,
                                              char* __restrict__ k_cache, char* __restrict__ v_cache,
                                              const int32_t* __restrict__ slot_mapping, int i,
                                              int first, int stride, int32_t num_kv_heads,
                                              int32_t chunks, int32_t block_size, int64_t num_slots) {
  const int32_t slot = slot_mapping[i];
  const int per_tok = num_kv_heads * chunks;        // 16-byte pieces of one token
  const char* ks = k + (size_t)i * per_tok * 16;
  const char* vs = v + (size_t)i * per_tok * 16;
  for (int j0 = first; j0 < per_tok; j0 += stride * kScatterAhead) {
    u32x4 a[kScatterAhead], b[kScatterAhead];
#pragma unroll
    for (int u = 0; u < kScatterAhead; ++u) {
      const int j = j0 + u * stride;
      if (j < per_tok) {
        a[u] = load16(ks + (size_t)j * 16);
        b[u] = load16(vs + (size_t)j * 16);
      }
    }
    if (slot < 0 || (int64_t)slot >= num_slots) continue;
    const int blk = slot / block_size, off = slot % block_size;
#pragma unroll
    for (int u = 0; u < kScatterAhead; ++u) {
      const int j = j0 + u * stride;
      if (j >= per_tok) break;
      const int h = j / chunks, c = j - h * chunks;
      const size_t dst = ((((size_t)blk * num_kv_heads + h) * block_size + off) * chunks + c) * 16;
      store16(k_cache + dst, a[u]);
      store16(v_cache + dst, b[u]);
    }
  }
}

// The same store into 8-bit E4M3 caches.  Each output piece of 16 codes
// reads 16 input values (f32/f16/bf16, IT) and stores the code of
// fp32(x) / scale: IEEE fp32 division, clamp to [-448, 448] (saturation;
// the conversion alone would turn an overflow into NaN), round to nearest
// even by the hardware conversion, NaN stored as 0x7F.
template <int IT>
__device__ __forceinline__ uint32_t e4m3_pack4(const float* x, float scale) {
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[e] / scale, -448.f), 448.f);
  int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);    // bytes 0, 1
  packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], packed, true);    // bytes 2, 3
  uint32_t out = (uint32_t)packed;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (__builtin_isnan(x[e] / scale)) out = (out & ~(0xffu << (8 * e))) | (0x7fu << (8 * e));
  return out;
}

template <int IT>
__device__ __forceinline__ void scatter_token_fp8(const char* __restrict__ k, const char* __restrict__ v,
                                                  char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                  const int32_t* __restrict__ slot_mapping, int i,
                                                  int first, int stride, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t block_size,
                                                  int64_t num_slots, float k_scale, float v_scale) {
  constexpr int ES = Format<IT>::kBytes;
  constexpr int LOADS = 16 * ES / 16;                 // 16-byte input loads per 16 codes
  constexpr int AHEAD = kScatterAhead / 2;            // 16-code pieces whose inputs load together
  const int32_t slot = slot_mapping[i];
  const int chunks = head_dim / 16;                   // 16-code pieces per (token, head) row
  const int per_tok = num_kv_heads * chunks;
  for (int j0 = first; j0 < per_tok; j0 += stride * AHEAD) {
    u32x4 kr[AHEAD][LOADS], vr[AHEAD][LOADS];
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) {
      const int j = j0 + u * stride;
      if (j < per_tok) {
        const char* ks = k + ((size_t)i * per_tok + j) * 16 * ES;
        const char* vs = v + ((size_t)i * per_tok + j) * 16 * ES;
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
          kr[u][l] = load16(ks + 16 * l);
          vr[u][l] = load16(vs + 16 * l);
        }
      }
    }
    if (slot < 0 || (int64_t)slot >= num_slots) continue;
    const int blk = slot / block_size, off = slot % block_size;
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) {
      const int j = j0 + u * stride;
      if (j >= per_tok) break;
      float kx[16], vx[16];
#pragma unroll
      for (int l = 0; l < LOADS; ++l) {
        widen16<IT>(kr[u][l], kx + l * (16 / ES));
        widen16<IT>(vr[u][l], vx + l * (16 / ES));
      }
      u32x4 kc, vc;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kc[w] = e4m3_pack4<IT>(kx + 4 * w, k_scale);
        vc[w] = e4m3_pack4<IT>(vx + 4 * w, v_scale);
      }
      const int h = j / chunks, c = j - h * chunks;
      const size_t dst = ((((size_t)blk * num_kv_heads + h) * block_size + off) * chunks + c) * 16;
      store16(k_cache + dst, kc);
      store16(v_cache + dst, vc);
    }
  }
}

}  // namespace pkv
