// Storing one new token's key and value rows into the slot the block
// manager reserved for it ("What is PagedAttention" (tecyfy), How it works:
// blocks handed out as a sequence grows).  Shared by the reshape_and_cache
// kernel and the fused append-and-plan kernel of a decode step.
#pragma once

#include "device_common.h"

namespace pkv {

// k_cache[slot / B][h][slot % B][:] = k[i][h][:] (and v) for every KV head h,
// moved in 16-byte pieces by the threads of the calling workgroup.  A slot
// outside [0, num_slots) stores nothing.  The slot and the first key/value
// loads are independent, so they are in flight together.
__device__ __forceinline__ void scatter_token(const char* __restrict__ k, const char* __restrict__ v,
                                              char* __restrict__ k_cache, char* __restrict__ v_cache,
                                              const int32_t* __restrict__ slot_mapping, int i,
                                              int32_t num_kv_heads, int32_t chunks,
                                              int32_t block_size, int64_t num_slots) {
  const int32_t slot = slot_mapping[i];
  const int per_tok = num_kv_heads * chunks;        // 16-byte pieces of one token
  const char* ks = k + (size_t)i * per_tok * 16;
  const char* vs = v + (size_t)i * per_tok * 16;
  const bool ok = slot >= 0 && (int64_t)slot < num_slots;
  const int blk = ok ? slot / block_size : 0, off = ok ? slot % block_size : 0;
  for (int j = threadIdx.x; j < per_tok; j += blockDim.x) {
    const u32x4 a = load16(ks + (size_t)j * 16);
    const u32x4 b = load16(vs + (size_t)j * 16);
    if (!ok) continue;
    const int h = j / chunks, c = j - h * chunks;
    const size_t dst = ((((size_t)blk * num_kv_heads + h) * block_size + off) * chunks + c) * 16;
    store16(k_cache + dst, a);
    store16(v_cache + dst, b);
  }
}

}  // namespace pkv
