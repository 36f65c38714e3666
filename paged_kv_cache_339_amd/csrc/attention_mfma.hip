// Matrix-core decode attention for grouped-query heads
// (attention_mfma_impl.h), instances whose key and value loads carry the
// nontemporal hint: caches streamed once per step.
#include "attention_mfma_impl.h"

namespace pkv {

bool launch_attention_mfma_stream(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                                  int block_size, int cap, hipStream_t stream, hipError_t* err) {
  return mfma_dispatch<true>(p, dt, kv, head_dim, block_size, cap, stream, err);
}

bool launch_attention_mfma(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                           int block_size, int cap, bool keep, hipStream_t stream, hipError_t* err) {
  return keep ? launch_attention_mfma_keep(p, dt, kv, head_dim, block_size, cap, stream, err)
              : launch_attention_mfma_stream(p, dt, kv, head_dim, block_size, cap, stream, err);
}

}  // namespace pkv
