// Matrix-core decode attention for grouped-query heads
// (attention_mfma_impl.h), instances with plain key and value loads: blocks
// shared by several sequences of the batch stay in L2 and the Infinity
// Cache between their readers.
#include "attention_mfma_impl.h"

namespace pkv {

bool launch_attention_mfma_keep(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                                int block_size, int cap, hipStream_t stream, hipError_t* err) {
  return mfma_dispatch<false>(p, dt, kv, head_dim, block_size, cap, stream, err);
}

}  // namespace pkv
