// Vector-ALU decode attention (attention_valu_impl.h), instances whose key
// and value loads carry the nontemporal hint: caches streamed once per step.
#include "attention_valu_impl.h"

namespace pkv {

bool launch_attention_valu_stream(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                                  int block_size, int cap, hipStream_t stream, hipError_t* err) {
  return valu_dispatch<true>(p, dt, kv, head_dim, block_size, cap, stream, err);
}

bool launch_attention_valu(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                           int block_size, int cap, bool keep, hipStream_t stream, hipError_t* err) {
  return keep ? launch_attention_valu_keep(p, dt, kv, head_dim, block_size, cap, stream, err)
              : launch_attention_valu_stream(p, dt, kv, head_dim, block_size, cap, stream, err);
}

}  // namespace pkv
