// Split-K merge for long contexts: each partition of a sequence left its
// normalised output o_p and (m_p, l_p) in the workspace; with
// M = max_p m_p and w_p = l_p 2^(m_p - M),
//     out = sum_p w_p o_p / sum_p w_p,
// which is the softmax over all of the sequence's tokens (the block-by-block
// evaluation the "pagedattention vllm" glossary describes under Attention
// Computation, Block-Wise Attention, carried across workgroups).
// One workgroup per (sequence, query head), one lane per element of the head.
#include "attention_common.h"

namespace pkv {

template <int DT, int D>
__global__ __launch_bounds__(D) void attn_reduce_kernel(AttnParams p, int B) {
  const int s = blockIdx.x / p.num_q_heads;
  const int hq = blockIdx.x % p.num_q_heads;
  const SeqWork sw = seq_work(p, s, B);
  if (sw.bad || sw.nparts <= 1) return;     // written by the main kernel
  const size_t base = ((size_t)s * p.num_q_heads + hq) * p.max_parts;
  const float* ml = p.ws_ml + base * 2;
  float M = -INFINITY;
  for (int i = 0; i < sw.nparts; ++i) M = fmaxf(M, ml[2 * i]);
  const float ref = softmax_ref(M);
  const int d = threadIdx.x;
  float tot = 0.f, o = 0.f;
  for (int i = 0; i < sw.nparts; ++i) {
    const float wgt = ml[2 * i + 1] * fast_exp2(ml[2 * i] - ref);
    tot += wgt;
    o = fmaf(wgt, p.ws_o[(base + i) * D + d], o);
  }
  store_elem<DT>(p.out, ((size_t)s * p.num_q_heads + hq) * D + d, o / tot);
}

namespace {
template <int DT, int D>
hipError_t launch_reduce(const AttnParams& p, int B, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.num_seqs * p.num_q_heads));
  hipLaunchKernelGGL((attn_reduce_kernel<DT, D>), grid, dim3(D), 0, st, p, B);
  return hipGetLastError();
}

template <int DT>
bool by_dim(const AttnParams& p, int D, int B, hipStream_t st, hipError_t* e) {
  switch (D) {
    case 64: *e = launch_reduce<DT, 64>(p, B, st); return true;
    case 128: *e = launch_reduce<DT, 128>(p, B, st); return true;
    default: return false;
  }
}
}  // namespace

bool launch_attention_reduce(const AttnParams& p, pkv_dtype dt, int head_dim, int block_size,
                             hipStream_t stream, hipError_t* err) {
  switch (dt) {
    case PKV_F32: return by_dim<PKV_F32>(p, head_dim, block_size, stream, err);
    case PKV_F16: return by_dim<PKV_F16>(p, head_dim, block_size, stream, err);
    case PKV_BF16: return by_dim<PKV_BF16>(p, head_dim, block_size, stream, err);
    default: return false;
  }
}

}  // namespace pkv
