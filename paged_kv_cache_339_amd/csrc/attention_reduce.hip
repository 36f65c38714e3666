// Split-K merge for long contexts: each partition of a sequence left its
// normalised output o_p and (m_p, l_p) in the workspace; with
// M = max_p m_p and w_p = l_p 2^(m_p - M),
//     out = sum_p w_p o_p / sum_p w_p,
// which is the softmax over all of the sequence's tokens (the block-by-block
// evaluation the "pagedattention vllm" glossary describes under Attention
// Computation, Block-Wise Attention, carried across workgroups).
#include "attention_common.h"

namespace pkv {

// One workgroup per (sequence, head chunk): the chunk's rows of a partition
// are one contiguous run, read 8 elements (one 16-byte load of a 16-bit
// row) per lane.  The merge runs over the partitions in order, as online
// softmax:
// M' = max(M, m_p), W = W 2^(M - M') + l_p 2^(m_p - M'), and O likewise with
// l_p 2^(m_p - M') o_p; the result O / W equals the two-pass form above.
constexpr int kReduceThreads = 256;
constexpr int kReduceElems = 8;     // consecutive row elements per lane
constexpr int kReduceAhead = 8;     // partitions whose loads are in flight together

template <int DT, int D>
__global__ __launch_bounds__(kReduceThreads) void attn_reduce_kernel(AttnParams p, int B) {
  constexpr int E = kReduceElems;
  const int slots = p.num_kv_heads * p.chunks;
  const int s = blockIdx.x / slots;
  const int slot = blockIdx.x - s * slots;
  const int c = slot % p.chunks;
  const int q0 = slot / p.chunks * p.group + c * p.chunk_rows;
  const int rows = min(p.chunk_rows, p.group - c * p.chunk_rows);
  const SeqWork sw = seq_work(p, s, B);
  if (sw.bad || sw.nparts <= 1) return;     // written by the main kernel
  const int G = p.cap;                      // rows per run in the workspace
  const size_t run0 = ((size_t)s * slots + slot) * p.max_parts;   // partition 0's first row is run0 * G
  for (int e = threadIdx.x * E; e < rows * D; e += blockDim.x * E) {
    const int g = e / D, d = e - g * D;
    float M = -INFINITY, W = 0.f, O[E];
#pragma unroll
    for (int k = 0; k < E; ++k) O[k] = 0.f;
    for (int i0 = 0; i0 < sw.nparts; i0 += kReduceAhead) {
      float m[kReduceAhead], l[kReduceAhead], o[kReduceAhead][E];
#pragma unroll
      for (int k = 0; k < kReduceAhead; ++k) {
        const int i = min(i0 + k, sw.nparts - 1);
        const size_t row = (run0 + i) * G + g;
        const f32x2v ml = *reinterpret_cast<const f32x2v*>(p.ws_ml + row * 2);
        m[k] = ml[0];
        l[k] = ml[1];
        load8<DT>(p.ws_o, row * D + d, o[k]);
      }
#pragma unroll
      for (int k = 0; k < kReduceAhead; ++k) {
        if (i0 + k >= sw.nparts) break;
        const float Mn = fmaxf(M, m[k]);
        const float ref = softmax_ref(Mn);
        const float a = fast_exp2(M - ref);
        const float b = l[k] * fast_exp2(m[k] - ref);
        W = fmaf(W, a, b);
#pragma unroll
        for (int j = 0; j < E; ++j) O[j] = fmaf(O[j], a, o[k][j] * b);
        M = Mn;
      }
    }
    float r[E];
#pragma unroll
    for (int j = 0; j < E; ++j) r[j] = O[j] / W;
    store_row8<DT, false>(p.out, ((size_t)s * p.num_q_heads + q0 + g) * D + d, r);
    if (p.lse != nullptr && d == 0) p.lse[(size_t)s * p.num_q_heads + q0 + g] = M + log2f(W);
  }
}

namespace {
template <int DT, int D>
hipError_t launch_reduce(const AttnParams& p, int B, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.num_seqs * p.num_kv_heads * p.chunks));
  // Lanes take 8 elements each; small groups need fewer lanes.
  const int rows = p.chunk_rows * D / kReduceElems;
  const int threads = min(kReduceThreads, max(kWave, (rows + kWave - 1) / kWave * kWave));
  hipLaunchKernelGGL((attn_reduce_kernel<DT, D>), grid, dim3(threads), 0, st, p, B);
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
