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
// are one contiguous run, read 4 elements per lane.  The merge runs over the
// partitions in order, as online softmax:
// M' = max(M, m_p), W = W 2^(M - M') + l_p 2^(m_p - M'), and O likewise with
// l_p 2^(m_p - M') o_p; the result O / W equals the two-pass form above.
constexpr int kReduceThreads = 256;

// Four consecutive partition-output elements (stored in the output format).
template <int DT>
__device__ __forceinline__ float4 load4(const void* base, size_t idx) {
  if constexpr (DT == PKV_F32) {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
    return make_float4(widen_half<DT>(w.x, false), widen_half<DT>(w.x, true),
                       widen_half<DT>(w.y, false), widen_half<DT>(w.y, true));
  }
}
constexpr int kReduceAhead = 4;     // partitions whose loads are in flight together

template <int DT, int D>
__global__ __launch_bounds__(kReduceThreads) void attn_reduce_kernel(AttnParams p, int B) {
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
  for (int e = threadIdx.x * 4; e < rows * D; e += blockDim.x * 4) {
    const int g = e / D, d = e - g * D;
    float M = -INFINITY, W = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = 0; i0 < sw.nparts; i0 += kReduceAhead) {
      float m[kReduceAhead], l[kReduceAhead];
      float4 o[kReduceAhead];
#pragma unroll
      for (int k = 0; k < kReduceAhead; ++k) {
        const int i = min(i0 + k, sw.nparts - 1);
        const size_t row = (run0 + i) * G + g;
        m[k] = p.ws_ml[row * 2];
        l[k] = p.ws_ml[row * 2 + 1];
        o[k] = load4<DT>(p.ws_o, row * D + d);
      }
#pragma unroll
      for (int k = 0; k < kReduceAhead; ++k) {
        if (i0 + k >= sw.nparts) break;
        const float Mn = fmaxf(M, m[k]);
        const float ref = softmax_ref(Mn);
        const float a = fast_exp2(M - ref);
        const float b = l[k] * fast_exp2(m[k] - ref);
        W = fmaf(W, a, b);
        O.x = fmaf(O.x, a, o[k].x * b);
        O.y = fmaf(O.y, a, o[k].y * b);
        O.z = fmaf(O.z, a, o[k].z * b);
        O.w = fmaf(O.w, a, o[k].w * b);
        M = Mn;
      }
    }
    const size_t out0 = ((size_t)s * p.num_q_heads + q0 + g) * D + d;
    store_elem<DT>(p.out, out0, O.x / W);
    store_elem<DT>(p.out, out0 + 1, O.y / W);
    store_elem<DT>(p.out, out0 + 2, O.z / W);
    store_elem<DT>(p.out, out0 + 3, O.w / W);
  }
}

namespace {
template <int DT, int D>
hipError_t launch_reduce(const AttnParams& p, int B, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.num_seqs * p.num_kv_heads * p.chunks));
  // Lanes take 4 elements each; small groups need fewer lanes.
  const int rows = p.chunk_rows * D / 4;
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
