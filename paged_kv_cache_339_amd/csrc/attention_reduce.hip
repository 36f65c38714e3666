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
// row) per lane.  Up to kReduceSplit groups of lanes take the partitions in
// turn (group k of n: partitions k, k + n, ...), so the longest sequences
// wait on a quarter of the dependent load rounds.  Each group merges its
// partitions in order, as online softmax:
// M' = max(M, m_p), W = W 2^(M - M') + l_p 2^(m_p - M'), and O likewise with
// l_p 2^(m_p - M') o_p; group 0 then merges the groups' states in group
// order through LDS, and O / W equals the two-pass form above.
constexpr int kReduceLanes = 256;   // lanes per group at most
constexpr int kReduceSplit = 4;     // groups of lanes per workgroup
constexpr int kReduceElems = 8;     // consecutive row elements per lane
constexpr int kReduceAhead = 4;     // partitions per group whose loads are in flight together

// Online-softmax state of 8 elements of a row: running max, sum, output.
struct MergeState {
  float M, W, O[kReduceElems];
};

// Merge partition p: its normalised output o_p with (m_p, l_p).
__device__ __forceinline__ void merge_into(MergeState& st, float m, float l, const float (&o)[kReduceElems]) {
  const float Mn = fmaxf(st.M, m);
  const float ref = softmax_ref(Mn);
  const float a = fast_exp2(st.M - ref);
  const float b = l * fast_exp2(m - ref);
  st.W = fmaf(st.W, a, b);
#pragma unroll
  for (int j = 0; j < kReduceElems; ++j) st.O[j] = fmaf(st.O[j], a, o[j] * b);
  st.M = Mn;
}

// Merge another group's state, whose O is already weighted by its W.
__device__ __forceinline__ void merge_state(MergeState& st, const MergeState& o) {
  const float Mn = fmaxf(st.M, o.M);
  const float ref = softmax_ref(Mn);
  const float a = fast_exp2(st.M - ref);
  const float b = fast_exp2(o.M - ref);
  st.W = fmaf(st.W, a, o.W * b);
#pragma unroll
  for (int j = 0; j < kReduceElems; ++j) st.O[j] = fmaf(st.O[j], a, o.O[j] * b);
  st.M = Mn;
}

template <int DT, int D>
__global__ __launch_bounds__(kReduceLanes * kReduceSplit) void attn_reduce_kernel(AttnParams p, int B) {
  constexpr int E = kReduceElems;
  extern __shared__ MergeState lds[];      // [split - 1][per]
  const int slots = p.num_kv_heads * p.chunks;
  const int s = blockIdx.x / slots;
  const int slot = blockIdx.x - s * slots;
  const int c = slot % p.chunks;
  const int q0 = slot / p.chunks * p.group + c * p.chunk_rows;
  const int rows = min(p.chunk_rows, p.group - c * p.chunk_rows);
  const SeqWork sw = seq_work(p, s, B);
  if (sw.bad || sw.nparts <= 1) return;     // written by the main kernel (workgroup-uniform)
  const int G = p.cap;                      // rows per run in the workspace
  const size_t run0 = ((size_t)s * slots + slot) * p.max_parts;   // partition 0's first row is run0 * G
  const int split = min(kReduceSplit, p.max_parts);                // groups of lanes
  const int per = blockDim.x / split;                              // lanes per group
  const int grp = threadIdx.x / per, lt = threadIdx.x - grp * per;
  // Every lane runs the same number of rounds (barriers inside).
  for (int e0 = 0; e0 < rows * D; e0 += per * E) {
    const int e = e0 + lt * E;
    const bool live = e < rows * D;
    const int g = live ? e / D : 0, d = live ? e - g * D : 0;
    MergeState st;
    st.M = -INFINITY;
    st.W = 0.f;
#pragma unroll
    for (int k = 0; k < E; ++k) st.O[k] = 0.f;
    if (live) {
      for (int i0 = grp; i0 < sw.nparts; i0 += split * kReduceAhead) {
        float m[kReduceAhead], l[kReduceAhead], o[kReduceAhead][E];
#pragma unroll
        for (int k = 0; k < kReduceAhead; ++k) {
          const int i = min(i0 + k * split, sw.nparts - 1);
          const size_t row = (run0 + i) * G + g;
          const f32x2v ml = *reinterpret_cast<const f32x2v*>(p.ws_ml + row * 2);
          m[k] = ml[0];
          l[k] = ml[1];
          load8<DT>(p.ws_o, row * D + d, o[k]);
        }
#pragma unroll
        for (int k = 0; k < kReduceAhead; ++k) {
          if (i0 + k * split >= sw.nparts) break;
          merge_into(st, m[k], l[k], o[k]);
        }
      }
    }
    if (grp > 0) lds[(grp - 1) * per + lt] = st;
    __syncthreads();
    if (grp == 0 && live) {
#pragma unroll
      for (int k = 0; k < split - 1; ++k) merge_state(st, lds[k * per + lt]);
      float r[E];
#pragma unroll
      for (int j = 0; j < E; ++j) r[j] = st.O[j] / st.W;
      store_row8<DT, false>(p.out, ((size_t)s * p.num_q_heads + q0 + g) * D + d, r);
      if (p.lse != nullptr && d == 0) p.lse[(size_t)s * p.num_q_heads + q0 + g] = st.M + log2f(st.W);
    }
    __syncthreads();                        // the states are read before the next round writes them
  }
}

namespace {
template <int DT, int D>
hipError_t launch_reduce(const AttnParams& p, int B, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.num_seqs * p.num_kv_heads * p.chunks));
  // Lanes take 8 elements each: a group has the row's lanes rounded up to a
  // power of two (16 to 256), and a sequence of P partitions needs at most
  // P groups.
  const int lanes = p.chunk_rows * D / kReduceElems;
  int per = 16;
  while (per < lanes && per < kReduceLanes) per *= 2;
  const int split = min(kReduceSplit, p.max_parts);
  const size_t lds = (size_t)(split - 1) * per * sizeof(MergeState);
  hipLaunchKernelGGL((attn_reduce_kernel<DT, D>), grid, dim3(per * split), lds, st, p, B);
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
