// Decode attention for groups of sequences that share the blocks of a common
// prefix (parallel samples of one prompt, beams): the blocks shared by
// reference count ("pagedattention vllm" glossary, Copy-on-Write Sharing:
// Prefix Sharing, Reference Counting and Use Cases; "What is PagedAttention"
// (tecyfy), What it changes) are read once per group instead of once per
// member.
//
// Softmax over the tokens [0, L) of a sequence splits exactly over the two
// ranges [0, P) and [P, L): with each part's normalised output o_a, o_b and
// log2-denominator l_a, l_b,
//     out = (o_a 2^(l_a - m) + o_b 2^(l_b - m)) / (2^(l_a - m) + 2^(l_b - m)),
// m = max(l_a, l_b) -- the same merge the split-K reduce applies to
// partitions.  The prefix part of every member of a group reads the same
// keys and values, so the group's members become the query heads of one
// "virtual" sequence: G members x g heads per KV head form a query group
// of G g heads, which the grouped-query kernels (matrix cores for 16-bit
// data) serve with one read of each prefix tile.
//
// Launches: prefix_prep_kernel (queries of each group's members side by
// side, the group's table row and prefix length, and the work lists of both
// passes), the decode kernels on the virtual batch, the decode kernels on the
// real batch starting each sequence at its prefix length, and
// prefix_merge_kernel.
#include "attention_plan.h"

namespace pkv {

// The group's first valid member: its table row and prefix length describe
// the shared prefix; -1 when the group has no member.
__device__ __forceinline__ int first_member(const PrefixArgs& a, int vg) {
  for (int j = 0; j < a.group_size; ++j) {
    const int m = a.members[(size_t)vg * a.group_size + j];
    if ((unsigned)m < (unsigned)a.num_seqs) return m;
  }
  return -1;
}

// The group's prefix length: its first valid member's (0 without one).
__device__ __forceinline__ int group_prefix_len(const PrefixArgs& a, int vg) {
  const int m = first_member(a, vg);
  return m >= 0 ? a.prefix_lens[m] : 0;
}

// Workgroups 0 and 1 build the own-token and grouped passes' work lists (when
// asked; the grouped pass's workgroup first writes the virtual lengths it
// plans from, lane l the groups l + 64 k, the same groups it then reads).
// The other workgroups grid-stride over three index ranges: 16-byte pieces
// of the virtual query rows, the virtual table entries and (unless
// workgroup 1 writes them) the virtual lengths.  Virtual head
// vh = h Gs g + j g + i of group vg is query head h g + i of member j.
// Workgroups of one wave: the plan is one wave's work.
__global__ __launch_bounds__(kWave) void prefix_prep_kernel(PrefixArgs a, AttnParams pre, AttnParams suf,
                                                             int B) {
  if (blockIdx.x == 0) {
    if (a.plan_suf) plan_body(suf, B);
    return;
  }
  if (blockIdx.x == 1) {
    if (a.plan_pre) {
      for (int vg = threadIdx.x; vg < a.num_groups; vg += kWave) a.lens_v[vg] = group_prefix_len(a, vg);
      __syncthreads();
      plan_body(pre, B);
    }
    return;
  }
  const int64_t vrows = (int64_t)a.num_groups * a.q_heads * a.group_size;
  const int64_t n_q = vrows * a.row_pieces;
  const int64_t n_t = (int64_t)a.num_groups * a.tab_v;
  const int64_t n = n_q + n_t + (a.plan_pre ? 0 : a.num_groups);
  const int per_kv = a.group_size * a.group;
  for (int64_t i = (blockIdx.x - 2) * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)(gridDim.x - 2) * blockDim.x) {
    if (i < n_q) {
      const int64_t row = i / a.row_pieces;
      const int piece = (int)(i - row * a.row_pieces);
      const int vg = (int)(row / ((int64_t)a.q_heads * a.group_size));
      const int vh = (int)(row - (int64_t)vg * a.q_heads * a.group_size);
      const int h = vh / per_kv, r = vh - h * per_kv, j = r / a.group, hi = r - j * a.group;
      const int m = a.members[(size_t)vg * a.group_size + j];
      u32x4 v = u32x4{0, 0, 0, 0};
      if ((unsigned)m < (unsigned)a.num_seqs)
        v = load16(a.q + (((size_t)m * a.q_heads + h * a.group + hi) * a.row_pieces + piece) * 16);
      store16(a.q_v + (size_t)i * 16, v);
    } else if (i < n_q + n_t) {
      const int64_t k = i - n_q;
      const int vg = (int)(k / a.tab_v), b = (int)(k - (int64_t)vg * a.tab_v);
      const int m = first_member(a, vg);
      a.tables_v[k] = m >= 0 ? a.tables[(size_t)m * a.max_blocks + b] : -1;
    } else {
      const int vg = (int)(i - n_q - n_t);
      a.lens_v[vg] = group_prefix_len(a, vg);
    }
  }
}

// One thread per 8 consecutive elements of a member's output row.
template <int DT, int D>
__global__ __launch_bounds__(256) void prefix_merge_kernel(PrefixMergeArgs a) {
  constexpr int RU = D / 8;
  const int64_t n = (int64_t)a.num_groups * a.group_size * a.q_heads * RU;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t row = i / RU;
  const int d = (int)(i - row * RU) * 8;
  const int hq = (int)(row % a.q_heads);
  const int64_t slot = row / a.q_heads;           // vg * Gs + j
  const int m = a.members[slot];
  if ((unsigned)m >= (unsigned)a.num_seqs) return;
  const int vg = (int)(slot / a.group_size), j = (int)(slot - (int64_t)vg * a.group_size);
  const int h = hq / a.group, hi = hq - h * a.group;
  const size_t vrow = (size_t)vg * a.q_heads * a.group_size + (size_t)h * a.group_size * a.group +
                      (size_t)j * a.group + hi;
  const size_t orow = (size_t)m * a.q_heads + hq;
  const float la = a.lse[orow], lb = a.lse_v[vrow];
  float x[8], y[8], r[8];
  load8<DT>(a.out, orow * D + d, x);
  load8<DT>(a.o_v, vrow * D + d, y);
  if (__builtin_isnan(la) || __builtin_isnan(lb)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = __builtin_nanf("");
  } else {
    const float mx = fmaxf(la, lb);
    const float ref = softmax_ref(mx);               // both empty: weights 0, result 0
    const float wa = fast_exp2(la - ref), wb = fast_exp2(lb - ref);
    const float tot = wa + wb;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = tot > 0.f ? fmaf(x[e], wa, y[e] * wb) / tot : 0.f;
  }
  store_row8<DT, false>(a.out, orow * D + d, r);
}

hipError_t launch_prefix_prep(const PrefixArgs& a, const AttnParams& pre, const AttnParams& suf,
                              int block_size, hipStream_t st) {
  const int64_t n = (int64_t)a.num_groups * a.q_heads * a.group_size * a.row_pieces +
                    (int64_t)a.num_groups * a.tab_v + a.num_groups;
  const int64_t blocks = 2 + std::min<int64_t>((n + kWave - 1) / kWave, 32768);
  hipLaunchKernelGGL(prefix_prep_kernel, dim3((unsigned)blocks), dim3(kWave), 0, st, a, pre, suf, block_size);
  return hipGetLastError();
}

namespace {
template <int DT>
bool merge_by_dim(const PrefixMergeArgs& a, int D, hipStream_t st, hipError_t* e) {
  const int64_t n = (int64_t)a.num_groups * a.group_size * a.q_heads * (D / 8);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (n == 0) {
    *e = hipSuccess;
    return true;
  }
  switch (D) {
    case 64: hipLaunchKernelGGL((prefix_merge_kernel<DT, 64>), dim3(blocks), dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((prefix_merge_kernel<DT, 128>), dim3(blocks), dim3(256), 0, st, a); break;
    default: return false;
  }
  *e = hipGetLastError();
  return true;
}
}  // namespace

bool launch_prefix_merge(const PrefixMergeArgs& a, pkv_dtype dt, int head_dim, hipStream_t st,
                         hipError_t* err) {
  switch (dt) {
    case PKV_F32: return merge_by_dim<PKV_F32>(a, head_dim, st, err);
    case PKV_F16: return merge_by_dim<PKV_F16>(a, head_dim, st, err);
    case PKV_BF16: return merge_by_dim<PKV_BF16>(a, head_dim, st, err);
    default: return false;
  }
}

}  // namespace pkv
