// Work list of a decode call.  The grid of the attention kernels is sized on
// the host from the largest context length, but how much work each sequence
// brings is only known on the device (context_lens lives there).  One
// workgroup turns context_lens into the list of (sequence, split-K
// partition) pairs the attention kernels walk, ordered longest first:
//   1. every full partition (part_blocks blocks), sequence by sequence;
//   2. the shorter last partitions, by decreasing size (coarse size bins);
//   3. empty or invalid sequences (their rows are zero- or NaN-filled).
// Workgroups are dispatched in grid order, so the long pieces start first
// and the kernel ends on the shortest ones instead of on a straggler; grid
// slots past the end of the list do nothing and come last.
// The order only schedules work: each pair's result does not depend on it.
#include "attention_plan.h"
#include "scatter.h"

namespace pkv {

__global__ __launch_bounds__(kWave) void attn_plan_kernel(AttnParams p, int B) { plan_body(p, B); }

// A decode step's first launch: workgroup 0 builds the work list (unless the
// caller reuses the one the workspace holds), the next a.split workgroups
// store sequence 0's new token, the next a.split sequence 1's, and so on.
// Neither part reads what the other writes (the plan reads only
// context_lens), so they share one launch.
__global__ __launch_bounds__(kWave) void append_and_plan_kernel(AttnParams p, int B, AppendArgs a) {
  if (blockIdx.x == 0) {
    if (a.plan) plan_body(p, B);
    return;
  }
  const int i = (blockIdx.x - 1) / a.split;
  const int first = (blockIdx.x - 1 - i * a.split) * kWave + threadIdx.x;
  const int stride = a.split * kWave;
  if (!a.fp8) {
    scatter_token(a.k, a.v, a.k_cache, a.v_cache, a.slot_mapping, i, first, stride, p.num_kv_heads,
                  a.chunks, B, a.num_slots);
  } else if (a.in_dtype == PKV_F16) {
    scatter_token_fp8<PKV_F16>(a.k, a.v, a.k_cache, a.v_cache, a.slot_mapping, i, first, stride,
                               p.num_kv_heads, a.head_dim, B, a.num_slots, a.k_scale, a.v_scale);
  } else if (a.in_dtype == PKV_BF16) {
    scatter_token_fp8<PKV_BF16>(a.k, a.v, a.k_cache, a.v_cache, a.slot_mapping, i, first, stride,
                                p.num_kv_heads, a.head_dim, B, a.num_slots, a.k_scale, a.v_scale);
  }
}

hipError_t launch_append_and_plan(const AttnParams& p, int block_size, const AppendArgs& a,
                                  hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)p.num_seqs * a.split + 1);
  hipLaunchKernelGGL(append_and_plan_kernel, dim3(grid), dim3(kWave), 0, stream, p, block_size, a);
  return hipGetLastError();
}

hipError_t launch_attention_plan(const AttnParams& p, int block_size, hipStream_t stream) {
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kWave), 0, stream, p, block_size);
  return hipGetLastError();
}

}  // namespace pkv
