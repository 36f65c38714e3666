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
#include "attention_common.h"
#include "scatter.h"

namespace pkv {

// One wave does the whole plan: the work is a few hundred sequences, and a
// single wave needs no workgroup barriers.  Sequences s = lane + 64 k are
// held by lane `lane`; up to kPlanCached of them per lane stay in registers
// between the two passes, longer batches re-read context_lens.
constexpr int kPlanBins = 256;
constexpr int kPlanCached = 8;

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int x = __shfl_up(v, off, kWave);
    if (lane >= off) v += x;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Bin of a last partition of r blocks (1 <= r < P): larger r, larger bin;
// bin 0 is kept for sequences without work.
__device__ __forceinline__ int size_bin(int r, int P) {
  return 1 + (int)((int64_t)(r - 1) * (kPlanBins - 1) / P);
}

// What one sequence contributes: `nfull` full partitions, and one item in
// bin `bin` (a shorter last partition, or bin 0 for no work), or none (-1).
struct SeqPlan { int nfull, bin; };

__device__ __forceinline__ SeqPlan seq_plan(const AttnParams& p, int s, int B) {
  const SeqWork w = seq_work(p, s, B);
  SeqPlan sp;
  if (w.bad || w.L == 0) {
    sp.nfull = 0;
    sp.bin = 0;
  } else {
    sp.nfull = w.nblk / p.part_blocks;
    const int r = w.nblk % p.part_blocks;
    sp.bin = r ? size_bin(r, p.part_blocks) : -1;
  }
  return sp;
}

// Pass-2 step for one chunk of 64 sequences: full partitions at the running
// prefix `carry` (sequence order), the other item at the next slot of its bin.
__device__ __forceinline__ void write_pairs(const AttnParams& p, int s, SeqPlan sp, int* carry,
                                            int* bins) {
  const int incl = wave_inclusive_scan(sp.nfull);
  const int first = *carry + incl - sp.nfull;
  *carry += __shfl(incl, kWave - 1, kWave);
  for (int k = 0; k < sp.nfull && first + k < p.max_pairs; ++k) p.pairs[first + k] = WorkPair{s, k};
  if (sp.bin >= 0) {
    const int pos = atomicAdd(&bins[sp.bin], 1);
    if (pos < p.max_pairs) p.pairs[pos] = WorkPair{s, sp.nfull};
  }
}

__device__ __forceinline__ void plan_body(const AttnParams& p, int B) {
  __shared__ int bins[kPlanBins];
  const int lane = lane_id();
  const int S = p.num_seqs;
  const int chunks = (S + kWave - 1) / kWave;
#pragma unroll
  for (int i = 0; i < kPlanBins / kWave; ++i) bins[lane + i * kWave] = 0;
  __syncthreads();

  // Pass 1: count full partitions, histogram the rest.
  SeqPlan cached[kPlanCached];
  int full_total = 0;
#pragma unroll
  for (int c = 0; c < kPlanCached; ++c) {
    const int s = c * kWave + lane;
    cached[c] = SeqPlan{0, -1};
    if (s < S) cached[c] = seq_plan(p, s, B);
  }
#pragma unroll
  for (int c = 0; c < kPlanCached; ++c) {
    full_total += cached[c].nfull;
    if (cached[c].bin >= 0) atomicAdd(&bins[cached[c].bin], 1);
  }
  for (int c = kPlanCached; c < chunks; ++c) {
    const int s = c * kWave + lane;
    SeqPlan sp{0, -1};
    if (s < S) sp = seq_plan(p, s, B);
    full_total += sp.nfull;
    if (sp.bin >= 0) atomicAdd(&bins[sp.bin], 1);
  }
  full_total = wave_sum(full_total);
  __syncthreads();

  // Start of each bin: full partitions first, then bins from the largest
  // size down, bin 0 last.  Lane l owns the four bins 255-4l .. 252-4l.
  {
    int cnt[kPlanBins / kWave], local = 0;
#pragma unroll
    for (int i = 0; i < kPlanBins / kWave; ++i) {
      cnt[i] = bins[kPlanBins - 1 - (lane * (kPlanBins / kWave) + i)];
      local += cnt[i];
    }
    const int incl = wave_inclusive_scan(local);
    int start = full_total + incl - local;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPlanBins / kWave; ++i) {
      const int b = kPlanBins - 1 - (lane * (kPlanBins / kWave) + i);
      // bin 0 goes after every other bin: the scan order puts it last already.
      bins[b] = start;
      start += cnt[i];
    }
    if (lane == kWave - 1) p.work->n_pairs = min(full_total + incl, p.max_pairs);
    __syncthreads();
  }

  // Pass 2: full partitions in sequence order, the rest into their bins.
  int carry = 0;
#pragma unroll
  for (int c = 0; c < kPlanCached; ++c) {
    if (c < chunks) write_pairs(p, c * kWave + lane, cached[c], &carry, bins);
  }
  for (int c = kPlanCached; c < chunks; ++c) {
    const int s = c * kWave + lane;
    SeqPlan sp{0, -1};
    if (s < S) sp = seq_plan(p, s, B);
    write_pairs(p, s, sp, &carry, bins);
  }
}

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
