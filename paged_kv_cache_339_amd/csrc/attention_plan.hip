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

namespace pkv {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanBins = kPlanThreads;

// Exclusive prefix sum over the workgroup: a scan within each wave by lane
// shuffles, then the wave totals through LDS.  *total receives the sum.
__device__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = lane_id(), w = wave_id();
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int x = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += x;
  }
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    before += i < w ? wave_tot[i] : 0;
    sum += wave_tot[i];
  }
  __syncthreads();
  *total = sum;
  return before + incl - v;
}

// Bin of a last partition of r blocks (1 <= r < P): larger r, larger bin;
// bin 0 is kept for sequences without work.
__device__ __forceinline__ int size_bin(int r, int P) {
  return 1 + (int)((int64_t)(r - 1) * (kPlanBins - 1) / P);
}

__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(AttnParams p, int B) {
  __shared__ int bins[kPlanBins];
  __shared__ int wave_tot[kPlanWaves];
  __shared__ int full_total;
  const int t = threadIdx.x;
  const int P = p.part_blocks;
  bins[t] = 0;
  if (t == 0) full_total = 0;
  __syncthreads();

  // Pass 1: count full partitions, histogram the rest.
  for (int s = t; s < p.num_seqs; s += kPlanThreads) {
    const SeqWork w = seq_work(p, s, B);
    if (w.bad || w.L == 0) {
      atomicAdd(&bins[0], 1);
    } else {
      atomicAdd(&full_total, w.nblk / P);
      const int r = w.nblk % P;
      if (r) atomicAdd(&bins[size_bin(r, P)], 1);
    }
  }
  __syncthreads();

  // Start of each bin: full partitions first, then bins from the largest
  // size down, bin 0 last (thread t takes bin kPlanBins-1-t, the last thread
  // bin 0).
  {
    const int bin = t < kPlanBins - 1 ? kPlanBins - 1 - t : 0;
    int total;
    const int start = block_exclusive_scan(bins[bin], wave_tot, &total);
    const int nfull = full_total;
    __syncthreads();
    bins[bin] = nfull + start;
    if (t == 0) p.work->n_pairs = min(nfull + total, p.max_pairs);
    __syncthreads();
  }

  // Pass 2: write the pairs.  Full partitions keep sequence order (prefix sum
  // of their counts, chunk by chunk); the others take the next slot of their bin.
  int carry = 0;
  for (int base = 0; base < p.num_seqs; base += kPlanThreads) {
    const int s = base + t;
    SeqWork w;
    int nfull = 0;
    if (s < p.num_seqs) {
      w = seq_work(p, s, B);
      if (!w.bad && w.L > 0) nfull = w.nblk / P;
    }
    int chunk_total;
    const int first = carry + block_exclusive_scan(nfull, wave_tot, &chunk_total);
    carry += chunk_total;
    if (s < p.num_seqs) {
      for (int k = 0; k < nfull && first + k < p.max_pairs; ++k) p.pairs[first + k] = WorkPair{s, k};
      int pos = -1, part = 0;
      if (w.bad || w.L == 0) {
        pos = atomicAdd(&bins[0], 1);
      } else if (w.nblk % P) {
        pos = atomicAdd(&bins[size_bin(w.nblk % P, P)], 1);
        part = nfull;
      }
      if (pos >= 0 && pos < p.max_pairs) p.pairs[pos] = WorkPair{s, part};
    }
  }
}

hipError_t launch_attention_plan(const AttnParams& p, int block_size, hipStream_t stream) {
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p, block_size);
  return hipGetLastError();
}

}  // namespace pkv
