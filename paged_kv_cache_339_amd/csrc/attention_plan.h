// Building the work list of a decode call (device code shared by the
// launches that build it): see attention_plan.hip.
#pragma once

#include "attention_common.h"

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

__device__ __forceinline__ SeqPlan plan_of(const AttnParams& p, const SeqWork& w) {
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

__device__ __forceinline__ SeqPlan seq_plan(const AttnParams& p, int s, int B) {
  return plan_of(p, seq_work(p, s, B));
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

  // Pass 1: count full partitions, histogram the rest.  The lengths (and
  // first tokens) of the cached chunks are all requested before any is
  // used, so the loads overlap instead of waiting one after another;
  // indices past the batch are clamped to its last sequence and their
  // values never used.
  SeqPlan cached[kPlanCached];
  int full_total = 0;
  int len[kPlanCached], first[kPlanCached];
#pragma unroll
  for (int c = 0; c < kPlanCached; ++c) len[c] = p.context_lens[min(c * kWave + lane, S - 1)];
#pragma unroll
  for (int c = 0; c < kPlanCached; ++c) first[c] = 0;
  if (p.seq_start != nullptr) {
#pragma unroll
    for (int c = 0; c < kPlanCached; ++c) first[c] = p.seq_start[min(c * kWave + lane, S - 1)];
  }
#pragma unroll
  for (int c = 0; c < kPlanCached; ++c) {
    const int s = c * kWave + lane;
    cached[c] = SeqPlan{0, -1};
    if (s < S) cached[c] = plan_of(p, seq_work_from(p, len[c], first[c], B));
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

}  // namespace pkv
