// Pieces shared by the two decode-attention kernels (vector-ALU and MFMA)
// and the split-K reduce: per-sequence bookkeeping and the epilogue that
// merges the waves of a workgroup and stores either the final row or a
// partition's partial result.
//
// Online softmax state, per query head, kept in log2 units: m = running max
// of scale*log2(e)*<q,k_t>, l = sum_t 2^(x_t - m), o = sum_t 2^(x_t - m) v_t.
// Two states merge as m = max(m1, m2), l = l1 a1 + l2 a2, o = o1 a1 + o2 a2
// with ai = 2^(mi - m); a state that has seen no token has m = -inf, l = 0.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pkv {

// What one sequence asks of the kernels.  Attended tokens are [t0, L): all
// of them, or the last `window` with a sliding window ("pagedattention vllm"
// glossary, Advanced Features > Sliding Window).  Partition p covers blocks
// [blk0 + p*part_blocks, ...) of the nblk blocks from blk0 to the block of
// token L-1; blocks before blk0 are never read (their table entries may be
// -1 once released).
struct SeqWork {
  int L;        // one past the last attended token
  int t0;       // first attended token
  int blk0;     // logical block holding t0
  int nblk;     // blocks blk0 .. (L-1)/B
  int nparts;   // split-K partitions of the sequence
  bool bad;     // context length outside what the table / launch covers
};

// From the sequence's context length `raw` and, when the call has
// per-sequence first tokens (p.seq_start), its first token `start`.
__device__ __forceinline__ SeqWork seq_work_from(const AttnParams& p, int raw, int start, int B) {
  SeqWork w;
  w.bad = raw < 0 || raw > p.max_context_len ||
          (int64_t)raw > (int64_t)p.max_blocks_per_seq * B;
  w.L = w.bad ? 0 : raw;
  w.t0 = (p.window > 0 && w.L > p.window) ? w.L - p.window : 0;
  if (p.seq_start != nullptr) {
    if (start > w.t0) w.t0 = start;
    if (w.t0 >= w.L) w.L = w.t0 = 0;     // nothing left to attend to
  }
  w.blk0 = w.t0 / B;
  w.nblk = w.L > 0 ? (w.L + B - 1) / B - w.blk0 : 0;
  w.nparts = (w.nblk + p.part_blocks - 1) / p.part_blocks;
  return w;
}

__device__ __forceinline__ SeqWork seq_work(const AttnParams& p, int s, int B) {
  return seq_work_from(p, p.context_lens[s], p.seq_start != nullptr ? p.seq_start[s] : 0, B);
}

// Safe reference point for 2^(x - m) when m may be -inf.
__device__ __forceinline__ float softmax_ref(float m) { return m == -INFINITY ? 0.f : m; }

// Workgroup -> (sequence, KV head, head chunk, partition) through the plan.
// Work item u covers pair u / Hkv of the list and KV head u % Hkv; the grid
// covers every pair the list could hold, and workgroups past its end (and
// entries that do not name a sequence and partition of this call) do
// nothing.  With one chunk per KV head, workgroup u is item u.  With C > 1
// chunks the C workgroups of one item are numbered 8 apart: workgroups are
// dealt to the 8 XCDs in turn, so the chunks of an item run on one XCD at
// about the same time and read the item's key/value tiles through the same
// L2.
struct WorkItem {
  int s, h, part;  // sequence, KV head, partition
  int slot;        // h * C + chunk: the item's run in the workspace
  int q0, rows;    // first query head, query heads of the chunk
  bool valid;
};

__device__ __forceinline__ WorkItem work_item(const AttnParams& p) {
  const int lin = blockIdx.x;
  int u = lin, c = 0;
  if (p.chunks > 1) {
    const int j = lin >> 3, jc = j / p.chunks;
    u = jc * 8 + (lin & 7);
    c = j - jc * p.chunks;
  }
  const bool in_grid = u < p.items;
  const int pair = in_grid ? u / p.num_kv_heads : 0;
  WorkItem it;
  it.h = u - pair * p.num_kv_heads;
  it.slot = it.h * p.chunks + c;
  it.q0 = it.h * p.group + c * p.chunk_rows;
  it.rows = min(p.chunk_rows, p.group - c * p.chunk_rows);
  if (p.direct) {
    it.s = pair / p.max_parts;
    it.part = pair - it.s * p.max_parts;
    it.valid = in_grid && it.s < p.num_seqs && it.rows > 0;
    return it;
  }
  // The pair is loaded before the list length so that both loads are in
  // flight together (the other order made the compiler wait in between).
  const WorkPair wp = p.pairs[pair];
  const int n_pairs = min(p.work->n_pairs, p.max_pairs);
  it.s = wp.s;
  it.part = wp.part;
  it.valid = in_grid && pair < n_pairs && (unsigned)wp.s < (unsigned)p.num_seqs &&
             (unsigned)wp.part < (unsigned)p.max_parts && it.rows > 0;
  return it;
}

// Rows that cannot be computed (data error) become NaN, with a NaN
// log-denominator; empty sequences 0, with -inf.
template <int DT, int D, int NT>
__device__ __forceinline__ void fill_rows(const AttnParams& p, const WorkItem& it, float value) {
  for (int idx = threadIdx.x; idx < it.rows * D; idx += NT) {
    const int g = idx / D, d = idx % D;
    store_elem<DT>(p.out, ((size_t)it.s * p.num_q_heads + it.q0 + g) * D + d, value);
  }
  if (p.lse != nullptr)
    for (int g = threadIdx.x; g < it.rows; g += NT)
      p.lse[(size_t)it.s * p.num_q_heads + it.q0 + g] = value == 0.f ? -INFINITY : value;
}

// LDS staging for the cross-wave merge.
template <int D, int G, int NW>
struct MergeSmem {
  float o[NW][G][D];
  float m[NW][G];
  float l[NW][G];
  int bad[NW];
};

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Eight values rounded to a 16-bit format DT (nearest even), packed in
// element order into 16 bytes.
template <int DT>
__device__ __forceinline__ u32x4 pack_row8(const float (&x)[8]) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = DT == PKV_F16 ? narrow_f16(x[2 * k]) : narrow_bf16(x[2 * k]);
    const uint32_t hi = DT == PKV_F16 ? narrow_f16(x[2 * k + 1]) : narrow_bf16(x[2 * k + 1]);
    w[k] = lo | (hi << 16);
  }
  return w;
}

// Eight consecutive elements of one row, rounded to the stored format and
// written with one 16-byte store (two for fp32 rows); NTS: with the
// nontemporal hint.
template <int DT, bool NTS>
__device__ __forceinline__ void store_row8(void* base, size_t idx, const float (&x)[8]) {
  if constexpr (DT == PKV_F32) {
    float* dst = reinterpret_cast<float*>(base) + idx;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4v v = f32x4v{x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
      if constexpr (NTS) __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(dst + 4 * h));
      else *reinterpret_cast<f32x4v*>(dst + 4 * h) = v;
    }
  } else {
    const u32x4 w = pack_row8<DT>(x);
    u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + idx);
    if constexpr (NTS) __builtin_nontemporal_store(w, dst);
    else *dst = w;
  }
}

// Eight consecutive elements of a row stored in format DT, widened to fp32.
template <int DT>
__device__ __forceinline__ void load8(const void* base, size_t idx, float (&x)[8]) {
  if constexpr (DT == PKV_F32) {
    const f32x4v* src = reinterpret_cast<const f32x4v*>(reinterpret_cast<const float*>(base) + idx);
    const f32x4v a = src[0], b = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  } else {
    const u32x4 w = load16(reinterpret_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wi = w[i];
      x[2 * i] = widen_half<DT>(wi, false);
      x[2 * i + 1] = widen_half<DT>(wi, true);
    }
  }
}

// Raw-buffer descriptor word 3 on gfx9: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of a buffer store: sc1 (system-coherent scope), the data
// written through to memory.
constexpr int kStoreSc1 = 16;

// Eight consecutive elements of a split-K partial row, stored with the sc1
// policy into the workgroup's run of partial rows (`run`, `run_bytes`; a
// wave-uniform base, so the descriptor lives in scalar registers); `idx`:
// element offset in the run.
template <int DT>
__device__ __forceinline__ void store_partial8(void* run, uint32_t run_bytes, int idx, const float (&x)[8]) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(run, 0, run_bytes, kBufferWord3);
  if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 v = u32x4{__builtin_bit_cast(uint32_t, x[4 * h]), __builtin_bit_cast(uint32_t, x[4 * h + 1]),
                            __builtin_bit_cast(uint32_t, x[4 * h + 2]), __builtin_bit_cast(uint32_t, x[4 * h + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, (idx + 4 * h) * 4, 0, kStoreSc1);
    }
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(pack_row8<DT>(x), rs, idx * 2, 0, kStoreSc1);
  }
}

// After every wave has put its (m, l, o) for the chunk's heads into `sm`:
// merge the waves and store.  A sequence with one partition gets its final
// output rows; otherwise the partition's normalised output and (m, l) go to
// the workspace for the reduce kernel, laid out [S, Hkv*C, P, cap, D] (in
// the output format) and [S, Hkv*C, P, cap, 2] (fp32): one workgroup's rows
// form one contiguous run, and the partitions of a (sequence, chunk) follow
// each other.  Measured on the 512-token split of the 70B-style GQA layer,
// these rows cost ~12% of the main kernel although they are 0.8% of its
// bytes: the cost goes with the partial lines that leave L2 (the same
// stores aimed at a 4 KiB run that stays in L2 cost nothing, at a 64 MB run
// as much as at the whole workspace), so they are kept as narrow as the
// output itself.  NT (streamed key/value loads): the rows are written
// through with the sc1 policy, 1.2% faster on that layer than nontemporal
// or plain stores; with plain loads, whose blocks are meant to stay in
// cache, plain stores measured faster.
template <int DT, int D, int G, int NW, bool NT>
__device__ __forceinline__ void merge_and_store(const AttnParams& p, const MergeSmem<D, G, NW>& sm,
                                                const WorkItem& it, int nparts) {
  bool bad = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) bad |= sm.bad[w] != 0;
  // Each thread merges and stores eight consecutive elements of a row: every
  // store is a whole 16-byte run, and a wave writes whole cache lines.
  constexpr int V = 8, RU = D / V;   // elements per thread, threads per row
  for (int u = threadIdx.x; u < it.rows * RU; u += NW * kWave) {
    const int g = u / RU, d = (u - g * RU) * V;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][g]);
    const float ref = softmax_ref(M);
    float tot = 0.f, o[V];
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = fast_exp2(sm.m[w][g] - ref);
      tot = fmaf(sm.l[w][g], a, tot);
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = fmaf(sm.o[w][g][d + e], a, o[e]);
    }
    float r[V];
#pragma unroll
    for (int e = 0; e < V; ++e) r[e] = bad ? __builtin_nanf("") : o[e] / tot * p.v_scale;
    if (nparts == 1) {
      store_row8<DT, false>(p.out, ((size_t)it.s * p.num_q_heads + it.q0 + g) * D + d, r);
      if (p.lse != nullptr && d == 0)
        p.lse[(size_t)it.s * p.num_q_heads + it.q0 + g] = bad ? __builtin_nanf("") : M + log2f(tot);
    } else {
      const size_t row0 =
          (((size_t)it.s * p.num_kv_heads * p.chunks + it.slot) * p.max_parts + it.part) * G;
      if constexpr (NT) {
        constexpr int ES = DT == PKV_F32 ? 4 : 2;
        store_partial8<DT>(static_cast<char*>(p.ws_o) + row0 * D * ES, (uint32_t)(G * D * ES), g * D + d, r);
      } else {
        store_row8<DT, false>(p.ws_o, (row0 + g) * D + d, r);
      }
      if (d == 0) {
        const f32x2v ml = f32x2v{M, bad ? __builtin_nanf("") : tot};
        f32x2v* dst = reinterpret_cast<f32x2v*>(p.ws_ml + (row0 + g) * 2);
        if constexpr (NT) __builtin_nontemporal_store(ml, dst);
        else *dst = ml;
      }
    }
  }
}

}  // namespace pkv
