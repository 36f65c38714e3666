// Internal interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Work list of one decode call, written by the plan kernel into the head of
// the workspace and read by the attention kernels: (sequence, partition)
// pairs, longest work first.
struct WorkHeader {
  int32_t n_pairs;
  int32_t pad[63];
};
struct WorkPair {
  int32_t s;
  int32_t part;
};

// Everything the decode-attention kernels read.  Sizes are validated by the
// C ABI before a launch.
struct AttnParams {
  void* out;                  // [S, Hq, D]
  const void* q;              // [S, Hq, D]
  const void* k_cache;        // [N, Hkv, B, D]
  const void* v_cache;
  const int32_t* block_tables;  // [S, M]
  const int32_t* context_lens;  // [S]
  void* ws_o;                 // [S, Hkv*C, P, cap, D] partition outputs, normalised, output format
  float* ws_ml;               // [S, Hkv*C, P, cap, 2] (running max in log2 units, sum)
  WorkHeader* work;           // plan written by the plan kernel
  WorkPair* pairs;            // [max_pairs]
  float scale_log2;           // scale * log2(e), times k_scale for 8-bit caches
  float v_scale;              // 1, or the value-cache scale of 8-bit caches
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t num_blocks;
  int32_t part_blocks;        // blocks per split-K partition
  int32_t max_parts;          // partitions per sequence covered by the grid
  int32_t max_pairs;          // num_seqs * max_parts, the room of `pairs`
  int32_t window;             // sliding window in tokens, 0 = attend to all
  // Query heads: the G = Hq / Hkv heads of one KV head are served in C
  // chunks of at most R = ceil(G / C) heads, one workgroup per chunk; a
  // workgroup holds room for `cap` heads (its kernel's compile-time group).
  int32_t group;              // G
  int32_t chunks;             // C
  int32_t chunk_rows;         // R
  int32_t cap;                // rows per (sequence, chunk, partition) in the workspace
  int32_t items;              // S * Hkv * max_parts, work items per chunk
  // Optional (nullptr = none): first attended token of each sequence [S]
  // (tokens before it are skipped as before a sliding window), and the
  // log2 of each output row's softmax denominator [S, Hq], in the units of
  // scale_log2: log2 sum_t 2^(scale_log2 <q, k_t>) (-inf for an empty row).
  const int32_t* seq_start;
  float* lse;
  // Nonzero: the grid is small enough to be resident at once, so the order
  // of the work items does not matter; workgroup u takes pair u / Hkv as
  // (sequence, partition) = (pair / max_parts, pair % max_parts) and no
  // work list is built or read.
  int32_t direct;
  // Optional (new_k = nullptr: none), for a small-grid decode step on the
  // vector kernel with caches in the query format: the step's new tokens
  // [S, Hkv, D], stored by the workgroup of (sequence, KV head, partition 0,
  // chunk 0) at new_slots[s] (skipped outside [0, num_slots)), and read
  // from here instead of the cache as token L - 1 of their sequence.
  const char* new_k;
  const char* new_v;
  const int32_t* new_slots;
  int64_t num_slots;
  char* store_k_cache;        // the caches, writable (the decode step's own pointers)
  char* store_v_cache;
};

// Workgroups of a main-kernel launch: one per work item and head chunk;
// with several chunks the grid is rounded up to whole rounds of the 8 XCDs
// (the numbering work_item undoes).
inline size_t attn_grid(const AttnParams& p) {
  if (p.chunks <= 1) return (size_t)p.items;
  return ((size_t)p.items + 7) / 8 * 8 * (size_t)p.chunks;
}

// Returns false when no kernel instance exists for the combination; `cap`
// selects the instance (rows per workgroup, AttnParams::cap).
// dt: the query / output format; kv: the caches' (dt, or PKV_FP8_E4M3);
// keep: plain key/value loads (blocks shared across the batch are served
// again from cache) instead of nontemporal ones.
bool launch_attention_valu(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                           int block_size, int cap, bool keep, hipStream_t stream, hipError_t* err);
bool launch_attention_mfma(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                           int block_size, int cap, bool keep, hipStream_t stream, hipError_t* err);
// The two load policies' instances, each built in a translation unit of its own.
bool launch_attention_valu_stream(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                                  int block_size, int cap, hipStream_t stream, hipError_t* err);
bool launch_attention_valu_keep(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                                int block_size, int cap, hipStream_t stream, hipError_t* err);
bool launch_attention_mfma_stream(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                                  int block_size, int cap, hipStream_t stream, hipError_t* err);
bool launch_attention_mfma_keep(const AttnParams& p, pkv_dtype dt, pkv_dtype kv, int head_dim,
                                int block_size, int cap, hipStream_t stream, hipError_t* err);
hipError_t launch_attention_plan(const AttnParams& p, int block_size, hipStream_t stream);

// Host checks of pkv_paged_attention_decode except those on the workspace:
// PKV_OK (then *workspace_bytes = what the call needs) or the status the call
// would return.  Touches neither the runtime nor any pointer.
int decode_arg_status(const void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                      int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t max_context_len, int32_t num_blocks, pkv_dtype dtype,
                      const pkv_attn_options* opts, size_t* workspace_bytes);

// New tokens of a decode step (one per sequence), stored by the launch that
// builds the work list.
struct AppendArgs {
  const char* k;              // [num_seqs, Hkv, D]
  const char* v;
  char* k_cache;
  char* v_cache;
  const int32_t* slot_mapping;  // [num_seqs]
  int32_t chunks;             // 16-byte pieces per (token, head) row of the cache
  int64_t num_slots;          // num_blocks * block_size
  int32_t fp8;                // store E4M3 codes of x / scale (in_dtype rows)
  int32_t in_dtype;           // format of k, v when fp8
  int32_t head_dim;
  float k_scale, v_scale;
  int32_t split;              // workgroups (of one wave) per new token, >= 1
  int32_t plan;               // 0: workgroup 0 leaves the work list as it is
};
hipError_t launch_append_and_plan(const AttnParams& p, int block_size, const AppendArgs& a,
                                  hipStream_t stream);
bool launch_attention_reduce(const AttnParams& p, pkv_dtype dt, int head_dim, int block_size,
                             hipStream_t stream, hipError_t* err);

// Shared-prefix decode: the prep launch (virtual queries, tables, lengths
// of each group) and the merge of prefix and suffix parts.
struct PrefixArgs {
  const char* q;              // [S, Hq, D] query rows
  char* q_v;                  // [Gn, Hq * Gs, D] virtual query rows (workspace)
  const int32_t* tables;      // [S, M]
  int32_t* tables_v;          // [Gn, Mv] (workspace)
  const int32_t* prefix_lens; // [S]
  int32_t* lens_v;            // [Gn] (workspace)
  const int32_t* members;     // [Gn, Gs], -1 = unused slot
  int32_t num_seqs, num_groups, group_size, q_heads, group, row_pieces, max_blocks, tab_v;
  // Work lists the same launch builds: the grouped pass's (which then also
  // writes lens_v, from which it plans) and the own-token pass's.
  int32_t plan_pre, plan_suf;
};

struct PrefixMergeArgs {
  void* out;                  // [S, Hq, D]: the suffix parts on entry, the results on exit
  const float* lse;           // [S, Hq] log2-denominators of the suffix parts
  const void* o_v;            // [Gn, Hq * Gs, D] prefix parts of the virtual batch
  const float* lse_v;         // [Gn, Hq * Gs]
  const int32_t* members;     // [Gn, Gs]
  int32_t num_seqs, num_groups, group_size, q_heads, group;
};

// The shared-prefix call's first launch: the virtual batch (queries side by
// side, tables, lengths) and the two passes' work lists.  `pre` / `suf`: the
// grouped and own-token passes' parameters (used when a.plan_pre / a.plan_suf).
hipError_t launch_prefix_prep(const PrefixArgs& a, const AttnParams& pre, const AttnParams& suf,
                              int block_size, hipStream_t stream);
bool launch_prefix_merge(const PrefixMergeArgs& a, pkv_dtype dt, int head_dim, hipStream_t stream,
                         hipError_t* err);

hipError_t launch_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                        const int32_t* slot_mapping, int32_t num_tokens,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, pkv_dtype in_dtype, float k_scale,
                                        float v_scale, hipStream_t stream);
hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                                    int32_t num_blocks, hipStream_t stream);
hipError_t launch_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              int32_t num_src, int32_t num_dst, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, int32_t num_blocks, hipStream_t stream);
hipError_t launch_gather_kv(void* dst, const void* cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t max_context_len, int32_t kv_head,
                            int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                            int32_t num_blocks, hipStream_t stream);

}  // namespace pkv
