// C ABI of libpkv: argument checks, split-K planning and kernel dispatch.
// Nothing here touches device memory; every device pointer is handed to a
// kernel launched on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "kernels.h"
#include "pkv.h"

namespace {

// Most workgroups one launch may have: a dispatch counts work-items in 32
// bits, and the kernels run up to 256 threads per workgroup.
constexpr int64_t kMaxGrid = 0xffffffffll / 256;
// Automatic split-K partition.  With at least kNoSplitPairs (sequence, KV
// head) pairs, one partition per sequence: an MI355X keeps 768 (MFMA
// kernel) to 1280 (vector kernel) workgroups resident, the plan orders the
// items longest first so the last ones are short, and a split would only
// add partial results, whose writes into the saturated read stream cost far
// more than their bytes (measured on the 7B/13B/GQA layers).  Fewer pairs
// leave the chip underfilled: then the span is cut into equal partitions of
// about the smallest power of two of at least kMinAutoPartition tokens that
// gives kFillItems work items when every sequence is as long as the longest
// (one GPU's share of the GQA layer under 4- and 8-way tensor parallelism:
// 73% -> 78% and 71% -> 73% of peak).  A sliding window makes every long
// sequence's span the same, so there is no long item to break up: windowed
// batches split only below kNoSplitPairs / 4 pairs (the 512-pair
// sliding-window layer measured ~1% slower split into five).
constexpr int64_t kNoSplitPairs = 2048;
constexpr int64_t kFillItems = 4096;
constexpr int64_t kMinAutoPartition = 1024;
// A grid of at most this many workgroups (one per compute unit) is resident
// at once: the order of its items does not matter, so no work list is built.
constexpr int64_t kDirectGrid = 256;

int dtype_bytes(pkv_dtype dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_block(int32_t b) { return b == 8 || b == 16 || b == 32 || b == 64; }

// Workspace layout: [work header][work pairs][partition outputs][partition (m, l)].
struct Plan {
  int kernel;
  bool fp8;
  bool keep;          // plain key/value loads (PKV_CACHE_KEEP, or head chunks)
  bool direct;        // small grid: items taken in grid order, no work list
  int32_t chunks;     // workgroups per (sequence, KV head, partition)
  int32_t chunk_rows; // query heads per chunk (the last may have fewer)
  int32_t cap;        // instance's query heads per workgroup, >= chunk_rows
  int32_t window;
  int32_t part_blocks;
  int32_t max_parts;
  int64_t max_pairs;
  size_t pairs_off;
  size_t ws_o_off;
  size_t ws_ml_off;
  size_t ws_bytes;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size, int32_t max_context_len, pkv_dtype dtype,
              const pkv_attn_options* opts, Plan* plan) {
  if (dtype_bytes(dtype) == 0 || dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0)
    return PKV_ERR_SHAPE;
  const int32_t cache_policy = opts ? opts->cache_policy : PKV_CACHE_STREAM;
  if (cache_policy != PKV_CACHE_STREAM && cache_policy != PKV_CACHE_KEEP) return PKV_ERR_SHAPE;
  plan->keep = cache_policy == PKV_CACHE_KEEP;
  const int32_t kv_format = opts ? opts->kv_format : PKV_KV_SAME;
  if (kv_format != PKV_KV_SAME && kv_format != PKV_KV_FP8_E4M3) return PKV_ERR_DTYPE;
  const bool fp8 = kv_format == PKV_KV_FP8_E4M3;
  if (fp8) {
    if (dtype == PKV_F32) return PKV_ERR_UNSUPPORTED;
    if (!good_scale(opts->k_scale) || !good_scale(opts->v_scale)) return PKV_ERR_SHAPE;
  }
  if (num_q_heads % num_kv_heads) return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (!pow2_block(block_size)) return PKV_ERR_UNSUPPORTED;
  // Query heads per KV head: any G.  The matrix-core kernel pads a chunk's
  // heads to whole 16-column tiles of its products (up to 64 heads), the
  // vector kernel computes up to 8 per workgroup; a larger group is cut into
  // C equal chunks, each a workgroup of its own that reads the same
  // key/value tiles.
  const int group = num_q_heads / num_kv_heads;
  const bool sixteen_bit = dtype != PKV_F32;
  int kernel = opts ? opts->kernel : PKV_KERNEL_AUTO;
  if (kernel == PKV_KERNEL_AUTO)
    kernel = (sixteen_bit && group >= 3) ? PKV_KERNEL_MFMA : PKV_KERNEL_VALU;
  if (kernel != PKV_KERNEL_MFMA && kernel != PKV_KERNEL_VALU) return PKV_ERR_SHAPE;
  if (kernel == PKV_KERNEL_MFMA && !sixteen_bit) return PKV_ERR_UNSUPPORTED;
  if (fp8 && (block_size == 8 || block_size == 64)) return PKV_ERR_UNSUPPORTED;
  // Matrix cores: up to 4 (head_dim 64) or 2 (128) column tiles of 16
  // heads per wave with 16- and 32-token blocks, one tile otherwise.
  const int tiles = kernel != PKV_KERNEL_MFMA ? 1
                    : (block_size == 16 || block_size == 32) ? (head_dim == 64 ? 4 : 2) : 1;
  const int max_rows = kernel == PKV_KERNEL_MFMA ? 16 * tiles : 8;
  plan->chunks = (group + max_rows - 1) / max_rows;
  plan->chunk_rows = (group + plan->chunks - 1) / plan->chunks;
  if ((int64_t)(plan->chunks - 1) * plan->chunk_rows >= group) return PKV_ERR_SHAPE;
  const int rows = plan->chunk_rows;
  if (kernel == PKV_KERNEL_MFMA)
    plan->cap = rows <= 4 ? 4 : rows <= 8 ? 8 : (rows + 15) / 16 * 16;
  else
    plan->cap = rows <= 2 ? rows : rows <= 4 ? 4 : 8;
  // Chunks of one item share its key/value tiles through L2, which the
  // nontemporal loads would not fill.
  if (plan->chunks > 1) plan->keep = true;

  // Partition boundaries must fall on block boundaries, and on 32-token
  // chunk boundaries for the MFMA kernel.
  const int32_t align = kernel == PKV_KERNEL_MFMA ? (block_size > 32 ? block_size : 32) : block_size;
  int32_t part = opts ? opts->partition_size : 0;
  const int32_t window = opts ? opts->sliding_window : 0;
  if (part < 0 || window < 0) return PKV_ERR_SHAPE;
  if (part > 0 && part % align) return PKV_ERR_SHAPE;

  // Blocks one sequence can ask for: its whole context, or those a window of
  // `window` tokens can touch (it may start inside a block).
  const int64_t ctx_blocks = ((int64_t)max_context_len + block_size - 1) / block_size;
  int64_t span_blocks = ctx_blocks;
  if (window > 0) {
    const int64_t w_blocks = ((int64_t)window + block_size - 1) / block_size + 1;
    if (w_blocks < span_blocks) span_blocks = w_blocks;
  }
  const int64_t span_tokens = span_blocks * block_size;
  if (part == 0) {
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    int64_t p = span_tokens;
    if (pairs < (window > 0 ? kNoSplitPairs / 4 : kNoSplitPairs)) {
      const int64_t want = (span_tokens * pairs + kFillItems - 1) / kFillItems;
      int64_t p2 = kMinAutoPartition;
      while (p2 < want && p2 < span_tokens) p2 <<= 1;
      // A span at most a quarter past p2 stays whole; a longer one is cut
      // into equal pieces, so no sliver of a block or two is left over.
      if (span_tokens > p2 + p2 / 4) {
        const int64_t n = (span_tokens + p2 - 1) / p2;
        p = (span_tokens + n - 1) / n;
      }
    }
    part = (int32_t)(p < 0x40000000 ? p : 0x40000000);
  }
  part = (int32_t)round_up(part, align);

  if (span_tokens <= part) {
    plan->part_blocks = (int32_t)(span_blocks > 0 ? span_blocks : 1);
    plan->max_parts = 1;
  } else {
    plan->part_blocks = part / block_size;
    plan->max_parts = (int32_t)((span_blocks + plan->part_blocks - 1) / plan->part_blocks);
  }
  plan->window = window;
  plan->fp8 = fp8;
  const int64_t items = (int64_t)num_seqs * num_kv_heads * plan->max_parts;
  const int64_t grid = plan->chunks > 1 ? (items + 7) / 8 * 8 * plan->chunks : items;
  if (grid > kMaxGrid) return PKV_ERR_SHAPE;
  plan->kernel = kernel;
  plan->direct = grid <= kDirectGrid;
  plan->max_pairs = (int64_t)num_seqs * plan->max_parts;
  plan->pairs_off = round_up(sizeof(pkv::WorkHeader), 256);
  plan->ws_o_off = plan->pairs_off + round_up((size_t)plan->max_pairs * sizeof(pkv::WorkPair), 256);
  plan->ws_ml_off = plan->ws_o_off;
  if (plan->max_parts > 1) {
    const size_t rows =
        (size_t)num_seqs * num_kv_heads * plan->chunks * plan->max_parts * plan->cap;
    // Partition outputs are kept in the output format: the split-K writes
    // are the dearest bytes of a split (written into a saturated read stream).
    plan->ws_ml_off = plan->ws_o_off + round_up(rows * head_dim * dtype_bytes(dtype), 256);
    plan->ws_bytes = plan->ws_ml_off + round_up(rows * 2 * sizeof(float), 256);
  } else {
    plan->ws_bytes = plan->ws_o_off;
  }
  if (num_seqs == 0) plan->ws_bytes = 0;
  return PKV_OK;
}

thread_local char g_last_error[256] = "";

int launch_status(hipError_t e) {
  if (e == hipSuccess) return PKV_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s (hipError %d)", hipGetErrorString(e), (int)e);
  return PKV_ERR_LAUNCH;
}

// Clear an error left pending by earlier runtime calls of the caller, so the
// check after a launch reports that launch only.
void clear_pending_error() { (void)hipGetLastError(); }

// A kernel may address `p` as is: device memory, or pinned host memory that
// the runtime maps at the same address on the device.  Pageable host memory
// and unknown pointers are refused instead of being dereferenced.
bool device_addressable(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type == hipMemoryTypeDevice) return true;
  return a.type == hipMemoryTypeHost && a.devicePointer != nullptr &&
         a.devicePointer == a.hostPointer;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error; }

const char* pkv_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid or inconsistent size";
    case PKV_ERR_DTYPE: return "unknown dtype";
    case PKV_ERR_UNSUPPORTED: return "no kernel for this combination";
    case PKV_ERR_ALIGN: return "data pointer not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_NO_BLOCKS: return "block pool exhausted";
    case PKV_ERR_STATE: return "invalid block manager state or sequence";
    case PKV_ERR_CAPACITY: return "output buffer too small";
    case PKV_ERR_SCRATCH: return "needs more than the fixed scratch buffer holds";
    default: return "unknown status";
  }
}

int pkv_paged_attention_plan_info(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                  pkv_dtype dtype, const pkv_attn_options* opts,
                                  int32_t* partition_size, int32_t* max_parts, int32_t* kernel) {
  Plan plan;
  const int st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, dtype, opts, &plan);
  if (st != PKV_OK) return st;
  if (partition_size) *partition_size = plan.part_blocks * block_size;
  if (max_parts) *max_parts = plan.max_parts;
  if (kernel) *kernel = plan.kernel;
  return PKV_OK;
}

size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_context_len,
                                           pkv_dtype dtype, const pkv_attn_options* opts) {
  Plan plan;
  if (make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len, dtype,
                opts, &plan) != PKV_OK)
    return 0;
  return plan.ws_bytes;
}

}  // extern "C"

namespace {

// Every host check of a decode call except those on the workspace, which
// needs plan->ws_bytes bytes (after PKV_OK).
int decode_checks(const void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, float scale,
                  int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                  int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                  int32_t num_blocks, pkv_dtype dtype, const pkv_attn_options* opts, Plan* plan) {
  const int st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, dtype, opts, plan);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_NULL;
  if (max_blocks_per_seq <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_ALIGN;
  return PKV_OK;
}

}  // namespace

namespace pkv {

int decode_arg_status(const void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                      int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t max_context_len, int32_t num_blocks, pkv_dtype dtype,
                      const pkv_attn_options* opts, size_t* workspace_bytes) {
  Plan plan;
  const int st = decode_checks(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                               block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                               max_blocks_per_seq, max_context_len, num_blocks, dtype, opts, &plan);
  if (st == PKV_OK) *workspace_bytes = plan.ws_bytes;
  return st;
}

}  // namespace pkv

namespace {

// The checks of a decode call on its workspace, then its kernel
// parameters (no new tokens).  Touches no device memory.
int decode_setup(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                 int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                 int32_t num_blocks, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                 const pkv_attn_options* opts, const int32_t* seq_start, float* lse, Plan* plan,
                 pkv::AttnParams* pp) {
  const int st = decode_checks(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                               block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                               max_blocks_per_seq, max_context_len, num_blocks, dtype, opts, plan);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!workspace || workspace_bytes < plan->ws_bytes) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_ALIGN;

  pkv::AttnParams& p = *pp;
  p = pkv::AttnParams{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  p.work = reinterpret_cast<pkv::WorkHeader*>(ws);
  p.pairs = reinterpret_cast<pkv::WorkPair*>(ws + plan->pairs_off);
  p.ws_o = plan->max_parts > 1 ? static_cast<void*>(ws + plan->ws_o_off) : nullptr;
  p.ws_ml = plan->max_parts > 1 ? reinterpret_cast<float*>(ws + plan->ws_ml_off) : nullptr;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634 * (plan->fp8 ? (double)opts->k_scale : 1.0));
  p.v_scale = plan->fp8 ? opts->v_scale : 1.f;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.num_blocks = num_blocks;
  p.part_blocks = plan->part_blocks;
  p.max_parts = plan->max_parts;
  p.max_pairs = (int32_t)plan->max_pairs;
  p.window = plan->window;
  p.group = num_q_heads / num_kv_heads;
  p.chunks = plan->chunks;
  p.chunk_rows = plan->chunk_rows;
  p.cap = plan->cap;
  p.items = (int32_t)((int64_t)num_seqs * num_kv_heads * plan->max_parts);
  p.seq_start = seq_start;
  p.lse = lse;
  p.direct = plan->direct ? 1 : 0;
  return PKV_OK;
}

// A call whose work list is in place (or not needed): the main kernel
// between the optional timing events, then the split-K reduce.
int decode_attend(const Plan& plan, const pkv::AttnParams& p, pkv_dtype dtype, int32_t head_dim,
                  int32_t block_size, const pkv_attn_options* opts, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (opts && opts->main_begin_event) {
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(opts->main_begin_event), s);
    if (e != hipSuccess) return launch_status(e);
  }
  const bool have = plan.kernel == PKV_KERNEL_MFMA
                        ? pkv::launch_attention_mfma(p, dtype, plan.fp8 ? PKV_FP8_E4M3 : dtype,
                                                     head_dim, block_size, plan.cap, plan.keep, s, &err)
                        : pkv::launch_attention_valu(p, dtype, plan.fp8 ? PKV_FP8_E4M3 : dtype,
                                                     head_dim, block_size, plan.cap, plan.keep, s, &err);
  if (!have) return PKV_ERR_UNSUPPORTED;
  if (err != hipSuccess) return launch_status(err);
  if (opts && opts->main_end_event) {
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(opts->main_end_event), s);
    if (e != hipSuccess) return launch_status(e);
  }
  if (plan.max_parts > 1) {
    if (!pkv::launch_attention_reduce(p, dtype, head_dim, block_size, s, &err))
      return PKV_ERR_UNSUPPORTED;
    if (err != hipSuccess) return launch_status(err);
  }
  return PKV_OK;
}

// Decode attention; with `append`, the launch that builds the work list also
// stores every sequence's new token (a decode step in two launches).
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, float scale,
                int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                int32_t num_blocks, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                const pkv_attn_options* opts, void* stream, pkv::AppendArgs* append) {
  Plan plan;
  pkv::AttnParams p;
  const int st = decode_setup(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                              num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                              max_context_len, num_blocks, dtype, workspace, workspace_bytes, opts,
                              nullptr, nullptr, &plan, &p);
  if (st != PKV_OK || num_seqs == 0) return st;
  // A small-grid decode step on the vector kernel (caches in the query
  // format) runs in one launch: the attention workgroups store the new
  // tokens and read them from the inputs.
  const bool fuse = append != nullptr && plan.direct && plan.kernel == PKV_KERNEL_VALU && !plan.fp8 &&
                    !append->fp8;
  p.new_k = fuse ? append->k : nullptr;
  p.new_v = fuse ? append->v : nullptr;
  p.new_slots = fuse ? append->slot_mapping : nullptr;
  p.num_slots = fuse ? append->num_slots : 0;
  p.store_k_cache = fuse ? append->k_cache : nullptr;
  p.store_v_cache = fuse ? append->v_cache : nullptr;

  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_pending_error();
  const bool reuse = opts && opts->reuse_plan;
  hipError_t err = hipSuccess;
  if (append && !fuse) {
    append->plan = (reuse || plan.direct) ? 0 : 1;
    err = pkv::launch_append_and_plan(p, block_size, *append, s);
  } else if (!append && !reuse && !plan.direct) {
    err = pkv::launch_attention_plan(p, block_size, s);
  }
  if (err != hipSuccess) return launch_status(err);
  return decode_attend(plan, p, dtype, head_dim, block_size, opts, s);
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, int32_t block_size, int32_t num_kv_heads,
                               int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int32_t num_blocks, pkv_dtype dtype, void* workspace,
                               size_t workspace_bytes, const pkv_attn_options* opts,
                               void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                     num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                     max_context_len, num_blocks, dtype, workspace, workspace_bytes, opts, stream,
                     nullptr);
}

int pkv_decode_step(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, const int32_t* slot_mapping, const int32_t* block_tables,
                    const int32_t* context_lens, float scale, int32_t block_size,
                    int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks,
                    pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                    const pkv_attn_options* opts, void* stream) {
  const int es = dtype_bytes(dtype);
  if (!es) return PKV_ERR_DTYPE;
  if (num_seqs > 0) {
    if (!k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_ALIGN;
  }
  const bool fp8 = opts && opts->kv_format == PKV_KV_FP8_E4M3;
  pkv::AppendArgs a;
  a.plan = 1;
  a.k = static_cast<const char*>(k_new);
  a.v = static_cast<const char*>(v_new);
  a.k_cache = static_cast<char*>(k_cache);
  a.v_cache = static_cast<char*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.chunks = fp8 ? head_dim / 16 : head_dim * es / 16;
  a.num_slots = (int64_t)num_blocks * block_size;
  a.fp8 = fp8 ? 1 : 0;
  a.in_dtype = dtype;
  a.head_dim = head_dim;
  a.k_scale = fp8 ? opts->k_scale : 1.f;
  a.v_scale = fp8 ? opts->v_scale : 1.f;
  // Workgroups of 64 lanes per new token: about two 16-byte pieces per lane,
  // one for 8-bit caches (each code takes an IEEE division).
  const int64_t per_tok = (int64_t)(num_kv_heads > 0 ? num_kv_heads : 1) * a.chunks;
  const int64_t per_wg = 64 * (fp8 ? 1 : 2);
  a.split = (int32_t)std::min<int64_t>(16, std::max<int64_t>(1, (per_tok + per_wg - 1) / per_wg));
  if ((int64_t)num_seqs * a.split + 1 > kMaxGrid) return PKV_ERR_SHAPE;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                     num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                     max_context_len, num_blocks, dtype, workspace, workspace_bytes, opts, stream, &a);
}

}  // extern "C"

namespace {

// Workspace of a shared-prefix call: the virtual batch (queries, tables,
// lengths, outputs and log-denominators), the real batch's log-denominators,
// then the workspaces of the two decode passes.
struct PrefixLayout {
  int32_t tab_v;
  size_t q_v, tables_v, lens_v, o_v, lse_v, lse_t, ws_pre, ws_suf, bytes;
  size_t ws_pre_bytes, ws_suf_bytes;
  pkv_attn_options pre, suf;
};

int prefix_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t max_context_len, int32_t num_groups,
                  int32_t group_size, int32_t max_prefix_len, pkv_dtype dtype,
                  const pkv_attn_options* opts, PrefixLayout* L) {
  pkv_attn_options o{};
  if (opts) o = *opts;
  if (o.sliding_window != 0) return PKV_ERR_UNSUPPORTED;
  if (num_groups < 0 || max_prefix_len < 0 || max_prefix_len > max_context_len) return PKV_ERR_SHAPE;
  if (num_groups > 0 && group_size <= 0) return PKV_ERR_SHAPE;
  if (num_groups == 0) group_size = 1;
  const int64_t vheads = (int64_t)num_q_heads * group_size;
  if (vheads > 0x7fffffff || (int64_t)num_groups * group_size > 0x7fffffff) return PKV_ERR_SHAPE;
  L->suf = o;
  L->pre = o;
  L->pre.kernel = PKV_KERNEL_AUTO;       // the virtual batch is grouped-query
  // A partition size valid for the whole-batch pass may not suit the matrix
  // cores (whole 32-token chunks): the grouped pass rounds it up.
  if (o.partition_size > 0)
    L->pre.partition_size = (int32_t)round_up((size_t)o.partition_size, block_size > 32 ? block_size : 32);
  L->pre.main_begin_event = L->pre.main_end_event = nullptr;
  Plan suf, pre;
  int st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                     dtype, &L->suf, &suf);
  if (st != PKV_OK) return st;
  st = make_plan(num_groups, (int32_t)vheads, num_kv_heads, head_dim, block_size, max_prefix_len,
                 dtype, &L->pre, &pre);
  if (st != PKV_OK) return st;
  L->tab_v = max_prefix_len > 0 ? (max_prefix_len + block_size - 1) / block_size : 1;
  const size_t es = (size_t)dtype_bytes(dtype);
  const size_t vrows = (size_t)num_groups * (size_t)vheads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes, 256);
    return at;
  };
  L->q_v = take(vrows * head_dim * es);
  L->tables_v = take((size_t)num_groups * L->tab_v * sizeof(int32_t));
  L->lens_v = take((size_t)num_groups * sizeof(int32_t));
  L->o_v = take(vrows * head_dim * es);
  L->lse_v = take(vrows * sizeof(float));
  L->lse_t = take((size_t)num_seqs * num_q_heads * sizeof(float));
  L->ws_pre_bytes = pre.ws_bytes;
  L->ws_suf_bytes = suf.ws_bytes;
  L->ws_pre = take(pre.ws_bytes);
  L->ws_suf = take(suf.ws_bytes);
  L->bytes = num_seqs > 0 ? off : 0;
  return PKV_OK;
}

}  // namespace

extern "C" {

size_t pkv_paged_attention_shared_prefix_workspace_bytes(
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_context_len, int32_t num_groups, int32_t group_size,
    int32_t max_prefix_len, pkv_dtype dtype, const pkv_attn_options* opts) {
  PrefixLayout L;
  if (prefix_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                    num_groups, group_size, max_prefix_len, dtype, opts, &L) != PKV_OK)
    return 0;
  return L.bytes;
}

int pkv_paged_attention_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* prefix_lens,
    const int32_t* group_members, int32_t num_groups, int32_t group_size, int32_t max_prefix_len,
    float scale, int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
    int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks,
    pkv_dtype dtype, void* workspace, size_t workspace_bytes, const pkv_attn_options* opts,
    void* stream) {
  PrefixLayout L;
  int st = prefix_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_context_len, num_groups, group_size, max_prefix_len, dtype, opts, &L);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_NULL;
  if (num_groups > 0 && (!prefix_lens || !group_members)) return PKV_ERR_NULL;
  // Every check of the two decode passes is made here, before the first launch.
  if (max_blocks_per_seq <= 0 || L.tab_v > max_blocks_per_seq || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_ALIGN;
  if (!workspace || workspace_bytes < L.bytes) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t vheads = num_q_heads * (num_groups > 0 ? group_size : 1);
  if (num_groups == 0) {
    return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                       max_context_len, num_blocks, dtype, ws + L.ws_suf, L.ws_suf_bytes, &L.suf,
                       stream, nullptr);
  }
  pkv::PrefixArgs a;
  a.q = static_cast<const char*>(q);
  a.q_v = ws + L.q_v;
  a.tables = block_tables;
  a.tables_v = reinterpret_cast<int32_t*>(ws + L.tables_v);
  a.prefix_lens = prefix_lens;
  a.lens_v = reinterpret_cast<int32_t*>(ws + L.lens_v);
  a.members = group_members;
  a.num_seqs = num_seqs;
  a.num_groups = num_groups;
  a.group_size = group_size;
  a.q_heads = num_q_heads;
  a.group = num_q_heads / num_kv_heads;
  a.row_pieces = head_dim * dtype_bytes(dtype) / 16;
  a.max_blocks = max_blocks_per_seq;
  a.tab_v = L.tab_v;
  // The two passes: the groups' shared prefixes (the virtual batch), then
  // every sequence's own tokens from its prefix length on.
  Plan pre_plan, suf_plan;
  pkv::AttnParams pre, suf;
  st = decode_setup(ws + L.o_v, ws + L.q_v, k_cache, v_cache, a.tables_v, a.lens_v, scale, block_size,
                    num_kv_heads, num_groups, vheads, head_dim, L.tab_v, max_prefix_len, num_blocks,
                    dtype, ws + L.ws_pre, L.ws_pre_bytes, &L.pre, nullptr,
                    reinterpret_cast<float*>(ws + L.lse_v), &pre_plan, &pre);
  if (st != PKV_OK) return st;
  st = decode_setup(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                    num_kv_heads, num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                    max_context_len, num_blocks, dtype, ws + L.ws_suf, L.ws_suf_bytes, &L.suf,
                    prefix_lens, reinterpret_cast<float*>(ws + L.lse_t), &suf_plan, &suf);
  if (st != PKV_OK) return st;
  // One launch builds the virtual batch and both work lists.
  const bool reuse = opts && opts->reuse_plan;
  a.plan_pre = !reuse && !pre_plan.direct;
  a.plan_suf = !reuse && !suf_plan.direct;
  clear_pending_error();
  const hipError_t e = pkv::launch_prefix_prep(a, pre, suf, block_size, s);
  if (e != hipSuccess) return launch_status(e);
  st = decode_attend(pre_plan, pre, dtype, head_dim, block_size, &L.pre, s);
  if (st != PKV_OK) return st;
  st = decode_attend(suf_plan, suf, dtype, head_dim, block_size, &L.suf, s);
  if (st != PKV_OK) return st;
  pkv::PrefixMergeArgs m;
  m.out = out;
  m.lse = reinterpret_cast<const float*>(ws + L.lse_t);
  m.o_v = ws + L.o_v;
  m.lse_v = reinterpret_cast<const float*>(ws + L.lse_v);
  m.members = group_members;
  m.num_seqs = num_seqs;
  m.num_groups = num_groups;
  m.group_size = group_size;
  m.q_heads = num_q_heads;
  m.group = num_q_heads / num_kv_heads;
  hipError_t err = hipSuccess;
  clear_pending_error();
  if (!pkv::launch_prefix_merge(m, dtype, head_dim, s, &err)) return PKV_ERR_UNSUPPORTED;
  return launch_status(err);
}

int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                          pkv_dtype dtype, void* stream) {
  const int es = dtype_bytes(dtype);
  if (!es) return PKV_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (((int64_t)head_dim * es) % 16) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)num_kv_heads * head_dim * es / 16 > 0x7fffffff / 16) return PKV_ERR_SHAPE;
  if (num_tokens > kMaxGrid) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_ALIGN;
  clear_pending_error();
  return launch_status(pkv::launch_reshape_and_cache(
      k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim * es, block_size,
      num_blocks, static_cast<hipStream_t>(stream)));
}

int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              pkv_dtype in_dtype, float k_scale, float v_scale, void* stream) {
  const int es = dtype_bytes(in_dtype);
  if (!es || in_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (!good_scale(k_scale) || !good_scale(v_scale)) return PKV_ERR_SHAPE;
  if (head_dim % 16) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)num_kv_heads * head_dim / 16 > 0x7fffffff / 64) return PKV_ERR_SHAPE;
  if (num_tokens > kMaxGrid) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_ALIGN;
  clear_pending_error();
  return launch_status(pkv::launch_reshape_and_cache_fp8(
      k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
      num_blocks, in_dtype, k_scale, v_scale, static_cast<hipStream_t>(stream)));
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs, int32_t num_pairs,
                    int32_t num_kv_heads, int32_t block_size, int32_t head_dim, int32_t num_blocks,
                    pkv_dtype dtype, void* stream) {
  const int es = dtype_bytes(dtype);
  if (!es) return PKV_ERR_DTYPE;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (((int64_t)head_dim * es) % 16) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return PKV_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_ALIGN;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * es;
  if ((int64_t)num_pairs * 2 * ((block_bytes + 16383) / 16384) > kMaxGrid) return PKV_ERR_SHAPE;
  clear_pending_error();
  return launch_status(pkv::launch_copy_blocks(k_cache, v_cache, src_dst_pairs, num_pairs,
                                               block_bytes, num_blocks,
                                               static_cast<hipStream_t>(stream)));
}

int pkv_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                    const int32_t* src_dst_pairs, int32_t num_pairs, int32_t num_src_blocks,
                    int32_t num_dst_blocks, int32_t num_kv_heads, int32_t block_size,
                    int32_t head_dim, pkv_dtype dtype, void* stream) {
  const int es = dtype_bytes(dtype);
  if (!es) return PKV_ERR_DTYPE;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_src_blocks < 0 ||
      num_dst_blocks < 0)
    return PKV_ERR_SHAPE;
  if (((int64_t)head_dim * es) % 16) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !src_dst_pairs) return PKV_ERR_NULL;
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v))
    return PKV_ERR_ALIGN;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * es;
  if ((int64_t)num_pairs * 2 * ((block_bytes + 16383) / 16384) > kMaxGrid) return PKV_ERR_SHAPE;
  if (!device_addressable(dst_k) || !device_addressable(dst_v) || !device_addressable(src_k) ||
      !device_addressable(src_v) || !device_addressable(src_dst_pairs))
    return PKV_ERR_UNSUPPORTED;
  clear_pending_error();
  return launch_status(pkv::launch_swap_blocks(dst_k, dst_v, src_k, src_v, src_dst_pairs, num_pairs,
                                               block_bytes, num_src_blocks, num_dst_blocks,
                                               static_cast<hipStream_t>(stream)));
}

int pkv_gather_kv(void* dst, const void* cache, const int32_t* block_tables,
                  const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                  int32_t max_context_len, int32_t kv_head, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks, pkv_dtype dtype,
                  void* stream) {
  const int es = dtype_bytes(dtype);
  if (!es) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || num_kv_heads <= 0 ||
      kv_head < 0 || kv_head >= num_kv_heads || head_dim <= 0 || block_size <= 0 ||
      num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (((int64_t)head_dim * es) % 16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_context_len == 0) return PKV_OK;
  if (!dst || !cache || !block_tables || !context_lens) return PKV_ERR_NULL;
  if (!aligned16(dst) || !aligned16(cache)) return PKV_ERR_ALIGN;
  if ((int64_t)num_seqs * max_context_len * head_dim * es / 16 / 256 >= kMaxGrid) return PKV_ERR_SHAPE;
  clear_pending_error();
  return launch_status(pkv::launch_gather_kv(dst, cache, block_tables, context_lens, num_seqs,
                                             max_blocks_per_seq, max_context_len, kv_head,
                                             num_kv_heads, head_dim * es, block_size, num_blocks,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
