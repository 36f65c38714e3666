/*
 * pkv.h — paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Plain pointers and sizes only.  "Device pointer" means
 * memory the HIP runtime allocated on the GPU the call runs on; "stream" is a
 * hipStream_t passed as void* (NULL = the default stream of the current
 * device).  Device calls are asynchronous and ordered on `stream`; none of
 * them synchronises, allocates or frees memory.  The caller owns every
 * buffer.  Every entry point returns PKV_OK (0) or a negative status; host
 * argument checks run before anything is launched, so a failed check leaves
 * all memory untouched.  No C++ exception crosses this boundary.
 *
 * What the operations are (pages on PagedAttention):
 *  - "PagedAttention" (lastdictionary): the KV cache of a sequence lives in
 *    fixed-size blocks of e.g. 16 tokens scattered anywhere in GPU memory; a
 *    per-sequence block table maps token positions to physical blocks; the
 *    attention kernel reads keys and values through that table; blocks are
 *    shared copy-on-write among sequences with a common prefix.
 *  - "pagedattention vllm" glossary (chipfoundryservices), "Attention
 *    Computation": block-wise attention equals standard attention over the
 *    gathered blocks; address translation maps virtual to physical blocks,
 *    loads them, computes and stores the result.  "Copy-on-Write Sharing":
 *    reference counts; copy a shared block before a sequence modifies it.
 *    "Memory Management": a free list, allocate on demand, release when the
 *    sequence completes.  "Implementation Details": block table entries are
 *    4 bytes.
 *
 * Layouts (all row-major, densely packed):
 *   q, out            [num_seqs, num_q_heads, head_dim]
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_dim]
 *   block_tables      int32 [num_seqs, max_blocks_per_seq]; entry t of row s
 *                     is the physical block holding tokens [t*B, (t+1)*B)
 *   context_lens      int32 [num_seqs]; tokens attended by each sequence
 *   k, v (new tokens) [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping      int32 [num_tokens]; slot = block * block_size + offset
 *   src_dst_pairs     int32 [num_pairs, 2]; (source block, destination block)
 * Query head j reads KV head j / (num_q_heads / num_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  PKV_FP8_E4M3 (OCP 8-bit E4M3, finite: bias 7, no
 * infinities, S.1111.111 = NaN, largest magnitude 448) is a KV-cache format
 * only: queries and outputs stay f32/f16/bf16.  A pkv_dtype argument is a
 * plain 32-bit integer, so any value a caller passes is representable and
 * an unknown one is refused with PKV_ERR_DTYPE. */
typedef int32_t pkv_dtype;
enum pkv_dtype_value { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 };

/* KV-cache format of the attention calls (pkv_attn_options.kv_format). */
enum pkv_kv_format {
  PKV_KV_SAME = 0,       /* caches hold the query's format */
  PKV_KV_FP8_E4M3 = 1    /* caches hold E4M3 codes; value = e4m3(code) * k_scale (v_scale) */
};

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* a size is negative, zero where it may not be, or inconsistent */
  PKV_ERR_DTYPE = -3,       /* unknown dtype */
  PKV_ERR_UNSUPPORTED = -4, /* a valid combination this build has no kernel for */
  PKV_ERR_ALIGN = -5,       /* a data pointer is not 16-byte aligned */
  PKV_ERR_WORKSPACE = -6,   /* workspace missing or too small */
  PKV_ERR_LAUNCH = -7,      /* the HIP runtime refused a launch */
  PKV_ERR_NO_BLOCKS = -8,   /* block manager: the free list is empty */
  PKV_ERR_STATE = -9,       /* block manager: unknown/duplicate sequence, bad block */
  PKV_ERR_CAPACITY = -10,   /* an output buffer is too small */
  PKV_ERR_SCRATCH = -11     /* the call needs more than the library's fixed scratch buffer */
};

/* Human-readable name of a status code (static storage). */
const char* pkv_status_str(int status);

/* Description of the HIP runtime error behind the last PKV_ERR_LAUNCH
 * returned on the calling thread ("" if none); valid until the next call. */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------------ */
/* Decode attention                                                          */
/* ------------------------------------------------------------------------ */

/* Both kernels take any number G of query heads per KV head (grouped-query
 * attention: heads sharing one set of keys and values, "Paged Attention"
 * glossary of systemdesign.academy; G = 1 is multi-head, Hkv = 1 multi-query).
 * A workgroup computes up to 8 of them on the vector ALUs; on the matrix
 * cores up to 16, or with 16- and 32-token blocks up to 64 (head_dim 64) or
 * 32 (head_dim 128) as several 16-column tiles that share each key/value
 * load.  A larger group is cut into C equal chunks, one workgroup each, and
 * the C workgroups of a (sequence, KV head, partition) run on one XCD so
 * they read its key/value tiles through the same L2 (with plain loads,
 * whatever the cache policy). */
enum pkv_kernel {
  PKV_KERNEL_AUTO = 0,  /* MFMA for 16-bit queries with 3 or more query heads per KV head, else VALU */
  PKV_KERNEL_VALU = 1,  /* vector-ALU kernel: every query / cache format */
  PKV_KERNEL_MFMA = 2   /* matrix-core kernel: f16/bf16 queries (8-bit caches decoded to that
                           format); each chunk's heads padded to the 16 columns of the products */
};

/* How the attention kernels load keys and values (pkv_attn_options.cache_policy). */
enum pkv_cache_policy {
  PKV_CACHE_STREAM = 0,  /* nontemporal loads: each block is read once per call (the default) */
  PKV_CACHE_KEEP = 1     /* plain loads: blocks several sequences of the batch share (a common
                            prompt of parallel samples or beams) are served again from L2 and
                            the Infinity Cache while their readers run close together */
};

typedef struct pkv_attn_options {
  /* Tokens per split-K partition.  0 = automatic: one partition per sequence
   * when there are at least 2048 (sequence, KV head) pairs (512 with a
   * sliding window); with fewer, the longest span (max_context_len, or the
   * window) is cut into equal partitions of about the smallest power of two
   * of at least 1024 tokens that gives ~4096 (sequence, KV head, partition)
   * work items, a span at most a quarter past it staying whole.
   * pkv_paged_attention_plan_info reports the choice.  Otherwise a positive
   * multiple of block_size (and of 32 for the MFMA kernel).  A sequence of
   * length L is cut into ceil(L / partition_size) partitions that separate
   * workgroups process; a reduce kernel merges them. */
  int32_t partition_size;
  int32_t kernel;            /* enum pkv_kernel */
  /* Optional hipEvent_t handles (NULL = none), recorded on the stream right
   * before and right after the main attention kernel, so a caller can time
   * that kernel alone.  The plan kernel runs before main_begin, the reduce
   * kernel (if any) after main_end.  Recording an event between two kernels
   * delays the second one by a few microseconds. */
  void* main_begin_event;
  void* main_end_event;
  /* Sliding window ("pagedattention vllm" glossary, Advanced Features >
   * Sliding Window): > 0 attends to the last sliding_window tokens of each
   * sequence only, t in [max(0, L - W), L); 0 attends to all L tokens.
   * Table entries of blocks wholly before the window are never read (they
   * may be -1 once pkv_bm_slide_window released them). */
  int32_t sliding_window;
  /* Cache format (enum pkv_kv_format) and, for PKV_KV_FP8_E4M3, the
   * per-tensor scales: a stored code c stands for e4m3(c) * k_scale in the
   * key cache and e4m3(c) * v_scale in the value cache ("pagedattention
   * vllm" glossary, Comparison with Alternatives > vs Compression: paging
   * combined with quantization).  Scales must be finite and > 0; they are
   * ignored for PKV_KV_SAME. */
  int32_t kv_format;
  float k_scale;
  float v_scale;
  /* Nonzero: skip building the work list and use the one the workspace
   * already holds, from an earlier call on the same stream with the same
   * arguments except the data (out, q, caches, new tokens, slot mapping)
   * and the same context_lens contents.  The list depends only on the batch
   * (context_lens, max_context_len, block size, heads, partition, window,
   * kernel), so the layers of one decode step can share it: build it on the
   * first layer, reuse it on the others.  A stale list (changed lengths, or
   * a workspace that never held one) leaves output rows undefined but stays
   * memory-safe: every read is still bounded by the current context_lens,
   * block tables and pool size. */
  int32_t reuse_plan;
  /* enum pkv_cache_policy.  Results are bit-identical under both; only the
   * speed differs.  Measured on MI355X: streaming reads unshared caches ~11%
   * faster; keeping made the shared-prefix sampling layer (8 samples per
   * 1000-token prompt, 1024-token partitions) 1.4x faster. */
  int32_t cache_policy;
} pkv_attn_options;

/* What pkv_paged_attention_decode will launch for these sizes and options:
 * the partition size in tokens after the automatic choice, the partitions
 * per sequence its grid covers (1: no split-K reduce), and the main kernel
 * (enum pkv_kernel, never PKV_KERNEL_AUTO).  Out-pointers may be NULL.
 * Returns the status the decode call's argument checks would give. */
int pkv_paged_attention_plan_info(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                  pkv_dtype dtype, const pkv_attn_options* opts,
                                  int32_t* partition_size, int32_t* max_parts, int32_t* kernel);

/* Bytes of workspace pkv_paged_attention_decode needs for these sizes and
 * options: a 256-byte header and the work list (8 bytes per sequence and
 * partition), plus partition results when a sequence can span several
 * partitions: per sequence, query head and partition, head_dim elements in
 * the output format (dtype) and 2 floats.  0 for an empty batch, and 0 on
 * invalid arguments (the decode call reports those). */
size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_context_len,
                                           pkv_dtype dtype, const pkv_attn_options* opts);

/*
 * Single-token decode attention through the block tables
 * ("pagedattention vllm" glossary, Attention Computation: Block-Wise
 * Attention and Address Translation; "What is PagedAttention" (tecyfy),
 * How it works: attention rewritten to read keys and values from scattered
 * blocks).  For every sequence s and query head j, with h = j / (Hq / Hkv)
 * and L = context_lens[s]:
 *
 *   K_t = k_cache[block_tables[s][t / B]][h][t % B][:],  V_t likewise,
 *   out[s][j][:] = sum_t softmax_t(scale * <q[s][j], K_t>) * V_t
 *
 * over t in [0, L), or [max(0, L - W), L) with a sliding window W.
 *
 * computed in fp32 and rounded to the data type (round to nearest even).
 * L = 0 gives a zero row.  Only the first ceil(L/B) table entries of a row
 * are read and only the first L tokens are used; other pool slots may hold
 * anything (NaN included) without affecting the result.
 *
 * Device pointers: out, q, k_cache, v_cache (16-byte aligned), block_tables,
 * context_lens, workspace.  max_context_len (host) must be >= every
 * context_lens[s]; it sizes the launch.  num_blocks is the pool size.
 *
 * Launches, in stream order: a one-workgroup plan kernel that reads
 * context_lens and writes the work list into the workspace (the
 * (sequence, partition) pairs, longest first, so long pieces start early
 * and the grid ends on short ones), then the main kernel, one workgroup per
 * (pair, KV head, head chunk); and, when a sequence can span several partitions, the
 * split-K reduce, which merges the partial softmax states in partition
 * order.  A main grid of at most 256 workgroups is resident at once: it
 * takes its items in grid order and no plan kernel runs.  The schedule
 * does not change any result.
 * Data errors are contained, never dereferenced: a table entry outside
 * [0, num_blocks), or context_lens[s] above max_context_len or
 * max_blocks_per_seq * B, makes that sequence's output rows NaN.
 * num_q_heads: any multiple of num_kv_heads.  head_dim: 64 or 128.
 * block_size: 8, 16, 32 or 64 (16 or 32 with 8-bit caches).
 * workspace: device memory of at least pkv_paged_attention_workspace_bytes,
 * 16-byte aligned, required whenever num_seqs > 0; its contents need no
 * initialisation and are overwritten.  Calls that overlap in time must not
 * share a workspace.
 * opts may be NULL (automatic everything).
 */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, int32_t block_size, int32_t num_kv_heads,
                               int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int32_t num_blocks, pkv_dtype dtype,
                               void* workspace, size_t workspace_bytes,
                               const pkv_attn_options* opts, void* stream);

/*
 * pkv_paged_attention_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments minus the workspace, the same kernels and
 * bit-identical results.  The work list and split-K partial results live in
 * one fixed device array of PKV_NOALLOC_SCRATCH_BYTES bytes that the library
 * reserves on every GPU it runs on, held until the process ends; nothing is
 * allocated or freed by the call.
 * The array is shared by every call on one GPU and keeps what the last call
 * left: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give undefined rows.  Nothing in it needs to start at
 * zero (the work list and the partials are written before they are read);
 * opts->reuse_plan reuses the work list the previous call on that GPU left.
 * A call whose workspace (pkv_paged_attention_workspace_bytes) exceeds the
 * array is refused with PKV_ERR_SCRATCH before anything runs: the 64 MiB
 * hold about 250k split-K partial rows of head_dim 128 in a 16-bit format
 * (D * 2 + 8 bytes each), while an unsplit batch needs only its 8-byte work
 * list entry per sequence.
 * The stream's device (the current device for NULL) is the GPU used; the
 * array's address on it is looked up on the first call there.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale,
                                       int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t num_blocks, pkv_dtype dtype,
                                       const pkv_attn_options* opts, void* stream);

/*
 * One decode step in two launches: every sequence's new token is stored as
 * pkv_reshape_and_cache would (token i = sequence i, slot slot_mapping[i])
 * by the same launch that builds the attention work list, then attention
 * runs as pkv_paged_attention_decode over context_lens (which count the new
 * token).  Results are bit-identical to those two calls in sequence; the
 * step saves one launch.  slot_mapping[i] must be the slot of token L_i - 1
 * of sequence i's table (as the block manager hands it out): a small batch
 * on the vector kernel with caches in the query format runs the whole step
 * in one launch, whose attention takes that token's key and value from
 * k_new and v_new rather than from the cache (a slot outside the pool is
 * neither stored nor substituted).  With opts->reuse_plan the first launch only
 * stores the tokens.  With an 8-bit cache format the tokens are stored as
 * pkv_reshape_and_cache_fp8 would, with the options' scales.  k_new, v_new:
 * device [num_seqs, num_kv_heads, head_dim] in the query format, 16-byte
 * aligned; slot_mapping: device int32 [num_seqs].  Other arguments,
 * workspace and errors as pkv_paged_attention_decode.
 */
int pkv_decode_step(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, const int32_t* slot_mapping, const int32_t* block_tables,
                    const int32_t* context_lens, float scale, int32_t block_size,
                    int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks,
                    pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                    const pkv_attn_options* opts, void* stream);

/*
 * Decode attention for groups of sequences that share the first blocks of
 * their tables: the parallel samples of one prompt, or beams, whose common
 * prefix blocks the block manager shares by reference count ("pagedattention
 * vllm" glossary, Copy-on-Write Sharing: Prefix Sharing, Reference Counting
 * and Use Cases; "What is PagedAttention" (tecyfy), What it changes).  The output is that of
 * pkv_paged_attention_decode on the same arguments (the same softmax over
 * t in [0, L) of every sequence); only the reads differ: the shared prefix
 * is read once per group instead of once per member.
 *
 * group_members: device int32 [num_groups, group_size]: sequence indices,
 *   -1 for an unused slot; a sequence appears in at most one group.
 * prefix_lens: device int32 [num_seqs]: P_s, the tokens at the start of
 *   sequence s whose keys and values are the same for every member of its
 *   group (the same physical blocks); all members of a group give the same
 *   P, with 0 <= P <= L_s, and sequences in no group give 0.  Tokens
 *   [0, P) of a group are read through the table of its first member.
 * max_prefix_len (host): >= every prefix_lens[s], <= max_context_len and
 *   <= max_blocks_per_seq * block_size; it sizes the prefix launch.
 *
 * Launches, in stream order: a gather of each group's member queries (and
 * its first member's table row and prefix length) into the workspace; the
 * decode kernels on the groups, whose G members x g heads per KV head form
 * a query group of G g heads (matrix cores for 16-bit data), giving each
 * member's prefix part and its log-denominator; the decode kernels on the
 * whole batch over t in [P_s, L_s); a merge of the two parts
 *   out = (o_a 2^(l_a - m) + o_b 2^(l_b - m)) / (2^(l_a - m) + 2^(l_b - m)),
 * m = max(l_a, l_b), where l is log2 of a part's softmax denominator in
 * units of log2(e) * scale * <q, k>.  The parts are rounded to the output
 * format before the merge (one more rounding than the plain call).
 * Arguments that break the rules above give undefined rows but stay
 * memory-safe; a data error (table entry, length) makes the affected rows
 * NaN as in pkv_paged_attention_decode.
 * opts: as pkv_paged_attention_decode, except sliding_window (must be 0:
 * PKV_ERR_UNSUPPORTED) and kernel and the events, which apply to the
 * whole-batch pass only; the grouped pass rounds partition_size up to a
 * multiple of 32 tokens (and of block_size) when it is not one.  workspace: at least
 * pkv_paged_attention_shared_prefix_workspace_bytes bytes, 16-byte aligned.
 * num_groups = 0 is a plain decode.
 */
size_t pkv_paged_attention_shared_prefix_workspace_bytes(
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_context_len, int32_t num_groups, int32_t group_size,
    int32_t max_prefix_len, pkv_dtype dtype, const pkv_attn_options* opts);

int pkv_paged_attention_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* prefix_lens,
    const int32_t* group_members, int32_t num_groups, int32_t group_size, int32_t max_prefix_len,
    float scale, int32_t block_size, int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
    int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks,
    pkv_dtype dtype, void* workspace, size_t workspace_bytes, const pkv_attn_options* opts,
    void* stream);

/* ------------------------------------------------------------------------ */
/* Cache write and copy-on-write                                             */
/* ------------------------------------------------------------------------ */

/*
 * Store each new token's key and value into the block slot the block
 * manager reserved for it, in the caches' own format (f32/f16/bf16; for
 * 8-bit caches see pkv_reshape_and_cache_fp8) ("What is PagedAttention"
 * (tecyfy), How it works:
 * blocks handed out as the sequence grows):
 *   k_cache[slot / B][h][slot % B][:] = k[i][h][:]   (and v), all h,
 * for every i with 0 <= slot = slot_mapping[i] < num_blocks * B.  Negative
 * slots are skipped (padding); slots at or beyond the pool are skipped too
 * (a data error, never written).  Bitwise copy.  Two tokens naming the same
 * slot is a caller error (which one lands is unspecified).
 * Device pointers: k, v, k_cache, v_cache (16-byte aligned), slot_mapping.
 */
int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                          pkv_dtype dtype, void* stream);

/*
 * reshape_and_cache into 8-bit caches: every value x of the new token's key
 * (value) row, in format in_dtype (f32/f16/bf16), is stored as the E4M3 code
 * of fp32(x) / k_scale (v_scale): fp32 division, round to nearest with ties
 * to the even code, saturating at +-448 (448 itself included), NaN stored as
 * 0x7F.  Caches: uint8 [num_blocks, num_kv_heads, block_size, head_dim].
 * Slots as in pkv_reshape_and_cache.  k_scale, v_scale finite and > 0.
 */
int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              pkv_dtype in_dtype, float k_scale, float v_scale, void* stream);

/*
 * Copy-on-write block copies ("pagedattention vllm" glossary, Copy-on-Write
 * Sharing: Divergence Handling): for every pair p, block dst = pairs[p][1]
 * of both caches becomes a bitwise copy of block src = pairs[p][0], all KV
 * heads and offsets.  Destinations must be distinct and must not be sources
 * in the same call (the block manager guarantees it); then pair order does
 * not matter.  Pairs naming a block outside [0, num_blocks) are skipped.
 * Device pointers: k_cache, v_cache (16-byte aligned), src_dst_pairs.
 */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs, int32_t num_pairs,
                    int32_t num_kv_heads, int32_t block_size, int32_t head_dim, int32_t num_blocks,
                    pkv_dtype dtype, void* stream);

/*
 * Swapping ("pagedattention vllm" glossary, Memory Management > Swapping):
 * for every pair p, block dst = pairs[p][1] of the destination pools becomes
 * a bitwise copy of block src = pairs[p][0] of the source pools (keys and
 * values, all heads).  Either side may be device memory or pinned host
 * memory the device can address at the same address (hipHostMalloc / torch
 * pin_memory); any other pointer (pageable memory) is refused with
 * PKV_ERR_UNSUPPORTED before anything runs.  Swap out is device -> host,
 * swap in host -> device; the copy runs as one kernel, bounded by PCIe for
 * host pools.  pairs: device int32
 * [num_pairs, 2]; destinations distinct; pairs naming a block outside its
 * pool are skipped.  Same element layout and sizes as the caches.
 */
int pkv_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                    const int32_t* src_dst_pairs, int32_t num_pairs, int32_t num_src_blocks,
                    int32_t num_dst_blocks, int32_t num_kv_heads, int32_t block_size,
                    int32_t head_dim, pkv_dtype dtype, void* stream);

/*
 * Debug/test helper: materialise one KV head's keys of a set of sequences
 * contiguously, through the block tables:
 *   dst[s][t][:] = cache[block_tables[s][t / B]][kv_head][t % B][:],  t < context_lens[s],
 * rows t >= context_lens[s] (up to max_context_len) are left untouched.
 * dst: device [num_seqs, max_context_len, head_dim].  Out-of-pool table
 * entries are skipped.  Same layout rules as the attention call.
 */
int pkv_gather_kv(void* dst, const void* cache, const int32_t* block_tables,
                  const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                  int32_t max_context_len, int32_t kv_head, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks, pkv_dtype dtype,
                  void* stream);

/* ------------------------------------------------------------------------ */
/* Host block manager (free list, reference counts, block tables, CoW)       */
/* ------------------------------------------------------------------------ */
/*
 * "What is PagedAttention" (tecyfy), How it works: blocks are handed out as a
 * sequence grows; a sequence holds the blocks it filled plus part of the
 * last.  "pagedattention vllm" glossary: Memory Management > Block
 * Allocation (free list, allocate on demand, release on completion);
 * Copy-on-Write Sharing > Reference Counting and Divergence Handling.
 *
 * Policy: blocks leave the free list from its front; blocks whose count
 * drops to zero return to its front in table order.  Appending at position
 * t allocates a new block when t % B == 0; otherwise, if the last block has
 * more than one reference, it takes a fresh block for this sequence, reports
 * (shared, fresh) for pkv_copy_blocks, and drops one reference of the
 * shared block.  Host memory only, no GPU needed; a handle is not
 * thread-safe.  Sequence ids are in [0, max_seqs).
 */
typedef struct pkv_block_manager pkv_block_manager;

/* free_order: NULL (0, 1, ..., num_blocks-1) or a permutation of the pool,
 * front first.  Returns NULL on invalid arguments or out of memory. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                                 const int32_t* free_order);
void pkv_bm_destroy(pkv_block_manager* bm);
int pkv_bm_add_seq(pkv_block_manager* bm, int32_t seq);
/* child gets parent's table and length; each shared block gains a reference */
int pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t child);
/* children[i] = fork of parents[i] for i in order (beam search: every new
 * beam continues a chosen parent).  On an error at i the forks before i
 * stay done, *num_done = i, and the error is returned. */
int pkv_bm_fork_batch(pkv_block_manager* bm, const int32_t* parents, const int32_t* children,
                      int32_t n, int32_t* num_done);
/* pkv_bm_free_seq for each of seqs[0..n), in order; errors as fork_batch. */
int pkv_bm_free_batch(pkv_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* num_done);
/* Reserve the next token's slot.  *cow_src / *cow_dst receive the pair to
 * copy before the write, or -1 / -1.  PKV_ERR_NO_BLOCKS leaves all state
 * unchanged. */
int pkv_bm_append(pkv_block_manager* bm, int32_t seq, int32_t* slot, int32_t* cow_src,
                  int32_t* cow_dst);
/* One append for each of n sequences, in order.  slots[n]; copy pairs are
 * written to pairs[2*k], pairs[2*k+1] and counted in *num_pairs (pairs_cap
 * pairs of room).  On an error at sequence i the appends before i stay
 * done, the return value is the error, and *num_done = i. */
int pkv_bm_append_batch(pkv_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* slots,
                        int32_t* pairs, int32_t pairs_cap, int32_t* num_pairs, int32_t* num_done);
/* Release a finished sequence's blocks. */
int pkv_bm_free_seq(pkv_block_manager* bm, int32_t seq);
/* Swapping ("pagedattention vllm" glossary, Memory Management > Swapping:
 * blocks move to CPU memory to serve more sequences than the GPU holds):
 * move sequence `seq` from manager `from` to manager `to` (say, the GPU
 * pool's and a pinned host pool's).  Each of its blocks gets a fresh block
 * of `to` (front of its free list, table order) and loses this sequence's
 * reference in `from`; released entries (-1) stay -1; the id and length
 * move along.  pairs[2k], pairs[2k+1] receive (block in from, block in to)
 * for pkv_swap_blocks, *num_pairs their number.  PKV_ERR_NO_BLOCKS (too few
 * free blocks in `to`) and every other error leave both managers as they
 * were.  Shared blocks are copied for this sequence, not shared in `to`. */
int pkv_bm_move_seq(pkv_block_manager* from, pkv_block_manager* to, int32_t seq, int32_t* pairs,
                    int32_t pairs_cap, int32_t* num_pairs);
/* Sliding window ("pagedattention vllm" glossary, Advanced Features >
 * Sliding Window: keep only recent blocks): release the blocks of `seq` that
 * hold no token of its last `window` tokens, i.e. table positions
 * 0 .. (len - window) / B - 1.  Their table entries become -1 (positions do
 * not move; attention with that window never reads them) and each loses one
 * reference (back to the free list at zero).  Returns the number of entries
 * released (>= 0) or a negative status. */
int pkv_bm_slide_window(pkv_block_manager* bm, int32_t seq, int32_t window);
/* Length of a sequence (>= 0) or a negative status. */
int pkv_bm_seq_len(const pkv_block_manager* bm, int32_t seq);
/* Copy a sequence's table into out[cap]; returns its number of blocks, or a
 * negative status (PKV_ERR_CAPACITY if cap is too small). */
int pkv_bm_block_table(const pkv_block_manager* bm, int32_t seq, int32_t* out, int32_t cap);
/* Rows of a batch: tables[n][max_blocks] (-1 padded) and context_lens[n]. */
int pkv_bm_export(const pkv_block_manager* bm, const int32_t* seqs, int32_t n, int32_t* tables,
                  int32_t max_blocks, int32_t* context_lens);
int pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);
int pkv_bm_num_free(const pkv_block_manager* bm);
/* Copy the free list (front first) into out[cap]; returns its length. */
int pkv_bm_free_list(const pkv_block_manager* bm, int32_t* out, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
