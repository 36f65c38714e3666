// Byte-moving kernels of the KV block pool: the new-token scatter
// (reshape_and_cache), the copy-on-write block copy (copy_blocks) and a
// gather through the block tables used to check addressing.  All of them
// move 16-byte units with vector loads and stores; none looks at values.
#include "device_common.h"
#include "kernels.h"
#include "scatter.h"

namespace pkv {

// One workgroup per new token.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int32_t num_kv_heads,
    int32_t chunks, int32_t block_size, int64_t num_slots) {
  scatter_token(k, v, k_cache, v_cache, slot_mapping, blockIdx.x, threadIdx.x, blockDim.x,
                num_kv_heads, chunks, block_size, num_slots);
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                                    int32_t num_blocks, hipStream_t stream) {
  const int32_t chunks = row_bytes / 16;
  if (num_tokens == 0) return hipSuccess;
  const int per_tok = num_kv_heads * chunks;
  const int threads = per_tok >= 256 ? 256 : (per_tok + 63) / 64 * 64;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)num_tokens), dim3(threads), 0, stream,
                     static_cast<const char*>(k), static_cast<const char*>(v),
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), slot_mapping,
                     num_kv_heads, chunks, block_size, (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

// Quantizing store into 8-bit caches, one workgroup per new token.
template <int IT>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int64_t num_slots, float k_scale, float v_scale) {
  scatter_token_fp8<IT>(k, v, k_cache, v_cache, slot_mapping, blockIdx.x, threadIdx.x, blockDim.x,
                        num_kv_heads, head_dim, block_size, num_slots, k_scale, v_scale);
}

hipError_t launch_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                        const int32_t* slot_mapping, int32_t num_tokens,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, pkv_dtype in_dtype, float k_scale,
                                        float v_scale, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int per_tok = num_kv_heads * (head_dim / 16);
  const int threads = per_tok >= 256 ? 256 : (per_tok + 63) / 64 * 64;
  const int64_t slots = (int64_t)num_blocks * block_size;
  const char* kk = static_cast<const char*>(k);
  const char* vv = static_cast<const char*>(v);
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  switch (in_dtype) {
    case PKV_F32:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<PKV_F32>, dim3((unsigned)num_tokens), dim3(threads), 0,
                         stream, kk, vv, kc, vc, slot_mapping, num_kv_heads, head_dim, block_size, slots,
                         k_scale, v_scale);
      break;
    case PKV_F16:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<PKV_F16>, dim3((unsigned)num_tokens), dim3(threads), 0,
                         stream, kk, vv, kc, vc, slot_mapping, num_kv_heads, head_dim, block_size, slots,
                         k_scale, v_scale);
      break;
    case PKV_BF16:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<PKV_BF16>, dim3((unsigned)num_tokens), dim3(threads), 0,
                         stream, kk, vv, kc, vc, slot_mapping, num_kv_heads, head_dim, block_size, slots,
                         k_scale, v_scale);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Each workgroup copies one 16 KiB piece of one block of one cache (keys or
// values) from the source pools to the destination pools; copy_blocks uses
// one pool as both, swap_blocks a device pool and a pinned host pool.
constexpr int kCopyPiece = 16384;

__global__ __launch_bounds__(256) void copy_pool_blocks_kernel(
    char* __restrict__ dst_k, char* __restrict__ dst_v, const char* src_k, const char* src_v,
    const int32_t* __restrict__ pairs, int64_t block_bytes, int32_t pieces, int32_t num_src,
    int32_t num_dst) {
  const int pair = blockIdx.x / (2 * pieces);
  const int rest = blockIdx.x % (2 * pieces);
  const int which = rest / pieces, piece = rest % pieces;
  const int32_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if ((unsigned)src >= (unsigned)num_src || (unsigned)dst >= (unsigned)num_dst) return;
  const char* from = (which ? src_v : src_k) + (size_t)src * block_bytes;
  char* to = (which ? dst_v : dst_k) + (size_t)dst * block_bytes;
  const int64_t begin = (int64_t)piece * kCopyPiece;
  u32x4 buf[kCopyPiece / (256 * 16)];
#pragma unroll
  for (int j = 0; j < kCopyPiece / (256 * 16); ++j) {
    const int64_t off = begin + ((int64_t)j * 256 + threadIdx.x) * 16;
    if (off < block_bytes) buf[j] = load16(from + off);
  }
#pragma unroll
  for (int j = 0; j < kCopyPiece / (256 * 16); ++j) {
    const int64_t off = begin + ((int64_t)j * 256 + threadIdx.x) * 16;
    if (off < block_bytes) store16(to + off, buf[j]);
  }
}

hipError_t launch_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              int32_t num_src, int32_t num_dst, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int32_t pieces = (int32_t)((block_bytes + kCopyPiece - 1) / kCopyPiece);
  const dim3 grid((unsigned)((int64_t)num_pairs * 2 * pieces));
  hipLaunchKernelGGL(copy_pool_blocks_kernel, grid, dim3(256), 0, stream, static_cast<char*>(dst_k),
                     static_cast<char*>(dst_v), static_cast<const char*>(src_k),
                     static_cast<const char*>(src_v), pairs, block_bytes, pieces, num_src, num_dst);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, int32_t num_blocks, hipStream_t stream) {
  return launch_swap_blocks(k_cache, v_cache, k_cache, v_cache, pairs, num_pairs, block_bytes,
                            num_blocks, num_blocks, stream);
}

// One thread per 16-byte chunk of dst[s][t][:].
__global__ __launch_bounds__(256) void gather_kv_kernel(
    char* __restrict__ dst, const char* __restrict__ cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, int64_t total, int32_t max_blocks, int32_t max_len,
    int32_t kv_head, int32_t num_kv_heads, int32_t chunks, int32_t block_size,
    int32_t num_blocks) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % chunks);
  const int64_t row = idx / chunks;          // s * max_len + t
  const int t = (int)(row % max_len);
  const int64_t s = row / max_len;
  const int32_t L = lens[s];
  if (t >= L || t / block_size >= max_blocks) return;
  const int32_t blk = tables[s * max_blocks + t / block_size];
  if ((unsigned)blk >= (unsigned)num_blocks) return;
  const size_t src =
      ((((size_t)blk * num_kv_heads + kv_head) * block_size + t % block_size) * chunks + c) * 16;
  store16(dst + ((size_t)row * chunks + c) * 16, load16(cache + src));
}

hipError_t launch_gather_kv(void* dst, const void* cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t max_context_len, int32_t kv_head,
                            int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                            int32_t num_blocks, hipStream_t stream) {
  const int32_t chunks = row_bytes / 16;
  const int64_t total = (int64_t)num_seqs * max_context_len * chunks;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(gather_kv_kernel, grid, dim3(256), 0, stream, static_cast<char*>(dst),
                     static_cast<const char*>(cache), block_tables, context_lens, total,
                     max_blocks_per_seq, max_context_len, kv_head, num_kv_heads, chunks,
                     block_size, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
