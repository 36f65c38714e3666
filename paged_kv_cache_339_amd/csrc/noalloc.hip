// Decode attention without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// pkv_paged_attention_decode keeps its work list and split-K partial results
// in a workspace the caller passes.  This variant takes that memory from one
// fixed device array, `scratch` below, of PKV_NOALLOC_SCRATCH_BYTES bytes:
// the code object reserves it on every GPU the library is loaded on, and it
// lives until the process ends.  The kernels are the same ones; only where
// their workspace lives differs.
//
// In host code `scratch` names a host-side stand-in, not the device memory,
// so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; only that
// address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "pkv.h"

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `device`, looked up on first use.
int scratch_on_device(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    int current = -1;
    if (hipGetDevice(&current) != hipSuccess) {
      (void)hipGetLastError();
      return PKV_ERR_LAUNCH;
    }
    if (current != device && hipSetDevice(device) != hipSuccess) {
      (void)hipGetLastError();
      return PKV_ERR_LAUNCH;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != device) (void)hipSetDevice(current);
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PKV_ERR_LAUNCH;
    }
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return PKV_OK;
}

// The device a call on `stream` runs on: the stream's, or the current one
// for the null stream.
int stream_device(void* stream, int* device) {
  hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), device)
                                   : hipGetDevice(device);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_LAUNCH;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale,
                                       int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t num_blocks, pkv_dtype dtype,
                                       const pkv_attn_options* opts, void* stream) {
  // Every host check of the decode call first, then the size: a call whose
  // work list and partials would not fit is refused before any runtime call.
  size_t need = 0;
  int st = pkv::decode_arg_status(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                  block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                                  max_blocks_per_seq, max_context_len, num_blocks, dtype, opts,
                                  &need);
  if (st != PKV_OK) return st;
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  if (num_seqs == 0) return PKV_OK;
  int device = -1;
  st = stream_device(stream, &device);
  if (st != PKV_OK) return st;
  void* ws = nullptr;
  st = scratch_on_device(device, &ws);
  if (st != PKV_OK) return st;
  return pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                    block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                                    max_blocks_per_seq, max_context_len, num_blocks, dtype, ws,
                                    (size_t)PKV_NOALLOC_SCRATCH_BYTES, opts, stream);
}

}  // extern "C"
