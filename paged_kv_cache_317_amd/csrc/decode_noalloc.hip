// Decode attention for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): pkv_paged_attn_decode with its split workspace in a device
// array of this library instead of caller memory.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/pkv.h"
#include "status.hpp"

namespace {

// The array every call on a device uses for the split workspace.  Each GPU
// the library runs on holds its own copy at its own address from the moment
// the code object is loaded until the process ends.  Host code must not use
// this name as a device address; it uses the address looked up below.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
pkv_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "device %d is beyond the %d devices the no-allocation "
                     "decode keeps a scratch address for", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pkv::fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

PKV_EXPORT size_t pkv_decode_noalloc_max_workspace(void) { return kScratchBytes; }

PKV_EXPORT pkv_status pkv_paged_attn_decode_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* cache,
    const int32_t* block_table, int32_t table_width, const int32_t* seq_lens, int32_t num_seqs,
    int32_t q_heads, int32_t max_seq_len, float scale, void* out, int32_t part_tokens,
    void* stream) {
  // The size check runs on the host before any HIP call.
  const size_t need =
      pkv_decode_workspace_size(cache, num_seqs, q_heads, max_seq_len, part_tokens);
  if (need == 0 && pkv_last_error()[0] != '\0') {
    // Invalid arguments: the regular entry point reports them.
    return pkv_paged_attn_decode(q, k_cache, v_cache, cache, block_table, table_width, seq_lens,
                                 num_seqs, q_heads, max_seq_len, scale, out, part_tokens, nullptr,
                                 0, stream);
  }
  if (need > kScratchBytes)
    return pkv::fail(PKV_ERR_WORKSPACE, "this call needs a %zu-byte workspace; the no-allocation "
                     "decode holds %zu bytes (use pkv_paged_attn_decode with a workspace)", need,
                     kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    pkv_status st = scratch_address(&ws);
    if (st != PKV_OK) return st;
  }
  return pkv_paged_attn_decode(q, k_cache, v_cache, cache, block_table, table_width, seq_lens,
                               num_seqs, q_heads, max_seq_len, scale, out, part_tokens, ws,
                               need > 0 ? kScratchBytes : 0, stream);
}
