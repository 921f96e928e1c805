// Slot write: each new token's K and V rows ([kv_heads, head_dim]) are copied
// bit for bit into the row of the slot the caller assigned.  In the
// [num_blocks, block_size, kv_heads, head_dim] layout the row of slot s starts
// at s * row_bytes, so the write is a scatter of whole rows; the page
// "PagedAttention Explained" describes the one-row-per-new-token growth of the
// cache ("The problem: the KV cache is big and unpredictable") and where the
// row lands ("How PagedAttention works", steps 2-4).
//
// Work split: one thread per 16-byte piece of a row; consecutive threads take
// consecutive pieces of the same row, so each wave reads and writes 1 KiB
// contiguous spans.  Pure data movement, HBM bound.
#include "device_common.hpp"
#include "cache_ops.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_write_kernel(KvWriteArgs a) {
  const int64_t row_vecs = a.row_bytes >> 4;
  const int64_t total = a.num_tokens * row_vecs;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += stride) {
    const int64_t tok = idx / row_vecs;
    const int64_t vec = idx - tok * row_vecs;
    const int64_t slot = a.slot_mapping[tok];
    if (slot < 0 || slot >= a.num_slots) continue;   // padding, or an id outside the pool
    const int64_t src = tok * row_vecs + vec;
    const int64_t dst = slot * row_vecs + vec;
    const uint4 kv = reinterpret_cast<const uint4*>(a.k)[src];
    const uint4 vv = reinterpret_cast<const uint4*>(a.v)[src];
    reinterpret_cast<uint4*>(a.k_cache)[dst] = kv;
    reinterpret_cast<uint4*>(a.v_cache)[dst] = vv;
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  const int64_t total = a.num_tokens * (a.row_bytes >> 4);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(kv_write_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
