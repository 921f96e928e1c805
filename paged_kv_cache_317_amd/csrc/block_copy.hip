// Whole-block copies between two pools of the same block shape.
//
// Copy-on-write: for every (src, dst) pair the block dst of the K pool and of
// the V pool becomes a bit copy of block src of the same pool -- the copy a
// sequence takes before writing into a block that others still reference
// ("PagedAttention Explained", "Sharing blocks between sequences").
// Swapping: the same copy between the device pool and a pool in pinned host
// memory, moving a preempted sequence's blocks out and back ("PagedAttention
// Explained", "Preemption and scheduling").
//
// Work split: each workgroup copies one 32 KiB chunk of one block of one pool;
// every thread issues all its loads before its stores so that eight 16-byte
// loads per thread are in flight.  Pure data movement, bound by HBM (or by
// the host link when one side is host memory).  Device-to-device copies use
// non-temporal loads and stores: 255 copy-on-write pairs of 32 KiB blocks
// (both pools) took 5.3 us that way, 10.2 us with regular accesses; over
// the host link the regular accesses were 2-4% faster, so moves to and from
// host memory keep them.
#include "device_common.hpp"
#include "cache_ops.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kVecsPerThread = 8;
constexpr int kChunkVecs = kThreads * kVecsPerThread;   // 32 KiB

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool kNt>
__global__ __launch_bounds__(kThreads) void block_move_kernel(BlockMoveArgs a, int chunks) {
  const int per_pair = 2 * chunks;
  const int pair = blockIdx.x / per_pair;
  const int rem = blockIdx.x - pair * per_pair;
  const int pool = rem / chunks;                   // 0: K, 1: V
  const int chunk = rem - pool * chunks;
  const int64_t src = a.pairs[2 * pair];
  const int64_t dst = a.pairs[2 * pair + 1];
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
  const int64_t block_vecs = a.block_bytes >> 4;
  const uint4* from = reinterpret_cast<const uint4*>(pool ? a.src_v : a.src_k) + src * block_vecs;
  uint4* to = reinterpret_cast<uint4*>(pool ? a.dst_v : a.dst_k) + dst * block_vecs;
  const int64_t first = (int64_t)chunk * kChunkVecs + threadIdx.x;
  // Every load is issued (an index past the block re-reads its last
  // element), so that all of them are in flight before the first store;
  // conditional loads into the array made the compiler wait for each one.
  // Elements stay uint4; the non-temporal builtins take the ext-vector form.
  uint4 buf[kVecsPerThread];
#pragma unroll
  for (int i = 0; i < kVecsPerThread; ++i) {
    const int64_t e = min(first + i * kThreads, block_vecs - 1);
    if constexpr (kNt) {
      const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(from + e));
      buf[i] = uint4{t[0], t[1], t[2], t[3]};
    } else {
      buf[i] = from[e];
    }
  }
#pragma unroll
  for (int i = 0; i < kVecsPerThread; ++i) {
    const int64_t e = first + i * kThreads;
    if (e < block_vecs) {
      if constexpr (kNt)
        __builtin_nontemporal_store(u32x4_t{buf[i].x, buf[i].y, buf[i].z, buf[i].w},
                                    reinterpret_cast<u32x4_t*>(to + e));
      else
        to[e] = buf[i];
    }
  }
}

}  // namespace

int64_t block_move_workgroups(const BlockMoveArgs& a) {
  const int64_t block_vecs = a.block_bytes >> 4;
  return (int64_t)a.num_pairs * 2 * ((block_vecs + kChunkVecs - 1) / kChunkVecs);
}

hipError_t launch_block_move(const BlockMoveArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  const int64_t block_vecs = a.block_bytes >> 4;
  const int chunks = (int)((block_vecs + kChunkVecs - 1) / kChunkVecs);
  const int64_t grid = block_move_workgroups(a);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (a.streaming)
    hipLaunchKernelGGL(block_move_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       a, chunks);
  else
    hipLaunchKernelGGL(block_move_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       a, chunks);
  return hipGetLastError();
}

}  // namespace pkv
