// Internal launchers of the slot-write and block-move kernels (host side).
// The C ABI in pkv_api.cpp validates every argument and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct KvWriteArgs {
  const void* k;
  const void* v;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  void* k_cache;
  void* v_cache;
  int64_t num_slots;     // num_blocks * block_size
  int64_t row_bytes;     // kv_heads * head_dim * element bytes, multiple of 16
};

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v); the two pools
// may be the same (copy-on-write) or differ (swapping).
struct BlockMoveArgs {
  const int64_t* pairs;  // [num_pairs, 2] (src block, dst block)
  int32_t num_pairs;
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  int64_t src_blocks;
  int64_t dst_blocks;
  int64_t block_bytes;   // block_size * kv_heads * head_dim * element bytes
  bool streaming;        // both pools on the device: non-temporal loads and stores
};

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
// Workgroups launch_block_move starts for these arguments (the API refuses
// calls above INT32_MAX before launching).
int64_t block_move_workgroups(const BlockMoveArgs& a);
hipError_t launch_block_move(const BlockMoveArgs& a, hipStream_t stream);

}  // namespace pkv
