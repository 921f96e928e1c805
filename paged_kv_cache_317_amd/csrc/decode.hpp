// Internal launchers of the decode kernels (host side).  The C ABI in
// pkv_api.cpp validates every argument and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Largest number of table entries one decode partition stages in LDS.
constexpr int kMaxPartBlocks = 512;

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* part_ml;          // [S, P, Hq, 2] (running max in log2 units, sum); split only
  void* part_o;            // [S, P, Hq, D]: bf16 caches o / l in bf16, f32 caches o in fp32
  int64_t num_blocks;
  int32_t table_width;
  int32_t num_seqs;
  int32_t q_heads;
  int32_t kv_heads;
  int32_t max_seq_len;
  int32_t part_tokens;     // multiple of the block size
  int32_t num_parts;       // partitions per sequence (1: no split)
  int32_t parts_per_unit;  // consecutive partitions one workgroup walks
  int32_t num_chunks;      // ceil(num_parts / parts_per_unit)
  int32_t heads_per_wg;    // kv heads per workgroup (one wave each)
  uint32_t row_bytes;      // one slot: kv_heads * head_dim * element bytes
  uint32_t tile_bytes;     // 16 slots
  uint32_t block_bytes;    // block_size slots
  float scale_log2;        // scale * log2(e)
};

// dtype: 0 f32, 1 bf16.  Returns hipErrorInvalidValue for a combination
// with no instantiated kernel (the API layer checks first).
bool decode_supported(int dtype, int head_dim, int block_size, int group);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                         int group, hipStream_t stream);

}  // namespace pkv
