// Internal launchers of the decode kernels (host side).  The C ABI in
// pkv_api.cpp validates every argument and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Tiles (16 token positions each) one workgroup's run of the work stream may
// hold: the run's table entries are staged in LDS, one per tile.
constexpr int kMaxRangeTiles = 1024;
// Longest partition a call may ask for, in tiles (8192 positions).
constexpr int kMaxPartTiles = 512;

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  const int32_t* block_table;
  const int32_t* seq_lens;
  // Split calls (num_ranges > 1) only, all in the workspace:
  int32_t* plan;           // [S+1] stream prefix (units), [groups] shared tiles, [2] run lengths
  float* part_ml;          // [slots, rows, 2]: running max (log2 units), sum
  float* part_o;           // [slots, rows, D]: unnormalised output, fp32
  int64_t num_blocks;
  int32_t table_width;
  int32_t num_seqs;
  int32_t q_heads;
  int32_t kv_heads;
  int32_t max_seq_len;
  int32_t part_tiles;      // tiles per partition, the unit of the work stream
  int32_t num_ranges;      // runs of the work stream (1: no merge)
  int32_t odd_q10;         // odd runs' share of an even run's work, in 1/1024
  int32_t heads_per_wg;    // kv heads per workgroup (one wave each)
  uint32_t row_bytes;      // one slot: kv_heads * head_dim * element bytes
  uint32_t tile_bytes;     // 16 slots
  float scale_log2;        // scale * log2(e)
};

// Sequences whose query heads share one wave's 16 matrix columns: 16 / G for
// bf16 caches, 1 for f32 caches.
constexpr int decode_group_size(int dtype, int group) { return dtype == 1 ? 16 / group : 1; }

// Bytes of dynamically sized LDS a decode workgroup needs for num_seqs
// sequences (the per-sequence plan of the work stream).
int64_t decode_plan_lds_bytes(int dtype, int group, int64_t num_seqs);

// Largest dynamically sized LDS a decode workgroup may use.
int64_t decode_max_plan_lds_bytes();

// dtype: 0 f32, 1 bf16.  Returns hipErrorInvalidValue for a combination
// with no instantiated kernel (the API layer checks first).
bool decode_supported(int dtype, int head_dim, int block_size, int group);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                         int group, hipStream_t stream);

}  // namespace pkv
