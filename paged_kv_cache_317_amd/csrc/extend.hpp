// Internal launcher of the multi-token (prefill / extend) attention kernel
// (host side).  The C ABI in pkv_api.cpp validates every argument first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct ExtendArgs {
  const void* q;               // [T, q_heads, head_dim]
  const void* k_cache;
  const void* v_cache;
  void* out;                   // [T, q_heads, head_dim]
  const int32_t* block_table;  // [num_seqs, table_width]
  const int32_t* seq_lens;     // [num_seqs], new tokens included
  const int32_t* query_start;  // [num_seqs + 1]
  int64_t num_blocks;
  int32_t table_width;
  int32_t num_seqs;
  int32_t num_tokens;          // rows of q and out; rows at or past it are never touched
  int32_t q_heads;
  int32_t kv_heads;
  int32_t max_query_len;       // host bound on query_start[s+1] - query_start[s]
  int32_t max_seq_len;         // host bound on seq_lens; keys at or past it are not read
  int32_t q_tiles;             // query tiles per (sequence, kv head)
  int32_t units;               // num_seqs * kv_heads * q_tiles * num_parts
  int32_t part_tokens;         // keys per partition (a multiple of 64)
  int32_t num_parts;           // partitions per query tile (1: no split)
  float* part_ml;              // split: [T, Hq, P, 2] (max in log2 units, sum)
  float* part_o;               // split: [T, Hq, P, D] fp32, normalised
  uint32_t row_bytes;          // one slot: kv_heads * head_dim * element bytes
  uint32_t block_bytes;        // block_size slots
  float scale_log2;            // scale * log2(e)
};

// Waves per workgroup and 16-column MFMA groups per wave.
#ifndef PKV_EXTEND_WAVES
#define PKV_EXTEND_WAVES 8
#endif
#ifndef PKV_EXTEND_GROUPS
#define PKV_EXTEND_GROUPS 2
#endif
// Query columns (token, head) one workgroup covers; a workgroup holds
// kExtendCols / G query tokens of one sequence.
constexpr int kExtendCols = PKV_EXTEND_WAVES * 16 * PKV_EXTEND_GROUPS;

// Keys per LDS tile of the extend kernel: partition lengths are multiples.
constexpr int kExtendKeys = 64;

bool extend_supported(int dtype, int head_dim, int block_size, int group);
hipError_t launch_extend(const ExtendArgs& a, int block_size, int group, hipStream_t stream);

}  // namespace pkv
