// C ABI of libpkv: argument checks, the split decision, and dispatch to the
// kernel launchers.  Every check runs on the host before any HIP call, so an
// invalid call launches nothing and touches no device state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/pkv.h"
#include "cache_ops.hpp"
#include "decode.hpp"
#include "extend.hpp"
#include "status.hpp"

namespace pkv {
const char* last_error();
}

// Kv heads (one wave each) per decode workgroup, when kv_heads allows it.
#ifndef PKV_DECODE_HEADS_PER_WG
#define PKV_DECODE_HEADS_PER_WG 4
#endif

// Waves a decode grid aims for: the work stream is cut into this many waves'
// worth of runs (kv_heads waves per run).
#ifndef PKV_DECODE_WAVE_TARGET
#define PKV_DECODE_WAVE_TARGET 2048
#endif

// Work of a run on an odd XCD relative to one on an even XCD, in 1/1024.  On
// the HBM-bound decode gather the odd XCDs of an MI355X take about 8% longer
// per tile than the even ones (per-wave timing, several batches and boxes),
// so equal runs leave the even XCDs idle at the end of the call.
#ifndef PKV_DECODE_ODD_XCD_Q10
#define PKV_DECODE_ODD_XCD_Q10 942
#endif

namespace pkv {
namespace {
thread_local std::string g_last_error;
}  // namespace

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

const char* last_error() { return g_last_error.c_str(); }

}  // namespace pkv

namespace {

using pkv::fail;
using pkv::ok;

pkv_status from_hip(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }

pkv_status check_cache(const pkv_cache_desc* c) {
  if (!c) return fail(PKV_ERR_NULL, "cache descriptor is NULL");
  if (c->dtype != PKV_F32 && c->dtype != PKV_BF16)
    return fail(PKV_ERR_DTYPE, "unknown dtype code %d", (int)c->dtype);
  if (c->num_blocks < 1 || c->block_size < 1 || c->kv_heads < 1 || c->head_dim < 1)
    return fail(PKV_ERR_SHAPE, "cache sizes must be positive (num_blocks %d, block_size %d, "
                "kv_heads %d, head_dim %d)", (int)c->num_blocks, (int)c->block_size,
                (int)c->kv_heads, (int)c->head_dim);
  const int64_t row = (int64_t)c->head_dim * elem_bytes(c->dtype);
  if (row % 16) return fail(PKV_ERR_UNSUPPORTED, "head_dim * element size must be a multiple of 16 bytes");
  return PKV_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Split policy.  The work stream (every sequence's tiles of 16 positions, in
// partitions of part_tiles tiles) is cut into num_ranges equal runs, one
// workgroup of up to four waves (kv heads) per run and kv-head group.  The
// host sees only max_seq_len, so the run count comes from the largest
// stream the call can have: enough runs for about kWaveTarget waves, no run
// shorter than kMinRunTiles tiles on a full-length batch, and no run longer
// than the kMaxRangeTiles tile slots a workgroup stages in LDS.  A batch too
// small for kFillWaves waves at that run length still gets that many waves
// (one partition per run at most): with the chip that empty, a tile costs
// the latency of its loads, so shorter runs finish sooner than the merge
// they add costs.  With one run the call needs no workspace and no merge.
constexpr int64_t kWaveTarget = PKV_DECODE_WAVE_TARGET;
constexpr int64_t kMinRunTiles = 32;
constexpr int64_t kFillWaves = 1024;   // 256 CUs, one four-wave workgroup each

struct DecodePlan {
  int64_t part_tiles = 1;
  int64_t num_ranges = 1;
  int64_t odd_q10 = 1024;
  int64_t lds = 0;
  size_t plan_bytes = 0;    // workspace: stream plan (int32)
  size_t ml_bytes = 0;      //            run states' (max, sum)
  size_t workspace = 0;
};

int64_t ceil_div64(int64_t x, int64_t y) { return (x + y - 1) / y; }

pkv_status plan_decode(const pkv_cache_desc* c, int32_t num_seqs, int32_t q_heads,
                       int32_t max_seq_len, int32_t part_tokens, DecodePlan* plan) {
  pkv_status st = check_cache(c);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_seq_len < 0 || part_tokens < 0)
    return fail(PKV_ERR_SHAPE, "num_seqs, max_seq_len and part_tokens must be >= 0");
  if (q_heads < 1 || q_heads % c->kv_heads)
    return fail(PKV_ERR_SHAPE, "q_heads (%d) must be a positive multiple of kv_heads (%d)",
                (int)q_heads, (int)c->kv_heads);
  const int group = q_heads / c->kv_heads;
  if (!pkv::decode_supported(c->dtype, c->head_dim, c->block_size, group))
    return fail(PKV_ERR_UNSUPPORTED, "no decode kernel for dtype %d, head_dim %d, block_size %d, "
                "group %d (built: f32 head_dim 64, bf16 head_dim 128; block 16 or 32; group 1, "
                "2, 4 or 8)", (int)c->dtype, (int)c->head_dim, (int)c->block_size, group);
  // Staged tile addresses (block * tiles per block + tile) keep the top bit
  // free for a flag.
  if ((int64_t)c->num_blocks * (c->block_size / 16) > (int64_t{1} << 31) - 16)
    return fail(PKV_ERR_UNSUPPORTED, "a pool of %d blocks of %d tokens is too large for decode",
                (int)c->num_blocks, (int)c->block_size);
  const int64_t pt =
      part_tokens > 0 ? std::min<int64_t>(ceil_div64(part_tokens, 16), pkv::kMaxPartTiles) : 1;
  // Tiles a member can own: its own tiles, or (block 32) the shared tiles of
  // its group, one more at most.
  const int64_t tmax = ceil_div64(max_seq_len, 16) + (c->block_size / 16 - 1);
  const int64_t units_bound = (int64_t)num_seqs * ceil_div64(tmax, pt);
  if (units_bound > INT32_MAX / 2)
    return fail(PKV_ERR_SHAPE, "num_seqs * max_seq_len is too large for one decode call");
  int64_t n = ceil_div64(kWaveTarget, c->kv_heads);
  const int64_t fill = std::min(ceil_div64(kFillWaves, c->kv_heads), units_bound);
  n = std::min(n, std::max({int64_t{1}, ceil_div64(units_bound, ceil_div64(kMinRunTiles, pt)), fill}));
  n = std::max(n, ceil_div64(units_bound, pkv::kMaxRangeTiles / pt));
  n = std::max<int64_t>(1, std::min(n, std::max<int64_t>(units_bound, 1)));
  // From 8 runs on: a multiple of 8, each run on one XCD, odd XCDs' runs
  // shorter; the longest (even) run still fits the staged tile slots.
  int64_t odd_q10 = 1024;
  if (n >= 8) {
    n = round_up(n, 8);
    odd_q10 = PKV_DECODE_ODD_XCD_Q10;
    auto longest = [&](int64_t nn) {
      const int64_t pairs_q10 = (nn / 2) * (1024 + odd_q10);
      return ceil_div64(units_bound * 1024, pairs_q10);
    };
    while (longest(n) * pt > pkv::kMaxRangeTiles) n += 8;
  }
  plan->part_tiles = pt;
  plan->num_ranges = n;
  plan->odd_q10 = odd_q10;
  plan->lds = pkv::decode_plan_lds_bytes(c->dtype, group, num_seqs);
  if (plan->lds > pkv::decode_max_plan_lds_bytes())
    return fail(PKV_ERR_UNSUPPORTED, "%d sequences exceed what one decode call plans in LDS "
                "(split the batch)", (int)num_seqs);
  plan->plan_bytes = plan->ml_bytes = plan->workspace = 0;
  if (n > 1) {
    const int64_t gs = pkv::decode_group_size(c->dtype, group);
    const int64_t groups = ceil_div64(num_seqs, gs);
    const int64_t slots = n + groups;
    const int64_t rows = slots * c->kv_heads * gs * group;
    plan->plan_bytes = (size_t)round_up(num_seqs + 1 + groups + 2, 4) * sizeof(int32_t);
    plan->ml_bytes = (size_t)round_up(2 * rows, 4) * sizeof(float);
    plan->workspace = plan->plan_bytes + plan->ml_bytes + (size_t)(rows * c->head_dim) * sizeof(float);
  }
  return PKV_OK;
}

}  // namespace

PKV_EXPORT const char* pkv_last_error(void) { return pkv::last_error(); }

PKV_EXPORT const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }

PKV_EXPORT pkv_status pkv_paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping,
                                         int64_t num_tokens, void* k_cache, void* v_cache,
                                         const pkv_cache_desc* cache, void* stream) {
  pkv_status st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return fail(PKV_ERR_SHAPE, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_ERR_NULL, "k, v, slot_mapping, k_cache and v_cache must be non-NULL");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_ALIGN, "k, v, k_cache and v_cache must be 16-byte aligned");
  pkv::KvWriteArgs a;
  a.k = k;
  a.v = v;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_slots = (int64_t)cache->num_blocks * cache->block_size;
  a.row_bytes = (int64_t)cache->kv_heads * cache->head_dim * elem_bytes(cache->dtype);
  return from_hip(pkv::launch_kv_write(a, (hipStream_t)stream), "paged_kv_write launch");
}

PKV_EXPORT int32_t pkv_decode_partition_tokens(const pkv_cache_desc* cache, int32_t num_seqs,
                                               int32_t q_heads, int32_t max_seq_len,
                                               int32_t part_tokens) {
  DecodePlan plan;
  if (plan_decode(cache, num_seqs, q_heads, max_seq_len, part_tokens, &plan) != PKV_OK) return 0;
  ok();
  return (int32_t)(plan.part_tiles * 16);
}

PKV_EXPORT int32_t pkv_decode_runs(const pkv_cache_desc* cache, int32_t num_seqs,
                                   int32_t q_heads, int32_t max_seq_len, int32_t part_tokens) {
  DecodePlan plan;
  if (plan_decode(cache, num_seqs, q_heads, max_seq_len, part_tokens, &plan) != PKV_OK) return 0;
  ok();
  return (int32_t)plan.num_ranges;
}

PKV_EXPORT size_t pkv_decode_workspace_size(const pkv_cache_desc* cache, int32_t num_seqs,
                                            int32_t q_heads, int32_t max_seq_len,
                                            int32_t part_tokens) {
  DecodePlan plan;
  if (plan_decode(cache, num_seqs, q_heads, max_seq_len, part_tokens, &plan) != PKV_OK) return 0;
  ok();
  return plan.workspace;
}

PKV_EXPORT pkv_status pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                            const pkv_cache_desc* cache, const int32_t* block_table,
                                            int32_t table_width, const int32_t* seq_lens,
                                            int32_t num_seqs, int32_t q_heads, int32_t max_seq_len,
                                            float scale, void* out, int32_t part_tokens,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan plan;
  pkv_status st = plan_decode(cache, num_seqs, q_heads, max_seq_len, part_tokens, &plan);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return ok();
  if (table_width < 1) return fail(PKV_ERR_SHAPE, "table_width must be >= 1");
  if ((int64_t)table_width * cache->block_size > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "table_width * block_size exceeds the int32 token range");
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out)
    return fail(PKV_ERR_NULL, "q, k_cache, v_cache, block_table, seq_lens and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PKV_ERR_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (plan.workspace > 0) {
    if (!workspace) return fail(PKV_ERR_WORKSPACE, "this call splits into %lld runs and needs "
                                "a %zu-byte workspace", (long long)plan.num_ranges, plan.workspace);
    if (workspace_bytes < plan.workspace)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed",
                  workspace_bytes, plan.workspace);
    if (!aligned16(workspace)) return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  int heads_per_wg = 1;
  for (int w : {PKV_DECODE_HEADS_PER_WG, 4, 2}) {
    if (cache->kv_heads % w == 0) {
      heads_per_wg = w;
      break;
    }
  }
  const int group = q_heads / cache->kv_heads;
  const int64_t block_bytes =
      (int64_t)cache->block_size * cache->kv_heads * cache->head_dim * elem_bytes(cache->dtype);
  if (block_bytes > UINT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "a block of %lld bytes exceeds 4 GiB", (long long)block_bytes);
  const int64_t units = plan.num_ranges * (cache->kv_heads / heads_per_wg);
  if (units > INT32_MAX || (int64_t)num_seqs * q_heads > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)units);

  pkv::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.plan = nullptr;
  a.part_ml = nullptr;
  a.part_o = nullptr;
  if (plan.workspace > 0) {
    char* ws = static_cast<char*>(workspace);
    a.plan = reinterpret_cast<int32_t*>(ws);
    a.part_ml = reinterpret_cast<float*>(ws + plan.plan_bytes);
    a.part_o = reinterpret_cast<float*>(ws + plan.plan_bytes + plan.ml_bytes);
  }
  a.num_blocks = cache->num_blocks;
  a.table_width = table_width;
  a.num_seqs = num_seqs;
  a.q_heads = q_heads;
  a.kv_heads = cache->kv_heads;
  a.max_seq_len = max_seq_len;
  a.part_tiles = (int32_t)plan.part_tiles;
  a.num_ranges = (int32_t)plan.num_ranges;
  a.odd_q10 = (int32_t)plan.odd_q10;
  a.heads_per_wg = heads_per_wg;
  a.row_bytes = (uint32_t)((int64_t)cache->kv_heads * cache->head_dim * elem_bytes(cache->dtype));
  a.tile_bytes = 16u * a.row_bytes;
  a.scale_log2 = scale * 1.4426950408889634f;
  return from_hip(pkv::launch_decode(a, cache->dtype, cache->head_dim, cache->block_size, group,
                                     (hipStream_t)stream),
                  "paged_attn_decode launch");
}

namespace {

// Extend split policy.  The grid has num_seqs * kv_heads * q_tiles
// workgroups, and one of them (8 waves at two waves per SIMD) fills a CU;
// with fewer than kExtendUnitTarget of them and long keys, each query tile's
// keys are cut into partitions so that the grid reaches the target, never
// shorter than kMinExtendPart keys.
constexpr int64_t kExtendUnitTarget = 256;
constexpr int64_t kMinExtendPart = 1024;

struct ExtendPlan {
  int64_t q_tiles = 0;
  int64_t part_tokens = 0;
  int64_t num_parts = 1;
  size_t workspace = 0;
};

pkv_status plan_extend(const pkv_cache_desc* c, int32_t num_seqs, int32_t num_tokens,
                       int32_t q_heads, int32_t max_query_len, int32_t max_seq_len,
                       int32_t part_tokens, ExtendPlan* plan) {
  pkv_status st = check_cache(c);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || max_seq_len < 0 || part_tokens < 0)
    return fail(PKV_ERR_SHAPE, "num_seqs, num_tokens, max_query_len, max_seq_len and "
                "part_tokens must be >= 0");
  if (q_heads < 1 || q_heads % c->kv_heads)
    return fail(PKV_ERR_SHAPE, "q_heads (%d) must be a positive multiple of kv_heads (%d)",
                (int)q_heads, (int)c->kv_heads);
  const int group = q_heads / c->kv_heads;
  if (!pkv::extend_supported(c->dtype, c->head_dim, c->block_size, group))
    return fail(PKV_ERR_UNSUPPORTED, "extend attention supports bf16 caches with head_dim 128, "
                "block_size 16 or 32 and G in {1, 2, 4, 8} (got dtype %d, head_dim %d, "
                "block_size %d, G %d)", (int)c->dtype, (int)c->head_dim,
                (int)c->block_size, group);
  const int64_t tokens_per_wg = pkv::kExtendCols / group;
  plan->q_tiles = (max_query_len + tokens_per_wg - 1) / tokens_per_wg;
  const int64_t keys = std::max<int64_t>(max_seq_len, 1);
  const int64_t units = (int64_t)num_seqs * c->kv_heads * plan->q_tiles;
  int64_t pt;
  if (part_tokens > 0) {
    pt = part_tokens;
  } else if (units >= kExtendUnitTarget || keys <= kMinExtendPart || units == 0) {
    pt = keys;
  } else {
    const int64_t parts = (kExtendUnitTarget + units - 1) / units;
    pt = std::max<int64_t>((keys + parts - 1) / parts, kMinExtendPart);
  }
  pt = round_up(std::min<int64_t>(pt, keys), pkv::kExtendKeys);
  if (pt > INT32_MAX / 2) return fail(PKV_ERR_SHAPE, "partition of %lld keys is too long", (long long)pt);
  plan->part_tokens = pt;
  plan->num_parts = (keys + pt - 1) / pt;
  plan->workspace = 0;
  if (plan->num_parts > 1) {
    // fp32 (max, sum) and fp32 normalised output per row and partition
    const int64_t rows = (int64_t)num_tokens * q_heads * plan->num_parts;
    plan->workspace = (size_t)(round_up(2 * rows, 4) + rows * c->head_dim) * sizeof(float);
  }
  return PKV_OK;
}

}  // namespace

PKV_EXPORT int32_t pkv_extend_partition_tokens(const pkv_cache_desc* cache, int32_t num_seqs,
                                               int32_t num_tokens, int32_t q_heads,
                                               int32_t max_query_len, int32_t max_seq_len,
                                               int32_t part_tokens) {
  ExtendPlan plan;
  if (plan_extend(cache, num_seqs, num_tokens, q_heads, max_query_len, max_seq_len, part_tokens,
                  &plan) != PKV_OK)
    return 0;
  ok();
  return (int32_t)plan.part_tokens;
}

PKV_EXPORT size_t pkv_extend_workspace_size(const pkv_cache_desc* cache, int32_t num_seqs,
                                            int32_t num_tokens, int32_t q_heads,
                                            int32_t max_query_len, int32_t max_seq_len,
                                            int32_t part_tokens) {
  ExtendPlan plan;
  if (plan_extend(cache, num_seqs, num_tokens, q_heads, max_query_len, max_seq_len, part_tokens,
                  &plan) != PKV_OK)
    return 0;
  ok();
  return plan.workspace;
}

PKV_EXPORT pkv_status pkv_paged_attn_extend(const void* q, const void* k_cache, const void* v_cache,
                                            const pkv_cache_desc* cache, const int32_t* block_table,
                                            int32_t table_width, const int32_t* seq_lens,
                                            const int32_t* query_start, int32_t num_seqs,
                                            int32_t num_tokens, int32_t q_heads,
                                            int32_t max_query_len, int32_t max_seq_len,
                                            float scale, void* out, int32_t part_tokens,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
  ExtendPlan plan;
  pkv_status st = plan_extend(cache, num_seqs, num_tokens, q_heads, max_query_len, max_seq_len,
                              part_tokens, &plan);
  if (st != PKV_OK) return st;
  if (!(scale > 0.f) || !(scale < INFINITY))
    return fail(PKV_ERR_SHAPE, "scale must be positive and finite");
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return ok();
  if (table_width < 1) return fail(PKV_ERR_SHAPE, "table_width must be >= 1");
  if ((int64_t)table_width * cache->block_size > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "table_width * block_size exceeds the int32 token range");
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !query_start || !out)
    return fail(PKV_ERR_NULL, "q, k_cache, v_cache, block_table, seq_lens, query_start and out "
                "must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PKV_ERR_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (plan.workspace > 0) {
    if (!workspace)
      return fail(PKV_ERR_WORKSPACE, "this call splits into %lld partitions and needs a "
                  "%zu-byte workspace", (long long)plan.num_parts, plan.workspace);
    if (workspace_bytes < plan.workspace)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed",
                  workspace_bytes, plan.workspace);
    if (!aligned16(workspace)) return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  const int group = q_heads / cache->kv_heads;
  const int64_t row_bytes = (int64_t)cache->kv_heads * cache->head_dim * elem_bytes(cache->dtype);
  const int64_t block_bytes = row_bytes * cache->block_size;
  if (block_bytes > UINT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "a block of %lld bytes exceeds 4 GiB", (long long)block_bytes);
  const int64_t units = (int64_t)num_seqs * cache->kv_heads * plan.q_tiles * plan.num_parts;
  // The launch rounds the (sequence, kv head) pairs up to a multiple of 8.
  const int64_t grid =
      ((int64_t)num_seqs * cache->kv_heads + 7) / 8 * 8 * plan.q_tiles * plan.num_parts;
  const int64_t merge_rows = (int64_t)num_seqs * max_query_len * q_heads;
  if (grid > INT32_MAX || merge_rows > (int64_t)INT32_MAX * 4)
    return fail(PKV_ERR_SHAPE, "grid of %lld workgroups is too large", (long long)grid);

  pkv::ExtendArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.query_start = query_start;
  a.num_blocks = cache->num_blocks;
  a.table_width = table_width;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.q_heads = q_heads;
  a.kv_heads = cache->kv_heads;
  a.max_query_len = max_query_len;
  a.max_seq_len = std::max(max_seq_len, 1);
  a.q_tiles = (int32_t)plan.q_tiles;
  a.units = (int32_t)units;
  a.part_tokens = (int32_t)plan.part_tokens;
  a.num_parts = (int32_t)plan.num_parts;
  a.part_ml = nullptr;
  a.part_o = nullptr;
  if (plan.workspace > 0) {
    const int64_t rows = (int64_t)num_tokens * q_heads * plan.num_parts;
    a.part_ml = static_cast<float*>(workspace);
    a.part_o = a.part_ml + round_up(2 * rows, 4);
  }
  a.row_bytes = (uint32_t)row_bytes;
  a.block_bytes = (uint32_t)block_bytes;
  a.scale_log2 = scale * 1.4426950408889634f;
  return from_hip(pkv::launch_extend(a, cache->block_size, group, (hipStream_t)stream),
                  "paged_attn_extend launch");
}

PKV_EXPORT pkv_status pkv_paged_block_copy(const int64_t* pairs, int32_t num_pairs, void* k_cache,
                                           void* v_cache, const pkv_cache_desc* cache,
                                           void* stream) {
  pkv_status st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return fail(PKV_ERR_SHAPE, "num_pairs must be >= 0");
  if (num_pairs == 0) return ok();
  if (!pairs || !k_cache || !v_cache)
    return fail(PKV_ERR_NULL, "pairs, k_cache and v_cache must be non-NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_ALIGN, "k_cache and v_cache must be 16-byte aligned");
  pkv::BlockMoveArgs a;
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.src_k = k_cache;
  a.src_v = v_cache;
  a.dst_k = k_cache;
  a.dst_v = v_cache;
  a.src_blocks = a.dst_blocks = cache->num_blocks;
  a.streaming = true;
  a.block_bytes = (int64_t)cache->block_size * cache->kv_heads * cache->head_dim *
                  elem_bytes(cache->dtype);
  if (pkv::block_move_workgroups(a) > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "too many pairs for one launch");
  return from_hip(pkv::launch_block_move(a, (hipStream_t)stream), "paged_block_copy launch");
}

namespace {

// The address a kernel uses for `p`: device memory as is, pinned host memory
// through its device mapping.  Pageable host memory (or anything the runtime
// does not know) is refused, so a kernel never dereferences it.
pkv_status device_address(const void* p, const char* name, void** out) {
  hipPointerAttribute_t attr{};
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKV_ERR_UNSUPPORTED, "%s is neither device memory nor pinned host memory", name);
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = const_cast<void*>(p);
    return PKV_OK;
  }
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, const_cast<void*>(p), 0);
    if (e != hipSuccess || !d) {
      (void)hipGetLastError();
      return fail(PKV_ERR_UNSUPPORTED, "%s is host memory without a device mapping", name);
    }
    *out = d;
    return PKV_OK;
  }
  return fail(PKV_ERR_UNSUPPORTED, "%s is neither device memory nor pinned host memory", name);
}

}  // namespace

PKV_EXPORT pkv_status pkv_paged_block_move(const int64_t* pairs, int32_t num_pairs,
                                           const void* src_k, const void* src_v,
                                           const pkv_cache_desc* src, void* dst_k, void* dst_v,
                                           const pkv_cache_desc* dst, void* stream) {
  pkv_status st = check_cache(src);
  if (st != PKV_OK) return st;
  st = check_cache(dst);
  if (st != PKV_OK) return st;
  if (src->block_size != dst->block_size || src->kv_heads != dst->kv_heads ||
      src->head_dim != dst->head_dim || src->dtype != dst->dtype)
    return fail(PKV_ERR_SHAPE, "source and destination pools must have the same block shape and dtype");
  if (num_pairs < 0) return fail(PKV_ERR_SHAPE, "num_pairs must be >= 0");
  if (num_pairs == 0) return ok();
  if (!pairs || !src_k || !src_v || !dst_k || !dst_v)
    return fail(PKV_ERR_NULL, "pairs and the four pool pointers must be non-NULL");
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return fail(PKV_ERR_ALIGN, "pool pointers must be 16-byte aligned");
  pkv::BlockMoveArgs a;
  void* p = nullptr;
  if ((st = device_address(pairs, "pairs", &p)) != PKV_OK) return st;
  a.pairs = static_cast<const int64_t*>(p);
  if ((st = device_address(src_k, "src_k", &p)) != PKV_OK) return st;
  a.src_k = p;
  if ((st = device_address(src_v, "src_v", &p)) != PKV_OK) return st;
  a.src_v = p;
  if ((st = device_address(dst_k, "dst_k", &p)) != PKV_OK) return st;
  a.dst_k = p;
  if ((st = device_address(dst_v, "dst_v", &p)) != PKV_OK) return st;
  a.dst_v = p;
  a.num_pairs = num_pairs;
  a.src_blocks = src->num_blocks;
  a.dst_blocks = dst->num_blocks;
  a.block_bytes = (int64_t)src->block_size * src->kv_heads * src->head_dim * elem_bytes(src->dtype);
  if (pkv::block_move_workgroups(a) > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "too many pairs for one launch");
  a.streaming = false;
  return from_hip(pkv::launch_block_move(a, (hipStream_t)stream), "paged_block_move launch");
}
