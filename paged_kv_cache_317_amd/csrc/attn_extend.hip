// Block-aware attention of several new tokens per sequence (prefill and
// chunked extend) for gfx950.
//
// The keys and values of a sequence sit in fixed-size blocks reached through
// its block table, and the attention gathers them from there ("PagedAttention
// Explained: Virtual Memory for the KV Cache", "How PagedAttention works",
// steps 2, 3 and 5).  Here a sequence brings n new tokens at once -- the
// prefill pass that recomputes a preempted sequence ("Preemption and
// scheduling"), or a chunk of a long prompt.  Query j sits at position
// p = L - n + j and attends causally to positions 0 .. p; query head h reads
// kv head h / G.
//
// Unlike decode, each cached key is used by many query rows, so the work is
// a dense contraction and runs on the matrix cores.
//
// Work decomposition
//   column    one (query token, query head) pair of one kv head; the G heads
//             of a token are adjacent columns
//   workgroup 256 columns (256 / G tokens) of one sequence and kv head;
//             eight waves of 32 columns (two 16-column MFMA groups each;
//             wave and group counts are build options)
//   tile      64 consecutive key positions, staged in LDS once per
//             workgroup and read by all eight waves
//   partition a split call (num_parts > 1) also cuts the keys into
//             part_tokens-long ranges, one workgroup per range; each writes
//             its running max, sum and normalised output per column, and a
//             second kernel merges them in a fixed order (the same
//             max-rescaled combination the online softmax applies per tile)
// Workgroups are ordered so that the query tiles of one (sequence, kv head)
// land on one XCD (workgroup b runs on XCD b mod 8) and share its L2.
//
// Per tile and wave (bf16, head_dim 128):
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16; keys are the M rows (A operand,
//                 read from the K tile in LDS), the 16 columns of a
//                 group the N columns (B operand, held in registers for the
//                 whole call).  Lane (r, c) gets keys 4r..4r+3 of column c
//                 for each 16-key block.
//   softmax       online, base 2, scale folded with log2 e into one fma per
//                 weight; the tile max of a column is an in-lane max plus
//                 two row swaps; the running max moves only when passed by
//                 more than 8 (log2 units), so O is rarely rescaled; the
//                 causal and length mask is applied only on tiles that need
//                 it.
//   O^T += V^T P^T  v_mfma_f32_16x16x32_bf16 with the 32 keys of two 16-key
//                 blocks as the K dimension in the order that matches the
//                 logits' lane layout: P stays in its lanes (rounded to
//                 bf16), V^T comes from the V tile through
//                 ds_read_b64_tr_b16 transpose reads, shared by both groups.
// Loads: the next tile's K and V rows go straight from global memory into
// the other LDS buffer (buffer_load_dwordx4 ... lds, 16 bytes per lane, 1 KB
// per wave instruction) while the current tile computes; one barrier per
// tile.  The LDS rows are unpadded and their 16-byte chunks XOR-swizzled by
// row, which spreads both operand reads over the LDS banks.
#include "device_common.hpp"
#include "extend.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kD = 128;                  // head_dim
constexpr int kKeys = kExtendKeys;       // key positions per tile
constexpr int kWaves = PKV_EXTEND_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = kThreads / 16;     // K/V rows one pass of the workgroup loads
constexpr int kRowsPerThread = kKeys / kStep;
constexpr int kGroups = PKV_EXTEND_GROUPS;   // 16-column groups per wave
constexpr int kWaveCols = 16 * kGroups;
constexpr int kRow = kD * 2;             // LDS row of a K or V tile (bytes, unpadded)
constexpr int kTile = kKeys * kRow;
constexpr float kLazyLog2 = 8.f;         // running-max slack before O is rescaled
// Fourth word of a buffer resource for raw loads: 32-bit data format, no
// swizzle, no stride (num_records then counts bytes).
constexpr int kBufferWord3 = 0x00020000;
static_assert(kExtendCols == kWaves * 16 * kGroups, "kWaves waves of kGroups 16-column groups");
static_assert(kKeys % kStep == 0, "whole rows per thread");
static_assert(kStep % 16 == 0, "a load pass keeps every row's index mod 16");

#ifndef PKV_EXTEND_WAVES_PER_EU
#define PKV_EXTEND_WAVES_PER_EU 2
#endif

__device__ __forceinline__ bf16x8_t cat(bf16x4_t lo, bf16x4_t hi) {
  return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ bf16x4_t tr_read(const char* lds, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4_t*)((__attribute__((address_space(3))) char*)lds + byte_off));
}

// The 16-byte chunks of LDS row r are stored at chunk ^ chunk_swizzle(r).
// The LDS rows are unpadded (the tile loads write whole 1 KB runs), so
// without it the K operand reads (16 rows at one chunk) and the V transpose
// reads (4 rows x 2 adjacent chunks per 16 lanes) would hit the same banks.
// Of the XOR patterns measured this one was fastest; leaving it out halves
// the kernel's speed.
__device__ __forceinline__ int chunk_swizzle(int r) { return (r & 15) ^ ((r >> 2) & 3); }

// Sequences a workgroup ranks by their work to order the units (each thread
// ranks one sequence against all of them, so the cost grows with the square
// of this bound; larger batches have many units and keep their order).
constexpr int kRankSeqs = 64;

// (sequence, kv head) pairs an XCD orders by their live units (below).
constexpr int kOrderPairs = 64;

// New tokens of a sequence the kernel computes: its query rows clamped to
// max_query_len and to the packed rows; none when query_start is negative.
__device__ __forceinline__ int live_tokens(const ExtendArgs& a, int q0, int n_raw) {
  if (q0 < 0) return 0;
  return max(min(min(n_raw, a.max_query_len), a.num_tokens - q0), 0);
}

// Keys a query tile may read, before the scan for table entries outside the
// pool: below its last query's position + 1 (ctx + j1) and the sequence's
// bounds.  In a split call a tile whose bound fits the first partition is
// complete in that partition's workgroup, which stores its rows itself; the
// merge leaves them alone.
__device__ __forceinline__ int tile_key_bound(const ExtendArgs& a, int L, int ctx, int j1, int BS) {
  const int kv_end = max(min(min(L, a.max_seq_len), a.table_width * BS), 0);
  return max(min(ctx + j1, kv_end), 0);
}

// Causal work of a sequence in key visits: n new tokens after ctx cached
// positions see n * ctx + n (n + 1) / 2 keys (n and ctx as the kernel clamps
// them; only the order of these values is used).
__device__ __forceinline__ long long causal_work(const ExtendArgs& a, int q0, int n_raw, int L) {
  const long long n = live_tokens(a, q0, n_raw);
  const long long ctx = max(min(L, a.max_seq_len) - n_raw, 0);
  return n * ctx + n * (n + 1) / 2;
}

template <int BS, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PKV_EXTEND_WAVES_PER_EU)))
void extend_kernel(ExtendArgs a) {
  static_assert(BS == 16 || BS == 32, "block_size 16 or 32");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "G in {1, 2, 4, 8}");
  constexpr int kTokens = kExtendCols / G;       // query tokens per workgroup

  // Two tile buffers, one LDS object each: the compiler then sees that the
  // loads streaming into one buffer do not touch the other, and adds no
  // wait for them before reading it.
  __shared__ __attribute__((aligned(16))) char s_k0[kTile];
  __shared__ __attribute__((aligned(16))) char s_k1[kTile];
  __shared__ __attribute__((aligned(16))) char s_v0[kTile];
  __shared__ __attribute__((aligned(16))) char s_v1[kTile];
  char* const s_k[2] = {s_k0, s_k1};
  char* const s_v[2] = {s_v0, s_v1};
  __shared__ int s_first_bad;
  __shared__ long long s_work[kRankSeqs];
  __shared__ int s_seq[kRankSeqs][3];    // query_start, new tokens, length
  __shared__ int s_order[kRankSeqs];     // sequence of each rank
  __shared__ int s_units[kOrderPairs];   // live units of this XCD's pairs
  __shared__ int s_pick[2];              // this unit's pair slot, index in the pair

  // (sequence, kv head) pairs go round-robin over the XCDs (workgroup b runs
  // on XCD b mod 8); on its XCD a pair's query tiles are consecutive, so they
  // run side by side and read the pair's keys and values through one L2.
  // A split call (num_parts > 1) also cuts each query tile's keys into
  // partitions of part_tokens; the query tiles of one partition are adjacent.
  // Later (longer) query tiles come first.  The grid has q_tiles * num_parts
  // slots per pair, q_tiles counted from max_query_len.
  const int unit = (int)blockIdx.x;
  const int xcd = unit % 8;
  const int local = unit / 8;
  const int per_pair = a.q_tiles * a.num_parts;
  int pair = (local / per_pair) * 8 + xcd;
  int li = local % per_pair;
  int qtiles = a.q_tiles;
  // Longest sequences first: pair p of the order is kv head p % kv_heads of
  // the sequence ranked p / kv_heads by causal work (descending; ties by
  // index), so that on every XCD the units that take longest start first and
  // the last ones to finish are short.  Every workgroup ranks the sequences
  // itself (batches of up to kRankSeqs sequences; larger ones keep the order
  // of the batch), from one round of loads that also gives its own
  // sequence's start, new tokens and length.  When the XCD has at most
  // kOrderPairs pairs, its slots also skip the query tiles a sequence does
  // not have (fewer new tokens than max_query_len): each pair takes only its
  // live units, one after another, and the empty slots move to the end of the
  // grid, where they return at once instead of sitting between two pairs.
  int s, q0, n_raw, L;
  if (a.num_seqs > 1 && a.num_seqs <= kRankSeqs) {
    const int npairs = a.num_seqs * a.kv_heads;
    const int nx = npairs > xcd ? (npairs - xcd + 7) / 8 : 0;   // pairs xcd + 8 k
    const bool compact = nx <= kOrderPairs;
    if (!compact && pair >= npairs) return;          // uniform over the workgroup
    for (int i = threadIdx.x; i < a.num_seqs; i += kThreads) {
      const int qa = a.query_start[i];
      const int nr = a.query_start[i + 1] - qa;
      const int len = a.seq_lens[i];
      s_seq[i][0] = qa;
      s_seq[i][1] = nr;
      s_seq[i][2] = len;
      s_work[i] = causal_work(a, qa, nr, len);
    }
    if (threadIdx.x == 0) s_pick[0] = -1;
    __syncthreads();
    for (int i = threadIdx.x; i < a.num_seqs; i += kThreads) {
      const long long wi = s_work[i];
      int r = 0;
      for (int j = 0; j < a.num_seqs; ++j) {
        const long long wj = s_work[j];
        r += (wj > wi || (wj == wi && j < i)) ? 1 : 0;
      }
      s_order[r] = i;
    }
    __syncthreads();
    if (compact) {
      for (int k = threadIdx.x; k < nx; k += kThreads) {
        const int sq = s_order[(8 * k + xcd) / a.kv_heads];
        const int nl = live_tokens(a, s_seq[sq][0], s_seq[sq][1]);
        s_units[k] = (nl + kTokens - 1) / kTokens * a.num_parts;
      }
      __syncthreads();
      for (int k = threadIdx.x; k < nx; k += kThreads) {
        int before = 0;
        for (int k2 = 0; k2 < k; ++k2) before += s_units[k2];
        if (local >= before && local < before + s_units[k]) {
          s_pick[0] = k;
          s_pick[1] = local - before;
        }
      }
      __syncthreads();
      if (s_pick[0] < 0) return;                     // past this XCD's live units
      pair = 8 * s_pick[0] + xcd;
      li = s_pick[1];
      qtiles = s_units[s_pick[0]] / a.num_parts;
    }
    s = s_order[pair / a.kv_heads];
    q0 = s_seq[s][0];
    n_raw = s_seq[s][1];
    L = s_seq[s][2];
  } else {
    s = pair / a.kv_heads;
    if (s >= a.num_seqs) return;                     // uniform over the workgroup
    q0 = a.query_start[s];
    n_raw = a.query_start[s + 1] - q0;
    L = a.seq_lens[s];
  }
  const int g = pair % a.kv_heads;
  const int part = li / qtiles;
  const int qt = qtiles - 1 - li % qtiles;

  // Rows outside [0, num_tokens) are never read or written, whatever
  // query_start holds.
  if (q0 < 0) return;
  const int n = live_tokens(a, q0, n_raw);
  const int j0 = qt * kTokens;
  if (j0 >= n) return;
  const int j1 = min(j0 + kTokens, n);
  const int ctx = L - n_raw;                       // position of query 0

  // Keys this workgroup may read: below every query's position + 1 and the
  // sequence length; a table entry outside the pool ends the sequence at
  // that block.
  int kv_end = max(min(min(L, a.max_seq_len), a.table_width * BS), 0);
  int kv_hi = tile_key_bound(a, L, ctx, j1, BS);
  const bool direct = a.num_parts > 1 && kv_hi <= a.part_tokens;
  if (direct && part > 0) return;                  // uniform: its keys are all in partition 0
  const int nblk = (kv_hi + BS - 1) / BS;
  const int32_t* trow = a.block_table + (int64_t)s * a.table_width;
  if (threadIdx.x == 0) s_first_bad = nblk;
  __syncthreads();
  for (int j = threadIdx.x; j < nblk; j += kThreads) {
    const int b = trow[j];
    if (b < 0 || b >= a.num_blocks) atomicMin(&s_first_bad, j);
  }
  __syncthreads();
  kv_end = min(kv_end, s_first_bad * BS);
  kv_hi = min(kv_hi, kv_end);
  const int last_blk = max((kv_hi - 1) / BS, 0);
  // This unit's tiles: keys [part * part_tokens, min(+part_tokens, kv_hi)).
  const int t_first = part * (a.part_tokens / kKeys);
  const int t_stop = min(t_first + a.part_tokens / kKeys, (kv_hi + kKeys - 1) / kKeys);
  const int ntiles = max(t_stop - t_first, 0);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = lane >> 4;
  const int lc = lane & 15;

  // This lane's columns, their positions and the query rows as B operands.
  int qpos[kGroups];
  bool cvalid[kGroups];
  u32x4_t qv[kGroups][4];
#pragma unroll
  for (int cg = 0; cg < kGroups; ++cg) {
    const int col = kWaveCols * wave + 16 * cg + lc;
    const int j = j0 + col / G;
    cvalid[cg] = j < j1;
    const int jc = min(j, j1 - 1);
    qpos[cg] = ctx + jc;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((int64_t)(q0 + jc) * a.q_heads + g * G + col % G) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qv[cg][ks] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks + 8 * rg);
  }
  const bool wave_active = j0 + (kWaveCols * wave) / G < j1;
  const int qmin_w = ctx + min(j0 + (kWaveCols * wave) / G, j1 - 1);
  const int qmax_w = ctx + min(j0 + (kWaveCols * wave + kWaveCols - 1) / G, j1 - 1);

  // Tile loader: each wave instruction moves 4 rows (1 KB) straight from
  // global memory into LDS; lane l of wave w writes the l-th 16 bytes of
  // rows 4 w .. 4 w + 3 (+ kStep i), i.e. row lrow = l / 16 + 4 w, physical
  // chunk lchunk = l % 16, so it fetches the logical chunk lchunk ^ swizzle.
  // The loads are buffer loads through a resource spanning the one block
  // they read: with the flat-encoded global form the compiler cannot keep
  // partial LDS wait counts and drains every operand read (measured 3-6%
  // slower).
  const int lchunk = threadIdx.x & 15;
  const int lrow = threadIdx.x >> 4;
  const uint32_t lane_off =
      (uint32_t)(g * kD * 2 + 16 * (lchunk ^ chunk_swizzle(lrow & 15)));
  const char* kcache = reinterpret_cast<const char*>(a.k_cache);
  const char* vcache = reinterpret_cast<const char*>(a.v_cache);

  // Table entries of this thread's rows of a tile (the same for a whole
  // wave; vector loads, so that waiting for them never holds up the LDS
  // traffic of the tile being computed).
  // A wave's 64 threads load 4 consecutive rows (row base 4 * wave), which
  // lie in one 16-row block, so the entry index is wave-uniform.
  const int wave_row = uniform_int(4 * wave);
  auto fetch_entries = [&](int tile, int (&e)[kRowsPerThread]) {
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i)
      e[i] = trow[min((tile * kKeys + wave_row + kStep * i) / BS, last_blk)];
  };
  auto load_tile = [&](const int (&e)[kRowsPerThread], int buf) {
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const uint32_t phys = (uint32_t)uniform_int(e[i]);
      const uint64_t base = (uint64_t)phys * a.block_bytes;
      const uint32_t off = (uint32_t)(((lrow + kStep * i) % BS) * a.row_bytes) + lane_off;
      const int lds_row = uniform_int(wave_row + kStep * i);
      // Sizes and offsets are unsigned 32-bit in the hardware; the builtins
      // take them as int, bit for bit.
      const int nrec = __builtin_bit_cast(int, a.block_bytes);
      const int voff = __builtin_bit_cast(int, off);
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(kcache + base), 0, nrec, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(vcache + base), 0, nrec, kBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(s_k[buf] + lds_row * kRow), 16, voff, 0,
          0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)(s_v[buf] + lds_row * kRow), 16, voff, 0,
          0, 0);
    }
  };
  // Once this lane's loads of `tile` have landed: the rows it loaded at or
  // past kv_hi (only in the last tile) become zeros; they may be unused
  // slots holding any bits.
  auto zero_tail = [&](int tile, int buf) {
    const int t0 = tile * kKeys;
    if (uniform_int(t0 + kKeys > kv_hi ? 1 : 0)) {
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i) {
        if (t0 + lrow + kStep * i >= kv_hi) {
          const int at = (lrow + kStep * i) * kRow + 16 * lchunk;
          *reinterpret_cast<u32x4_t*>(s_k[buf] + at) = u32x4_t{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4_t*>(s_v[buf] + at) = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  // Running max per column; the softmax denominator accumulates in the
  // matrix pipe as the product of an all-ones operand with the weights
  // (every element of lsum[cg] holds the column's sum of the bf16 weights,
  // the same weights the value sum uses).
  float m_run[kGroups];
  f32x4_t lsum[kGroups];
  f32x4_t ot[kGroups][kD / 16];
#pragma unroll
  for (int cg = 0; cg < kGroups; ++cg) {
    m_run[cg] = -INFINITY;
    lsum[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) ot[cg][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Per-lane LDS offsets of the operand reads.
  // Swizzled rows: K chunk rg + 4 ks of row lc; V bytes 8 (lc & 3) + 32 db of
  // row 4 rg + lc / 4, i.e. chunk 2 db + (lc & 3) / 2, 8 (lc & 1) bytes in.
  // Blocks of 16 rows keep the row index mod 16, hence the swizzle.
  int ka_off[4], tr_off[kD / 16];
  {
    const int sk = chunk_swizzle(lc);
    const int vrow = 4 * rg + (lc >> 2);
    const int sv = chunk_swizzle(vrow);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka_off[ks] = lc * kRow + 16 * ((rg + 4 * ks) ^ sk);
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
      tr_off[db] = vrow * kRow + 16 * ((2 * db + ((lc & 3) >> 1)) ^ sv) + 8 * (lc & 1);
  }

  // The three stages of a tile.  A wave whose columns all sit before the
  // tile (tile_active false) skips all three.
  f32x4_t sacc[kGroups][4];   // logits of the tile between qk and softmax
  bf16x4_t pb[kGroups][4];    // its weights between softmax and pv
  auto tile_active = [&](int tile) { return wave_active && tile * kKeys <= qmax_w; };

  auto qk = [&](int buf) {
    const char* kt = s_k[buf];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4_t ka[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        ka[ks] = *reinterpret_cast<const u32x4_t*>(kt + ka_off[ks] + 16 * kb * kRow);
#pragma unroll
      for (int cg = 0; cg < kGroups; ++cg) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[ks]),
                                                        __builtin_bit_cast(bf16x8_t, qv[cg][ks]),
                                                        acc, 0, 0, 0);
        sacc[cg][kb] = acc;
      }
    }
  };

  auto softmax = [&](int tile) {
    const int t0 = tile * kKeys;
    // Only tiles that reach past the wave's first query position, or past
    // the readable keys, need the mask (a wave-uniform test).
    const bool need_mask =
        uniform_int((t0 + kKeys - 1 > qmin_w) || (t0 + kKeys > kv_hi) ? 1 : 0) != 0;
    if (need_mask) {
#pragma unroll
      for (int cg = 0; cg < kGroups; ++cg) {
        // keys 16 kb + i of this lane are visible while below `lim`
        const int lim = min(qpos[cg] + 1, kv_hi) - t0 - 4 * rg;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * kb + i >= lim) sacc[cg][kb][i] = -INFINITY;
      }
    }
#pragma unroll
    for (int cg = 0; cg < kGroups; ++cg) {
      // The scale is positive, so the tile max is taken on the raw logits.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[cg][kb][i]);
      mx = max_xor32(max_xor16(mx)) * a.scale_log2;
      // Lazy rescaling: the running max only moves when the tile max passes
      // it by more than kLazyLog2, so the weights stay below 2^kLazyLog2 and
      // most tiles skip the rescale of O.
      const float m_old = m_run[cg];
      const float m_new = mx > m_old + kLazyLog2 ? mx : m_old;
      // A column with nothing visible yet keeps weight 0 everywhere.
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      if (__any(m_new != m_old)) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_use);
        lsum[cg] *= alpha;
#pragma unroll
        for (int db = 0; db < kD / 16; ++db) ot[cg][db] *= alpha;
      }
      m_run[cg] = m_new;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pb[cg][kb][i] =
              (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[cg][kb][i], a.scale_log2, -m_use));
      }
    }
  };

  auto pv = [&](int buf) {
    const char* vt = s_v[buf];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) {
        const bf16x4_t a0 = tr_read(vt, tr_off[db] + 32 * kp * kRow);
        const bf16x4_t a1 = tr_read(vt, tr_off[db] + (32 * kp + 16) * kRow);
        const bf16x8_t av = cat(a0, a1);
#pragma unroll
        for (int cg = 0; cg < kGroups; ++cg)
          ot[cg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av, cat(pb[cg][2 * kp], pb[cg][2 * kp + 1]), ot[cg][db], 0, 0, 0);
      }
      const bf16x8_t ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                             (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int cg = 0; cg < kGroups; ++cg)
        lsum[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            ones, cat(pb[cg][2 * kp], pb[cg][2 * kp + 1]), lsum[cg], 0, 0, 0);
    }
  };

  if (ntiles > 0) {
    // Tile i+1 streams into LDS buffer (i+1) & 1 while tile i computes; that
    // buffer held tile i-1, released by the previous barrier.  The end of
    // step i waits for this wave's loads, clears the tail rows it loaded,
    // and the barrier publishes the tile.  Local tile i is absolute tile
    // t_first + i.
    int ent[kRowsPerThread];
    fetch_entries(t_first, ent);
    load_tile(ent, 0);
    fetch_entries(t_first + 1, ent);
    __builtin_amdgcn_s_waitcnt(0);
    zero_tail(t_first, 0);
    __syncthreads();
    // Unrolled by two so that every buffer index is a constant.
    auto step = [&](int i, auto cur) {
      constexpr int kCur = decltype(cur)::value;
      const int t = t_first + i;
      const bool more = i + 1 < ntiles;
      if (more) {
        load_tile(ent, kCur ^ 1);
        fetch_entries(t + 2, ent);
      }
      if (tile_active(t)) {
        qk(kCur);
        softmax(t);
        pv(kCur);
      }
      if (more) {
        __builtin_amdgcn_s_waitcnt(0);
        zero_tail(t + 1, kCur ^ 1);
      }
      __syncthreads();
    };
    for (int i = 0; i < ntiles; i += 2) {
      step(i, std::integral_constant<int, 0>());
      if (i + 1 >= ntiles) break;
      step(i + 1, std::integral_constant<int, 1>());
    }
  }

  if (a.num_parts > 1 && !direct) {
    // Split: each valid column's state for this partition -- running max
    // (log2 units) and sum in fp32, the output normalised by the sum in
    // bf16 -- at workspace row ((query row) * q_heads + head) * num_parts +
    // part.  A partition with no keys for a column leaves (-inf, 0, 0).
#pragma unroll
    for (int cg = 0; cg < kGroups; ++cg) {
      const float l_tot = lsum[cg][0];
      if (cvalid[cg]) {
        const int col = kWaveCols * wave + 16 * cg + lc;
        const int j = j0 + col / G;
        const int64_t idx =
            ((int64_t)(q0 + j) * a.q_heads + g * G + col % G) * a.num_parts + part;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* po = a.part_o + idx * kD + 4 * rg;
#pragma unroll
        for (int db = 0; db < kD / 16; ++db)
          *reinterpret_cast<f32x4_t*>(po + 16 * db) = ot[cg][db] * inv;
        if (rg == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * idx) = float2{m_run[cg], l_tot};
      }
    }
    return;
  }

#pragma unroll
  for (int cg = 0; cg < kGroups; ++cg) {
    const float l_tot = lsum[cg][0];
    if (cvalid[cg]) {
      const int col = kWaveCols * wave + 16 * cg + lc;
      const int j = j0 + col / G;
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      __bf16* out = reinterpret_cast<__bf16*>(a.out) +
                    ((int64_t)(q0 + j) * a.q_heads + g * G + col % G) * kD + 4 * rg;
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) {
        bf16x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(ot[cg][db][i] * inv);
        *reinterpret_cast<bf16x4_t*>(out + 16 * db) = w;
      }
    }
  }
}

// Merge of a split call: 32 lanes per (query row, head) of every computed
// row, lane i owning output elements 4i .. 4i + 3.  The partitions are folded
// in order with the online rescaling the kernel applies per tile: M the
// running max, each state weighted by 2^(m_p - M) l_p and the running sums
// rescaled when M moves; out = sum / weight.  Every load of a row is
// independent of the others, so a row costs one round trip.
constexpr int kMergeLanes = 32;
constexpr int kMergeRowsPerWg = 8;

__global__ __launch_bounds__(kMergeLanes * kMergeRowsPerWg) void extend_merge_kernel(ExtendArgs a) {
  const int sub = threadIdx.x % kMergeLanes;
  const int64_t u = (int64_t)blockIdx.x * kMergeRowsPerWg + threadIdx.x / kMergeLanes;
  const int h = (int)(u % a.q_heads);
  const int64_t rest = u / a.q_heads;
  const int j = (int)(rest % a.max_query_len);
  const int s = (int)(rest / a.max_query_len);
  if (s >= a.num_seqs) return;
  const int q0 = a.query_start[s];
  if (q0 < 0) return;
  const int n_raw = a.query_start[s + 1] - q0;
  const int n = live_tokens(a, q0, n_raw);
  if (j >= n) return;
  // Rows of a query tile whose keys fit the first partition: stored by the
  // kernel.
  const int tokens = kExtendCols / (a.q_heads / a.kv_heads);
  const int L = a.seq_lens[s];
  const int BS = (int)(a.block_bytes / a.row_bytes);
  if (tile_key_bound(a, L, L - n_raw, min((j / tokens + 1) * tokens, n), BS) <= a.part_tokens)
    return;
  const int64_t base = ((int64_t)(q0 + j) * a.q_heads + h) * a.num_parts;
  const float* ml = a.part_ml + 2 * base;
  const float* po = a.part_o + base * kD + 4 * sub;
  float M = -INFINITY, lsum = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.num_parts; ++p) {
    const float2 st = *reinterpret_cast<const float2*>(ml + 2 * p);
    const f32x4_t o4 = *reinterpret_cast<const f32x4_t*>(po + (int64_t)p * kD);
    if (st.x == -INFINITY) continue;              // no key of this partition for the row
    if (st.x > M) {
      const float c = __builtin_amdgcn_exp2f(M - st.x);   // 0 while M is -inf
      lsum *= c;
      acc *= c;
      M = st.x;
    }
    const float w = __builtin_amdgcn_exp2f(st.x - M) * st.y;
    lsum += w;
    acc += w * o4;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  bf16x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x4_t*>(reinterpret_cast<__bf16*>(a.out) +
                               ((int64_t)(q0 + j) * a.q_heads + h) * kD + 4 * sub) = r;
}

template <int BS, int G>
hipError_t launch_one(const ExtendArgs& a, hipStream_t stream) {
  // Unit u maps to pair (u / 8 / per_pair) * 8 + u % 8: the grid covers every
  // pair index below num_seqs * kv_heads rounded up to 8.
  const int pairs8 = 8 * ((a.num_seqs * a.kv_heads + 7) / 8);
  const int grid = pairs8 * a.q_tiles * a.num_parts;
  hipLaunchKernelGGL((extend_kernel<BS, G>), dim3(grid), dim3(kThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_parts == 1) return err;
  const int64_t rows = (int64_t)a.num_seqs * a.max_query_len * a.q_heads;
  hipLaunchKernelGGL(extend_merge_kernel, dim3((unsigned)((rows + kMergeRowsPerWg - 1) / kMergeRowsPerWg)),
                     dim3(kMergeLanes * kMergeRowsPerWg), 0, stream, a);
  return hipGetLastError();
}

template <int BS>
hipError_t launch_bs(const ExtendArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<BS, 1>(a, stream);
    case 2: return launch_one<BS, 2>(a, stream);
    case 4: return launch_one<BS, 4>(a, stream);
    case 8: return launch_one<BS, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool extend_supported(int dtype, int head_dim, int block_size, int group) {
  return dtype == 1 && head_dim == kD && (block_size == 16 || block_size == 32) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_extend(const ExtendArgs& a, int block_size, int group, hipStream_t stream) {
  if (a.units <= 0) return hipSuccess;
  if (block_size == 16) return launch_bs<16>(a, group, stream);
  if (block_size == 32) return launch_bs<32>(a, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
