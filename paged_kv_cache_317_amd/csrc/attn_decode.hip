// Block-aware decode attention for gfx950.
//
// One query token per sequence attends over that sequence's cached keys and
// values, which live in fixed-size physical blocks reached through the
// sequence's block table ("PagedAttention Explained: Virtual Memory for the KV
// Cache", section "How PagedAttention works", steps 2, 3 and 5).  The result is
// standard scaled-dot-product softmax attention per query head; query head h
// reads kv head h / G (grouped-query attention, "Trade-offs and related
// techniques").
//
// Work decomposition
//   tile      16 consecutive token positions of one sequence (a block of 16
//             is one tile, a block of 32 two).
//   group     GS consecutive sequences whose query heads share one wave's 16
//             matrix columns: GS = 16 / G for bf16 caches (column c is head
//             c % G of member c / G), GS = 1 for f32 caches.
//   shared    the leading blocks every member of a group holds (same physical
//             block, "Sharing blocks between sequences"): member 0 processes
//             them once for all members' columns; each member then processes
//             its private tiles with only its own columns live.
//   stream    every member's own tiles, member after member, cut into
//             partitions of part_tiles tiles (the last one of a member may
//             be shorter).  Partition counts per member and their prefix sums
//             form the plan, which every workgroup computes for itself in LDS
//             from the lengths and the tables.
//   run       the stream is cut into num_ranges equal runs of partitions
//             (stream-K): every workgroup gets the same amount of work,
//             whatever the mix of lengths.  A run may end or start inside a
//             member's tiles and may cover several members and groups.
//   workgroup one run for up to four kv heads, one wave per kv head.  The
//             run's table entries (one per tile) are staged in LDS once; the
//             waves then walk the run's tiles, loading the next tile's K and V
//             rows while they compute on the current one.
// A member's result is complete in one workgroup when only one run touches
// its tiles (and, past member 0, its group's shared tiles): the workgroup
// stores the normalised row.  Otherwise each touching run stores the state
// of that member's columns -- running max, sum and unnormalised output, in
// fp32 -- and a second kernel merges the states in run order (deterministic,
// no atomics).
//
// Per tile (one wave), bf16 caches:
//   logits   S = K q^T with v_mfma_f32_16x16x32_bf16: the 16 tokens are the M
//            rows (A operand, K rows as stored), the group's query columns the
//            N columns (B operand).  Products of bf16 values are exact in fp32;
//            sums are fp32.  A token is masked per column past that column's
//            member length, and every column of another member is masked on
//            a private tile.
//   softmax  running max and sum per column (online softmax in base 2, the
//            scale folded with log2 e).  Lane (r, c) holds tokens 4r..4r+3 of
//            column c, so the tile max is an in-lane max plus two row swaps.
//   P.V      O^T += V^T P^T with v_mfma_f32_16x16x16bf16_1k over eight 16-dim
//            slices.  The logits tile's lane layout is exactly the B operand
//            layout, so P never moves between lanes; it is split into two
//            bf16 terms (hi + lo) whose sum keeps 16 significant bits, and
//            both are multiplied in.  V^T comes from the V tile staged in LDS
//            (padded rows) through ds_read_b64_tr_b16 transpose reads.
// f32 caches use v_mfma_f32_16x16x4_f32 for the logits and fp32 FMAs for P.V
// (each lane owns one 16-byte chunk of the value rows of four tokens).
//
// Loads: a K or V tile is four 16-byte loads per lane, each instruction
// covering 4 whole 256-byte rows: non-temporal for a member's own tiles
// (read once per call and kv head), through the caches for shared tiles
// (other groups may read the same blocks).  bf16 K is re-laid out through a
// padded LDS tile into the operand layout.
#include <climits>
#include <utility>

#include "device_common.hpp"
#include "decode.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kTile = 16;
// Staged tile addresses: physical block * tiles per block + tile in block, or
// one of these markers.
constexpr uint32_t kBadTile = 0xffffffffu;   // table entry outside the pool
constexpr uint32_t kNoTile = 0xfffffffeu;    // partition slot past a member's tiles
// Running max of a column that has seen no token yet: finite, so that a tile
// on which a column is masked leaves its state exactly as it was.
constexpr float kStateFloor = -1.0e30f;
// Fourth word of a buffer resource for raw accesses: 32-bit data format, no
// swizzle, no stride (num_records then counts bytes).
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load: the non-temporal bit.
constexpr int kLoadNonTemporal = 2;
// Kv heads (one wave each) a decode workgroup can hold.
#ifndef PKV_DECODE_MAX_WAVES
#define PKV_DECODE_MAX_WAVES 4
#endif
constexpr int kMaxWavesPerWg = PKV_DECODE_MAX_WAVES;

template <typename T>
struct Storage;
template <>
struct Storage<float> {
  static constexpr int kPerVec = 4;    // elements per 16-byte chunk
};
template <>
struct Storage<uint16_t> {             // bf16 held as raw bits
  static constexpr int kPerVec = 8;
};

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int ceil_div(int x, int y) { return (x + y - 1) / y; }

// Logits of one 16-token tile: acc[i] in lane (r, c) is q_column(c) . K_token(4r + i).
__device__ __forceinline__ f32x4_t tile_logits(const u32x4_t (&k)[4], const u32x4_t (&q)[4],
                                               uint16_t) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k[c]),
                                                  __builtin_bit_cast(bf16x8_t, q[c]), acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ f32x4_t tile_logits(const u32x4_t (&k)[4], const u32x4_t (&q)[4],
                                               float) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[c][e]), __uint_as_float(q[c][e]),
                                                 acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int s, int block_size) {
  int L = a.seq_lens[s];
  L = min(L, a.max_seq_len);
  L = min(L, a.table_width * block_size);
  return max(L, 0);
}

// Tiles a member processes itself: member 0 of a group its whole sequence or
// the group's shared tiles, whichever reaches further; any other member the
// tiles past the shared ones.
__device__ __forceinline__ int own_tiles(int len, int member, int shared_tiles) {
  const int t = ceil_div(len, kTile);
  return member == 0 ? max(t, shared_tiles) : max(t - shared_tiles, 0);
}

// Runs of the work stream.  Runs alternate between two lengths: even runs
// hold `ce` partitions, odd runs `co` <= ce (the launch puts every run on XCD
// run % 8, and the odd XCDs move fewer bytes per second on this gather).
// Run r starts at partition ceil(r / 2) * ce + floor(r / 2) * co; runs past
// the stream are empty and all come last.
struct RunMap {
  int ce, co;
  __device__ __forceinline__ int start(int r) const { return ((r + 1) >> 1) * ce + (r >> 1) * co; }
  __device__ __forceinline__ int run_of(int u) const {
    const int pair = ce + co;
    return 2 * (u / pair) + ((u % pair) >= ce ? 1 : 0);
  }
};

// The runs whose tiles contribute to one member: the runs over its own
// partitions [own_lo, own_hi) of the stream, and, for members past the
// first, the runs over member 0's partitions that hold shared tiles
// [shared_lo, shared_lo + shared_units).  The second interval ends at or
// before the first begins, so the two overlap in at most one run.
struct Contrib {
  int q0, q1;   // runs of the shared partitions (empty when nq == 0)
  int r0, r1;   // runs of the own partitions (empty when nr == 0)
  int nq, nr, count;

  __device__ __forceinline__ Contrib(int own_lo, int own_hi, int shared_lo, int shared_units,
                                     int member, const RunMap& rm) {
    nq = 0;
    nr = 0;
    q0 = q1 = r0 = r1 = 0;
    if (member != 0 && shared_units > 0) {
      q0 = rm.run_of(shared_lo);
      q1 = rm.run_of(shared_lo + shared_units - 1);
      nq = q1 - q0 + 1;
    }
    if (own_hi > own_lo) {
      r0 = rm.run_of(own_lo);
      r1 = rm.run_of(own_hi - 1);
      nr = r1 - r0 + 1;
    }
    count = nq + nr - ((nq > 0 && nr > 0 && r0 == q1) ? 1 : 0);
  }
  __device__ __forceinline__ bool has(int r) const {
    return (nq > 0 && q0 <= r && r <= q1) || (nr > 0 && r0 <= r && r <= r1);
  }
  // The idx-th contributing run, in increasing order.
  __device__ __forceinline__ int at(int idx) const {
    if (idx < nq) return q0 + idx;
    const int skip = (nq > 0 && nr > 0 && r0 == q1) ? 1 : 0;
    return r0 + (idx - nq) + skip;
  }
};

// Exclusive prefix sum of one int per thread over the workgroup; `total`
// receives the sum.  s_tmp holds one int per wave.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int t = s_tmp[w];
    if (w < wave) base += t;
    total += t;
  }
  __syncthreads();
  return base + x - v;
}

// Shared leading blocks of every group of GS consecutive sequences: the
// longest run of table entries from logical block 0 that all members hold
// (the same physical block, inside the pool, within every member's length).
// Groups of fewer than two members share nothing.  Writes s_sh[k] in tiles.
// Block 0's entries (s_e0, loaded with the lengths) settle most groups; a
// group that shares block 0 then compares 64 further blocks per round, every
// member's entries of several blocks in flight per thread.
template <int GS, int BS>
__device__ void find_shared_prefixes(const DecodeArgs& a, const int* s_len, const int* s_e0,
                                     int* s_sh, int* scr) {
  constexpr int kTilesPerBlock = BS / kTile;
  constexpr int kBatch = 256;          // candidate groups per batch
  constexpr int kSpan = 64;            // blocks compared per round and group
  constexpr int kPairs = GS >= 16 ? 2 : 32 / GS;   // (group, block) pairs per thread in flight
  const int S = a.num_seqs;
  const int ngroups = ceil_div(S, GS);
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int64_t MB = a.table_width;
  int* s_cand = scr;                   // group ids of the candidates
  int* s_mis = scr + kBatch;           // first block not shared (so far)
  int* s_nb = scr + 2 * kBatch;        // fewest blocks of a member, per group
  int* s_eq = scr + 3 * kBatch;        // every member's block 0 is member 0's
  int* s_count = scr + 4 * kBatch;
  for (int kb = 0; kb < ngroups; kb += kBatch) {
    if (tid == 0) *s_count = 0;
    const int kend = min(ngroups, kb + kBatch);
    for (int k = kb + tid; k < kend; k += nthr) {
      s_nb[k - kb] = INT_MAX;
      s_eq[k - kb] = 1;
    }
    __syncthreads();
    // One thread per sequence of the batch's groups.
    for (int s = kb * GS + tid; s < min(S, kend * GS); s += nthr) {
      const int k = s / GS;
      atomicMin(&s_nb[k - kb], ceil_div(s_len[s], BS));
      if (s % GS != 0 && s_e0[s] != s_e0[k * GS]) s_eq[k - kb] = 0;
    }
    __syncthreads();
    for (int k = kb + tid; k < kend; k += nthr) {
      const int s0 = k * GS;
      const int nm = min(GS, S - s0);
      const int nb = s_nb[k - kb];
      int shared_blocks = 0;
      if (nm >= 2 && nb >= 1) {
        const int e0 = s_e0[s0];
        const bool eq = e0 >= 0 && e0 < a.num_blocks && s_eq[k - kb] != 0;
        if (eq) {
          if (nb == 1) {
            shared_blocks = 1;
          } else {
            const int c = atomicAdd(s_count, 1);
            s_cand[c] = k;
            s_mis[c] = nb;
          }
        }
      }
      s_sh[k] = shared_blocks * kTilesPerBlock;
    }
    __syncthreads();
    const int ncand = *s_count;
    for (int j0 = 1; ncand > 0; j0 += kSpan) {
      const int npairs = ncand * kSpan;
      for (int base = 0; base < npairs; base += nthr * kPairs) {
        // Every pair's candidate first (the LDS reads issue together), then
        // every member's entry of every pair as plain loads from indices
        // clamped into the table (a pair past the round or past a member
        // reads an entry it then ignores), so that no load waits on a branch.
        int jv[kPairs], cv[kPairs], nmv[kPairs], kv[kPairs], misv[kPairs];
        const int32_t* rp[kPairs];
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
          const int t = base + u * nthr + tid;
          cv[u] = min(t / kSpan, ncand - 1);
          kv[u] = s_cand[cv[u]];
          misv[u] = s_mis[cv[u]];
        }
        // Keep the LDS reads above together: one wait for all of them.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
          const int t = base + u * nthr + tid;
          const int j = j0 + t % kSpan;
          const int s0 = kv[u] * GS;
          nmv[u] = min(GS, S - s0);
          jv[u] = ((t < npairs) & (j < misv[u])) ? j : INT_MAX;
          rp[u] = a.block_table + (int64_t)s0 * MB + min(j, (int)MB - 1);
        }
        int e[kPairs][GS];
#pragma unroll
        for (int u = 0; u < kPairs; ++u)
#pragma unroll
          for (int m = 0; m < GS; ++m) e[u][m] = rp[u][(int64_t)min(m, nmv[u] - 1) * MB];
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
          bool same = e[u][0] >= 0 && e[u][0] < a.num_blocks;
#pragma unroll
          for (int m = 1; m < GS; ++m) same = same && e[u][m] == e[u][0];
          if (jv[u] != INT_MAX && !same) atomicMin(&s_mis[cv[u]], jv[u]);
        }
      }
      __syncthreads();
      int open = 0;
      for (int c = tid; c < ncand; c += nthr) open |= s_mis[c] > j0 + kSpan;
      if (!__syncthreads_or(open)) break;
    }
    for (int c = tid; c < ncand; c += nthr) s_sh[s_cand[c]] = s_mis[c] * kTilesPerBlock;
    __syncthreads();
  }
}

// Occupancy request: waves per SIMD the register allocation must allow.  The
// launches put about two waves on each SIMD; with room for more than 128
// registers the bf16 instantiations take 131-134 and spill nothing.
#ifndef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_WAVES_PER_EU 2
#endif
template <typename T, int D, int BS, int G>
__global__ __launch_bounds__(64 * kMaxWavesPerWg)
__attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU)))
void decode_stream_kernel(DecodeArgs a) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int E = Storage<T>::kPerVec;
  constexpr int GS = kBf16 ? 16 / G : 1;
  constexpr int CW = GS * G;           // matrix columns that hold query heads
  static_assert(D / E == 16, "a token row must be sixteen 16-byte chunks");
  static_assert(BS % kTile == 0, "block_size must be a multiple of 16");
  static_assert(G >= 1 && G <= 16 && CW <= 16, "a group's query heads fit the 16 MFMA columns");
  constexpr int kTilesPerBlock = BS / kTile;
  // bf16: one V tile per wave in LDS, rows padded by 32 bytes so that the
  // transpose reads of a 16-lane group hit distinct banks.
  constexpr int kVRow = D * 2 + 32;
  constexpr int kVTileBytes = kBf16 ? kTile * kVRow : 16;
  // bf16 K tile: rows padded by 16 bytes so that the 16 rows one operand read
  // touches fall in distinct banks.
  constexpr int kKRow = D * 2 + 16;
  constexpr int kKTileBytes = kBf16 ? kTile * kKRow : 16;
  constexpr int kDimTiles = D / 16;
  static_assert(!kBf16 || kMaxWavesPerWg * kKTileBytes >= 4 * (4 * 256 + 1),
                "the prologue scratch fits the K tiles");

  // Plan of the work stream (dynamic size): clamped lengths [S], prefix of
  // partitions per member [S + 1], shared tiles per group [groups].
  extern __shared__ int s_dyn[];
  __shared__ uint32_t s_addr[kMaxRangeTiles];
  __shared__ int s_scan[kMaxWavesPerWg];
  __shared__ __attribute__((aligned(16))) char s_vtile[kMaxWavesPerWg][kVTileBytes];
  __shared__ __attribute__((aligned(16))) char s_ktile[kMaxWavesPerWg][kKTileBytes];

  const int S = a.num_seqs;
  const int ngroups = ceil_div(S, GS);
  int* s_len = s_dyn;
  int* s_wpre = s_dyn + S;
  int* s_sh = s_dyn + 2 * S + 1;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane >> 4;            // row group: logits rows 4rg..4rg+3
  const int lc = lane & 15;            // K row / matrix column / V chunk
  const int kvgroups = a.kv_heads / a.heads_per_wg;
  const int P = a.part_tiles;

  // ---- plan (every workgroup computes the same one) ----
  // Lengths, and (groups of several sequences) each table's block-0 entry,
  // in one round of loads; s_wpre holds the entries until the prefix sum.
  for (int s = tid; s < S; s += nthr) {
    s_len[s] = clamp_len(a, s, BS);
    if constexpr (GS > 1) s_wpre[s] = a.block_table[(int64_t)s * a.table_width];
  }
  __syncthreads();
  if constexpr (GS > 1)
    find_shared_prefixes<GS, BS>(a, s_len, s_wpre, s_sh, reinterpret_cast<int*>(s_ktile));
  auto shared_of = [&](int k) { return GS > 1 ? s_sh[k] : 0; };
  auto units_of = [&](int s) {
    return ceil_div(own_tiles(s_len[s], s % GS, shared_of(s / GS)), P);
  };
  {
    const int per = ceil_div(S, nthr);
    const int c0 = min(S, tid * per);
    const int c1 = min(S, c0 + per);
    int local = 0;
    for (int s = c0; s < c1; ++s) local += units_of(s);
    int total;
    int pre = block_exclusive_scan(local, s_scan, total);
    for (int s = c0; s < c1; ++s) {
      s_wpre[s] = pre;
      pre += units_of(s);
    }
    if (tid == 0) s_wpre[S] = total;
  }
  // Does any group share tiles?  (Every workgroup reaches the same answer.)
  int any_sh = 0;
  if constexpr (GS > 1)
    for (int k = tid; k < ngroups; k += nthr) any_sh |= s_sh[k] > 0 ? 1 : 0;
  const bool sharing = __syncthreads_or(any_sh) != 0;
  const int W = s_wpre[S];

  // Workgroup b runs on XCD b % 8.  With a multiple of 8 runs, run r's
  // kv-head groups are the workgroups r % 8 + 8 * (kvgroups * (r / 8) + i),
  // all on XCD r % 8, and even runs are longer (the odd XCDs gather more
  // slowly).  When groups share tiles and 2, 4 or 8 kv-head groups split a
  // run, XCD x takes kv-head group x % kvgroups of every run instead, so
  // that an XCD's L2 holds the shared blocks of fewer heads; the runs are
  // then equal.  Otherwise run r is workgroups r * kvgroups + i.
  const bool by_heads = sharing && a.num_ranges % 8 == 0 && kvgroups > 1 && 8 % kvgroups == 0;
  int r, kvg;
  if (by_heads) {
    const int x = blockIdx.x & 7;
    kvg = x % kvgroups;
    r = x / kvgroups + (8 / kvgroups) * (int)(blockIdx.x >> 3);
  } else if (a.num_ranges % 8 == 0) {
    const int j = blockIdx.x >> 3;
    r = (blockIdx.x & 7) + 8 * (j / kvgroups);
    kvg = j % kvgroups;
  } else {
    r = blockIdx.x / kvgroups;
    kvg = blockIdx.x % kvgroups;
  }
  const int g = kvg * a.heads_per_wg + wave;                       // kv head
  RunMap rm;
  if (by_heads) {
    rm.ce = rm.co = max(1, ceil_div(W, a.num_ranges));
  } else {
    // Even runs hold ce partitions, odd runs co = ceil(ce * odd_q10 / 1024):
    // (N / 2) * (ce + co) >= W covers the stream.
    const int64_t pairs_q10 = (int64_t)(a.num_ranges >> 1) * (1024 + a.odd_q10) +
                              (a.num_ranges & 1) * 1024;
    rm.ce = max(1, (int)(((int64_t)W * 1024 + pairs_q10 - 1) / pairs_q10));
    rm.co = max(1, (int)(((int64_t)rm.ce * a.odd_q10 + 1023) >> 10));
  }
  if (blockIdx.x == 0 && a.plan) {
    for (int i = tid; i <= S; i += nthr) a.plan[i] = s_wpre[i];
    for (int k = tid; k < ngroups; k += nthr) a.plan[S + 1 + k] = shared_of(k);
    if (tid == 0) {
      a.plan[S + 1 + ngroups] = rm.ce;
      a.plan[S + 2 + ngroups] = rm.co;
    }
  }
  const int ua = rm.start(r);
  if (r >= a.num_ranges || ua >= max(W, 1)) return;   // uniform over the workgroup

  // ---- this run's table entries, one per tile slot, once per workgroup ----
  const int ub = min(W, rm.start(r + 1));
  // The host sizes the grid so that a run never exceeds the staged slots;
  // the clamp only keeps LDS accesses in bounds whatever the arguments.
  const int nslots = min((ub - ua) * P, kMaxRangeTiles);
  auto member_of = [&](int u) {        // the member whose partitions hold unit u
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_wpre[mid] <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  for (int i = tid; i < nslots; i += nthr) {
    const int u = ua + i / P;
    const int s = member_of(u);
    const int m = s % GS;
    const int sh = shared_of(s / GS);
    const int ot = (u - s_wpre[s]) * P + i % P;
    uint32_t addr = kNoTile;
    if (ot < own_tiles(s_len[s], m, sh)) {
      const int st = ot + (m ? sh : 0);
      const int e = a.block_table[(int64_t)s * a.table_width + st / kTilesPerBlock];
      addr = (e >= 0 && e < a.num_blocks) ? (uint32_t)e * kTilesPerBlock + st % kTilesPerBlock
                                          : kBadTile;
    }
    s_addr[i] = addr;
  }
  __syncthreads();

  // Byte offsets.  A tile's rows start at a wave-uniform address (SGPR pair);
  // each lane adds fixed 32-bit offsets, so every load is SGPR base + VGPR
  // offset (+ immediate).
  const uint32_t row_u32 = a.row_bytes;                                  // one slot
  const uint32_t head_bytes = (uint32_t)(g * D * sizeof(T));
  // bf16: K and V both as 4 whole rows per instruction (tokens 4rg + i,
  // chunk lc).  f32: K in the operand layout (row lc, chunks rg + 4c).
  const uint32_t k_lane = kBf16 ? 4 * rg * row_u32 + head_bytes + lc * 16
                                : lc * row_u32 + head_bytes + rg * 16;
  const uint32_t v_lane0 = 4 * rg * row_u32 + head_bytes + lc * 16;     // token 4rg
  const char* kcache = reinterpret_cast<const char*>(a.k_cache);
  const char* vcache = reinterpret_cast<const char*>(a.v_cache);

  // bf16 V tile in LDS: lane (r, c) writes chunk c of tokens 4r..4r+3; the
  // transpose read of lane 16j + 4r' + q covers token 4j + r', dims 4q..4q+3
  // of each 16-dim slice (offset 32 bytes per slice).
  char* vt = s_vtile[wave];
  const int tr_lane = (4 * rg + (lc >> 2)) * kVRow + 8 * (lc & 3);
  // bf16 K tile in LDS: written like V; the operand read of lane (r, c) takes
  // row c, chunk r + 4k for k-step k.
  char* kt = s_ktile[wave];
  const int ka_lane = lc * kKRow + 16 * rg;

  float m_run = kStateFloor;  // per column, in log2 units
  float l_run = 0.f;          // per lane: this row group's share of the column's sum
  // bf16: O^T slices (lane (r, c): dims 16dt + 4r .. +3 of column c);
  // f32: O rows (lane (r, c): chunk c of every head, tokens of row group r).
  f32x4_t ot[kBf16 ? kDimTiles : 1];
  float o[kBf16 ? 1 : G][E];
  u32x4_t qv[4];
  int col_len = 0;            // length of this lane's column's member (bf16)
  int max_len = 0;            // longest member of the group (uniform)

  auto reset_state = [&] {
    m_run = kStateFloor;
    l_run = 0.f;
    if constexpr (kBf16) {
#pragma unroll
      for (int dt = 0; dt < kDimTiles; ++dt) ot[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = 0.f;
    }
  };

  // Query columns of group k as the MFMA B operand (same chunk order as K).
  auto start_group = [&](int k) {
    const int s0 = k * GS;
    const int mc = kBf16 ? lc / G : 0;       // member of this lane's column
    const int hc = kBf16 ? lc % G : min(lc, G - 1);
    const bool live = kBf16 ? s0 + mc < S : lc < G;
    const int sq = min(s0 + mc, S - 1);
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((int64_t)sq * a.q_heads + g * G + hc) * D;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qrow + (rg + 4 * c) * E);
#pragma unroll
      for (int j = 0; j < 4; ++j) qv[c][j] = live ? w[j] : 0u;
    }
    col_len = live ? s_len[sq] : 0;
    // The group's longest member: a max over the 16 columns of a row.
    int mx = col_len;
    if constexpr (kBf16) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = max(mx, __shfl_xor(mx, off, 64));
    }
    max_len = uniform_int(mx);
    reset_state();
  };

  // Loads of one tile.  Tiles every member of a group reads go through the
  // caches (`cached`); every other tile is read once per call and kv head
  // and is loaded non-temporally.  Buffer loads over the tile's 16 rows: the
  // cache policy is an immediate of the instruction, so the two flavours are
  // two instruction sequences under one uniform branch.
  auto load_tile = [&](uint32_t taddr, bool cached, u32x4_t (&kr)[4], u32x4_t (&vr)[4]) {
    // A table entry outside the pool reads tile 0 instead (in the pool); its
    // tokens are masked.
    const uint32_t t = (uint32_t)uniform_int((int)(taddr >= kNoTile ? 0u : taddr));
    const uint64_t base = (uint64_t)t * a.tile_bytes;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kcache + base), 0, a.tile_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vcache + base), 0, a.tile_bytes, kBufferWord3);
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      koff[i] = kBf16 ? v_lane0 + i * row_u32 : k_lane + 64 * i;
      voff[i] = v_lane0 + i * row_u32;
    }
    if (cached) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[i], 0, 0));
        vr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i], 0, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[i], 0, kLoadNonTemporal));
        vr[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i], 0, kLoadNonTemporal));
      }
    }
  };

  // One tile, with its K and V rows in registers as loaded.  Token
  // tok0 + 4rg + i counts for this lane's column when it is below `lim`;
  // value rows at or past `vlim` (a bound for every column: unused slots,
  // any bits) are replaced by zeros first.
  //
  // bf16: the rows are staged in LDS first, then `next` (the loads of the
  // following tile into the same registers) is issued, so one register set
  // serves both the tile in flight and the tile being computed.
  auto process = [&](int tok0, int lim, int vlim, u32x4_t (&kr)[4], u32x4_t (&vr)[4],
                     auto&& next) {
    if (tok0 + kTile > vlim) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool keep = tok0 + 4 * rg + i < vlim;
#pragma unroll
        for (int j = 0; j < 4; ++j) vr[i][j] = keep ? vr[i][j] : 0u;
      }
    }
    f32x4_t acc;
    u32x4_t vkeep[kBf16 ? 1 : 4];
    if constexpr (kBf16) {
      // K and V rows to LDS as loaded (padded rows), then the next loads.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4_t*>(kt + (4 * rg + i) * kKRow + lc * 16) = kr[i];
        *reinterpret_cast<u32x4_t*>(vt + (4 * rg + i) * kVRow + lc * 16) = vr[i];
      }
      next();
      __builtin_amdgcn_wave_barrier();
      u32x4_t ka[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) ka[c] = *reinterpret_cast<const u32x4_t*>(kt + ka_lane + 64 * c);
      acc = tile_logits(ka, qv, T{});
    } else {
      u32x4_t kc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kc[i] = kr[i];
        vkeep[i] = vr[i];
      }
      next();
      acc = tile_logits(kc, qv, T{});
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = acc[i] * a.scale_log2;
      if (tok0 + 4 * rg + i >= lim) x[i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = max_xor32(max_xor16(mx));
    // m_run is finite, so m_new is too, even for a column masked on the
    // whole tile (its weights are then 0 and alpha 1).
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    if constexpr (kBf16) {
      // Rescale this lane's column where the running max moved.
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) ot[dt] *= alpha;
      }
      // P as two bf16 terms; lane (r, c) already holds P[4r..4r+3][c], the
      // B operand layout of the 16x16x16 MFMA.
      bf16x4_t phi, plo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        phi[i] = (__bf16)p[i];
        plo[i] = (__bf16)(p[i] - (float)phi[i]);
      }
      const s16x4_t bhi = __builtin_bit_cast(s16x4_t, phi);
      const s16x4_t blo = __builtin_bit_cast(s16x4_t, plo);
#pragma unroll
      for (int dt = 0; dt < kDimTiles; ++dt) {
        const bf16x4_t av = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_t*)((__attribute__((address_space(3))) char*)vt + tr_lane + 32 * dt));
        const s16x4_t as = __builtin_bit_cast(s16x4_t, av);
        ot[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as, bhi, ot[dt], 0, 0, 0);
        ot[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as, blo, ot[dt], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      if (__any(lc < G && alpha != 1.f)) {
        static_for<G>([&](auto H) {
          const float al = read_lane(alpha, H);
#pragma unroll
          for (int e = 0; e < E; ++e) o[H][e] *= al;
        });
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        static_for<G>([&](auto H) {
          const float ph = row_bcast<H>(p[i]);
#pragma unroll
          for (int e = 0; e < E; ++e) o[H][e] = fmaf(ph, __uint_as_float(vkeep[i][e]), o[H][e]);
        });
      }
    }
  };

  const int Hq = a.q_heads;
  const int rows_per_slot = a.kv_heads * CW;

  // End of group k in this run: every member this run contributes to gets
  // either its output row (this run is its only contributor) or the state of
  // its columns in workspace slot r + k.
  auto finish_group = [&](int k) {
    const float l_tot = sum_xor32(sum_xor16(l_run));     // per column
    if constexpr (!kBf16) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = sum_xor32(sum_xor16(o[h][e]));
    }
    const int s0 = k * GS;
    const int nm = min(GS, S - s0);
    const int shared_units = ceil_div(shared_of(k), P);
    const int p0 = s_wpre[s0];
    const int64_t slot = (int64_t)r + k;
    if constexpr (kBf16) {
      // Each lane settles its own column's member (m = c / G): all members
      // of the group at once.
      const int m = lc / G;
      if (m < nm) {
        const int s = s0 + m;
        const Contrib cb(s_wpre[s], s_wpre[s + 1], p0, shared_units, m, rm);
        if (cb.has(r)) {
          if (cb.count == 1) {
            // Lane (r, c) owns dims 16dt + 4r .. +3 of column c.
            const int64_t orow = (int64_t)s * Hq + g * G + lc % G;
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            __bf16* out = reinterpret_cast<__bf16*>(a.out) + orow * D + 4 * rg;
#pragma unroll
            for (int dt = 0; dt < kDimTiles; ++dt) {
              bf16x4_t w;
#pragma unroll
              for (int i = 0; i < 4; ++i) w[i] = (__bf16)(ot[dt][i] * inv);
              *reinterpret_cast<bf16x4_t*>(out + 16 * dt) = w;
            }
          } else {
            const int64_t prow = slot * rows_per_slot + g * CW + lc;
            float* po = a.part_o + prow * D + 4 * rg;
#pragma unroll
            for (int dt = 0; dt < kDimTiles; ++dt)
              *reinterpret_cast<f32x4_t*>(po + 16 * dt) = ot[dt];
            if (rg == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * prow) = float2{m_run, l_tot};
          }
        }
      }
    } else {
      for (int m = 0; m < nm; ++m) {
        const int s = s0 + m;
        const Contrib cb(s_wpre[s], s_wpre[s + 1], p0, shared_units, m, rm);
        if (!cb.has(r)) continue;
        const bool final_row = cb.count == 1;
        // Lanes of row group h % 4 store head h (chunk lc each).
        static_for<G>([&](auto H) {
          constexpr int h = H;
          const float l_h = read_lane(l_tot, h);
          const float m_h = read_lane(m_run, h);
          if (rg == (h & 3)) {
            if (final_row) {
              const int64_t orow = (int64_t)s * Hq + g * G + h;
              const float inv = l_h > 0.f ? 1.f / l_h : 0.f;
              *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.out) + orow * D + lc * E) =
                  f32x4_t{o[h][0] * inv, o[h][1] * inv, o[h][2] * inv, o[h][3] * inv};
            } else {
              const int64_t prow = slot * rows_per_slot + g * G + h;
              *reinterpret_cast<f32x4_t*>(a.part_o + prow * D + lc * E) =
                  f32x4_t{o[h][0], o[h][1], o[h][2], o[h][3]};
              if (lc == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * prow) = float2{m_h, l_h};
            }
          }
        });
      }
    }
  };

  // ---- walk the run's tiles ----
  // Pieces: the run's tiles of one member, and for member 0 of a sharing
  // group its shared and its private tiles as two pieces.  Per piece the
  // member, its length, the column masks and the load flavour are fixed, so
  // the tile loop reads only the next tile's staged address from LDS.  The
  // load issued for the first tile of the next piece takes the current
  // piece's flavour.
  int i = 0;
  while (i < nslots && s_addr[i] == kNoTile) ++i;
  if (i < nslots) {
    int s = member_of(ua);
    int k_cur = -1;
    u32x4_t kr[4], vr[4];
    uint32_t taddr = (uint32_t)uniform_int((int)s_addr[i]);
    bool loaded = false;
    while (i < nslots) {
      const int u = ua + i / P;
      while (s_wpre[s + 1] <= u) ++s;
      s = uniform_int(s);
      const int k = s / GS;
      const int m = s % GS;
      if (k != k_cur) {
        if (k_cur >= 0) finish_group(k_cur);
        start_group(k);
        k_cur = k;
      }
      const int sh = uniform_int(shared_of(k));
      const int len = uniform_int(s_len[s]);
      const int wlo = uniform_int(s_wpre[s]);
      // slots of this member in the run, and its first tile of the sequence
      int piece_end = min(nslots, (uniform_int(s_wpre[s + 1]) - ua) * P);
      int st = (u - wlo) * P + i % P + (m ? sh : 0);
      const bool shared = GS > 1 && m == 0 && st < sh;
      int lim, vlim;
      if (shared) {
        // The shared tiles end at slot i + (sh - st) (member 0's slots have
        // no gaps before its last partition).
        piece_end = min(piece_end, i + (sh - st));
        lim = col_len;                       // every member's own length
        vlim = max_len;
      } else {
        lim = (!kBf16 || lc / G == m) ? len : 0;
        vlim = len;
      }
      if (!loaded) {
        load_tile(taddr, shared, kr, vr);
        loaded = true;
      }
      while (i < piece_end) {
        int inext = i + 1;
        if (P > 1) {
          while (inext < nslots && s_addr[inext] == kNoTile) ++inext;
          inext = uniform_int(inext);
        }
        // Loads past the run's last tile re-read it (an L2 hit) so that every
        // iteration issues the same loads.
        const uint32_t naddr = inext < nslots ? (uint32_t)uniform_int((int)s_addr[inext]) : taddr;
        const bool bad = taddr == kBadTile;
        process(st * kTile, bad ? 0 : lim, bad ? 0 : vlim, kr, vr,
                [&] { load_tile(naddr, shared, kr, vr); });
        taddr = naddr;
        i = inext;
        ++st;
      }
    }
    finish_group(k_cur);
  }

  // A single run also writes the zero rows of members nothing contributes to
  // (length 0); with several runs the merge kernel does.
  if (a.num_ranges == 1) {
    for (int s = 0; s < S; ++s) {
      const int m = s % GS;
      if (s_wpre[s + 1] > s_wpre[s] || (m != 0 && shared_of(s / GS) > 0)) continue;
      T* orow = reinterpret_cast<T*>(a.out) + ((int64_t)s * Hq + g * G) * D;
      for (int idx = lane * E; idx < G * D; idx += 64 * E)
        *reinterpret_cast<u32x4_t*>(orow + idx) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

// Merge of the run states of one member's rows: with M = max_p m_p and
// w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p over the runs that
// contribute to the member, in increasing run order.  One wave per
// (sequence, kv head), the G query heads side by side (64 / G lanes per
// head, D * G / 64 elements per lane), four waves per workgroup; four
// states' loads are in flight per step and the running max is carried
// across steps (fixed order, so the result does not depend on timing).
// Members a single run completed are left alone; members no run
// contributes to (length 0) get zero rows.
constexpr int kMergeWaves = 4;

template <typename T, int D, int G>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(DecodeArgs a) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int GS = kBf16 ? 16 / G : 1;
  constexpr int CW = GS * G;
  constexpr int LPH = 64 / G;          // lanes per query head
  constexpr int PER = D / LPH;         // elements per lane
  constexpr int U = 4;
  static_assert(PER % 2 == 0 || PER == 1, "whole pairs of elements per lane");
  const int lane = threadIdx.x & 63;
  const int S = a.num_seqs;
  const int unit = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (unit >= S * a.kv_heads) return;
  const int s = unit / a.kv_heads;
  const int g = unit - s * a.kv_heads;
  const int k = s / GS;
  const int m = s % GS;
  const int ngroups = ceil_div(S, GS);
  const int* wpre = a.plan;
  RunMap rm;
  rm.ce = a.plan[S + 1 + ngroups];
  rm.co = a.plan[S + 2 + ngroups];
  const int shared_units = ceil_div(a.plan[S + 1 + k], a.part_tiles);
  const Contrib cb(wpre[s], wpre[s + 1], wpre[k * GS], shared_units, m, rm);
  if (cb.count == 1) return;
  const int hh = lane / LPH;
  const int e0 = (lane % LPH) * PER;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float lsum = 0.f;
  const int64_t rows_per_slot = (int64_t)a.kv_heads * CW;
  const int64_t srow = (int64_t)g * CW + m * G + hh;
  float M = kStateFloor;
  for (int base = 0; base < cb.count; base += U) {
    float mv[U], lv[U], ov[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = base + u < cb.count;
      const int run = cb.at(min(base + u, cb.count - 1));
      const int64_t pr = ((int64_t)run + k) * rows_per_slot + srow;
      const float2 ml = live ? *reinterpret_cast<const float2*>(a.part_ml + 2 * pr)
                             : float2{kStateFloor, 0.f};
      mv[u] = ml.x;
      lv[u] = ml.y;
      const float* po = a.part_o + pr * D + e0;
      if constexpr (PER % 4 == 0) {
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
          const f32x4_t v = live ? *reinterpret_cast<const f32x4_t*>(po + e)
                                 : f32x4_t{0.f, 0.f, 0.f, 0.f};
          ov[u][e] = v[0];
          ov[u][e + 1] = v[1];
          ov[u][e + 2] = v[2];
          ov[u][e + 3] = v[3];
        }
      } else if constexpr (PER == 2) {
        const float2 v = live ? *reinterpret_cast<const float2*>(po) : float2{0.f, 0.f};
        ov[u][0] = v.x;
        ov[u][1] = v.y;
      } else {
        ov[u][0] = live ? po[0] : 0.f;
      }
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < U; ++u) cm = fmaxf(cm, mv[u]);
    const float sc = __builtin_amdgcn_exp2f(M - cm);
    lsum *= sc;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= sc;
    M = cm;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __builtin_amdgcn_exp2f(mv[u] - M);
      lsum = fmaf(w, lv[u], lsum);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, ov[u][e], acc[e]);
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int64_t orow = (int64_t)s * a.q_heads + g * G + hh;
  if constexpr (kBf16) {
    __bf16* out = reinterpret_cast<__bf16*>(a.out) + orow * D + e0;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = (__bf16)(acc[e] * inv);
  } else {
    float* out = reinterpret_cast<float*>(a.out) + orow * D + e0;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = acc[e] * inv;
  }
}

template <typename T, int D, int BS, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  constexpr int dtype = sizeof(T) == 2 ? 1 : 0;
  const int kvgroups = a.kv_heads / a.heads_per_wg;
  const int64_t units = (int64_t)a.num_ranges * kvgroups;
  if (units == 0 || a.num_seqs == 0) return hipSuccess;
  const int64_t lds = decode_plan_lds_bytes(dtype, G, a.num_seqs);
  auto kern = decode_stream_kernel<T, D, BS, G>;
  if (lds > 48 * 1024) {
    // Large batches plan in more LDS than a launch gets by default.
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)decode_max_plan_lds_bytes());
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)units), dim3(64 * a.heads_per_wg), (size_t)lds, stream,
                     a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_ranges == 1) return err;
  const int64_t units_m = (int64_t)a.num_seqs * a.kv_heads;
  hipLaunchKernelGGL((decode_merge_kernel<T, D, G>),
                     dim3((unsigned)((units_m + kMergeWaves - 1) / kMergeWaves)),
                     dim3(64 * kMergeWaves), 0, stream, a);
  return hipGetLastError();
}

typedef hipError_t (*Launcher)(const DecodeArgs&, hipStream_t);

template <typename T, int D, int BS>
Launcher pick_group(int group) {
  switch (group) {
    case 1: return launch_typed<T, D, BS, 1>;
    case 2: return launch_typed<T, D, BS, 2>;
    case 4: return launch_typed<T, D, BS, 4>;
    case 8: return launch_typed<T, D, BS, 8>;
    default: return nullptr;
  }
}

Launcher pick(int dtype, int head_dim, int block_size, int group) {
  if (dtype == 1 && head_dim == 128) {
    if (block_size == 16) return pick_group<uint16_t, 128, 16>(group);
    if (block_size == 32) return pick_group<uint16_t, 128, 32>(group);
  }
  if (dtype == 0 && head_dim == 64) {
    if (block_size == 16) return pick_group<float, 64, 16>(group);
    if (block_size == 32) return pick_group<float, 64, 32>(group);
  }
  return nullptr;
}

}  // namespace

int64_t decode_plan_lds_bytes(int dtype, int group, int64_t num_seqs) {
  const int gs = decode_group_size(dtype, group);
  const int64_t groups = gs > 1 ? (num_seqs + gs - 1) / gs : 0;
  return (2 * num_seqs + 1 + groups) * 4;
}

// Static LDS of a decode workgroup is under 40 KB; the plan may use the rest
// of the 160 KB a gfx950 workgroup can hold, less a margin.
int64_t decode_max_plan_lds_bytes() { return 112 * 1024; }

bool decode_supported(int dtype, int head_dim, int block_size, int group) {
  return pick(dtype, head_dim, block_size, group) != nullptr;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
                         hipStream_t stream) {
  Launcher f = pick(dtype, head_dim, block_size, group);
  if (!f) return hipErrorInvalidValue;
  if (a.heads_per_wg > kMaxWavesPerWg) return hipErrorInvalidValue;
  return f(a, stream);
}

}  // namespace pkv
