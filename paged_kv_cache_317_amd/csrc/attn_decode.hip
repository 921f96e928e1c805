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
//   unit      = (sequence, partition, group of kv heads) -> one workgroup
//   wave      = one kv head of the unit and its G query heads
//   tile      = 16 consecutive token positions (a block of 16 is one tile,
//               a block of 32 two)
// A workgroup stages its partition's slice of the block table in LDS once;
// each wave then walks the tiles, loading the next tile's K and V rows while
// it computes on the current one.
//
// Per tile (one wave), bf16 caches:
//   logits   S = K q^T with v_mfma_f32_16x16x32_bf16: the 16 tokens are the M
//            rows (A operand, K rows as stored), the group's query heads the
//            N columns (B operand; columns >= G hold zero).  Products of bf16
//            values are exact in fp32; sums are fp32.
//   softmax  running max and sum per head (online softmax in base 2, the
//            scale folded with log2 e).  Lane (r, c) holds tokens 4r..4r+3 of
//            head c, so the tile max is an in-lane max plus two row swaps.
//   P.V      O^T += V^T P^T with v_mfma_f32_16x16x16bf16_1k over eight 16-dim
//            slices.  The logits tile's lane layout is exactly the B operand
//            layout, so P never moves between lanes; it is split into two
//            bf16 terms (hi + lo) whose sum keeps 16 significant bits, and
//            both are multiplied in.  V^T comes from the V tile staged in LDS
//            (padded rows) through ds_read_b64_tr_b16 transpose reads.
//            The accumulators are 8 x 4 fp32 per lane for any G <= 16.
// f32 caches use v_mfma_f32_16x16x4_f32 for the logits and fp32 FMAs for P.V
// (each lane owns one 16-byte chunk of the value rows of four tokens).
//
// Loads: a K or V tile is four 16-byte non-temporal loads per lane, each
// instruction covering 4 whole 256-byte rows.  (Loading K directly in the
// MFMA operand layout would touch 16 rows x 64 bytes per instruction, which
// measured about 13% slower on the same gather.)  bf16 K is then re-laid
// out through a padded LDS tile into the operand layout.  Every cached byte
// a sequence needs is read from HBM exactly once per call.
//
// Split-K (long contexts): with more than one partition per sequence each
// wave emits its partition's state per head -- running max and sum in fp32,
// the output normalised by the sum and rounded to bf16 for bf16 caches
// (unnormalised fp32 for f32 caches) -- into the workspace, ordered
// [sequence, partition, head] so that a wave's heads are adjacent and leave
// through its LDS tile in whole runs (device-scope stores).  A second kernel merges the
// partitions with the log-sum-exp rule in a fixed order (deterministic, no
// atomics).  A workgroup may walk several consecutive partitions (a build
// option), emitting each one's state at its last tile.
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
// Fourth word of a buffer resource for raw accesses: 32-bit data format, no
// swizzle, no stride (num_records then counts bytes).
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer store: the sc1 bit (device scope).
constexpr int kStoreDeviceScope = 16;
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

// Logits of one 16-token tile: acc[i] in lane (r, c) is q_head(c) . K_token(4r + i).
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

// Occupancy request: waves per SIMD the register allocation must allow.
#ifndef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_WAVES_PER_EU 4
#endif
template <typename T, int D, int BS, int G>
__global__ __launch_bounds__(64 * kMaxWavesPerWg)
__attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU)))
void decode_partition_kernel(DecodeArgs a) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int E = Storage<T>::kPerVec;
  static_assert(D / E == 16, "a token row must be sixteen 16-byte chunks");
  static_assert(BS % kTile == 0, "block_size must be a multiple of 16");
  static_assert(G >= 1 && G <= 16, "query heads per kv head must fit the 16 MFMA columns");
  constexpr int kTilesPerBlock = BS / kTile;
  // bf16: one V tile per wave in LDS, rows padded by 32 bytes so that the
  // transpose reads of a 16-lane group hit distinct banks.
  constexpr int kVRow = D * 2 + 32;
  constexpr int kVTileBytes = kBf16 ? kTile * kVRow : 16;
  // Staging rows of the split states in the V tile: D bf16 + 16 bytes of padding.
  constexpr int kStageRowBytes = 2 * D + 16;
  static_assert(!kBf16 || G * kStageRowBytes <= kVTileBytes, "split staging fits the V tile");
  // bf16 K tile: rows padded by 16 bytes so that the 16 rows one operand read
  // touches fall in distinct banks.
  constexpr int kKRow = D * 2 + 16;
  constexpr int kKTileBytes = kBf16 ? kTile * kKRow : 16;
  constexpr int kDimTiles = D / 16;

  __shared__ int32_t s_table[kMaxPartBlocks];
  __shared__ int s_first_bad;
  __shared__ __attribute__((aligned(16))) char s_vtile[kMaxWavesPerWg][kVTileBytes];
  __shared__ __attribute__((aligned(16))) char s_ktile[kMaxWavesPerWg][kKTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = lane >> 4;            // row group: logits rows 4rg..4rg+3
  const int lc = lane & 15;            // K row / query head column / V chunk
  const int groups = a.kv_heads / a.heads_per_wg;
  int unit = blockIdx.x;
  const int grp = unit % groups;
  unit /= groups;
  const int chunk = unit % a.num_chunks;           // parts_per_unit consecutive partitions
  const int s = unit / a.num_chunks;
  const int g = grp * a.heads_per_wg + wave;

  const int L = clamp_len(a, s, BS);
  const int span = a.part_tokens * a.parts_per_unit;
  const int t0 = chunk * span;
  if (a.num_parts > 1 && t0 >= L) return;          // uniform over the workgroup
  int t1 = min(L, t0 + span);
  const int nblk = max(t1 - t0, 0) / BS + ((max(t1 - t0, 0) % BS) != 0);
  const int j0 = t0 / BS;

  // The partition's slice of the block table, once per workgroup.  A table
  // entry outside the pool ends the sequence at that block: the partition is
  // cut back to the first such entry.
  if (threadIdx.x == 0) s_first_bad = nblk;
  __syncthreads();
  for (int j = threadIdx.x; j < nblk; j += blockDim.x) {
    const int b = a.block_table[(int64_t)s * a.table_width + j0 + j];
    s_table[j] = b;
    if (b < 0 || b >= a.num_blocks) atomicMin(&s_first_bad, j);
  }
  __syncthreads();
  t1 = min(t1, t0 + s_first_bad * BS);
  const int ntok = max(t1 - t0, 0);

  // Query heads hq0 .. hq0+G-1 as the MFMA B operand (same chunk order as K).
  const int hq0 = g * G;
  u32x4_t qv[4];
  {
    // Columns >= G read head G-1 and are then zeroed (no branch around loads).
    const int hc = min(lc, G - 1);
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((int64_t)s * a.q_heads + hq0 + hc) * D;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qrow + (rg + 4 * c) * E);
#pragma unroll
      for (int j = 0; j < 4; ++j) qv[c][j] = lc < G ? w[j] : 0u;
    }
  }

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

  float m_run = -INFINITY;   // per column (head), in log2 units
  float l_run = 0.f;         // per lane: this row group's share of the sum
  // bf16: O^T slices (lane (r, c): dims 16dt + 4r .. +3 of head c);
  // f32: O rows (lane (r, c): chunk c of every head, tokens of row group r).
  f32x4_t ot[kBf16 ? kDimTiles : 1];
  float o[kBf16 ? 1 : G][E];
  if constexpr (kBf16) {
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) ot[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) o[h][e] = 0.f;
  }

  auto load_tile = [&](int tile, u32x4_t (&kr)[4], u32x4_t (&vr)[4]) {
    const uint32_t phys = (uint32_t)uniform_int(s_table[tile / kTilesPerBlock]);
    const uint64_t base = (uint64_t)phys * a.block_bytes +
                          (uint32_t)((tile % kTilesPerBlock) * a.tile_bytes);
    const char* kp = kcache + base;
    const char* vp = vcache + base;
    // The offsets are re-materialised here so that each load is selected as
    // SGPR base + 32-bit VGPR offset rather than a 64-bit VGPR address.
    auto ld = [](const char* p) {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    };
    if constexpr (kBf16) {
      uint32_t v0 = v_lane0, v1 = v_lane0 + row_u32, v2 = v_lane0 + 2 * row_u32,
               v3 = v_lane0 + 3 * row_u32;
      asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
      kr[0] = ld(kp + v0);
      kr[1] = ld(kp + v1);
      kr[2] = ld(kp + v2);
      kr[3] = ld(kp + v3);
      vr[0] = ld(vp + v0);
      vr[1] = ld(vp + v1);
      vr[2] = ld(vp + v2);
      vr[3] = ld(vp + v3);
    } else {
      uint32_t kl = k_lane, v0 = v_lane0, v1 = v_lane0 + row_u32, v2 = v_lane0 + 2 * row_u32,
               v3 = v_lane0 + 3 * row_u32;
      asm volatile("" : "+v"(kl), "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
#pragma unroll
      for (int c = 0; c < 4; ++c) kr[c] = ld(kp + kl + c * 64);
      vr[0] = ld(vp + v0);
      vr[1] = ld(vp + v1);
      vr[2] = ld(vp + v2);
      vr[3] = ld(vp + v3);
    }
  };

  // One tile, with its K and V rows in registers as loaded.  `tb` is the
  // tile's first position; tokens at or past t1 get weight 0 (only the last
  // tile of a partition can hold such tokens, `ragged`), and their value rows
  // (unused slots, any bits) are replaced by zeros.
  //
  // bf16: the rows are staged in LDS first, then `next` (the loads of the
  // following tile into the same registers) is issued, so one register set
  // serves both the tile in flight and the tile being computed.
  auto process = [&](int tb, bool ragged, u32x4_t (&kr)[4], u32x4_t (&vr)[4], auto&& next) {
    if (ragged) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool keep = tb + 4 * rg + i < t1;
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
      if (tb + 4 * rg + i >= t1) x[i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = max_xor32(max_xor16(mx));
    // Every tile holds at least one unmasked token, so m_new is finite.
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    if constexpr (kBf16) {
      // Rescale this lane's head column where the running max moved.
      if (__any(lc < G && alpha != 1.f)) {
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

  // Split calls: this wave's unnormalised state (running max in log2 units,
  // sum, o) of partition p goes to the workspace, and the state restarts.
  auto emit_partial = [&](int p) {
    const float l_tot = sum_xor32(sum_xor16(l_run));
    // Partition p's states of this wave's G heads are adjacent in the
    // workspace ([S, P, Hq, ...] order): G * D floats of o, G (m, l) pairs.
    const int64_t row0 = ((int64_t)s * a.num_parts + p) * a.q_heads + hq0;
    if constexpr (kBf16) {
      // bf16 caches: the partition's output is stored normalised (o / l) in
      // bf16, next to its max and sum in fp32.  It goes through this wave's
      // V tile (free between tiles) so that the workspace is written in
      // whole runs, 16 bytes per lane.
      char* st = vt;
      if (lc < G) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) {
          bf16x4_t w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (__bf16)(ot[dt][i] * inv);
          *reinterpret_cast<bf16x4_t*>(st + lc * kStageRowBytes + 2 * (16 * dt + 4 * rg)) = w;
        }
        if (rg == 0)
          *reinterpret_cast<float2*>(a.part_ml + 2 * (row0 + lc)) = float2{m_run, l_tot};
      }
      __builtin_amdgcn_wave_barrier();
      // Buffer stores with device scope (the sc1 cache-policy bit): of the
      // store policies measured on the long-context split (regular,
      // non-temporal, sc0, sc1, both scopes, with and without nt) this one
      // disturbed the read stream least.
      __bf16* po = reinterpret_cast<__bf16*>(a.part_o) + row0 * D;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(po, 0, G * D * 2, kBufferWord3);
#pragma unroll
      for (int idx = 8 * lane; idx < G * D; idx += 8 * kWave)
        __builtin_amdgcn_raw_buffer_store_b128(
            *reinterpret_cast<const u32x4_t*>(st + (idx / D) * kStageRowBytes + 2 * (idx % D)),
            rs, idx * 2, 0, kStoreDeviceScope);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int dt = 0; dt < kDimTiles; ++dt) ot[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
      static_for<G>([&](auto H) {
        constexpr int h = H;
        const float l_h = read_lane(l_tot, h);
        const float m_h = read_lane(m_run, h);
        float oh[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          oh[e] = sum_xor32(sum_xor16(o[h][e]));
          o[h][e] = 0.f;
        }
        if (rg == (h & 3)) {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.part_o) + (row0 + h) * D + lc * E) =
              f32x4_t{oh[0], oh[1], oh[2], oh[3]};
          if (lc == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * (row0 + h)) = float2{m_h, l_h};
        }
      });
    }
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // One register set, refilled as soon as its tile is staged: while tile t
  // is computed, tile t+1 is in flight.  Loads past the last tile re-read it
  // (an L2 hit) so that every iteration issues the same loads.  A split
  // wave may walk several consecutive partitions: the loads run straight
  // through, and the state is emitted at every partition boundary.
  const bool split = a.num_parts > 1;
  const int p_first = chunk * a.parts_per_unit;
  int p_next = p_first;                            // first partition not emitted yet
  const int ntiles = (ntok + kTile - 1) / kTile;
  const int nfull = ntok / kTile;
  if (ntiles > 0) {
    const int last = ntiles - 1;
    u32x4_t kr[4], vr[4];
    load_tile(0, kr, vr);
    for (int t = 0; t < ntiles; ++t) {
      process(t0 + t * kTile, t == nfull, kr, vr, [&] { load_tile(min(t + 1, last), kr, vr); });
      const int tend = t0 + (t + 1) * kTile;
      if (split && (t == last || tend % a.part_tokens == 0)) {
        const int p = (tend - 1) / a.part_tokens;
        emit_partial(p);
        p_next = p + 1;
      }
    }
  }

  if (split) {
    // Partitions of this wave's span that hold no readable token (past a
    // table entry outside the pool) carry an empty state.
    const int p_end = min(p_first + a.parts_per_unit, (L + a.part_tokens - 1) / a.part_tokens);
    for (int p = p_next; p < p_end; ++p) emit_partial(p);
    return;
  }

  // Unsplit: sum the four row groups' shares of the softmax denominator and
  // store the normalised rows.
  const float l_tot = sum_xor32(sum_xor16(l_run));
  if constexpr (kBf16) {
    // Lane (r, c) owns dims 16dt + 4r .. +3 of head c.
    if (lc < G) {
      const int64_t orow = (int64_t)s * a.q_heads + hq0 + lc;
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      __bf16* out = reinterpret_cast<__bf16*>(a.out) + orow * D + 4 * rg;
#pragma unroll
      for (int dt = 0; dt < kDimTiles; ++dt) {
        bf16x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(ot[dt][i] * inv);
        *reinterpret_cast<bf16x4_t*>(out + 16 * dt) = w;
      }
    }
  } else {
    // Sum the row groups' partial outputs; lanes of row group h % 4 store head h.
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) o[h][e] = sum_xor32(sum_xor16(o[h][e]));
    static_for<G>([&](auto H) {
      constexpr int h = H;
      const float l_h = read_lane(l_tot, h);
      if (rg == (h & 3)) {
        const int64_t orow = (int64_t)s * a.q_heads + hq0 + h;
        const float inv = l_h > 0.f ? 1.f / l_h : 0.f;
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.out) + orow * D + lc * E) =
            f32x4_t{o[h][0] * inv, o[h][1] * inv, o[h][2] * inv, o[h][3] * inv};
      }
    });
  }
}

// Merge of the partition states of one (sequence, query head) row:
// M = max_p m_p, w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p.
// Four waves share a row: wave w takes partitions w, w + 4, ... (four of
// them in flight per step), lane i owns D / 64 output elements; the four
// partial sums are added in a fixed order through LDS, so the result does
// not depend on timing.
constexpr int kMergeWaves = 4;

template <typename T, int D, int BS>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  constexpr int kUnroll = 4;
  __shared__ float s_max[kMergeWaves];
  __shared__ float s_acc[kMergeWaves][D + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int orow = blockIdx.x;
  const int s = orow / a.q_heads;
  const int L = clamp_len(a, s, BS);
  const int P = (L + a.part_tokens - 1) / a.part_tokens;
  // Partition p of row (s, h) sits at workspace row (s * num_parts + p) * q_heads + h.
  const int h = orow - s * a.q_heads;
  const int64_t stride = a.q_heads;                 // rows between partitions
  const float* ml = a.part_ml + ((int64_t)s * a.num_parts * a.q_heads + h) * 2;
  // bf16 caches keep o / l in bf16 (the weight of partition p is then
  // w_p * l_p); f32 caches keep o unnormalised in fp32.
  constexpr bool kBf16 = sizeof(T) == 2;
  const int64_t o_off = ((int64_t)s * a.num_parts * a.q_heads + h) * D + lane * PER;
  const float* po32 = reinterpret_cast<const float*>(a.part_o) + o_off;
  const uint16_t* po16 = reinterpret_cast<const uint16_t*>(a.part_o) + o_off;

  float M = -INFINITY;
  for (int p = threadIdx.x; p < P; p += 64 * kMergeWaves) M = fmaxf(M, ml[2 * p * stride]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) s_max[wave] = M;
  __syncthreads();
  M = s_max[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, s_max[w]);

  float lsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int p0 = wave; p0 < P; p0 += kMergeWaves * kUnroll) {
    float mv[kUnroll], lv[kUnroll], ov[kUnroll][PER];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = min(p0 + u * kMergeWaves, P - 1);
      mv[u] = ml[2 * p * stride];
      lv[u] = ml[2 * p * stride + 1];
#pragma unroll
      for (int e = 0; e < PER; ++e)
        ov[u][e] = kBf16 ? __uint_as_float((uint32_t)po16[(int64_t)p * stride * D + e] << 16)
                         : po32[(int64_t)p * stride * D + e];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // A partition with no tokens (m = -inf), or past the row's last one,
      // carries no weight.
      const bool live = p0 + u * kMergeWaves < P && mv[u] != -INFINITY;
      const float w = live ? __builtin_amdgcn_exp2f(mv[u] - M) : 0.f;
      const float wl = w * lv[u];
      lsum += wl;
      const float wo = kBf16 ? wl : w;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wo, ov[u][e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) s_acc[wave][lane * PER + e] = acc[e];
  if (lane == 0) s_acc[wave][D] = lsum;
  __syncthreads();
  if (wave != 0) return;
  float tot[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) tot[e] = s_acc[0][lane * PER + e];
  float ltot = s_acc[0][D];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) {
#pragma unroll
    for (int e = 0; e < PER; ++e) tot[e] += s_acc[w][lane * PER + e];
    ltot += s_acc[w][D];
  }
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if constexpr (sizeof(T) == 2) {
    static_assert(PER == 2, "bf16 merge writes two elements per lane");
    __bf16* out = reinterpret_cast<__bf16*>(a.out) + (int64_t)orow * D + lane * PER;
    out[0] = (__bf16)(tot[0] * inv);
    out[1] = (__bf16)(tot[1] * inv);
  } else {
    float* out = reinterpret_cast<float*>(a.out) + (int64_t)orow * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = tot[e] * inv;
  }
}

// Merge for calls with few partitions per sequence (at most NP): one wave
// per (sequence, query head) row, four rows per workgroup.  Each lane loads
// the row's (m, l) of every partition and its own D / 64 output elements of
// each, all before any arithmetic, so the merge costs one round trip to
// memory; the max and the weighted sums then run in registers in partition
// order (fixed, so the result does not depend on timing).  Slots past the
// row's last partition re-read that partition (written by the partition
// kernel, so finite) and carry no weight.
template <typename T, int D, int BS, int NP>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_few_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  constexpr bool kBf16 = sizeof(T) == 2;
  const int lane = threadIdx.x & 63;
  const int orow = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (orow >= a.num_seqs * a.q_heads) return;
  const int s = orow / a.q_heads;
  const int h = orow - s * a.q_heads;
  const int L = clamp_len(a, s, BS);
  const int P = (L + a.part_tokens - 1) / a.part_tokens;
  const int64_t stride = a.q_heads;
  const int64_t row0 = (int64_t)s * a.num_parts * a.q_heads + h;
  const float* ml = a.part_ml + row0 * 2;
  const int64_t o_off = row0 * D + lane * PER;
  const float* po32 = reinterpret_cast<const float*>(a.part_o) + o_off;
  const uint16_t* po16 = reinterpret_cast<const uint16_t*>(a.part_o) + o_off;

  if (P == 0) {                       // empty sequence: zero row, nothing to read
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if constexpr (kBf16)
        reinterpret_cast<__bf16*>(a.out)[(int64_t)orow * D + lane * PER + e] = (__bf16)0.f;
      else
        reinterpret_cast<float*>(a.out)[(int64_t)orow * D + lane * PER + e] = 0.f;
    }
    return;
  }
  float mv[NP], lv[NP], ov[NP][PER];
  const int plast = P - 1;
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int p = min(u, plast);
    mv[u] = ml[2 * p * stride];
    lv[u] = ml[2 * p * stride + 1];
#pragma unroll
    for (int e = 0; e < PER; ++e)
      ov[u][e] = kBf16 ? __uint_as_float((uint32_t)po16[(int64_t)p * stride * D + e] << 16)
                       : po32[(int64_t)p * stride * D + e];
  }
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < NP; ++u) M = u < P ? fmaxf(M, mv[u]) : M;
  float lsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    // A partition with no tokens (m = -inf), or past the row's last one,
    // carries no weight.
    const bool live = u < P && mv[u] != -INFINITY;
    const float w = live ? __builtin_amdgcn_exp2f(mv[u] - M) : 0.f;
    const float wl = w * lv[u];
    lsum += wl;
    const float wo = kBf16 ? wl : w;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(wo, ov[u][e], acc[e]);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if constexpr (kBf16) {
    static_assert(PER == 2, "bf16 merge writes two elements per lane");
    __bf16* out = reinterpret_cast<__bf16*>(a.out) + (int64_t)orow * D + lane * PER;
    out[0] = (__bf16)(acc[0] * inv);
    out[1] = (__bf16)(acc[1] * inv);
  } else {
    float* out = reinterpret_cast<float*>(a.out) + (int64_t)orow * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = acc[e] * inv;
  }
}

template <typename T, int D, int BS, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const int groups = a.kv_heads / a.heads_per_wg;
  const int64_t units = (int64_t)a.num_seqs * a.num_chunks * groups;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_partition_kernel<T, D, BS, G>), dim3((unsigned)units),
                     dim3(64 * a.heads_per_wg), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_parts == 1) return err;
  const int64_t rows = (int64_t)a.num_seqs * a.q_heads;
  const dim3 few_grid((unsigned)((rows + kMergeWaves - 1) / kMergeWaves));
  const dim3 threads(64 * kMergeWaves);
  if (a.num_parts <= 2)
    hipLaunchKernelGGL((decode_merge_few_kernel<T, D, BS, 2>), few_grid, threads, 0, stream, a);
  else if (a.num_parts <= 4)
    hipLaunchKernelGGL((decode_merge_few_kernel<T, D, BS, 4>), few_grid, threads, 0, stream, a);
  else if (a.num_parts <= 8)
    hipLaunchKernelGGL((decode_merge_few_kernel<T, D, BS, 8>), few_grid, threads, 0, stream, a);
  else if (a.num_parts <= 16)
    hipLaunchKernelGGL((decode_merge_few_kernel<T, D, BS, 16>), few_grid, threads, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<T, D, BS>), dim3((unsigned)rows), threads, 0, stream,
                       a);
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
