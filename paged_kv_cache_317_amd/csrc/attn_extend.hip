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
//   workgroup 128 columns (128 / G tokens) of one sequence and kv head;
//             four waves of 32 columns (two 16-column MFMA groups each)
//   tile      64 consecutive key positions, staged in LDS once per
//             workgroup and read by all four waves
// Workgroups are ordered so that the query tiles of one (sequence, kv head)
// land on one XCD (workgroup b runs on XCD b mod 8) and share its L2.
//
// Per tile and wave (bf16, head_dim 128):
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16; keys are the M rows (A operand,
//                 read from the padded K tile in LDS), the 16 columns of a
//                 group the N columns (B operand, held in registers for the
//                 whole call).  Lane (r, c) gets keys 4r..4r+3 of column c
//                 for each 16-key block.
//   softmax       online, base 2, scale folded with log2 e; the tile max of
//                 a column is an in-lane max plus two row swaps; the causal
//                 and length mask is applied only on tiles that need it.
//   O^T += V^T P^T  v_mfma_f32_16x16x32_bf16 with the 32 keys of two 16-key
//                 blocks as the K dimension in the order that matches the
//                 logits' lane layout: P stays in its lanes (rounded to
//                 bf16), V^T comes from the padded V tile through
//                 ds_read_b64_tr_b16 transpose reads, shared by both groups.
// Loads: the next tile's K and V rows (16 bytes per lane, 16 lanes per
// 256-byte row) are issued before the current tile is computed and written
// to the other LDS buffer after it; one barrier per tile.
#include "device_common.hpp"
#include "extend.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kD = 128;                  // head_dim
constexpr int kKeys = 64;                // key positions per tile
constexpr int kThreads = 256;
constexpr int kGroups = 2;               // 16-column groups per wave
constexpr int kKRow = kD * 2 + 16;       // padded LDS row of the K tile (bytes)
constexpr int kVRow = kD * 2 + 32;       // padded LDS row of the V tile (bytes)
constexpr int kKTile = kKeys * kKRow;
constexpr int kVTile = kKeys * kVRow;
static_assert(kExtendCols == 4 * 16 * kGroups, "four waves of kGroups 16-column groups");

__device__ __forceinline__ bf16x8_t cat(bf16x4_t lo, bf16x4_t hi) {
  return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ bf16x4_t tr_read(const char* lds, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4_t*)((__attribute__((address_space(3))) char*)lds + byte_off));
}

template <int BS, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void extend_kernel(ExtendArgs a) {
  static_assert(BS == 16 || BS == 32, "block_size 16 or 32");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "G in {1, 2, 4, 8}");
  constexpr int kTokens = kExtendCols / G;       // query tokens per workgroup
  constexpr int kEntries = kKeys / BS;           // table entries per tile
  constexpr int kRowsPerThread = kKeys * 16 / kThreads;   // 16-byte chunks per thread per tile
  static_assert(kRowsPerThread == 4, "four rows per thread per tile");

  __shared__ __attribute__((aligned(16))) char s_k[2][kKTile];
  __shared__ __attribute__((aligned(16))) char s_v[2][kVTile];
  __shared__ int s_first_bad;

  const int per_xcd = (a.units + 7) / 8;
  const int unit = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (unit >= a.units) return;
  const int qt = a.q_tiles - 1 - unit % a.q_tiles;   // later (longer) query tiles first
  const int rest = unit / a.q_tiles;
  const int g = rest % a.kv_heads;
  const int s = rest / a.kv_heads;

  const int q0 = a.query_start[s];
  const int n_raw = a.query_start[s + 1] - q0;
  // Rows outside [0, num_tokens) are never read or written, whatever
  // query_start holds.
  if (q0 < 0) return;
  const int n = min(min(n_raw, a.max_query_len), a.num_tokens - q0);
  const int j0 = qt * kTokens;
  if (j0 >= n) return;
  const int j1 = min(j0 + kTokens, n);
  const int L = a.seq_lens[s];
  const int ctx = L - n_raw;                       // position of query 0

  // Keys this workgroup may read: below every query's position + 1 and the
  // sequence length; a table entry outside the pool ends the sequence at
  // that block.
  int kv_end = max(min(L, a.table_width * BS), 0);
  int kv_hi = max(min(ctx + j1, kv_end), 0);
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
  const int ntiles = (kv_hi + kKeys - 1) / kKeys;
  const int last_blk = max((kv_hi - 1) / BS, 0);

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
    const int col = 32 * wave + 16 * cg + lc;
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
  const bool wave_active = j0 + (32 * wave) / G < j1;
  const int qmin_w = ctx + min(j0 + (32 * wave) / G, j1 - 1);
  const int qmax_w = ctx + min(j0 + (32 * wave + 31) / G, j1 - 1);

  // Tile loader: thread t moves chunk t % 16 of rows t / 16 + 16 i.
  const int lchunk = threadIdx.x & 15;
  const int lrow = threadIdx.x >> 4;
  const uint32_t lane_off = (uint32_t)(g * kD * 2 + 16 * lchunk);
  const char* kcache = reinterpret_cast<const char*>(a.k_cache);
  const char* vcache = reinterpret_cast<const char*>(a.v_cache);

  // Table entries of a tile (vector loads, so that waiting for them never
  // holds up the LDS traffic of the tile being computed).
  auto fetch_entries = [&](int tile, int (&e)[kEntries]) {
#pragma unroll
    for (int k = 0; k < kEntries; ++k) e[k] = trow[min(tile * kEntries + k, last_blk)];
  };
  auto load_tile = [&](const int (&e)[kEntries], u32x4_t (&kr)[4], u32x4_t (&vr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t phys = (uint32_t)uniform_int(e[(16 * i) / BS]);
      const uint64_t base = (uint64_t)phys * a.block_bytes;
      uint32_t off = (uint32_t)((lrow + (16 * i) % BS) * a.row_bytes) + lane_off;
      asm volatile("" : "+v"(off));
      kr[i] = *reinterpret_cast<const u32x4_t*>(kcache + base + off);
      vr[i] = *reinterpret_cast<const u32x4_t*>(vcache + base + off);
    }
  };
  // Rows at or past kv_hi (only in the last tile) are stored as zeros: they
  // may be unused slots holding any bits.
  auto store_tile = [&](int tile, int buf, u32x4_t (&kr)[4], u32x4_t (&vr)[4]) {
    const int t0 = tile * kKeys;
    if (t0 + kKeys > kv_hi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (t0 + lrow + 16 * i >= kv_hi) {
          kr[i] = u32x4_t{0u, 0u, 0u, 0u};
          vr[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4_t*>(&s_k[buf][(lrow + 16 * i) * kKRow + 16 * lchunk]) = kr[i];
      *reinterpret_cast<u32x4_t*>(&s_v[buf][(lrow + 16 * i) * kVRow + 16 * lchunk]) = vr[i];
    }
  };

  float m_run[kGroups], l_run[kGroups];
  f32x4_t ot[kGroups][kD / 16];
#pragma unroll
  for (int cg = 0; cg < kGroups; ++cg) {
    m_run[cg] = -INFINITY;
    l_run[cg] = 0.f;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) ot[cg][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Per-lane LDS offsets of the operand reads.
  const int ka_lane = lc * kKRow + 16 * rg;                        // K row lc, chunk rg
  const int tr_lane = (4 * rg + (lc >> 2)) * kVRow + 8 * (lc & 3);  // V transpose read

  auto compute = [&](int tile, int buf) {
    const int t0 = tile * kKeys;
    if (!wave_active || t0 > qmax_w) return;
    const char* kt = s_k[buf];
    const char* vt = s_v[buf];
    f32x4_t sacc[kGroups][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4_t ka[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        ka[ks] = *reinterpret_cast<const u32x4_t*>(kt + ka_lane + 16 * kb * kKRow + 64 * ks);
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
    const bool need_mask = (t0 + kKeys - 1 > qmin_w) || (t0 + kKeys > kv_hi);
    bf16x4_t pb[kGroups][4];
#pragma unroll
    for (int cg = 0; cg < kGroups; ++cg) {
      float x[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[cg][kb][i] * a.scale_log2;
          if (need_mask) {
            const int kp = t0 + 16 * kb + 4 * rg + i;
            if (kp > qpos[cg] || kp >= kv_hi) v = -INFINITY;
          }
          x[kb][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = max_xor32(max_xor16(mx));
      const float m_new = fmaxf(m_run[cg], mx);
      // A column with nothing visible yet keeps weight 0 everywhere.
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[cg] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(x[kb][i] - m_use);
          psum += p;
          pb[cg][kb][i] = (__bf16)p;
        }
      }
      l_run[cg] = l_run[cg] * alpha + psum;
      m_run[cg] = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < kD / 16; ++db) ot[cg][db] *= alpha;
      }
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) {
        const bf16x4_t a0 = tr_read(vt, tr_lane + 32 * kp * kVRow + 32 * db);
        const bf16x4_t a1 = tr_read(vt, tr_lane + (32 * kp + 16) * kVRow + 32 * db);
        const bf16x8_t av = cat(a0, a1);
#pragma unroll
        for (int cg = 0; cg < kGroups; ++cg)
          ot[cg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av, cat(pb[cg][2 * kp], pb[cg][2 * kp + 1]), ot[cg][db], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) {
    int ent[kEntries];
    u32x4_t kr[4], vr[4];
    fetch_entries(0, ent);
    load_tile(ent, kr, vr);
    fetch_entries(1, ent);
    store_tile(0, 0, kr, vr);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      if (more) {
        load_tile(ent, kr, vr);
        fetch_entries(t + 2, ent);
      }
      compute(t, t & 1);
      if (more) store_tile(t + 1, (t + 1) & 1, kr, vr);
      __syncthreads();
    }
  }

#pragma unroll
  for (int cg = 0; cg < kGroups; ++cg) {
    const float l_tot = sum_xor32(sum_xor16(l_run[cg]));
    if (cvalid[cg]) {
      const int col = 32 * wave + 16 * cg + lc;
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

template <int BS, int G>
hipError_t launch_one(const ExtendArgs& a, hipStream_t stream) {
  const int per_xcd = (a.units + 7) / 8;
  hipLaunchKernelGGL((extend_kernel<BS, G>), dim3(8 * per_xcd), dim3(kThreads), 0, stream, a);
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
