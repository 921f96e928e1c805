// Host block manager: free list, reference counts, per-sequence block tables,
// on-demand allocation and copy-on-write ("PagedAttention Explained: Virtual
// Memory for the KV Cache", "How PagedAttention works" steps 1-4 and "Sharing
// blocks between sequences"; release on finish from "What does PagedAttention
// change in LLM KV allocation?", "Calculate unused block space").  Host memory
// only; every call checks its arguments and either completes or changes
// nothing.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "status.hpp"

namespace {

// 64-bit mixing (the splitmix64 finaliser) and the hash of one full block:
// its predecessor's hash followed by its token ids.
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
inline uint64_t block_hash(uint64_t parent, const int32_t* t, int32_t n) {
  uint64_t h = mix64(parent ^ 0x9E3779B97F4A7C15ull);
  for (int32_t i = 0; i < n; ++i) h = mix64(h + (uint32_t)t[i] + 0x9E3779B97F4A7C15ull);
  return h;
}
constexpr uint64_t kRootHash = 0x243F6A8885A308D3ull;   // predecessor of block 0

}  // namespace

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> table;   // logical block -> physical block
    int32_t len = 0;
    bool tracked = false;         // token ids known (prefix-cache registration)
    std::vector<int32_t> tokens;  // token ids, when tracked
    std::vector<uint64_t> hashes; // hash chain of the full blocks, when tracked
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> refcount;  // per physical block
  std::vector<int32_t> fill;      // token slots stored in the block
  std::deque<int32_t> free_list;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t copies = 0;
  int64_t preemptions = 0;
  // Prefix cache: hash -> block, and per registered block its hash, its
  // predecessor's hash and its token ids (to confirm hits).
  std::unordered_map<uint64_t, int32_t> cache;
  std::vector<char> registered;
  std::vector<uint64_t> reg_hash, reg_parent;
  std::vector<int32_t> reg_tokens;  // num_blocks x block_size, filled on registration
  int64_t reused = 0;
  // Swap space: host block free list and swapped-out sequences.
  struct Swapped {
    std::vector<int32_t> host;     // host block of each logical block
    int32_t len = 0;
  };
  int32_t host_blocks = 0;
  std::deque<int32_t> host_free;
  std::unordered_map<int64_t, Swapped> swapped;
  int64_t swap_outs = 0;

  void unregister(int32_t b) {
    if (!registered.empty() && registered[b]) {
      cache.erase(reg_hash[b]);
      registered[b] = 0;
    }
  }
  // Extend a tracked sequence's hash chain over its newly full blocks and
  // register each one that no entry covers yet.
  void register_full(Seq& q) {
    if (registered.empty()) {
      registered.assign(num_blocks, 0);
      reg_hash.assign(num_blocks, 0);
      reg_parent.assign(num_blocks, 0);
      reg_tokens.assign((size_t)num_blocks * block_size, 0);
    }
    const int32_t full = q.len / block_size;
    for (int32_t j = (int32_t)q.hashes.size(); j < full; ++j) {
      const int32_t* t = q.tokens.data() + (int64_t)j * block_size;
      const uint64_t parent = j > 0 ? q.hashes[j - 1] : kRootHash;
      const uint64_t h = block_hash(parent, t, block_size);
      q.hashes.push_back(h);
      const int32_t b = q.table[j];
      if (registered[b] || cache.count(h)) continue;
      cache.emplace(h, b);
      registered[b] = 1;
      reg_hash[b] = h;
      reg_parent[b] = parent;
      std::copy(t, t + block_size, reg_tokens.begin() + (size_t)b * block_size);
    }
  }
  // A registered block holding exactly these tokens after `parent`, or -1.
  int32_t lookup(uint64_t parent, const int32_t* t) const {
    const uint64_t h = block_hash(parent, t, block_size);
    auto it = cache.find(h);
    if (it == cache.end()) return -1;
    const int32_t b = it->second;
    if (reg_parent[b] != parent) return -1;
    if (!std::equal(t, t + block_size, reg_tokens.begin() + (size_t)b * block_size)) return -1;
    return b;
  }

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    refcount[b] = 1;
    fill[b] = 0;
    return b;
  }
  void drop(int32_t b) {
    if (--refcount[b] == 0) {
      fill[b] = 0;
      unregister(b);
      free_list.push_back(b);
    }
  }
  // Blocks an append of n tokens takes from the pool.
  int64_t needed(const Seq& q, int32_t n) const {
    if (n <= 0) return 0;
    const int64_t have = (q.len + (int64_t)block_size - 1) / block_size;
    const int64_t want = (q.len + (int64_t)n + block_size - 1) / block_size;
    const bool cow = q.len % block_size != 0 && refcount[q.table.back()] > 1;
    return want - have + (cow ? 1 : 0);
  }
  void release(int64_t id) {
    auto it = seqs.find(id);
    for (int32_t b : it->second.table) drop(b);
    seqs.erase(it);
  }
};

namespace {

using pkv::fail;
using pkv::ok;

pkv_status find(const pkv_block_manager* bm, int64_t seq) {
  if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
  if (!bm->seqs.count(seq)) return fail(PKV_ERR_KEY, "unknown sequence id %lld", (long long)seq);
  return PKV_OK;
}

}  // namespace

PKV_EXPORT pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                    const int32_t* free_order, pkv_block_manager** out) {
  if (!out) return fail(PKV_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1)
    return fail(PKV_ERR_SHAPE, "num_blocks and block_size must be positive");
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
  if (!bm) return fail(PKV_ERR_SHAPE, "out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  bm->fill.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return fail(PKV_ERR_SHAPE, "free_order must be a permutation of 0..num_blocks-1");
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  }
  *out = bm;
  return ok();
}

PKV_EXPORT void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

PKV_EXPORT pkv_status pkv_bm_add(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
  if (bm->seqs.count(seq) || bm->swapped.count(seq))
    return fail(PKV_ERR_KEY, "sequence id %lld exists", (long long)seq);
  bm->seqs.emplace(seq, pkv_block_manager::Seq{});
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  pkv_status st = find(bm, parent);
  if (st != PKV_OK) return st;
  if (bm->seqs.count(child) || bm->swapped.count(child))
    return fail(PKV_ERR_KEY, "sequence id %lld exists", (long long)child);
  pkv_block_manager::Seq copy = bm->seqs.at(parent);
  for (int32_t b : copy.table) ++bm->refcount[b];
  bm->seqs.emplace(child, std::move(copy));
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_blocks_needed(const pkv_block_manager* bm, int64_t seq, int32_t n,
                                           int32_t* blocks) {
  pkv_status st = find(bm, seq);
  if (st != PKV_OK) return st;
  if (!blocks) return fail(PKV_ERR_NULL, "blocks is NULL");
  if (n < 0) return fail(PKV_ERR_SHAPE, "n must be >= 0");
  *blocks = (int32_t)bm->needed(bm->seqs.at(seq), n);
  return ok();
}

namespace {

pkv_status append_impl(pkv_block_manager* bm, int64_t seq, bool with_tokens,
                       const int32_t* tokens, int32_t n, int64_t* slots, int64_t* copies,
                       int32_t copies_cap, int32_t* n_copies);

}  // namespace

PKV_EXPORT pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int32_t n, int64_t* slots,
                                    int64_t* copies, int32_t copies_cap, int32_t* n_copies) {
  return append_impl(bm, seq, false, nullptr, n, slots, copies, copies_cap, n_copies);
}

PKV_EXPORT pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, int64_t seq,
                                           const int32_t* tokens, int32_t n, int64_t* slots,
                                           int64_t* copies, int32_t copies_cap,
                                           int32_t* n_copies) {
  if (n > 0 && !tokens) return fail(PKV_ERR_NULL, "tokens is NULL");
  return append_impl(bm, seq, true, tokens, n, slots, copies, copies_cap, n_copies);
}

namespace {

pkv_status append_impl(pkv_block_manager* bm, int64_t seq, bool with_tokens,
                       const int32_t* tokens, int32_t n, int64_t* slots, int64_t* copies,
                       int32_t copies_cap, int32_t* n_copies) {
  pkv_status st = find(bm, seq);
  if (st != PKV_OK) return st;
  if (n < 0) return fail(PKV_ERR_SHAPE, "n must be >= 0");
  if ((n > 0 && !slots) || !n_copies) return fail(PKV_ERR_NULL, "slots and n_copies must be non-NULL");
  pkv_block_manager::Seq& q = bm->seqs.at(seq);
  if ((int64_t)q.len + n > INT32_MAX) return fail(PKV_ERR_SHAPE, "sequence length overflows int32");
  if (with_tokens && !q.tracked)
    return fail(PKV_ERR_SHAPE, "sequence %lld does not carry token ids", (long long)seq);
  const int64_t need = bm->needed(q, n);
  const bool cow = n > 0 && q.len % bm->block_size != 0 && bm->refcount[q.table.back()] > 1;
  if (cow && (copies_cap < 1 || !copies))
    return fail(PKV_ERR_SHAPE, "this append copies a shared block: copies needs room for 1 pair");
  if (need > (int64_t)bm->free_list.size())
    return fail(PKV_ERR_NO_BLOCKS, "append needs %lld free blocks, the pool has %zu",
                (long long)need, bm->free_list.size());
  const int32_t BS = bm->block_size;
  *n_copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t t = q.len;
    const int32_t off = t % BS;
    int32_t b;
    if (off == 0) {
      b = bm->take();
      q.table.push_back(b);
    } else {
      b = q.table.back();
      if (bm->refcount[b] > 1) {
        const int32_t nb = bm->take();
        copies[2 * *n_copies] = b;
        copies[2 * *n_copies + 1] = nb;
        ++*n_copies;
        ++bm->copies;
        bm->fill[nb] = bm->fill[b];
        --bm->refcount[b];
        q.table.back() = nb;
        b = nb;
      }
    }
    slots[i] = (int64_t)b * BS + off;
    bm->fill[b] = std::max(bm->fill[b], off + 1);
    q.len = t + 1;
  }
  if (with_tokens) {
    q.tokens.insert(q.tokens.end(), tokens, tokens + n);
    bm->register_full(q);
  } else if (n > 0) {
    q.tracked = false;
    q.tokens.clear();
    q.hashes.clear();
  }
  return ok();
}

}  // namespace

PKV_EXPORT pkv_status pkv_bm_add_cached(pkv_block_manager* bm, int64_t seq, const int32_t* tokens,
                                        int32_t n, int32_t* reused_tokens) {
  if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
  if (n < 0) return fail(PKV_ERR_SHAPE, "n must be >= 0");
  if ((n > 0 && !tokens) || !reused_tokens)
    return fail(PKV_ERR_NULL, "tokens and reused_tokens must be non-NULL");
  if (bm->seqs.count(seq) || bm->swapped.count(seq))
    return fail(PKV_ERR_KEY, "sequence id %lld exists", (long long)seq);
  pkv_block_manager::Seq q;
  q.tracked = true;
  const int32_t BS = bm->block_size;
  uint64_t parent = kRootHash;
  int32_t done = 0;
  while (!bm->cache.empty() && done + BS <= n) {
    const int32_t b = bm->lookup(parent, tokens + done);
    if (b < 0) break;
    parent = bm->reg_hash[b];
    q.table.push_back(b);
    done += BS;
  }
  for (int32_t b : q.table) {
    ++bm->refcount[b];
    q.hashes.push_back(bm->reg_hash[b]);
  }
  bm->reused += (int64_t)q.table.size();
  q.len = done;
  q.tokens.assign(tokens, tokens + done);
  bm->seqs.emplace(seq, std::move(q));
  *reused_tokens = done;
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq) {
  if (bm) {
    auto it = bm->swapped.find(seq);
    if (it != bm->swapped.end()) {      // finished while swapped out
      for (int32_t h : it->second.host) bm->host_free.push_back(h);
      bm->swapped.erase(it);
      return ok();
    }
  }
  pkv_status st = find(bm, seq);
  if (st != PKV_OK) return st;
  bm->release(seq);
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_preempt(pkv_block_manager* bm, int64_t seq) {
  pkv_status st = find(bm, seq);
  if (st != PKV_OK) return st;
  bm->release(seq);
  ++bm->preemptions;
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_set_swap_space(pkv_block_manager* bm, int32_t host_blocks) {
  if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
  if (host_blocks < 1) return fail(PKV_ERR_SHAPE, "host_blocks must be positive");
  if (bm->host_blocks) return fail(PKV_ERR_SHAPE, "swap space is already set");
  bm->host_blocks = host_blocks;
  for (int32_t b = 0; b < host_blocks; ++b) bm->host_free.push_back(b);
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq, int64_t* pairs,
                                      int32_t cap, int32_t* n) {
  pkv_status st = find(bm, seq);
  if (st != PKV_OK) return st;
  if (!n) return fail(PKV_ERR_NULL, "n is NULL");
  const auto& q = bm->seqs.at(seq);
  const int64_t need = (int64_t)q.table.size();
  if (need > 0 && (!pairs || cap < need))
    return fail(PKV_ERR_SHAPE, "pairs needs room for %lld pairs", (long long)need);
  if (need > (int64_t)bm->host_free.size())
    return fail(PKV_ERR_NO_BLOCKS, "swap-out needs %lld host blocks, %zu free", (long long)need,
                bm->host_free.size());
  pkv_block_manager::Swapped sw;
  sw.len = q.len;
  for (int64_t j = 0; j < need; ++j) {
    const int32_t h = bm->host_free.front();
    bm->host_free.pop_front();
    pairs[2 * j] = q.table[j];
    pairs[2 * j + 1] = h;
    sw.host.push_back(h);
  }
  *n = (int32_t)need;
  bm->swapped.emplace(seq, std::move(sw));
  bm->release(seq);
  ++bm->swap_outs;
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq, int64_t* pairs,
                                     int32_t cap, int32_t* n) {
  if (!bm || !n) return fail(PKV_ERR_NULL, "block manager and n must be non-NULL");
  auto it = bm->swapped.find(seq);
  if (it == bm->swapped.end())
    return fail(PKV_ERR_KEY, "sequence id %lld is not swapped out", (long long)seq);
  const auto& sw = it->second;
  const int64_t need = (int64_t)sw.host.size();
  if (need > 0 && (!pairs || cap < need))
    return fail(PKV_ERR_SHAPE, "pairs needs room for %lld pairs", (long long)need);
  if (need > (int64_t)bm->free_list.size())
    return fail(PKV_ERR_NO_BLOCKS, "swap-in needs %lld device blocks, %zu free", (long long)need,
                bm->free_list.size());
  pkv_block_manager::Seq q;
  q.len = sw.len;
  const int32_t BS = bm->block_size;
  for (int64_t j = 0; j < need; ++j) {
    const int32_t b = bm->take();
    bm->fill[b] = (int32_t)std::min<int64_t>(BS, sw.len - j * BS);
    q.table.push_back(b);
    pairs[2 * j] = sw.host[j];
    pairs[2 * j + 1] = b;
    bm->host_free.push_back(sw.host[j]);
  }
  *n = (int32_t)need;
  bm->swapped.erase(it);
  bm->seqs.emplace(seq, std::move(q));
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_length(const pkv_block_manager* bm, int64_t seq, int32_t* len) {
  pkv_status st = find(bm, seq);
  if (st != PKV_OK) return st;
  if (!len) return fail(PKV_ERR_NULL, "len is NULL");
  *len = bm->seqs.at(seq).len;
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_table(const pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                                   int32_t width, int32_t* table) {
  if (!bm) return fail(PKV_ERR_NULL, "block manager is NULL");
  if (n < 0 || width < 0) return fail(PKV_ERR_SHAPE, "n and width must be >= 0");
  if (n > 0 && (!seqs || (width > 0 && !table))) return fail(PKV_ERR_NULL, "seqs and table must be non-NULL");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PKV_ERR_KEY, "unknown sequence id %lld", (long long)seqs[i]);
    if ((int64_t)it->second.table.size() > width)
      return fail(PKV_ERR_SHAPE, "sequence %lld holds %zu blocks > width %d", (long long)seqs[i],
                  it->second.table.size(), (int)width);
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& t = bm->seqs.at(seqs[i]).table;
    int32_t* row = table + (int64_t)i * width;
    std::fill(row, row + width, -1);
    std::copy(t.begin(), t.end(), row);
  }
  return ok();
}

PKV_EXPORT pkv_status pkv_bm_get_stats(const pkv_block_manager* bm, pkv_bm_stats* out) {
  if (!bm || !out) return fail(PKV_ERR_NULL, "block manager and out must be non-NULL");
  pkv_bm_stats s{};
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->refcount[b] > 0) {
      ++s.allocated_blocks;
      s.used_slots += bm->fill[b];
    }
  }
  s.allocated_slots = s.allocated_blocks * bm->block_size;
  s.free_blocks = (int64_t)bm->free_list.size();
  s.sequences = (int64_t)bm->seqs.size();
  for (const auto& kv : bm->seqs) s.logical_tokens += kv.second.len;
  s.copies = bm->copies;
  s.preemptions = bm->preemptions;
  s.cached_blocks = (int64_t)bm->cache.size();
  s.reused_blocks = bm->reused;
  s.host_blocks_used = bm->host_blocks - (int64_t)bm->host_free.size();
  s.swapped_sequences = (int64_t)bm->swapped.size();
  s.swap_outs = bm->swap_outs;
  s.unused_slots = s.allocated_slots - s.used_slots;
  s.waste_fraction =
      s.allocated_slots > 0 ? (double)s.unused_slots / (double)s.allocated_slots : 0.0;
  *out = s;
  return ok();
}

PKV_EXPORT pkv_status pkv_capacity(int64_t num_blocks, int32_t block_size, const int32_t* lens,
                                   int32_t n, int32_t reserve_len, int32_t* paged,
                                   int32_t* contiguous) {
  if (!paged || !contiguous || (n > 0 && !lens))
    return fail(PKV_ERR_NULL, "lens, paged and contiguous must be non-NULL");
  if (num_blocks < 0 || block_size < 1 || n < 0 || reserve_len < 1)
    return fail(PKV_ERR_SHAPE, "num_blocks >= 0, block_size >= 1, n >= 0, reserve_len >= 1");
  for (int32_t i = 0; i < n; ++i)
    if (lens[i] < 0 || lens[i] > reserve_len)
      return fail(PKV_ERR_SHAPE, "length %d outside 0..reserve_len (%d)", (int)lens[i],
                  (int)reserve_len);
  int64_t used = 0;
  int32_t fit = 0;
  for (; fit < n; ++fit) {
    used += (lens[fit] + (int64_t)block_size - 1) / block_size;
    if (used > num_blocks) break;
  }
  *paged = fit;
  const int64_t slots = num_blocks * (int64_t)block_size;
  *contiguous = (int32_t)std::min<int64_t>(n, slots / reserve_len);
  return ok();
}
