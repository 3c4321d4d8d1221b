// Host-side block allocator with a chained-hash prefix cache: the producer
// of the block tables and slots the kernels consume.
//
// Behaviour follows "12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.8
// (BlockManager) and the trace of "对照 Nano-vLLM 实现：读懂 vLLM 调度", §1.2:
//   * blocks carry a reference count, the prefix hash of their contents (only
//     once full) and those token ids (to rule out hash collisions);
//   * free blocks form a FIFO: handed out from the front, returned to the back,
//     so a just-freed block keeps its cached contents as long as possible;
//   * a block's hash chains the previous block's hash (8 bytes, little endian;
//     none for the first block) with its int64 token ids, through xxh64;
//   * freeing keeps the hash and the index entry (a later prompt with the same
//     prefix revives the block); handing the block out again drops the entry.
// The allocator is host code: no device memory, no GPU calls.
#include <cstring>
#include <deque>
#include <unordered_map>
#include <vector>

#include "common.hpp"

namespace pa {
namespace {

// ---------------------------------------------------------------- xxh64
// The published xxHash64 algorithm (seed 0), one-shot over a byte buffer.
constexpr uint64_t kPrime1 = 0x9E3779B185EBCA87ULL;
constexpr uint64_t kPrime2 = 0xC2B2AE3D27D4EB4FULL;
constexpr uint64_t kPrime3 = 0x165667B19E3779F9ULL;
constexpr uint64_t kPrime4 = 0x85EBCA77C2B2AE63ULL;
constexpr uint64_t kPrime5 = 0x27D4EB2F165667C5ULL;

inline uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t load_le64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
  return v;
}
inline uint32_t load_le32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
inline uint64_t stripe_round(uint64_t acc, uint64_t lane) {
  return rotl64(acc + lane * kPrime2, 31) * kPrime1;
}
inline uint64_t merge_accumulator(uint64_t h, uint64_t acc) {
  return (h ^ stripe_round(0, acc)) * kPrime1 + kPrime4;
}

uint64_t xxh64(const uint8_t* p, size_t len) {
  const uint8_t* const end = p + len;
  uint64_t h;
  if (len >= 32) {
    uint64_t a1 = kPrime1 + kPrime2, a2 = kPrime2, a3 = 0, a4 = 0 - kPrime1;
    do {
      a1 = stripe_round(a1, load_le64(p));
      a2 = stripe_round(a2, load_le64(p + 8));
      a3 = stripe_round(a3, load_le64(p + 16));
      a4 = stripe_round(a4, load_le64(p + 24));
      p += 32;
    } while (end - p >= 32);
    h = rotl64(a1, 1) + rotl64(a2, 7) + rotl64(a3, 12) + rotl64(a4, 18);
    h = merge_accumulator(h, a1);
    h = merge_accumulator(h, a2);
    h = merge_accumulator(h, a3);
    h = merge_accumulator(h, a4);
  } else {
    h = kPrime5;
  }
  h += (uint64_t)len;
  for (; end - p >= 8; p += 8) h = rotl64(h ^ stripe_round(0, load_le64(p)), 27) * kPrime1 + kPrime4;
  if (end - p >= 4) {
    h = rotl64(h ^ ((uint64_t)load_le32(p) * kPrime1), 23) * kPrime2 + kPrime3;
    p += 4;
  }
  for (; p < end; ++p) h = rotl64(h ^ ((uint64_t)*p * kPrime5), 11) * kPrime1;
  h ^= h >> 33;
  h *= kPrime2;
  h ^= h >> 29;
  h *= kPrime3;
  h ^= h >> 32;
  return h;
}

uint64_t chained_hash(const int64_t* tokens, int32_t n, bool has_prefix, uint64_t prefix) {
  thread_local std::vector<uint8_t> buf;
  buf.resize((size_t)(has_prefix ? 8 : 0) + (size_t)n * 8);
  uint8_t* p = buf.data();
  if (has_prefix)
    for (int i = 0; i < 8; ++i) *p++ = (uint8_t)(prefix >> (8 * i));
  for (int32_t t = 0; t < n; ++t) {
    const uint64_t v = (uint64_t)tokens[t];
    for (int i = 0; i < 8; ++i) *p++ = (uint8_t)(v >> (8 * i));
  }
  return xxh64(buf.data(), buf.size());
}

}  // namespace
}  // namespace pa

struct pa_block_manager {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> ref;
  std::vector<uint64_t> hash;
  std::vector<uint8_t> hashed;
  std::vector<std::vector<int64_t>> tokens;
  std::vector<uint8_t> used;
  std::deque<int32_t> free_ids;
  std::unordered_map<uint64_t, int32_t> index;

  int32_t take_free_block() {
    const int32_t bid = free_ids.front();
    free_ids.pop_front();
    if (hashed[bid]) {
      auto it = index.find(hash[bid]);
      if (it != index.end() && it->second == bid) index.erase(it);
    }
    ref[bid] = 1;
    hashed[bid] = 0;
    tokens[bid].clear();
    used[bid] = 1;
    return bid;
  }

  void release_block(int32_t bid) {
    used[bid] = 0;
    free_ids.push_back(bid);
  }

  // Leading full blocks (all but the last block of the sequence) that the
  // index holds with identical tokens; `in_use` counts those referenced now.
  int32_t cached_prefix(const int64_t* toks, int32_t n, int32_t* in_use) const {
    const int32_t nblocks = (n + block_size - 1) / block_size;
    bool has = false;
    uint64_t h = 0;
    int32_t hits = 0;
    *in_use = 0;
    for (int32_t i = 0; i + 1 < nblocks; ++i) {
      const int64_t* b = toks + (int64_t)i * block_size;
      h = pa::chained_hash(b, block_size, has, h);
      has = true;
      auto it = index.find(h);
      if (it == index.end()) break;
      const int32_t bid = it->second;
      const auto& stored = tokens[bid];
      if ((int32_t)stored.size() != block_size ||
          std::memcmp(stored.data(), b, sizeof(int64_t) * block_size) != 0)
        break;
      ++hits;
      if (used[bid]) ++*in_use;
    }
    return hits;
  }
};

extern "C" pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) {
    pa::set_error("pa_bm_create: num_blocks and block_size must be positive");
    return nullptr;
  }
  auto* bm = new pa_block_manager();
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->hash.assign(num_blocks, 0);
  bm->hashed.assign(num_blocks, 0);
  bm->tokens.assign(num_blocks, {});
  bm->used.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) bm->free_ids.push_back(i);
  return bm;
}

extern "C" void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

extern "C" uint64_t pa_bm_chained_hash(const int64_t* token_ids, int32_t n, uint64_t prefix,
                                       int32_t has_prefix) {
  if (n < 0 || (n > 0 && !token_ids)) return 0;
  return pa::chained_hash(token_ids, n, has_prefix != 0, prefix);
}

extern "C" int32_t pa_bm_can_allocate(pa_block_manager* bm, const int64_t* token_ids,
                                      int32_t num_tokens, int32_t* num_cached_blocks) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !token_ids) || !num_cached_blocks)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_can_allocate: bad arguments");
  int32_t in_use = 0;
  *num_cached_blocks = bm->cached_prefix(token_ids, num_tokens, &in_use);
  const int32_t nblocks = (num_tokens + bm->block_size - 1) / bm->block_size;
  return (int32_t)bm->free_ids.size() >= nblocks - in_use ? 1 : 0;
}

extern "C" int32_t pa_bm_allocate(pa_block_manager* bm, const int64_t* token_ids,
                                  int32_t num_tokens, int32_t num_cached_blocks,
                                  int32_t* block_table, int32_t capacity) {
  using pa::fail;
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !token_ids) || !block_table)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: bad arguments");
  const int32_t nblocks = (num_tokens + bm->block_size - 1) / bm->block_size;
  if (capacity < nblocks) return fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: table capacity");
  if (num_cached_blocks < 0 || num_cached_blocks > nblocks)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: num_cached_blocks out of range");
  // check before mutating: cached blocks must be indexed, the rest must fit
  int32_t in_use = 0;
  if (bm->cached_prefix(token_ids, num_tokens, &in_use) < num_cached_blocks)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: prefix not cached");
  bool has = false;
  uint64_t h = 0;
  int32_t revive = 0;
  for (int32_t i = 0; i < num_cached_blocks; ++i) {
    h = pa::chained_hash(token_ids + (int64_t)i * bm->block_size, bm->block_size, has, h);
    has = true;
    if (!bm->used[bm->index.at(h)]) ++revive;
  }
  if ((int32_t)bm->free_ids.size() < revive + (nblocks - num_cached_blocks))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: not enough free blocks");
  has = false;
  h = 0;
  for (int32_t i = 0; i < num_cached_blocks; ++i) {
    h = pa::chained_hash(token_ids + (int64_t)i * bm->block_size, bm->block_size, has, h);
    has = true;
    const int32_t bid = bm->index.at(h);
    if (bm->used[bid]) {
      ++bm->ref[bid];
    } else {  // freed but not reused yet: take it back out of the FIFO
      bm->ref[bid] = 1;
      for (auto it = bm->free_ids.begin(); it != bm->free_ids.end(); ++it)
        if (*it == bid) {
          bm->free_ids.erase(it);
          break;
        }
      bm->used[bid] = 1;
    }
    block_table[i] = bid;
  }
  for (int32_t i = num_cached_blocks; i < nblocks; ++i) block_table[i] = bm->take_free_block();
  pa::clear_error();
  return nblocks;
}

extern "C" int32_t pa_bm_deallocate(pa_block_manager* bm, const int32_t* block_table,
                                    int32_t n_blocks) {
  if (!bm || n_blocks < 0 || (n_blocks > 0 && !block_table))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_deallocate: bad arguments");
  for (int32_t i = 0; i < n_blocks; ++i) {
    const int32_t bid = block_table[i];
    if (bid < 0 || bid >= bm->num_blocks || bm->ref[bid] <= 0)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_deallocate: block %d is not allocated", bid);
  }
  for (int32_t i = n_blocks - 1; i >= 0; --i) {
    const int32_t bid = block_table[i];
    if (--bm->ref[bid] == 0) bm->release_block(bid);
  }
  return PA_OK;
}

extern "C" int32_t pa_bm_can_append(const pa_block_manager* bm, int32_t seq_len) {
  if (!bm || seq_len < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_can_append: bad arguments");
  const int32_t need = (seq_len % bm->block_size == 1) ? 1 : 0;
  return (int32_t)bm->free_ids.size() >= need ? 1 : 0;
}

extern "C" int32_t pa_bm_may_append(pa_block_manager* bm, int32_t seq_len, int32_t* block_table,
                                    int32_t n_blocks, int32_t capacity) {
  if (!bm || seq_len < 0 || n_blocks < 0 || !block_table)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_may_append: bad arguments");
  if (seq_len % bm->block_size != 1) return n_blocks;
  if (n_blocks >= capacity) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_may_append: capacity");
  if (bm->free_ids.empty()) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_may_append: no free block");
  block_table[n_blocks] = bm->take_free_block();
  return n_blocks + 1;
}

extern "C" int32_t pa_bm_hash_blocks(pa_block_manager* bm, const int64_t* token_ids,
                                     int32_t num_tokens, const int32_t* block_table,
                                     int32_t n_blocks, int32_t num_cached_tokens,
                                     int32_t num_scheduled_tokens) {
  using pa::fail;
  if (!bm || !block_table || num_cached_tokens < 0 || num_scheduled_tokens < 0)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_hash_blocks: bad arguments");
  const int32_t bs = bm->block_size;
  const int32_t start = num_cached_tokens / bs;
  const int32_t end = (num_cached_tokens + num_scheduled_tokens) / bs;
  if (start == end) return 0;
  if (end > n_blocks || (int64_t)end * bs > num_tokens || !token_ids)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_hash_blocks: range past the sequence");
  bool has = false;
  uint64_t h = 0;
  if (start > 0 && bm->hashed[block_table[start - 1]]) {
    has = true;
    h = bm->hash[block_table[start - 1]];
  }
  for (int32_t i = start; i < end; ++i) {
    const int32_t bid = block_table[i];
    const int64_t* b = token_ids + (int64_t)i * bs;
    h = pa::chained_hash(b, bs, has, h);
    has = true;
    bm->hash[bid] = h;
    bm->hashed[bid] = 1;
    bm->tokens[bid].assign(b, b + bs);
    bm->index[h] = bid;
  }
  return end - start;
}

extern "C" int32_t pa_bm_num_free(const pa_block_manager* bm) {
  return bm ? (int32_t)bm->free_ids.size() : PA_ERR_INVALID_ARG;
}

extern "C" int32_t pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int32_t capacity) {
  if (!bm || (capacity > 0 && !out)) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_free_list");
  int32_t n = 0;
  for (int32_t bid : bm->free_ids) {
    if (n < capacity) out[n] = bid;
    ++n;
  }
  return n;
}

extern "C" int32_t pa_bm_block_state(const pa_block_manager* bm, int32_t block_id,
                                     int32_t* ref_count, uint64_t* hash, int32_t* hashed) {
  if (!bm || block_id < 0 || block_id >= bm->num_blocks)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_block_state: bad block");
  if (ref_count) *ref_count = bm->ref[block_id];
  if (hash) *hash = bm->hash[block_id];
  if (hashed) *hashed = bm->hashed[block_id];
  return PA_OK;
}

extern "C" int32_t pa_bm_lookup(const pa_block_manager* bm, uint64_t hash) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->index.find(hash);
  return it == bm->index.end() ? -1 : it->second;
}

extern "C" int32_t pa_bm_index_entries(const pa_block_manager* bm, uint64_t* hashes,
                                       int32_t* block_ids, int32_t capacity) {
  if (!bm) return PA_ERR_INVALID_ARG;
  int32_t n = 0;
  for (const auto& kv : bm->index) {
    if (n < capacity) {
      hashes[n] = kv.first;
      block_ids[n] = kv.second;
    }
    ++n;
  }
  return n;
}
