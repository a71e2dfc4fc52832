// Host-side block manager with a chain-hash prefix cache (C++, no device code).
//
// What is implemented follows "大模型推理引擎学习入门-2：带你理解 nano-vllm 的 KV Cache 以及
// Paged Attention" (juejin.cn), sections 2.2, 3.3 and 3.4, and the nano-vLLM lab manual
// ("5. 动手改造：从跑通到可测量的推理服务"), B.6:
//  * a block's fingerprint is a chain hash: XXH64 (seed 0) over the previous full block's
//    hash (8 bytes, little-endian; absent for the first block) followed by the block's
//    token ids as 64-bit little-endian integers, so equal fingerprints mean equal whole
//    prefixes; only full blocks get one;
//  * allocate walks the prompt's blocks: a fingerprint found in the table whose block still
//    holds the same tokens is a hit (REUSE if the block is in use: one more reference;
//    REACTIVATE if it was freed but not yet overwritten); the first miss ends the hits for
//    the rest of the prompt (ALLOCATE from the front of the free list); the last block of a
//    prompt is never taken from the cache (B.6: a 512-token prompt over 256-token blocks
//    hits at most one block), so at least one token is always computed;
//  * freeing drops one reference per block, last block first; a block at zero goes to the
//    back of the free list and keeps its fingerprint until it is reallocated (lazy
//    reclamation); reallocating it drops its old fingerprint from the table;
//  * appending a token: crossing into a new block allocates one, filling a block registers
//    its fingerprint.  A sequence forked from another shares all its blocks (one more
//    reference each); writing into a shared last block first gives the writer a private
//    copy (copy-on-write, section 2.2), and the caller copies the block's K/V rows on the
//    device with pa_copy_blocks.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace pa {
namespace {

// XXH64, from the published algorithm (Yann Collet's xxHash specification).
constexpr uint64_t kP1 = 0x9E3779B185EBCA87ULL, kP2 = 0xC2B2AE3D27D4EB4FULL,
                   kP3 = 0x165667B19E3779F9ULL, kP4 = 0x85EBCA77C2B2AE63ULL,
                   kP5 = 0x27D4EB2F165667C5ULL;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t read64(const uint8_t* p) {
  uint64_t v;
  std::memcpy(&v, p, 8);  // little-endian host
  return v;
}
inline uint32_t read32(const uint8_t* p) {
  uint32_t v;
  std::memcpy(&v, p, 4);
  return v;
}
inline uint64_t xround(uint64_t acc, uint64_t in) { return rotl(acc + in * kP2, 31) * kP1; }
inline uint64_t xmerge(uint64_t h, uint64_t v) { return (h ^ xround(0, v)) * kP1 + kP4; }

uint64_t xxh64(const uint8_t* p, size_t len, uint64_t seed) {
  const uint8_t* const end = p + len;
  uint64_t h;
  if (len >= 32) {
    uint64_t v1 = seed + kP1 + kP2, v2 = seed + kP2, v3 = seed, v4 = seed - kP1;
    const uint8_t* const limit = end - 32;
    do {
      v1 = xround(v1, read64(p));
      v2 = xround(v2, read64(p + 8));
      v3 = xround(v3, read64(p + 16));
      v4 = xround(v4, read64(p + 24));
      p += 32;
    } while (p <= limit);
    h = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
    h = xmerge(h, v1);
    h = xmerge(h, v2);
    h = xmerge(h, v3);
    h = xmerge(h, v4);
  } else {
    h = seed + kP5;
  }
  h += (uint64_t)len;
  for (; p + 8 <= end; p += 8) h = rotl(h ^ xround(0, read64(p)), 27) * kP1 + kP4;
  if (p + 4 <= end) {
    h = rotl(h ^ ((uint64_t)read32(p) * kP1), 23) * kP2 + kP3;
    p += 4;
  }
  for (; p < end; ++p) h = rotl(h ^ ((uint64_t)*p * kP5), 11) * kP1;
  h ^= h >> 33;
  h *= kP2;
  h ^= h >> 29;
  h *= kP3;
  h ^= h >> 32;
  return h;
}

uint64_t chain_hash(const int32_t* tokens, int n, bool has_prefix, uint64_t prefix) {
  std::vector<uint8_t> buf((has_prefix ? 8 : 0) + 8 * (size_t)n);
  size_t o = 0;
  if (has_prefix) {
    std::memcpy(buf.data(), &prefix, 8);
    o = 8;
  }
  for (int i = 0; i < n; ++i) {
    const int64_t t = tokens[i];
    std::memcpy(buf.data() + o + 8 * (size_t)i, &t, 8);
  }
  return xxh64(buf.data(), buf.size(), 0);
}

struct Block {
  int ref = 0;
  bool hashed = false;  // a full block with a registered fingerprint
  uint64_t hash = 0;
  std::vector<int32_t> tokens;  // the block's token ids once full (for the hit check)
};

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  int32_t cached = 0;
};

}  // namespace

struct BlockManager {
  int32_t bs;
  std::vector<Block> blocks;
  std::deque<int32_t> free_ids;
  std::unordered_set<int32_t> used;
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 0;

  BlockManager(int32_t n, int32_t block_size) : bs(block_size), blocks(n) {
    for (int32_t i = 0; i < n; ++i) free_ids.push_back(i);
  }

  // Takes block id off the free list (front or wherever it is) into use, cleared; a
  // fingerprint it still carried leaves the table.
  void take(int32_t id) {
    for (auto it = free_ids.begin(); it != free_ids.end(); ++it)
      if (*it == id) {
        free_ids.erase(it);
        break;
      }
    Block& b = blocks[id];
    if (b.hashed) {
      const auto it = by_hash.find(b.hash);
      if (it != by_hash.end() && it->second == id) by_hash.erase(it);
    }
    b.ref = 1;
    b.hashed = false;
    b.tokens.clear();
    used.insert(id);
  }
  void release(int32_t id) {
    used.erase(id);
    free_ids.push_back(id);
  }
  void register_full(int32_t id, uint64_t h, const int32_t* toks) {
    Block& b = blocks[id];
    b.hashed = true;
    b.hash = h;
    b.tokens.assign(toks, toks + bs);
    by_hash[h] = id;
  }
  // Fingerprint of logical block i of s (full), chained on block i-1's.
  uint64_t hash_of(const Seq& s, int i, uint64_t prev) const {
    return chain_hash(s.tokens.data() + (size_t)i * bs, bs, i > 0, prev);
  }
  int32_t free_count() const { return (int32_t)free_ids.size(); }
};

}  // namespace pa

using namespace pa;

struct pa_block_manager {
  BlockManager m;
  pa_block_manager(int32_t n, int32_t bs) : m(n, bs) {}
};

extern "C" uint64_t pa_chain_hash(const int32_t* token_ids, int32_t num_tokens,
                                  int32_t has_prefix, uint64_t prefix) {
  return chain_hash(token_ids, num_tokens < 0 ? 0 : num_tokens, has_prefix != 0, prefix);
}

extern "C" pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  clear_error();
  if (num_blocks <= 0 || block_size < 2) {
    fail(PA_ERR_SHAPE, "pa_bm_create: num_blocks %d, block_size %d", num_blocks, block_size);
    return nullptr;
  }
  return new (std::nothrow) pa_block_manager(num_blocks, block_size);
}

extern "C" void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

extern "C" int64_t pa_bm_allocate(pa_block_manager* bm, const int32_t* token_ids,
                                  int32_t num_tokens) {
  clear_error();
  if (!bm || (!token_ids && num_tokens > 0)) return -fail(PA_ERR_NULL, "pa_bm_allocate: null");
  if (num_tokens <= 0) return -fail(PA_ERR_SHAPE, "pa_bm_allocate: %d tokens", num_tokens);
  BlockManager& m = bm->m;
  const int nb = (num_tokens + m.bs - 1) / m.bs;
  if (nb > m.free_count()) {
    // The walk below may reuse blocks, but admission is decided on the worst case.
    return -fail(PA_ERR_CAPACITY, "pa_bm_allocate: %d blocks needed, %d free", nb, m.free_count());
  }
  Seq s;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  bool miss = false;
  uint64_t h = 0;
  for (int i = 0; i < nb; ++i) {
    const bool full = (i + 1) * m.bs <= num_tokens;
    if (full) h = m.hash_of(s, i, h);
    int32_t id = -1;
    if (full && i < nb - 1 && !miss) {  // the prompt's last block is always computed
      const auto it = m.by_hash.find(h);
      if (it != m.by_hash.end()) {
        const Block& b = m.blocks[it->second];
        if (b.hashed && b.hash == h &&
            std::memcmp(b.tokens.data(), s.tokens.data() + (size_t)i * m.bs,
                        sizeof(int32_t) * m.bs) == 0)
          id = it->second;
      }
    }
    if (id < 0) {
      miss = true;
      id = m.free_ids.front();
      m.take(id);  // ALLOCATE
    } else {
      s.cached += m.bs;
      if (m.used.count(id)) ++m.blocks[id].ref;  // REUSE
      else m.take(id);                             // REACTIVATE
    }
    if (full) m.register_full(id, h, s.tokens.data() + (size_t)i * m.bs);
    s.table.push_back(id);
  }
  const int64_t sid = m.next_id++;
  m.seqs.emplace(sid, std::move(s));
  return sid;
}

extern "C" int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t token_id,
                            int32_t* cow_src, int32_t* cow_dst) {
  clear_error();
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_append: null");
  BlockManager& m = bm->m;
  auto it = m.seqs.find(seq);
  if (it == m.seqs.end()) return fail(PA_ERR_SHAPE, "pa_bm_append: no sequence %lld", (long long)seq);
  Seq& s = it->second;
  if (cow_src) *cow_src = -1;
  if (cow_dst) *cow_dst = -1;
  const int len = (int)s.tokens.size() + 1;  // after the append
  if (len % m.bs == 1) {  // the token opens a new block
    if (m.free_count() == 0) return fail(PA_ERR_CAPACITY, "pa_bm_append: no free block");
    const int32_t id = m.free_ids.front();
    m.take(id);
    s.table.push_back(id);
  } else if (m.blocks[s.table.back()].ref > 1) {  // shared partial block: copy on write
    if (m.free_count() == 0) return fail(PA_ERR_CAPACITY, "pa_bm_append: no free block");
    const int32_t src = s.table.back();
    const int32_t id = m.free_ids.front();
    m.take(id);
    --m.blocks[src].ref;
    s.table.back() = id;
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = id;
  }
  s.tokens.push_back(token_id);
  if (len % m.bs == 0) {  // the token fills its block: register the fingerprint
    const int i = len / m.bs - 1;
    const uint64_t prev = i > 0 ? m.blocks[s.table[i - 1]].hash : 0;
    m.register_full(s.table[i], m.hash_of(s, i, prev), s.tokens.data() + (size_t)i * m.bs);
  }
  return PA_OK;
}

extern "C" int64_t pa_bm_fork(pa_block_manager* bm, int64_t seq) {
  clear_error();
  if (!bm) return -fail(PA_ERR_NULL, "pa_bm_fork: null");
  BlockManager& m = bm->m;
  auto it = m.seqs.find(seq);
  if (it == m.seqs.end()) return -fail(PA_ERR_SHAPE, "pa_bm_fork: no sequence %lld", (long long)seq);
  Seq child = it->second;
  for (int32_t id : child.table) ++m.blocks[id].ref;
  const int64_t sid = m.next_id++;
  m.seqs.emplace(sid, std::move(child));
  return sid;
}

extern "C" int pa_bm_free(pa_block_manager* bm, int64_t seq) {
  clear_error();
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_free: null");
  BlockManager& m = bm->m;
  auto it = m.seqs.find(seq);
  if (it == m.seqs.end()) return fail(PA_ERR_SHAPE, "pa_bm_free: no sequence %lld", (long long)seq);
  const std::vector<int32_t>& t = it->second.table;
  for (auto r = t.rbegin(); r != t.rend(); ++r)
    if (--m.blocks[*r].ref == 0) m.release(*r);
  m.seqs.erase(it);
  return PA_OK;
}

extern "C" int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq, int32_t* out,
                                     int32_t capacity) {
  clear_error();
  if (!bm) return -fail(PA_ERR_NULL, "pa_bm_block_table: null");
  auto it = bm->m.seqs.find(seq);
  if (it == bm->m.seqs.end()) return -fail(PA_ERR_SHAPE, "pa_bm_block_table: no sequence");
  const std::vector<int32_t>& t = it->second.table;
  const int32_t n = (int32_t)t.size();
  if (out)
    for (int32_t i = 0; i < n && i < capacity; ++i) out[i] = t[i];
  return n;
}

extern "C" int32_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq) {
  if (!bm) return -PA_ERR_NULL;
  auto it = bm->m.seqs.find(seq);
  return it == bm->m.seqs.end() ? -PA_ERR_SHAPE : (int32_t)it->second.tokens.size();
}

extern "C" int32_t pa_bm_num_cached_tokens(const pa_block_manager* bm, int64_t seq) {
  if (!bm) return -PA_ERR_NULL;
  auto it = bm->m.seqs.find(seq);
  return it == bm->m.seqs.end() ? -PA_ERR_SHAPE : it->second.cached;
}

extern "C" int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id) {
  if (!bm) return -PA_ERR_NULL;
  if (block_id < 0 || block_id >= (int32_t)bm->m.blocks.size()) return -PA_ERR_SHAPE;
  return bm->m.blocks[block_id].ref;
}

extern "C" int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? bm->m.free_count() : -PA_ERR_NULL;
}
