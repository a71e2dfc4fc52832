// Host-side block manager with a chain-hash prefix cache (C++, no device code).
//
// Behaviour ("大模型推理引擎学习入门-2：带你理解 nano-vllm 的 KV Cache 以及 Paged
// Attention" (juejin.cn), sections 2.2, 3.3 and 3.4; the nano-vLLM lab manual
// "5. 动手改造：从跑通到可测量的推理服务", B.6):
//  * a full block's fingerprint is a chain hash: XXH64 (seed 0) over the previous full
//    block's fingerprint (8 bytes, little-endian; absent for the first block) followed by
//    the block's token ids as 64-bit little-endian integers, so equal fingerprints stand
//    for equal whole prefixes;
//  * admitting a prompt matches its blocks against the cache from the first one on; the
//    first block without a match ends the matching, and the prompt's last block is never
//    matched (B.6), so at least one token is computed.  A matched block in use is shared
//    (one more reference), a matched block that was freed but not handed out again is
//    taken back; every other block is fresh, taken from the front of the free list and
//    emptied (its old fingerprint leaves the index).  All full blocks of the prompt
//    become findable under their fingerprints;
//  * a finished sequence gives back one reference per block, last block first; a block at
//    zero joins the back of the free list and stays findable until it is handed out
//    again (lazy reclamation);
//  * a generated token that starts a block gets a fresh one, a token that completes a
//    block makes it findable.  A forked sequence shares all blocks of its parent; writing
//    into a shared last block first moves the writer to a fresh block (copy-on-write,
//    section 2.2) and the caller copies the block's K/V rows with pa_copy_blocks.
//
// Layout: per-block arrays (references, fingerprint, token ids of findable blocks) and
// the free list as links threaded through the block ids, so that taking a freed block
// back, wherever it sits in the list, costs O(1).
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
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

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  int32_t cached = 0;
};

}  // namespace

struct BlockManager {
  const int32_t bs;
  const int32_t n;
  std::vector<int32_t> refs;
  std::vector<uint8_t> findable;  // the block holds a full block listed under fp
  std::vector<uint64_t> fp;
  std::vector<int32_t> held;      // [n][bs] token ids of findable blocks
  std::vector<int32_t> prev, next;  // free-list links, -1 at the ends
  int32_t head = -1, tail = -1, nfree = 0;
  std::unordered_map<uint64_t, int32_t> index;  // fingerprint -> block
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_handle = 0;

  BlockManager(int32_t num_blocks, int32_t block_size)
      : bs(block_size), n(num_blocks), refs(num_blocks, 0), findable(num_blocks, 0),
        fp(num_blocks, 0), held((size_t)num_blocks * block_size), prev(num_blocks, -1),
        next(num_blocks, -1) {
    for (int32_t b = 0; b < n; ++b) push_free(b);
  }

  void push_free(int32_t b) {  // to the back
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b;
    else head = b;
    tail = b;
    ++nfree;
  }
  void unlink_free(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b];
    else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b];
    else tail = prev[b];
    prev[b] = next[b] = -1;
    --nfree;
  }
  // The least recently freed block, emptied for new contents, with its first reference.
  int32_t fresh() {
    const int32_t b = head;
    unlink_free(b);
    if (findable[b]) {
      const auto it = index.find(fp[b]);
      if (it != index.end() && it->second == b) index.erase(it);
      findable[b] = 0;
    }
    refs[b] = 1;
    return b;
  }
  void make_findable(int32_t b, uint64_t h, const int32_t* toks) {
    findable[b] = 1;
    fp[b] = h;
    std::memcpy(&held[(size_t)b * bs], toks, sizeof(int32_t) * bs);
    index[h] = b;
  }
  // The block still holding exactly these tokens under this fingerprint, or -1.
  int32_t lookup(uint64_t h, const int32_t* toks) const {
    const auto it = index.find(h);
    if (it == index.end()) return -1;
    const int32_t b = it->second;
    if (!findable[b] || fp[b] != h ||
        std::memcmp(&held[(size_t)b * bs], toks, sizeof(int32_t) * bs) != 0)
      return -1;
    return b;
  }
  void unref(int32_t b) {
    if (--refs[b] == 0) push_free(b);  // keeps what it holds
  }
  // Chain fingerprints of the first `count` full blocks of a token list.
  void fingerprints(const int32_t* toks, int count, std::vector<uint64_t>& out) const {
    out.resize(count);
    for (int i = 0; i < count; ++i)
      out[i] = chain_hash(toks + (size_t)i * bs, bs, i > 0, i > 0 ? out[i - 1] : 0);
  }
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
  try {
    return new pa_block_manager(num_blocks, block_size);
  } catch (const std::bad_alloc&) {
    fail(PA_ERR_CAPACITY, "pa_bm_create: out of host memory for %d blocks", num_blocks);
    return nullptr;
  }
}

extern "C" void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

extern "C" int64_t pa_bm_allocate(pa_block_manager* bm, const int32_t* token_ids,
                                  int32_t num_tokens) {
  clear_error();
  if (!bm || (!token_ids && num_tokens > 0)) return -fail(PA_ERR_NULL, "pa_bm_allocate: null");
  if (num_tokens <= 0) return -fail(PA_ERR_SHAPE, "pa_bm_allocate: %d tokens", num_tokens);
  BlockManager& m = bm->m;
  const int need = (num_tokens + m.bs - 1) / m.bs;
  if (need > m.nfree)  // decided on the worst case: no block found in the cache
    return -fail(PA_ERR_CAPACITY, "pa_bm_allocate: %d blocks needed, %d free", need, m.nfree);
  const int full = num_tokens / m.bs;
  std::vector<uint64_t> fps;
  m.fingerprints(token_ids, full, fps);
  // The cached run at the front of the prompt (never its last block).
  std::vector<int32_t> table;
  table.reserve(need);
  for (int i = 0; i < full && i < need - 1; ++i) {
    const int32_t b = m.lookup(fps[i], token_ids + (size_t)i * m.bs);
    if (b < 0) break;
    table.push_back(b);
  }
  const int matched = (int)table.size();
  for (const int32_t b : table) {
    if (m.refs[b] > 0) {
      ++m.refs[b];  // shared with a live sequence
    } else {
      m.unlink_free(b);  // freed but intact: back in use
      m.refs[b] = 1;
    }
  }
  while ((int)table.size() < need) table.push_back(m.fresh());
  for (int i = 0; i < full; ++i) m.make_findable(table[i], fps[i], token_ids + (size_t)i * m.bs);
  Seq s;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  s.table = std::move(table);
  s.cached = matched * m.bs;
  const int64_t handle = m.next_handle++;
  m.seqs.emplace(handle, std::move(s));
  return handle;
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
  const int len = (int)s.tokens.size() + 1;  // with the new token
  const bool starts = len % m.bs == 1;  // block_size >= 2
  if (starts || m.refs[s.table.back()] > 1) {
    if (m.nfree == 0) return fail(PA_ERR_CAPACITY, "pa_bm_append: no free block");
    if (starts) {
      s.table.push_back(m.fresh());
    } else {  // the last block is shared: move to a private copy
      const int32_t src = s.table.back();
      s.table.back() = m.fresh();
      --m.refs[src];  // others still hold it
      if (cow_src) *cow_src = src;
      if (cow_dst) *cow_dst = s.table.back();
    }
  }
  s.tokens.push_back(token_id);
  if (len % m.bs == 0) {  // the token completes its block
    const int i = len / m.bs - 1;
    std::vector<uint64_t> fps;
    m.fingerprints(s.tokens.data(), i + 1, fps);
    m.make_findable(s.table[i], fps[i], s.tokens.data() + (size_t)i * m.bs);
  }
  return PA_OK;
}

extern "C" int64_t pa_bm_fork(pa_block_manager* bm, int64_t seq) {
  clear_error();
  if (!bm) return -fail(PA_ERR_NULL, "pa_bm_fork: null");
  BlockManager& m = bm->m;
  auto it = m.seqs.find(seq);
  if (it == m.seqs.end()) return -fail(PA_ERR_SHAPE, "pa_bm_fork: no sequence %lld", (long long)seq);
  for (const int32_t b : it->second.table) ++m.refs[b];
  Seq child = it->second;
  const int64_t handle = m.next_handle++;
  m.seqs.emplace(handle, std::move(child));
  return handle;
}

extern "C" int pa_bm_free(pa_block_manager* bm, int64_t seq) {
  clear_error();
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_free: null");
  BlockManager& m = bm->m;
  auto it = m.seqs.find(seq);
  if (it == m.seqs.end()) return fail(PA_ERR_SHAPE, "pa_bm_free: no sequence %lld", (long long)seq);
  const std::vector<int32_t>& t = it->second.table;
  for (auto r = t.rbegin(); r != t.rend(); ++r) m.unref(*r);  // last block first
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
  if (block_id < 0 || block_id >= bm->m.n) return -PA_ERR_SHAPE;
  return bm->m.refs[block_id];
}

extern "C" int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? bm->m.nfree : -PA_ERR_NULL;
}
