// Host-side KV block manager: free-block queue, allocate_slots, per-block prefix hashing
// with longest-hit lookup, and the step arrays the attention path reads. Declared in
// include/pa_blocks.h, which states the policy; this file follows it.
//
// Blocks: hn.213312.xyz "深入解析 vLLM", section 一 (engine construction: a queue of free
// blocks; scheduler: allocate_slots). Prefix hashing: same page, section 二, item 2, and
// shengyayun.com "读懂 vLLM 推理引擎内幕", section 关键实现细节, items 1 and 2.
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_blocks.h"
#include "pa_internal.h"

namespace {

constexpr int kBlockTokens = PA_BLOCK_SIZE;

// ---- hashes -------------------------------------------------------------------------

struct HashKey {
  uint8_t b[32];
  bool operator==(const HashKey& o) const { return std::memcmp(b, o.b, 32) == 0; }
};

struct HashKeyHasher {
  size_t operator()(const HashKey& k) const {
    uint64_t x;
    std::memcpy(&x, k.b, 8);
    uint64_t y;
    std::memcpy(&y, k.b + 8, 8);
    return static_cast<size_t>(x ^ (y * 0x9E3779B97F4A7C15ull));
  }
};

void put_le32(uint8_t* dst, uint32_t v) {
  for (int i = 0; i < 4; ++i) dst[i] = static_cast<uint8_t>(v >> (8 * i));
}

// 64-bit FNV-1a (Fowler, Noll, Vo): offset basis 14695981039346656037, prime 2^40 + 2^8 + 0xb3.
uint64_t fnv1a64(const uint8_t* data, size_t n) {
  uint64_t h = 14695981039346656037ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= data[i];
    h *= 1099511628211ull;
  }
  return h;
}

// SHA-256 (FIPS 180-4). The round constants are the first 32 fractional bits of the cube
// roots of the first 64 primes, the initial state those of the square roots of the first
// 8 primes; both are derived here with exact integer roots.
struct Sha256Tables {
  uint32_t k[64];
  uint32_t h0[8];
  Sha256Tables() {
    int primes[64];
    int n = 0;
    for (int c = 2; n < 64; ++c) {
      bool prime = true;
      for (int d = 2; d * d <= c; ++d)
        if (c % d == 0) {
          prime = false;
          break;
        }
      if (prime) primes[n++] = c;
    }
    using u128 = unsigned __int128;
    for (int i = 0; i < 64; ++i) {  // floor(cbrt(p * 2^96)) = floor(cbrt(p) * 2^32)
      const u128 x = static_cast<u128>(primes[i]) << 96;
      uint64_t lo = 0, hi = uint64_t(1) << 37;
      while (hi - lo > 1) {
        const uint64_t mid = (lo + hi) / 2;
        if (static_cast<u128>(mid) * mid * mid <= x) lo = mid; else hi = mid;
      }
      k[i] = static_cast<uint32_t>(lo);
    }
    for (int i = 0; i < 8; ++i) {  // floor(sqrt(p * 2^64)) = floor(sqrt(p) * 2^32)
      const u128 x = static_cast<u128>(primes[i]) << 64;
      uint64_t lo = 0, hi = uint64_t(1) << 38;
      while (hi - lo > 1) {
        const uint64_t mid = (lo + hi) / 2;
        if (static_cast<u128>(mid) * mid <= x) lo = mid; else hi = mid;
      }
      h0[i] = static_cast<uint32_t>(lo);
    }
  }
};

const Sha256Tables& sha_tables() {
  static const Sha256Tables t;
  return t;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void sha256(const uint8_t* msg, size_t len, uint8_t out[32]) {
  const Sha256Tables& t = sha_tables();
  uint32_t h[8];
  std::memcpy(h, t.h0, sizeof(h));
  // padded message: msg, 0x80, zeros, 64-bit big-endian bit length; a multiple of 64 bytes
  const size_t total = ((len + 9 + 63) / 64) * 64;
  std::vector<uint8_t> m(total, 0);
  std::memcpy(m.data(), msg, len);
  m[len] = 0x80;
  const uint64_t bits = static_cast<uint64_t>(len) * 8;
  for (int i = 0; i < 8; ++i) m[total - 1 - i] = static_cast<uint8_t>(bits >> (8 * i));
  for (size_t off = 0; off < total; off += 64) {
    uint32_t w[64];
    for (int i = 0; i < 16; ++i) {
      const uint8_t* p = &m[off + 4 * i];
      w[i] = (uint32_t(p[0]) << 24) | (uint32_t(p[1]) << 16) | (uint32_t(p[2]) << 8) | uint32_t(p[3]);
    }
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = hh + S1 + ch + t.k[i] + w[i];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + maj;
      hh = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h[0] += a;
    h[1] += b;
    h[2] += c;
    h[3] += d;
    h[4] += e;
    h[5] += f;
    h[6] += g;
    h[7] += hh;
  }
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = static_cast<uint8_t>(h[i] >> (24 - 8 * j));
}

HashKey block_hash(pa_block_hash kind, const HashKey* parent, const int32_t* tokens) {
  HashKey out{};
  uint8_t buf[32 + 4 * kBlockTokens];
  const size_t plen = kind == PA_HASH_SHA256 ? 32 : 8;
  if (parent) std::memcpy(buf, parent->b, plen); else std::memset(buf, 0, plen);
  for (int i = 0; i < kBlockTokens; ++i) put_le32(buf + plen + 4 * i, static_cast<uint32_t>(tokens[i]));
  const size_t n = plen + 4 * kBlockTokens;
  if (kind == PA_HASH_SHA256) {
    sha256(buf, n, out.b);
  } else {
    const uint64_t h = fnv1a64(buf, n);
    for (int i = 0; i < 8; ++i) out.b[i] = static_cast<uint8_t>(h >> (8 * i));
  }
  return out;
}

bool valid_hash(int kind) { return kind == PA_HASH_FNV1A64 || kind == PA_HASH_SHA256; }

pa_status fail(pa_status s, const std::string& msg) { return pa::report(s, msg.c_str()); }

std::string id_str(int64_t id) { return std::to_string(static_cast<long long>(id)); }

struct Request {
  std::vector<int32_t> tokens;  // known tokens: prompt, then appended ones
  std::vector<int32_t> blocks;  // block ids in logical order
  std::vector<HashKey> hashes;  // chain hashes of leading full blocks computed so far
  int64_t computed = 0;         // tokens whose KV is written or scheduled
  int64_t hit_tokens = 0;       // tokens served by the prefix cache at registration
  size_t registered = 0;        // leading full blocks already offered to the hash map
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  bool prefix = false;
  pa_block_hash kind = PA_HASH_FNV1A64;
  std::vector<int32_t> ref;
  // free queue: doubly linked list over block ids; -1 ends it
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1, free_count = 0;
  std::vector<uint8_t> has_hash;
  std::vector<HashKey> key;
  std::unordered_map<HashKey, int32_t, HashKeyHasher> cached;
  std::unordered_map<int64_t, Request> reqs;

  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++free_count;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --free_count;
  }
  int32_t pop_head() {
    const int32_t b = head;
    unlink(b);
    return b;
  }
  // Chain hash of the request's block j (j <= hashes.size()); computed once, kept.
  const HashKey& hash_of(Request& r, size_t j) {
    if (j == r.hashes.size())
      r.hashes.push_back(block_hash(kind, j ? &r.hashes[j - 1] : nullptr, r.tokens.data() + j * kBlockTokens));
    return r.hashes[j];
  }
};

extern "C" {

pa_status pa_block_hash_compute(pa_block_hash hash, const uint8_t* parent, const int32_t* tokens, uint8_t* out) {
  if (!tokens || !out) return fail(PA_E_NULL, "tokens and out are required");
  if (!valid_hash(hash)) return fail(PA_E_DTYPE, "unknown block hash " + std::to_string((int)hash));
  HashKey p{};
  if (parent) std::memcpy(p.b, parent, 32);
  const HashKey h = block_hash(hash, &p, tokens);
  std::memcpy(out, h.b, 32);
  return PA_OK;
}

pa_status pa_bm_create(int32_t num_blocks, int32_t prefix_caching, pa_block_hash hash, pa_block_manager** bm) {
  if (!bm) return fail(PA_E_NULL, "bm is required");
  *bm = nullptr;
  if (num_blocks < 1) return fail(PA_E_SHAPE, "num_blocks=" + std::to_string(num_blocks) + " must be >= 1");
  if (!valid_hash(hash)) return fail(PA_E_DTYPE, "unknown block hash " + std::to_string((int)hash));
  if (prefix_caching != 0 && prefix_caching != 1) return fail(PA_E_SHAPE, "prefix_caching must be 0 or 1");
  try {
    auto* m = new pa_block_manager;
    m->num_blocks = num_blocks;
    m->prefix = prefix_caching == 1;
    m->kind = hash;
    m->ref.assign(num_blocks, 0);
    m->prev.assign(num_blocks, -1);
    m->next.assign(num_blocks, -1);
    m->in_free.assign(num_blocks, 0);
    m->has_hash.assign(num_blocks, 0);
    m->key.assign(num_blocks, HashKey{});
    for (int32_t b = 0; b < num_blocks; ++b) m->push_tail(b);
    *bm = m;
  } catch (const std::bad_alloc&) {
    return fail(PA_E_SHAPE, "out of host memory for " + std::to_string(num_blocks) + " blocks");
  }
  return PA_OK;
}

pa_status pa_bm_destroy(pa_block_manager* bm) {
  delete bm;
  return PA_OK;
}

pa_status pa_bm_add_request(pa_block_manager* bm, int64_t request_id, const int32_t* token_ids, int64_t num_tokens,
                            int64_t* num_cached_tokens) {
  if (!bm || !token_ids) return fail(PA_E_NULL, "bm and token_ids are required");
  if (num_tokens < 1) return fail(PA_E_SHAPE, "a request needs at least one token");
  if (bm->reqs.count(request_id)) return fail(PA_E_REQUEST, "request " + id_str(request_id) + " already registered");
  try {
    Request r;
    r.tokens.assign(token_ids, token_ids + num_tokens);
    size_t hit = 0;
    if (bm->prefix) {
      // Longest run of leading full blocks already in the map, leaving one token to compute.
      const size_t max_hit = static_cast<size_t>((num_tokens - 1) / kBlockTokens);
      while (hit < max_hit && bm->cached.count(bm->hash_of(r, hit))) ++hit;
    }
    Request& stored = bm->reqs.emplace(request_id, std::move(r)).first->second;
    for (size_t j = 0; j < hit; ++j) {  // claim the hit
      const int32_t b = bm->cached.at(stored.hashes[j]);
      if (bm->ref[b] == 0) bm->unlink(b);
      ++bm->ref[b];
      stored.blocks.push_back(b);
    }
    stored.computed = stored.hit_tokens = static_cast<int64_t>(hit) * kBlockTokens;
    stored.registered = hit;
    if (num_cached_tokens) *num_cached_tokens = stored.hit_tokens;
  } catch (const std::bad_alloc&) {
    bm->reqs.erase(request_id);
    return fail(PA_E_SHAPE, "out of host memory");
  }
  return PA_OK;
}

pa_status pa_bm_append_tokens(pa_block_manager* bm, int64_t request_id, const int32_t* token_ids,
                              int64_t num_tokens) {
  if (!bm || !token_ids) return fail(PA_E_NULL, "bm and token_ids are required");
  if (num_tokens < 1) return fail(PA_E_SHAPE, "num_tokens must be >= 1");
  auto it = bm->reqs.find(request_id);
  if (it == bm->reqs.end()) return fail(PA_E_REQUEST, "unknown request " + id_str(request_id));
  try {
    it->second.tokens.insert(it->second.tokens.end(), token_ids, token_ids + num_tokens);
  } catch (const std::bad_alloc&) {
    return fail(PA_E_SHAPE, "out of host memory");
  }
  return PA_OK;
}

pa_status pa_bm_allocate_slots(pa_block_manager* bm, int64_t request_id, int64_t num_new_tokens) {
  if (!bm) return fail(PA_E_NULL, "bm is required");
  if (num_new_tokens < 1) return fail(PA_E_SHAPE, "num_new_tokens must be >= 1");
  auto it = bm->reqs.find(request_id);
  if (it == bm->reqs.end()) return fail(PA_E_REQUEST, "unknown request " + id_str(request_id));
  Request& r = it->second;
  const int64_t upto = r.computed + num_new_tokens;
  if (upto > static_cast<int64_t>(r.tokens.size()))
    return fail(PA_E_REQUEST, "request " + id_str(request_id) + ": tokens up to " + std::to_string(upto) +
                                  " are not known (" + std::to_string(r.tokens.size()) + " known)");
  const int64_t want = (upto + kBlockTokens - 1) / kBlockTokens;
  const int64_t need = want - static_cast<int64_t>(r.blocks.size());
  if (need > bm->free_count)
    return fail(PA_E_NO_SPACE, "request " + id_str(request_id) + " needs " + std::to_string(need) + " blocks, " +
                                   std::to_string(bm->free_count) + " free");
  try {
    r.blocks.reserve(static_cast<size_t>(want));
    r.hashes.reserve(static_cast<size_t>(upto / kBlockTokens));
    for (int64_t n = 0; n < need; ++n) {
      const int32_t b = bm->pop_head();
      if (bm->has_hash[b]) {  // evict the reused block's old content from the map
        auto c = bm->cached.find(bm->key[b]);
        if (c != bm->cached.end() && c->second == b) bm->cached.erase(c);
        bm->has_hash[b] = 0;
      }
      bm->ref[b] = 1;
      r.blocks.push_back(b);
    }
    if (bm->prefix) {  // offer the blocks this makes full to the map
      const size_t full = static_cast<size_t>(upto / kBlockTokens);
      for (size_t j = r.registered; j < full; ++j) {
        const HashKey& h = bm->hash_of(r, j);
        const int32_t b = r.blocks[j];
        if (!bm->has_hash[b] && !bm->cached.count(h)) {
          bm->cached.emplace(h, b);
          bm->has_hash[b] = 1;
          bm->key[b] = h;
        }
      }
      if (full > r.registered) r.registered = full;
    }
  } catch (const std::bad_alloc&) {
    return fail(PA_E_SHAPE, "out of host memory");
  }
  return PA_OK;
}

pa_status pa_bm_free_request(pa_block_manager* bm, int64_t request_id) {
  if (!bm) return fail(PA_E_NULL, "bm is required");
  auto it = bm->reqs.find(request_id);
  if (it == bm->reqs.end()) return fail(PA_E_REQUEST, "unknown request " + id_str(request_id));
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (size_t j = blocks.size(); j-- > 0;) {
    const int32_t b = blocks[j];
    if (--bm->ref[b] == 0) bm->push_tail(b);
  }
  bm->reqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_build_step(pa_block_manager* bm, const int64_t* request_ids, const int64_t* query_lens,
                           int32_t num_seqs, int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* seq_lens,
                           int32_t* query_start_loc, int32_t* context_lens, int64_t* slot_mapping,
                           int64_t num_tokens) {
  if (!bm || !query_start_loc) return fail(PA_E_NULL, "bm and query_start_loc are required");
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_E_SHAPE, "num_seqs and num_tokens must be >= 0");
  if (num_seqs > 0 && (!request_ids || !query_lens || !block_tables || !seq_lens || !context_lens))
    return fail(PA_E_NULL, "request_ids, query_lens, block_tables, seq_lens and context_lens are required");
  if (num_seqs > 0 && max_blocks_per_seq < 1) return fail(PA_E_SHAPE, "max_blocks_per_seq must be >= 1");
  if (num_tokens > 0 && !slot_mapping) return fail(PA_E_NULL, "slot_mapping is required");
  std::vector<Request*> rs(static_cast<size_t>(num_seqs));
  std::unordered_set<int64_t> seen;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {  // validate everything before writing anything
    const int64_t id = request_ids[i];
    auto it = bm->reqs.find(id);
    if (it == bm->reqs.end()) return fail(PA_E_REQUEST, "unknown request " + id_str(id));
    if (!seen.insert(id).second) return fail(PA_E_REQUEST, "request " + id_str(id) + " appears twice in the step");
    Request& r = it->second;
    const int64_t n = query_lens[i];
    if (n < 0) return fail(PA_E_SHAPE, "query_lens[" + std::to_string(i) + "] is negative");
    if (r.computed + n > static_cast<int64_t>(r.blocks.size()) * kBlockTokens ||
        r.computed + n > static_cast<int64_t>(r.tokens.size()))
      return fail(PA_E_REQUEST, "request " + id_str(id) + ": " + std::to_string(n) +
                                    " query tokens are not covered by allocate_slots");
    if (static_cast<int64_t>(r.blocks.size()) > max_blocks_per_seq)
      return fail(PA_E_SHAPE, "request " + id_str(id) + " holds " + std::to_string(r.blocks.size()) +
                                  " blocks, more than max_blocks_per_seq=" + std::to_string(max_blocks_per_seq));
    if (r.computed + n > INT32_MAX) return fail(PA_E_SHAPE, "sequence too long for int32 lengths");
    total += n;
    rs[i] = &r;
  }
  if (total > num_tokens)
    return fail(PA_E_SHAPE, "the step schedules " + std::to_string(total) + " tokens, num_tokens=" +
                                std::to_string(num_tokens));
  if (total > INT32_MAX) return fail(PA_E_SHAPE, "too many tokens for int32 offsets");
  int64_t row = 0;
  query_start_loc[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Request& r = *rs[i];
    const int64_t n = query_lens[i];
    int32_t* bt = block_tables + static_cast<int64_t>(i) * max_blocks_per_seq;
    const size_t nb = r.blocks.size();
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) bt[j] = static_cast<size_t>(j) < nb ? r.blocks[j] : 0;
    context_lens[i] = static_cast<int32_t>(r.computed);
    seq_lens[i] = static_cast<int32_t>(r.computed + n);
    for (int64_t t = 0; t < n; ++t) {
      const int64_t pos = r.computed + t;
      slot_mapping[row + t] = static_cast<int64_t>(r.blocks[pos / kBlockTokens]) * kBlockTokens + pos % kBlockTokens;
    }
    row += n;
    query_start_loc[i + 1] = static_cast<int32_t>(row);
    r.computed += n;
  }
  for (int64_t t = row; t < num_tokens; ++t) slot_mapping[t] = -1;
  return PA_OK;
}

pa_status pa_bm_num_free_blocks(const pa_block_manager* bm, int32_t* num_free) {
  if (!bm || !num_free) return fail(PA_E_NULL, "bm and num_free are required");
  *num_free = bm->free_count;
  return PA_OK;
}

pa_status pa_bm_num_cached_blocks(const pa_block_manager* bm, int32_t* num_cached) {
  if (!bm || !num_cached) return fail(PA_E_NULL, "bm and num_cached are required");
  *num_cached = static_cast<int32_t>(bm->cached.size());
  return PA_OK;
}

pa_status pa_bm_request_blocks(const pa_block_manager* bm, int64_t request_id, int32_t* blocks, int32_t capacity,
                               int32_t* num_blocks) {
  if (!bm || !num_blocks || (capacity > 0 && !blocks)) return fail(PA_E_NULL, "bm, num_blocks and blocks are required");
  auto it = bm->reqs.find(request_id);
  if (it == bm->reqs.end()) return fail(PA_E_REQUEST, "unknown request " + id_str(request_id));
  const std::vector<int32_t>& b = it->second.blocks;
  for (size_t j = 0; j < b.size() && static_cast<int64_t>(j) < capacity; ++j) blocks[j] = b[j];
  *num_blocks = static_cast<int32_t>(b.size());
  return PA_OK;
}

pa_status pa_bm_request_info(const pa_block_manager* bm, int64_t request_id, int64_t* info) {
  if (!bm || !info) return fail(PA_E_NULL, "bm and info are required");
  auto it = bm->reqs.find(request_id);
  if (it == bm->reqs.end()) return fail(PA_E_REQUEST, "unknown request " + id_str(request_id));
  const Request& r = it->second;
  info[0] = static_cast<int64_t>(r.tokens.size());
  info[1] = r.computed;
  info[2] = r.hit_tokens;
  info[3] = static_cast<int64_t>(r.blocks.size());
  return PA_OK;
}

pa_status pa_bm_block_state(const pa_block_manager* bm, int32_t block, int32_t* ref_count, int32_t* free_position) {
  if (!bm || !ref_count || !free_position) return fail(PA_E_NULL, "bm, ref_count and free_position are required");
  if (block < 0 || block >= bm->num_blocks) return fail(PA_E_SHAPE, "block " + std::to_string(block) + " out of range");
  *ref_count = bm->ref[block];
  int32_t pos = -1;
  if (bm->in_free[block]) {
    pos = 0;
    for (int32_t b = bm->head; b != block; b = bm->next[b]) ++pos;
  }
  *free_position = pos;
  return PA_OK;
}

}  // extern "C"
