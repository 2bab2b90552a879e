// block_manager.cpp -- host-side paged KV block manager with a hashed prefix
// cache, producing the block tables and cached-token counts that the packer
// (pack.cpp) turns into kernel metadata.
//
// Semantics follow "nano-vLLM-1" (BlockManager sections "1. Block", "2.
// BlockManager 初始化与链式哈希", "3. 核心方法一：分配 (allocate)", "4. 核心方法二：
// 追加 (may_append)", "5. 核心方法三：回收块 (deallocate)", "6. 辅助查询方法") and
// "【nano-vllm 学习】04 …", "PageAttention / 内/显存管理":
//  - a pool of num_blocks blocks of block_size tokens; free blocks wait in a
//    FIFO (taken from the front, returned to the back), a block is in use
//    while its reference count is positive;
//  - a full block is identified by a chained 64-bit hash: xxh64 (seed 0) over
//    the previous block's hash as 8 little-endian bytes (absent for the first
//    block) followed by the block's token ids as little-endian int64; the hash
//    table maps hashes to blocks, and a hit is only taken after comparing the
//    block's recorded tokens (a collision is a miss) and its recorded hash:
//    a freed block later reused under another prefix chain keeps an entry
//    under its old hash and may hold the same tokens, but its KV was computed
//    in the other context, so that stale entry must miss too;
//  - a new sequence's cached prefix is the longest run of its leading full
//    blocks whose chained hash is registered to a block holding exactly those
//    tokens. Those blocks are shared (one more holder each; a block nobody
//    held comes back out of the free FIFO with its K/V intact) and count as
//    cached tokens. Every later block is fresh from the front of the FIFO,
//    and the fresh full ones are registered;
//  - before a decode step writes the KV of a sequence's newest token (at
//    position len - 1), the sequence gets a new block when that position
//    lies past its table, and the block is hashed and registered when that
//    position is the block's last;
//  - deallocation drops one reference per block, last block first; blocks
//    reaching zero return to the back of the FIFO but keep their hash and
//    tokens, so a later allocation of the same prefix can still hit them.
// The pages' assertions become status codes; an allocation that might not
// fit fails before changing anything.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

int pkv_internal_fail(int code, const char *msg);

// ---------------------------------------------------------------------------
// XXH64, written from the xxHash specification (Yann Collet, "xxHash fast
// digest algorithm", XXH64 section): 32-byte stripes into four accumulators,
// then the tail in 8-, 4- and 1-byte steps, then the avalanche.
namespace {

constexpr uint64_t kP1 = 0x9E3779B185EBCA87ULL;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4FULL;
constexpr uint64_t kP3 = 0x165667B19E3779F9ULL;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ULL;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ULL;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t le64(const uint8_t *p) {
    uint64_t v = 0;
    for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
inline uint32_t le32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
inline uint64_t xx_round(uint64_t acc, uint64_t lane) {
    acc += lane * kP2;
    return rotl(acc, 31) * kP1;
}
inline uint64_t xx_merge(uint64_t acc, uint64_t v) {
    acc ^= xx_round(0, v);
    return acc * kP1 + kP4;
}

uint64_t xxh64(const void *data, size_t len, uint64_t seed) {
    const uint8_t *p = (const uint8_t *)data, *end = p + len;
    uint64_t acc;
    if (len >= 32) {
        uint64_t v1 = seed + kP1 + kP2, v2 = seed + kP2, v3 = seed, v4 = seed - kP1;
        for (; p + 32 <= end; p += 32) {
            v1 = xx_round(v1, le64(p));
            v2 = xx_round(v2, le64(p + 8));
            v3 = xx_round(v3, le64(p + 16));
            v4 = xx_round(v4, le64(p + 24));
        }
        acc = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
        acc = xx_merge(acc, v1);
        acc = xx_merge(acc, v2);
        acc = xx_merge(acc, v3);
        acc = xx_merge(acc, v4);
    } else {
        acc = seed + kP5;
    }
    acc += (uint64_t)len;
    for (; p + 8 <= end; p += 8) {
        acc ^= xx_round(0, le64(p));
        acc = rotl(acc, 27) * kP1 + kP4;
    }
    if (p + 4 <= end) {
        acc ^= (uint64_t)le32(p) * kP1;
        acc = rotl(acc, 23) * kP2 + kP3;
        p += 4;
    }
    for (; p < end; ++p) {
        acc ^= (uint64_t)(*p) * kP5;
        acc = rotl(acc, 11) * kP1;
    }
    acc ^= acc >> 33;
    acc *= kP2;
    acc ^= acc >> 29;
    acc *= kP3;
    acc ^= acc >> 32;
    return acc;
}

// Chained hash of one full block.
uint64_t block_hash(const int64_t *tokens, int32_t n, bool has_prefix, uint64_t prefix) {
    std::vector<uint8_t> buf((has_prefix ? 8 : 0) + (size_t)n * 8);
    uint8_t *w = buf.data();
    if (has_prefix) {
        for (int i = 0; i < 8; ++i) *w++ = (uint8_t)(prefix >> (8 * i));
    }
    for (int32_t t = 0; t < n; ++t) {
        const uint64_t v = (uint64_t)tokens[t];
        for (int i = 0; i < 8; ++i) *w++ = (uint8_t)(v >> (8 * i));
    }
    return xxh64(buf.data(), buf.size(), 0);
}

struct Block {
    int32_t ref = 0;
    bool hashed = false;   // a full block whose hash and tokens are recorded
    uint64_t hash = 0;
    std::vector<int64_t> tokens;
    int32_t prev = -1, next = -1;   // links in the free FIFO
    bool in_free = false;
};

struct SeqState {
    std::vector<int64_t> tokens;
    std::vector<int32_t> table;
    int32_t num_cached = 0;
};

}  // namespace

struct pkv_block_manager {
    int32_t num_blocks = 0, block_size = 0;
    std::vector<Block> blocks;
    int32_t free_head = -1, free_tail = -1, num_free = 0;
    std::unordered_map<uint64_t, int32_t> by_hash;
    std::unordered_map<int64_t, SeqState> seqs;

    void push_back_free(int32_t b) {
        Block &x = blocks[b];
        x.prev = free_tail;
        x.next = -1;
        x.in_free = true;
        if (free_tail >= 0) blocks[free_tail].next = b;
        else free_head = b;
        free_tail = b;
        ++num_free;
    }
    void unlink_free(int32_t b) {
        Block &x = blocks[b];
        if (x.prev >= 0) blocks[x.prev].next = x.next;
        else free_head = x.next;
        if (x.next >= 0) blocks[x.next].prev = x.prev;
        else free_tail = x.prev;
        x.prev = x.next = -1;
        x.in_free = false;
        --num_free;
    }
    // A free block handed to a sequence: one reference, no hash yet.
    void take(int32_t b) {
        unlink_free(b);
        Block &x = blocks[b];
        x.ref = 1;
        x.hashed = false;
        x.tokens.clear();
    }
    // A free block whose K/V a new holder reuses: it leaves the FIFO and keeps
    // its registration.
    void revive(int32_t b) {
        unlink_free(b);
        blocks[b].ref = 1;
    }
    void record(int32_t b, uint64_t h, const int64_t *tok, int32_t n) {
        Block &x = blocks[b];
        x.hashed = true;
        x.hash = h;
        x.tokens.assign(tok, tok + n);
        by_hash[h] = b;
    }
    // The block registered under hash h, if it still holds exactly these
    // tokens under that hash (a hash collision or a stale entry is a miss).
    int32_t lookup(uint64_t h, const int64_t *tok, int32_t n) const {
        auto it = by_hash.find(h);
        if (it == by_hash.end()) return -1;
        const Block &c = blocks[it->second];
        const bool same = c.hashed && c.hash == h && c.tokens.size() == (size_t)n &&
                          memcmp(c.tokens.data(), tok, (size_t)n * 8) == 0;
        return same ? it->second : -1;
    }
    int32_t blocks_for(int64_t len) const { return (int32_t)((len + block_size - 1) / block_size); }
};

extern "C" uint64_t pkv_xxh64(const void *data, size_t len, uint64_t seed) {
    return xxh64(data, len, seed);
}

extern "C" uint64_t pkv_block_hash(const int64_t *token_ids, int32_t num_tokens,
                                   int32_t has_prefix, uint64_t prefix) {
    return block_hash(token_ids, num_tokens < 0 ? 0 : num_tokens, has_prefix != 0, prefix);
}

extern "C" int pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager **out) {
    if (!out || num_blocks <= 0 || block_size <= 0)
        return pkv_internal_fail(PKV_EINVAL, "pkv_bm_create: need positive sizes and an out pointer");
    pkv_block_manager *m = new (std::nothrow) pkv_block_manager;
    if (!m) return pkv_internal_fail(PKV_ENOSPACE, "pkv_bm_create: out of host memory");
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->blocks.resize(num_blocks);
    for (int32_t b = 0; b < num_blocks; ++b) m->push_back_free(b);
    *out = m;
    return PKV_OK;
}

extern "C" void pkv_bm_destroy(pkv_block_manager *m) { delete m; }

extern "C" int32_t pkv_bm_num_free(const pkv_block_manager *m) { return m ? m->num_free : -1; }

extern "C" int pkv_bm_can_allocate(const pkv_block_manager *m, int32_t num_tokens) {
    return m && num_tokens >= 0 && m->num_free >= m->blocks_for(num_tokens);
}

extern "C" int pkv_bm_allocate(pkv_block_manager *m, int64_t seq_id, const int64_t *token_ids,
                               int32_t num_tokens, int32_t *num_cached_tokens) {
    if (!m || num_tokens < 1 || !token_ids)
        return pkv_internal_fail(PKV_EINVAL, "pkv_bm_allocate: bad arguments");
    if (m->seqs.count(seq_id)) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_allocate: sequence already holds blocks");
    const int32_t bs = m->block_size;
    const int32_t nb = m->blocks_for(num_tokens);
    const int32_t nfull = (int32_t)(num_tokens / bs);   // blocks the prompt fills completely
    // The worst case (no hit) must fit before anything changes.
    if (m->num_free < nb) return pkv_internal_fail(PKV_ENOSPACE, "pkv_bm_allocate: not enough free blocks");

    // 1. The identity of every full block: its hash chained to the block before.
    std::vector<uint64_t> ident((size_t)nfull);
    for (int32_t i = 0; i < nfull; ++i)
        ident[i] = block_hash(token_ids + (int64_t)i * bs, bs, i > 0, i > 0 ? ident[i - 1] : 0);

    // 2. The cached prefix: the longest run of leading full blocks whose
    //    identity is registered to a block holding exactly these tokens.
    SeqState st;
    st.tokens.assign(token_ids, token_ids + num_tokens);
    st.table.reserve(nb);
    int32_t shared = 0;
    for (; shared < nfull; ++shared) {
        const int32_t b = m->lookup(ident[shared], token_ids + (int64_t)shared * bs, bs);
        if (b < 0) break;
        st.table.push_back(b);
    }

    // 3. Claim the prefix: one more holder per block; a block nobody held
    //    leaves the free FIFO (its K/V is still valid, so it is reused as is).
    for (int32_t b : st.table) {
        if (m->blocks[b].ref > 0) ++m->blocks[b].ref;
        else m->revive(b);
    }
    st.num_cached = shared * bs;

    // 4. The rest are fresh blocks from the front of the FIFO. The full ones
    //    are registered, so that a later prompt with this prefix finds them.
    for (int32_t i = shared; i < nb; ++i) {
        const int32_t b = m->free_head;
        m->take(b);
        if (i < nfull) m->record(b, ident[i], token_ids + (int64_t)i * bs, bs);
        st.table.push_back(b);
    }
    if (num_cached_tokens) *num_cached_tokens = st.num_cached;
    m->seqs.emplace(seq_id, std::move(st));
    return PKV_OK;
}

extern "C" int pkv_bm_append_token(pkv_block_manager *m, int64_t seq_id, int64_t token_id) {
    if (!m) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_append_token: null manager");
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_append_token: unknown sequence");
    it->second.tokens.push_back(token_id);
    return PKV_OK;
}

extern "C" int pkv_bm_can_append(const pkv_block_manager *m, int64_t seq_id) {
    if (!m) return 0;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return 0;
    const SeqState &st = it->second;
    const bool opens = m->blocks_for((int64_t)st.tokens.size()) > (int32_t)st.table.size();
    return m->num_free >= (opens ? 1 : 0);
}

extern "C" int pkv_bm_may_append(pkv_block_manager *m, int64_t seq_id) {
    if (!m) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_may_append: null manager");
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_may_append: unknown sequence");
    SeqState &st = it->second;
    const int32_t bs = m->block_size;
    if (st.table.empty() || st.tokens.empty())
        return pkv_internal_fail(PKV_EINVAL, "pkv_bm_may_append: sequence has no blocks");
    // Where the newest token's K/V goes: logical block lb, offset off in it.
    const int64_t pos = (int64_t)st.tokens.size() - 1;
    const int64_t lb = pos / bs;
    const int32_t off = (int32_t)(pos % bs);
    const int64_t have = (int64_t)st.table.size();
    if (lb == have) {
        // A block past the table: the one before must be complete, and a
        // fresh block is needed for this token.
        if (!m->blocks[st.table.back()].hashed)
            return pkv_internal_fail(PKV_EINVAL, "pkv_bm_may_append: last block not complete");
        if (m->num_free < 1) return pkv_internal_fail(PKV_ENOSPACE, "pkv_bm_may_append: no free block");
        const int32_t b = m->free_head;
        m->take(b);
        st.table.push_back(b);
    } else if (lb != have - 1) {
        return pkv_internal_fail(PKV_EINVAL, "pkv_bm_may_append: sequence length out of step with its blocks");
    }
    const int32_t cur = st.table.back();
    if (m->blocks[cur].hashed)
        return pkv_internal_fail(PKV_EINVAL, "pkv_bm_may_append: last block already complete");
    if (off == bs - 1) {
        // This token completes its block: register it under its chained
        // identity so that a later prompt sharing these tokens can reuse it.
        const bool chained = lb > 0;
        const uint64_t before = chained ? m->blocks[st.table[lb - 1]].hash : 0;
        const int64_t *tok = st.tokens.data() + lb * bs;
        m->record(cur, block_hash(tok, bs, chained, before), tok, bs);
    }
    return PKV_OK;
}

extern "C" int pkv_bm_deallocate(pkv_block_manager *m, int64_t seq_id) {
    if (!m) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_deallocate: null manager");
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_deallocate: unknown sequence");
    // Released tail first: a sequence's leading blocks -- the ones other
    // prompts are most likely to share -- reach the back of the FIFO last and
    // are therefore the last to be handed out again (and lose their K/V).
    const std::vector<int32_t> &t = it->second.table;
    std::for_each(t.rbegin(), t.rend(), [m](int32_t b) {
        if (--m->blocks[b].ref == 0) m->push_back_free(b);
    });
    m->seqs.erase(it);
    return PKV_OK;
}

extern "C" int32_t pkv_bm_block_table(const pkv_block_manager *m, int64_t seq_id, int32_t *out,
                                      int32_t capacity) {
    if (!m) return -1;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return -1;
    const std::vector<int32_t> &t = it->second.table;
    if (out && capacity >= (int32_t)t.size()) memcpy(out, t.data(), t.size() * 4);
    return (int32_t)t.size();
}

extern "C" int pkv_bm_gather(const pkv_block_manager *m, int32_t num_seqs, const int64_t *seq_ids,
                             int32_t *seq_lens, int32_t *num_cached_tokens,
                             int64_t *bt_offsets, int32_t *bt_ids, int64_t bt_capacity) {
    if (!m || num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !seq_lens || !bt_offsets)))
        return pkv_internal_fail(PKV_EINVAL, "pkv_bm_gather: bad arguments");
    int64_t at = 0;
    if (bt_offsets) bt_offsets[0] = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        auto it = m->seqs.find(seq_ids[s]);
        if (it == m->seqs.end()) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_gather: unknown sequence");
        const SeqState &st = it->second;
        if (st.tokens.size() > (size_t)INT32_MAX) return pkv_internal_fail(PKV_EINVAL, "pkv_bm_gather: sequence too long");
        seq_lens[s] = (int32_t)st.tokens.size();
        if (num_cached_tokens) num_cached_tokens[s] = st.num_cached;
        if (at + (int64_t)st.table.size() > bt_capacity)
            return pkv_internal_fail(PKV_ENOSPACE, "pkv_bm_gather: block-table buffer too small");
        if (bt_ids) memcpy(bt_ids + at, st.table.data(), st.table.size() * 4);
        at += (int64_t)st.table.size();
        bt_offsets[s + 1] = at;
    }
    return PKV_OK;
}
