// Randomised host test of the metadata packers (pack.cpp) and the
// BlockManager (block_manager.cpp), built with AddressSanitizer and UBSan by
// tests/test_host_sanitizers.py. Packers: random batches (block sizes 1..256,
// ragged and empty sequences, too-short tables, invalid lengths, undersized
// buffers) -- every slot equals block_table[p / bs] * bs + p % bs, positions,
// prefix sums and -1 table padding are checked. BlockManager: random
// allocate / append / deallocate / gather sequences with shared prefixes, in
// the scheduler's order -- free blocks plus distinct blocks in use always
// equal the pool size. Usage: host_fuzz <packer iterations> <manager runs>.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
#include <map>
#include "pkv.h"
int pkv_internal_fail(int code, const char *) { return code; }
static std::mt19937_64 rng(12345);
static int ri(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "CHECK failed %s:%d %s \n", __FILE__, __LINE__, #c); std::abort(); } } while (0)

static void fuzz_pack(int iters) {
    for (int it = 0; it < iters; ++it) {
        const bool prefill = ri(0, 1);
        const int n = ri(0, 40);
        const int bs = std::vector<int>{1, 2, 16, 64, 256}[ri(0, 4)];
        std::vector<int32_t> lens(n), cached(n);
        std::vector<int64_t> off(n + 1, 0);
        std::vector<int32_t> ids;
        for (int s = 0; s < n; ++s) {
            lens[s] = prefill ? ri(0, 3000) : ri(1, 3000);
            cached[s] = prefill ? ri(0, lens[s]) : lens[s] - 1;
            int need = (lens[s] + bs - 1) / bs;
            int have = need + ri(0, 3);
            if (ri(0, 30) == 0) have = std::max(0, need - 1);   // sometimes too short
            for (int i = 0; i < have; ++i) ids.push_back(ri(0, 100000));
            off[s + 1] = off[s] + have;
        }
        if (n && ri(0, 40) == 0) lens[ri(0, n - 1)] = -5;          // sometimes invalid
        pkv_batch_layout L;
        int rc = prefill ? pkv_plan_prefill(n, lens.data(), cached.data(), off.data(), bs, &L)
                         : pkv_plan_decode(n, lens.data(), off.data(), bs, &L);
        if (rc != PKV_OK) continue;
        size_t bytes = (size_t)L.total_bytes;
        if (ri(0, 20) == 0 && bytes > 0) bytes -= 1;                // sometimes too small
        std::vector<unsigned char> buf(bytes ? bytes : 1);
        rc = prefill ? pkv_pack_prefill(n, lens.data(), cached.data(), ids.data(), off.data(), bs, &L, buf.data(), bytes)
                     : pkv_pack_decode(n, lens.data(), ids.data(), off.data(), bs, &L, buf.data(), bytes);
        if (rc != PKV_OK) { CHECK(bytes < (size_t)L.total_bytes || rc != PKV_OK); continue; }
        // slot formula and positions
        const int32_t *slots = (const int32_t *)(buf.data() + L.off_slot_mapping);
        const int32_t *pos = (const int32_t *)(buf.data() + L.off_positions);
        int k = 0;
        for (int s = 0; s < n; ++s) {
            int b0 = prefill ? cached[s] : lens[s] - 1;
            for (int p = b0; p < lens[s]; ++p, ++k) {
                CHECK(slots[k] == ids[off[s] + p / bs] * bs + p % bs);
                CHECK(pos[k] == p);
            }
        }
        CHECK(k == L.num_slots);
        if (prefill) {
            const int32_t *cq = (const int32_t *)(buf.data() + L.off_cu_seqlens_q);
            const int32_t *ck = (const int32_t *)(buf.data() + L.off_cu_seqlens_k);
            CHECK(cq[0] == 0 && ck[0] == 0);
            for (int s = 0; s < n; ++s) { CHECK(cq[s + 1] - cq[s] == lens[s] - cached[s]); CHECK(ck[s + 1] - ck[s] == lens[s]); }
        }
        if (L.off_block_tables >= 0) {
            const int32_t *bt = (const int32_t *)(buf.data() + L.off_block_tables);
            for (int s = 0; s < n; ++s)
                for (int j = 0; j < L.max_blocks_per_seq; ++j) {
                    int64_t have = off[s + 1] - off[s];
                    int need = (lens[s] + bs - 1) / bs;
                    int32_t v = bt[(int64_t)s * L.max_blocks_per_seq + j];
                    if (j < need) CHECK(v == ids[off[s] + j]);
                    else CHECK(v == -1 || (j < have && v == ids[off[s] + j]));
                }
        }
    }
}

static void fuzz_bm(int iters) {
    for (int it = 0; it < iters; ++it) {
        const int nb = ri(1, 200), bs = std::vector<int>{1, 2, 4, 16}[ri(0, 3)];
        pkv_block_manager *m = nullptr;
        CHECK(pkv_bm_create(nb, bs, &m) == PKV_OK);
        std::map<int64_t, std::vector<int64_t>> live;
        std::vector<int64_t> prefix;
        for (int i = 0; i < 64; ++i) prefix.push_back(ri(0, 50));
        for (int op = 0; op < 400; ++op) {
            int what = ri(0, 9);
            if (what <= 2) {
                int64_t id = ri(0, 30);
                int len = ri(0, 120);
                std::vector<int64_t> toks;
                int shared = ri(0, std::min<int>(len, 64));
                for (int i = 0; i < len; ++i) toks.push_back(i < shared ? prefix[i] : ri(0, 50));
                int32_t cached = -1;
                int rc = pkv_bm_allocate(m, id, toks.data(), len, &cached);
                if (rc == PKV_OK) { CHECK(!live.count(id)); CHECK(cached >= 0 && cached % bs == 0 && cached <= len); live[id] = toks; }
            } else if (what <= 5 && !live.empty()) {
                auto itr = live.begin(); std::advance(itr, ri(0, (int)live.size() - 1));
                // scheduler order: the sampled token is appended, then the next
                // step checks and reserves room for its KV (or preempts)
                int64_t tok = ri(0, 50);
                CHECK(pkv_bm_append_token(m, itr->first, tok) == PKV_OK);
                itr->second.push_back(tok);
                if (pkv_bm_can_append(m, itr->first) == 1) {
                    CHECK(pkv_bm_may_append(m, itr->first) == PKV_OK);
                } else {
                    CHECK(pkv_bm_deallocate(m, itr->first) == PKV_OK);
                    live.erase(itr);
                }
            } else if (what <= 7 && !live.empty()) {
                auto itr = live.begin(); std::advance(itr, ri(0, (int)live.size() - 1));
                CHECK(pkv_bm_deallocate(m, itr->first) == PKV_OK);
                live.erase(itr);
            } else if (!live.empty()) {
                std::vector<int64_t> ids; for (auto &kv : live) ids.push_back(kv.first);
                int n = (int)ids.size();
                std::vector<int32_t> lens(n), cached(n); std::vector<int64_t> off(n + 1);
                int64_t cap = ri(0, 1) ? 100000 : ri(0, 20);
                std::vector<int32_t> bt(cap ? cap : 1);
                int rc = pkv_bm_gather(m, n, ids.data(), lens.data(), cached.data(), off.data(), bt.data(), cap);
                if (rc == PKV_OK) for (int s = 0; s < n; ++s) {
                    CHECK(lens[s] == (int)live[ids[s]].size());
                    CHECK(off[s + 1] - off[s] == (lens[s] + bs - 1) / bs);
                    std::vector<int32_t> t(off[s + 1] - off[s] + 1);
                    int32_t got = pkv_bm_block_table(m, ids[s], t.data(), (int32_t)t.size());
                    CHECK(got == off[s + 1] - off[s]);
                    for (int j = 0; j < got; ++j) CHECK(t[j] == bt[off[s] + j] && t[j] >= 0 && t[j] < nb);
                }
            }
            // invariant: free + distinct blocks in use == nb
            std::map<int32_t, int> used;
            for (auto &kv : live) { std::vector<int32_t> t(200); int32_t g = pkv_bm_block_table(m, kv.first, t.data(), 200); CHECK(g >= 0); for (int j = 0; j < g; ++j) used[t[j]]++; }
            CHECK(pkv_bm_num_free(m) + (int)used.size() == nb);
        }
        pkv_bm_destroy(m);
    }
}

int main(int argc, char **argv) {
    fuzz_pack(argc > 1 ? atoi(argv[1]) : 3000);
    fuzz_bm(argc > 2 ? atoi(argv[2]) : 300);
    // hash smoke
    int64_t t[3] = {1, 2, 3};
    (void)pkv_block_hash(t, 3, 0, 0); (void)pkv_block_hash(t, 0, 1, 7); (void)pkv_xxh64(nullptr, 0, 0);
    printf("host fuzz ok\n");
    return 0;
}
