// prefill.hip -- varlen causal prefill attention over a flattened ragged batch.
//
// Sequence s owns query rows [cu_q[s], cu_q[s+1]) and keys [0, Lk); query i
// sits at position Lk - Lq + i and sees keys up to it ("Nano vLLM 解读（5）：
// 解析 ModelRunner", "FlashAttention Kernel 函参准备" and "prepare_prefill";
// "nano-vLLM-1", "4. prefill 输入打包": positions start at num_cached_tokens).
// Keys come from the call's contiguous k/v rows, or -- on a prefix-cache hit
// -- from the pool through the block table ("nano-vLLM-1", "5. deocde 输入打包",
// the block_table difference between prefill and decode). The result is
// softmax(scale * Q K^T + causal mask) V ("【nano-vllm 学习】04 - …源码学习2",
// "KV-Cache … 是什么？").
//
// prefill_mfma_kernel (bf16, head_dim 128) is a FlashAttention-2 style forward
// (Dao, 2023) laid out for CDNA4: a workgroup of 4 waves owns 128 query rows of
// one head (32 per wave) -- or, when every sequence is short, 64 or 32 rows of
// each of 2 or 4 query heads of a GQA group, which then share every staged
// K/V tile -- and streams 64-key tiles of K and V through two LDS
// buffers (the next tile's global loads are in flight while the current one
// is computed; one barrier per tile). Two workgroups per CU, so two waves
// share each SIMD: while one waits on LDS or runs its softmax on the VALU,
// the other keeps the matrix core busy. Both contractions run on
// v_mfma_f32_32x32x16_bf16 in the transposed form
//     S^T = K Q^T        (keys as MFMA rows, the wave's queries as columns)
//     O^T += V^T P^T     (head dims as rows, queries as columns)
// so that every lane owns one query row: the row max needs a single
// cross-lane exchange, the rescale by exp2(m_old - m_new) is lane-local, and
// P^T is fed to the second MFMA straight from the registers the first one
// produced. V stays row-major in LDS; the V^T operand comes from the gfx950
// transpose read (ds_read_b64_tr_b16), two reads of 4 consecutive keys per
// MFMA. A wave skips key tiles that lie entirely above its causal diagonal.
#include <stdlib.h>

#include <type_traits>
#include <utility>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kPfD = 128;
constexpr int kPfBN = 64;      // keys per tile
constexpr float kLazy = 8.f;   // log2 headroom before the running max is moved
// Persistent prefill grid: the largest per-XCD pair count and query-block
// count whose item tables fit in LDS (larger batches take the fixed grid).
constexpr int kPfMaxXcdPairs = 256;
constexpr int kPfMaxQblocks = 512;

// Element offset of key `key` of sequence s in its source (k rows or the
// pool), for kv head kvh; -1 when the table entry is outside the pool.
__device__ __forceinline__ int64_t prefill_key_off(const PrefillArgs &a, int s, int k_start,
                                                   int key, int kvh, int D) {
    if (!a.paged) return (int64_t)(k_start + key) * a.kv_stride + (int64_t)kvh * D;
    const int lb = key >> a.log2bs;
    if (lb >= a.maxb) return -1;
    const int blk = a.bt[(int64_t)s * a.maxb + lb];
    if (blk < 0 || blk >= a.num_blocks) return -1;
    const int64_t row = (int64_t)blk * a.bs + (key & (a.bs - 1));
    return (row * a.Hkv + kvh) * D;
}

// Where a 64-key tile of K/V comes from.
enum KeySource {
    kContiguous = 0,   // the call's k/v rows: one descriptor per tile
    kPoolBlocks = 1,   // the pool, block_size a multiple of 64: one descriptor per tile
    kPoolSmall = 2,    // the pool, block_size 4 or 8: one descriptor per 4 keys
    kPoolWave = 3      // the pool, block_size 16 or 32: one descriptor per wave's 16 keys
};

// LDS tile layout: 64 keys x 256 bytes, no padding; the 16-byte chunk c of key
// row t sits at chunk position c ^ tile_swz(t). With this swizzle the K
// operand reads (16 rows, one chunk each) and the V transpose reads (4 rows x
// 4 chunks per 32 lanes) each touch 16 distinct chunk positions, so neither
// has LDS bank conflicts.
__device__ __forceinline__ int tile_swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

// Maximum of three scores (IEEE maximum, one v_maximum3_f32).
__device__ __forceinline__ float fmax3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// A wave's direct loads of one tile operand from one descriptor: load i
// lands 1024*i bytes past the LDS base d and reads 1024*i bytes past
// voff[i] (the instruction offset moves both addresses).
template <int... I>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, __attribute__((address_space(3))) void *d,
                                         const int (&voff)[8], std::integer_sequence<int, I...>) {
    (__builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, voff[I], 0, 1024 * I, 0), ...);
}

// NW waves per workgroup, RB blocks of 32 query rows per wave. HPW query
// heads of one GQA group share the workgroup and every K/V tile it stages,
// NW / HPW waves each: the workgroup owns BM = 32 * RB * NW / HPW rows of each
// of its heads. WPE waves share one SIMD.
// STORE: store_kvcache fused into the attention launch. Each query block
// also copies its own rows of the call's k/v into the cache (shared out over
// the group's query heads), and keys at positions Lk - Lq and beyond -- the
// ones this call stores -- are read from those rows rather than the pool.
template <int SRC, int NW, int RB, int WPE, bool PERSIST, bool STORE, int HPW>
__device__ __forceinline__ void prefill_mfma_body(const PrefillArgs &a) {
    static_assert(!STORE || (RB == 1 && !PERSIST && SRC != kPoolSmall),
                  "the fused store is built for the fixed grid and tiles of whole 16-key slices");
    static_assert(HPW == 1 || (!STORE && !PERSIST && NW % HPW == 0),
                  "heads share a workgroup on the fixed grid of the attention-only kernel");
    constexpr int WPH = NW / HPW;            // waves per query head
    constexpr int BM = 32 * RB * WPH;        // query rows per workgroup and head
    constexpr int LPW = 16 / NW;   // 1 KiB direct-load instructions per wave per K (or V) tile
    static_assert(NW * LPW == 16 && NW >= 2, "waves must split a tile evenly");
    static_assert(RB == 1 || RB == 2, "row blocks per wave");
    // Arrays that the lambdas below capture are sized for the largest shape
    // (RB 2, LPW 8): clang does not emit the host launch stub of a kernel
    // whose lambdas capture arrays of template-dependent size. Only the
    // first RB (LPW) entries are ever touched.
    // Two buffers, each a K tile followed by a V tile, 64 keys x 256 bytes each.
    constexpr int kTileBytes = kPfBN * 256;
    // One LDS object: the tile buffers, then (persistent grid) its item
    // tables. With the tables in objects of their own the compiler stopped
    // telling the direct tile loads apart from the operand reads of the other
    // buffer, and waited for every load before each tile's reads.
    constexpr int kTabWords = PERSIST ? 3 * 256 + 512 + 2 : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_all[2 * 2 * kTileBytes + 4 * kTabWords];
    auto lds = reinterpret_cast<uint8_t (*)[2 * kTileBytes]>(lds_all);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Work order, XCD-aware. The hardware deals a launch's workgroups to the 8
    // XCDs round robin (starting wherever the previous launch left off), so
    // workgroups with equal p % 8 run on one XCD, and each XCD has its own
    // L2. Work is grouped by (sequence, kv head) pair, the unit that shares K
    // and V; pair pi runs on the XCD of class pi % 8, so all query blocks and
    // all query heads of that kv head read their K/V tiles through one L2. Two orders within an XCD, chosen on the host from the batch's
    // K/V bytes (a bound on them when the keys come through block tables):
    //  - K/V within half the 256 MB MALL: longest first across all the XCD's
    //    pairs (query-block rank major), so the tail holds only short blocks;
    //  - larger: pair by pair, each pair's longest blocks first, so only a few
    //    pairs' K/V are live at a time.
    // Either way the group's heads sit side by side and every (pair, query
    // block, head) is visited once.
    const int HG = a.group / HPW;            // head groups per kv head
    const int qblocks = (a.max_seqlen_q + BM - 1) / BM;
    const int npairs = a.num_seqs * a.Hkv;
    const int xcd = blockIdx.x & 7;
    const int hh = wave / WPH, wh = wave - hh * WPH;   // the wave's head in the group, its place in the head's rows

    // Persistent grid: the claim of the next item, issued by thread 0 once an
    // item's tile loop is done (so that the per-tile waits for vector memory
    // do not wait for it) and published after the item.
    uint32_t next_claim = 0;
    uint32_t *const claim_ctr = PERSIST ? a.work_ctr + xcd : nullptr;

    // One work item: query block qt of (sequence, kv head) pair `pair`, head group hg.
    auto run_item = [&](const int pair, const int qt, const int hg) {
    const int s = pair / a.Hkv;
    const int kvh = pair - s * a.Hkv;
    const int h = kvh * a.group + hg * HPW + hh;
    // Block-table entries are read through the scalar cache (a wave-uniform
    // index) one tile ahead of the loads that use them: a vector load here
    // would make every tile step wait for it (vmcnt counts in order) before
    // it could issue the next tile's loads. The first tile's entries go out
    // with the sequence bounds, before the key count is known (any entry of
    // the sequence's table row may be read), and count only for keys that
    // exist.
    typedef const __attribute__((address_space(4))) int32_t *bt_ptr;
    const bt_ptr bt_row = (bt_ptr)(a.bt + (int64_t)s * a.maxb);
    constexpr int NB = SRC == kPoolSmall ? LPW : 1;   // block ids per wave and tile
    // first key of block-id slot i of the wave in tile k0
    auto key_of = [&](int k0, int i) {
        return SRC == kPoolSmall ? k0 + 4 * (LPW * wave + i) : SRC == kPoolWave ? k0 + 4 * LPW * wave : k0;
    };
    // All four bounds in one round trip (a workgroup with no rows here
    // learns it from the first two and leaves).
    const int q_start = a.cu_q[s], q_end = a.cu_q[s + 1];
    const int k_start = a.cu_k[s], k_end = a.cu_k[s + 1];
    int first_blk[8];
    if constexpr (SRC != kContiguous) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int lb = key_of(0, i) >> a.log2bs;
            first_blk[i] = lb < a.maxb ? bt_row[lb] : -1;
        }
    }
    const int Lq = q_end - q_start, Lk = k_end - k_start;
    const int q0 = qt * BM;
    // One test, so that the four loads above issue together. Rows outside
    // [0, total_q) of q and out are never touched, whatever cu_seqlens_q
    // holds; keys must number between Lq and the host's max_seqlen_k (which
    // bounds the work); contiguous keys are this call's rows (Lk == Lq), so
    // they too lie in [0, total_q).
    const bool skip = (q0 >= Lq) | (q_start < 0) | (q_start > a.total_q - Lq) | (Lk < Lq) |
                      (Lk > a.max_seqlen_k) |
                      (SRC == kContiguous && ((k_start < 0) | (k_start > a.total_q - Lk)));
    if (skip) return;
    const int off = Lk - Lq;
    const int r32 = lane & 31, j = lane >> 5;
    // The wave owns rows q0 + 32*RB*wh + 32*rb + r32, rb < RB.
    int my_pos[2];
    bool row_ok[2];
    bf16x8 qb[2][8];   // B operand of S^T = K Q^T: Q[row][d = 16*kk + 8*j .. +8]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = q0 + 32 * RB * wh + 32 * rb + r32;
        row_ok[rb] = row < Lq;
        my_pos[rb] = off + row;
        const uint16_t *q = (const uint16_t *)a.q + (int64_t)(q_start + row) * a.q_stride +
                            (int64_t)h * kPfD + 8 * j;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row_ok[rb]) w = ld16(q + 16 * kk);
            qb[rb][kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    // Fused store: the cache slot of the wave's row r32 (row i of q, k and v
    // is the same token), loaded with q; -1 for rows past the sequence.
    int my_slot = -1;
    if constexpr (STORE) {
        if (row_ok[0]) my_slot = a.slots[q_start + q0 + 32 * wh + r32];
    }
    const int kend = min(Lk, off + min(q0 + BM, Lq));   // keys this block needs
    const int n_kt = (kend + kPfBN - 1) / kPfBN;
    // Position of the wave's last row: tiles starting past it hold only masked
    // keys for this wave, which skips their arithmetic (not their loads). A
    // wave whose rows all lie past the sequence's end (the last query block of
    // a sequence, or a short one such as a decode row) skips all of it.
    const int pos_last = off + q0 + 32 * RB * (wh + 1) - 1;
    const bool wave_rows = q0 + 32 * RB * wh < Lq;

    // Tile loads go global -> LDS directly (buffer_load_dwordx4 ... lds), no
    // registers in between. Instruction i of wave w fills LDS bytes
    // [1024*(LPW*w+i), +1024) of a tile: keys 4*(LPW*w+i) + lane/16, chunk
    // position lane%16. Keys at or past kend are outside the descriptor's
    // range and arrive as zeros; a tile wholly past them gets a zero record
    // count, so the loads carry no branches (the step after the last tile
    // loads nothing and writes zeros into a buffer no one reads). With one
    // descriptor per tile, a wave's loads of one operand share one LDS base
    // (M0) and step through the tile with the instruction offset 1024*i,
    // which the hardware adds to both the LDS and the source address; it is
    // taken out of the per-lane source offset, which stays non-negative
    // since key rows are at least 256 bytes apart. Small blocks take one
    // descriptor per 4 keys and an LDS base per load. Record counts go
    // through readfirstlane: the clamps select to vector med3, and a
    // descriptor word in a vector register would put every load in a loop
    // over its distinct values.
    const uint8_t *kbase = (const uint8_t *)(SRC == kContiguous ? a.k : a.kc) + (int64_t)kvh * kPfD * 2;
    const uint8_t *vbase = (const uint8_t *)(SRC == kContiguous ? a.v : a.vc) + (int64_t)kvh * kPfD * 2;
    const uint32_t stride_b = (uint32_t)(SRC == kContiguous ? a.kv_stride * 2 : (int64_t)a.Hkv * kPfD * 2);
    auto blk_of = [&](int key0) -> int {   // block holding key key0; -1 past the keys or the table
        const int lb = key0 >> a.log2bs;
        return (key0 < kend && lb < a.maxb) ? bt_row[lb] : -1;
    };
    int pre_blk[8];   // block ids for the next load_tile: NB entries
    auto fetch_blocks = [&](int k0) {
        if constexpr (SRC != kContiguous) {
#pragma unroll
            for (int i = 0; i < NB; ++i) pre_blk[i] = blk_of(key_of(k0, i));
        }
    };
    int voff[8];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int t = 4 * (LPW * wave + i) + (lane >> 4);
        const int chunk = (lane & 15) ^ tile_swz(t);
        voff[i] = SRC == kPoolSmall  ? (lane >> 4) * (int)stride_b + 16 * chunk
                  : SRC == kPoolWave ? (t - 4 * LPW * wave) * (int)stride_b + 16 * chunk - 1024 * i
                                     : t * (int)stride_b + 16 * chunk - 1024 * i;
    }
    typedef __attribute__((address_space(3))) void lds_t;
    // Fused store over the pool: keys at positions off and beyond come from
    // the call's k/v rows (position p is row q_start + p - off), the rows
    // this call stores; the others from the pool. voff_n is voff for those
    // rows' stride.
    const uint8_t *knbase = (const uint8_t *)a.k + (int64_t)kvh * kPfD * 2;
    const uint8_t *vnbase = (const uint8_t *)a.v + (int64_t)kvh * kPfD * 2;
    const uint32_t stride_n = (uint32_t)(a.kv_stride * 2);
    int voff_n[8];
    if constexpr (STORE && SRC != kContiguous) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int t = 4 * (LPW * wave + i) + (lane >> 4);
            const int chunk = (lane & 15) ^ tile_swz(t);
            voff_n[i] = t * (int)stride_n + 16 * chunk - 1024 * i;
        }
    }
    // Descriptor over the call's rows from key `key0` on (the base may lie
    // before the sequence's first row when key0 < off: only lanes at keys
    // off and beyond use it), nk keys long.
    auto rows_rsrc = [&](const uint8_t *base, int key0, int nk) {
        const int nrec = __builtin_amdgcn_readfirstlane(max(0, nk) * (int)stride_n);
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)(base + ((int64_t)q_start + key0 - off) * stride_n), (short)0, nrec, kBufWord3);
    };
    auto load_tile = [&](int k0, uint8_t *dst) {
        uint8_t *kd = dst + 1024 * LPW * wave;
        uint8_t *vd = dst + kTileBytes + 1024 * LPW * wave;
        if constexpr (STORE && SRC != kContiguous) {
            if (k0 >= off) {
                // every key of the tile is this call's: its rows, as in the contiguous form
                const int nkeys = min(kPfBN, kend - k0);
                dma_tile(rows_rsrc(knbase, k0, nkeys), (lds_t *)kd, voff_n, std::make_integer_sequence<int, LPW>{});
                dma_tile(rows_rsrc(vnbase, k0, nkeys), (lds_t *)vd, voff_n, std::make_integer_sequence<int, LPW>{});
                return;
            }
            if (k0 + kPfBN > off) {
                // The tile holds both (at most one such tile per item): each
                // load goes out twice with complementary lane masks, cached
                // keys from the pool and the rest from the rows, each at its
                // own LDS base. Masked-off lanes neither read nor write LDS.
                const int nkeys = min(kPfBN, kend - k0);
#pragma unroll
                for (int i = 0; i < LPW; ++i) {
                    const int t = 4 * (LPW * wave + i) + (lane >> 4);
                    const int chunk = (lane & 15) ^ tile_swz(t);
                    const int key0 = k0 + 4 * (LPW * wave + i);
                    // the cached keys' descriptor: its first key (the tile's, or the
                    // wave's slice's), block, and keys in range
                    const int pk = key_of(k0, 0);
                    const int blk = pre_blk[0];
                    const int np = min(SRC == kPoolWave ? 4 * LPW : kPfBN, off - pk);
                    const bool ok = (uint32_t)blk < (uint32_t)a.num_blocks;
                    const int nrec = __builtin_amdgcn_readfirstlane(ok ? max(0, np) * (int)stride_b : 0);
                    const int64_t rb_ = ((int64_t)(ok ? blk : 0) * a.bs + (pk & (a.bs - 1))) * stride_b;
                    const int vo_p = (k0 + t - pk) * (int)stride_b + 16 * chunk;
                    const int vo_n = t * (int)stride_n + 16 * chunk;
                    if (k0 + t < off) {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + rb_), (short)0, nrec, kBufWord3),
                            (lds_t *)(kd + 1024 * i), 16, vo_p, 0, 0, 0);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + rb_), (short)0, nrec, kBufWord3),
                            (lds_t *)(vd + 1024 * i), 16, vo_p, 0, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(knbase, k0, nkeys), (lds_t *)(kd + 1024 * i), 16, vo_n, 0, 0, 0);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(vnbase, k0, nkeys), (lds_t *)(vd + 1024 * i), 16, vo_n, 0, 0, 0);
                    }
                }
                return;
            }
        }
        if constexpr (SRC == kPoolSmall) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int key0 = k0 + 4 * (LPW * wave + i);
                const int blk = pre_blk[i];
                const bool ok = (uint32_t)blk < (uint32_t)a.num_blocks;
                const int nrec = __builtin_amdgcn_readfirstlane(ok ? min(4, max(0, kend - key0)) * (int)stride_b : 0);
                const int64_t rb_ = ((int64_t)(ok ? blk : 0) * a.bs + (key0 & (a.bs - 1))) * stride_b;
                const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + rb_), (short)0, nrec, kBufWord3);
                const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + rb_), (short)0, nrec, kBufWord3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_t *)(kd + 1024 * i), 16, voff[i], 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_t *)(vd + 1024 * i), 16, voff[i], 0, 0, 0);
            }
        } else {
            // kPoolWave: the same with the wave's 16 keys (one block) as the tile
            const int kw0 = key_of(k0, 0);
            const int nkeys = min(SRC == kPoolWave ? 4 * LPW : kPfBN, max(0, kend - kw0));
            int64_t row0;   // first key row of the tile (or the wave's slice) in its source
            bool ok = true;
            if constexpr (SRC == kContiguous) {
                row0 = (int64_t)k_start + k0;
            } else {
                const int blk = pre_blk[0];
                ok = (uint32_t)blk < (uint32_t)a.num_blocks;
                row0 = (int64_t)(ok ? blk : 0) * a.bs + (kw0 & (a.bs - 1));
            }
            const int nrec = __builtin_amdgcn_readfirstlane(ok ? nkeys * (int)stride_b : 0);
            const int64_t rb_ = row0 * stride_b;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + rb_), (short)0, nrec, kBufWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + rb_), (short)0, nrec, kBufWord3);
            dma_tile(rk, (lds_t *)kd, voff, std::make_integer_sequence<int, LPW>{});
            dma_tile(rv, (lds_t *)vd, voff, std::make_integer_sequence<int, LPW>{});
        }
    };

    // Per-lane LDS byte offsets of the operand reads (loop invariant).
    // K (A operand of S^T = K Q^T): key row 32*mt + r32, chunk 2*kk + j.
    int koff[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) koff[kk] = r32 * 256 + 16 * ((2 * kk + j) ^ tile_swz(r32));
    // V^T (A operand of O^T += V^T P^T) by transpose reads: lane reads 4
    // elements of key row 32*mt + 16*ap + 4*j + q16/4 (+8 for the upper
    // half), dims 32*nt + 16*g2 + 4*(q16%4) .. +4.
    const int q16 = lane & 15, g2 = (lane >> 4) & 1;
    int voffr[2][4];
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int t = 4 * j + 8 * hi + (q16 >> 2);
            const int chunk = 4 * nt + 2 * g2 + ((q16 & 3) >> 1);
            voffr[hi][nt] = t * 256 + 16 * (chunk ^ tile_swz(t)) + 8 * (q16 & 1);
        }

    float m[2], l[2];
    f32x16 o[2][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m[rb] = -INFINITY;
        l[rb] = 0.f;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][nt][r] = 0.f;
    const float c = a.scale_log2;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

    // One key tile: start the direct loads of the next tile into `nxt`, then
    // compute on `cur`. The two buffers are distinct objects (restrict), which
    // lets the compiler read `cur` without waiting for the loads into `nxt`.
    // `nmt`: key halves of the tile the wave computes: 2, or 1 (the lower
    // half) on a diagonal tile whose upper half lies wholly above the wave's
    // last row.
    auto tile_step = [&](auto nmt, auto masked, const uint8_t *__restrict__ cur, uint8_t *__restrict__ nxt,
                         int k0, bool more) {
        constexpr int NMT = decltype(nmt)::value;
        load_tile(k0 + kPfBN, nxt);
        const uint8_t *Ks = cur;
        const uint8_t *Vs = cur + kTileBytes;
        if (wave_rows && (!decltype(masked)::value || k0 <= pos_last)) {
            // S^T tiles: st[rb][mt][r] = S[row r32 of block rb][key k0 + 32*mt + 8*(r/4) + 4*j + r%4].
            // Every K operand read from LDS feeds both row blocks.
            f32x16 st[RB][2];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) st[rb][mt][r] = 0.f;
            // The two key halves' chains alternate, and the K operand reads
            // run kLook ahead of the MFMAs that use them: left to itself the
            // scheduler reused one register group per step and waited out the
            // LDS latency before every MFMA pair.
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
                    const bf16x8 kab = __builtin_bit_cast(bf16x8,
                        *reinterpret_cast<const u32x4 *>(Ks + 32 * 256 * mt + koff[kk]));
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        st[rb][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kab, qb[rb][kk], st[rb][mt], 0, 0, 0);
                }
            if constexpr (RB == 1) {
                constexpr int kLook = NMT == 2 ? 6 : 4;
                __builtin_amdgcn_sched_group_barrier(0x100, kLook, 0);   // the first K reads
#pragma unroll
                for (int i = 0; i < 8 * NMT - kLook; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // the next read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, kLook, 0);   // the last MFMAs
            }
            // Online softmax: causal mask (diagonal tiles only), max on raw
            // scores, one lazy-rescale decision for both row blocks, then
            // p = exp2(q.k * c - m * c) rounded to bf16 and row sums of the
            // rounded p via v_dot2.
            float mx[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                if constexpr (decltype(masked)::value) {
                    const int lim = my_pos[rb] - k0 - 4 * j;
#pragma unroll
                    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            st[rb][mt][r] = (32 * mt + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : st[rb][mt][r];
                }
                // four independent partial maxima, then a short tree. IEEE
                // maximum (NaN-propagating) pairs into v_maximum3_f32 and,
                // unlike fmaxf, needs no quieting of its inputs first.
                float xq[4];
#pragma unroll
                for (int g = 0; g < 2 * NMT; ++g) {
                    const int mt = g >> 1, r0 = 8 * (g & 1);
                    xq[g] = fmax3(st[rb][mt][r0], st[rb][mt][r0 + 1], st[rb][mt][r0 + 2]);
                    xq[g] = fmax3(xq[g], st[rb][mt][r0 + 3], st[rb][mt][r0 + 4]);
                    xq[g] = fmax3(xq[g], st[rb][mt][r0 + 5], st[rb][mt][r0 + 6]);
                    xq[g] = fmax3(xq[g], st[rb][mt][r0 + 7], xq[g]);
                }
                const float x4 = NMT == 2 ? fmax3(fmax3(xq[0], xq[1], xq[2]), xq[3], xq[3])
                                          : __builtin_elementwise_maximum(xq[0], xq[1]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x4), __float_as_uint(x4), false, false);
                mx[rb] = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            bool grow = false;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) grow = grow || mx[rb] * c > m[rb] * c + kLazy;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const float m_new = fmaxf(m[rb], mx[rb]);
                    const float alpha = m[rb] == m_new ? 1.f : fast_exp2((m[rb] - m_new) * c);
                    l[rb] *= alpha;
                    // A plain multiply: the compiler then keeps every
                    // accumulator in ordinary VGPRs (206 of them, no AGPRs,
                    // nothing spilled), so the scores need no copies out of
                    // the accumulation registers either.
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) o[rb][nt] *= alpha;
                    m[rb] = m_new;
                }
            }
            bf16x8 pb[RB][2][2];   // [rb][mt][ap]
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float mc = m[rb] * c;
                float ls[4] = {0.f, 0.f, 0.f, 0.f};   // four short sum chains
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                    for (int ap = 0; ap < 2; ++ap) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            pb[rb][mt][ap][e] = (__bf16)fast_exp2(__builtin_fmaf(st[rb][mt][8 * ap + e], c, -mc));
#pragma unroll
                        for (int e = 0; e < 8; e += 2)
                            ls[2 * mt + ap] = __builtin_amdgcn_fdot2_f32_bf16(
                                bf16x2{pb[rb][mt][ap][e], pb[rb][mt][ap][e + 1]}, ones, ls[2 * mt + ap], false);
                    }
                l[rb] += NMT == 2 ? (ls[0] + ls[1]) + (ls[2] + ls[3]) : ls[0] + ls[1];
            }
            // O^T += V^T P^T over 4 steps of 16 keys; each V^T operand (two
            // transpose reads of 4 consecutive key rows) feeds both row blocks.
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int ap = 0; ap < 2; ++ap) {
                    const uint8_t *vrow = Vs + (32 * mt + 16 * ap) * 256;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        typedef short s16x4 __attribute__((ext_vector_type(4)));
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(vrow + voffr[0][nt]));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(vrow + voffr[1][nt]));
                        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
                            o[rb][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[rb][mt][ap], o[rb][nt], 0, 0, 0);
                    }
                }
        }
        // the block ids of the tile after next, behind this step's LDS reads
        // (a scalar load shares their counter); the wait before the barrier
        // covers it
        if (more) fetch_blocks(k0 + 2 * kPfBN);
    };

    if constexpr (SRC != kContiguous) {
#pragma unroll
        for (int i = 0; i < NB; ++i) pre_blk[i] = key_of(0, i) < kend ? first_blk[i] : -1;
    }
    load_tile(0, lds[0]);
    fetch_blocks(kPfBN);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Tiles below the diagonal of every row of this wave need no mask; the
    // last few do. Waves of one workgroup may split the tiles differently:
    // every wave still passes one barrier per tile, and a barrier counts
    // arrivals whatever instruction a wave reached it at.
    const int n_full = min(n_kt, max(0, (off + q0 + 32 * RB * wh + 1) / kPfBN));
    // Unrolled by two, so that each step's buffer is a constant and the
    // operand read addresses need no per-tile arithmetic. The other buffer
    // was last read before the previous barrier; the next tile's direct loads
    // must have landed before the barrier hands its buffer to the other waves.
    int kt = 0;
    for (; kt + 1 < n_full; kt += 2) {
        tile_step(std::integral_constant<int, 2>{}, std::false_type{}, lds[0], lds[1], kt * kPfBN, true);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        tile_step(std::integral_constant<int, 2>{}, std::false_type{}, lds[1], lds[0], (kt + 1) * kPfBN, kt + 2 < n_kt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (kt < n_full) {   // kt is even here
        tile_step(std::integral_constant<int, 2>{}, std::false_type{}, lds[0], lds[1], kt * kPfBN, kt + 1 < n_kt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        ++kt;
    }
    for (; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        if (kt * kPfBN + 32 > pos_last)   // the upper key half is masked for every row of the wave
            tile_step(std::integral_constant<int, 1>{}, std::true_type{}, lds[buf], lds[buf ^ 1], kt * kPfBN, kt + 1 < n_kt);
        else
            tile_step(std::integral_constant<int, 2>{}, std::true_type{}, lds[buf], lds[buf ^ 1], kt * kPfBN, kt + 1 < n_kt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    if constexpr (PERSIST) {
        if (tid == 0)
            next_claim = __hip_atomic_fetch_add(claim_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (RB == 1) {
        // Through LDS (the tile buffers are free after the last barrier): the
        // wave's 32 x 128 output tile goes in with 8-byte writes, rows 272
        // bytes apart, and comes back as whole 256-byte rows, so each global
        // store writes four full rows instead of 32 scattered 16-byte pieces.
        constexpr int kPitch = 272;
        uint8_t *stg = &lds[0][0] + kPitch * 32 * wave;
        const int rbase = q0 + 32 * wh;
        // Fused store: the K/V rows of the wave's 32 query rows go to their
        // cache slots, four whole 256-byte rows per instruction. The G query
        // heads of a kv head share them out (instruction i falls to head
        // i % G), and the loads go out before the output epilogue, so the
        // round trip overlaps it; the last two tile steps read these rows,
        // so this XCD's L2 serves them. Rows past the sequence and slots
        // outside the pool are skipped, as in store_kvcache.
        u32x4 kw[8], vw[8];
        int slot[8];
        if constexpr (STORE) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int rr = 4 * i + (lane >> 4), chunk = lane & 15;
                slot[i] = -1;
                if (i % HG == hg) {   // wave-uniform
                    slot[i] = __shfl(my_slot, rr);
                    if ((uint32_t)slot[i] < (uint32_t)a.num_slots) {
                        const int64_t src = (int64_t)(q_start + rbase + rr) * a.kv_stride + kvh * kPfD + 8 * chunk;
                        kw[i] = ld16((const uint16_t *)a.k + src);
                        vw[i] = ld16((const uint16_t *)a.v + src);
                    }
                }
            }
        }
        const float lt = xor32_sum(l[0]);
        const float inv = row_ok[0] ? 1.f / lt : 0.f;
        // o[0][nt][4*g + c] = O[row][d = 32*nt + 8*g + 4*j + c]
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(o[0][nt][4 * g] * inv, o[0][nt][4 * g + 1] * inv);
                w[1] = pack_bf16x2(o[0][nt][4 * g + 2] * inv, o[0][nt][4 * g + 3] * inv);
                *reinterpret_cast<u32x2 *>(stg + r32 * kPitch + 2 * (32 * nt + 8 * g + 4 * j)) = w;
            }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int rr = 4 * i + (lane >> 4), chunk = lane & 15;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + rr * kPitch + 16 * chunk);
            if (rbase + rr < Lq) {
                uint16_t *out = (uint16_t *)a.out + ((int64_t)(q_start + rbase + rr) * a.Hq + h) * kPfD;
                *reinterpret_cast<u32x4 *>(out + 8 * chunk) = v;
            }
        }
        if constexpr (STORE) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int chunk = lane & 15;
                if ((uint32_t)slot[i] < (uint32_t)a.num_slots) {
                    const int64_t dst = ((int64_t)slot[i] * a.Hkv + kvh) * kPfD + 8 * chunk;
                    *reinterpret_cast<u32x4 *>((uint16_t *)a.store_kc + dst) = kw[i];
                    *reinterpret_cast<u32x4 *>((uint16_t *)a.store_vc + dst) = vw[i];
                }
            }
        }
    } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float lt = xor32_sum(l[rb]);
        if (!row_ok[rb]) continue;
        const float inv = 1.f / lt;
        const int row = q0 + 32 * RB * wh + 32 * rb + r32;
        uint16_t *out = (uint16_t *)a.out + ((int64_t)(q_start + row) * a.Hq + h) * kPfD;
        // o[rb][nt][4*g + c] = O[row][d = 32*nt + 8*g + 4*j + c]
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(o[rb][nt][4 * g] * inv, o[rb][nt][4 * g + 1] * inv);
                w[1] = pack_bf16x2(o[rb][nt][4 * g + 2] * inv, o[rb][nt][4 * g + 3] * inv);
                *reinterpret_cast<u32x2 *>(out + 32 * nt + 8 * g + 4 * j) = w;
            }
    }
    }
    };

    if constexpr (!PERSIST) {
        // One workgroup per item, in a fixed XCD-aware order. Workgroups with
        // equal p % 8 run on one XCD (the hardware deals them round robin),
        // and each XCD has its own L2. Work is grouped by (sequence, kv head)
        // pair, the unit that shares K and V; pair pi runs in class pi % 8, so
        // all query blocks and heads of that kv head read their K/V tiles
        // through one L2. Two orders within an XCD,
        // chosen on the host from the batch's K/V bytes (a bound on them when
        // the keys come through block tables):
        //  - K/V within half the 256 MB MALL: longest first across all the
        //    XCD's pairs (query-block rank major), so the tail holds only
        //    short blocks;
        //  - larger: pair by pair, each pair's longest blocks first, so only a
        //    few pairs' K/V are live at a time.
        const int local = blockIdx.x >> 3;
        int lp, rank, hg;
        if (a.by_rank) {
            const int per_rank = ((npairs + 7) / 8) * HG;
            rank = local / per_rank;
            const int within = local - rank * per_rank;
            lp = within / HG;
            hg = within - lp * HG;
        } else {
            const int per_pair = qblocks * HG;
            lp = local / per_pair;
            const int within = local - lp * per_pair;
            rank = within / HG;
            hg = within - rank * HG;
        }
        const int pair = 8 * lp + xcd;
        if (pair >= npairs) return;
        run_item(pair, qblocks - 1 - rank, hg);
    } else {
        // Persistent grid: a fixed number of workgroups per XCD, each claiming
        // items of its XCD's list from a counter in the workspace (an
        // agent-scope atomic). The list holds only the non-empty items of the
        // XCD's pairs (pair = 8 * lp + xcd), in the same two orders as above,
        // with pairs of more query blocks first; every workgroup builds it in
        // LDS from cu_seqlens_q. An item's successor is claimed when its tile
        // loop is done. A workgroup leaves when its claim passes the end of
        // the list; the last one to leave zeroes the counters for the next call.
        static_assert(kPfMaxXcdPairs == 256 && kPfMaxQblocks == 512, "table sizes");
        int32_t *const tab = reinterpret_cast<int32_t *>(lds_all + 2 * 2 * kTileBytes);
        int32_t *const s_nq = tab;                    // query blocks per pair, sorted descending
        int32_t *const s_lp = tab + 256;              // the pair (lp) at each sorted position
        int32_t *const s_raw = tab + 512;             // query blocks per pair, by lp
        int32_t *const s_pre = tab + 768;             // items before rank r (or before sorted pair i)
        uint32_t &s_claim = *reinterpret_cast<uint32_t *>(tab + 768 + 513);
        uint32_t *ctr = a.work_ctr;
        const int npx = (npairs + 7 - xcd) / 8;       // pairs of this XCD: lp < npx
        for (int lp = tid; lp < npx; lp += 64 * NW) {
            const int pair = 8 * lp + xcd;
            const int sq = pair / a.Hkv;
            const int lq = a.cu_q[sq + 1] - a.cu_q[sq];
            s_raw[lp] = lq > 0 ? min((lq + BM - 1) / BM, qblocks) : 0;
        }
        if (tid == 0) s_claim = __hip_atomic_fetch_add(ctr + xcd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        // stable sort by query-block count, descending (rank by counting)
        for (int lp = tid; lp < npx; lp += 64 * NW) {
            const int v = s_raw[lp];
            int pos = 0;
            for (int o = 0; o < npx; ++o) {
                const int w = s_raw[o];
                pos += (w > v) | ((w == v) & (o < lp));
            }
            s_nq[pos] = v;
            s_lp[pos] = lp;
        }
        __syncthreads();
        // prefix counts: rank-major over ranks r (query block qblocks-1-r; the
        // pairs holding it are the first cnt of the sorted list), or
        // pair-major over sorted pairs
        const int nent = a.by_rank ? qblocks : npx;
        if (tid < 64) {
            int run = 0;
            for (int base = 0; base < nent; base += 64) {
                const int e = base + lane;
                int cnt = 0;
                if (e < nent) {
                    if (a.by_rank) {
                        const int qt = qblocks - 1 - e;   // pairs with s_nq > qt: binary search
                        int lo = 0, hi = npx;
                        while (lo < hi) {
                            const int mid = (lo + hi) >> 1;
                            if (s_nq[mid] > qt) lo = mid + 1; else hi = mid;
                        }
                        cnt = lo * HG;
                    } else {
                        cnt = s_nq[e] * HG;
                    }
                }
                int incl = cnt;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    if (lane >= o) incl += y;
                }
                if (e < nent) s_pre[e] = run + incl - cnt;
                run += __shfl(incl, 63);
            }
            if (lane == 0) s_pre[nent] = run;
        }
        __syncthreads();
        const uint32_t n_items = (uint32_t)s_pre[nent];
        uint32_t c = s_claim;
        while (c < n_items) {
            // the entry e with s_pre[e] <= c < s_pre[e + 1]
            int lo = 0, hi = nent;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if ((uint32_t)s_pre[mid] <= c) lo = mid; else hi = mid;
            }
            const int rem = (int)(c - (uint32_t)s_pre[lo]);
            int lp, qt, hg;
            if (a.by_rank) {
                qt = qblocks - 1 - lo;
                lp = s_lp[rem / HG];
                hg = rem % HG;
            } else {
                lp = s_lp[lo];
                qt = s_nq[lo] - 1 - rem / HG;
                hg = rem % HG;
            }
            next_claim = 0xffffffffu;
            run_item(__builtin_amdgcn_readfirstlane(8 * lp + xcd), __builtin_amdgcn_readfirstlane(qt),
                     __builtin_amdgcn_readfirstlane(hg));
            __syncthreads();   // every wave is past the item (its LDS is free) and has read c
            if (tid == 0) {
                // an item that left early (bad metadata) made no claim yet
                if (next_claim == 0xffffffffu)
                    next_claim = __hip_atomic_fetch_add(claim_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_claim = next_claim;
            }
            __syncthreads();
            c = s_claim;
        }
        if (tid == 0) {
            const uint32_t d = __hip_atomic_fetch_add(ctr + 8, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (d == gridDim.x - 1) {
                // every workgroup has made its last claim: reset for the next call
#pragma unroll
                for (int x = 0; x < 9; ++x)
                    __hip_atomic_store(ctr + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <int SRC, int NW, int RB, int WPE, bool PERSIST, int HPW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void prefill_mfma_kernel(PrefillArgs a) {
    prefill_mfma_body<SRC, NW, RB, WPE, PERSIST, false, HPW>(a);
}

// The call's K/V rows also stored into the cache.
template <int SRC, int NW, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void prefill_store_mfma_kernel(PrefillArgs a) {
    prefill_mfma_body<SRC, NW, 1, WPE, false, true, 1>(a);
}

template <typename T>
__device__ __forceinline__ float pf_load(const T *p, int64_t i);
template <>
__device__ __forceinline__ float pf_load<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float pf_load<uint16_t>(const uint16_t *p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
template <typename T>
__device__ __forceinline__ void pf_store(T *p, int64_t i, float x);
template <>
__device__ __forceinline__ void pf_store<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void pf_store<uint16_t>(uint16_t *p, int64_t i, float x) {
    p[i] = (uint16_t)f32_to_bf16(x);
}

// One wave per (query row, q head): plain online softmax with wave reductions.
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_generic_kernel(PrefillArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave, h = blockIdx.y, s = blockIdx.z;
    const int q_start = a.cu_q[s];
    const int Lq = a.cu_q[s + 1] - q_start;
    if (row >= Lq || q_start < 0 || q_start > a.total_q - Lq) return;
    const int k_start = a.cu_k[s];
    const int Lk = a.cu_k[s + 1] - k_start;
    if (Lk < Lq || Lk > a.max_seqlen_k) return;
    if (!a.paged && (k_start < 0 || k_start > a.total_q - Lk)) return;
    const int pos = Lk - Lq + row;
    const int kvh = h / a.group;
    const T *q = (const T *)a.q + (int64_t)(q_start + row) * a.q_stride + (int64_t)h * D;
    const T *kb = (const T *)(a.paged ? a.kc : a.k);
    const T *vb = (const T *)(a.paged ? a.vc : a.v);
    float qv[EPL], acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        qv[e] = pf_load<T>(q, lane * EPL + e) * a.scale_log2;
        acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int last = min(pos, Lk - 1);
    for (int key = 0; key <= last; ++key) {
        const int64_t eo = prefill_key_off(a, s, k_start, key, kvh, D);
        float kv[EPL], vv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kv[e] = eo >= 0 ? pf_load<T>(kb, eo + lane * EPL + e) : 0.f;
            vv[e] = eo >= 0 ? pf_load<T>(vb, eo + lane * EPL + e) : 0.f;
        }
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], kv[e], dot);
        dot = wave_sum(dot);
        const float m_new = fmaxf(m, dot);
        const float alpha = fast_exp2(m - m_new);
        const float pw = fast_exp2(dot - m_new);
        l = l * alpha + pw;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pw, vv[e], acc[e] * alpha);
        m = m_new;
    }
    const float inv = last >= 0 ? 1.f / l : 0.f;
    T *o = (T *)a.out + ((int64_t)(q_start + row) * a.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) pf_store<T>(o, lane * EPL + e, acc[e] * inv);
}

// Compute units of the current device (cached per device).
static int prefill_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

// The fused store's copy as a store_kvcache launch (for the shapes that run
// it as a kernel of its own).
static hipError_t launch_store_of(const PrefillArgs &a, int dtype, hipStream_t stream) {
    const int es = dtype == 1 ? 2 : 4;
    StoreArgs sa;
    sa.k = (const uint8_t *)a.k;
    sa.v = (const uint8_t *)a.v;
    sa.k_stride_bytes = sa.v_stride_bytes = a.kv_stride * es;
    sa.kc = (uint8_t *)a.store_kc;
    sa.vc = (uint8_t *)a.store_vc;
    sa.slots = a.slots;
    sa.num_tokens = a.total_q;
    sa.chunks_per_row = a.Hkv * a.d * es / 16;
    sa.num_slots = a.num_slots;
    return launch_store(sa, stream);
}

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    if (a.num_seqs == 0 || a.max_seqlen_q == 0) return hipSuccess;
    // The MFMA kernel's direct tile loads address up to 64 key rows per
    // descriptor with 32-bit offsets, and the small-block form needs blocks of
    // at least 4 keys; anything else takes the generic kernel.
    const int64_t row_bytes = a.paged ? (int64_t)a.Hkv * a.d * 2 : a.kv_stride * 2;
    // The fused store over the pool also addresses 64 of the call's rows.
    const bool rows_ok = !(a.slots && a.paged) || a.kv_stride * 2 * kPfBN < (1ll << 31);
    if (dtype == 1 && a.d == 128 && (!a.paged || a.bs >= 4) && row_bytes * kPfBN < (1ll << 31) && rows_ok) {
        // Four waves of 32 query rows per workgroup (one head, 128 rows), two
        // waves per SIMD: while one wave waits on LDS or runs its softmax the
        // other keeps the matrix core busy.
        constexpr int NW = 4, RB = 1;
        // One query head per workgroup, 128 rows, when any sequence has more
        // query rows than a shared workgroup would give each head: there two
        // heads of a GQA group sharing a workgroup's K/V tiles (64 rows each)
        // measured equal on prefix hits and 9% slower on a mixed step. When
        // every sequence fits (decode rows, short chunks: at most 64 rows,
        // or 32 with a group of 4), HPW heads share it and each K/V tile is
        // staged once for all of them: 64 decode rows took 122 us this way
        // against 168 us with one head per workgroup.
        const bool store = a.slots && (!a.paged || a.bs >= 4 * (16 / NW));
        const int hpw = store ? 1
                        : (a.group % 4 == 0 && a.max_seqlen_q <= 32 * RB * (NW / 4)) ? 4
                        : (a.group % 2 == 0 && a.max_seqlen_q <= 32 * RB * (NW / 2)) ? 2 : 1;
        const int bm = 32 * RB * (NW / hpw);
        const int64_t pairs = (int64_t)a.num_seqs * a.Hkv;
        const int64_t qblocks = (a.max_seqlen_q + bm - 1) / bm;
        // The persistent grid (two workgroups per CU claiming items) only when
        // the caller gave a workspace, the item tables fit in LDS and every
        // workgroup takes one head.
        const bool persist = a.work_ctr != nullptr && hpw == 1 && (pairs + 7) / 8 <= kPfMaxXcdPairs &&
                             qblocks <= kPfMaxQblocks;
        const int64_t nwg_fixed = 8 * ((pairs + 7) / 8) * qblocks * (a.group / hpw);
        if (nwg_fixed > 0x7fffffff) return hipErrorInvalidValue;
        const int64_t nwg = persist ? 8 * ((2 * prefill_cus() + 7) / 8) : nwg_fixed;
        const dim3 grid((unsigned)nwg), block(64 * NW);
#define PKV_MFMA_LAUNCH(P, H)                                                                                \
    do {                                                                                                     \
        if (!a.paged)                                                                                        \
            hipLaunchKernelGGL((prefill_mfma_kernel<kContiguous, NW, RB, 2, P, H>), grid, block, 0, stream, a); \
        else if (a.bs % kPfBN == 0)                                                                          \
            hipLaunchKernelGGL((prefill_mfma_kernel<kPoolBlocks, NW, RB, 2, P, H>), grid, block, 0, stream, a); \
        else if (a.bs >= 4 * (16 / NW))                                                                      \
            hipLaunchKernelGGL((prefill_mfma_kernel<kPoolWave, NW, RB, 2, P, H>), grid, block, 0, stream, a);   \
        else                                                                                                 \
            hipLaunchKernelGGL((prefill_mfma_kernel<kPoolSmall, NW, RB, 2, P, H>), grid, block, 0, stream, a);  \
    } while (0)
        if (store) {
            const dim3 g((unsigned)nwg_fixed);
            if (!a.paged)
                hipLaunchKernelGGL((prefill_store_mfma_kernel<kContiguous, NW, 2>), g, block, 0, stream, a);
            else if (a.bs % kPfBN == 0)
                hipLaunchKernelGGL((prefill_store_mfma_kernel<kPoolBlocks, NW, 2>), g, block, 0, stream, a);
            else
                hipLaunchKernelGGL((prefill_store_mfma_kernel<kPoolWave, NW, 2>), g, block, 0, stream, a);
        } else if (a.slots) {
            // Blocks of 4 or 8 keys: the store kernel, then attention. (The
            // fused form of the per-4-key loads ran out of scalar registers
            // and was slower than the two launches.)
            const hipError_t e = launch_store_of(a, dtype, stream);
            if (e != hipSuccess) return e;
            if (hpw == 4) PKV_MFMA_LAUNCH(false, 4);
            else if (hpw == 2) PKV_MFMA_LAUNCH(false, 2);
            else PKV_MFMA_LAUNCH(false, 1);
        } else if (persist) {
            PKV_MFMA_LAUNCH(true, 1);
        } else if (hpw == 4) {
            PKV_MFMA_LAUNCH(false, 4);
        } else if (hpw == 2) {
            PKV_MFMA_LAUNCH(false, 2);
        } else {
            PKV_MFMA_LAUNCH(false, 1);
        }
#undef PKV_MFMA_LAUNCH
    } else {
        if (a.slots) {
            // Other dtypes, head sizes and block sizes: the store kernel, then
            // attention (over the pool when there are block tables).
            const hipError_t e = launch_store_of(a, dtype, stream);
            if (e != hipSuccess) return e;
        }
        const dim3 grid((a.max_seqlen_q + 3) / 4, a.Hq, a.num_seqs);
        if (dtype == 0 && a.d == 64)
            hipLaunchKernelGGL((prefill_generic_kernel<float, 64>), grid, dim3(256), 0, stream, a);
        else if (dtype == 0 && a.d == 128)
            hipLaunchKernelGGL((prefill_generic_kernel<float, 128>), grid, dim3(256), 0, stream, a);
        else if (dtype == 1 && a.d == 64)
            hipLaunchKernelGGL((prefill_generic_kernel<uint16_t, 64>), grid, dim3(256), 0, stream,
                               a);
        else if (dtype == 1 && a.d == 128)
            hipLaunchKernelGGL((prefill_generic_kernel<uint16_t, 128>), grid, dim3(256), 0, stream,
                               a);
        else
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace pkv
