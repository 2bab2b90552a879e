// pkv_internal.h -- launchers shared between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct StoreArgs {
    const uint8_t *k, *v;
    int64_t k_stride_bytes, v_stride_bytes;
    uint8_t *kc, *vc;
    const int32_t *slots;
    int32_t num_tokens;
    int32_t chunks_per_row;   // row bytes / 16
    int64_t num_slots;
};
hipError_t launch_store(const StoreArgs &a, hipStream_t stream);

struct RopeStoreArgs {
    uint8_t *q;                  // rotated in place
    uint8_t *k;                  // read; written back when write_k
    const uint8_t *v;
    int64_t q_stride_bytes, k_stride_bytes, v_stride_bytes;
    uint8_t *kc, *vc;
    const int32_t *slots, *positions;
    const float *cos_sin;        // [max_positions][rot_dim]
    int32_t max_positions, rot_dim, style, write_k, d;
    int64_t row_bytes;           // one cache slot row (all kv heads)
    int64_t num_slots;
    // work items: per token q_items + k_items + v_items
    int32_t r_items;             // rotated items per head vector
    int32_t p_items;             // unrotated tail chunks per k head vector
    int32_t q_items, k_items, items_per_token;
    int64_t total_items;
};
hipError_t launch_rope_store(const RopeStoreArgs &a, int dtype, hipStream_t stream);

struct DecodeArgs {
    const void *q;
    int64_t q_stride;          // elements between consecutive sequences' q rows
    const void *kc, *vc;
    const int32_t *bt;
    int32_t maxb;
    const int32_t *ctx;
    int32_t ctx_cap;           // max_context_len: every context is read as min(max(ctx, 0), ctx_cap)
    int32_t num_seqs, num_blocks, bs, log2bs;
    int32_t Hq, Hkv, d, group;
    float scale_log2;          // scale * log2(e): scores live in the exp2 domain
    void *out;
    int32_t P;                 // tokens per partition
    int32_t maxparts;          // ceil(max_context_len / P)
    float *ws_acc;             // fixed partitions: [num_seqs][maxparts][Hq][d]
                               // balanced split:   [waves][2][group][d]
    float *ws_ml;              // the matching (max, sum) pairs
    int32_t *ws_cum;           // balanced split: chunk-count prefix sums [num_seqs + 1]
    int32_t waves;             // balanced split: waves in the grid
    // Store fused into the fixed-partition kernel (null st_k otherwise): row b
    // of st_k / st_v (st_stride_bytes apart) goes to slot st_slots[b] of
    // st_kc / st_vc before the attention reads that slot.
    const uint8_t *st_k = nullptr, *st_v = nullptr;
    int64_t st_stride_bytes = 0;
    uint8_t *st_kc = nullptr, *st_vc = nullptr;
    const int32_t *st_slots = nullptr;
    int64_t st_num_slots = 0;
};
// How a decode call is carried out, and the workspace it needs (the same
// plan serves pkv_decode_workspace_bytes and the call).
struct DecodePlan {
    bool balanced;             // decode_sk_kernel (work split evenly over all waves)
    int32_t P, maxparts;       // fixed-partition kernels
    int32_t waves;             // balanced split
    int64_t acc_bytes, ml_bytes, cum_bytes, total;
};
DecodePlan plan_decode(int32_t num_seqs, int32_t max_ctx, int32_t Hq, int32_t Hkv, int32_t d,
                       int32_t bs, int dtype, int32_t partition_size);
// Returns hipErrorNotSupported when no kernel covers the shape/dtype.
hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &plan, int dtype, hipStream_t stream);
// Whether launch_decode runs the fixed-partition kernel that can take the
// store (a.st_k set) into its own launch.
bool decode_store_fusable(const DecodeArgs &a, const DecodePlan &plan, int dtype);

struct PrefillArgs {
    const void *q;
    int64_t q_stride;
    const void *k, *v;         // contiguous source (paged == 0)
    int64_t kv_stride;
    const void *kc, *vc;       // paged source (paged == 1)
    const int32_t *bt;
    int32_t maxb;
    int32_t paged;
    const int32_t *cu_q, *cu_k;
    int32_t num_seqs, num_blocks, bs, log2bs;
    int32_t Hq, Hkv, d, group;
    float scale_log2;
    void *out;
    int32_t max_seqlen_q;
    int32_t max_seqlen_k;      // a sequence with more keys (or fewer than its queries) is skipped
    int32_t total_q;           // rows of q and out; a sequence outside them is skipped
    int32_t by_rank;           // grid order: longest query blocks first across pairs (set by the host)
    uint32_t *work_ctr;        // persistent grid: 8 per-XCD claim counters + 1 exit counter, or null
    // Fused store (contiguous keys only): k/v row i is also copied to row
    // slots[i] of these caches ([num_slots, Hkv, d]) when 0 <= slots[i] < num_slots.
    void *store_kc = nullptr, *store_vc = nullptr;
    const int32_t *slots = nullptr;
    int32_t num_slots = 0;
};
// Bytes of the prefill workspace (the persistent grid's counters).
constexpr size_t kPrefillWorkspaceBytes = 256;
hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream);

}  // namespace pkv
