// store.hip -- store_kvcache: write each new token's K/V row into the pool
// slot named by slot_mapping.
//
// ("Nano vLLM 解读（5）：解析 ModelRunner", ModelRunner init and
//  "prepare_prefill": the attention layer writes new K/V via slot_mapping into
//  the per-layer cache view [num_blocks, block_size, kv_heads, head_dim] of
//  "nano-vLLM-1", "3. KV cache 分配".)
//
// A pure bit copy bound by HBM: every (token, 16-byte chunk) pair of the K row
// and of the V row is one work item. Consecutive lanes take consecutive chunks
// of one row, so each wave instruction moves whole 64-byte segments; every
// thread keeps kStoreUnroll items (2 * kStoreUnroll loads) in flight before
// its stores. Workgroups of 1024 threads, one item each. The K/V loads do not wait for the slot: they are issued with
// the slot load (every token row is readable), and only the stores depend on
// it.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// 1024 threads x 1 item measured best among 64..1024 threads x 1..4 items and
// grid-stride forms (16k tokens: 24.6 us against 25.2 for 256 x 2; 49k
// tokens: 77.8 against 79.4); 4 items per thread were the slowest.
constexpr int kStoreThreads = 1024;
constexpr int kStoreUnroll = 1;

__global__ __launch_bounds__(kStoreThreads) void store_kvcache_kernel(StoreArgs a) {
    const int64_t total = (int64_t)a.num_tokens * a.chunks_per_row;
    const int64_t base = (int64_t)blockIdx.x * (kStoreThreads * kStoreUnroll) + threadIdx.x;
    const int64_t row_bytes = (int64_t)a.chunks_per_row * 16;
    const bool narrow = total <= 0x7fffffffLL;   // item indices fit 32-bit division
    u32x4 kx[kStoreUnroll], vx[kStoreUnroll];
    int64_t dst[kStoreUnroll];
#pragma unroll
    for (int u = 0; u < kStoreUnroll; ++u) {
        const int64_t item = base + (int64_t)u * kStoreThreads;
        dst[u] = -1;
        if (item < total) {
            int32_t t, c;
            if (narrow) {
                t = (int32_t)item / a.chunks_per_row;
                c = (int32_t)item - t * a.chunks_per_row;
            } else {
                t = (int32_t)(item / a.chunks_per_row);
                c = (int32_t)(item - (int64_t)t * a.chunks_per_row);
            }
            const int32_t s = a.slots[t];
            kx[u] = ld16(a.k + t * a.k_stride_bytes + c * 16);
            vx[u] = ld16(a.v + t * a.v_stride_bytes + c * 16);
            if (s >= 0 && s < a.num_slots) dst[u] = (int64_t)s * row_bytes + c * 16;
        }
    }
#pragma unroll
    for (int u = 0; u < kStoreUnroll; ++u) {
        if (dst[u] >= 0) {
            st16(a.kc + dst[u], kx[u]);
            st16(a.vc + dst[u], vx[u]);
        }
    }
}

hipError_t launch_store(const StoreArgs &a, hipStream_t stream) {
    const int64_t total = (int64_t)a.num_tokens * a.chunks_per_row;
    if (total == 0) return hipSuccess;
    const int64_t per_block = (int64_t)kStoreThreads * kStoreUnroll;
    const int64_t blocks = (total + per_block - 1) / per_block;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(store_kvcache_kernel, dim3((unsigned)blocks), dim3(kStoreThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace pkv
