// rope.hip -- rotary position embedding fused with store_kvcache.
//
// The attention layer rotates q and k by each token's position and then writes
// k and v into the pool slot named by slot_mapping ("Nano vLLM 解读（5）：解析
// ModelRunner", the attention layer's forward; "nano-vLLM-1", "4. prefill 输入
// 打包", where positions are packed next to slot_mapping). Fusing the two
// reads each k row once instead of twice and drops one launch. The rotation is
// RoFormer's (Su et al., 2021): pair j of a head vector at position p turns by
// theta_j(p) = p * base^(-2j / rot_dim); its cos and sin come from a float
// table [max_positions][rot_dim] (cos in the first half, sin in the second)
// built once on the host in double precision.
//
// HBM-bound elementwise work. One work item is one 16-byte chunk of a head
// vector, or for the "rotate half" layout the matching pair of chunks
// (elements [cV, cV+V) and [rot/2 + cV, rot/2 + cV + V)), so a thread's loads
// and stores are whole 16-byte vectors and consecutive lanes walk consecutive
// chunks of a row. Items of one token, in order: q heads (rotated in place),
// k heads (rotated chunks, then the unrotated tail chunks past rot_dim, all
// written to the cache row and optionally back to k), v heads (copied).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kRopeThreads = 256;

template <typename T>
__device__ __forceinline__ void unpack16(const u32x4 &w, float (&x)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const u32x4 &w, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4 &w, float (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
}

template <typename T>
__device__ __forceinline__ u32x4 pack16(const float (&x)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ u32x4 pack16<uint16_t>(const float (&x)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    return w;
}
template <>
__device__ __forceinline__ u32x4 pack16<float>(const float (&x)[4]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x[i]);
    return w;
}

// Rotated chunk c of one head vector `src` (elements, not bytes); results in
// r0 (the chunk itself) and, for the rotate-half layout, r1 (its partner chunk
// rot/2 elements further on).
template <typename T, int STYLE>
__device__ __forceinline__ void rotate_chunk(const T *src, int c, const float *cs, int half,
                                             u32x4 &r0, u32x4 &r1) {
    constexpr int V = 16 / sizeof(T);
    float x0[V], out0[V];
    unpack16<T>(ld16(src + c * V), x0);
    if constexpr (STYLE == 0) {
        // pairs (j, j + half), j = cV .. cV+V-1
        float x1[V], out1[V], cv[V], sv[V];
        unpack16<T>(ld16(src + half + c * V), x1);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            cv[e] = cs[c * V + e];
            sv[e] = cs[half + c * V + e];
        }
#pragma unroll
        for (int e = 0; e < V; ++e) {
            out0[e] = __builtin_fmaf(x0[e], cv[e], -x1[e] * sv[e]);
            out1[e] = __builtin_fmaf(x1[e], cv[e], x0[e] * sv[e]);
        }
        r1 = pack16<T>(out1);
    } else {
        // pairs (2j, 2j+1), j = cV/2 .. cV/2 + V/2 - 1
#pragma unroll
        for (int e = 0; e < V / 2; ++e) {
            const float cj = cs[c * (V / 2) + e], sj = cs[half + c * (V / 2) + e];
            out0[2 * e] = __builtin_fmaf(x0[2 * e], cj, -x0[2 * e + 1] * sj);
            out0[2 * e + 1] = __builtin_fmaf(x0[2 * e + 1], cj, x0[2 * e] * sj);
        }
    }
    r0 = pack16<T>(out0);
}

template <typename T, int STYLE>
__global__ __launch_bounds__(kRopeThreads) void rope_store_kernel(RopeStoreArgs a) {
    constexpr int V = 16 / sizeof(T);
    const int64_t idx = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    if (idx >= a.total_items) return;
    const int32_t t = (int32_t)(idx / a.items_per_token);
    int32_t u = (int32_t)(idx - (int64_t)t * a.items_per_token);
    const int half = a.rot_dim / 2;
    if (u < a.q_items) {
        const int h = u / a.r_items, c = u - h * a.r_items;
        const int p = min(max(a.positions[t], 0), a.max_positions - 1);
        const float *cs = a.cos_sin + (int64_t)p * a.rot_dim;
        T *row = (T *)(a.q + (int64_t)t * a.q_stride_bytes) + (int64_t)h * a.d;
        u32x4 r0, r1;
        rotate_chunk<T, STYLE>(row, c, cs, half, r0, r1);
        st16(row + c * V, r0);
        if (STYLE == 0) st16(row + half + c * V, r1);
        return;
    }
    u -= a.q_items;
    const int32_t slot = a.slots[t];
    const bool store = slot >= 0 && slot < a.num_slots;
    if (u < a.k_items) {
        const int per = a.r_items + a.p_items;
        const int h = u / per, c = u - h * per;
        T *src = (T *)(a.k + (int64_t)t * a.k_stride_bytes) + (int64_t)h * a.d;
        T *dst = store ? (T *)(a.kc + (int64_t)slot * a.row_bytes) + (int64_t)h * a.d : nullptr;
        if (c < a.r_items) {
            const int p = min(max(a.positions[t], 0), a.max_positions - 1);
            const float *cs = a.cos_sin + (int64_t)p * a.rot_dim;
            u32x4 r0, r1;
            rotate_chunk<T, STYLE>(src, c, cs, half, r0, r1);
            if (dst) {
                st16(dst + c * V, r0);
                if (STYLE == 0) st16(dst + half + c * V, r1);
            }
            if (a.write_k) {
                st16(src + c * V, r0);
                if (STYLE == 0) st16(src + half + c * V, r1);
            }
        } else if (dst) {
            // unrotated tail past rot_dim: copied to the cache, k unchanged
            const int e0 = a.rot_dim + (c - a.r_items) * V;
            st16(dst + e0, ld16(src + e0));
        }
        return;
    }
    u -= a.k_items;
    // v: chunk u of the row (all heads), copied bit for bit; the load is
    // issued with the slot's, only the store depends on it
    const u32x4 vv = ld16(a.v + (int64_t)t * a.v_stride_bytes + (int64_t)u * 16);
    if (store) st16(a.vc + (int64_t)slot * a.row_bytes + (int64_t)u * 16, vv);
}

hipError_t launch_rope_store(const RopeStoreArgs &a, int dtype, hipStream_t stream) {
    if (a.total_items == 0) return hipSuccess;
    const int64_t blocks = (a.total_items + kRopeThreads - 1) / kRopeThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g((unsigned)blocks), b(kRopeThreads);
    if (dtype == 1) {
        if (a.style == 0) hipLaunchKernelGGL((rope_store_kernel<uint16_t, 0>), g, b, 0, stream, a);
        else hipLaunchKernelGGL((rope_store_kernel<uint16_t, 1>), g, b, 0, stream, a);
    } else {
        if (a.style == 0) hipLaunchKernelGGL((rope_store_kernel<float, 0>), g, b, 0, stream, a);
        else hipLaunchKernelGGL((rope_store_kernel<float, 1>), g, b, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace pkv
