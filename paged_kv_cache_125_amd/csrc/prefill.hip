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
// one head (32 per wave) and streams 64-key tiles of K and V through LDS. Both
// contractions run on v_mfma_f32_32x32x16_bf16 in the transposed form
//     S^T = K Q^T        (keys as MFMA rows, the wave's queries as columns)
//     O^T += V^T P^T     (head dims as rows, queries as columns)
// so that every lane owns one query row: the row max needs a single
// cross-lane exchange, the rescale by exp2(m_old - m_new) is lane-local, and
// P^T is fed to the second MFMA straight from the registers the first one
// produced. V is written to LDS transposed; within each 16-key group, key
// index bits 2 and 3 are swapped so that the 8 keys one lane contributes to
// an MFMA step sit in 16 contiguous bytes.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kPfD = 128;
constexpr int kPfBM = 128;     // query rows per workgroup
constexpr int kPfBN = 64;      // keys per tile
constexpr int kKsPitch = 136;  // LDS row pitch of K tile (elements)
constexpr int kVtPitch = 72;   // LDS row pitch of the transposed V tile (elements)

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

__device__ __forceinline__ int swap_bits23(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kPfBN * kKsPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[kPfD * kVtPitch];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.x, s = blockIdx.y;
    const int qt = gridDim.z - 1 - blockIdx.z;   // longest (last) query tiles first
    const int q_start = a.cu_q[s];
    const int Lq = a.cu_q[s + 1] - q_start;
    const int q0 = qt * kPfBM;
    if (q0 >= Lq) return;
    const int k_start = a.cu_k[s];
    const int Lk = a.cu_k[s + 1] - k_start;
    const int off = Lk - Lq;
    const int kvh = h / a.group;
    const int r32 = lane & 31, j = lane >> 5;
    const int my_row = q0 + 32 * wave + r32;
    const bool row_ok = my_row < Lq;
    const int my_pos = off + my_row;
    const uint8_t *kbase = (const uint8_t *)(a.paged ? a.kc : a.k);
    const uint8_t *vbase = (const uint8_t *)(a.paged ? a.vc : a.v);

    // B operand of S^T = K Q^T: lane holds Q[row r32][d = 16*kk + 8*j .. +8].
    bf16x8 qb[8];
    {
        const uint16_t *q = (const uint16_t *)a.q + (int64_t)(q_start + my_row) * a.q_stride +
                            (int64_t)h * kPfD + 8 * j;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row_ok) w = ld16(q + 16 * kk);
            qb[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    const int kend = min(Lk, off + min(q0 + kPfBM, Lq));   // keys this block needs
    const int n_kt = (kend + kPfBN - 1) / kPfBN;
    const int wave_pos0 = off + q0 + 32 * wave;            // first row's position

    float m = -INFINITY, l = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nt][r] = 0.f;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * kPfBN;
        __syncthreads();
        // K tile, row-major: thread -> key (tid/16 + 16*it), 16-byte chunk tid%16.
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int kl = (tid >> 4) + 16 * it;
            const int key = k0 + kl;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (key < kend) {
                const int64_t eo = prefill_key_off(a, s, k_start, key, kvh, kPfD);
                if (eo >= 0) w = ld16(kbase + eo * 2 + (tid & 15) * 16);
            }
            *reinterpret_cast<u32x4 *>(&Ks[kl * kKsPitch + 8 * (tid & 15)]) = w;
        }
        // V tile, transposed: thread -> key lane, chunk (wave + 4*it); one
        // wave instruction writes 64 keys of one head-dim row.
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int c = wave + 4 * it;
            const int key = k0 + lane;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (key < kend) {
                const int64_t eo = prefill_key_off(a, s, k_start, key, kvh, kPfD);
                if (eo >= 0) w = ld16(vbase + eo * 2 + c * 16);
            }
            const int col = swap_bits23(lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Vt[(8 * c + 2 * e) * kVtPitch + col] = (uint16_t)(w[e] & 0xffffu);
                Vt[(8 * c + 2 * e + 1) * kVtPitch + col] = (uint16_t)(w[e] >> 16);
            }
        }
        __syncthreads();

        // S^T tiles: st[mt][r] = S[row r32][key k0 + 32*mt + 8*(r/4) + 4*j + r%4].
        f32x16 st[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[mt][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const u32x4 ka =
                    *reinterpret_cast<const u32x4 *>(&Ks[(32 * mt + r32) * kKsPitch + 16 * kk + 8 * j]);
                st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka),
                                                                 qb[kk], st[mt], 0, 0, 0);
            }
        }
        const bool need_mask = row_ok && (k0 + kPfBN - 1 > wave_pos0);
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 32 * mt + 8 * (r >> 2) + 4 * j + (r & 3);
                float x = st[mt][r] * a.scale_log2;
                if (need_mask && key > my_pos) x = -INFINITY;
                st[mt][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2(m - m_new);
        float ls = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(st[mt][r] - m_new);
                st[mt][r] = e;
                ls += e;
            }
        l = l * alpha + ls;
        m = m_new;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[nt][r] *= alpha;

        // O^T += V^T P^T over 4 steps of 16 keys.
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int ap = 0; ap < 2; ++ap) {
                bf16x8 pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[e] = (__bf16)st[mt][8 * ap + e];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const u32x4 va = *reinterpret_cast<const u32x4 *>(
                        &Vt[(32 * nt + r32) * kVtPitch + 32 * mt + 16 * ap + 8 * j]);
                    o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                                    pb, o[nt], 0, 0, 0);
                }
            }
    }

    l += shfl_xor(l, 32);
    if (row_ok) {
        const float inv = 1.f / l;
        uint16_t *out = (uint16_t *)a.out + ((int64_t)(q_start + my_row) * a.Hq + h) * kPfD;
        // o[nt][4*g + c] = O[row][d = 32*nt + 8*g + 4*j + c]
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(o[nt][4 * g] * inv, o[nt][4 * g + 1] * inv);
                w[1] = pack_bf16x2(o[nt][4 * g + 2] * inv, o[nt][4 * g + 3] * inv);
                *reinterpret_cast<u32x2 *>(out + 32 * nt + 8 * g + 4 * j) = w;
            }
    }
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
    if (row >= Lq) return;
    const int k_start = a.cu_k[s];
    const int Lk = a.cu_k[s + 1] - k_start;
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

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    if (a.num_seqs == 0 || a.max_seqlen_q == 0) return hipSuccess;
    if (dtype == 1 && a.d == 128) {
        const dim3 grid(a.Hq, a.num_seqs, (a.max_seqlen_q + kPfBM - 1) / kPfBM);
        hipLaunchKernelGGL(prefill_mfma_kernel, grid, dim3(256), 0, stream, a);
    } else {
        const dim3 grid((a.max_seqlen_q + 3) / 4, a.Hq, a.num_seqs);
        if (dtype == 0 && a.d == 64)
            hipLaunchKernelGGL((prefill_generic_kernel<float, 64>), grid, dim3(256), 0, stream, a);
        else if (dtype == 0 && a.d == 128)
            hipLaunchKernelGGL((prefill_generic_kernel<float, 128>), grid, dim3(256), 0, stream, a);
        else if (dtype == 1 && a.d == 64)
            hipLaunchKernelGGL((prefill_generic_kernel<uint16_t, 64>), grid, dim3(256), 0, stream,
                               a);
        else
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace pkv
