// decode.hip -- paged decode attention with split-context partitions.
//
// One query token per sequence attends to context_lens[b] keys gathered
// through the sequence's block table ("Nano vLLM 解读（5）：解析 ModelRunner",
// "prepare_decode"; "nano-vLLM-1", "5. deocde 输入打包"): position j lives at
// slot block_tables[b][j / bs] * bs + j % bs of the per-layer pool
// [num_blocks, bs, Hkv, d]. The output is softmax(scale * q K^T) V
// ("【nano-vllm 学习】04 - …源码学习2", "KV-Cache … 是什么？").
//
// Long contexts are cut into partitions of P tokens, each reduced to an
// unnormalised (acc, max, sum) triple and combined by a log-sum-exp rule
// afterwards (Flash-Decoding, Dao et al. 2023; online softmax, Milakov &
// Gimelshein 2018). A sequence that fits one partition is finished in place.
//
// Kernels:
//  decode_mfma_kernel<G, CHUNK>   bf16, head_dim 128, GQA group G <= 8. One
//      wave per (sequence, kv head, partition). The K/V rows of the kv head are
//      loaded once into registers with 16-byte loads and serve all G query
//      heads of the group: q.K^T runs on MFMA (16x16x32 bf16, the G heads as
//      rows), P.V on the VALU in fp32. Softmax statistics use DPP row
//      reductions; LDS carries only the slot rows, P and per-head statistics.
//  decode_generic_kernel<T, D>    any dtype/group, fp32 math, one wave per
//      (sequence, q head, partition); used for fp32 and small head dims.
//  decode_reduce_kernel<T>        the log-sum-exp combine of partitions.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kDecWaves = 4;    // kv heads (waves) per workgroup, MFMA kernel
constexpr int kDecChunk = 64;   // tokens per online-softmax step, MFMA kernel

// Slot row of position t of sequence b, or -1 for an entry outside the table
// or the pool (such positions read as zeros; outputs are then unspecified).
__device__ __forceinline__ int32_t decode_row(const DecodeArgs &a, int b, int t) {
    const int lb = t >> a.log2bs;
    if (lb >= a.maxb) return -1;
    const int blk = a.bt[(int64_t)b * a.maxb + lb];
    if (blk < 0 || blk >= a.num_blocks) return -1;
    return blk * a.bs + (t & (a.bs - 1));
}

template <int G, int CHUNK>
__global__ __launch_bounds__(64 * kDecWaves) void decode_mfma_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int TILES = CHUNK / 16;   // 16-token MFMA tiles per chunk
    constexpr int TPL = CHUNK / 4;      // tokens each lane accumulates in P.V
    static_assert(G >= 1 && G <= 8, "group");
    __shared__ int32_t rows_s[kDecWaves][CHUNK];
    __shared__ float p_s[kDecWaves][CHUNK * G];
    __shared__ float st_s[kDecWaves][3][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kvh = blockIdx.z * kDecWaves + wave;
    const int b = blockIdx.y, p = blockIdx.x;
    if (kvh >= a.Hkv) return;
    const int n = a.ctx[b];
    const int t_begin = p * a.P;
    if (t_begin >= n && p > 0) return;
    const int nparts = (n + a.P - 1) / a.P;
    const int t_end = min(n, t_begin + a.P);
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t row_bytes = (int64_t)a.Hkv * D * 2;
    const uint8_t *kbase = (const uint8_t *)a.kc + (int64_t)kvh * D * 2;
    const uint8_t *vbase = (const uint8_t *)a.vc + (int64_t)kvh * D * 2;

    // A operand: row = head lr of the group (zero rows above G), k = d.
    bf16x8 qa[4];
    {
        const uint16_t *q = (const uint16_t *)a.q + (int64_t)b * a.q_stride + (int64_t)kvh * G * D;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (lr < G) w = ld16(q + lr * D + 32 * kk + 8 * lg);
            qa[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    float m_run[4], l_run[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    for (int t0 = t_begin; t0 < t_end; t0 += CHUNK) {
        for (int i = lane; i < CHUNK; i += 64) {
            const int t = t0 + i;
            rows_s[wave][i] = t < t_end ? decode_row(a, b, t) : -1;
        }
        wave_lds_fence();
        // K: lane (lr, lg) reads token 16*tile + lr, d = 32*kk + 8*lg .. +8.
        u32x4 kx[TILES][4];
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) {
            const int row = rows_s[wave][16 * tile + lr];
            const uint8_t *src = kbase + (int64_t)row * row_bytes + lg * 16;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                u32x4 w = {0u, 0u, 0u, 0u};
                if (row >= 0) w = ld16(src + kk * 64);
                kx[tile][kk] = w;
            }
        }
        // V: lane (lr, lg) reads d = 8*lr .. +8 of tokens lg + 4*i.
        u32x4 vx[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int row = rows_s[wave][lg + 4 * i];
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row >= 0) w = ld16(vbase + (int64_t)row * row_bytes + lr * 16);
            vx[i] = w;
        }
        // S = q . K^T: lane holds S[head 4*lg + r][token 16*tile + lr].
        f32x4 s[TILES];
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) {
            s[tile] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                s[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    qa[kk], __builtin_bit_cast(bf16x8, kx[tile][kk]), s[tile], 0, 0, 0);
        }
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mx = -INFINITY;
#pragma unroll
            for (int tile = 0; tile < TILES; ++tile) {
                const bool ok = t0 + 16 * tile + lr < t_end;
                const float x = ok ? s[tile][r] * a.scale_log2 : -INFINITY;
                s[tile][r] = x;
                mx = fmaxf(mx, x);
            }
            mx = row16_max(mx);
            const float m_new = fmaxf(m_run[r], mx);
            alpha[r] = fast_exp2(m_run[r] - m_new);
            float ls = 0.f;
#pragma unroll
            for (int tile = 0; tile < TILES; ++tile) {
                const float e = fast_exp2(s[tile][r] - m_new);
                s[tile][r] = e;
                ls += e;
            }
            l_run[r] = l_run[r] * alpha[r] + ls;
            m_run[r] = m_new;
        }
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * lg + r;
                if (h < G) p_s[wave][(16 * tile + lr) * G + h] = s[tile][r];
            }
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * lg + r;
                if (h < G) st_s[wave][0][h] = alpha[r];
            }
        }
        wave_lds_fence();
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = st_s[wave][0][h];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= al;
        }
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int tl = lg + 4 * i;
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16lo(vx[i][e]);
                v[2 * e + 1] = bf16hi(vx[i][e]);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ph = p_s[wave][tl * G + h];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, v[e], acc[h][e]);
            }
        }
        wave_lds_fence();
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) l_run[r] = row16_sum(l_run[r]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += shfl_xor(acc[h][e], 16);
            acc[h][e] += shfl_xor(acc[h][e], 32);
        }
    if (lr == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * lg + r;
            if (h < G) {
                st_s[wave][1][h] = m_run[r];
                st_s[wave][2][h] = l_run[r];
            }
        }
    }
    wave_lds_fence();
    if (lane < 16) {
        const int c = lane;  // d = 8c .. 8c+7
        const int h0 = kvh * G;
        if (n == 0 || nparts == 1) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = n == 0 ? 0.f : 1.f / st_s[wave][2][h];
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(acc[h][2 * e] * inv, acc[h][2 * e + 1] * inv);
                st16((uint16_t *)a.out + ((int64_t)b * a.Hq + h0 + h) * D + 8 * c, w);
            }
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float *dst = a.ws_acc + (((int64_t)b * a.maxparts + p) * a.Hq + h0 + h) * D + 8 * c;
                st16(dst, u32x4{__float_as_uint(acc[h][0]), __float_as_uint(acc[h][1]),
                                __float_as_uint(acc[h][2]), __float_as_uint(acc[h][3])});
                st16(dst + 4, u32x4{__float_as_uint(acc[h][4]), __float_as_uint(acc[h][5]),
                                    __float_as_uint(acc[h][6]), __float_as_uint(acc[h][7])});
                if (c == 0) {
                    float *ml = a.ws_ml + (((int64_t)b * a.maxparts + p) * a.Hq + h0 + h) * 2;
                    ml[0] = st_s[wave][1][h];
                    ml[1] = st_s[wave][2][h];
                }
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ float load_elem(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
template <typename T>
__device__ __forceinline__ void store_elem(T *p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t *p, int64_t i, float x) {
    p[i] = (uint16_t)f32_to_bf16(x);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x;
    const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int kvh = h / a.group;
    const int n = a.ctx[b];
    const int t_begin = p * a.P;
    if (t_begin >= n && p > 0) return;
    const int nparts = (n + a.P - 1) / a.P;
    const int t_end = min(n, t_begin + a.P);
    const T *q = (const T *)a.q + (int64_t)b * a.q_stride + (int64_t)h * D;
    const T *kc = (const T *)a.kc;
    const T *vc = (const T *)a.vc;
    float qv[EPL], acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        qv[e] = load_elem<T>(q, lane * EPL + e) * a.scale_log2;
        acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int t = t_begin; t < t_end; ++t) {
        const int row = decode_row(a, b, t);
        float kv[EPL], vv[EPL];
        const int64_t off = ((int64_t)(row < 0 ? 0 : row) * a.Hkv + kvh) * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kv[e] = row >= 0 ? load_elem<T>(kc, off + e) : 0.f;
            vv[e] = row >= 0 ? load_elem<T>(vc, off + e) : 0.f;
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
    if (n == 0 || nparts == 1) {
        const float inv = n == 0 ? 0.f : 1.f / l;
        T *o = (T *)a.out + ((int64_t)b * a.Hq + h) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) store_elem<T>(o, lane * EPL + e, acc[e] * inv);
    } else {
        float *dst = a.ws_acc + (((int64_t)b * a.maxparts + p) * a.Hq + h) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[lane * EPL + e] = acc[e];
        if (lane == 0) {
            float *ml = a.ws_ml + (((int64_t)b * a.maxparts + p) * a.Hq + h) * 2;
            ml[0] = m;
            ml[1] = l;
        }
    }
}

// Combine: M = max_p m_p; out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x * 4 + wave, b = blockIdx.y;
    if (h >= a.Hq) return;
    const int n = a.ctx[b];
    const int nparts = (n + a.P - 1) / a.P;
    if (nparts <= 1) return;
    const int64_t pstride = (int64_t)a.Hq;
    const float *ml = a.ws_ml + ((int64_t)b * a.maxparts * a.Hq + h) * 2;
    float M = -INFINITY;
    for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[p * pstride * 2]);
    M = wave_max(M);
    float o[EPL], den = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    const float *acc = a.ws_acc + ((int64_t)b * a.maxparts * a.Hq + h) * D + lane * EPL;
    for (int p = 0; p < nparts; ++p) {
        const float w = fast_exp2(ml[p * pstride * 2] - M);
        den = fmaf(w, ml[p * pstride * 2 + 1], den);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = fmaf(w, acc[p * pstride * D + e], o[e]);
    }
    const float inv = 1.f / den;
    T *out = (T *)a.out + ((int64_t)b * a.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) store_elem<T>(out, lane * EPL + e, o[e] * inv);
}

bool decode_has_mfma_path(int dtype, int32_t d, int32_t group) {
    return dtype == 1 && d == 128 && (group == 1 || group == 2 || group == 4 || group == 8);
}

int32_t decode_auto_partition(int32_t num_seqs, int32_t max_ctx, int32_t Hkv, int32_t bs,
                              int dtype, int32_t d, int32_t group) {
    (void)bs;
    if (!decode_has_mfma_path(dtype, d, group)) return 256;
    // Enough (sequence, kv head, partition) waves to fill 256 CUs several times
    // over, but partitions long enough that the combine stays a small cost.
    const int64_t pairs = (int64_t)num_seqs * Hkv;
    const int64_t ctx = max_ctx > 0 ? max_ctx : 1;
    int32_t P = 256;
    while (P > 64 && pairs * ((ctx + P - 1) / P) < 4096) P /= 2;
    while (P < 512 && pairs * ((ctx + P - 1) / P) > 65536) P *= 2;
    return P;
}

template <typename T, int D>
static void launch_generic(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_generic_kernel<T, D>), dim3(a.maxparts, a.Hq, a.num_seqs),
                       dim3(64), 0, stream, a);
}

template <int G>
static void launch_mfma(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid(a.maxparts, a.num_seqs, (a.Hkv + kDecWaves - 1) / kDecWaves);
    hipLaunchKernelGGL((decode_mfma_kernel<G, kDecChunk>), grid, dim3(64 * kDecWaves), 0,
                       stream, a);
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (decode_has_mfma_path(dtype, a.d, a.group)) {
        switch (a.group) {
            case 1: launch_mfma<1>(a, stream); break;
            case 2: launch_mfma<2>(a, stream); break;
            case 4: launch_mfma<4>(a, stream); break;
            case 8: launch_mfma<8>(a, stream); break;
            default: return hipErrorNotSupported;
        }
    } else if (dtype == 0 && a.d == 64) {
        launch_generic<float, 64>(a, stream);
    } else if (dtype == 0 && a.d == 128) {
        launch_generic<float, 128>(a, stream);
    } else if (dtype == 1 && a.d == 64) {
        launch_generic<uint16_t, 64>(a, stream);
    } else if (dtype == 1 && a.d == 128) {
        launch_generic<uint16_t, 128>(a, stream);
    } else {
        return hipErrorNotSupported;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.maxparts <= 1) return e;
    const dim3 grid((a.Hq + 3) / 4, a.num_seqs);
    if (dtype == 0 && a.d == 64)
        hipLaunchKernelGGL((decode_reduce_kernel<float, 64>), grid, dim3(256), 0, stream, a);
    else if (dtype == 0)
        hipLaunchKernelGGL((decode_reduce_kernel<float, 128>), grid, dim3(256), 0, stream, a);
    else if (a.d == 64)
        hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
