// pkv_device.h -- device helpers shared by the gfx950 kernels of libpkv.
//
// Written for CDNA4 only: 64-wide wavefronts, bf16 MFMA, DPP row operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Word 3 of a raw (stride 0) buffer resource on CDNA: 32-bit data format, so
// buffer loads range-check against num_records and return zeros beyond it.
constexpr int kBufWord3 = 0x00020000;

// A bf16 value is the upper half of an fp32: widening is a shift or a mask.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (the hardware conversion,
// v_cvt_pk_bf16_f32); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global loads/stores through the vector memory path.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// DPP lane exchange inside a 16-lane row (the controls are the CDNA DPP
// encodings: quad_perm, row_half_mirror, row_mirror).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Max / sum over the 16 lanes of a row; every lane of the row gets the result.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<kQuadSwap1>(x));
    x = fmaxf(x, dpp<kQuadSwap2>(x));
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    x += dpp<kRowHalfMirror>(x);
    x += dpp<kRowMirror>(x);
    return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
    int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}
__device__ __forceinline__ float shfl(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// Exchange across lane rows with the gfx950 permlane swaps (VALU, no LDS):
// permlane32_swap(x, x) hands each lane the values of lanes (l & 31) and
// (l & 31) + 32; permlane16_swap(x, x) those of lanes (l & ~16) and (l | 16).
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum over a whole wave (64 lanes).
__device__ __forceinline__ float wave_max(float x) { return xor32_max(xor16_max(row16_max(x))); }
__device__ __forceinline__ float wave_sum(float x) { return xor32_sum(xor16_sum(row16_sum(x))); }

// Compiler-level ordering point for LDS traffic exchanged between lanes of
// one wave (DS instructions of a wave execute in order).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pkv
