// fa_device.hpp - gfx950 device helpers shared by the attention kernels:
// vector types, MFMA wrappers, bf16 packing, exp2 and wave-level exchanges.
//
// MFMA register layouts used throughout (CDNA3/CDNA4 wave64):
//   v_mfma_f32_32x32x16_bf16  A (32 x 16): lane i holds row i%32, eight k-slots
//                             of half i/32; B (16 x 32): lane i holds column
//                             i%32, the same eight k-slots; C (32 x 32) fp32:
//                             lane i, register r holds
//                             row 8*(r/4) + 4*(i/32) + r%4, column i%32.
//   v_mfma_f32_32x32x2_f32    A: lane i holds row i%32, k = i/32; B: column
//                             i%32, k = i/32; C as above.
// A and B always receive the same logical k in the same (half, slot), so the
// hardware's internal k order never matters; only the row/column/C mapping
// above does.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// exp2 on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values -> two bf16 (round to nearest even) packed in one dword,
// first argument in the low half (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Value held by lane (lane ^ 32): swaps the two halves of the wave.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace fa
