// fa_calib.hip - synthetic matrix-core loops that measure what rate this part
// reaches for a given instruction mix per bf16 product (fa_calib.h).
//
// An attention kernel cannot beat the rate at which the chip runs its own mix
// of work per matrix instruction: each v_mfma_f32_32x32x16_bf16 of the
// prefill forward needs its A operand (1 KB per wave) from LDS, and the
// softmax adds about one exp2 and several fp32 vector instructions per
// product.  These loops run the same mixes with nothing else (no HBM traffic,
// no barriers, no masking), so their rate is a ceiling measured on the part,
// next to the nominal 2.5 PFLOP/s.
//
// Each wave keeps NACC independent accumulator chains.  Per product it takes
// its A operand from registers or, with FROM_LDS, by one ds_read_b128 from a
// wave-private LDS area (64 lanes x 16 bytes, conflict-free), and issues NFMA
// fp32 FMAs on eight independent chains and NEXP exp2 (each followed by one
// FMA that maps the result back into [0, 1), so the chains stay finite).
// The operand bits change from product to product (four A and four B
// operands in rotation, or a different LDS row per product).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_calib.h"

namespace {

typedef __bf16 cal_bf16x8 __attribute__((ext_vector_type(8)));
typedef float cal_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSeedChunks = 4096;   // 16-byte operand chunks in the seed buffer (64 KB)

template <int NACC, int NFMA, int NEXP, bool FROM_LDS>
__global__ __launch_bounds__(256) void calib_kernel(const uint4* __restrict__ seed, float* __restrict__ out,
                                                    int iters) {
    // LDS rows (1 KB each) per wave: 2*NACC read in one pass of the unrolled
    // pair of steps, plus 8 so that consecutive pairs read different rows.
    constexpr int ROWS = FROM_LDS ? 2 * NACC + 8 : 1;
    __shared__ uint4 lds[4][ROWS * 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = (blockIdx.x * 256 + threadIdx.x) & (kSeedChunks - 1);
    uint4 A[4], B[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        A[i] = seed[(g + 512 * i) & (kSeedChunks - 1)];
        B[i] = seed[(g + 512 * i + 2048) & (kSeedChunks - 1)];
    }
    if constexpr (FROM_LDS) {
        for (int i = 0; i < ROWS; ++i) lds[w][i * 64 + lane] = seed[(g + 97 * i) & (kSeedChunks - 1)];
        __syncthreads();
    }
    cal_f32x16 acc[NACC];
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = (cal_f32x16){};
    float z[8], x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        z[j] = 0.01f * (lane + j);
        x[j] = 0.001f * (lane + 3 * j);
    }
    for (int it = 0; it < iters; it += 2) {
        const uint4* rows = &lds[w][lane] + (FROM_LDS ? ((it >> 1) & 1) * 8 * 64 : 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int k = 0; k < NACC; ++k) {
                const uint4 a = FROM_LDS ? rows[(h * NACC + k) * 64] : A[k & 3];
                const uint4 b = B[(k + 2 * h) & 3];
                acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(cal_bf16x8, a),
                                                                  __builtin_bit_cast(cal_bf16x8, b), acc[k], 0, 0,
                                                                  0);
#pragma unroll
                for (int f = 0; f < NFMA; ++f) {
                    const int j = (k * NFMA + f) & 7;
                    z[j] = __builtin_fmaf(z[j], 0.999f, 0.001f);
                }
#pragma unroll
                for (int e = 0; e < NEXP; ++e) {
                    const int j = (k * NEXP + e) & 7;
                    x[j] = __builtin_fmaf(__builtin_amdgcn_exp2f(x[j]), -0.5f, 1.0f);
                }
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NACC; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[k][r];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += z[j] + x[j];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

struct Mix {
    const char* name;
    int nacc;
    void (*launch)(int grid, const uint4* seed, float* out, int iters, hipStream_t st);
};

template <int NACC, int NFMA, int NEXP, bool FROM_LDS>
void launch_mix(int grid, const uint4* seed, float* out, int iters, hipStream_t st) {
    calib_kernel<NACC, NFMA, NEXP, FROM_LDS><<<grid, 256, 0, st>>>(seed, out, iters);
}

// Accumulator chains per wave set the occupancy: eight chains (128 accumulator
// registers) leave one wave per SIMD, four chains two.
const Mix kMixes[] = {
    {"products only, operands in registers, 1 wave per SIMD", 8, launch_mix<8, 0, 0, false>},
    {"A operand from LDS (1 KB ds_read_b128 per product), 2 waves per SIMD", 4, launch_mix<4, 0, 0, true>},
    {"A from LDS + 1 exp2 and 3 fp32 FMA per product, 2 waves per SIMD", 4, launch_mix<4, 2, 1, true>},
    {"A from LDS + 1 exp2 and 5 fp32 FMA per product, 2 waves per SIMD", 4, launch_mix<4, 4, 1, true>},
    {"A from LDS + 1 exp2 and 7 fp32 FMA per product, 2 waves per SIMD", 4, launch_mix<4, 6, 1, true>},
};
constexpr int kNumMixes = sizeof(kMixes) / sizeof(kMixes[0]);

}  // namespace

extern "C" int fa_calib_mix_count(void) { return kNumMixes; }

extern "C" const char* fa_calib_mix_name(int mix) {
    return (mix >= 0 && mix < kNumMixes) ? kMixes[mix].name : nullptr;
}

extern "C" double fa_calib_flops(int mix, int grid, int iters) {
    if (mix < 0 || mix >= kNumMixes || grid < 1 || iters < 2) return 0.0;
    // per wave: iters steps of NACC products of 2 * 32 * 32 * 16 flops; 4 waves per workgroup
    return (double)grid * 4.0 * (double)iters * kMixes[mix].nacc * 32768.0;
}

extern "C" fa_status fa_calib_mfma(int mix, int grid, int iters, const void* seed, float* out, void* stream) {
    if (!seed || !out) return FA_ERR_NULL;
    if (((uintptr_t)seed | (uintptr_t)out) & 15) return FA_ERR_ALIGN;
    if (mix < 0 || mix >= kNumMixes || grid < 1 || grid > FA_CALIB_MAX_GRID || iters < 2 ||
        iters > FA_CALIB_MAX_ITERS || (iters & 1))
        return FA_ERR_ARG;
    kMixes[mix].launch(grid, static_cast<const uint4*>(seed), out, iters, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
