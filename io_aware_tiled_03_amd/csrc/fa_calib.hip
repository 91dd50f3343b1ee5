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

// ---------------------------------------------------------------------------
// LDS read patterns of the attention kernels' operand reads, each alone: eight
// waves per workgroup read one pattern eight times per step from a 64-row tile
// of `stride`-byte rows.  Row reads: ds_read_b128, lane i at row kperm(i % 32)
// (the kernels' row order), 16 bytes at column 16 * (i / 32) (+32 per read).
// Transposing reads: ds_read_b64_tr_b16, lane s of 16-lane group G at row
// 8 * (G / 2) + s / 4, column 32 * (G % 2) + 8 * (s % 4) bytes (+64 per read),
// and the second read of each pair four rows on; with SPACED, the rows go
// through the backward kernels' permutation inside each 16-row block (tile row
// 4a + b at LDS row 4b + a).

namespace {

__device__ __forceinline__ int cal_kperm(int m) {
    const int j = 4 * (m >> 3) + (m & 3);
    return 16 * (j >> 3) + 8 * ((m >> 2) & 1) + (j & 7);
}
__device__ __forceinline__ int cal_spaced(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

typedef short cal_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) cal_v4i16 cal_lds_v4i16;

template <bool TR, bool SPACED, int STRIDE, int D>
__global__ __launch_bounds__(512) void calib_lds_kernel(uint32_t* __restrict__ out, int iters) {
    __shared__ __attribute__((aligned(16))) unsigned char tile[64 * STRIDE + 256];
    const int lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < (64 * STRIDE + 256) / 4; i += 512)
        reinterpret_cast<uint32_t*>(tile)[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    const int G = lane >> 4, sl = lane & 15;
    int off;
    if constexpr (TR) {
        // tile rows r0 + s/4 and r0 + 4 + s/4: LDS rows 4*(s/4) + r0/4 (+1) when spaced
        off = (SPACED ? 4 * (sl >> 2) + 2 * (G >> 1) : 8 * (G >> 1) + (sl >> 2)) * STRIDE + 32 * (G & 1) + 8 * (sl & 3);
    } else {
        const int r = cal_kperm(lane & 31);
        off = (SPACED ? cal_spaced(r) : r) * STRIDE + 16 * (lane >> 5);
    }
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        int o = off;
        asm volatile("" : "+v"(o));   // the address is opaque: every step reads again
        const unsigned char* base = tile + o;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (TR) {
                constexpr int NC = D / 32;   // 64-byte column groups per row
                const int hi = (r / NC) * (SPACED ? 1 : 4) * STRIDE;
                const cal_v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((cal_lds_v4i16*)(base + (r % NC) * 64 + hi));
                acc += (uint32_t)(uint16_t)v.x ^ ((uint32_t)(uint16_t)v.y << 16) ^ (uint32_t)(uint16_t)v.z ^
                       ((uint32_t)(uint16_t)v.w << 16);
            } else {
                constexpr int NC = D / 16;   // 32-byte column steps per row
                const uint4 v = *reinterpret_cast<const uint4*>(base + (r % NC) * 32 + (r / NC) * 32 * STRIDE);
                acc += v.x ^ v.y ^ v.z ^ v.w;
            }
        }
    }
    out[blockIdx.x * 512 + threadIdx.x] = acc;
}

struct LdsPattern {
    const char* name;
    int bytes_per_read;   // per wave
    void (*launch)(int grid, uint32_t* out, int iters, hipStream_t st);
};

template <bool TR, bool SPACED, int STRIDE, int D>
void launch_lds(int grid, uint32_t* out, int iters, hipStream_t st) {
    calib_lds_kernel<TR, SPACED, STRIDE, D><<<grid, 512, 0, st>>>(out, iters);
}

const LdsPattern kLds[] = {
    {"row reads, 272-byte rows (d=128)", 1024, launch_lds<false, false, 272, 128>},
    {"row reads, 288-byte rows (d=128)", 1024, launch_lds<false, false, 288, 128>},
    {"row reads, 320-byte rows (d=128)", 1024, launch_lds<false, false, 320, 128>},
    {"row reads, 272-byte rows, rows permuted (d=128)", 1024, launch_lds<false, true, 272, 128>},
    {"transposing reads, 272-byte rows (d=128)", 512, launch_lds<true, false, 272, 128>},
    {"transposing reads, 288-byte rows (d=128)", 512, launch_lds<true, false, 288, 128>},
    {"transposing reads, 304-byte rows (d=128)", 512, launch_lds<true, false, 304, 128>},
    {"transposing reads, 320-byte rows (d=128)", 512, launch_lds<true, false, 320, 128>},
    {"transposing reads, 272-byte rows, rows permuted (d=128)", 512, launch_lds<true, true, 272, 128>},
    {"row reads, 144-byte rows (d=64)", 1024, launch_lds<false, false, 144, 64>},
    {"transposing reads, 144-byte rows (d=64)", 512, launch_lds<true, false, 144, 64>},
    {"transposing reads, 144-byte rows, rows permuted (d=64)", 512, launch_lds<true, true, 144, 64>},
};
constexpr int kNumLds = sizeof(kLds) / sizeof(kLds[0]);

}  // namespace

extern "C" int fa_calib_lds_count(void) { return kNumLds; }

extern "C" const char* fa_calib_lds_name(int pattern) {
    return (pattern >= 0 && pattern < kNumLds) ? kLds[pattern].name : nullptr;
}

extern "C" double fa_calib_lds_bytes(int pattern, int grid, int iters) {
    if (pattern < 0 || pattern >= kNumLds || grid < 1 || iters < 1) return 0.0;
    // 8 waves per workgroup, 8 reads per step
    return (double)grid * 8.0 * (double)iters * 8.0 * kLds[pattern].bytes_per_read;
}

extern "C" fa_status fa_calib_lds(int pattern, int grid, int iters, unsigned int* out, void* stream) {
    if (!out) return FA_ERR_NULL;
    if ((uintptr_t)out & 15) return FA_ERR_ALIGN;
    if (pattern < 0 || pattern >= kNumLds || grid < 1 || grid > FA_CALIB_MAX_GRID || iters < 1 ||
        iters > FA_CALIB_MAX_ITERS)
        return FA_ERR_ARG;
    kLds[pattern].launch(grid, reinterpret_cast<uint32_t*>(out), iters, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// HBM streaming read: each workgroup reads its own contiguous share of a
// buffer in 16-byte chunks with non-temporal loads (the load form of the
// decode kernels), its 256 lanes on consecutive chunks and 8 chunks in flight
// per lane (32 KB per workgroup and step); the chunks are folded into one
// checksum per lane.

namespace {

typedef uint32_t cal_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void calib_read_kernel(const cal_u32x4* __restrict__ buf, size_t nchunks,
                                                         uint32_t* __restrict__ out) {
    const size_t per = (nchunks + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * per;
    const size_t end = beg + per < nchunks ? beg + per : nchunks;
    uint32_t acc = 0;
    size_t i = beg + threadIdx.x;
    for (; i + 7 * 256 < end; i += 8 * 256) {
        cal_u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * 256);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += 256) {
        const cal_u32x4 v = __builtin_nontemporal_load(buf + i);
        acc += v.x ^ v.y ^ v.z ^ v.w;
    }
    out[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" fa_status fa_calib_hbm_read(const void* buf, size_t bytes, int grid, unsigned int* out, void* stream) {
    if (!buf || !out) return FA_ERR_NULL;
    if (((uintptr_t)buf | (uintptr_t)out) & 15) return FA_ERR_ALIGN;
    if (bytes == 0 || (bytes & 15) || grid < 1 || grid > FA_CALIB_MAX_GRID) return FA_ERR_ARG;
    calib_read_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const cal_u32x4*>(buf), bytes / 16,
                                                                        reinterpret_cast<uint32_t*>(out));
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
