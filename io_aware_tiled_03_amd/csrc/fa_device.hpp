// fa_device.hpp - gfx950 device helpers shared by the attention kernels:
// vector types, MFMA wrappers, bf16 packing, exp2 and wave-level exchanges.
//
// MFMA register layouts used throughout (CDNA3/CDNA4 wave64):
//   v_mfma_f32_32x32x16_bf16  A (32 x 16): lane i holds row i%32, eight k-slots
//                             of half i/32; B (16 x 32): lane i holds column
//                             i%32, the same eight k-slots; C (32 x 32) fp32:
//                             lane i, register r holds
//                             row 8*(r/4) + 4*(i/32) + r%4, column i%32.
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

// First product of an accumulation chain: C = 0 as the inline constant operand.
__device__ __forceinline__ f32x16 mfma32x32x16_zero(const u32x4& a, const u32x4& b) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), f32x16{}, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: A (16 x 32): lane i holds row i%16, eight k-slots
// of group i/16; B (32 x 16): column i%16, the same k-slots; C (16 x 16) fp32:
// lane i, register r holds row 4*(i/16) + r, column i%16.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32_zero(const u32x4& a, const u32x4& b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), f32x4{}, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: as above with four k-slots per lane (k = 4*(i/16) + j).
__device__ __forceinline__ f32x4 mfma16x16x16(const u32x2& a, const u32x2& b, const f32x4& c) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, a),
                                                      __builtin_bit_cast(v4i16, b), c, 0, 0, 0);
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

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// DPP lane moves inside a row of 16 lanes (no LDS round trip).
enum : int {
    kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppRowRor4 = 0x124,    // rotate the 16-lane row by 4
    kDppRowRor8 = 0x128,    // rotate the 16-lane row by 8
    kDppHalfMirror = 0x141  // reverse each group of 8 lanes
};
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8 or 16); every lane gets its group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 8 || G == 16, "group of 8 or 16 lanes");
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    if constexpr (G == 8) {
        x += dpp_mov<kDppHalfMirror>(x);
    } else {
        x += dpp_mov<kDppRowRor4>(x);
        x += dpp_mov<kDppRowRor8>(x);
    }
    return x;
}

// Value held by lane (lane ^ 32): swaps the two halves of the wave.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives 16-bit element (i % 4) of the 8-byte pieces addressed by
// lanes 4j + i/4 of its group, for j = 0..3.  So if lane s of a group
// addresses row r0 + s/4, columns c0 + 4*(s%4) .. +3 of a row-major 16-bit
// matrix, lane i receives rows r0..r0+3 of column c0 + i: a column-major piece
// of a row-major tile, ready as MFMA operand slots.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds));
    return __builtin_bit_cast(u32x2, r);
}

// An MFMA A operand (8 bf16: four keys of one column, then the next four) from
// two transposing reads, assembled in place.
__device__ __forceinline__ u32x4 lds_read_tr16_x2(const void* lds_lo, const void* lds_hi) {
    u32x4 r;
    r.xy = lds_read_tr16(lds_lo);
    r.zw = lds_read_tr16(lds_hi);
    return r;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3 =
// 0x00020000).  Loads at byte offsets at or past `bytes` return zero, so a
// tile that runs past the end of a tensor needs no branch and no clamp.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// The same load marked non-temporal (data read once: keep it from displacing
// reused lines in the caches).
__device__ __forceinline__ u32x4 buf_ld16_nt(rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2));
}
// a ^ b ^ c in one instruction (v_bitop3_b32 with the three-input parity
// table 0x96; the compiler emits two XORs for the plain expression).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32 with 10 rounds (J. K. Salmon et al., "Parallel random numbers:
// as easy as 1, 2, 3", SC11): each round multiplies counter words 0 and 2 by
// the two round constants (one 32x32 -> 64-bit product each) and outputs
// (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key advances by the two Weyl
// constants before every round after the first.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return u32x4{c0, c1, c2, c3};
}

// Dropout of the (query, key) pairs of one 4 x 4 block: one Philox call with
// counter (key/4, query/4, b*H + h, offset) and key = the 64-bit seed; pair
// (query, key) is kept iff byte key%4 of word query%4 is >= thr.
struct Dropout {
    uint32_t seed_lo, seed_hi, offset;
    int thr;        // round(256 p), 1..255 when dropout is on
    float scale;    // 1 / (1 - thr/256)
    __device__ __forceinline__ u32x4 block(int key, int query, int bh) const {
        return philox4x32_10((uint32_t)key >> 2, (uint32_t)query >> 2, (uint32_t)bh, offset,
                             seed_lo, seed_hi);
    }
    // The word of a fixed query row (query % 4 = row): keep bits of keys 4k..4k+3.
    __device__ __forceinline__ static uint32_t row_word(const u32x4& w, int row) {
        const uint32_t a = (row & 1) ? w[1] : w[0];
        const uint32_t b = (row & 1) ? w[3] : w[2];
        return (row & 2) ? b : a;
    }
    __device__ __forceinline__ bool keep(uint32_t word, int byte) const {
        return (int)((word >> (8 * byte)) & 0xFFu) >= thr;
    }
};

// 4 x 4 transpose across each group of four lanes: lane r (0..3 within its
// quad) holds row r, a[0..3]; afterwards it holds column r, b[g] = lane g's
// a[r].  Two butterfly stages (partner lane r^1, then r^2) exchange one
// element per pair of indices through DPP quad permutes.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 a, int r) {
    // The four words as named scalars: indexing the vector with a choice of
    // two positions made the compiler build run-time-indexed extracts
    // (compares and select chains) around every exchange.
    uint32_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
    const bool h1 = (r & 1) != 0, h2 = (r & 2) != 0;
    {   // partner r ^ 1: pairs (0, 1) and (2, 3)
        const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(h1 ? a0 : a1), kDppXor1, 0xF, 0xF, false);
        const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(h1 ? a2 : a3), kDppXor1, 0xF, 0xF, false);
        a0 = h1 ? t0 : a0;
        a1 = h1 ? a1 : t0;
        a2 = h1 ? t1 : a2;
        a3 = h1 ? a3 : t1;
    }
    {   // partner r ^ 2: pairs (0, 2) and (1, 3)
        const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(h2 ? a0 : a2), kDppXor2, 0xF, 0xF, false);
        const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(h2 ? a1 : a3), kDppXor2, 0xF, 0xF, false);
        a0 = h2 ? t0 : a0;
        a2 = h2 ? a2 : t0;
        a1 = h2 ? t1 : a1;
        a3 = h2 ? a3 : t1;
    }
    return u32x4{a0, a1, a2, a3};
}

// 4 x 4 byte transpose inside one lane: out[e] holds byte e of in[0..3]
// (byte w of out[e] = byte e of in[w]).  v_perm_b32 picks bytes of {hi, lo}
// (selectors 0..3 address lo, 4..7 hi).
__device__ __forceinline__ u32x4 byte_transpose(const u32x4& a) {
    const uint32_t t01 = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);   // a0b0 a1b0 a0b1 a1b1
    const uint32_t t23 = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
    const uint32_t u01 = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);   // a0b2 a1b2 a0b3 a1b3
    const uint32_t u23 = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
    return u32x4{__builtin_amdgcn_perm(t23, t01, 0x05040100u), __builtin_amdgcn_perm(t23, t01, 0x07060302u),
                 __builtin_amdgcn_perm(u23, u01, 0x05040100u), __builtin_amdgcn_perm(u23, u01, 0x07060302u)};
}

// Block-sparse tile lists: writes to list[] (LDS), in increasing order, the
// tiles t < ntiles for which active(t) holds, and returns how many there are.
// Waves ballot chunks of 64 tiles, one thread places the chunks by a prefix
// sum, then every wave writes its tiles.  bal and off are LDS scratch of
// ceil(ntiles / 64) and ceil(ntiles / 64) + 1 entries.  Every thread of the
// workgroup must call it (it synchronises the workgroup).
template <int NW, typename F>
__device__ __forceinline__ int build_tile_list(F active, int ntiles, uint16_t* list, uint64_t* bal,
                                               int* off, int wave, int lane, int tid) {
    const int nchunks = (ntiles + 63) / 64;
    for (int c = wave; c < nchunks; c += NW) {
        const int t = 64 * c + lane;
        const bool act = t < ntiles && active(t);
        const uint64_t b = __builtin_amdgcn_ballot_w64(act);
        if (lane == 0) bal[c] = b;
    }
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int c = 0; c < nchunks; ++c) {
            off[c] = acc;
            acc += __builtin_popcountll(bal[c]);
        }
        off[nchunks] = acc;
    }
    __syncthreads();
    for (int c = wave; c < nchunks; c += NW) {
        const uint64_t b = bal[c];
        if ((b >> lane) & 1)
            list[off[c] + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u))] =
                (uint16_t)(64 * c + lane);
    }
    const int n = off[nchunks];
    __syncthreads();
    return n;
}

// Direct global -> LDS copy of 16 bytes per lane: lane i's bytes land at
// lds_base + 16*i (lds_base must be the same for the whole wave).  Completion
// is tracked by vmcnt, not by any register: wait with wait_vmem() before a
// barrier that publishes the data.
__device__ __forceinline__ void buf_ld16_lds(rsrc_t r, uint32_t byte_off, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                             byte_off, 0, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Epilogue stores through LDS.  The accumulators of the O^T-shaped products
// leave each lane 16 head-dim entries per 32-wide block of one row, so direct
// stores write 8-byte pieces of 32 different rows per instruction.  A wave
// instead writes its 32 rows, packed to bf16, into a wave-private LDS tile
// (stage_piece), then stores whole rows, 16 bytes per lane (store_rows).  A
// wave reads back only what it wrote, and one wave's LDS operations complete
// in order, so no barrier is needed between the two.
//
// stage_piece: row `row` (this lane's), head-dim entries d .. d+3.  The write
// is an asm ds_write_b64 (a store: no register result; the memory clobber
// orders it before the reads in store_rows).  As an ordinary C++ store into
// the staging buffers, which the main loops fill only with direct-to-LDS
// copies, it changed how the compiler treats the loops' LDS reads and pushed
// the 128-key-tile forward from 224 VGPRs to 256 plus spills.
__device__ __forceinline__ void stage_piece(uint16_t* tile, int stride, int row, int d, float a,
                                            float b, float c, float e) {
    u32x2 w;
    w[0] = pack_bf16x2(a, b);
    w[1] = pack_bf16x2(c, e);
    // the low 32 bits of a generic LDS address are the LDS byte address
    const uint32_t p = (uint32_t)(uintptr_t)(tile + row * stride + d);
    asm volatile("ds_write_b64 %0, %1" ::"v"(p), "v"(w) : "memory");
}
// store_rows: rows 0 .. nrows-1 (at most 32) of the tile to dst (row-major, D
// entries per row).
template <int D>
__device__ __forceinline__ void store_rows(const uint16_t* tile, int stride, uint16_t* dst, int nrows,
                                           int lane) {
    constexpr int CPR = D / 8;   // 16-byte pieces per row
#pragma unroll
    for (int t = 0; t < 32 * CPR / 64; ++t) {
        const int pos = t * 64 + lane, row = pos / CPR, c = (pos % CPR) * 8;
        const u32x4 v = ld16(tile + row * stride + c);
        if (row < nrows) st16(dst + (size_t)row * D + c, v);
    }
}

}  // namespace fa
