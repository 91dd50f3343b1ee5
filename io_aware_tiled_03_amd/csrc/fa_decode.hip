// fa_decode.hip - split-KV decode for gfx950: one query row per (b, h)
// against its KV cache, the HBM-bound case ("Atenção eficiente —
// FlashAttention, sparse e híbrida", "FlashAttention não acelera o decode").
//
// decode_split_kernel: one workgroup per (split, h, b) streams the contiguous
//   key range [s*chunk, min((s+1)*chunk, L_b)) of its sequence.  Lanes cover
//   16-byte pieces of a key row (16 lanes per d=128 row), so every load
//   instruction of a wave reads whole consecutive rows; the dot products are
//   reduced across the lanes of a row, and each wave keeps its own running
//   max m, sum l and output o (the block recurrence of the "flash-attention"
//   page, "como funciona").  The four waves are merged through LDS and the
//   split writes o_s = o/l and lse_s = tau*m + ln(l) (or -inf when empty).
// decode_merge_kernel: one wave per (b, h) combines the splits with the same
//   merge rule: LSE = ln sum_s exp(lse_s), O = sum_s exp(lse_s - LSE) o_s.
// Key rows at or beyond L_b are never read: padding may hold anything.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {   // bf16: 8 elements per 16-byte piece
    static constexpr int PER16 = 8;
    __device__ static void unpack(const u32x4& w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf16lo(w[i]); f[2 * i + 1] = bf16hi(w[i]); }
    }
};
template <> struct Elem<float> {      // fp32: 4 elements per 16-byte piece
    static constexpr int PER16 = 4;
    __device__ static void unpack(const u32x4& w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // copy the element first: bit-casting the vector element lvalue
            // directly reads element 0 with this compiler
            const uint32_t x = w[i];
            f[i] = __builtin_bit_cast(float, x);
        }
    }
};

// Sum of a partial dot product over the CPR lanes that hold one key row.
template <int CPR>
__device__ __forceinline__ float row_sum(float x) {
    if constexpr (CPR <= 16) {
        return group_sum<CPR>(x);
    } else {
        x = group_sum<16>(x);
        return x + __shfl_xor(x, 16, 64);
    }
}

#ifndef FA_DECODE_U
#define FA_DECODE_U 4
#endif
#ifndef FA_DECODE_ROTATE
#define FA_DECODE_ROTATE 0
#endif
#ifndef FA_DECODE_NT
#define FA_DECODE_NT 1
#endif

// Streaming 16-byte load of the KV cache (read once: optionally non-temporal).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
#if FA_DECODE_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
    return ld16(p);
#endif
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int* __restrict__ seqlens, int B, int H, int N_max, int chunk, float scale_log2,
    float tau, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
    constexpr int PER = Elem<T>::PER16;
    constexpr int CPR = D / PER;          // lanes per key row
    constexpr int KPL = 64 / CPR;         // keys per wave load instruction
    constexpr int U = FA_DECODE_U;        // loads per operand per pipeline stage
    constexpr int KPI = U * KPL;          // keys per wave per stage
    // Linear grid with (b, h) fastest: consecutive workgroups, which the
    // dispatcher deals round-robin to the 8 XCDs, belong to different
    // sequences, so every XCD gets a share of every split index (high splits
    // are often empty); split 0, always full, is dispatched first.
    const int BH = H * B;
    const int s = (int)(blockIdx.x / (unsigned)BH);
    const int bhi = (int)(blockIdx.x % (unsigned)BH);
    const int b = bhi / H, h = bhi % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % CPR, g = lane / CPR;
    const size_t bh = (size_t)bhi;
    const size_t wsi = (size_t)s * BH + bhi;

    const int L = min(max(seqlens[b], 0), N_max);
    const int kb = s * chunk, ke = min(L, kb + chunk);
    if (kb >= ke) {   // empty split: contributes nothing to the merge
        if (tid < D) ws_o[wsi * D + tid] = 0.f;
        if (tid == 0) ws_lse[wsi] = neg_inf();
        return;
    }

    float qv[PER];
    Elem<T>::unpack(ld16(Q + bh * D + c * PER), qv);
    const T* Kb = K + bh * (size_t)N_max * D + c * PER;
    const T* Vb = V + bh * (size_t)N_max * D + c * PER;

    float m = neg_inf(), l = 0.f, o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;

    // Keys past ke are clamped to row ke-1 (always a valid row, so finite) and
    // their scores are masked to -inf: no branch around any load.
    auto load = [&](u32x4* kr, u32x4* vr, int k0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t row = (size_t)min(k0 + u * KPL + g, ke - 1) * D;
            kr[u] = ld16_stream(Kb + row);
            vr[u] = ld16_stream(Vb + row);
        }
    };
    auto consume = [&](const u32x4* kr, const u32x4* vr, int k0) {
        float sc[U];
        float mx = neg_inf();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kv[PER];
            Elem<T>::unpack(kr[u], kv);
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc = __builtin_fmaf(qv[i], kv[i], acc);
            acc = row_sum<CPR>(acc);
            sc[u] = (k0 + u * KPL + g < ke) ? acc : neg_inf();
            mx = fmaxf(mx, sc[u]);
        }
#pragma unroll
        for (int off = CPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2((m - mnew) * scale_log2);
        const float mc = mnew * scale_log2;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = fast_exp2(__builtin_fmaf(sc[u], scale_log2, -mc));
            l += p;
            float vv[PER];
            Elem<T>::unpack(vr[u], vv);
#pragma unroll
            for (int i = 0; i < PER; ++i) o[i] = __builtin_fmaf(p, vv[i], o[i]);
        }
        m = mnew;
    };

    // The chunk is walked in stages of KPI keys; wave w takes stages w, w+4, ...
    // Each workgroup starts at a rotated stage so that concurrently running
    // workgroups, whose chunks begin at large power-of-two offsets, do not all
    // hit the same HBM channels in lock step (the softmax merge does not depend
    // on the order of the keys).  Two register stages: the loads of the next
    // keys are in flight while the current ones are consumed.
    const int nst = (ke - kb + KPI - 1) / KPI;
    const int rot = (int)(blockIdx.x % (unsigned)nst) * FA_DECODE_ROTATE;
    auto stage_key = [&](int t) {
        int p = t + rot;
        p = p >= nst ? p - nst : p;
        return kb + p * KPI;
    };
    int t = wave;
    if (t < nst) {
        u32x4 ka[U], va[U], kn[U], vn[U];
        load(ka, va, stage_key(t));
        while (true) {
            const int t1 = t + 4;
            if (t1 < nst) load(kn, vn, stage_key(t1));
            consume(ka, va, stage_key(t));
            if (t1 >= nst) break;
            const int t2 = t1 + 4;
            if (t2 < nst) load(ka, va, stage_key(t2));
            consume(kn, vn, stage_key(t1));
            if (t2 >= nst) break;
            t = t2;
        }
    }
    // combine the KPL key groups of the wave (lanes with equal c)
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) {
        const float mo = __shfl_xor(m, off, 64);
        const float lo = __shfl_xor(l, off, 64);
        const float mn = fmaxf(m, mo);
        const float a0 = (m == neg_inf()) ? 0.f : fast_exp2((m - mn) * scale_log2);
        const float a1 = (mo == neg_inf()) ? 0.f : fast_exp2((mo - mn) * scale_log2);
        l = l * a0 + lo * a1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const float oo = __shfl_xor(o[i], off, 64);
            o[i] = o[i] * a0 + oo * a1;
        }
        m = mn;
    }
    // combine the four waves
    __shared__ float sm[4], sl[4], so[4][D];
    if (g == 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) so[wave][c * PER + i] = o[i];
        if (c == 0) { sm[wave] = m; sl[wave] = l; }
    }
    __syncthreads();
    if (tid < D) {
        float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a = (sm[w] == neg_inf()) ? 0.f : fast_exp2((sm[w] - M) * scale_log2);
            lt += sl[w] * a;
            ot += so[w][tid] * a;
        }
        ws_o[wsi * D + tid] = ot / lt;
        if (tid == 0) ws_lse[wsi] = M * tau + __logf(lt);
    }
}

// One wave per (b, h): lane t owns head-dim entries t and t + 64.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int S, int BH,
    T* __restrict__ O, float* __restrict__ LSE) {
    const int bh = blockIdx.x, t = threadIdx.x;
    float M = neg_inf();
    for (int s = 0; s < S; ++s) M = fmaxf(M, ws_lse[(size_t)s * BH + bh]);
    constexpr int PL = D / 64;
    float acc[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) acc[i] = 0.f;
    float sum = 0.f;
    if (M != neg_inf()) {
        for (int s = 0; s < S; ++s) {
            const float ls = ws_lse[(size_t)s * BH + bh];
            if (ls == neg_inf()) continue;
            const float w = __expf(ls - M);
            sum += w;
#pragma unroll
            for (int i = 0; i < PL; ++i) acc[i] += w * ws_o[((size_t)s * BH + bh) * D + t + 64 * i];
        }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const float v = acc[i] * inv;
        if constexpr (sizeof(T) == 2) {
            typedef __bf16 bf;
            reinterpret_cast<bf*>(O)[(size_t)bh * D + t + 64 * i] = (bf)v;
        } else {
            O[(size_t)bh * D + t + 64 * i] = v;
        }
    }
    if (t == 0) LSE[bh] = (M == neg_inf()) ? neg_inf() : M + __logf(sum);
}

template <typename T, int D>
void launch(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(a.num_splits * a.B * a.H), dim3(256), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.seqlens, a.B, a.H, a.N_max,
                       a.chunk, a.tau * kLog2e, a.tau, a.ws_o, a.ws_lse);
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.B * a.H), dim3(64), 0, st, a.ws_o,
                       a.ws_lse, a.num_splits, a.B * a.H, (T*)a.o, a.lse);
}

}  // namespace

int decode_chunk(int N_max, int splits) {
    int c = (N_max + splits - 1) / splits;
    return (c + 63) / 64 * 64;
}

int decode_splits(int B, int H, int N_max, int d, int requested) {
    (void)d;
    if (requested > 0) {
        const int c = decode_chunk(N_max, requested);
        return (N_max + c - 1) / c;
    }
    // Automatic: the shortest chunk (>= 256 keys) that keeps the grid at or
    // below 16384 workgroups.
    const long bh = (long)B * H;
    int c = 256;
    while (c < N_max && bh * ((N_max + c - 1) / c) > 16384) c *= 2;
    return (N_max + c - 1) / c;
}

size_t decode_ws_bytes(int B, int H, int d, int splits) {
    return (size_t)splits * B * H * (size_t)(d + 1) * sizeof(float);
}

void launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.dtype == kBF16) {
        a.d == 64 ? launch<uint16_t, 64>(a, st) : launch<uint16_t, 128>(a, st);
    } else {
        a.d == 64 ? launch<float, 64>(a, st) : launch<float, 128>(a, st);
    }
}

}  // namespace fa
