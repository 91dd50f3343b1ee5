// fa_f32.hip - the fp32 (FA_F32) forward and backward: float inputs, float
// arithmetic throughout, for the tight 1e-5 comparisons of debugging runs.
//
// Same mathematics as the bf16 kernels ("flash-attention" encyclopedia page,
// "como funciona": scores tau q.k, running max m and sum l with rescaling,
// LSE = m + ln l saved; backward D_i = dO_i . O_i, dV = P^T dO, dS = P o (dP -
// D), dQ = tau dS K, dK = tau dS^T Q), computed with vector FMAs rather than
// MFMA: on this part the fp32 matrix and vector peaks are the same, so MFMA
// buys nothing here, and the vector form keeps each dot product in a fixed
// order.  Each row (query or key) is spread over LPR lanes of a wave, each
// lane holding D / LPR of its head-dim entries, so the per-row registers
// stay within one wave's budget at d = 128 (no scratch); the LPR partial dot
// products are added across lanes.  Rows of K, V (forward, dQ) or Q, dO (dK
// and dV) are read straight from global memory: every row of the wave reads
// the same key (query) at once, so the loads are served by the caches.
//
// Masks: causal, with a sliding window and sinks; dropout with the mask of
// Dropout::block (the bf16 kernels' layout).  Block-sparse masks are bf16 only.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

// Sum of x over the LPR lanes that share a row (lanes r, r + 64/LPR, ...).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16, "lanes per row");
    if constexpr (LPR >= 16) x += __shfl_xor(x, 4, 64);
    if constexpr (LPR >= 8) x += __shfl_xor(x, 8, 64);
    if constexpr (LPR >= 4) x += __shfl_xor(x, 16, 64);
    if constexpr (LPR >= 2) x += __shfl_xor(x, 32, 64);
    return x;
}

// Key j visible to query i (causal: j <= i and (i - j < window or j < sinks)).
__device__ __forceinline__ bool visible(int i, int j, bool causal, int window, int sinks) {
    return !causal || (j <= i && (i - j < window || j < sinks));
}

__device__ __forceinline__ bool kept(const Dropout& drop, int i, int j, int bh) {
    const uint32_t w = Dropout::row_word(drop.block(j, i, bh), i & 3);
    return drop.keep(w, j & 3);
}

// Forward: a workgroup of NS waves takes 64 / LPR query rows; wave w walks
// the w-th of NS equal slices of the rows' key range, keys in chunks of 8
// (the chunk's scores in registers, max, rescale, exp, accumulate), and the
// NS partial (m, l, o) of each row are combined through LDS with the same
// rescaling rule.  The row reads have no branch around them, so a chunk's
// reads are in flight together; 8 keys keep them within the register budget
// (32 spilled at d = 128) and measured fastest (the 1x1x256x64 forward 114 ->
// 77 us against chunks of 32 read one key at a time).  The key split shortens
// each wave's chain of dependent reads NS-fold.
template <int D, int LPR, int NS>
__global__ __launch_bounds__(64 * NS) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int N, float scale_log2, float tau,
    int causal, int window, int sinks, Dropout drop) {
    constexpr int RPW = 64 / LPR, DS = D / LPR, KC = 8;
    __shared__ float s_o[NS][RPW][D], s_m[NS][RPW], s_l[NS][RPW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = (int)(blockIdx.x % BH);
    const int rt = (int)(blockIdx.x / BH);
    const int rr = lane % RPW, row = rt * RPW + rr, c0 = (lane / RPW) * DS;
    const size_t base = (size_t)bh * N * D;
    const bool live = row < N;
    float q[DS], o[DS];
#pragma unroll
    for (int c = 0; c < DS; c += 4) {
        const f32x4 t = live ? *reinterpret_cast<const f32x4*>(Q + base + (size_t)row * D + c0 + c)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
        q[c] = t[0]; q[c + 1] = t[1]; q[c + 2] = t[2]; q[c + 3] = t[3];
        o[c] = o[c + 1] = o[c + 2] = o[c + 3] = 0.f;
    }
    float m = neg_inf(), l = 0.f;
    const int last_row = min(N, rt * RPW + RPW) - 1;
    const int kend = causal ? last_row + 1 : N;
    // this wave's slice of the keys, whole chunks
    const int nch = (kend + KC - 1) / KC;
    const int kb = KC * (nch * wave / NS), ke = min(kend, KC * (nch * (wave + 1) / NS));
    for (int k0 = kb; k0 < ke; k0 += KC) {
        float s[KC];
        float mx = neg_inf();
        // Keys past kend read the row kend - 1 instead (their scores are
        // masked to -inf, so their p is 0): no branch around any load, so the
        // chunk's row reads can all be in flight together.
#pragma unroll
        for (int u = 0; u < KC; ++u) {
            const int j = k0 + u;
            float acc = 0.f;
            const float* kr = K + base + (size_t)min(j, kend - 1) * D + c0;
#pragma unroll
            for (int c = 0; c < DS; c += 4) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(kr + c);
                acc = __builtin_fmaf(q[c], t[0], acc);
                acc = __builtin_fmaf(q[c + 1], t[1], acc);
                acc = __builtin_fmaf(q[c + 2], t[2], acc);
                acc = __builtin_fmaf(q[c + 3], t[3], acc);
            }
            acc = row_sum<LPR>(acc);
            s[u] = (j < kend && visible(row, j, causal, window, sinks)) ? acc : neg_inf();
            mx = fmaxf(mx, s[u]);
        }
        const float mnew = fmaxf(m, mx);
        // a row with no visible key so far (window) keeps m = -inf, l = 0, o = 0
        const float alpha = m == mnew ? 1.f : fast_exp2((m - mnew) * scale_log2);
        const float mc = mnew == neg_inf() ? 0.f : mnew * scale_log2;
        l *= alpha;
#pragma unroll
        for (int c = 0; c < DS; ++c) o[c] *= alpha;
#pragma unroll
        for (int u = 0; u < KC; ++u) {
            const int j = k0 + u;
            float p = fast_exp2(__builtin_fmaf(s[u], scale_log2, -mc));   // 0 past kend
            l += p;
            if (drop.thr > 0 && !kept(drop, row, j, bh)) p = 0.f;
            const float* vr = V + base + (size_t)min(j, kend - 1) * D + c0;
#pragma unroll
            for (int c = 0; c < DS; c += 4) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(vr + c);
                o[c] = __builtin_fmaf(p, t[0], o[c]);
                o[c + 1] = __builtin_fmaf(p, t[1], o[c + 1]);
                o[c + 2] = __builtin_fmaf(p, t[2], o[c + 2]);
                o[c + 3] = __builtin_fmaf(p, t[3], o[c + 3]);
            }
        }
        m = mnew;
    }
    if constexpr (NS > 1) {   // combine the slices: rescale each to the largest m
#pragma unroll
        for (int c = 0; c < DS; ++c) s_o[wave][rr][c0 + c] = o[c];
        if (c0 == 0) {
            s_m[wave][rr] = m;
            s_l[wave][rr] = l;
        }
        __syncthreads();
        if (wave != 0) return;
        float mm = neg_inf();
#pragma unroll
        for (int w = 0; w < NS; ++w) mm = fmaxf(mm, s_m[w][rr]);
        l = 0.f;
#pragma unroll
        for (int c = 0; c < DS; ++c) o[c] = 0.f;
#pragma unroll
        for (int w = 0; w < NS; ++w) {
            const float mw = s_m[w][rr];
            const float a = mw == neg_inf() ? 0.f : fast_exp2((mw - mm) * scale_log2);
            l = __builtin_fmaf(a, s_l[w][rr], l);
#pragma unroll
            for (int c = 0; c < DS; ++c) o[c] = __builtin_fmaf(a, s_o[w][rr][c0 + c], o[c]);
        }
        m = mm;
    }
    if (live) {
        const float inv = (drop.thr > 0 ? drop.scale : 1.f) / l;
#pragma unroll
        for (int c = 0; c < DS; c += 4)
            *reinterpret_cast<f32x4*>(O + base + (size_t)row * D + c0 + c) =
                f32x4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
        if (c0 == 0) LSE[(size_t)bh * N + row] = m * tau + logf(l);
    }
}

// Backward, dQ (and D): one wave = 64 / LPR query rows; walks the keys.
template <int D, int LPR>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ Dv, float* __restrict__ dQ, int BH, int N, float scale_log2, float tau,
    int causal, int window, int sinks, Dropout drop) {
    constexpr int RPW = 64 / LPR, DS = D / LPR;
    const int lane = threadIdx.x;
    const int bh = (int)(blockIdx.x % BH);
    const int rt = (int)(blockIdx.x / BH);
    const int row = rt * RPW + lane % RPW, c0 = (lane / RPW) * DS;
    const size_t base = (size_t)bh * N * D;
    const bool live = row < N;
    float q[DS], g[DS], dq[DS];
    float dpart = 0.f;
#pragma unroll
    for (int c = 0; c < DS; c += 4) {
        const size_t off = base + (size_t)row * D + c0 + c;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 tq = live ? *reinterpret_cast<const f32x4*>(Q + off) : z;
        const f32x4 tg = live ? *reinterpret_cast<const f32x4*>(dO + off) : z;
        const f32x4 to = live ? *reinterpret_cast<const f32x4*>(O + off) : z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            q[c + e] = tq[e];
            g[c + e] = tg[e];
            dq[c + e] = 0.f;
            dpart = __builtin_fmaf(tg[e], to[e], dpart);
        }
    }
    // D_i = dO_i . O_i ("como funciona": D_i = P_i . dP_i = dO_i . O_i)
    const float Di = row_sum<LPR>(dpart);
    if (live && c0 == 0) Dv[(size_t)bh * N + row] = Di;
    const float lse2 = live ? LSE[(size_t)bh * N + row] * kLog2e : __builtin_inff();
    const int last_row = min(N, rt * RPW + RPW) - 1;
    const int kend = causal ? last_row + 1 : N;
    for (int j = 0; j < kend; ++j) {
        const float* kr = K + base + (size_t)j * D + c0;
        const float* vr = V + base + (size_t)j * D + c0;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < DS; c += 4) {
            const f32x4 tk = *reinterpret_cast<const f32x4*>(kr + c);
            const f32x4 tv = *reinterpret_cast<const f32x4*>(vr + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = __builtin_fmaf(q[c + e], tk[e], s);
                dp = __builtin_fmaf(g[c + e], tv[e], dp);
            }
        }
        s = row_sum<LPR>(s);
        dp = row_sum<LPR>(dp);
        const float p = (live && visible(row, j, causal, window, sinks))
                            ? fast_exp2(__builtin_fmaf(s, scale_log2, -lse2)) : 0.f;
        if (drop.thr > 0) dp = kept(drop, row, j, bh) ? dp * drop.scale : 0.f;
        const float ds = p * (dp - Di);
#pragma unroll
        for (int c = 0; c < DS; c += 4) {
            const f32x4 tk = *reinterpret_cast<const f32x4*>(kr + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) dq[c + e] = __builtin_fmaf(ds, tk[e], dq[c + e]);
        }
    }
    if (live) {
#pragma unroll
        for (int c = 0; c < DS; c += 4)
            *reinterpret_cast<f32x4*>(dQ + base + (size_t)row * D + c0 + c) =
                f32x4{dq[c] * tau, dq[c + 1] * tau, dq[c + 2] * tau, dq[c + 3] * tau};
    }
}

// Backward, dK and dV: one wave = 64 / LPR keys; walks the queries that can
// see them (it reads the D the dQ kernel wrote).
template <int D, int LPR>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int N, float scale_log2, float tau,
    int causal, int window, int sinks, Dropout drop) {
    constexpr int RPW = 64 / LPR, DS = D / LPR;
    const int lane = threadIdx.x;
    const int bh = (int)(blockIdx.x % BH);
    const int kt = (int)(blockIdx.x / BH);
    const int key = kt * RPW + lane % RPW, c0 = (lane / RPW) * DS;
    const size_t base = (size_t)bh * N * D;
    const bool live = key < N;
    float k[DS], v[DS], dk[DS], dv[DS];
#pragma unroll
    for (int c = 0; c < DS; c += 4) {
        const size_t off = base + (size_t)key * D + c0 + c;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 tk = live ? *reinterpret_cast<const f32x4*>(K + off) : z;
        const f32x4 tv = live ? *reinterpret_cast<const f32x4*>(V + off) : z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            k[c + e] = tk[e];
            v[c + e] = tv[e];
            dk[c + e] = dv[c + e] = 0.f;
        }
    }
    const int k_lo = kt * RPW;   // the wave's first key: no query before it sees any of its keys
    const int i0 = causal ? k_lo : 0;
    for (int i = i0; i < N; ++i) {
        const float* qr = Q + base + (size_t)i * D + c0;
        const float* gr = dO + base + (size_t)i * D + c0;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < DS; c += 4) {
            const f32x4 tq = *reinterpret_cast<const f32x4*>(qr + c);
            const f32x4 tg = *reinterpret_cast<const f32x4*>(gr + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = __builtin_fmaf(tq[e], k[c + e], s);
                dp = __builtin_fmaf(tg[e], v[c + e], dp);
            }
        }
        s = row_sum<LPR>(s);
        dp = row_sum<LPR>(dp);
        const float lse2 = LSE[(size_t)bh * N + i] * kLog2e;
        const float Di = Dv[(size_t)bh * N + i];
        const float p = (live && visible(i, key, causal, window, sinks))
                            ? fast_exp2(__builtin_fmaf(s, scale_log2, -lse2)) : 0.f;
        float pz = p;
        if (drop.thr > 0) {
            const bool kp = kept(drop, i, key, bh);
            pz = kp ? p * drop.scale : 0.f;
            dp = kp ? dp * drop.scale : 0.f;
        }
        const float ds = p * (dp - Di);
#pragma unroll
        for (int c = 0; c < DS; c += 4) {
            const f32x4 tq = *reinterpret_cast<const f32x4*>(qr + c);
            const f32x4 tg = *reinterpret_cast<const f32x4*>(gr + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dv[c + e] = __builtin_fmaf(pz, tg[e], dv[c + e]);
                dk[c + e] = __builtin_fmaf(ds, tq[e], dk[c + e]);
            }
        }
    }
    if (live) {
#pragma unroll
        for (int c = 0; c < DS; c += 4) {
            const size_t off = base + (size_t)key * D + c0 + c;
            *reinterpret_cast<f32x4*>(dK + off) =
                f32x4{dk[c] * tau, dk[c + 1] * tau, dk[c + 2] * tau, dk[c + 3] * tau};
            *reinterpret_cast<f32x4*>(dV + off) = f32x4{dv[c], dv[c + 1], dv[c + 2], dv[c + 3]};
        }
    }
}

Dropout make_drop(int thr, unsigned long long seed, unsigned int offset) {
    Dropout d;
    d.seed_lo = (uint32_t)seed;
    d.seed_hi = (uint32_t)(seed >> 32);
    d.offset = offset;
    d.thr = thr;
    d.scale = thr > 0 ? 256.f / (256.f - (float)thr) : 1.f;
    return d;
}

// Lanes per row: 8 in all three kernels, so a wave holds 8 rows and each lane
// 8 (d = 64) or 16 (d = 128) entries of a row.  Measured against 2 lanes per
// row (forward, dQ) and 4 (dK/dV): the 1x1x256x64 forward 136 -> 115 us, the
// causal 1x4x1024x128 forward 0.65 -> 0.46 ms and backward 1.76 -> 0.82 ms;
// 16 lanes per row was slower at 2x8x2048x64.
constexpr int kFwdLPR = 8, kDqLPR = 8, kDkvLPR = 8;
// Waves per forward workgroup, each taking a slice of the key range: 8
// measured fastest (1x1x256x64 forward 77 -> 23 us with 4, 15 us with 8;
// causal 1x4x1024x128 0.33 -> 0.10 ms).
constexpr int kFwdSplit = 8;

template <int D>
void fwd_d(const FwdArgs& a, hipStream_t st) {
    constexpr int RPW = 64 / kFwdLPR;
    const int bh = a.B * a.H;
    const int nt = (a.N + RPW - 1) / RPW;
    hipLaunchKernelGGL((fwd_f32_kernel<D, kFwdLPR, kFwdSplit>), dim3(nt * bh), dim3(64 * kFwdSplit), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       bh, a.N, a.tau * kLog2e, a.tau, a.causal, a.window, a.sinks,
                       make_drop(a.drop_thr, a.seed, a.offset));
}

template <int D>
void bwd_d(const BwdArgs& a, int stages, hipStream_t st) {
    const int bh = a.B * a.H;
    const Dropout drop = make_drop(a.drop_thr, a.seed, a.offset);
    if (stages & 1) {
        constexpr int RPW = 64 / kDqLPR;
        const int nt = (a.N + RPW - 1) / RPW;
        hipLaunchKernelGGL((bwd_dq_f32_kernel<D, kDqLPR>), dim3(nt * bh), dim3(64), 0, st,
                           (const float*)a.q, (const float*)a.k, (const float*)a.v,
                           (const float*)a.o, (const float*)a.dout, a.lse, a.D, (float*)a.dq, bh,
                           a.N, a.tau * kLog2e, a.tau, a.causal, a.window, a.sinks, drop);
    }
    if (stages & 2) {
        constexpr int RPW = 64 / kDkvLPR;
        const int nt = (a.N + RPW - 1) / RPW;
        hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, kDkvLPR>), dim3(nt * bh), dim3(64), 0, st,
                           (const float*)a.q, (const float*)a.k, (const float*)a.v,
                           (const float*)a.dout, a.lse, a.D, (float*)a.dk, (float*)a.dv, bh, a.N,
                           a.tau * kLog2e, a.tau, a.causal, a.window, a.sinks, drop);
    }
}

}  // namespace

void launch_fwd_f32(const FwdArgs& a, hipStream_t st) {
    a.d == 64 ? fwd_d<64>(a, st) : fwd_d<128>(a, st);
}

void launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t st) {
    a.d == 64 ? bwd_d<64>(a, stages, st) : bwd_d<128>(a, stages, st);
}

}  // namespace fa
