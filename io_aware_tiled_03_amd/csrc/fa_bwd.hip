// fa_bwd.hip - recomputing backward of exact attention for gfx950.
//
// The backward keeps only O and the per-row statistic (here LSE = m + ln l)
// and rebuilds S and P on chip ("flash-attention" encyclopedia page, "como
// funciona", backward paragraph).  With P = exp(tau S - LSE):
//   D_i  = dO_i . O_i                       (the page's D_i = P_i . dP_i identity)
//   dV   = P^T dO,   dP = dO V^T,   dS = P o (dP - D),
//   dK   = tau dS^T Q,               dQ = tau dS K.
//
// Kernels (bf16 in, fp32 accumulation on MFMA, bf16 out; no atomics):
//  bwd_pre_kernel  : D for every row, an inner product of length d.
//  bwd_dkdv_kernel : one workgroup per 128-key tile (32 keys per wave, K and V
//                    of those keys held in registers); loops over 64-query
//                    tiles staged in LDS both row-major (for S = Q K^T and
//                    dP = dO V^T, whose results put one key per lane) and
//                    transposed (for dV^T += dO^T P and dK^T += Q^T dS, whose B
//                    operands are P and dS straight from registers).
//  bwd_dq_kernel   : one workgroup per 128-query tile (32 queries per wave, Q
//                    and dO rows in registers); loops over 64-key tiles up to
//                    the diagonal, recomputing S^T = K Q^T and dP^T = V dO^T
//                    (one query per lane) and accumulating dQ^T += K^T dS^T.
// Query rows are read from LDS in the kperm order so that the C registers of
// each lane half hold 8 consecutive rows, ready to be packed as a B operand.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

__device__ __forceinline__ int kperm(int m) {
    const int j = 4 * (m >> 3) + (m & 3);
    return 16 * (j >> 3) + 8 * ((m >> 2) & 1) + (j & 7);
}
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row & 8) >> 1); }
__device__ __forceinline__ int swz_t(int row) { return row & 7; }

__device__ __forceinline__ uint16_t half_of(const u32x4& w, int e) {
    const uint32_t x = w[e >> 1];
    return (uint16_t)((e & 1) ? (x >> 16) : (x & 0xffff));
}

// D_i = sum_d dO_id O_id in fp32; D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ Dv, size_t rows) {
    constexpr int LPR = D / 8;
    const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t row = gid / LPR;
    const int c = (int)(gid % LPR);
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = ld16(O + row * D + c * 8), b = ld16(dO + row * D + c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc += bf16lo(a[i]) * bf16lo(b[i]) + bf16hi(a[i]) * bf16hi(b[i]);
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && c == 0) Dv[row] = acc;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int N, float scale_log2,
    float tau) {
    constexpr int BC = 128, BR = 64;
    constexpr int KCH = D / 8, TCH = BR / 8, SPT = KCH / 4;
    __shared__ u32x4 sQ[BR * KCH], sdO[BR * KCH], sQt[D * TCH], sdOt[D * TCH];
    __shared__ float sL[BR], sD[BR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, hf = lane >> 5;
    const int kt = (int)(blockIdx.x / BH);      // causal: low key tiles carry the most work
    const int bh = (int)(blockIdx.x % BH);
    const size_t base = (size_t)bh * N * D;
    const int k0 = kt * BC, kw = k0 + 32 * wave, key = kw + ln;

    u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const size_t off = base + (size_t)key * D + ks * 16 + hf * 8;
        kf[ks] = key < N ? ld16(K + off) : u32x4{0, 0, 0, 0};
        vf[ks] = key < N ? ld16(V + off) : u32x4{0, 0, 0, 0};
    }
    f32x16 dvacc[D / 32], dkacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvacc[db][r] = 0.f; dkacc[db][r] = 0.f; }

    const int prow = kperm(ln);
    const int n_qt = (N + BR - 1) / BR;
    const int qt0 = CAUSAL ? k0 / BR : 0;
    uint16_t* sQt16 = reinterpret_cast<uint16_t*>(sQt);
    uint16_t* sdOt16 = reinterpret_cast<uint16_t*>(sdOt);

    for (int qt = qt0; qt < n_qt; ++qt) {
        const int q0 = qt * BR;
        __syncthreads();
        {
            const int q = q0 + lane;
#pragma unroll
            for (int u = 0; u < SPT; ++u) {
                const int c = wave + 4 * u;
                const size_t off = base + (size_t)q * D + c * 8;
                const u32x4 a = q < N ? ld16(Q + off) : u32x4{0, 0, 0, 0};
                const u32x4 b = q < N ? ld16(dO + off) : u32x4{0, 0, 0, 0};
                sQ[lane * KCH + (c ^ swz_k(lane))] = a;
                sdO[lane * KCH + (c ^ swz_k(lane))] = b;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = c * 8 + e;
                    const int pos = d * BR + (((lane >> 3) ^ swz_t(d)) << 3) + (lane & 7);
                    sQt16[pos] = half_of(a, e);
                    sdOt16[pos] = half_of(b, e);
                }
            }
            if (wave == 0) sL[lane] = q < N ? LSE[(size_t)bh * N + q] * kLog2e : __builtin_inff();
            if (wave == 1) sD[lane] = q < N ? Dv[(size_t)bh * N + q] : 0.f;
        }
        __syncthreads();
        if (CAUSAL && q0 + BR - 1 < kw) continue;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qs = q0 + qb * 32;
            if (CAUSAL && qs + 31 < kw) continue;
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
            const int row = qb * 32 + prow;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const int ch = row * KCH + ((ks * 2 + hf) ^ swz_k(row));
                s = mfma32x32x16(sQ[ch], kf[ks], s);
                dp = mfma32x32x16(sdO[ch], vf[ks], dp);
            }
            const bool mask = CAUSAL && (kw + 31 > qs);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = qb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7);
                float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -sL[ql]));
                if (mask && key > q0 + ql) p = 0.f;
                s[r] = p;
                dp[r] = p * (dp[r] - sD[ql]);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u32x4 pf, dsf;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pf[w] = pack_bf16x2(s[8 * t + 2 * w], s[8 * t + 2 * w + 1]);
                    dsf[w] = pack_bf16x2(dp[8 * t + 2 * w], dp[8 * t + 2 * w + 1]);
                }
                const int ch = qb * 4 + 2 * t + hf;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const int d = db * 32 + ln;
                    const int idx = d * TCH + (ch ^ swz_t(d));
                    dvacc[db] = mfma32x32x16(sdOt[idx], pf, dvacc[db]);
                    dkacc[db] = mfma32x32x16(sQt[idx], dsf, dkacc[db]);
                }
            }
        }
    }
    if (key < N) {
        uint16_t* dkr = dK + base + (size_t)key * D;
        uint16_t* dvr = dV + base + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hf;
                u32x2 wk, wv;
                wk[0] = pack_bf16x2(dkacc[db][4 * g] * tau, dkacc[db][4 * g + 1] * tau);
                wk[1] = pack_bf16x2(dkacc[db][4 * g + 2] * tau, dkacc[db][4 * g + 3] * tau);
                wv[0] = pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]);
                wv[1] = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                *reinterpret_cast<u32x2*>(dkr + d) = wk;
                *reinterpret_cast<u32x2*>(dvr + d) = wv;
            }
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dQ, int BH, int N, float scale_log2, float tau, int n_qtiles) {
    constexpr int BR = 128, BC = 64;
    constexpr int KCH = D / 8, TCH = BC / 8, SPT = KCH / 4;
    __shared__ u32x4 sK[BC * KCH], sV[BC * KCH], sKt[D * TCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, hf = lane >> 5;
    const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
    const int bh = (int)(blockIdx.x % BH);
    const size_t base = (size_t)bh * N * D;
    const int q0 = qt * BR, qw = q0 + 32 * wave, qrow = qw + ln;

    u32x4 qf[D / 16], df[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const size_t off = base + (size_t)qrow * D + ks * 16 + hf * 8;
        qf[ks] = qrow < N ? ld16(Q + off) : u32x4{0, 0, 0, 0};
        df[ks] = qrow < N ? ld16(dO + off) : u32x4{0, 0, 0, 0};
    }
    const float lse2 = qrow < N ? LSE[(size_t)bh * N + qrow] * kLog2e : __builtin_inff();
    const float Dq = qrow < N ? Dv[(size_t)bh * N + qrow] : 0.f;
    f32x16 dqacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

    const int prow = kperm(ln);
    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kend + BC - 1) / BC;
    uint16_t* sKt16 = reinterpret_cast<uint16_t*>(sKt);

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BC;
        __syncthreads();
        {
            const int kr = k0 + lane;
#pragma unroll
            for (int u = 0; u < SPT; ++u) {
                const int c = wave + 4 * u;
                const size_t off = base + (size_t)kr * D + c * 8;
                const u32x4 a = kr < N ? ld16(K + off) : u32x4{0, 0, 0, 0};
                const u32x4 b = kr < N ? ld16(V + off) : u32x4{0, 0, 0, 0};
                sK[lane * KCH + (c ^ swz_k(lane))] = a;
                sV[lane * KCH + (c ^ swz_k(lane))] = b;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = c * 8 + e;
                    sKt16[d * BC + (((lane >> 3) ^ swz_t(d)) << 3) + (lane & 7)] = half_of(a, e);
                }
            }
        }
        __syncthreads();
        if (CAUSAL && k0 > qw + 31) continue;
        const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
            const int row = kb * 32 + prow;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const int ch = row * KCH + ((ks * 2 + hf) ^ swz_k(row));
                s = mfma32x32x16(sK[ch], qf[ks], s);
                dp = mfma32x32x16(sV[ch], df[ks], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -lse2));
                if (need_mask) {
                    const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7);
                    if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
                }
                s[r] = p * (dp[r] - Dq);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u32x4 dsf;
#pragma unroll
                for (int w = 0; w < 4; ++w) dsf[w] = pack_bf16x2(s[8 * t + 2 * w], s[8 * t + 2 * w + 1]);
                const int ch = kb * 4 + 2 * t + hf;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const int d = db * 32 + ln;
                    dqacc[db] = mfma32x32x16(sKt[d * TCH + (ch ^ swz_t(d))], dsf, dqacc[db]);
                }
            }
        }
    }
    if (qrow < N) {
        uint16_t* dqr = dQ + base + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hf;
                u32x2 w;
                w[0] = pack_bf16x2(dqacc[db][4 * g] * tau, dqacc[db][4 * g + 1] * tau);
                w[1] = pack_bf16x2(dqacc[db][4 * g + 2] * tau, dqacc[db][4 * g + 3] * tau);
                *reinterpret_cast<u32x2*>(dqr + d) = w;
            }
    }
}

template <int D, bool C>
void launch(const BwdArgs& a, int stages, hipStream_t st) {
    const int bh = a.B * a.H;
    if (stages & 1) {
        const size_t rows = (size_t)bh * a.N;
        const size_t pre_blocks = (rows * (D / 8) + 255) / 256;
        hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)pre_blocks), dim3(256), 0, st,
                           (const uint16_t*)a.o, (const uint16_t*)a.dout, a.D, rows);
    }
    if (stages & 2) {
        const int nk = (a.N + 127) / 128;
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, C>), dim3(nk * bh), dim3(256), 0, st,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, a.lse, a.D, (uint16_t*)a.dk, (uint16_t*)a.dv,
                           bh, a.N, a.tau * kLog2e, a.tau);
    }
    if (stages & 4) {
        const int nq = (a.N + 127) / 128;
        hipLaunchKernelGGL((bwd_dq_kernel<D, C>), dim3(nq * bh), dim3(256), 0, st,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, a.lse, a.D, (uint16_t*)a.dq, bh, a.N,
                           a.tau * kLog2e, a.tau, nq);
    }
}

}  // namespace

void launch_bwd(const BwdArgs& a, int stages, hipStream_t st) {
    if (a.d == 64) a.causal ? launch<64, true>(a, stages, st) : launch<64, false>(a, stages, st);
    else a.causal ? launch<128, true>(a, stages, st) : launch<128, false>(a, stages, st);
}

}  // namespace fa
