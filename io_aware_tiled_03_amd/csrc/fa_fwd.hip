// fa_fwd.hip - fused exact-attention forward for gfx950.
//
// What is computed ("flash-attention" encyclopedia page, "como funciona"):
// for every query row, O = softmax(tau * q K^T [+ causal mask]) V and
// LSE = m + ln(l), walking the keys block by block with a running maximum m
// and running sum l that rescale the partial output when a block is merged.
// Scores and probabilities exist only in registers; HBM sees Q, K, V once per
// tile and O, LSE once ("FlashAttention e o gargalo real de inferência",
// "FlashAttention: eliminar a viagem").
//
// bf16 kernel layout (one workgroup = 4 waves = 128 query rows, key tile 64):
//  * each wave owns 32 query rows; its Q rows sit in registers as the B
//    operand of S^T = K Q^T, so in the result every lane holds one query
//    (column) and 16 keys per 32-key block (rows): the row max/sum of the
//    softmax is a register loop plus one exchange between wave halves;
//  * K rows are read from LDS in the order pi(m) (see kperm) chosen so that
//    the registers of S^T already hold, per lane half, 8 consecutive keys:
//    the bf16-rounded P^T feeds the P V product as the B operand directly;
//  * V is staged transposed in LDS (V^T rows = head-dim index) so the A
//    operand of O^T = V^T P^T is one 16-byte read per lane;
//  * the loop runs over key tiles in order and, under the causal mask, stops
//    at the diagonal tile; waves whose rows precede the whole tile skip it;
//  * exp2 with tau*log2(e) folded into one FMA; O is normalised once at the end.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

// Row of the K tile that lane-row m reads so that C-register r of lane half h
// holds key 16*(r/8) + 8*h + r%8 of the 32-key block (see header comment).
__device__ __forceinline__ int kperm(int m) {
    const int j = 4 * (m >> 3) + (m & 3);
    return 16 * (j >> 3) + 8 * ((m >> 2) & 1) + (j & 7);
}

// XOR swizzles of the 16-byte chunk index inside an LDS row.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row & 8) >> 1); }
__device__ __forceinline__ int swz_vt(int row) { return row & 7; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int N, float scale_log2, float tau,
    int n_qtiles) {
    constexpr int BR = 128, BC = 64;
    constexpr int KCH = D / 8;             // 16-byte chunks per K row
    constexpr int KPT = BC * KCH / 256;    // K chunks staged per thread
    constexpr int VPT = KCH / 4;           // V chunks staged per thread
    constexpr int VTCH = BC / 8;           // 16-byte chunks per V^T row
    __shared__ u32x4 sK[BC * KCH];
    __shared__ u32x4 sVt[D * VTCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, hf = lane >> 5;
    const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);   // heaviest tiles first
    const int bh = (int)(blockIdx.x % BH);
    const size_t base = (size_t)bh * N * D;
    const int q0 = qt * BR;
    const int qw = q0 + wave * 32;
    const int qrow = qw + ln;

    u32x4 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = qrow < N ? ld16(Q + base + (size_t)qrow * D + ks * 16 + hf * 8) : u32x4{0, 0, 0, 0};

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m = neg_inf(), l = 0.f;

    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kend + BC - 1) / BC;
    const int prow = kperm(ln);

    u32x4 kreg[KPT], vreg[VPT];
    auto gload = [&](int j) {
        const int k0 = j * BC;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int idx = tid + 256 * u, row = idx / KCH, ch = idx % KCH, key = k0 + row;
            kreg[u] = key < N ? ld16(K + base + (size_t)key * D + ch * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int ch = wave + 4 * u, key = k0 + lane;
            vreg[u] = key < N ? ld16(V + base + (size_t)key * D + ch * 8) : u32x4{0, 0, 0, 0};
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int idx = tid + 256 * u, row = idx / KCH, ch = idx % KCH;
            sK[row * KCH + (ch ^ swz_k(row))] = kreg[u];
        }
        uint16_t* vt = reinterpret_cast<uint16_t*>(sVt);
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int ch = wave + 4 * u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = ch * 8 + e;
                const uint32_t w = vreg[u][e >> 1];
                vt[d * BC + (((lane >> 3) ^ swz_vt(d)) << 3) + (lane & 7)] =
                    (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffff));
            }
        }
    };

    gload(0);
    for (int j = 0; j < ntiles; ++j) {
        lstore();
        __syncthreads();
        if (j + 1 < ntiles) gload(j + 1);
        const int k0 = j * BC;
        const bool active = !CAUSAL || k0 <= qw + 31;
        if (active) {
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
                const int row = kb * 32 + prow;
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const u32x4 a = sK[row * KCH + ((ks * 2 + hf) ^ swz_k(row))];
                    s[kb] = mfma32x32x16(a, qf[ks], s[kb]);
                }
            }
            const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7);
                        if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = neg_inf();
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, xor32(mx));
            const float mnew = fmaxf(m, mx);
            const float alpha = fast_exp2((m - mnew) * scale_log2);
            const float mc = mnew * scale_log2;
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -mc));
                    s[kb][r] = p;
                    rs += p;
                }
            l = l * alpha + rs;
            m = mnew;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    u32x4 pf;
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        pf[w] = pack_bf16x2(s[kb][8 * t + 2 * w], s[kb][8 * t + 2 * w + 1]);
                    const int vch = kb * 4 + 2 * t + hf;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const int d = db * 32 + ln;
                        const u32x4 a = sVt[d * VTCH + (vch ^ swz_vt(d))];
                        oacc[db] = mfma32x32x16(a, pf, oacc[db]);
                    }
                }
        }
        __syncthreads();
    }

    l += xor32(l);
    const float inv = 1.f / l;
    if (qrow < N) {
        uint16_t* orow = O + base + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hf;
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + d) = w;
            }
        if (hf == 0) LSE[(size_t)bh * N + qrow] = m * tau + __logf(l);
    }
}

// fp32 path: one wave per 64 query rows, one row per lane, VALU arithmetic in
// fp32, K/V tiles of 32 rows in LDS (read as broadcasts).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int N, float scale_log2, float tau,
    int n_qtiles) {
    constexpr int BR = 64, BC = 32;
    __shared__ float sK[BC][D];
    __shared__ float sV[BC][D];
    const int lane = threadIdx.x;
    const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
    const int bh = (int)(blockIdx.x % BH);
    const size_t base = (size_t)bh * N * D;
    const int q0 = qt * BR, row = q0 + lane;

    float q[D], o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = row < N ? Q[base + (size_t)row * D + d] : 0.f;
        o[d] = 0.f;
    }
    float m = neg_inf(), l = 0.f;
    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    for (int k0 = 0; k0 < kend; k0 += BC) {
        __syncthreads();
        for (int idx = lane; idx < BC * D; idx += 64) {
            const int r = idx / D, d = idx % D, key = k0 + r;
            sK[r][d] = key < N ? K[base + (size_t)key * D + d] : 0.f;
            sV[r][d] = key < N ? V[base + (size_t)key * D + d] : 0.f;
        }
        __syncthreads();
        float s[BC];
        float mx = neg_inf();
        for (int c = 0; c < BC; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], sK[c][d], acc);
            const int key = k0 + c;
            s[c] = (key < N && (!CAUSAL || key <= row)) ? acc : neg_inf();
            mx = fmaxf(mx, s[c]);
        }
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2((m - mnew) * scale_log2);
        const float mc = mnew * scale_log2;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
        for (int c = 0; c < BC; ++c) {
            const float p = fast_exp2(__builtin_fmaf(s[c], scale_log2, -mc));
            l += p;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, sV[c][d], o[d]);
        }
        m = mnew;
    }
    if (row < N) {
        const float inv = 1.f / l;
#pragma unroll
        for (int d = 0; d < D; ++d) O[base + (size_t)row * D + d] = o[d] * inv;
        LSE[(size_t)bh * N + row] = m * tau + logf(l);
    }
}

template <int D, bool C>
void launch_bf16(const FwdArgs& a, hipStream_t st) {
    const int nq = (a.N + 127) / 128;
    const int bh = a.B * a.H;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, C>), dim3(nq * bh), dim3(256), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, bh, a.N, a.tau * kLog2e, a.tau, nq);
}

template <int D, bool C>
void launch_f32(const FwdArgs& a, hipStream_t st) {
    const int nq = (a.N + 63) / 64;
    const int bh = a.B * a.H;
    hipLaunchKernelGGL((fwd_f32_kernel<D, C>), dim3(nq * bh), dim3(64), 0, st, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, bh, a.N,
                       a.tau * kLog2e, a.tau, nq);
}

}  // namespace

void launch_fwd(const FwdArgs& a, hipStream_t st) {
    if (a.dtype == kBF16) {
        if (a.d == 64) a.causal ? launch_bf16<64, true>(a, st) : launch_bf16<64, false>(a, st);
        else a.causal ? launch_bf16<128, true>(a, st) : launch_bf16<128, false>(a, st);
    } else {
        if (a.d == 64) a.causal ? launch_f32<64, true>(a, st) : launch_f32<64, false>(a, st);
        else a.causal ? launch_f32<128, true>(a, st) : launch_f32<128, false>(a, st);
    }
}

}  // namespace fa
