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
//   page, "como funciona").  The waves (4, or 16 in a grid smaller than
//   the part's CU count) are merged through LDS and the split writes
//   o_s = o/l and lse_s = tau*m + ln(l) (or -inf when empty).
// decode_merge_kernel: one wave per (b, h) combines the splits with the same
//   merge rule: LSE = ln sum_s exp(lse_s), O = sum_s exp(lse_s - LSE) o_s.
// Key rows at or beyond L_b are never read: padding may hold anything.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

template <int N_> using ic = std::integral_constant<int, N_>;

// One output element in the output dtype (bf16: round to nearest even).
__device__ __forceinline__ void store_out(uint16_t* p, float v) {
    *reinterpret_cast<__bf16*>(p) = (__bf16)v;
}
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }

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
// Keys [kb, ke) of split s of S for a sequence of L keys (L <= S * chunk),
// as the paged decode assigns them.  Splits below L / chunk take whole chunks
// in order; the last split takes the remainder (L mod chunk keys after the
// whole chunks, possibly none); the splits in between are empty.  The grid
// runs split-major, so the short remainders are dispatched after every whole
// chunk and the grid drains on short work instead of on whole chunks of the
// longest sequences (measured on 64 sequences of 1024-8192 keys with 1024-key
// chunks: 208.7 -> 203.8 us).  The dense decode keeps chunk s = keys
// [s * chunk, (s + 1) * chunk): its grid runs many more rounds of workgroups,
// and the same order measured no faster there.
__device__ __forceinline__ void split_range(int s, int S, int chunk, int L, int& kb, int& ke) {
    const int nfull = L / chunk;
    if (s < nfull) {
        kb = s * chunk;
        ke = kb + chunk;
    } else if (s == S - 1) {
        kb = nfull * chunk;
        ke = L;
    } else {
        kb = ke = 0;
    }
}

// Streaming 16-byte load of the KV cache (read once: non-temporal, so it does
// not displace reused lines in the caches).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int* __restrict__ seqlens, int B, int H, int N_max, int chunk, float scale_log2,
    float tau, float* __restrict__ ws_o, float* __restrict__ ws_lse, T* __restrict__ O,
    float* __restrict__ LSE) {
    // O and LSE non-null: there is a single split, whose normalised partial
    // is already the result, so it is stored as the merge would store it
    // (the merge of one split multiplies by exp(0) = 1 and adds ln 1 = 0) and
    // the merge is not launched.
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
        if (O) {          // an empty sequence: O = 0, LSE = -inf (the empty sum)
            if (tid < D) store_out(O + bh * D + tid, 0.f);
            if (tid == 0) LSE[bh] = neg_inf();
            return;
        }
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

    // The chunk is walked in stages of KPI keys; wave w takes stages w, w+NW, ...
    // Two register stages: the loads of the next keys are in flight while the
    // current ones are consumed.
    const int nst = (ke - kb + KPI - 1) / KPI;
    auto stage_key = [&](int t) { return kb + t * KPI; };
    int t = wave;
    if (t < nst) {
        u32x4 ka[U], va[U], kn[U], vn[U];
        load(ka, va, stage_key(t));
        while (true) {
            const int t1 = t + NW;
            if (t1 < nst) load(kn, vn, stage_key(t1));
            consume(ka, va, stage_key(t));
            if (t1 >= nst) break;
            const int t2 = t1 + NW;
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
    // combine the NW waves
    __shared__ float sm[NW], sl[NW], so[NW][D];
    if (g == 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) so[wave][c * PER + i] = o[i];
        if (c == 0) { sm[wave] = m; sl[wave] = l; }
    }
    __syncthreads();
    if (tid < D) {
        float M = sm[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w]);
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float a = (sm[w] == neg_inf()) ? 0.f : fast_exp2((sm[w] - M) * scale_log2);
            lt += sl[w] * a;
            ot += so[w][tid] * a;
        }
        if (O) {
            store_out(O + bh * D + tid, ot / lt);
            if (tid == 0) LSE[bh] = M * tau + __logf(lt);
        } else {
            ws_o[wsi * D + tid] = ot / lt;
            if (tid == 0) ws_lse[wsi] = M * tau + __logf(lt);
        }
    }
}

// One wave per (b, h): lane t owns head-dim entries t and t + 64 (d = 128) or
// t (d = 64).  The split LSEs are read by the lanes in parallel (64 at a
// time) and reduced across the wave; the partial outputs are loaded
// independently of them (the first 16 splits' before the reduction).
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int S, int BH,
    T* __restrict__ O, float* __restrict__ LSE) {
    const int bh = blockIdx.x, t = threadIdx.x;
    constexpr int PL = D / 64;
    // The partial outputs of the first PRE splits are loaded before the LSEs
    // are reduced (their addresses do not depend on the weights), so that a
    // call with at most PRE splits waits for memory once.
    constexpr int PRE = 16;
    float po[PRE][PL];
#pragma unroll
    for (int j = 0; j < PRE; ++j)
#pragma unroll
        for (int i = 0; i < PL; ++i)
            po[j][i] = j < S ? ws_o[((size_t)j * BH + bh) * D + t + 64 * i] : 0.f;
    float M = neg_inf();
    for (int s0 = 0; s0 < S; s0 += 64)
        if (s0 + t < S) M = fmaxf(M, ws_lse[(size_t)(s0 + t) * BH + bh]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float acc[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) acc[i] = 0.f;
    float sum = 0.f;
    // (with every split empty, M = -inf and every weight is 0: O = 0, LSE = -inf)
    for (int s0 = 0; s0 < S; s0 += 64) {
        // lane t holds the weight of split s0 + t
        const float ls = s0 + t < S ? ws_lse[(size_t)(s0 + t) * BH + bh] : neg_inf();
        const float wt = ls == neg_inf() ? 0.f : __expf(ls - M);
        const int n = min(64, S - s0);
        if (s0 == 0) {
#pragma unroll
            for (int j = 0; j < PRE; ++j) {
                const float w = __shfl(wt, j, 64);   // 0 for j >= S
                sum += w;
#pragma unroll
                for (int i = 0; i < PL; ++i) acc[i] += w * po[j][i];
            }
        }
        for (int j = s0 == 0 ? PRE : 0; j < n; ++j) {
            const float w = __shfl(wt, j, 64);
            sum += w;
            const float* src = ws_o + ((size_t)(s0 + j) * BH + bh) * D + t;
#pragma unroll
            for (int i = 0; i < PL; ++i) acc[i] += w * src[64 * i];
        }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        store_out(O + (size_t)bh * D + t + 64 * i, acc[i] * inv);
    }
    if (t == 0) LSE[bh] = (M == neg_inf()) ? neg_inf() : M + __logf(sum);
}

// ---------------------------------------------------------------------------
// Paged cache, grouped KV heads.  One workgroup serves up to 16 query heads
// that share one KV head (h0 .. h0+15 of the group), for one sequence and one
// split, so each KV byte is read from HBM once per group.  Each wave streams
// its own 16-key blocks (blocks w, w+4, ... of the split) into registers,
// two blocks in flight (the next block's loads are issued before the current
// one is consumed), and computes
//   S^T [16 keys x 16 heads] = K Q^T     (16x16x32 MFMA; the K registers are
//                                         loaded directly in A-operand layout)
//   O^T [d x 16 heads]      += V^T P^T   (16x16x16 MFMA; V goes through a
//                                         per-wave LDS tile for the transposing
//                                         read, P^T comes straight from S^T's
//                                         accumulator registers)
// with the running max / sum per head kept in the lanes of that head.  The
// four waves are merged through LDS at the end as in decode_split_kernel.
// With G query heads per KV head these are G-row contractions; heads beyond
// G in the last group of 16 carry Q = 0 and are never stored.  A 16-key block
// starting at a multiple of 16 lies in one page (page_size >= 16), so its
// page base is wave-uniform.
constexpr int kPagedBK = 16;   // keys per wave block
#ifndef FA_PAGED_MINB
#define FA_PAGED_MINB 2        // workgroups per CU the register budget is sized for
#endif

template <int D>
struct PagedShape {
    static constexpr int LGD = D == 64 ? 6 : 7;
    static constexpr int VSTR = D + 16;          // padded LDS row of the V tile (elements)
    static constexpr int CPR = D / 8;            // 16-byte pieces per row
    static constexpr int VRPI = 64 / CPR;        // V rows per wave load instruction
    static constexpr int NVL = kPagedBK / VRPI;  // V load instructions per block
    static constexpr int TILE = kPagedBK * VSTR; // V tile elements per wave
};

template <int D>
struct PagedRegs {
    u32x4 k[D / 32];                    // K rows, A-operand layout (d slice kk)
    u32x4 v[PagedShape<D>::NVL];        // V rows, 16 bytes per lane per instruction
};

template <int D>
__global__ __launch_bounds__(256, FA_PAGED_MINB) void decode_paged_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kp, const uint16_t* __restrict__ Vp,
    const int* __restrict__ table, const int* __restrict__ seqlens, int B, int Hq, int Hkv, int G,
    int NG, int num_pages, int lgP, int max_pages, int chunk, float scale_log2, float tau,
    float* __restrict__ ws_o, float* __restrict__ ws_lse) {
    using S = PagedShape<D>;
    // V tiles during the sweep; the cross-wave merge reuses the same bytes.
    constexpr int LDS_BYTES = 4 * S::TILE * 2 > (128 + 64 * D) * 4 ? 4 * S::TILE * 2 : (128 + 64 * D) * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

    // Grid: (b, kv head, head group) fastest, then the split, so consecutive
    // workgroups (dealt round-robin to the XCDs) belong to different sequences.
    const int per_s = B * Hkv * NG;
    const int s = (int)(blockIdx.x / (unsigned)per_s);
    int rem = (int)(blockIdx.x % (unsigned)per_s);
    const int hg = rem % NG;
    rem /= NG;
    const int hkv = rem % Hkv, b = rem / Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane & 15, gq = lane >> 4;
    const int pmask = (1 << lgP) - 1;
    const int L = min(max(seqlens[b], 0), max_pages << lgP);
    int kb, ke;
    split_range(s, (int)(gridDim.x / (unsigned)per_s), chunk, L, kb, ke);
    const int h0 = hkv * G + hg * 16;          // first query head served here
    const int nh = min(16, G - hg * 16);       // query heads served here
    const size_t ws_row0 = (size_t)s * B * Hq + (size_t)b * Hq + h0;

    if (kb >= ke) {   // empty split: contributes nothing to the merge
        for (int i = tid; i < nh * D; i += 256) ws_o[ws_row0 * D + i] = 0.f;
        if (tid < nh) ws_lse[ws_row0 + tid] = neg_inf();
        return;
    }

    // B operand of S^T = K Q^T: lane i holds head i%16, the same d slots as K.
    u32x4 qf[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        qf[kk] = hl < nh ? ld16(Q + ((size_t)b * Hq + h0 + hl) * D + 32 * kk + 8 * gq)
                         : u32x4{0, 0, 0, 0};

    const int* trow = table + (size_t)b * max_pages;
    const size_t page_stride = (size_t)Hkv << (lgP + S::LGD);   // elements per page
    const size_t head_off = (size_t)hkv << (lgP + S::LGD);
    // Per-lane byte offsets inside a block, loop-invariant: K row hl, d slice
    // 8 gq (+32 kk); V row t * VRPI + lane / CPR, column 8 (lane % CPR).
    const int vr = lane / S::CPR, vc = (lane % S::CPR) * 8;
    const uint32_t koff = (uint32_t)(hl * D + 8 * gq) * 2;
    const uint32_t voff_g = (uint32_t)(vr * D + vc) * 2;

    // Buffer descriptors of the block at key k0: base = the block's first
    // row in its page (a 16-key block starting at a multiple of 16 lies in
    // one page), size = its rows before ke, so rows past ke read as zero (their
    // scores are masked; their V rows meet p = 0).  Page ids are clamped into
    // [0, num_pages) so that any table content keeps the reads in the cache.
    // (The block's element offset and size pass through readfirstlane so that
    // the compiler treats the descriptors as wave-uniform scalars.)
    struct BlockRsrc { size_t base; uint32_t bytes; };
    auto block_rsrc = [&](int k0) __attribute__((always_inline)) {
        const int kc = min(k0, ke - 1);
        const int pg = min(max(trow[kc >> lgP], 0), num_pages - 1);
        const size_t base = (size_t)pg * page_stride + head_off + ((size_t)(kc & pmask) << S::LGD);
        const uint32_t bytes = (uint32_t)max(min(ke - k0, kPagedBK), 0) * (D * 2);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
        return BlockRsrc{((size_t)hi << 32) | lo, (uint32_t)__builtin_amdgcn_readfirstlane(bytes)};
    };
    auto load = [&](PagedRegs<D>& R, const BlockRsrc& br) __attribute__((always_inline)) {
        const rsrc_t kr = make_rsrc(Kp + br.base, br.bytes);
        const rsrc_t vr_ = make_rsrc(Vp + br.base, br.bytes);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) R.k[kk] = buf_ld16_nt(kr, koff + 64 * kk);
#pragma unroll
        for (int t = 0; t < S::NVL; ++t) R.v[t] = buf_ld16_nt(vr_, voff_g + t * S::VRPI * D * 2);
    };

    // V^T operand: lane s of 16-lane group gq addresses key 4 gq + s/4,
    // columns 16 db + 4 (s%4); the transposing read hands lane i keys
    // 4 gq .. 4 gq + 3 of column 16 db + i%16, the keys whose probabilities
    // S^T's accumulator registers leave in lane i.
    uint16_t* const tile = reinterpret_cast<uint16_t*>(smem) + wave * S::TILE;
    const int voff = (4 * gq + (hl >> 2)) * S::VSTR + 4 * (hl & 3);
    f32x4 oacc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = neg_inf(), l = 0.f;   // running max (raw score units), lane-partial sum

    auto consume = [&](const PagedRegs<D>& R, int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < S::NVL; ++t) st16(tile + (t * S::VRPI + vr) * S::VSTR + vc, R.v[t]);
        f32x4 sc = mfma16x16x32_zero(R.k[0], qf[0]);   // register r: key 4 gq + r, head hl
#pragma unroll
        for (int kk = 1; kk < D / 32; ++kk) sc = mfma16x16x32(R.k[kk], qf[kk], sc);
        if (k0 + kPagedBK > ke) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (k0 + 4 * gq + r >= ke) sc[r] = neg_inf();
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2((m - mnew) * scale_log2);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
        const float mc = mnew * scale_log2;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = fast_exp2(__builtin_fmaf(sc[r], scale_log2, -mc));
            l += p[r];
        }
        const u32x2 pf = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
            oacc[db] = mfma16x16x16(lds_read_tr16(tile + voff + 16 * db), pf, oacc[db]);
    };

    // Blocks of this wave: keys kb + 16 (wave + 4 i), i < nbw.  Two register
    // sets; the loads of block i + 1 are issued before block i is consumed,
    // and block i + 2's descriptor (page id) is fetched meanwhile.  The
    // loads are unconditional so that every wait the compiler places is
    // exact: past the last block they go through a descriptor of zero bytes
    // (key ke), which returns zeros without touching memory.  (Repeating the
    // last block instead re-fetched part of it from HBM: the streaming loads
    // do not keep it in the caches.)  A scheduling barrier after each batch
    // keeps the loads ahead of the MFMAs.  (A third register set, two blocks
    // in flight, measured no faster.)
    const int nblk = (ke - kb + kPagedBK - 1) / kPagedBK;
    const int nbw = nblk > wave ? (nblk - wave + 3) / 4 : 0;
    if (nbw > 0) {
        auto key0 = [&](int i) { return i < nbw ? kb + kPagedBK * (wave + 4 * i) : ke; };
        PagedRegs<D> ra, rb;
        load(ra, block_rsrc(key0(0)));
        BlockRsrc rn = block_rsrc(key0(1));
        for (int i = 0; i < nbw; i += 2) {
            load(rb, rn);
            rn = block_rsrc(key0(i + 2));
            __builtin_amdgcn_sched_barrier(0);
            consume(ra, key0(i));
            if (i + 1 >= nbw) break;
            load(ra, rn);
            rn = block_rsrc(key0(i + 3));
            __builtin_amdgcn_sched_barrier(0);
            consume(rb, key0(i + 1));
        }
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);

    // Merge the four waves through LDS.
    __syncthreads();
    float* sm = reinterpret_cast<float*>(smem);   // [4][16] maxima
    float* sl = sm + 64;                          // [4][16] sums
    float* so = sl + 64;                          // [4][16][D] outputs
    if (gq == 0) {
        sm[wave * 16 + hl] = m;
        sl[wave * 16 + hl] = l;
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4*>(&so[(wave * 16 + hl) * D + 16 * db + 4 * gq]) = oacc[db];
    __syncthreads();
    for (int i = tid; i < nh * D; i += 256) {
        const int h = i / D, dd = i % D;
        const float M = fmaxf(fmaxf(sm[h], sm[16 + h]), fmaxf(sm[32 + h], sm[48 + h]));
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = sm[w * 16 + h];
            const float a = mw == neg_inf() ? 0.f : fast_exp2((mw - M) * scale_log2);
            lt += sl[w * 16 + h] * a;
            ot += so[(w * 16 + h) * D + dd] * a;
        }
        ws_o[ws_row0 * D + i] = ot / lt;
        if (dd == 0) ws_lse[ws_row0 + h] = M * tau + __logf(lt);
    }
}

template <int D>
void launch_paged(const PagedDecodeArgs& a, hipStream_t st) {
    const int G = a.Hq / a.Hkv, NG = (G + 15) / 16;
    const int lgP = __builtin_ctz((unsigned)a.page_size);
    const unsigned grid = (unsigned)a.num_splits * a.B * a.Hkv * NG;
    hipLaunchKernelGGL((decode_paged_kernel<D>), dim3(grid), dim3(256), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_pages, (const uint16_t*)a.v_pages,
                       a.block_table, a.seqlens, a.B, a.Hq, a.Hkv, G, NG, a.num_pages, lgP,
                       a.max_pages, a.chunk, a.tau * kLog2e, a.tau, a.ws_o, a.ws_lse);
    hipLaunchKernelGGL((decode_merge_kernel<uint16_t, D>), dim3(a.B * a.Hq), dim3(64), 0, st,
                       a.ws_o, a.ws_lse, a.num_splits, a.B * a.Hq, (uint16_t*)a.o, a.lse);
}

template <typename T, int D>
void launch(const DecodeArgs& a, hipStream_t st) {
    // A grid with fewer workgroups than the part has CUs (a small decode in
    // one split) takes 16 waves per workgroup, so that enough rows are in
    // flight per sequence; larger grids take 4.
    const unsigned grid = (unsigned)a.num_splits * a.B * a.H;
    T* const o1 = a.num_splits == 1 ? (T*)a.o : nullptr;
    float* const lse1 = a.num_splits == 1 ? a.lse : nullptr;
    if (grid < 256)
        hipLaunchKernelGGL((decode_split_kernel<T, D, 16>), dim3(grid), dim3(1024), 0, st,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, a.seqlens, a.B, a.H,
                           a.N_max, a.chunk, a.tau * kLog2e, a.tau, a.ws_o, a.ws_lse, o1, lse1);
    else
        hipLaunchKernelGGL((decode_split_kernel<T, D, 4>), dim3(grid), dim3(256), 0, st,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, a.seqlens, a.B, a.H,
                           a.N_max, a.chunk, a.tau * kLog2e, a.tau, a.ws_o, a.ws_lse, o1, lse1);
    if (a.num_splits > 1)
        hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.B * a.H), dim3(64), 0, st, a.ws_o,
                           a.ws_lse, a.num_splits, a.B * a.H, (T*)a.o, a.lse);
}

}  // namespace

void launch_decode_paged(const PagedDecodeArgs& a, hipStream_t st) {
    a.d == 64 ? launch_paged<64>(a, st) : launch_paged<128>(a, st);
}

void launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.dtype == kBF16) {
        a.d == 64 ? launch<uint16_t, 64>(a, st) : launch<uint16_t, 128>(a, st);
    } else {
        a.d == 64 ? launch<float, 64>(a, st) : launch<float, 128>(a, st);
    }
}

}  // namespace fa
