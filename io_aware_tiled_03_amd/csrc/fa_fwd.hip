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
// bf16 kernel layout (one workgroup = NW waves of 32 query rows, key tile BC):
//  * each wave owns 32 query rows; its Q rows sit in registers as the B
//    operand of S^T = K Q^T, so in the result every lane holds one query
//    (column) and 16 keys per 32-key block (rows): the row max/sum of the
//    softmax is a register loop plus one exchange between wave halves;
//  * K rows are stored in LDS permuted (see kperm) so that lane m reading
//    physical row m gets key kperm(m), chosen such that the
//    registers of S^T already hold, per lane half, 8 consecutive keys: the
//    bf16-rounded P^T feeds the P V product as the B operand directly;
//  * V stays row-major in LDS; the A operand of O^T = V^T P^T comes from the
//    transposing LDS read, four keys of one head-dim column per 8-byte read;
//  * K and V tiles are double-buffered in LDS (one barrier per tile), the next
//    tile's global loads are in flight during the current tile's math;
//  * the loop runs over key tiles in order and, under the causal mask, stops
//    at the diagonal tile; waves whose rows precede the whole tile skip it;
//  * the causal mask may carry a sliding window with sink tokens ("Atenção
//    eficiente — FlashAttention, sparse e híbrida", sections "Atenção híbrida"
//    and "Attention sinks"): key j is visible to query i iff j <= i and
//    (i - j < window or j < sinks).  The workgroup then visits the tiles
//    holding sink keys below its window, then the tiles from its window's
//    lower edge to the diagonal; tiles that are entirely visible to every row
//    run the unmasked body, the window's lower edge and the diagonal the
//    masked one (plain causal attention is window >= N, no sinks);
//  * exp2 with tau*log2(e) folded into one FMA; the running reference max is
//    only moved (and O rescaled) when a score exceeds it by more than 2^8, so
//    most tiles skip the rescale; O is normalised once at the end.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

// Key (within a 32-key block) that lane-row m of the S^T MFMA must hold so
// that C-register r of lane half h holds key 16*(r/8) + 8*h + r%8.
__device__ __forceinline__ int kperm(int m) {
    const int j = 4 * (m >> 3) + (m & 3);
    return 16 * (j >> 3) + 8 * ((m >> 2) & 1) + (j & 7);
}

#ifndef FA_FWD_RESCALE_LOG2
#define FA_FWD_RESCALE_LOG2 8.0f
#endif
#ifndef FA_FWD_KPAD
#define FA_FWD_KPAD 8        // K row padding (bf16 elements)
#endif
#ifndef FA_FWD_VPAD
#define FA_FWD_VPAD 16       // V row padding (bf16 elements), natural row order
#endif

// V tiles are read only by the transposing read, each 16-lane group on 64 bytes
// of four consecutive keys, which share banks at rows of 16 x odd bytes and
// partly at the padded 288-byte rows.  The d = 128 causal kernel (the long
// prefill) instead stores key r of a tile at LDS row vrow(r) of 272-byte rows:
// vrow swaps the two 2-bit fields of r inside each 16-row block, so the four keys
// of a read sit four rows apart (4 x 16 x odd bytes = 64 mod 256: the pieces
// cover the banks once).  Long causal prefill 1.906 -> 1.892 ms, outputs
// identical.  The other kernels keep natural order: with the permutation the
// d = 128 non-causal kernel spilled 20 bytes and the d = 64 dropout kernels
// went over the registers of three waves per SIMD, for at most 1% elsewhere.
__device__ __forceinline__ int vrow(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }
// d=128: the score products' K operand reads are issued this many ahead of
// the products that use them (the compiler's own order kept two in flight,
// exposing the LDS latency before every other product; four measured 2%
// faster on the long causal prefill, more gave nothing further; at d=64,
// with more waves per SIMD to hide the latency, it gave nothing).  0 leaves
// the order to the compiler.
#ifndef FA_FWD_SCHED
#define FA_FWD_SCHED 4
#endif

template <int N_> using ic = std::integral_constant<int, N_>;

// Mask modes of the bf16 forward (kMaskBlock*: block-sparse, without or with
// the causal mask).
enum : int { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2, kMaskBlock = 3, kMaskBlockCausal = 4 };
// V rows through vrow (above) in the d = 128 causal kernel only
template <int D, int MODE, bool DROP>
constexpr bool fwd_vperm() { return D == 128 && MODE == kMaskCausal && !DROP; }

// BC keys per tile, NW waves per workgroup (32 query rows each); MODE is one
// of the mask modes (kMaskWindow: causal with a sliding window and sinks).
// DROP: dropout on P after the softmax (mask from Dropout::block); the row
// sum l and the LSE use the undropped P, O is scaled by 1/(1 - p) at the end.
template <int D, int MODE, int BC, int NW, bool DROP>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int N, float scale_log2, float tau,
    int n_qtiles, int window, int sinks, Dropout drop, BlockSparse bs) {
    constexpr bool CAUSAL = MODE == kMaskCausal || MODE == kMaskWindow || MODE == kMaskBlockCausal;
    constexpr bool WIN = MODE == kMaskWindow, BLK = MODE >= kMaskBlock;
    // rows that may meet tiles before their first visible key (-inf guards)
    constexpr bool SPARSE_ROWS = WIN || BLK;
    constexpr int BR = 32 * NW, NKB = BC / 32;
    constexpr int KCH = D / 8;             // 16-byte chunks per row
    constexpr int KSTR = D + FA_FWD_KPAD;  // K row stride (elements), padded against bank conflicts
    constexpr bool VPERM = fwd_vperm<D, MODE, DROP>();
    constexpr int VSTR = VPERM ? D + 8 : D + FA_FWD_VPAD;  // V row stride (elements)
    // Two staging buffers per operand, as distinct LDS variables chosen at
    // compile time: the compiler then knows a read of one buffer cannot alias
    // the direct-to-LDS copies still landing in the other, and does not wait
    // for those copies before the reads.  (With one array indexed by a run-time
    // buffer number it waits for every outstanding copy, serialising the next
    // tile's load with this tile's compute.)
    __shared__ __attribute__((aligned(16))) uint16_t sK0[BC * KSTR], sK1[BC * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[BC * VSTR], sV1[BC * VSTR];
    // block-sparse: the workgroup's active key tiles, in order
    __shared__ uint16_t s_list[BLK ? kMaxSparseTiles : 1];
    __shared__ uint64_t s_bal[BLK ? kMaxSparseTiles / 64 : 1];
    __shared__ int s_off[BLK ? kMaxSparseTiles / 64 + 1 : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
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
    float m = neg_inf(), l = 0.f;   // reference max (raw score units) and lane-partial sum

    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kend + BC - 1) / BC;
    const int nfull = N / BC;       // tiles with no key past N

    // Staging: direct global -> LDS copies.  A wave instruction fills 1 KB of
    // LDS (lane i -> 16 bytes at +16*i), so each lane loads whichever global
    // 16-byte chunk belongs at its LDS position: K rows are stored permuted
    // (physical row p holds key kperm(p)), rows are padded, and padding
    // positions load a duplicate chunk that is never read.  Rows past N read
    // as zeros through the buffer descriptor (their scores are masked to -inf
    // and their V rows meet p = 0).  Wave w issues instructions w, w+4, ...
    constexpr int KCPR = KSTR / 8, VCPR = VSTR / 8;      // 16-byte chunks per padded row
    constexpr int KNI = BC * KCPR / 64, VNI = BC * VCPR / 64;   // wave instructions per tile
    constexpr int KPW = (KNI + NW - 1) / NW, VPW = (VNI + NW - 1) / NW;   // per wave (upper bound)
    static_assert(BC * KCPR % 64 == 0 && BC * VCPR % 64 == 0, "whole wave instructions");
    const rsrc_t krs = make_rsrc(K + base, (uint32_t)N * D * 2);
    const rsrc_t vrs = make_rsrc(V + base, (uint32_t)N * D * 2);
    uint32_t kgo[KPW], vgo[VPW];   // byte offsets inside a tile (tile start added per tile)
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
        const int pos = (wave + NW * t) * 64 + lane, prow = pos / KCPR, c = pos % KCPR;
        const int key = (prow & ~31) + kperm(prow & 31);
        kgo[t] = (uint32_t)(key * D + (c < KCH ? c : 0) * 8) * 2;
    }
#pragma unroll
    for (int t = 0; t < VPW; ++t) {
        const int pos = (wave + NW * t) * 64 + lane, row = pos / VCPR, c = pos % VCPR;
        const int key = VPERM ? vrow(row) : row;   // LDS row `row` holds this key of the tile
        vgo[t] = (uint32_t)(key * D + (c < KCH ? c : 0) * 8) * 2;
    }
    auto stage = [&](int j, auto bufc) __attribute__((always_inline)) {   // copies of tile j into buffer bufc
        constexpr bool B1 = decltype(bufc)::value != 0;
        uint16_t* const sk = B1 ? sK1 : sK0;
        uint16_t* const sv = B1 ? sV1 : sV0;
        const uint32_t t0 = (uint32_t)j * (BC * D * 2);
#pragma unroll
        for (int t = 0; t < KPW; ++t)
            if (wave + NW * t < KNI) buf_ld16_lds(krs, kgo[t] + t0, &sk[(wave + NW * t) * 512]);
#pragma unroll
        for (int t = 0; t < VPW; ++t)
            if (wave + NW * t < VNI) buf_ld16_lds(vrs, vgo[t] + t0, &sv[(wave + NW * t) * 512]);
    };
    // Block-sparse: the mask row of this wave's query block (waves hold 32
    // rows and blocks are at least 32 rows, so one row per wave).
    const unsigned char* bmrow = nullptr;
    if constexpr (BLK) {
        const int head = bs.heads > 1 ? bh % bs.H : 0;
        bmrow = bs.mask + ((size_t)head * bs.nbq + (min(qw, N - 1) >> bs.lgbq)) * bs.nbk;
    }
    auto block_bit = [&](int key) { return bmrow[min(key >> bs.lgbk, bs.nbk - 1)] != 0; };

    // Per-lane offsets of the operand reads.  K: physical row kb*32 + ln.
    // V (transposing read): lane s of 16-lane group G reads key 8*(G/2) + s/4
    // (+4 for slots 4..7), columns 16*(G%2) + 4*(s%4); through vrow that key (plus
    // a multiple of 16) is LDS row 4*(s/4) + 2*(G/2), and key +4 the next LDS row.
    const int k_off = ln * KSTR + hf * 8;
    const int G = lane >> 4, sl = lane & 15;
    const int v_off = (VPERM ? 4 * (sl >> 2) + 2 * (G >> 1) : 8 * (G >> 1) + (sl >> 2)) * VSTR + 16 * (G & 1) +
                      4 * (sl & 3);
    constexpr int V_HI = VPERM ? VSTR : 4 * VSTR;   // offset of the second read (keys +4)

    // One key tile from LDS buffer BUF; MASK selects the masked variant (tail
    // tile, or a tile crossing this wave's diagonal under the causal mask).
    auto compute = [&](auto bufc, auto maskc, int k0) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(maskc)::value != 0;
        const uint16_t* const sk = decltype(bufc)::value ? sK1 : sK0;
        const uint16_t* const sv = decltype(bufc)::value ? sV1 : sV0;
        bool bbit[NKB];   // block-sparse: the wave's bit for each 32-key block
        if constexpr (BLK) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) bbit[kb] = block_bit(k0 + 32 * kb);
        }
        // S^T = K Q^T for the tile (rows: keys in kperm order, columns: this
        // wave's queries), with -inf where a key is not visible
        auto scores = [&](f32x16 (&s)[NKB]) __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                u32x4 ka[D / 16];   // all operands of the block first, then the MFMA chain
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) ka[ks] = ld16(&sk[k_off + kb * 32 * KSTR + ks * 16]);
                s[kb] = mfma32x32x16_zero(ka[0], qf[0]);
#pragma unroll
                for (int ks = 1; ks < D / 16; ++ks) s[kb] = mfma32x32x16(ka[ks], qf[ks], s[kb]);
            }
#if FA_FWD_SCHED
            if constexpr (D == 128 && !DROP && !BLK) {
                // the score products as a scheduling region of their own: AH K
                // operand reads first, then two products per two further reads
                constexpr int NR = NKB * D / 16, AH = FA_FWD_SCHED;
                __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
                for (int i = 0; i < (NR - AH) / 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
#endif
            if constexpr (MASK) {
                // register r of block kb holds key kb0 + d_r, with kb0 per lane
                // and d_r = 16 (r / 8) + r % 8 fixed: each test below compares
                // the constant d_r with one per-lane limit
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const int kb0 = k0 + kb * 32 + 8 * hf;
                    const int lim_n = N - kb0, lim_c = qrow - kb0;
                    const int lim_w = qrow - kb0 - window, lim_s = sinks - kb0;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int dr = 16 * (r >> 3) + (r & 7);
                        if (dr >= lim_n || (CAUSAL && (dr > lim_c || (WIN && dr <= lim_w && dr >= lim_s))) ||
                            (BLK && !bbit[kb]))
                            s[kb][r] = neg_inf();
                    }
                }
            }
        };
        // Move the reference to the tile's maximum where that exceeds it by
        // more than 2^min_log2 (rescaling O and l); returns the reference in
        // log2 units for the exponent.
        auto rebase = [&](const f32x16 (&s)[NKB], float min_log2) __attribute__((always_inline)) {
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, xor32(mx));
            const bool grow = (mx - m) * scale_log2 > min_log2;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float mnew = fmaxf(m, mx);
                // under a window or a block mask a row may have seen no visible key
                // yet (m = mnew = -inf, l and O still zero): keep it as it is
                const float alpha = (SPARSE_ROWS && m == mnew) ? 1.f : fast_exp2((m - mnew) * scale_log2);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m = mnew;
            }
            // a row with no visible key so far keeps m = -inf; its scores are all
            // -inf as well, so any finite reference gives p = 0
            return (SPARSE_ROWS && m == neg_inf()) ? 0.f : m * scale_log2;
        };
        // P = exp2(S tau log2(e) - mc) for the tile, packed to bf16 as the B
        // operand of the P V product; returns this lane's sum of the
        // (undropped) probabilities.
        auto probs = [&](const f32x16 (&s)[NKB], float mc, u32x4 (&pf)[NKB][2]) __attribute__((always_inline)) {
            // Dropout words, one generator call per lane per 32-key block: the four
            // lanes of a quad hold rows of one 4-row block, so lane r computes the
            // block of key group r (keys 16(r/2) + 8hf + 4(r%2) + 0..3) and a quad
            // transpose hands every lane its own row's word of all four groups.
            u32x4 dwq[NKB];
            if constexpr (DROP) {
                const int r4 = qrow & 3;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    dwq[kb] = quad_transpose(
                        drop.block(k0 + kb * 32 + 16 * (r4 >> 1) + 8 * hf + 4 * (r4 & 1), qrow, bh), r4);
            }
            float lt = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    // dropout words of this lane's row for keys k0+32kb+16t+8hf+0..3 and +4..7
                    uint32_t dw[2] = {0u, 0u};
                    if constexpr (DROP) {
                        dw[0] = dwq[kb][2 * t];
                        dw[1] = dwq[kb][2 * t + 1];
                    }
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const int r = 8 * t + 2 * w;
                        float p0 = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -mc));
                        float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], scale_log2, -mc));
                        lt += p0 + p1;
                        if constexpr (DROP) {   // keys 2(w%2), 2(w%2)+1 of the 4-key group w/2
                            p0 = drop.keep(dw[w >> 1], 2 * (w & 1)) ? p0 : 0.f;
                            p1 = drop.keep(dw[w >> 1], 2 * (w & 1) + 1) ? p1 : 0.f;
                        }
                        pf[kb][t][w] = pack_bf16x2(p0, p1);
                    }
                }
            return lt;
        };
        f32x16 s[NKB];
        u32x4 pf[NKB][2];
        scores(s);
        l += probs(s, rebase(s, FA_FWD_RESCALE_LOG2), pf);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int vb = v_off + (kb * 32 + 16 * t) * VSTR;
                u32x4 va[D / 32];
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    va[db] = lds_read_tr16_x2(&sv[vb + db * 32], &sv[vb + db * 32 + V_HI]);
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] = mfma32x32x16(va[db], pf[kb][t], oacc[db]);
            }
    };

    // Key tiles are visited in a sequence of positions p: under a window with
    // sinks first the nsk tiles holding sink keys below the window, then the
    // tiles tlo .. ntiles-1 (window's lower edge to the diagonal).  Position p
    // lives in buffer p % 2; the copies of position p + 1 go to the other
    // buffer while position p is computed.
    int nsk = 0, tlo = 0, tfull = 0;
    if constexpr (WIN) {
        const int q1 = min(q0 + BR, N) - 1;                 // last row of the workgroup
        const int lo_min = q0 - window + 1, lo_max = q1 - window + 1;
        tlo = max(lo_min, 0) / BC;                          // first tile any row's window reaches
        tfull = max(tlo, (max(lo_max, 0) + BC - 1) / BC);   // first tile inside every row's window
        nsk = min((sinks + BC - 1) / BC, tlo);              // sink tiles below the window
    }
    // Block-sparse: list the workgroup's active key tiles (those holding a
    // set block for one of its query blocks) in LDS, in order.  Pass 1 ballots
    // tiles in chunks of 64 per wave, a prefix sum places the chunks, pass 2
    // writes the tile numbers.
    int nact = 0;
    if constexpr (BLK) {
        const int head = bs.heads > 1 ? bh % bs.H : 0;
        const unsigned char* mh = bs.mask + (size_t)head * bs.nbq * bs.nbk;
        const int rb0 = q0 >> bs.lgbq, rb1 = (min(q0 + BR, N) - 1) >> bs.lgbq;
        auto active = [&](int t) {
            const int kb0 = (t * BC) >> bs.lgbk, kb1 = min((t * BC + BC - 1) >> bs.lgbk, bs.nbk - 1);
            bool act = false;
            for (int rb = rb0; rb <= rb1; ++rb)
                for (int kb = kb0; kb <= kb1; ++kb) act |= mh[(size_t)rb * bs.nbk + kb] != 0;
            return act;
        };
        nact = build_tile_list<NW>(active, ntiles, s_list, s_bal, s_off, wave, lane, tid);
    }
    auto tile_at = [&](int p) {
        if constexpr (BLK) return (int)s_list[min(p, max(nact - 1, 0))];
        return p < nsk ? p : tlo + (p - nsk);
    };
    // Whether any row of this wave sees a key of the tile at k0.
    auto wave_sees = [&](int k0) {
        if constexpr (BLK) {
            bool any = false;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) any |= block_bit(k0 + 32 * kb);
            if (!any) return false;
        }
        if constexpr (!CAUSAL) return true;
        if constexpr (!WIN) return k0 <= qw + 31;
        return k0 <= qw + 31 && (k0 + BC - 1 >= qw - window + 1 || k0 < sinks);
    };
    auto tile = [&](int p, auto bufc, auto maskc) __attribute__((always_inline)) {
        stage(tile_at(p + 1), ic<1 - decltype(bufc)::value>{});   // past the end: never read back
        const int k0 = tile_at(p) * BC;
        if constexpr (decltype(maskc)::value != 0) {
            if (wave_sees(k0)) compute(bufc, maskc, k0);
        } else {
            compute(bufc, maskc, k0);
        }
        wait_vmem();
        __syncthreads();
    };
    // Positions [pb, pe) with position p in buffer p % 2: an odd first
    // position alone, then pairs, then an even last one, so every buffer
    // choice is fixed at compile time.
    auto phase = [&](int pb, int pe, auto maskc) __attribute__((always_inline)) {
        int p = pb;
        if (p < pe && (p & 1)) { tile(p, ic<1>{}, maskc); ++p; }
        for (; p + 1 < pe; p += 2) {
            tile(p, ic<0>{}, maskc);
            tile(p + 1, ic<1>{}, maskc);
        }
        if (p < pe) tile(p, ic<0>{}, maskc);
    };
    // Tiles in [tfull, tdiag) need no mask in any wave: no key past N, every
    // key precedes the workgroup's first row and lies inside every row's
    // window.  The others (sinks, window edge, diagonal, sequence end) are masked.
    const int jsplit = min(CAUSAL ? q0 / BC : ntiles, nfull);
    const int tdiag = max(tfull, jsplit);
    int p1 = nsk + (tfull - tlo), p2 = nsk + (tdiag - tlo), p3 = nsk + (ntiles - tlo);
    if constexpr (BLK) p1 = p2 = 0, p3 = nact;   // block-sparse: every listed tile masked
    if (p3 > 0) stage(tile_at(0), ic<0>{});
    wait_vmem();
    __syncthreads();
    phase(0, p1, ic<1>{});
    phase(p1, p2, ic<0>{});
    phase(p2, p3, ic<1>{});

    l += xor32(l);
    // a row that saw no key (block-sparse) keeps the empty sum: O = 0, LSE = -inf
    const float inv = (BLK && l == 0.f) ? 0.f : (DROP ? drop.scale : 1.f) / l;
    if (qrow < N && hf == 0)
        LSE[(size_t)bh * N + qrow] = (BLK && l == 0.f) ? neg_inf() : m * tau + __logf(l);
    // O through LDS (stage_piece / store_rows): the staging buffers are free
    // (every tile ended with a wait for its copies and a barrier).  Wave w
    // takes 32-row block w of the K buffers, then of the V buffers.
    {
        constexpr int RB = BC / 32;   // 32-row blocks per staging buffer
        static_assert(NW <= 4 * RB, "the staging buffers hold every wave's rows");
        uint16_t* tile;
        int stride = KSTR;
        if constexpr (NW <= 2 * RB) {
            tile = (wave < RB ? sK0 : sK1) + (wave % RB) * 32 * KSTR;
        } else {
            const int blk = wave % RB, buf = wave / RB;
            if (buf < 2) {
                tile = (buf == 0 ? sK0 : sK1) + blk * 32 * KSTR;
            } else {
                tile = (buf == 2 ? sV0 : sV1) + blk * 32 * VSTR;
                stride = VSTR;
            }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16& a = oacc[db];
                stage_piece(tile, stride, ln, db * 32 + 8 * g + 4 * hf, a[4 * g] * inv,
                            a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv);
            }
        store_rows<D>(tile, stride, O + base + (size_t)qw * D, N - qw, lane);
    }
}

// Tile shapes measured on MI355X: d=128 runs 128-key tiles in 8-wave (256-row)
// workgroups, one per CU (143 KB of LDS); d=64 runs 64-key tiles in 4-wave
// workgroups, several per CU.
// The d=128 variants with dropout or a block mask carry more live registers
// (generator words, block bits) and take 64-key tiles, which halves the
// per-tile scores and probabilities and keeps them out of scratch.  The
// block-mask variants also take 4-wave workgroups: their workgroups are short
// (a tile list, a few tiles), and two of them per CU overlap each other's
// serial phases (1x32x16384x128 with 3.9% of the causal pairs: 220 -> 194 us
// against 8 waves).
template <int D, int MODE, bool DROP> struct FwdShape { static constexpr int BC = 64, NW = 4; };
template <int MODE, bool DROP> struct FwdShape<128, MODE, DROP> {
    static constexpr int BC = (DROP || MODE >= kMaskBlock) ? 64 : 128;
    static constexpr int NW = MODE >= kMaskBlock ? 4 : 8;
};

Dropout make_dropout(int thr, unsigned long long seed, unsigned int offset) {
    Dropout d;
    d.seed_lo = (uint32_t)seed;
    d.seed_hi = (uint32_t)(seed >> 32);
    d.offset = offset;
    d.thr = thr;
    d.scale = thr > 0 ? 256.f / (256.f - (float)thr) : 1.f;
    return d;
}

template <int D, int MODE, bool DROP>
void launch_bf16(const FwdArgs& a, hipStream_t st) {
    constexpr int BC = FwdShape<D, MODE, DROP>::BC, NW = FwdShape<D, MODE, DROP>::NW;
    const int bh = a.B * a.H;
    const int nq = (a.N + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MODE, BC, NW, DROP>), dim3(nq * bh), dim3(64 * NW), 0,
                       st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, a.lse, bh, a.N, a.tau * kLog2e, a.tau, nq, a.window,
                       a.sinks, make_dropout(a.drop_thr, a.seed, a.offset), a.blk);
}

template <int D>
void launch_bf16_d(const FwdArgs& a, hipStream_t st) {
    const bool win = a.causal && (a.window < a.N || a.sinks > 0);
    if (a.blk.mask) {       // block-sparse (no window, no dropout)
        a.causal ? launch_bf16<D, kMaskBlockCausal, false>(a, st)
                 : launch_bf16<D, kMaskBlock, false>(a, st);
    } else if (a.drop_thr > 0) {   // dropout: with no mask or the plain causal mask
        a.causal ? launch_bf16<D, kMaskCausal, true>(a, st) : launch_bf16<D, kMaskNone, true>(a, st);
    } else if (!a.causal) {
        launch_bf16<D, kMaskNone, false>(a, st);
    } else {
        // a window shorter than N or sinks: the window variant; otherwise the
        // plain causal mask (at d = 128 it measured 1.3% faster on the long
        // causal prefill than the window variant with window = N, both
        // without spills)
        win ? launch_bf16<D, kMaskWindow, false>(a, st) : launch_bf16<D, kMaskCausal, false>(a, st);
    }
}

}  // namespace

void launch_fwd(const FwdArgs& a, hipStream_t st) {
    if (a.dtype == kBF16) {
        a.d == 64 ? launch_bf16_d<64>(a, st) : launch_bf16_d<128>(a, st);
    } else {
        launch_fwd_f32(a, st);
    }
}

}  // namespace fa
