// fa_bwd.hip - recomputing backward of exact attention for gfx950.
//
// The backward keeps only O and the per-row statistic (here LSE = m + ln l)
// and rebuilds S and P on chip ("flash-attention" encyclopedia page, "como
// funciona", backward paragraph).  With P = exp(tau S - LSE):
//   D_i  = dO_i . O_i                       (the page's D_i = P_i . dP_i identity)
//   dV   = P^T dO,   dP = dO V^T,   dS = P o (dP - D),
//   dK   = tau dS^T Q,               dQ = tau dS K.
//
// Kernels (bf16 in, fp32 accumulation on MFMA, bf16 out; no atomics), run in
// this order:
//  bwd_dq_kernel   : one workgroup per 128-query tile (32 queries per wave, Q
//                    and dO rows in registers); first forms D for its rows
//                    from O and dO (an inner product of length d) and writes
//                    it out, then loops over 64-key tiles of K and V up to the
//                    diagonal, recomputing S^T = K Q^T and dP^T = V dO^T (one
//                    query per lane) and accumulating dQ^T += K^T dS^T with
//                    K^T from the transposing read.
//  bwd_dkdv_kernel : one workgroup per 128-key tile (32 keys per wave, K and V
//                    of those keys held in registers); loops over query tiles
//                    (128 rows at d = 64, 64 at d = 128 and under a block
//                    mask) of Q and dO copied straight into LDS (double
//                    buffered, one barrier per tile).  S = Q K^T and dP = dO V^T
//                    read their A operands row-wise (one key per result lane);
//                    dV^T += dO^T P and dK^T += Q^T dS read dO^T and Q^T with
//                    the transposing LDS read and take P and dS straight from
//                    registers as B operands; it reads the D that the dQ
//                    kernel wrote.
// A-operand rows are read in the kperm order so that the C registers of each
// lane half hold 8 consecutive rows, ready to be packed as a B operand.  Only
// tiles that cross the causal diagonal run the masked variant.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {

__device__ __forceinline__ int kperm(int m) {
    const int j = 4 * (m >> 3) + (m & 3);
    return 16 * (j >> 3) + 8 * ((m >> 2) & 1) + (j & 7);
}

template <int N_> using ic = std::integral_constant<int, N_>;

// Staged tiles (Q and dO in the dK/dV kernel, K and V in the dQ kernel) are read two ways: by
// rows (ds_read_b128, lane i at row kperm(i), 16 lanes on 16 rows of one 16-row block) and
// transposed (ds_read_b64_tr_b16, each 16-lane group on four consecutive rows, 64 bytes of each).
// With rows padded to 16 x odd bytes the row reads are free of bank conflicts, but four
// consecutive rows of the transposing reads fall on overlapping banks.  Logical row r is therefore
// stored at physical row lds_row(r): inside each 16-row block the two 2-bit fields of r trade
// places (r = 4a + b goes to 4b + a; the map is its own inverse), so the four consecutive logical
// rows of a transposing read sit four physical rows apart (4 x 16 x odd bytes = 64 mod 256: the
// four 64-byte pieces tile the banks), and the 16 rows of a row read still go to 16 distinct
// physical rows of their block.  Measured on gfx950 with the two patterns alone (fa_calib_lds,
// eight waves per workgroup): transposing reads at 272-byte rows 63 B per clock per CU before,
// about 180 after; at 144-byte rows 120 before, about 185 after; row reads about 235 either way.
// The block-sparse kernels keep plain row order (PERM = false): their few, scattered query or key
// tiles measured 2.5% slower with the permutation (the 1x32x16384x128 band-and-global backward,
// 0.739 -> 0.759 ms), while the dense and window backward gained.
template <bool PERM>
__device__ __forceinline__ int lds_row(int r) {
    return PERM ? (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3) : r;
}
// Per-lane offsets (elements) of the operand reads.  Row reads: tile row kperm(lane % 32), column
// 8 * (lane / 32).  Transposing reads (lane s of 16-lane group G): tile row 8*(G/2) + s/4, and
// four rows on for the second read of a pair, column 16*(G%2) + 4*(s%4); with the permutation that
// tile row (plus a multiple of 16) is LDS row 4*(s/4) + 2*(G/2), and the second read's row the next
// LDS row.
template <bool PERM, int STR>
__device__ __forceinline__ int row_read_off(int lane) { return lds_row<PERM>(kperm(lane & 31)) * STR + (lane >> 5) * 8; }
template <bool PERM, int STR>
__device__ __forceinline__ int tr_read_off(int lane) {
    const int G = lane >> 4, sl = lane & 15;
    return (PERM ? 4 * (sl >> 2) + 2 * (G >> 1) : 8 * (G >> 1) + (sl >> 2)) * STR + 16 * (G & 1) + 4 * (sl & 3);
}
template <bool PERM, int STR>
constexpr int tr_second_row() { return PERM ? STR : 4 * STR; }

// Direct global -> LDS staging of a tile of ROWS rows of a [N, D] bf16 matrix
// into padded LDS rows of STR elements (STR*2 = 16 * odd bytes), tile row r at LDS row
// lds_row<PERM>(r).  One wave instruction fills 1 KB of LDS; every lane loads the 16-byte chunk that
// belongs at its LDS position (padding positions load a duplicate chunk that
// is never read).  Rows past N read as zeros through the buffer descriptor.
// The byte offsets are recomputed at each issue (a few integer operations):
// held in an array inside the struct, which the kernels' lambdas capture by
// reference, they were kept in scratch memory in some variants.
template <int ROWS, int D, int STR, int NWAVES, bool PERM>
struct TileCopy {
    static constexpr int CPR = STR / 8, NI = ROWS * CPR / 64, PW = (NI + NWAVES - 1) / NWAVES;
    static_assert(ROWS * CPR % 64 == 0, "whole wave instructions");
    int wave, lane;
    __device__ void init(int wave_, int lane_) { wave = wave_; lane = lane_; }
    __device__ void issue(rsrc_t rs, int row0, uint16_t* lds, int) const {
        const uint32_t t0 = (uint32_t)row0 * (D * 2);
#pragma unroll
        for (int t = 0; t < PW; ++t)
            if (wave + NWAVES * t < NI) {
                const int pos = (wave + NWAVES * t) * 64 + lane, row = pos / CPR, c = pos % CPR;
                // LDS row `row` holds tile row lds_row(row) (the map is its own inverse)
                const uint32_t off = (uint32_t)(lds_row<PERM>(row) * D + (c < D / 8 ? c : 0) * 8) * 2;
                buf_ld16_lds(rs, off + t0, lds + (wave + NWAVES * t) * 512);
            }
    }
};

// Mask modes: none, causal, causal with a sliding window and sink tokens
// (key j visible to query i iff j <= i and (i - j < window or j < sinks)).
enum : int { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2, kMaskBlock = 3, kMaskBlockCausal = 4 };

// Block-sparse dK/dV: whether query tile t (rows t*BR .. t*BR+BR-1) holds a
// set block against key blocks kb0 .. kb1 of mask head mh (before the causal
// diagonal, t < qt0, it never does).
template <int BR, bool CAUSAL>
__device__ __forceinline__ bool blk_qtile_active(const BlockSparse& bs, const unsigned char* mh, int t,
                                                 int qt0, int kb0, int kb1) {
    if (CAUSAL && t < qt0) return false;
    const int rb0 = (t * BR) >> bs.lgbq, rb1 = min((t * BR + BR - 1) >> bs.lgbq, bs.nbq - 1);
    bool act = false;
    for (int rb = rb0; rb <= rb1; ++rb)
        for (int kb = kb0; kb <= kb1; ++kb) act |= mh[(size_t)rb * bs.nbk + kb] != 0;
    return act;
}

// Split plan, pass 1: one wave per (key tile, head) item counts the active
// query tiles of its list (the same predicate the dK/dV workgroup lists them
// with) into plan[4 item] and clears the item's arrival count.
template <int BR, bool CAUSAL>
__global__ __launch_bounds__(256) void blk_count_kernel(BlockSparse bs, int BH, int N, int n_items,
                                                        int* __restrict__ plan) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int item = (int)blockIdx.x * 4 + wave;
    if (item >= n_items) return;
    const int kt = item / BH, bh = item % BH, k0 = kt * kBlkKeys;
    const int head = bs.heads > 1 ? bh % bs.H : 0;
    const unsigned char* mh = bs.mask + (size_t)head * bs.nbq * bs.nbk;
    const int kb0 = k0 >> bs.lgbk, kb1 = (min(k0 + kBlkKeys, N) - 1) >> bs.lgbk;
    const int n_qt = (N + BR - 1) / BR, qt0 = CAUSAL ? k0 / BR : 0;
    int count = 0;
    for (int c = 0; c < n_qt; c += 64) {
        const int t = c + lane;
        const bool act = t < n_qt && blk_qtile_active<BR, CAUSAL>(bs, mh, t, qt0, kb0, kb1);
        count += __builtin_popcountll(__builtin_amdgcn_ballot_w64(act));
    }
    if (lane == 0) {
        plan[4 * item] = count;
        plan[4 * item + 3] = 0;
    }
}

// Exclusive prefix sum over the 1024 threads of a workgroup; *total receives
// the sum.  sh: 16 ints of LDS.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int w = lane < 16 ? sh[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(w, o);
            if (lane >= o) w += y;
        }
        if (lane < 16) sh[lane] = w;
    }
    __syncthreads();
    const int off = wave ? sh[wave - 1] : 0;
    *total = sh[15];
    __syncthreads();
    return off + x - v;
}

// Split plan, pass 2 (one workgroup of 1024 threads, each taking a run of
// consecutive items): a part holds at most T query tiles, T = max(kBlkMinPart, twice
// the mean list length, the total over the resident workgroups); an item of
// two or more parts gets one slot per part and one helper per part after the
// first, in item order while slots last (later items keep nh = 0 and are
// walked whole by their owner).  Writes plan[4 i] = helpers, [4 i + 1] =
// first helper, [4 i + 2] = first slot and meta[0] = helpers in use.
__global__ __launch_bounds__(1024) void blk_plan_kernel(int* __restrict__ plan, int* __restrict__ meta,
                                                        int n_items, int slots, int conc) {
    __shared__ int sh[16];
    __shared__ long long shl[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n_items + 1023) / 1024, i0 = min(tid * per, n_items), i1 = min(i0 + per, n_items);
    long long mine = 0;
    for (int i = i0; i < i1; ++i) mine += plan[4 * i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o);
    if (lane == 0) shl[wave] = mine;
    __syncthreads();
    long long total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) total += shl[w];
    const long long t = max((long long)kBlkMinPart, max((2 * total + n_items - 1) / n_items, (total + conc - 1) / conc));
    const int T = (int)min(t, 1LL << 30);
    auto parts_of = [&](int i) { return (plan[4 * i] + T - 1) / T; };
    // Slot demand per thread, capped at slots + 1: the prefix stays exact
    // below the slot count and exceeds it whenever the true sum does.
    int need_sum = 0;
    for (int i = i0; i < i1; ++i) {
        const int p = parts_of(i);
        need_sum = min(need_sum + (p >= 2 ? p : 0), slots + 1);
    }
    int tot_s;
    int sb = min(block_excl_scan(need_sum, sh, &tot_s), slots + 1);
    // helpers: the items that fit take parts - 1 each (slots run out in item order)
    int nh_sum = 0;
    {
        int run = sb;
        for (int i = i0; i < i1; ++i) {
            const int p = parts_of(i), need = p >= 2 ? p : 0;
            if (need && run + need <= slots) nh_sum += p - 1;
            run = min(run + need, slots + 1);
        }
    }
    int tot_h;
    int hb = block_excl_scan(nh_sum, sh, &tot_h);
    for (int i = i0; i < i1; ++i) {
        const int p = parts_of(i), need = p >= 2 ? p : 0;
        const int nh = (need && sb + need <= slots) ? p - 1 : 0;
        // every read of plan[4 i] above precedes this store (same thread)
        plan[4 * i] = nh;
        plan[4 * i + 1] = hb;
        plan[4 * i + 2] = sb;
        sb = min(sb + need, slots + 1);
        hb += nh;
    }
    if (tid == 0) meta[0] = tot_h;
}

// DROP: the forward dropped P with the mask of Dropout::block; with
// Z = keep / (1 - p): dV = (P o Z)^T dO and dS = P o (Z o dP - D).
template <int D, int MODE, bool DROP>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int N, float scale_log2,
    float tau, int window, int sinks, Dropout drop, BlockSparse bs, BlkSplit split) {
    constexpr bool CAUSAL = MODE == kMaskCausal || MODE == kMaskWindow || MODE == kMaskBlockCausal;
    constexpr bool WIN = MODE == kMaskWindow, BLK = MODE >= kMaskBlock;
    // d = 64 streams 128-query tiles (measured 4% faster than 64 on the 1k and
    // 4k causal backward); d = 128 and the block-sparse variants keep 64, where
    // the larger tile would cost occupancy or is unmeasured.
    constexpr int BC = 128, BR = (D == 64 && !BLK) ? 128 : 64;
    static_assert(!BLK || (BC == kBlkKeys && BR == 64), "the split plan counts 64-row query tiles of 128 keys");
    constexpr int STR = D + 8;                 // padded row (16 * odd bytes)
    // Without dropout, dS = P o (dP - D) takes -D as the starting accumulator
    // of the dP = dO V^T product, so the subtraction costs nothing; LDS then
    // holds -D.  (With dropout, dS = P o (Z o dP - D) scales dP alone.)  This
    // saves one vector operation per probability: 7% on the 4k causal backward.
    constexpr bool DNEG = !DROP;
    // Double buffers as distinct LDS variables picked at compile time, so that
    // reads of one buffer are not made to wait for the copies landing in the
    // other (see the forward kernel).
    __shared__ __attribute__((aligned(16))) uint16_t sQ0[BR * STR], sQ1[BR * STR];
    __shared__ __attribute__((aligned(16))) uint16_t sdO0[BR * STR], sdO1[BR * STR];
    __shared__ __attribute__((aligned(16))) float sL0[BR], sL1[BR];
    __shared__ __attribute__((aligned(16))) float sD0[BR], sD1[BR];
    // block-sparse: the workgroup's active query tiles, in order
    __shared__ uint16_t s_list[BLK ? kMaxSparseTiles : 1];
    __shared__ uint64_t s_bal[BLK ? kMaxSparseTiles / 64 : 1];
    __shared__ int s_off[BLK ? kMaxSparseTiles / 64 + 1 : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int ln = lane & 31, hf = lane >> 5;
    // Block-sparse with a split plan: the first split.slots workgroups are
    // helpers (helper g takes part g - first + 1 of the item whose helper range
    // holds g; unused helpers leave at once), the rest own one item each.
    int item = (int)blockIdx.x, part = 0, nparts = 1, sbase = 0;
    if constexpr (BLK) {
        if (split.plan) {
            const int n_items = (int)gridDim.x - split.slots;
            if ((int)blockIdx.x < split.slots) {
                const int g = (int)blockIdx.x;
                if (g >= split.meta[0]) return;
                int lo = 0, hi = n_items - 1;   // the last item whose first helper is <= g
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (split.plan[4 * mid + 1] <= g) lo = mid;
                    else hi = mid - 1;
                }
                item = lo;
                part = g - split.plan[4 * item + 1] + 1;
                nparts = split.plan[4 * item] + 1;
                sbase = split.plan[4 * item + 2];
            } else {
                item = (int)blockIdx.x - split.slots;   // reads its plan entry once its list is known
            }
        }
    }
    const int kt = item / BH;      // causal: low key tiles carry the most work
    const int bh = item % BH;
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

    const rsrc_t qrs = make_rsrc(Q + base, (uint32_t)N * D * 2);
    const rsrc_t ors = make_rsrc(dO + base, (uint32_t)N * D * 2);
    TileCopy<BR, D, STR, 4, !BLK> cp;
    cp.init(wave, lane);
    // operand read offsets: A operand rows (queries) in kperm order; transposed
    // operands via the transposing read
    const int a_off = row_read_off<!BLK, STR>(lane);
    const int t_off = tr_read_off<!BLK, STR>(lane);
    constexpr int T2 = tr_second_row<!BLK, STR>();

    const int n_qt = (N + BR - 1) / BR;
    const int qt0 = CAUSAL ? k0 / BR : 0;
    // The next tile's LSE (threads < BR) or D (threads BR .. 2BR-1) value of
    // this thread, raw: one register whose load is only waited for when it is
    // written to LDS after the current tile's math.  (Two variables assigned
    // under the thread test became a private array in scratch, and the store
    // into it waited for every outstanding load, the next tile's Q and dO
    // copies included, before the current tile could start.)
    const bool ld_is_l = tid < BR;
    const float* const ld_src = (ld_is_l ? LSE : Dv) + (size_t)bh * N;
    float ld_v = 0.f;
    auto stage = [&](int qt, auto bufc) __attribute__((always_inline)) {
        constexpr bool B1 = decltype(bufc)::value != 0;
        const int q0 = qt * BR;
        cp.issue(qrs, q0, B1 ? sQ1 : sQ0, wave);
        cp.issue(ors, q0, B1 ? sdO1 : sdO0, wave);
        if (tid < 2 * BR) {
            const int q = q0 + (tid & (BR - 1));
            ld_v = q < N ? ld_src[q] : (ld_is_l ? __builtin_inff() : 0.f);
        }
    };
    auto stage_ld = [&](auto bufc) __attribute__((always_inline)) {
        constexpr bool B1 = decltype(bufc)::value != 0;
        if (ld_is_l) (B1 ? sL1 : sL0)[tid] = ld_v * kLog2e;
        else if (tid < 2 * BR) (B1 ? sD1 : sD0)[tid - BR] = DNEG ? -ld_v : ld_v;
    };

    // Block-sparse: this wave's key block (waves hold 32 keys, blocks >= 32)
    // and the bit of the query block holding row q.
    const unsigned char* bmcol = nullptr;
    if constexpr (BLK) {
        const int head = bs.heads > 1 ? bh % bs.H : 0;
        bmcol = bs.mask + (size_t)head * bs.nbq * bs.nbk + (min(kw, N - 1) >> bs.lgbk);
    }
    auto block_bit = [&](int q) { return bmcol[(size_t)min(q >> bs.lgbq, bs.nbq - 1) * bs.nbk] != 0; };

    // Unmasked tiles without dropout or a block mask (every 32-query block
    // runs, dS = P o (dP - D) with -D in dP's accumulator): the same arithmetic
    // as compute() below, software-pipelined over the blocks.  Block qb's S
    // and dP products are issued before block qb-1's dV and dK products, and
    // block qb's softmax does not depend on those, so one wave's vector and
    // matrix work can overlap instead of waiting on each other in turn (4k
    // causal backward, outputs bit-identical: dK/dV 2% faster at d = 64, 7% at
    // d = 128).  The general body keeps its order: held across a block, the
    // packed operands cost 16 registers, which the dropout variants lack.
    auto compute_pipe = [&](auto bufc, int q0) __attribute__((always_inline)) {
        constexpr bool B1 = decltype(bufc)::value != 0;
        const uint16_t* q_lds = B1 ? sQ1 : sQ0;
        const uint16_t* o_lds = B1 ? sdO1 : sdO0;
        const float* l_lds = B1 ? sL1 : sL0;
        const float* d_lds = B1 ? sD1 : sD0;
        auto sdp = [&](int qb, f32x16& sacc, f32x16& dp, f32x4* lq) __attribute__((always_inline)) {
            u32x4 qa[D / 16], oa[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                qa[ks] = ld16(q_lds + qb * 32 * STR + a_off + ks * 16);
                oa[ks] = ld16(o_lds + qb * 32 * STR + a_off + ks * 16);
            }
            f32x4 dq4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lq[i] = *reinterpret_cast<const f32x4*>(&l_lds[qb * 32 + 16 * (i >> 1) + 8 * hf + 4 * (i & 1)]);
                dq4[i] = *reinterpret_cast<const f32x4*>(&d_lds[qb * 32 + 16 * (i >> 1) + 8 * hf + 4 * (i & 1)]);
            }
            f32x16 negd;
#pragma unroll
            for (int r = 0; r < 16; ++r) negd[r] = dq4[r >> 2][r & 3];
            sacc = mfma32x32x16_zero(qa[0], kf[0]);
            dp = mfma32x32x16(oa[0], vf[0], negd);
#pragma unroll
            for (int ks = 1; ks < D / 16; ++ks) {
                sacc = mfma32x32x16(qa[ks], kf[ks], sacc);
                dp = mfma32x32x16(oa[ks], vf[ks], dp);
            }
        };
        auto soft = [&](const f32x16& sacc, const f32x16& dp, const f32x4* lq, u32x4* pf, u32x4* dsf)
            __attribute__((always_inline)) {
            float pv[16], dv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pv[r] = fast_exp2(__builtin_fmaf(sacc[r], scale_log2, -lq[r >> 2][r & 3]));
                dv[r] = pv[r] * dp[r];
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pf[t][w] = pack_bf16x2(pv[8 * t + 2 * w], pv[8 * t + 2 * w + 1]);
                    dsf[t][w] = pack_bf16x2(dv[8 * t + 2 * w], dv[8 * t + 2 * w + 1]);
                }
        };
        auto acc = [&](int qb, const u32x4* pf, const u32x4* dsf) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int tb = t_off + (qb * 32 + 16 * t) * STR;
                u32x4 ot[D / 32], qt4[D / 32];
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    ot[db] = lds_read_tr16_x2(o_lds + tb + db * 32, o_lds + tb + db * 32 + T2);
                    qt4[db] = lds_read_tr16_x2(q_lds + tb + db * 32, q_lds + tb + db * 32 + T2);
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    dvacc[db] = mfma32x32x16(ot[db], pf[t], dvacc[db]);
                    dkacc[db] = mfma32x32x16(qt4[db], dsf[t], dkacc[db]);
                }
            }
        };
        f32x16 sacc, dp;
        f32x4 lq[4];
        u32x4 pf[2], dsf[2];
        sdp(0, sacc, dp, lq);
        soft(sacc, dp, lq, pf, dsf);
#pragma unroll
        for (int qb = 1; qb < BR / 32; ++qb) {
            sdp(qb, sacc, dp, lq);
            acc(qb - 1, pf, dsf);
            soft(sacc, dp, lq, pf, dsf);
        }
        acc(BR / 32 - 1, pf, dsf);
    };

    auto compute = [&](auto bufc, int q0, auto maskc) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(maskc)::value != 0;
        if constexpr (!MASK && !BLK && !DROP) {
            compute_pipe(bufc, q0);
            return;
        }
        constexpr bool B1 = decltype(bufc)::value != 0;
        const uint16_t* q_lds = B1 ? sQ1 : sQ0;
        const uint16_t* o_lds = B1 ? sdO1 : sdO0;
        const float* l_lds = B1 ? sL1 : sL0;
        const float* d_lds = B1 ? sD1 : sD0;
#pragma unroll
        for (int qb = 0; qb < BR / 32; ++qb) {
            const int qs = q0 + qb * 32;
            if (MASK && CAUSAL && qs + 31 < kw) continue;   // all these queries precede the keys
            if (MASK && WIN && qs - (kw + 31) >= window && kw >= sinks) continue;   // all past the window
            if (BLK && !block_bit(qs)) continue;   // the 32 x 32 block is clear
            u32x4 qa[D / 16], oa[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                qa[ks] = ld16(q_lds + qb * 32 * STR + a_off + ks * 16);
                oa[ks] = ld16(o_lds + qb * 32 * STR + a_off + ks * 16);
            }
            // register r holds query qb*32 + 16*(r/8) + 8*hf + r%8 (key = this lane's)
            f32x4 lq[4], dq4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lq[i] = *reinterpret_cast<const f32x4*>(&l_lds[qb * 32 + 16 * (i >> 1) + 8 * hf + 4 * (i & 1)]);
                dq4[i] = *reinterpret_cast<const f32x4*>(&d_lds[qb * 32 + 16 * (i >> 1) + 8 * hf + 4 * (i & 1)]);
            }
            f32x16 sacc = mfma32x32x16_zero(qa[0], kf[0]);
            f32x16 dp;
            if constexpr (DNEG) {
                f32x16 negd;   // -D of each register's query
#pragma unroll
                for (int r = 0; r < 16; ++r) negd[r] = dq4[r >> 2][r & 3];
                dp = mfma32x32x16(oa[0], vf[0], negd);
            } else {
                dp = mfma32x32x16_zero(oa[0], vf[0]);
            }
#pragma unroll
            for (int ks = 1; ks < D / 16; ++ks) {
                sacc = mfma32x32x16(qa[ks], kf[ks], sacc);
                dp = mfma32x32x16(oa[ks], vf[ks], dp);
            }
            // dropout bits: 4-query group g = r/4 holds queries
            // qs + 16 (g/2) + 8 hf + 4 (g%2) + 0..3.  The four lanes of a quad
            // hold keys of one 4-key block, so lane e computes the block of
            // query group e, byte-transposes it (byte w of word e' = byte e'
            // of word w) and a quad transpose hands lane key%4 its byte of
            // every word of all four groups: byte w of kb4[g] = bit (query
            // 4-group g + w, this key).
            u32x4 kb4;
            if constexpr (DROP) {
                const int e = key & 3;
                kb4 = quad_transpose(byte_transpose(
                          drop.block(key, qs + 16 * (e >> 1) + 8 * hf + 4 * (e & 1), bh)), e);
            }
            // register r holds query qb0 + d_r, d_r = 16 (r / 8) + r % 8: the mask
            // tests compare the constant d_r with per-lane limits
            const int qb0 = qs + 8 * hf;
            const int lim_c = key - qb0, lim_w = key - qb0 + window;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(__builtin_fmaf(sacc[r], scale_log2, -lq[r >> 2][r & 3]));
                if constexpr (MASK) {
                    const int dr = 16 * (r >> 3) + (r & 7);
                    if (CAUSAL && (dr < lim_c || (WIN && dr >= lim_w && key >= sinks))) p = 0.f;
                }
                if constexpr (DROP) {
                    const bool kept = drop.keep(kb4[r >> 2], r & 3);
                    sacc[r] = kept ? p : 0.f;
                    dp[r] = p * ((kept ? dp[r] * drop.scale : 0.f) - dq4[r >> 2][r & 3]);
                } else {
                    sacc[r] = p;
                    dp[r] = DNEG ? p * dp[r] : p * (dp[r] - dq4[r >> 2][r & 3]);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u32x4 pf, dsf;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pf[w] = pack_bf16x2(sacc[8 * t + 2 * w], sacc[8 * t + 2 * w + 1]);
                    dsf[w] = pack_bf16x2(dp[8 * t + 2 * w], dp[8 * t + 2 * w + 1]);
                }
                const int tb = t_off + (qb * 32 + 16 * t) * STR;
                u32x4 ot[D / 32], qt4[D / 32];
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    ot[db] = lds_read_tr16_x2(o_lds + tb + db * 32, o_lds + tb + db * 32 + T2);
                    qt4[db] = lds_read_tr16_x2(q_lds + tb + db * 32, q_lds + tb + db * 32 + T2);
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    dvacc[db] = mfma32x32x16(ot[db], pf, dvacc[db]);
                    dkacc[db] = mfma32x32x16(qt4[db], dsf, dkacc[db]);
                }
            }
        }
    };

    // query tiles that reach into this workgroup's keys need the causal mask
    const int qmask_end = CAUSAL ? min(n_qt, (k0 + BC + BR - 1) / BR) : qt0;
    // Under a window: no query past the last key's window sees the tile
    // unless it holds sink keys (qt_end), and query tiles from qwin on have a
    // query beyond some key's window (masked).
    int qt_end = n_qt, qwin = n_qt;
    if constexpr (WIN) {
        if (k0 >= sinks) qt_end = min(n_qt, (k0 + BC - 1 + window - 1) / BR + 1);
        qwin = max(0, (k0 + window - BR + 1 + BR - 1) / BR);
    }
    const int qu_end = max(qmask_end, min(qwin, qt_end));   // end of the unmasked query tiles
    // Query tiles are visited as positions p = 0, 1, ...: tile qt0 + p, or
    // under a block mask the p-th listed active tile; position p lives in
    // buffer p % 2.
    int npos = qt_end - qt0, pm1 = qmask_end - qt0, pu = max(pm1, qu_end - qt0);
    if constexpr (BLK) {
        const int head = bs.heads > 1 ? bh % bs.H : 0;
        const unsigned char* mh = bs.mask + (size_t)head * bs.nbq * bs.nbk;
        const int kb0 = k0 >> bs.lgbk, kb1 = (min(k0 + BC, N) - 1) >> bs.lgbk;
        auto active = [&](int t) { return blk_qtile_active<BR, CAUSAL>(bs, mh, t, qt0, kb0, kb1); };
        npos = build_tile_list<4>(active, n_qt, s_list, s_bal, s_off, wave, lane, tid);
        pm1 = pu = 0;   // every listed tile runs the masked body
    }
    // positions [pbeg, pend) of the list are this workgroup's part
    int pbeg = 0, pend = npos;
    if constexpr (BLK) {
        // An owner's list can only have been split if it is longer than the
        // smallest part (kBlkMinPart tiles); a short list skips the plan read.
        if (split.plan && (int)blockIdx.x >= split.slots && npos > kBlkMinPart) {
            nparts = split.plan[4 * item] + 1;
            sbase = split.plan[4 * item + 2];
        }
        if (nparts > 1) {   // npos <= 4096 and nparts <= npos: no overflow
            pbeg = part * npos / nparts;
            pend = (part + 1) * npos / nparts;
        }
    }
    auto qt_at = [&](int p) {
        if constexpr (BLK) return (int)s_list[min(p, max(npos - 1, 0))];
        return qt0 + p;
    };
    if (pbeg < pend) {
        if (pbeg & 1) {
            stage(qt_at(pbeg), ic<1>{});
            stage_ld(ic<1>{});
        } else {
            stage(qt_at(pbeg), ic<0>{});
            stage_ld(ic<0>{});
        }
        wait_vmem();
        __syncthreads();
    }
    auto tile_b = [&](int p, auto bufc, auto maskc) __attribute__((always_inline)) {   // position p lives in buffer bufc
        constexpr ic<1 - decltype(bufc)::value> other{};
        if (p + 1 < pend) stage(qt_at(p + 1), other);
        const int q0 = qt_at(p) * BR;
        if (!(CAUSAL && q0 + BR - 1 < kw) && !(WIN && q0 - (kw + 31) >= window && kw >= sinks))
            compute(bufc, q0, maskc);
        if (p + 1 < pend) stage_ld(other);
        wait_vmem();
        __syncthreads();
    };
    // Positions [pb, pe), position p in buffer p % 2: an odd first position
    // alone, then pairs, then an even last one (buffers fixed at compile time).
    auto phase = [&](int pb, int pe, auto maskc) __attribute__((always_inline)) {
        int p = pb;
        if (p < pe && (p & 1)) { tile_b(p, ic<1>{}, maskc); ++p; }
        for (; p + 1 < pe; p += 2) {
            tile_b(p, ic<0>{}, maskc);
            tile_b(p + 1, ic<1>{}, maskc);
        }
        if (p < pe) tile_b(p, ic<0>{}, maskc);
    };
    if constexpr (BLK) {
        phase(pbeg, pend, ic<1>{});
    } else {
        phase(0, pm1, ic<1>{});
        phase(max(0, pm1), pu, ic<0>{});
        phase(max(0, pu), npos, ic<1>{});
    }

    // A part of a split list: write this part's fp32 partials to its slot
    // (lane-contiguous float4 pieces in the accumulator layout), publish them,
    // count the arrival; the part that arrives last adds every part's slot in
    // part order (so the sum does not depend on which part finished last) and
    // goes on to the epilogue, the others leave.  No workgroup waits for another.
    if constexpr (BLK) {
        if (nparts > 1) {
            constexpr int SLOT = 2 * kBlkKeys * D;   // floats per slot
            auto piece = [&](int which, int db, int g) {
                return ((((which * 4 + wave) * (D / 32) + db) * 4 + g) * 64 + lane) * 4;
            };
            float* const mine = split.pool + (size_t)(sbase + part) * SLOT;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    *reinterpret_cast<f32x4*>(mine + piece(0, db, g)) =
                        f32x4{dkacc[db][4 * g], dkacc[db][4 * g + 1], dkacc[db][4 * g + 2], dkacc[db][4 * g + 3]};
                    *reinterpret_cast<f32x4*>(mine + piece(1, db, g)) =
                        f32x4{dvacc[db][4 * g], dvacc[db][4 * g + 1], dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]};
                }
            __shared__ int s_last;
            __threadfence();
            __syncthreads();
            if (tid == 0)
                s_last = __hip_atomic_fetch_add(split.plan + 4 * item + 3, 1, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
            __syncthreads();
            if (!s_last) return;
            __threadfence();
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) { dkacc[db][r] = 0.f; dvacc[db][r] = 0.f; }
            for (int pp = 0; pp < nparts; ++pp) {
                const float* const src = split.pool + (size_t)(sbase + pp) * SLOT;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(src + piece(0, db, g));
                        const f32x4 b = *reinterpret_cast<const f32x4*>(src + piece(1, db, g));
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            dkacc[db][4 * g + e] += a[e];
                            dvacc[db][4 * g + e] += b[e];
                        }
                    }
            }
        }
    }

    // Epilogue through LDS (stage_piece / store_rows); the staging buffers are
    // free: every tile ended with a barrier and no copy is in flight.
    {
        constexpr int WPB = BR / 32;   // waves' row blocks per staging buffer
        uint16_t* const kr = (wave < WPB ? sQ0 : sQ1) + (wave % WPB) * 32 * STR;
        uint16_t* const vr = (wave < WPB ? sdO0 : sdO1) + (wave % WPB) * 32 * STR;
        const float vs = DROP ? drop.scale : 1.f;   // Z's scale, factored out of dV
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hf;
                const f32x16& ka = dkacc[db];
                const f32x16& va = dvacc[db];
                stage_piece(kr, STR, ln, d, ka[4 * g] * tau, ka[4 * g + 1] * tau, ka[4 * g + 2] * tau,
                            ka[4 * g + 3] * tau);
                stage_piece(vr, STR, ln, d, va[4 * g] * vs, va[4 * g + 1] * vs, va[4 * g + 2] * vs,
                            va[4 * g + 3] * vs);
            }
        store_rows<D>(kr, STR, dK + base + (size_t)kw * D, N - kw, lane);
        store_rows<D>(vr, STR, dV + base + (size_t)kw * D, N - kw, lane);
    }
}

template <int D, int MODE, bool DROP>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ Dv, uint16_t* __restrict__ dQ, int BH, int N, float scale_log2, float tau,
    int n_qtiles, int window,
    int sinks, Dropout drop, BlockSparse bs) {
    constexpr bool CAUSAL = MODE == kMaskCausal || MODE == kMaskWindow || MODE == kMaskBlockCausal;
    constexpr bool WIN = MODE == kMaskWindow, BLK = MODE >= kMaskBlock;
    constexpr int BR = 128, BC = 64;
    constexpr int STR = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sK0[BC * STR], sK1[BC * STR];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[BC * STR], sV1[BC * STR];
    // block-sparse: the workgroup's active key tiles, in order
    __shared__ uint16_t s_list[BLK ? kMaxSparseTiles : 1];
    __shared__ uint64_t s_bal[BLK ? kMaxSparseTiles / 64 : 1];
    __shared__ int s_off[BLK ? kMaxSparseTiles / 64 + 1 : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int ln = lane & 31, hf = lane >> 5;
    const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
    const int bh = (int)(blockIdx.x % BH);
    const size_t base = (size_t)bh * N * D;
    const int q0 = qt * BR, qw = q0 + 32 * wave, qrow = qw + ln;

    // D_i = dO_i . O_i (the page's identity D_i = P_i . dP_i = dO_i . O_i),
    // formed here from the rows this wave owns: each lane holds half of its
    // row's d entries (the same slices as its dO operands), the two wave
    // halves are added, and the value is written to the workspace for the
    // dK/dV kernel, which runs after this one.
    u32x4 qf[D / 16], df[D / 16];
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const size_t off = base + (size_t)qrow * D + ks * 16 + hf * 8;
        qf[ks] = qrow < N ? ld16(Q + off) : u32x4{0, 0, 0, 0};
        df[ks] = qrow < N ? ld16(dO + off) : u32x4{0, 0, 0, 0};
        const u32x4 of = qrow < N ? ld16(O + off) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dpart += bf16lo(of[i]) * bf16lo(df[ks][i]) + bf16hi(of[i]) * bf16hi(df[ks][i]);
    }
    const float lse2 = qrow < N ? LSE[(size_t)bh * N + qrow] * kLog2e : __builtin_inff();
    const float Dq = dpart + xor32(dpart);
    if (hf == 0 && qrow < N) Dv[(size_t)bh * N + qrow] = Dq;
    // Without dropout the dP = dO V^T products start from -D (one query per
    // lane), so dS = P o (dP - D) needs no subtraction.
    constexpr bool DNEG = !DROP;
    f32x16 negd;
#pragma unroll
    for (int r = 0; r < 16; ++r) negd[r] = -Dq;
    f32x16 dqacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

    const rsrc_t krs = make_rsrc(K + base, (uint32_t)N * D * 2);
    const rsrc_t vrs = make_rsrc(V + base, (uint32_t)N * D * 2);
    TileCopy<BC, D, STR, 4, !BLK> cp;
    cp.init(wave, lane);
    // operand read offsets as in the dK/dV kernel
    const int a_off = row_read_off<!BLK, STR>(lane);
    const int t_off = tr_read_off<!BLK, STR>(lane);
    constexpr int T2 = tr_second_row<!BLK, STR>();

    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kend + BC - 1) / BC;

    // Keys past N are zero rows (buffer descriptor) but still get a
    // probability exp2(-LSE) from their zero score, which overflows to inf
    // for a row whose LSE is below about -88; inf times their K = 0 would
    // make the row's dQ NaN, so the tile holding them runs the masked body,
    // which gives them p = 0 (as the forward does).
    // Block-sparse: the mask row of this wave's query block (waves hold 32
    // rows, blocks >= 32) and the bit of the key block holding key j.
    const unsigned char* bmrow = nullptr;
    if constexpr (BLK) {
        const int head = bs.heads > 1 ? bh % bs.H : 0;
        bmrow = bs.mask + ((size_t)head * bs.nbq + (min(qw, N - 1) >> bs.lgbq)) * bs.nbk;
    }
    auto block_bit = [&](int j) { return bmrow[min(j >> bs.lgbk, bs.nbk - 1)] != 0; };

    auto compute = [&](auto bufc, int k0, auto maskc) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(maskc)::value != 0;
        const uint16_t* k_lds = decltype(bufc)::value ? sK1 : sK0;
        const uint16_t* v_lds = decltype(bufc)::value ? sV1 : sV0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (BLK && !block_bit(k0 + 32 * kb)) continue;   // the 32 x 32 block is clear
            u32x4 ka[D / 16], va[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                ka[ks] = ld16(k_lds + kb * 32 * STR + a_off + ks * 16);
                va[ks] = ld16(v_lds + kb * 32 * STR + a_off + ks * 16);
            }
            f32x16 sacc = mfma32x32x16_zero(ka[0], qf[0]);
            f32x16 dp = DNEG ? mfma32x32x16(va[0], df[0], negd) : mfma32x32x16_zero(va[0], df[0]);
#pragma unroll
            for (int ks = 1; ks < D / 16; ++ks) {
                sacc = mfma32x32x16(ka[ks], qf[ks], sacc);
                dp = mfma32x32x16(va[ks], df[ks], dp);
            }
            // dropout words of this lane's row for the 4-key groups g = r/4:
            // keys k0 + 32 kb + 16 (g/2) + 8 hf + 4 (g%2) + 0..3, byte r%4
            // (one generator call per lane: lane r of the quad computes key
            // group r, a quad transpose hands out the rows' words)
            u32x4 dw = {0u, 0u, 0u, 0u};
            if constexpr (DROP) {
                const int r4 = qrow & 3;
                dw = quad_transpose(
                    drop.block(k0 + kb * 32 + 16 * (r4 >> 1) + 8 * hf + 4 * (r4 & 1), qrow, bh), r4);
            }
            // register r holds key kb0 + d_r, d_r = 16 (r / 8) + r % 8: the mask
            // tests compare the constant d_r with per-lane limits
            const int kb0 = k0 + kb * 32 + 8 * hf;
            const int lim_n = N - kb0, lim_c = qrow - kb0, lim_w = qrow - kb0 - window, lim_s = sinks - kb0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(__builtin_fmaf(sacc[r], scale_log2, -lse2));
                if constexpr (MASK) {
                    const int dr = 16 * (r >> 3) + (r & 7);
                    if (dr >= lim_n || (CAUSAL && (dr > lim_c || (WIN && dr <= lim_w && dr >= lim_s))))
                        p = 0.f;
                }
                if constexpr (DROP) {
                    const bool kept = drop.keep(dw[r >> 2], r & 3);
                    dp[r] = kept ? dp[r] * drop.scale : 0.f;
                }
                sacc[r] = DNEG ? p * dp[r] : p * (dp[r] - Dq);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u32x4 dsf;
#pragma unroll
                for (int w = 0; w < 4; ++w) dsf[w] = pack_bf16x2(sacc[8 * t + 2 * w], sacc[8 * t + 2 * w + 1]);
                const int tb = t_off + (kb * 32 + 16 * t) * STR;
                u32x4 kt4[D / 32];
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    kt4[db] = lds_read_tr16_x2(k_lds + tb + db * 32, k_lds + tb + db * 32 + T2);
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db) dqacc[db] = mfma32x32x16(kt4[db], dsf, dqacc[db]);
            }
        }
    };

    // Key tiles in a sequence of positions p (as in the forward): under a
    // window first the nsk tiles of sink keys below the window, then tiles
    // tlo .. ntiles-1; masked, unmasked, masked phases.  Position p lives in
    // buffer p % 2.
    int nsk = 0, tlo = 0, tfull = 0;
    if constexpr (WIN) {
        const int q1 = min(q0 + BR, N) - 1;
        const int lo_min = q0 - window + 1, lo_max = q1 - window + 1;
        tlo = max(lo_min, 0) / BC;
        tfull = max(tlo, (max(lo_max, 0) + BC - 1) / BC);
        nsk = min((sinks + BC - 1) / BC, tlo);
    }
    // Block-sparse: the workgroup's active key tiles in LDS.
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
        nact = build_tile_list<4>(active, ntiles, s_list, s_bal, s_off, wave, lane, tid);
    }
    auto tile_at = [&](int p) {
        if constexpr (BLK) return (int)s_list[min(p, max(nact - 1, 0))];
        return p < nsk ? p : tlo + (p - nsk);
    };
    // tiles in [tfull, tdiag) precede every query of the workgroup, lie
    // inside every row's window and hold no key past N: no mask
    const int jsplit = min(ntiles, CAUSAL ? q0 / BC : N / BC);
    const int tdiag = max(tfull, jsplit);
    int p1 = nsk + (tfull - tlo), p2 = nsk + (tdiag - tlo), p3 = nsk + (ntiles - tlo);
    if constexpr (BLK) p1 = p2 = 0, p3 = nact;   // every listed tile masked
    if (p3 > 0) {
        cp.issue(krs, tile_at(0) * BC, sK0, wave);
        cp.issue(vrs, tile_at(0) * BC, sV0, wave);
    }
    wait_vmem();
    __syncthreads();
    auto tile_b = [&](int p, auto bufc, auto maskc) __attribute__((always_inline)) {   // position p lives in buffer bufc
        constexpr bool B1 = decltype(bufc)::value != 0;
        if (p + 1 < p3) {
            const int k1 = tile_at(p + 1) * BC;
            cp.issue(krs, k1, B1 ? sK0 : sK1, wave);
            cp.issue(vrs, k1, B1 ? sV0 : sV1, wave);
        }
        const int k0 = tile_at(p) * BC;
        if constexpr (decltype(maskc)::value != 0) {
            const bool sees = !(CAUSAL && k0 > qw + 31) &&
                              !(WIN && k0 + BC - 1 < qw - window + 1 && k0 >= sinks) &&
                              !(BLK && !block_bit(k0) && !block_bit(k0 + 32));
            if (sees) compute(bufc, k0, maskc);
        } else {
            compute(bufc, k0, maskc);
        }
        wait_vmem();
        __syncthreads();
    };
    // Positions [pb, pe), position p in buffer p % 2 (buffers fixed at compile time).
    auto phase = [&](int pb, int pe, auto maskc) __attribute__((always_inline)) {
        int p = pb;
        if (p < pe && (p & 1)) { tile_b(p, ic<1>{}, maskc); ++p; }
        for (; p + 1 < pe; p += 2) {
            tile_b(p, ic<0>{}, maskc);
            tile_b(p + 1, ic<1>{}, maskc);
        }
        if (p < pe) tile_b(p, ic<0>{}, maskc);
    };
    phase(0, p1, ic<1>{});
    phase(p1, p2, ic<0>{});
    phase(p2, p3, ic<1>{});

    // Epilogue through LDS (stage_piece / store_rows); the K staging buffers
    // are free: every tile ended with a barrier and no copy is in flight.
    {
        uint16_t* const tile = (wave < BC / 32 ? sK0 : sK1) + (wave % (BC / 32)) * 32 * STR;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16& a = dqacc[db];
                stage_piece(tile, STR, ln, db * 32 + 8 * g + 4 * hf, a[4 * g] * tau, a[4 * g + 1] * tau,
                            a[4 * g + 2] * tau, a[4 * g + 3] * tau);
            }
        store_rows<D>(tile, STR, dQ + base + (size_t)qw * D, N - qw, lane);
    }
}

template <int D, int MODE, bool DROP>
void launch(const BwdArgs& a, int stages, hipStream_t st) {
    const int bh = a.B * a.H;
    Dropout drop;
    drop.seed_lo = (uint32_t)a.seed;
    drop.seed_hi = (uint32_t)(a.seed >> 32);
    drop.offset = a.offset;
    drop.thr = a.drop_thr;
    drop.scale = a.drop_thr > 0 ? 256.f / (256.f - (float)a.drop_thr) : 1.f;
    // stage bit 0: dQ, which also writes D; bit 1: dK and dV, which read D
    if (stages & 1) {
        const int nq = (a.N + 127) / 128;
        hipLaunchKernelGGL((bwd_dq_kernel<D, MODE, DROP>), dim3(nq * bh), dim3(256), 0, st,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, (const uint16_t*)a.o, a.lse, a.D,
                           (uint16_t*)a.dq, bh, a.N, a.tau * kLog2e, a.tau, nq, a.window, a.sinks,
                           drop, a.blk);
    }
    if (stages & 2) {
        const int nk = (a.N + kBlkKeys - 1) / kBlkKeys;
        BlkSplit split;
        int helpers = 0;
        if constexpr (MODE >= kMaskBlock) {
            if (a.split.plan) {   // plan the parts, then helpers first in the grid
                split = a.split;
                helpers = split.slots;
                int dev = 0, cus = 0;
                if (hipGetDevice(&dev) != hipSuccess ||
                    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                    cus < 1)
                    cus = 256;
                split.conc = 2 * cus;   // two dK/dV workgroups per CU
                const int n_items = nk * bh;
                constexpr bool CAUSAL = MODE == kMaskBlockCausal;
                hipLaunchKernelGGL((blk_count_kernel<64, CAUSAL>), dim3((n_items + 3) / 4), dim3(256), 0,
                                   st, a.blk, bh, a.N, n_items, split.plan);
                hipLaunchKernelGGL(blk_plan_kernel, dim3(1), dim3(1024), 0, st, split.plan, split.meta,
                                   n_items, split.slots, split.conc);
            }
        }
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MODE, DROP>), dim3(helpers + nk * bh), dim3(256), 0, st,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, a.lse, a.D, (uint16_t*)a.dk, (uint16_t*)a.dv,
                           bh, a.N, a.tau * kLog2e, a.tau, a.window, a.sinks, drop, a.blk, split);
    }
}

template <int D>
void launch_d(const BwdArgs& a, int stages, hipStream_t st) {
    if (a.blk.mask) {       // block-sparse (no window, no dropout)
        a.causal ? launch<D, kMaskBlockCausal, false>(a, stages, st)
                 : launch<D, kMaskBlock, false>(a, stages, st);
    } else if (a.drop_thr > 0) {   // dropout: with no mask or the plain causal mask
        a.causal ? launch<D, kMaskCausal, true>(a, stages, st)
                 : launch<D, kMaskNone, true>(a, stages, st);
    } else if (!a.causal) {
        launch<D, kMaskNone, false>(a, stages, st);
    } else if (a.window < a.N || a.sinks > 0) {
        launch<D, kMaskWindow, false>(a, stages, st);
    } else {
        launch<D, kMaskCausal, false>(a, stages, st);
    }
}

}  // namespace

void launch_bwd(const BwdArgs& a, int stages, hipStream_t st) {
    if (a.dtype == kF32) {
        launch_bwd_f32(a, stages, st);
        return;
    }
    a.d == 64 ? launch_d<64>(a, stages, st) : launch_d<128>(a, stages, st);
}

}  // namespace fa
