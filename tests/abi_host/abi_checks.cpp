// abi_checks.cpp - host-only check of the C ABI's argument validation and
// launch planning, built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_abi_sanitizer.py builds and runs it).
//
// It links the library's own host sources (fa_api.cpp, fa_plan.cpp) with stub
// launchers that record the arguments a call resolved instead of launching
// kernels, and a stub hipGetLastError.  Every entry point is called with
// valid arguments and with each kind of invalid one, including sizes near the
// int range; the sanitizers abort on any overflow or bad access in the
// checks, and the program exits non-zero if a status or a resolved launch
// argument differs from what fa.h documents.  No device memory exists here:
// the tensor pointers are fake aligned addresses that nothing dereferences.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "fa.h"
#include "fa_internal.h"

namespace {
int fails = 0, checks = 0;
int n_fwd = 0, n_dec = 0, n_paged = 0, n_bwd = 0;
fa::FwdArgs last_fwd{};
fa::DecodeArgs last_dec{};
fa::PagedDecodeArgs last_paged{};
fa::BwdArgs last_bwd{};
int last_stages = 0;
}  // namespace

namespace fa {
void launch_fwd(const FwdArgs& a, hipStream_t) { ++n_fwd; last_fwd = a; }
void launch_decode(const DecodeArgs& a, hipStream_t) { ++n_dec; last_dec = a; }
void launch_decode_paged(const PagedDecodeArgs& a, hipStream_t) { ++n_paged; last_paged = a; }
void launch_bwd(const BwdArgs& a, int stages, hipStream_t) {
    ++n_bwd;
    last_bwd = a;
    last_stages = stages;
}
}  // namespace fa

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

#define CHECK(cond)                                                          \
    do {                                                                     \
        ++checks;                                                            \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++fails;                                                         \
        }                                                                    \
    } while (0)

namespace {

void* const P = reinterpret_cast<void*>(uintptr_t{1} << 20);     // fake, 16-byte aligned
void* const P8 = reinterpret_cast<void*>((uintptr_t{1} << 20) + 8);
float* const L = static_cast<float*>(P);
const int* const I = static_cast<const int*>(P);
const unsigned char* const M = static_cast<const unsigned char*>(P);
const float kNaN = std::numeric_limits<float>::quiet_NaN();
const float kInf = std::numeric_limits<float>::infinity();

// A failing call returns `want` and launches nothing.
template <typename F>
void expect_reject(int want, F call, int line = __builtin_LINE()) {
    const int before = n_fwd + n_dec + n_paged + n_bwd;
    const int st = call();
    CHECK(st == want);
    CHECK(n_fwd + n_dec + n_paged + n_bwd == before);
    if (st != want) std::fprintf(stderr, "  line %d: status %d, expected %d\n", line, st, want);
}

int fwd(int B, int H, int N, int d, float tau, int causal, int dtype, const void* q = P,
        float* lse = L) {
    return fa_fwd(q, P, P, P, lse, B, H, N, d, tau, causal, dtype, nullptr);
}

void check_fwd() {
    expect_reject(FA_ERR_NULL, [] { return fwd(1, 1, 16, 64, 0.125f, 0, FA_BF16, nullptr); });
    expect_reject(FA_ERR_NULL, [] { return fwd(1, 1, 16, 64, 0.125f, 0, FA_BF16, P, nullptr); });
    expect_reject(FA_ERR_SHAPE, [] { return fwd(1, 1, 0, 64, 0.125f, 0, FA_BF16); });
    expect_reject(FA_ERR_SHAPE, [] { return fwd(-1, 1, 16, 64, 0.125f, 0, FA_BF16); });
    expect_reject(FA_ERR_SHAPE, [] { return fwd(1, 1, (1 << 20) + 1, 64, 0.125f, 0, FA_BF16); });
    expect_reject(FA_ERR_SHAPE, [] { return fwd(INT_MAX, INT_MAX, 16, 64, 0.125f, 0, FA_BF16); });
    expect_reject(FA_ERR_SHAPE, [] { return fwd(46341, 46341, 1 << 20, 128, 0.1f, 1, FA_BF16); });
    expect_reject(FA_ERR_SHAPE, [] { return fwd(INT_MAX, 1, 1 << 20, 64, 0.1f, 0, FA_BF16); });
    expect_reject(FA_ERR_UNSUPPORTED, [] { return fwd(1, 1, 16, 96, 0.125f, 0, FA_BF16); });
    expect_reject(FA_ERR_UNSUPPORTED, [] { return fwd(1, 1, 16, 64, 0.125f, 0, 7); });
    expect_reject(FA_ERR_UNSUPPORTED, [] { return fwd(1, 1, 16, 64, 0.125f, 2, FA_BF16); });
    for (float t : {0.f, -1.f, kNaN, kInf, -kInf})
        expect_reject(FA_ERR_ARG, [t] { return fwd(1, 1, 16, 64, t, 0, FA_BF16); });
    expect_reject(FA_ERR_ALIGN, [] { return fwd(1, 1, 16, 64, 0.125f, 0, FA_BF16, P8); });
    expect_reject(FA_ERR_ALIGN, [] {
        return fwd(1, 1, 16, 64, 0.125f, 0, FA_BF16, P, reinterpret_cast<float*>((uintptr_t)P + 2));
    });
    const int n0 = n_fwd;
    CHECK(fwd(3, 5, 1000, 128, 0.088f, 1, FA_BF16) == FA_OK);
    CHECK(n_fwd == n0 + 1);
    CHECK(last_fwd.B == 3 && last_fwd.H == 5 && last_fwd.N == 1000 && last_fwd.d == 128);
    CHECK(last_fwd.causal == 1 && last_fwd.dtype == FA_BF16 && last_fwd.drop_thr == 0);
    CHECK(last_fwd.blk.mask == nullptr && last_fwd.sinks == 0 && last_fwd.window >= (1 << 20));
    CHECK(fwd(1, 1, 1 << 20, 64, 0.125f, 0, FA_F32) == FA_OK);
}

void check_fwd_window() {
    auto win = [](int N, int w, int s) {
        return fa_fwd_window(P, P, P, P, L, 1, 2, N, 64, 0.125f, w, s, FA_BF16, nullptr);
    };
    expect_reject(FA_ERR_ARG, [&] { return win(16, 0, 0); });
    expect_reject(FA_ERR_ARG, [&] { return win(16, 4, -1); });
    expect_reject(FA_ERR_ARG, [&] { return win(16, INT_MIN, 0); });
    CHECK(win(100, 1000, 500) == FA_OK);
    CHECK(last_fwd.window == 100 && last_fwd.sinks == 100 && last_fwd.causal == 1);
    CHECK(win(100, 7, 3) == FA_OK);
    CHECK(last_fwd.window == 7 && last_fwd.sinks == 3);
    CHECK(win(100, INT_MAX, INT_MAX) == FA_OK);
    CHECK(last_fwd.window == 100 && last_fwd.sinks == 100);
}

void check_fwd_dropout() {
    auto drop = [](float p) {
        return fa_fwd_dropout(P, P, P, P, L, 1, 2, 64, 64, 0.125f, 0, p, ~0ULL, ~0U, FA_BF16,
                              nullptr);
    };
    for (float p : {-0.1f, 1.f, 0.999f, kNaN, kInf})
        expect_reject(FA_ERR_ARG, [&] { return drop(p); });
    CHECK(drop(0.1f) == FA_OK);
    CHECK(last_fwd.drop_thr == 26 && last_fwd.seed == ~0ULL && last_fwd.offset == ~0U);
    CHECK(drop(0.f) == FA_OK && last_fwd.drop_thr == 0);
    CHECK(drop(255.f / 256.f) == FA_OK && last_fwd.drop_thr == 255);
}

void check_block_sparse() {
    auto bs = [](const unsigned char* m, int heads, int bq, int bk, int N, int dtype) {
        return fa_fwd_block_sparse(P, P, P, P, L, 2, 3, N, 128, 0.1f, 1, m, heads, bq, bk, dtype,
                                   nullptr);
    };
    expect_reject(FA_ERR_NULL, [&] { return bs(nullptr, 1, 64, 64, 1000, FA_BF16); });
    for (int b : {0, 16, 48, 2048, INT_MIN})
        expect_reject(FA_ERR_ARG, [&] { return bs(M, 1, b, 64, 1000, FA_BF16); });
    expect_reject(FA_ERR_SHAPE, [&] { return bs(M, 2, 64, 64, 1000, FA_BF16); });
    expect_reject(FA_ERR_SHAPE, [&] { return bs(M, 1, 64, 64, 64 * 4096 + 1, FA_BF16); });
    expect_reject(FA_ERR_UNSUPPORTED, [&] { return bs(M, 1, 64, 64, 1000, FA_F32); });
    CHECK(bs(M, 3, 64, 256, 1000, FA_BF16) == FA_OK);
    CHECK(last_fwd.blk.mask == M && last_fwd.blk.nbq == 16 && last_fwd.blk.nbk == 4);
    CHECK(last_fwd.blk.lgbq == 6 && last_fwd.blk.lgbk == 8 && last_fwd.blk.heads == 3);
    const int n0 = n_bwd;
    CHECK(fa_bwd_block_sparse(P, P, P, P, L, P, P, P, P, 2, 3, 1000, 64, 0.125f, 0, M, 1, 32, 1024,
                              P, 2 * 3 * 1000 * 4, FA_BF16, nullptr) == FA_OK);
    CHECK(n_bwd == n0 + 1 && last_bwd.blk.nbq == 32 && last_bwd.blk.nbk == 1);
    CHECK(last_bwd.split.plan == nullptr && last_bwd.split.slots == 0);   // D only: no split
    // the split workspace: D, the plan (4 ints per 128-key tile and head), 256 bytes of totals,
    // then slots of 2 * 128 * d floats, here the default 32
    const size_t Dbytes = (size_t)2 * 3 * 1000 * 4, items = (size_t)2 * 3 * 8;
    const size_t fixed = (Dbytes + 255) / 256 * 256 + (items * 16 + 255) / 256 * 256 + 256;
    const size_t need = fa_bwd_block_sparse_workspace_bytes(2, 3, 1000, 64);
    CHECK(need == fixed + 32 * (size_t)2 * 128 * 64 * 4);
    CHECK(fa_bwd_block_sparse_workspace_bytes(2, 3, 1000, 96) == 0);
    CHECK(fa_bwd_block_sparse_workspace_bytes(0, 3, 1000, 64) == 0);
    char* const W = static_cast<char*>(P);
    CHECK(fa_bwd_block_sparse(P, P, P, P, L, P, P, P, P, 2, 3, 1000, 64, 0.125f, 0, M, 1, 32, 1024,
                              P, need, FA_BF16, nullptr) == FA_OK);
    CHECK(last_bwd.split.plan == reinterpret_cast<int*>(W + (Dbytes + 255) / 256 * 256));
    CHECK(last_bwd.split.meta == reinterpret_cast<int*>(W + fixed - 256));
    CHECK(last_bwd.split.pool == reinterpret_cast<float*>(W + fixed) && last_bwd.split.slots == 32);
    CHECK(fa_bwd_block_sparse(P, P, P, P, L, P, P, P, P, 2, 3, 1000, 64, 0.125f, 0, M, 1, 32, 1024,
                              P, fixed + 2 * 2 * 128 * 64 * 4 - 1, FA_BF16, nullptr) == FA_OK);
    CHECK(last_bwd.split.plan == nullptr);   // fewer than two slots: no split
    CHECK(fa_bwd_block_sparse(P, P, P, P, L, P, P, P, P, 2, 3, 1000, 64, 0.125f, 0, M, 1, 32, 1024,
                              P, fixed + (size_t)5000 * 2 * 128 * 64 * 4, FA_BF16, nullptr) == FA_OK);
    CHECK(last_bwd.split.slots == fa::kBlkMaxSlots);
    expect_reject(FA_ERR_UNSUPPORTED, [&] {
        return fa_bwd_block_sparse(P, P, P, P, L, P, P, P, P, 2, 3, 1000, 64, 0.125f, 0, M, 1, 32, 1024,
                                   P, 2 * 3 * 1000 * 4, FA_F32, nullptr);
    });
}

void check_decode() {
    CHECK(fa_decode_num_splits(0, 1, 16, 64, 0) == 0);
    CHECK(fa_decode_num_splits(1, 1, 16, 96, 0) == 0);
    CHECK(fa_decode_num_splits(1, 1, 16, 64, -1) == 0);
    CHECK(fa_decode_num_splits(1, 1, 16, 64, 1025) == 0);
    CHECK(fa_decode_workspace_bytes(1, 1, 0, 64, 0) == 0);
    CHECK(fa_decode_num_splits(64, 32, 8192, 128, 0) == 8);
    CHECK(fa_decode_num_splits(8, 16, 1024, 64, 0) == 1);
    CHECK(fa_decode_num_splits(INT_MAX, INT_MAX, 1 << 20, 128, 0) >= 1);
    const int B = 4, H = 3, Nm = 5000, d = 128;
    for (int req : {0, 1, 3, 7, 1024}) {
        const int S = fa_decode_num_splits(B, H, Nm, d, req);
        const size_t need = fa_decode_workspace_bytes(B, H, Nm, d, req);
        CHECK(S >= 1 && need == (size_t)S * B * H * (d + 1) * sizeof(float));
        auto call = [&](void* ws, size_t bytes) {
            return fa_decode(P, P, P, I, B, H, Nm, d, 0.1f, P, L, req, ws, bytes, FA_BF16, nullptr);
        };
        expect_reject(FA_ERR_WORKSPACE, [&] { return call(nullptr, need); });
        expect_reject(FA_ERR_WORKSPACE, [&] { return call(P, need - 1); });
        expect_reject(FA_ERR_ALIGN, [&] { return call(P8, need); });
        CHECK(call(P, need) == FA_OK);
        CHECK(last_dec.num_splits == S && (long long)last_dec.chunk * S >= Nm);
        CHECK((long long)last_dec.chunk * (S - 1) < Nm && last_dec.chunk % 64 == 0);
        CHECK(last_dec.ws_o == static_cast<float*>(P));
        CHECK(last_dec.ws_lse == static_cast<float*>(P) + (size_t)S * B * H * d);
    }
    expect_reject(FA_ERR_NULL, [] {
        return fa_decode(P, P, P, nullptr, 1, 1, 16, 64, 0.1f, P, L, 0, P, 1 << 20, FA_BF16, nullptr);
    });
    expect_reject(FA_ERR_ARG, [] {
        return fa_decode(P, P, P, I, 1, 1, 16, 64, 0.1f, P, L, -2, P, 1 << 20, FA_BF16, nullptr);
    });
    expect_reject(FA_ERR_ALIGN, [] {
        return fa_decode(P, P, P, reinterpret_cast<const int*>((uintptr_t)P + 2), 1, 1, 16, 64, 0.1f,
                         P, L, 0, P, 1 << 20, FA_BF16, nullptr);
    });
}

void check_decode_paged() {
    CHECK(fa_decode_paged_num_splits(1, 6, 4, 16, 8, 128, 0) == 0);     // Hq % Hkv
    CHECK(fa_decode_paged_num_splits(1, 8, 4, 8, 8, 128, 0) == 0);      // page_size < 16
    CHECK(fa_decode_paged_num_splits(1, 8, 4, 24, 8, 128, 0) == 0);     // not a power of two
    CHECK(fa_decode_paged_num_splits(1, 8, 4, 16, 65537, 128, 0) == 0); // > 2^20 keys
    CHECK(fa_decode_paged_num_splits(1, 8, 4, 65536, INT_MAX, 128, 0) == 0);
    CHECK(fa_decode_paged_workspace_bytes(1, 8, 4, 16, 8, 96, 0) == 0);
    const int B = 5, Hq = 32, Hkv = 8, ps = 16, mp = 512, d = 128;
    for (int req : {0, 1, 5, 64}) {
        const int S = fa_decode_paged_num_splits(B, Hq, Hkv, ps, mp, d, req);
        const size_t need = fa_decode_paged_workspace_bytes(B, Hq, Hkv, ps, mp, d, req);
        CHECK(S >= 1 && need == (size_t)S * B * Hq * (d + 1) * sizeof(float));
        auto call = [&](int num_pages, size_t bytes, int dtype) {
            return fa_decode_paged(P, P, P, I, I, B, Hq, Hkv, num_pages, ps, mp, d, 0.1f, P, L, req, P,
                                   bytes, dtype, nullptr);
        };
        expect_reject(FA_ERR_SHAPE, [&] { return call(0, need, FA_BF16); });
        expect_reject(FA_ERR_UNSUPPORTED, [&] { return call(100, need, FA_F32); });
        expect_reject(FA_ERR_WORKSPACE, [&] { return call(100, need - 1, FA_BF16); });
        CHECK(call(100, need, FA_BF16) == FA_OK);
        CHECK(last_paged.num_splits == S && last_paged.chunk % 128 == 0);
        CHECK((long long)last_paged.chunk * S >= (long long)ps * mp);
        CHECK(last_paged.ws_lse == static_cast<float*>(P) + (size_t)S * B * Hq * d);
    }
    // a cache of 2^71 bytes: page offsets would leave the 64-bit range
    expect_reject(FA_ERR_SHAPE, [] {
        return fa_decode_paged(P, P, P, I, I, 1, 65536, 65536, INT_MAX, 65536, 16, 128, 0.1f, P, L,
                               0, P, SIZE_MAX, FA_BF16, nullptr);
    });
    // 2^56 bytes is addressable: accepted (page offsets are 64-bit on the device)
    CHECK(fa_decode_paged(P, P, P, I, I, 1, 4, 2, INT_MAX, 65536, 16, 128, 0.1f, P, L, 0, P,
                          SIZE_MAX, FA_BF16, nullptr) == FA_OK);
}

void check_bwd() {
    const int B = 2, H = 3, N = 500, d = 64;
    const size_t ws = fa_bwd_workspace_bytes(B, H, N);
    CHECK(ws == (size_t)B * H * N * sizeof(float));
    CHECK(fa_bwd_workspace_bytes(0, 1, 1) == 0);
    CHECK(fa_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX) ==
          (size_t)INT_MAX * INT_MAX * INT_MAX * sizeof(float));
    auto bwd = [&](int causal, size_t bytes, int dtype, const void* dout = P) {
        return fa_bwd(P, P, P, P, L, dout, P, P, P, B, H, N, d, 0.125f, causal, P, bytes, dtype,
                      nullptr);
    };
    expect_reject(FA_ERR_NULL, [&] { return bwd(1, ws, FA_BF16, nullptr); });
    expect_reject(FA_ERR_WORKSPACE, [&] { return bwd(1, ws - 1, FA_BF16); });
    expect_reject(FA_ERR_UNSUPPORTED, [&] { return bwd(2, ws, FA_BF16); });
    expect_reject(FA_ERR_UNSUPPORTED, [&] { return bwd(1, ws, 9); });
    CHECK(bwd(0, ws, FA_F32) == FA_OK && last_bwd.dtype == FA_F32);
    CHECK(bwd(1, ws, FA_BF16) == FA_OK);
    CHECK(last_stages == 3 && last_bwd.D == static_cast<float*>(P) && last_bwd.causal == 1);
    for (int stage : {0, 1}) {
        CHECK(fa_bwd_stage(stage, P, P, P, P, L, P, P, P, P, B, H, N, d, 0.125f, 1, P, ws, FA_BF16,
                           nullptr) == FA_OK);
        CHECK(last_stages == (1 << stage));
    }
    for (int stage : {-1, 2, INT_MAX})
        expect_reject(FA_ERR_ARG, [&] {
            return fa_bwd_stage(stage, P, P, P, P, L, P, P, P, P, B, H, N, d, 0.125f, 1, P, ws,
                                FA_BF16, nullptr);
        });
    auto win = [&](int w, int s) {
        return fa_bwd_window(P, P, P, P, L, P, P, P, P, B, H, N, d, 0.125f, w, s, P, ws, FA_BF16,
                             nullptr);
    };
    expect_reject(FA_ERR_ARG, [&] { return win(0, 0); });
    expect_reject(FA_ERR_ARG, [&] { return win(10, -1); });
    CHECK(win(INT_MAX, INT_MAX) == FA_OK && last_bwd.window == N && last_bwd.sinks == N);
    CHECK(win(33, 2) == FA_OK && last_bwd.window == 33 && last_bwd.sinks == 2);
    auto drop = [&](float p) {
        return fa_bwd_dropout(P, P, P, P, L, P, P, P, P, B, H, N, d, 0.125f, 0, p, 5, 6, P, ws,
                              FA_BF16, nullptr);
    };
    expect_reject(FA_ERR_ARG, [&] { return drop(kNaN); });
    expect_reject(FA_ERR_ARG, [&] { return drop(1.5f); });
    CHECK(drop(0.5f) == FA_OK && last_bwd.drop_thr == 128 && last_bwd.seed == 5);
}

void check_status_strings() {
    for (int s = 0; s <= 7; ++s) CHECK(fa_status_string(s) != nullptr);
    CHECK(fa_status_string(-1) != nullptr && fa_status_string(INT_MAX) != nullptr);
}

}  // namespace

int main() {
    check_fwd();
    check_fwd_window();
    check_fwd_dropout();
    check_block_sparse();
    check_decode();
    check_decode_paged();
    check_bwd();
    check_status_strings();
    std::printf("%d checks, %d failed\n", checks, fails);
    return fails == 0 ? 0 : 1;
}
