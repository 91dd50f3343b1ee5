// fa_api.cpp - the extern "C" entry points of libfa.so (declared in fa.h).
// Validates every argument on the host, resolves the launch configuration and
// enqueues the kernels on the caller's stream.  Nothing here allocates or
// touches device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int check_common(int B, int H, int N, int d, float tau, int dtype) {
    if (B < 1 || H < 1 || N < 1 || N > (1 << 20)) return FA_ERR_SHAPE;
    if ((long long)B * H > 0x7fffffffLL) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!(tau > 0.f) || !isfinite(tau)) return FA_ERR_ARG;
    return FA_OK;
}

// Workgroups of the largest grid a call launches must stay addressable.
bool grid_ok(long long blocks, int threads) {
    return blocks >= 1 && blocks * threads < (1LL << 32) && blocks < 0x7fffffffLL;
}

int after_launch() {
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

namespace fa {

int decode_prepare(const void* q, const void* k, const void* v, const int* seqlens_k, int B, int H,
                   int N_max, int d, float tau, void* o, float* lse, int num_splits, int dtype,
                   DecodeArgs* a, size_t* ws_bytes) {
    if (!q || !k || !v || !seqlens_k || !o || !lse) return FA_ERR_NULL;
    int st = check_common(B, H, N_max, d, tau, dtype);
    if (st != FA_OK) return st;
    if (num_splits < 0 || num_splits > 1024) return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) ||
        !aligned4(seqlens_k))
        return FA_ERR_ALIGN;
    const int S = decode_splits(B, H, N_max, d, num_splits);
    if (!grid_ok((long long)S * B * H, 256)) return FA_ERR_SHAPE;
    *a = DecodeArgs{q, k, v, seqlens_k, B, H, N_max, d, tau, o, lse, S,
                    decode_chunk(N_max, S), nullptr, nullptr, dtype};
    *ws_bytes = decode_ws_bytes(B, H, d, S);
    return FA_OK;
}

void decode_set_workspace(DecodeArgs* a, void* ws) {
    float* w = static_cast<float*>(ws);
    a->ws_o = w;
    a->ws_lse = w + (size_t)a->num_splits * a->B * a->H * a->d;
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float tau, int causal, int dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    int st = check_common(B, H, N, d, tau, dtype);
    if (st != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
        return FA_ERR_ALIGN;
    const long long bh = (long long)B * H;
    if (!grid_ok(bh * ((N + 63) / 64), 256)) return FA_ERR_SHAPE;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, tau, causal, dtype};
    (void)hipGetLastError();
    fa::launch_fwd(a, (hipStream_t)stream);
    return after_launch();
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, int d, float tau, int window, int sinks, int dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    int st = check_common(B, H, N, d, tau, dtype);
    if (st != FA_OK) return st;
    if (window < 1 || sinks < 0) return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
        return FA_ERR_ALIGN;
    const long long bh = (long long)B * H;
    if (!grid_ok(bh * ((N + 63) / 64), 256)) return FA_ERR_SHAPE;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, tau, 1, dtype};
    a.window = window < N ? window : N;   // a window of N or more keys is the causal mask
    a.sinks = sinks < N ? sinks : N;
    (void)hipGetLastError();
    fa::launch_fwd(a, (hipStream_t)stream);
    return after_launch();
}

// Byte threshold round(256 p) of a dropout probability; -1 if out of range.
static int drop_threshold(float p) {
    if (!(p >= 0.f) || !(p < 1.f)) return -1;
    const int t = (int)lrintf(p * 256.f);
    return t <= 255 ? t : -1;
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, float tau, int causal, float p_drop, unsigned long long seed,
                   unsigned int offset, int dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    int st = check_common(B, H, N, d, tau, dtype);
    if (st != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    const int thr = drop_threshold(p_drop);
    if (thr < 0) return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
        return FA_ERR_ALIGN;
    const long long bh = (long long)B * H;
    if (!grid_ok(bh * ((N + 63) / 64), 256)) return FA_ERR_SHAPE;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, tau, causal, dtype};
    a.drop_thr = thr;
    a.seed = seed;
    a.offset = offset;
    (void)hipGetLastError();
    fa::launch_fwd(a, (hipStream_t)stream);
    return after_launch();
}

// Block-sparse arguments: fills bs or returns the status to report.
static int block_sparse_args(const unsigned char* mask, int mask_heads, int block_q, int block_k,
                             int H, int N, fa::BlockSparse* bs) {
    if (!mask) return FA_ERR_NULL;
    auto pow2 = [](int x) { return x >= 32 && x <= 1024 && (x & (x - 1)) == 0; };
    if (!pow2(block_q) || !pow2(block_k)) return FA_ERR_ARG;
    if (mask_heads != 1 && mask_heads != H) return FA_ERR_SHAPE;
    if (N > 64 * fa::kMaxSparseTiles) return FA_ERR_SHAPE;   // tile lists live in LDS
    bs->mask = mask;
    bs->nbq = (N + block_q - 1) / block_q;
    bs->nbk = (N + block_k - 1) / block_k;
    bs->lgbq = __builtin_ctz((unsigned)block_q);
    bs->lgbk = __builtin_ctz((unsigned)block_k);
    bs->heads = mask_heads;
    bs->H = H;
    return FA_OK;
}

int fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int N, int d, float tau, int causal, const unsigned char* block_mask,
                        int mask_heads, int block_q, int block_k, int dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    int st = check_common(B, H, N, d, tau, dtype);
    if (st != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    fa::BlockSparse bs;
    st = block_sparse_args(block_mask, mask_heads, block_q, block_k, H, N, &bs);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
        return FA_ERR_ALIGN;
    const long long bh = (long long)B * H;
    if (!grid_ok(bh * ((N + 63) / 64), 256)) return FA_ERR_SHAPE;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, tau, causal, dtype};
    a.blk = bs;
    (void)hipGetLastError();
    fa::launch_fwd(a, (hipStream_t)stream);
    return after_launch();
}

int fa_decode_num_splits(int B, int H, int N_max, int d, int num_splits) {
    if (B < 1 || H < 1 || N_max < 1 || N_max > (1 << 20) || (d != 64 && d != 128)) return 0;
    if (num_splits < 0 || num_splits > 1024) return 0;
    return fa::decode_splits(B, H, N_max, d, num_splits);
}

size_t fa_decode_workspace_bytes(int B, int H, int N_max, int d, int num_splits) {
    const int s = fa_decode_num_splits(B, H, N_max, d, num_splits);
    if (s == 0) return 0;
    return fa::decode_ws_bytes(B, H, d, s);
}

int fa_decode(const void* q, const void* k, const void* v, const int* seqlens_k, int B, int H,
              int N_max, int d, float tau, void* o, float* lse, int num_splits, void* workspace,
              size_t workspace_bytes, int dtype, void* stream) {
    fa::DecodeArgs a;
    size_t need = 0;
    int st = fa::decode_prepare(q, k, v, seqlens_k, B, H, N_max, d, tau, o, lse, num_splits, dtype,
                                &a, &need);
    if (st != FA_OK) return st;
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    fa::decode_set_workspace(&a, workspace);
    (void)hipGetLastError();
    fa::launch_decode(a, (hipStream_t)stream);
    return after_launch();
}

// Paged cache sizes: returns FA_OK or the status fa_decode_paged reports.
static int check_paged(int B, int Hq, int Hkv, int page_size, int max_pages, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if ((long long)B * Hq > 0x7fffffffLL) return FA_ERR_SHAPE;
    if (page_size < 16 || page_size > 65536 || (page_size & (page_size - 1)) != 0) return FA_ERR_SHAPE;
    if (max_pages < 1 || (long long)page_size * max_pages > (1LL << 20)) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

int fa_decode_paged_num_splits(int B, int Hq, int Hkv, int page_size, int max_pages, int d,
                               int num_splits) {
    if (check_paged(B, Hq, Hkv, page_size, max_pages, d) != FA_OK) return 0;
    if (num_splits < 0 || num_splits > 1024) return 0;
    return fa::decode_paged_splits(B, Hq, Hkv, page_size * max_pages, num_splits);
}

size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int page_size, int max_pages, int d,
                                       int num_splits) {
    const int s = fa_decode_paged_num_splits(B, Hq, Hkv, page_size, max_pages, d, num_splits);
    if (s == 0) return 0;
    return fa::decode_ws_bytes(B, Hq, d, s);
}

int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                    const int* block_table, const int* seqlens_k, int B, int Hq, int Hkv,
                    int num_pages, int page_size, int max_pages, int d, float tau, void* o,
                    float* lse, int num_splits, void* workspace, size_t workspace_bytes,
                    int dtype, void* stream) {
    if (!q || !k_pages || !v_pages || !block_table || !seqlens_k || !o || !lse) return FA_ERR_NULL;
    int st = check_paged(B, Hq, Hkv, page_size, max_pages, d);
    if (st != FA_OK) return st;
    if (num_pages < 1) return FA_ERR_SHAPE;
    if ((double)num_pages * Hkv * page_size * d * 2.0 > 9.0e18) return FA_ERR_SHAPE;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!(tau > 0.f) || !isfinite(tau)) return FA_ERR_ARG;
    if (num_splits < 0 || num_splits > 1024) return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) ||
        !aligned4(lse) || !aligned4(block_table) || !aligned4(seqlens_k))
        return FA_ERR_ALIGN;
    const int max_keys = page_size * max_pages;
    const int S = fa::decode_paged_splits(B, Hq, Hkv, max_keys, num_splits);
    const size_t need = fa::decode_ws_bytes(B, Hq, d, S);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    const long long groups = (Hq / Hkv + 15) / 16;
    if (!grid_ok((long long)S * B * Hkv * groups, 256)) return FA_ERR_SHAPE;
    float* ws = (float*)workspace;
    const size_t n_o = (size_t)S * B * Hq * d;
    fa::PagedDecodeArgs a{q, k_pages, v_pages, block_table, seqlens_k, B, Hq, Hkv, num_pages,
                          page_size, max_pages, d, tau, o, lse, S,
                          fa::decode_paged_chunk(max_keys, S), ws, ws + n_o};
    (void)hipGetLastError();
    fa::launch_decode_paged(a, (hipStream_t)stream);
    return after_launch();
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1) return 0;
    return (size_t)B * H * N * sizeof(float);
}

namespace {

int bwd_common(int stages, const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int H,
               int N, int d, float tau, int causal, void* workspace, size_t workspace_bytes,
               int dtype, void* stream, int window = 0, int sinks = 0, int drop_thr = 0,
               unsigned long long seed = 0, unsigned int offset = 0,
               const fa::BlockSparse* bs = nullptr, bool split = false) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    int st = check_common(B, H, N, d, tau, dtype);
    if (st != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (bs && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;   // block-sparse: bf16 only
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
        return FA_ERR_ALIGN;
    if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, N)) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    if (!grid_ok((long long)B * H * ((N + 63) / 64), 256)) return FA_ERR_SHAPE;
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, (float*)workspace, B, H, N, d, tau, causal,
                  dtype};
    if (window > 0) {   // causal with a sliding window (a window of N or more is the causal mask)
        a.window = window < N ? window : N;
        a.sinks = sinks < N ? sinks : N;
    }
    a.drop_thr = drop_thr;
    a.seed = seed;
    a.offset = offset;
    if (bs) a.blk = *bs;
    if (bs && split) {   // room for the split plan and at least two slots: split long lists
        const size_t fixed = fa::blk_split_fixed_bytes(B, H, N), slot = fa::blk_split_slot_bytes(d);
        if (workspace_bytes >= fixed + 2 * slot) {
            char* const w = (char*)workspace;
            a.split.plan = (int*)(w + fa::align256((size_t)B * H * N * sizeof(float)));
            a.split.meta = (int*)(w + fixed - 256);
            a.split.pool = (float*)(w + fixed);
            const size_t n = (workspace_bytes - fixed) / slot;
            a.split.slots = (int)(n < (size_t)fa::kBlkMaxSlots ? n : fa::kBlkMaxSlots);
        }
    }
    (void)hipGetLastError();
    fa::launch_bwd(a, stages, (hipStream_t)stream);
    return after_launch();
}

}  // namespace

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, float tau,
           int causal, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
    return bwd_common(3, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, tau, causal, workspace,
                      workspace_bytes, dtype, stream);
}

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                  float tau, int window, int sinks, void* workspace, size_t workspace_bytes,
                  int dtype, void* stream) {
    if (window < 1 || sinks < 0) return FA_ERR_ARG;
    return bwd_common(3, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, tau, 1, workspace,
                      workspace_bytes, dtype, stream, window, sinks);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float tau, int causal, float p_drop, unsigned long long seed,
                   unsigned int offset, void* workspace, size_t workspace_bytes, int dtype,
                   void* stream) {
    const int thr = drop_threshold(p_drop);
    if (thr < 0) return FA_ERR_ARG;
    return bwd_common(3, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, tau, causal, workspace,
                      workspace_bytes, dtype, stream, 0, 0, thr, seed, offset);
}

int fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                        int H, int N, int d, float tau, int causal,
                        const unsigned char* block_mask, int mask_heads, int block_q, int block_k,
                        void* workspace, size_t workspace_bytes, int dtype, void* stream) {
    fa::BlockSparse bs;
    const int st = block_sparse_args(block_mask, mask_heads, block_q, block_k, H, N, &bs);
    if (st != FA_OK) return st;
    return bwd_common(3, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, tau, causal, workspace,
                      workspace_bytes, dtype, stream, 0, 0, 0, 0, 0, &bs, true);
}

size_t fa_bwd_block_sparse_workspace_bytes(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
    const size_t items = fa::blk_split_items(B, H, N);
    size_t slots = items / 16;   // every slot also launches one (possibly idle) helper workgroup
    slots = slots < 32 ? 32 : (slots > 256 ? 256 : slots);
    return fa::blk_split_fixed_bytes(B, H, N) + slots * fa::blk_split_slot_bytes(d);
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int H,
                 int N, int d, float tau, int causal, void* workspace, size_t workspace_bytes,
                 int dtype, void* stream) {
    if (stage < 0 || stage > 1) return FA_ERR_ARG;
    return bwd_common(1 << stage, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, tau, causal,
                      workspace, workspace_bytes, dtype, stream);
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "a size is out of range";
        case FA_ERR_UNSUPPORTED: return "unsupported dtype, head dimension or flag";
        case FA_ERR_WORKSPACE: return "workspace missing or too small";
        case FA_ERR_HIP: return "HIP launch error";
        case FA_ERR_ALIGN: return "a pointer is not aligned (16 bytes for tensors)";
        case FA_ERR_SCRATCH:
            return "the call needs more than the fixed scratch of fa_decode_noalloc "
                   "(FA_DECODE_NOALLOC_SCRATCH_BYTES)";
        case FA_ERR_ARG:
            return "bad argument value (tau finite and > 0, num_splits 0..1024, window >= 1, "
                   "sinks >= 0, stage 0..1, dropout probability in [0, 255/256], block sizes "
                   "powers of two in [32, 1024])";
        default: return "unknown status";
    }
}

}  // extern "C"
