// fa_internal.h - argument bundles and launcher declarations shared by the
// C-ABI layer (fa_api.cpp) and the kernel translation units.  Launchers assume
// arguments were validated by the ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

enum { kF32 = 0, kBF16 = 1 };

// Largest number of key (or query) tiles a block-sparse workgroup lists in LDS.
constexpr int kMaxSparseTiles = 4096;

// Block-sparse attention: key j is visible to query i only if
// mask[head][i >> lgbq][j >> lgbk] != 0 (head = h when heads == H, else 0).
struct BlockSparse {
    const unsigned char* mask = nullptr;   // [heads, nbq, nbk] uint8
    int nbq = 0, nbk = 0, lgbq = 0, lgbk = 0, heads = 0, H = 1;
};

// Block-sparse backward: a key tile whose list of active query tiles is long
// is walked in parts by several dK/dV workgroups (its owner and helpers).
// Each part writes fp32 partial dK and dV to a slot, and the last part to
// finish adds the slots in part order and stores dK and dV.  The workspace
// holds, after D: the plan, four ints per (key tile, head) item (helpers,
// first helper, first slot, arrivals; the count pass leaves the list length
// in the first), 64 ints of totals (helpers in use), then the slots.
struct BlkSplit {
    int* plan = nullptr;     // nullptr: no splitting, every owner walks its whole list
    int* meta = nullptr;
    float* pool = nullptr;   // [slots][2 (dK, dV)][128 * d] in the workgroup's register layout
    int slots = 0;
    int conc = 0;            // dK/dV workgroups resident at once (sizes the parts; set at launch)
};
constexpr int kBlkKeys = 128;   // keys per dK/dV workgroup
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
inline size_t blk_split_items(int B, int H, int N) {
    return (size_t)B * H * ((N + kBlkKeys - 1) / kBlkKeys);
}
inline size_t blk_split_fixed_bytes(int B, int H, int N) {   // D, plan, totals
    return align256((size_t)B * H * N * sizeof(float)) +
           align256(blk_split_items(B, H, N) * 4 * sizeof(int)) + 256;
}
inline size_t blk_split_slot_bytes(int d) { return (size_t)2 * kBlkKeys * d * sizeof(float); }
constexpr int kBlkMaxSlots = 4096;
constexpr int kBlkMinPart = 4;   // smallest planned part (query tiles): shorter lists are never split

struct FwdArgs {
    const void *q, *k, *v;
    void* o;
    float* lse;
    int B, H, N, d;
    float tau;
    int causal, dtype;
    int window = 0x40000000;   // causal only: key j visible to query i iff j <= i and
    int sinks = 0;             // (i - j < window or j < sinks); the defaults give plain causal
    int drop_thr = 0;          // dropout: byte threshold round(256 p); 0 = no dropout
    unsigned long long seed = 0;
    unsigned int offset = 0;
    BlockSparse blk;           // block-sparse when blk.mask != nullptr
};
void launch_fwd(const FwdArgs& a, hipStream_t st);
void launch_fwd_f32(const FwdArgs& a, hipStream_t st);   // dtype kF32 (no block mask)

struct DecodeArgs {
    const void *q, *k, *v;
    const int* seqlens;
    int B, H, N_max, d;
    float tau;
    void* o;
    float* lse;
    int num_splits;       // resolved (>= 1)
    int chunk;            // keys per split: ceil(N_max / num_splits) rounded up to 64
    float* ws_o;          // [num_splits, B, H, d] normalised partial outputs
    float* ws_lse;        // [num_splits, B, H] partial LSE (-inf for empty splits)
    int dtype;
};
void launch_decode(const DecodeArgs& a, hipStream_t st);
// Host checks of a decode call (every argument except the workspace, in the
// order fa_decode documents); on FA_OK fills *a without workspace pointers and
// *ws_bytes with the workspace the call needs.  Touches no device memory.
int decode_prepare(const void* q, const void* k, const void* v, const int* seqlens_k, int B, int H,
                   int N_max, int d, float tau, void* o, float* lse, int num_splits, int dtype,
                   DecodeArgs* a, size_t* ws_bytes);
// Points the partial outputs and partial LSEs of *a into a workspace of at
// least decode_ws_bytes bytes: [S, B, H, d] floats, then [S, B, H] floats.
void decode_set_workspace(DecodeArgs* a, void* ws);
int decode_splits(int B, int H, int N_max, int d, int requested);
int decode_chunk(int N_max, int splits);
size_t decode_ws_bytes(int B, int H, int d, int splits);

struct PagedDecodeArgs {
    const void *q, *k_pages, *v_pages;
    const int* block_table;   // [B, max_pages] page ids
    const int* seqlens;       // [B]
    int B, Hq, Hkv, num_pages, page_size, max_pages, d;
    float tau;
    void* o;
    float* lse;
    int num_splits;           // resolved (>= 1)
    int chunk;                // keys per split, a multiple of 128
    float* ws_o;              // [num_splits, B, Hq, d]
    float* ws_lse;            // [num_splits, B, Hq]
};
void launch_decode_paged(const PagedDecodeArgs& a, hipStream_t st);
int decode_paged_splits(int B, int Hq, int Hkv, int max_keys, int requested);
int decode_paged_chunk(int max_keys, int splits);

struct BwdArgs {
    const void *q, *k, *v, *o;
    const float* lse;
    const void* dout;
    void *dq, *dk, *dv;
    float* D;             // [B, H, N] workspace
    int B, H, N, d;
    float tau;
    int causal, dtype;
    int window = 0x40000000;   // as in FwdArgs
    int sinks = 0;
    int drop_thr = 0;
    unsigned long long seed = 0;
    unsigned int offset = 0;
    BlockSparse blk;
    BlkSplit split;       // block-sparse only
};
// stages: bit 0 = dQ (which also writes D), bit 1 = dK/dV (reads D); launched in that order
void launch_bwd(const BwdArgs& a, int stages, hipStream_t st);
void launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t st);   // dtype kF32 (no block mask)

}  // namespace fa
