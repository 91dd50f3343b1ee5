// fa_plan.cpp - host-side launch planning of the decode calls: how many key
// splits a call uses, how many keys each split covers and how much workspace
// the split partials need.  Plain C++ with no device code, so the same
// source builds into the library and into the host-only sanitizer check of
// the C ABI's argument validation.
#include <stddef.h>

#include "fa_internal.h"

namespace fa {

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
    // Automatic: one split when no sequence can hold more than 1024 keys
    // (such a decode is bound by launch and memory latency: the split kernel
    // then stores the result itself and the merge launch is saved, 9 us
    // instead of 11-12 us at 8x16x1024x64); otherwise the shortest chunk
    // (>= 256 keys) that keeps the grid at or below 16384 workgroups.
    if (N_max <= 1024) return 1;
    // bh * splits > 16384  <=>  splits > 16384 / bh (integer division; no
    // product that could overflow for huge B * H)
    const long long bh = (long long)B * H;
    int c = 256;
    while (c < N_max && (N_max + c - 1) / c > 16384 / bh) c *= 2;
    return (N_max + c - 1) / c;
}

size_t decode_ws_bytes(int B, int H, int d, int splits) {
    return (size_t)splits * B * H * (size_t)(d + 1) * sizeof(float);
}

int decode_paged_chunk(int max_keys, int splits) {
    const int c = (max_keys + splits - 1) / splits;
    return (c + 127) / 128 * 128;
}

int decode_paged_splits(int B, int Hq, int Hkv, int max_keys, int requested) {
    if (requested > 0) {
        const int c = decode_paged_chunk(max_keys, requested);
        return (max_keys + c - 1) / c;
    }
    // Automatic: the shortest chunk (>= 512 keys) that keeps the grid at or
    // below 4096 workgroups (each workgroup holds a whole CU's worth of LDS).
    const long long units = (long long)B * Hkv * ((Hq / Hkv + 15) / 16);
    int c = 512;
    while (c < max_keys && (max_keys + c - 1) / c > 4096 / units) c *= 2;
    c = decode_paged_chunk(max_keys, (max_keys + c - 1) / c);
    return (max_keys + c - 1) / c;
}

}  // namespace fa
