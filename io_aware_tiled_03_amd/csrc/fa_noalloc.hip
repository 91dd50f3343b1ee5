// fa_noalloc.hip - fa_decode_noalloc: split-KV decode whose partial results
// live in a fixed array in device memory instead of a caller-supplied
// workspace, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below is allocated with the library's code object on
// each GPU the library runs on and kept until the process ends.  Its name is
// only a host-side stand-in for the symbol: host code never passes it to a
// kernel or a copy.  On the first call on a device (with that device current)
// the device address is looked up once with hipGetSymbolAddress and cached
// per device; every later use goes through that cached pointer.  Calls that
// overlap on one GPU share the array and race: a caller issues them on one
// stream, or orders them.  The split kernel writes every partial the merge
// reads in the same call (empty splits write 0 and -inf), so nothing has to
// start at zero and the previous call's contents are never read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

static_assert(FA_DECODE_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");

// The partial outputs and LSEs of fa_decode_noalloc ([S, B, H, d] floats, then
// [S, B, H] floats), at most FA_DECODE_NOALLOC_SCRATCH_BYTES bytes.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per
// device); FA_OK or the status to report.
int scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return FA_OK;
}

}  // namespace

extern "C" int fa_decode_noalloc(const void* q, const void* k, const void* v, const int* seqlens_k,
                                 int B, int H, int N_max, int d, float tau, void* o, float* lse,
                                 int num_splits, int dtype, void* stream) {
    fa::DecodeArgs a;
    size_t need = 0;
    int st = fa::decode_prepare(q, k, v, seqlens_k, B, H, N_max, d, tau, o, lse, num_splits, dtype,
                                &a, &need);
    if (st != FA_OK) return st;
    if (need > (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_ptr(&ws);
    if (st != FA_OK) return st;
    fa::decode_set_workspace(&a, ws);
    (void)hipGetLastError();
    fa::launch_decode(a, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
