/*
 * fa_calib.h - measurement aid exported by libfa.so beside the attention
 * entry points of fa.h: synthetic matrix-core loops that give the rate this
 * part reaches for a given mix of work per bf16 product.
 *
 * The attention kernels are rated against the nominal dense bf16 peak
 * (2.5 PFLOP/s at 2.4 GHz).  What a kernel can reach is lower: the clock the
 * part holds under a busy matrix pipe, the LDS bandwidth that feeds one
 * operand of every product, and the vector instructions (exp2, fp32
 * arithmetic) issued between products all take their share.  Each mix below
 * runs one such combination with nothing else in the loop, so its rate is
 * measured on the same part, under the same clock behaviour, as the kernel it
 * is compared with.  A second set runs the kernels' LDS read patterns alone,
 * which is how their row layouts were chosen, and a third streams a buffer from
 * HBM, the ceiling of the decode kernels.  None of this is part of the
 * attention path.
 *
 * Conventions follow fa.h (fa_status results, device pointers, stream).
 */
#ifndef FA_CALIB_H
#define FA_CALIB_H

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

#define FA_CALIB_MAX_GRID 65536
#define FA_CALIB_MAX_ITERS (1 << 24)

/* Number of mixes fa_calib_mfma runs (mix ids 0 .. count-1). */
int fa_calib_mix_count(void);

/* A static description of mix `mix`, or NULL when the id is out of range. */
const char* fa_calib_mix_name(int mix);

/* Floating-point operations of the bf16 products in one
 * fa_calib_mfma(mix, grid, iters, ...) launch (2 * 32 * 32 * 16 per product);
 * 0 for an invalid mix, grid < 1 or iters < 2. */
double fa_calib_flops(int mix, int grid, int iters);

/* Enqueues one launch of mix `mix` on `stream`: `grid` workgroups of four
 * waves, each wave running `iters` steps.
 * seed : device pointer, 16-byte aligned, to at least 65536 bytes of operand
 *        data (any bf16 values; read only).
 * out  : device pointer, 16-byte aligned, to grid * 256 floats (one per lane,
 *        a checksum that keeps the loop's results live; overwritten).
 * grid in [1, FA_CALIB_MAX_GRID], iters even and in [2, FA_CALIB_MAX_ITERS]
 * (FA_ERR_ARG otherwise, also for an unknown mix); FA_ERR_NULL, FA_ERR_ALIGN
 * for bad pointers; FA_ERR_HIP for a launch error. */
fa_status fa_calib_mfma(int mix, int grid, int iters, const void* seed, float* out, void* stream);

/* LDS read patterns of the kernels' operand reads, each run alone (eight waves
 * per workgroup, 64-row tiles): row reads (ds_read_b128 in the kernels' row
 * order) and transposing reads (ds_read_b64_tr_b16) at several row strides, with
 * and without the backward kernels' row permutation.  Count and descriptions: */
int fa_calib_lds_count(void);
const char* fa_calib_lds_name(int pattern);   /* NULL when out of range */

/* LDS bytes that one fa_calib_lds(pattern, grid, iters, ...) launch reads; 0 for
 * an invalid pattern, grid < 1 or iters < 1. */
double fa_calib_lds_bytes(int pattern, int grid, int iters);

/* Enqueues one launch of LDS read pattern `pattern`: `grid` workgroups of eight
 * waves, `iters` steps of eight reads per wave.
 * out : device pointer, 16-byte aligned, to grid * 512 unsigned ints (a
 *       checksum per lane; overwritten).
 * grid in [1, FA_CALIB_MAX_GRID], iters in [1, FA_CALIB_MAX_ITERS] (FA_ERR_ARG
 * otherwise, also for an unknown pattern); FA_ERR_NULL, FA_ERR_ALIGN for a bad
 * pointer; FA_ERR_HIP for a launch error. */
fa_status fa_calib_lds(int pattern, int grid, int iters, unsigned int* out, void* stream);

/* Enqueues one streaming read of `bytes` bytes at `buf` (non-temporal 16-byte
 * loads, the load form of the decode kernels; `grid` workgroups of 256 lanes,
 * each on its own contiguous share of the buffer): the HBM read rate the part
 * reaches with nothing else in the loop.
 * buf  : device pointer, 16-byte aligned, `bytes` readable bytes (read only).
 * out  : device pointer, 16-byte aligned, to grid * 256 unsigned ints (a
 *        checksum per lane; overwritten).
 * bytes a positive multiple of 16, grid in [1, FA_CALIB_MAX_GRID] (FA_ERR_ARG
 * otherwise); FA_ERR_NULL, FA_ERR_ALIGN for a bad pointer; FA_ERR_HIP for a
 * launch error. */
fa_status fa_calib_hbm_read(const void* buf, size_t bytes, int grid, unsigned int* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_CALIB_H */
