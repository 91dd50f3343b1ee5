/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The library computes exact attention O = softmax(tau * Q K^T [+ causal mask]) V
 * without ever writing the N x N score matrix to HBM: Q is tiled, K/V tiles are
 * staged on chip, and the softmax is carried through the key blocks with a
 * running row maximum m and row sum l that rescale the partial output whenever
 * a block is merged ("flash-attention" encyclopedia page, sections "a ideia"
 * and "como funciona").  The forward saves only O and the per-row
 * log-sum-exp, and the backward recomputes S and P from them (same page,
 * backward paragraph of "como funciona").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors   : device pointers to contiguous row-major [B, H, N, d] arrays, d
 *             fastest, 16-byte aligned.  The caller owns every buffer; the
 *             library allocates nothing and keeps no global state.
 * dtype     : FA_BF16 (bfloat16) or FA_F32 (IEEE float).  O, dQ, dK and dV
 *             take the input dtype; LSE and D are always float.
 * Arithmetic: products are accumulated in fp32 (bf16 MFMA with fp32
 *             accumulation for FA_BF16; fp32 throughout for FA_F32).  The
 *             probabilities P are rounded to bf16 before the P V product on the
 *             FA_BF16 path.
 * tau       : the scale applied to Q K^T before the softmax (typically
 *             1/sqrt(d)); must be finite and > 0.
 * causal    : 0 or 1.  When 1, key j is visible to query i iff j <= i
 *             (diagonal included; as many queries as keys).
 * LSE       : natural-log log-sum-exp of each row of the tau-scaled scores,
 *             LSE_i = m_i + ln(l_i), float [B, H, N].
 * stream    : a hipStream_t (NULL = the default stream).  Every call only
 *             validates on the host and enqueues kernels; it returns before
 *             the work finishes.
 * Errors    : every entry point returns an fa_status.  Arguments are checked
 *             on the host before anything is launched; a failed check launches
 *             nothing and writes nothing.  FA_ERR_HIP reports a launch error
 *             (hipGetLastError after the launches).  Nothing is thrown across
 *             the ABI.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,         /* a required pointer is NULL                     */
    FA_ERR_SHAPE = 2,        /* B, H, N, d or a length out of range            */
    FA_ERR_UNSUPPORTED = 3,  /* dtype, head dim or flag value not supported    */
    FA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required        */
    FA_ERR_HIP = 5,          /* the HIP runtime reported a launch error        */
    FA_ERR_ALIGN = 6,        /* a pointer is not 16-byte aligned               */
    FA_ERR_ARG = 7,          /* a value out of range: tau, split count, window,
                                sinks, stage, dropout probability, block size   */
    FA_ERR_SCRATCH = 8       /* fa_decode_noalloc: the call needs more than the
                                library's fixed scratch array                   */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/* Supported head dimensions: 64 and 128.  Sizes: B, H, N >= 1 and
 * B*H <= 2^31-1, N <= 2^20 (FA_ERR_SHAPE otherwise). */

/*
 * fa_fwd - fused exact-attention forward (prefill).
 *
 * Defined by the standard statement S = tau Q K^T, P = softmax(S), O = P V
 * ("flash-attention" page, sections "o problema" and "como funciona"), computed
 * tile by tile with the running (m, l) statistics so that S and P never leave
 * the chip ("FlashAttention e o gargalo real de inferência", section
 * "FlashAttention: eliminar a viagem").
 *
 * q, k, v : [B, H, N, d] inputs of dtype `dtype`.
 * o       : [B, H, N, d] output, dtype `dtype`.
 * lse     : [B, H, N] float output (the statistic the backward needs).
 * Fully masked causal tiles are never visited.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float tau, int causal, int dtype, void* stream);

/*
 * fa_fwd_window - fa_fwd under the causal mask restricted to a sliding window
 * with sink tokens.
 *
 * Local layers of hybrid attention attend to a window of recent tokens only
 * ("Atenção eficiente — FlashAttention, sparse e híbrida", section "Atenção
 * híbrida: local + global intercalados"), and StreamingLLM keeps the first
 * few tokens visible besides the window (same page, "Attention sinks — o
 * paradoxo do primeiro token").  Key j is visible to query i iff j <= i and
 * (i - j < window or j < sinks).  Tiles outside every row's window are never
 * visited.  window >= N with sinks = 0 is exactly fa_fwd with causal = 1.
 *
 * window : >= 1 (the query's own key always counts); sinks: >= 0 (FA_ERR_ARG
 *          otherwise).  Other arguments as fa_fwd; LSE is over the visible keys.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float tau, int window, int sinks,
                  int dtype, void* stream);

/*
 * fa_fwd_dropout - fa_fwd with dropout on the attention probabilities.
 *
 * Standard attention applies dropout to P as one of its memory-bound steps
 * ("flash-attention" page, "o problema"); the fused kernel applies it on chip
 * and the backward regenerates the mask from the generator state instead of
 * storing it (same page, "como funciona", backward paragraph).  After the
 * softmax each P_ij is kept with probability 1 - p and scaled by 1/(1 - p),
 * else zeroed; LSE is that of the undropped scores.  The mask is a pure
 * function of (seed, offset, b, h, i, j): one Philox4x32-10 call (Salmon et
 * al., "Parallel random numbers: as easy as 1, 2, 3", SC11) per 4 x 4 block of
 * (query, key) pairs with counter (j/4, i/4, b*H + h, offset) and key = seed
 * (low word first); the pair is kept iff byte j%4 of output word i%4 is
 * >= round(256 p).  p is therefore used as a multiple of 1/256.
 *
 * p_drop : 0 <= p_drop and round(256 p_drop) <= 255 (FA_ERR_ARG otherwise);
 *          p_drop = 0 is exactly fa_fwd.
 * seed, offset : the generator state; fa_bwd_dropout must get the same.
 * Other arguments as fa_fwd (causal 0 or 1; no sliding window).
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float tau, int causal, float p_drop,
                   unsigned long long seed, unsigned int offset, int dtype, void* stream);

/*
 * fa_fwd_block_sparse - block-sparse attention forward.
 *
 * The pages' answer to sequences too long for exact attention is the
 * block-sparse variant of the fused kernel, an approximation ("flash-attention"
 * page, "o que isso custou"): a mask over (query block, key block) pairs
 * switches whole blocks of the score matrix off, and tiles that hold no set
 * block are never loaded.  Key j is visible to query i only if
 * block_mask[head][i / block_q][j / block_k] != 0 (and j <= i when causal).
 * A row with no visible key gets the empty sum: O = 0, LSE = -inf.
 *
 * block_mask : device uint8 [mask_heads, ceil(N/block_q), ceil(N/block_k)],
 *              shared by all batch entries; mask_heads = 1 (one mask for all
 *              heads) or H (head h uses block_mask[h]).
 * block_q, block_k : powers of two in [32, 1024] (FA_ERR_ARG otherwise).
 * N <= 262144 (FA_ERR_SHAPE otherwise); bf16 only.  Other arguments as fa_fwd.
 */
int fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, float tau, int causal,
                        const unsigned char* block_mask, int mask_heads, int block_q,
                        int block_k, int dtype, void* stream);

/*
 * fa_decode_workspace_bytes - workspace that fa_decode needs.
 *
 * num_splits = 0 asks for the size of the split count that fa_decode chooses
 * by itself for these sizes; otherwise the size for that explicit count.
 * Returns 0 for arguments fa_decode would reject.
 */
size_t fa_decode_workspace_bytes(int B, int H, int N_max, int d, int num_splits);

/*
 * fa_decode_num_splits - the split count fa_decode uses for these sizes
 * (num_splits = 0 picks it from B*H and N_max; otherwise returns num_splits).
 */
int fa_decode_num_splits(int B, int H, int N_max, int d, int num_splits);

/*
 * fa_decode - one query per sequence against a KV cache, split over the keys.
 *
 * The decode step is a single query row reading the whole KV cache from HBM
 * ("Atenção eficiente — FlashAttention, sparse e híbrida", section
 * "FlashAttention não acelera o decode").  Each (b, h) key range [0, L_b) is cut
 * into num_splits contiguous chunks of equal length (the last ones may be
 * short or empty); each chunk yields its normalised partial output o_s and its
 * lse_s in the workspace, and a merge kernel combines them with the block-merge
 * rule of the running (m, l) statistics ("flash-attention" page, "como
 * funciona"): LSE = ln sum_s exp(lse_s), O = sum_s exp(lse_s - LSE) o_s.
 * With a single split that partial is the result: the split kernel stores O
 * and LSE itself (the same values the merge would store) and no merge runs.
 * The automatic count is one split when N_max <= 1024.
 *
 * q         : [B, H, 1, d] queries (the newest token of each sequence).
 * k, v      : [B, H, N_max, d] caches; rows at and beyond L_b are never read.
 * seqlens_k : device int32 [B], L_b.  Values are clamped to [0, N_max] on the
 *             device; a sequence with L_b = 0 yields O = 0 and LSE = -inf.
 * o         : [B, H, 1, d] output (dtype `dtype`); lse: [B, H] float output.
 * num_splits: 0 = automatic, else 1..1024.
 * workspace : device memory of at least fa_decode_workspace_bytes(...) bytes,
 *             16-byte aligned; its contents on entry do not matter.
 * No mask: all L_b keys are visible to the decode query.
 */
int fa_decode(const void* q, const void* k, const void* v, const int* seqlens_k,
              int B, int H, int N_max, int d, float tau, void* o, float* lse,
              int num_splits, void* workspace, size_t workspace_bytes,
              int dtype, void* stream);

/*
 * fa_decode_noalloc - fa_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, split count and results as fa_decode, but
 * the split partials live in a fixed array the library holds on each GPU
 * (FA_DECODE_NOALLOC_SCRATCH_BYTES, allocated with the library's code object
 * and kept until the process ends) instead of a workspace argument.
 *
 * Arguments as for fa_decode, without the workspace.  The call allocates
 * nothing; its first call on a device looks up that device's array address.
 * It returns FA_ERR_SCRATCH (launching nothing) when
 * fa_decode_workspace_bytes(B, H, N_max, d, num_splits) exceeds
 * FA_DECODE_NOALLOC_SCRATCH_BYTES; one split (automatic for N_max <= 1024)
 * uses no partials at all.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  Nothing in the array needs clearing: each
 * call writes every partial it reads.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_noalloc(const void* q, const void* k, const void* v, const int* seqlens_k,
                      int B, int H, int N_max, int d, float tau, void* o, float* lse,
                      int num_splits, int dtype, void* stream);

/*
 * fa_decode_paged_num_splits / fa_decode_paged_workspace_bytes - the split
 * count fa_decode_paged uses (num_splits = 0: chosen from B, Hkv, the head
 * groups and page_size * max_pages; otherwise num_splits) and the workspace
 * it needs, 4 * splits * B * Hq * (d + 1) bytes.  Both return 0 for sizes
 * fa_decode_paged would reject.
 */
int fa_decode_paged_num_splits(int B, int Hq, int Hkv, int page_size, int max_pages, int d,
                               int num_splits);
size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int page_size, int max_pages,
                                       int d, int num_splits);

/*
 * fa_decode_paged - decode with grouped KV heads over a paged KV cache.
 *
 * Decode reads the whole KV cache once per generated token ("Atenção
 * eficiente — FlashAttention, sparse e híbrida", section "FlashAttention não
 * acelera o decode token a token"); sharing each KV head among several query
 * heads (MQA, GQA: the page's "Veja também" list) shrinks that cache, and
 * Paged Attention keeps it in fixed-size pages located through a per-sequence
 * table (table of section "Sparse e híbrida").  Per (b, h) the result is
 * exactly fa_decode's: one query against keys [0, L_b), split over the keys
 * and merged by LSE.
 *
 * q           : [B, Hq, 1, d] bfloat16.
 * k_pages,
 * v_pages     : [num_pages, Hkv, page_size, d] bfloat16.  Query head h uses
 *               KV head h / (Hq / Hkv); Hq must be a multiple of Hkv (Hkv = Hq
 *               is multi-head, Hkv = 1 multi-query attention).
 * block_table : device int32 [B, max_pages]: key t of sequence b is row
 *               t % page_size of page block_table[b][t / page_size].  Entries
 *               past the sequence's last page are never read; a page id
 *               outside [0, num_pages) is clamped into that range (the reads
 *               stay inside the cache; the result for that sequence is then
 *               meaningless).
 * seqlens_k   : device int32 [B], L_b, clamped on the device to
 *               [0, page_size * max_pages]; L_b = 0 yields O = 0, LSE = -inf.
 *               Rows of a page at or beyond L_b are never read.
 * page_size   : a power of two in [16, 65536]; page_size * max_pages <= 2^20.
 * o           : [B, Hq, 1, d] bfloat16 output; lse: [B, Hq] float output.
 * num_splits  : 0 = automatic, else 1..1024 (chunks are multiples of 128 keys).
 * workspace   : >= fa_decode_paged_workspace_bytes(...) bytes, 16-byte aligned.
 * dtype       : FA_BF16 only (FA_ERR_UNSUPPORTED otherwise).
 */
int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                    const int* block_table, const int* seqlens_k, int B, int Hq, int Hkv,
                    int num_pages, int page_size, int max_pages, int d, float tau, void* o,
                    float* lse, int num_splits, void* workspace, size_t workspace_bytes,
                    int dtype, void* stream);

/*
 * fa_bwd_workspace_bytes - workspace of fa_bwd: D, B*H*N floats.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_bwd - recomputing backward of fa_fwd.
 *
 * Uses only O and LSE saved by the forward ("flash-attention" page, "como
 * funciona", backward paragraph).  Two kernels: one per query tile that first
 * forms D_i = dO_i . O_i for its rows (the page's identity D_i = P_i . dP_i =
 * dO_i . O_i, an inner product of length d), writes it to the workspace and
 * accumulates dQ = tau dS K with dS = P o (dO V^T - D); then one per key tile
 * that recomputes S = tau Q K^T and P = exp(S - LSE) on chip and accumulates
 * dV = P^T dO and dK = tau dS^T Q, reading D.  No atomics: the result is
 * deterministic.
 *
 * q, k, v, o, dout : [B, H, N, d], dtype `dtype`; o is fa_fwd's output.
 * lse              : [B, H, N] float, fa_fwd's output.
 * dq, dk, dv       : [B, H, N, d] outputs, dtype `dtype`.
 * workspace        : >= fa_bwd_workspace_bytes(B, H, N) bytes; on return it
 *                    holds D as float [B, H, N].
 * dtype            : FA_BF16 (bf16 MFMA products, fp32 accumulation) or FA_F32
 *                    (float vector arithmetic throughout, for tight checks;
 *                    not a performance path).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float tau, int causal,
           void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_bwd_window - backward of fa_fwd_window (causal mask with a sliding
 * window of `window` keys and `sinks` sink keys; same visibility rule).
 * Query tiles no key of a tile can reach, and key tiles outside every row's
 * window, are skipped.  Arguments as fa_bwd without `causal`, plus window >= 1
 * and sinks >= 0 (FA_ERR_ARG otherwise); o and lse must come from
 * fa_fwd_window with the same window and sinks.
 */
int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv,
                  int B, int H, int N, int d, float tau, int window, int sinks,
                  void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_bwd_dropout - backward of fa_fwd_dropout: regenerates the same mask from
 * (p_drop, seed, offset); with Z = keep / (1 - p): dV = (P o Z)^T dO,
 * dS = P o (Z o dP - D) and D_i = dO_i . O_i as before.  o and lse must come
 * from fa_fwd_dropout with the same arguments.  Arguments as fa_bwd plus the
 * dropout state.
 */
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float tau, int causal, float p_drop,
                   unsigned long long seed, unsigned int offset,
                   void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_bwd_block_sparse_workspace_bytes - workspace with which
 * fa_bwd_block_sparse splits long key-tile lists: D, a split plan and
 * clamp(items / 16, 32, 256) slots of 2 * 128 * d floats (items = B * H *
 * ceil(N / 128)).  0 for invalid sizes or d other than 64 and 128.  A larger
 * workspace gives more slots (at most 4096).
 */
size_t fa_bwd_block_sparse_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd_block_sparse - backward of fa_fwd_block_sparse (same mask and block
 * sizes; o and lse from that forward).  Query and key tiles holding no set
 * block are skipped; rows with no visible key receive zero gradient.
 * Arguments as fa_bwd plus the block mask.
 *
 * The dK/dV pass walks, for each 128-key tile, the list of query tiles that
 * hold a set block for it; under a mask with global key blocks one such list
 * can be far longer than the rest.  With a workspace of at least
 * fa_bwd_block_sparse_workspace_bytes (anything from D plus the plan plus two
 * slots on), the call first counts every list on the device, cuts lists
 * longer than a planned part into parts taken by extra workgroups, and the
 * last part of each list to finish adds the fp32 partials of all its parts in
 * part order (deterministic; lists beyond the slots are walked whole).  With
 * fa_bwd_workspace_bytes(B, H, N) bytes every list is walked whole by one
 * workgroup.  Calls that share a workspace must not overlap.
 */
int fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, float tau, int causal,
                        const unsigned char* block_mask, int mask_heads, int block_q,
                        int block_k, void* workspace, size_t workspace_bytes, int dtype,
                        void* stream);

/*
 * fa_bwd_stage - enqueue one of fa_bwd's two kernels.
 *
 * stage 0 computes dQ and writes D into the workspace, stage 1 dK and dV
 * (it reads D, so stage 0 must have run on the same inputs).  Enqueuing
 * stages 0, 1 in order on one stream is exactly fa_bwd.  Same arguments and
 * checks as fa_bwd, plus FA_ERR_ARG for a stage outside 0..1.  Meant for
 * per-kernel timing.
 */
int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, float tau, int causal,
                 void* workspace, size_t workspace_bytes, int dtype, void* stream);

/* fa_status_string - static, human-readable text of a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
