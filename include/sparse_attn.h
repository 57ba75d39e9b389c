/*
 * sparse_attn.h: C ABI of the MI355X (gfx950) top-k sparse attention library.
 *
 * The library computes two forms of the same attention:
 *   1. sparse_attn_fwd: each query token attends to K rows of a shared
 *      key/value cache picked by an index list (-1 = empty slot), with a
 *      per-head "sink" logit that takes part in the softmax normalisation only.
 *   2. topk_bitmask_build + masked_attn_fwd: the index lists scattered into a
 *      bit-packed mask, consumed by a dense attention that reads the mask
 *      words 4 at a time (one 16-byte load per 128 keys).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device memory on the current device;
 *    "host" pointers are ordinary CPU memory. bf16 data is passed as raw
 *    16-bit storage (the high half of an IEEE single). Every tensor is dense
 *    and row-major in the layout stated; the caller owns every buffer.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    on it; no entry point synchronises, allocates device memory or keeps
 *    state between calls.
 *  - All arguments are checked on the host before any HIP call; a rejected
 *    call returns a nonzero sa_status and touches no memory. Launch failures
 *    return SA_ERR_HIP; faults inside a kernel surface at the caller's next
 *    synchronisation.
 *  - Zero-sized work returns SA_OK without launching anything.
 *  - Outputs must not alias inputs.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,       /* a size is negative or sizes are inconsistent */
  SA_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  SA_ERR_UNSUPPORTED = 4, /* a head dimension / head count the library has no kernel for */
  SA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  SA_ERR_HIP = 6          /* a HIP call (launch) failed */
} sa_status;

/* Static, human-readable name of a status code. Never NULL. */
const char* sa_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Top-k sparse attention.                                                   */
/* Operation ("DeepSeek V4 源码剖析", ch. 5, sections 5.1-5.2, 5.4-5.5):     */
/*   for every batch b, token s, head h, with V = { k : 0 <= idx[b,s,k] < T }  */
/*   (duplicates counted; -1 or any index outside [0, T) is an empty slot):    */
/*     x_k  = scale * dot(q[b,s,h,:], kv[b, idx[b,s,k], :])                    */
/*     w    = softmax over { x_k : k in V } plus one extra logit sink[h]       */
/*     o[b,s,h,:] = sum_{k in V} w_k * kv[b, idx[b,s,k], :]   (sink has no row) */
/*   The same kv row serves as key and value (one shared row for all heads).   */
/*   sink[h] = +inf gives o = 0; -inf means no sink; NaN gives a NaN row;      */
/*   no valid slot and sink -inf gives o = 0.                                  */
/*   Arithmetic: bf16 products, fp32 accumulation, fp32 softmax; the softmax   */
/*   weights are rounded to bf16 before the weighted row sum; o is rounded to  */
/*   bf16 (nearest even). When a token's slots are split over workgroups, each */
/*   split's unnormalised weighted row sum (its weights relative to its own    */
/*   reference maximum) is rounded to bf16 once before the merge.             */
/* ------------------------------------------------------------------------ */

/*
 * Bytes of device workspace sparse_attn_fwd needs for this shape and split
 * count (num_splits = 0 picks the library's choice, as sparse_attn_fwd does).
 * Returns 0 when no workspace is needed, and also for invalid sizes.
 */
size_t sparse_attn_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K, int num_splits);

/*
 * The split count sparse_attn_fwd uses for num_splits = 0 (each token's K
 * slots are cut into this many contiguous ranges processed by separate
 * workgroups and merged afterwards), per token and head group (see
 * sparse_attn_head_groups: the count applies to the B*S*groups pairs). It
 * never gives more than 256 workgroups (one per CU) in all, at most K's
 * 32-slot tile count and 16, and within that the count that balances each
 * workgroup's tile loop against the partials written and merged (a cost
 * fitted to measured decode calls). Returns 1 for invalid sizes.
 */
int sparse_attn_num_splits(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K);

/*
 * The number of head groups sparse_attn_fwd (fp8 = 0) or sparse_attn_fp8_fwd
 * (fp8 = 1) cuts each token's heads into: 1, or 2 (groups of H / 2 heads, each
 * processed by its own workgroups like a token of H / 2 heads) at D = 512 with
 * 64 or more heads (a multiple of 32) when B*S <= 32, and for bf16 rows also
 * when two groups keep at least 2 splits and as many workgroups as one. The
 * split count of sparse_attn_num_splits is per token and head group. Returns 1
 * for invalid sizes. Pure host function (no HIP call).
 */
int sparse_attn_head_groups(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K, int fp8);

/*
 * The split count sparse_attn_fp8_fwd uses for num_splits = 0 (D = 512; per
 * token and head group, as sparse_attn_num_splits for bf16 rows). Returns 1
 * for invalid sizes.
 */
int sparse_attn_fp8_num_splits(int64_t B, int64_t S, int64_t H, int64_t K);

/*
 * q          device, bf16 [B][S][H][D]
 * kv         device, bf16 [B][T][D]
 * attn_sink  device, fp32 [H]
 * topk_idxs  device, int32 [B][S][K]
 * out        device, bf16 [B][S][H][D] (written in full)
 * scale      the softmax scale (the pages use D^-0.5)
 * num_splits 0 = library choice, else 1..64 (clamped to K's tile count)
 * workspace  device, >= sparse_attn_workspace_bytes(...) bytes, 256-byte
 *            aligned; may be NULL when that size is 0. Scratch for the split
 *            partials: contents on entry do not matter, on return they are
 *            unspecified. Calls that may run at the same time need separate
 *            workspaces.
 * Supported: D in {64, 512}; 1 <= H <= 128. q, kv, out 16-byte aligned.
 * Sizes: B*S <= 2^30, T < 2^31, K <= 2^30, and B*S times the split count
 * below 2^31; larger sizes return SA_ERR_SHAPE.
 */
int sparse_attn_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* out,
                    int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same operation, arguments, checks and results as sparse_attn_fwd with
 * num_splits resolved the same way, but without a workspace argument. The
 * split partials live in a device array inside the library: 40 MiB per GPU,
 * held from when the library is loaded until the process ends. A call whose
 * sparse_attn_workspace_bytes(...) exceeds 40 MiB returns SA_ERR_WORKSPACE
 * before any HIP call. Every call on one GPU shares that array, which keeps
 * the last call's contents: calls that may overlap on one GPU (other streams
 * or threads) race and give wrong results. The array's device address is
 * looked up once per GPU, on that GPU's first call; the call allocates
 * nothing.
 */
int sparse_attn_fwd_noalloc(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs,
                            void* out, int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale,
                            int num_splits, void* stream);

/*
 * The two phases of sparse_attn_fwd, for callers that schedule them apart (to
 * overlap the merge with other work) or time them: sparse_attn_split_fwd runs
 * the attention over each token's split slot ranges and leaves, per split,
 * the unnormalised weighted row sum O_p (bf16), its reference maximum m_p
 * (log2 units) and weight sum l_p in the workspace; sparse_attn_merge_fwd
 * merges them into `out`, adding the sink once (the identity
 * o = sum_p 2^(m_p - M) O_p / (sum_p 2^(m_p - M) l_p + 2^(sink log2 e - M)),
 * M the largest exponent).
 * When the split count resolves to 1, sparse_attn_split_fwd writes `out` in full
 * and sparse_attn_merge_fwd does nothing. Both take exactly sparse_attn_fwd's
 * arguments and checks; call them in this order on one stream with the same
 * arguments and workspace. Merge identity: "DeepSeek V4 源码剖析", ch. 5,
 * section 5.5 (FlashMLA's split combine with the sink).
 */
int sparse_attn_split_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* out,
                          int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);
int sparse_attn_merge_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* out,
                          int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_attn_fwd over FP8 rows (D = 512): the MODEL1 row of FlashMLA (DeepSeek V4
 * source notes, ch. 5, section 5.7): 584 bytes per row of kv8 [B][T][584]:
 *   bytes 0..447    e4m3 (OCP FP8 E4M3) values of dims 0..447,
 *   bytes 448..575  bf16 (little-endian) dims 448..511 (the RoPE part, used as is),
 *   bytes 576..582  one scale byte s per 64-dim tile of dims 0..447, byte 583 unused;
 *   dim d < 448 is e4m3(byte d) * 2^(s[d / 64] - 127).
 * The page prints the layout but not the scale byte's encoding; the unsigned
 * power-of-two (UE8M0) reading above is this library's. Rows are dequantized to
 * bf16 inside the kernel (exact for scale bytes in [15, 239], where every scaled
 * e4m3 value is a normal bf16) and the call is otherwise sparse_attn_fwd with
 * D = 512: same q, attn_sink, topk_idxs, out, scale, num_splits and workspace
 * (size it with sparse_attn_workspace_bytes(B, S, H, 512, K, num_splits)).
 * Requires kv8 8-byte aligned and T * 584 < 2^31.
 */
int sparse_attn_fp8_fwd(const void* q, const void* kv8, const float* attn_sink, const int32_t* topk_idxs, void* out,
                        int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, float scale, int num_splits,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two phases of sparse_attn_fp8_fwd, as sparse_attn_split_fwd and
 * sparse_attn_merge_fwd are of sparse_attn_fwd: the split phase leaves the same
 * partials (O_p, m_p, l_p) in the workspace, and the merge phase combines them
 * into `out` with the sink added once ("DeepSeek V4 源码剖析", ch. 5, section
 * 5.5). Both take exactly sparse_attn_fp8_fwd's arguments and checks; call them
 * in this order on one stream with the same arguments and workspace. When the
 * split count resolves to 1, the split phase writes `out` in full and the merge
 * phase does nothing.
 */
int sparse_attn_fp8_split_fwd(const void* q, const void* kv8, const float* attn_sink, const int32_t* topk_idxs,
                              void* out, int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, float scale,
                              int num_splits, void* workspace, size_t workspace_bytes, void* stream);
int sparse_attn_fp8_merge_fwd(const void* q, const void* kv8, const float* attn_sink, const int32_t* topk_idxs,
                              void* out, int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, float scale,
                              int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Bit-packed top-k mask.                                                    */
/* Shape rule and row layout: prhub summary of vLLM PR #52217, key source    */
/* (_topk_mask_shape, _build_topk_mask) and its tests; bit order: prhub      */
/* summary of vLLM PR #48770, key source (dense_mask_mod: word j >> 5,       */
/* bit j & 31, least significant bit first).                                 */
/* ------------------------------------------------------------------------ */

/*
 * Host-only. Writes {B, padded_q, words} to out_shape (host, 3 entries):
 *   padded_q = max_q_len rounded up to 128 when max_q_len <= 128, else to 256;
 *   words    = ceil(max_key_len / 32) + (reserve_key_start_word ? 1 : 0),
 *              rounded up to a multiple of 4 (rows are whole 16-byte chunks).
 */
int topk_bitmask_shape(int64_t B, int64_t max_q_len, int64_t max_key_len, int reserve_key_start_word,
                       int64_t* out_shape);

/*
 * topk_idxs  device, int32 [B][Q][topk]
 * q_lens     device, int32 [B] or NULL (NULL: all Q rows of every batch are live)
 * key_starts device, int32 [B] or NULL; when given, words must hold the reserved
 *            word: words >= ceil(key_len / 32) + 1
 * mask       device, uint32 [B][padded_q][words], written in FULL (no pre-zeroing):
 *              bit (j & 31) of mask[b][q][j >> 5] is set iff q < q_len[b] and
 *              some slot of topk_idxs[b][q] equals j with 0 <= j < key_len;
 *              mask[b][0][words-1] = key_starts[b] when key_starts is given;
 *              every other word is 0.
 * Requires padded_q >= Q, words % 4 == 0, 32 * words >= key_len, mask 16-byte aligned;
 * words <= 32768 (else SA_ERR_UNSUPPORTED); B * padded_q < 2^31, topk < 2^31 and
 * B * Q * topk <= 2^40 (else SA_ERR_SHAPE).
 */
int topk_bitmask_build(const int32_t* topk_idxs, const int32_t* q_lens, const int32_t* key_starts, uint32_t* mask,
                       int64_t B, int64_t Q, int64_t topk, int64_t key_len, int64_t padded_q, int64_t words,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Masked dense attention (the masked-MHA form).                             */
/* prhub summary of vLLM PR #48770 (masked MHA emulating sparse attention    */
/* for short prefills; dense_mask_mod) and of vLLM PR #52217 (mask words     */
/* loaded 4 at a time, bitwise-identical results).                           */
/*   for b, query q, head h, with J = { j < KV : mask == NULL or bit j of     */
/*   mask[b][q] is set } (one mask row shared by all heads, no sink):         */
/*     o[b,q,h,:] = sum_{j in J} softmax_j(scale * q[b,q,h,:].k[b,j,h,:]) v[b,j,h,:] */
/*   J empty gives o = 0.                                                     */
/* ------------------------------------------------------------------------ */

/*
 * q     device, bf16 [B][Q][H][Dqk]
 * k     device, bf16 [B][KV][H][Dqk]
 * v     device, bf16 [B][KV][H][Dv]
 * mask  device, uint32 [B][padded_q][words] or NULL (NULL: every key visible)
 * out   device, bf16 [B][Q][H][Dv] (written in full)
 * mask_load_bits  128: the mask is read as aligned 16-byte chunks (4 words per
 *                 128 keys); 32: one 32-bit word per 32 keys (control variant).
 *                 Both give bitwise-identical outputs.
 * Supported: (Dqk, Dv) = (192, 128), H <= 4096 (else SA_ERR_UNSUPPORTED).
 * Requires padded_q >= Q, words % 4 == 0, words <= 2^21, 32 * words >= KV,
 * KV <= 2^30, Q < 2^31 (else SA_ERR_SHAPE); q, k, v, mask, out 16-byte aligned.
 */
int masked_attn_fwd(const void* q, const void* k, const void* v, const uint32_t* mask, void* out,
                    int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv, int64_t padded_q,
                    int64_t words, float scale, int mask_load_bits, void* stream);

/*
 * Chunked-context form (prhub summary of vLLM PR #48770, key source:
 * offset_dense_mask_mod). k and v hold one chunk of KV keys of a longer
 * context; chunk key j is key p = key_start[b] + j of the mask rows, where
 * key_start[b] = mask[b][0][words-1] (the reserved word that
 * topk_bitmask_build writes from key_starts), read as unsigned 32-bit:
 *   J = { j < KV : p < 32 * (words - 1) and bit (p & 31) of mask[b][q][p >> 5] }
 * Positions at or past the reserved word are never visible, so a start past
 * every bit word gives o = 0. Otherwise as masked_attn_fwd: same arguments
 * (no mask_load_bits: the words of a chunk tile sit at any bit offset and are
 * read 4 bytes at a time), same layouts, no sink, o = 0 for an empty J.
 * lse        device fp32 [B][Q][H], or NULL: the natural-log log-sum-exp of
 *            each query's scaled logits over J (-inf for an empty J), so that
 *            the outputs of the chunks of one context can be merged:
 *            o = sum_c exp(lse_c - LSE) o_c, LSE = log sum_c exp(lse_c) (the
 *            fallback from one global mask to per-chunk masks, prhub summary of
 *            vLLM PR #48770, review discussion). 4-byte aligned.
 * Requires mask != NULL (when B*Q*H > 0), words >= 4, words % 4 == 0,
 * padded_q >= Q; KV is not limited by words. Returns SA_ERR_NULL without a mask.
 * The size limits of masked_attn_fwd apply (H <= 4096, words <= 2^21, ...).
 */
int masked_attn_offset_fwd(const void* q, const void* k, const void* v, const uint32_t* mask, void* out, float* lse,
                           int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv, int64_t padded_q,
                           int64_t words, float scale, void* stream);

/* ------------------------------------------------------------------------ */
/* Candidate mask of the indexer's decode logits.                           */
/* prhub summary of vLLM PR #56628 (ROCm DSA decode: the candidate mask      */
/* strides only up to each row's live end; the mask rule and the tests'      */
/* contract: agreement on [0, end), columns past it untouched, the launch     */
/* grid fixed by the shapes so graph replay follows changing ends).          */
/* ------------------------------------------------------------------------ */

/*
 * logits  device float32; element (r, c) at logits[r * stride_row + c * stride_col]
 *         (0 <= r < rows, 0 <= c < width), modified in place.
 * starts  device int32 or NULL (NULL: every start is 0); row r uses
 *         starts[(r / row_repeat) * stride_start].
 * ends    device int32; row r uses e = ends[(r / row_repeat) * stride_end].
 * flags   device uint8 [rows][nblocks + 1], nblocks = ceil(width / block_size):
 *         flags[r][b] != 0 keeps block b of row r, the columns
 *         start + b * block_size ... start + (b + 1) * block_size - 1;
 *         flags[r][nblocks] != 0 (the edge flag) keeps column width - 1.
 *         How the flags are derived from candidate blocks is not printed on
 *         the page; they are an input here.
 * For each row, a column c with start <= c < e is live; a live column keeps
 * its value iff its block flag is set (a block index outside [0, nblocks)
 * keeps nothing) or c == width - 1 and the edge flag is set. Every other
 * column c < min(e, width) becomes -inf. Columns c >= e are NOT written (the
 * whole-row form would set them to -inf too; no consumer reads them), so the
 * cost follows the live length, not the workspace width. e <= 0 writes nothing.
 * Launch: candidate_mask_grid(rows, width) workgroups, a function of the shapes
 * only, so a captured graph replays correctly with new starts / ends / flags.
 * Requires block_size >= 1, row_repeat >= 1, stride_col >= 1, other strides
 * >= 0, width < 2^31 - 4096; logits, starts, ends 4-byte aligned; ends (and
 * starts) hold ceil(rows / row_repeat) entries.
 */
int candidate_mask_apply(float* logits, const int32_t* starts, const int32_t* ends, const uint8_t* flags,
                         int64_t rows, int64_t width, int64_t stride_row, int64_t stride_col, int64_t stride_start,
                         int64_t stride_end, int64_t block_size, int64_t row_repeat, void* stream);

/* Host-only: the number of workgroups candidate_mask_apply launches (0 for no work). */
int candidate_mask_grid(int64_t rows, int64_t width);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
