// Host side of the C ABI declared in include/sparse_attn.h: argument checks (done before
// any HIP call, so a rejected call touches no memory), split and workspace policy, and
// dispatch to the kernel launchers.
#include <cmath>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sparse_attn.h"

extern "C" {
int sa_internal_launch_sparse(const void* q, const void* kv, const float* sink, const int32_t* idx, void* out,
                              int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale,
                              int nsplit, void* ws, int phases, int fp8, int G, void* stream);
int sa_internal_head_blocks(int64_t H);
size_t sa_internal_sparse_ws_bytes(int64_t ntok, int64_t H, int64_t D, int nsplit);
size_t sa_internal_scratch_bytes(void);
int sa_internal_scratch_ptr(void** out);
int sa_internal_launch_bitmask(const int32_t* idx, const int32_t* q_lens, const int32_t* key_starts, uint32_t* mask,
                               int64_t B, int64_t Q, int64_t topk, int64_t key_len, int64_t padded_q, int64_t words,
                               void* stream);
int64_t sa_internal_bitmask_max_words(void);
int sa_internal_launch_masked(const void* q, const void* k, const void* v, const uint32_t* mask, void* out,
                              float* lse, int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv,
                              int64_t padded_q, int64_t words, float scale, int mask_load_bits, int offset,
                              void* stream);
int sa_internal_candidate_gcols(int64_t rows, int64_t width);
int sa_internal_launch_candidate_mask(float* logits, const int32_t* starts, const int32_t* ends, const uint8_t* flags,
                                      int64_t rows, int64_t width, int64_t stride_row, int64_t stride_col,
                                      int64_t stride_start, int64_t stride_end, int64_t block_size, int64_t row_repeat,
                                      void* stream);
}

namespace {

constexpr int kTileRows = 32;   // slot tile of the sparse kernel
constexpr int kMaxSplits = 16;  // combine kernel limit
constexpr int64_t kTargetWorkgroups = 256;  // one per CU on MI355X
constexpr int64_t kInt32Max = ((int64_t)1 << 31) - 1;
// Masked attention: the kernel's per-tile byte offsets are 32-bit; with at most kMaskedMaxHeads
// heads and kMaskedMaxWords mask words they stay below 2^31 (64 key rows of H * 384 bytes; 256
// mask rows of 4 * words bytes).
constexpr int64_t kMaskedMaxHeads = 4096;
constexpr int64_t kMaskedMaxWords = (int64_t)1 << 21;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool sparse_sizes_ok(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K) {
  return B >= 0 && S >= 0 && H >= 0 && D >= 0 && K >= 0;
}

// The library's split count: at most one workgroup per CU in all (a second, partial wave of
// workgroups made decode calls 39-51 % slower), and within that the n that minimises a per-call
// cost fitted to decode-shaped calls (D = 512, H = 128; 8-256 tokens, K = 512, 1152 and 2048):
// t(n) ~ c + 1.30 us * tiles / n + 0.024 us * tokens * n + 0.36 us * n, i.e. the tile loop of one
// workgroup against the split partials written and merged. Its choice was within 2.9 % of the
// best measured split count at every one of those 24 shapes (filling every CU instead: up to 51 %).
int choose_splits(int64_t B, int64_t S, int64_t K, int requested) {
  const int64_t ntok = B * S;
  const int64_t tiles = cdiv(K, kTileRows);
  if (ntok <= 0 || tiles <= 0) return 1;
  int64_t n = requested;
  if (requested <= 0) {
    n = (int64_t)(std::sqrt(1.30 * (double)tiles / (0.024 * (double)ntok + 0.36)) + 0.5);
    const int64_t one_wave = kTargetWorkgroups / ntok;
    if (n > one_wave) n = one_wave;
  }
  if (n > kMaxSplits) n = kMaxSplits;
  if (n > tiles) n = tiles;
  if (n < 1) n = 1;
  return (int)n;
}

// Head groups: each token's H heads may be cut into G = 2 groups of H / 2, each processed like a
// token of its own (twice the workgroups, each with half the heads: half the query load and half the
// per-tile chain; a gathered row is then copied by both groups' workgroups). At D = 512 with 64 or
// more heads (a multiple of 32): with at most 32 tokens always (decode calls 10-19 % faster at 4-16
// tokens, 2-12 % at 24-32, FP8 rows 2-19 %), and for bf16 rows beyond that when two groups still get
// at least 2 splits and at least as many workgroups as one group (40 tokens 8 %, 64 tokens 2.4-3.5 %
// faster; 48 tokens, with fewer workgroups, 3 % slower, and 96, with one split, 14 % slower). FP8 rows
// beyond 32 tokens keep one group: each group expands every row it copies (48 and 64 tokens 15-28 %
// slower).
int head_groups(int64_t ntok, int64_t H, int64_t D, int64_t K, int fp8) {
  if (D != 512 || H < 64 || H % 32 != 0 || ntok <= 0) return 1;
  if (ntok <= 32) return 2;
  if (fp8) return 1;
  const int n1 = choose_splits(ntok, 1, K, 0), n2 = choose_splits(2 * ntok, 1, K, 0);
  return (n2 >= 2 && 2 * n2 >= n1) ? 2 : 1;
}

size_t sparse_ws_bytes(int64_t B, int64_t S, int64_t H, int64_t D, int G, int nsplit) {
  if (nsplit <= 1) return 0;
  return sa_internal_sparse_ws_bytes(B * S * G, H / G, D, nsplit);
}

// Workspace for a call of this shape, bf16 or FP8 rows alike (the larger of the two).
size_t sparse_ws_bytes_any(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K, int num_splits) {
  size_t need = 0;
  for (int fp8 = 0; fp8 < 2; fp8++) {
    const int G = head_groups(B * S, H, D, K, fp8);
    const size_t w = sparse_ws_bytes(B, S, H, D, G, choose_splits(B * G, S, K, num_splits));
    if (w > need) need = w;
  }
  return need;
}

// noalloc: take the workspace from the library's scratch array instead of the arguments
static int sparse_attn_run(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* out,
                           int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale,
                           int num_splits, void* workspace, size_t workspace_bytes, void* stream, int phases,
                           int fp8 = 0, int noalloc = 0) {
  if (!sparse_sizes_ok(B, S, H, D, K) || T < 0 || num_splits < 0 || num_splits > 64) return SA_ERR_SHAPE;
  if (B * S == 0 || H == 0) return SA_OK;
  if (D != 64 && D != 512) return SA_ERR_UNSUPPORTED;
  if (fp8 && (D != 512 || T * 584 > ((int64_t)1 << 31) - 1)) return fp8 && D != 512 ? SA_ERR_UNSUPPORTED : SA_ERR_SHAPE;
  if (fp8 && kv && ((uintptr_t)kv & 7u)) return SA_ERR_ALIGN;
  if (H > 128) return SA_ERR_UNSUPPORTED;
  if (B * S > (int64_t)1 << 30 || T > kInt32Max || K > (int64_t)1 << 30) return SA_ERR_SHAPE;
  if (!q || !attn_sink || !out || (K > 0 && !topk_idxs) || (T > 0 && K > 0 && !kv)) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (!fp8 && kv && !aligned16(kv))) return SA_ERR_ALIGN;
  if (((uintptr_t)attn_sink & 3u) || (topk_idxs && ((uintptr_t)topk_idxs & 3u))) return SA_ERR_ALIGN;
  const int G = head_groups(B * S, H, D, K, fp8);
  const int nsplit = choose_splits(B * G, S, K, num_splits);
  if (B * S * G * nsplit > ((int64_t)1 << 31) - 1) return SA_ERR_SHAPE;  // (token, split) pairs are int
  const size_t need = sparse_ws_bytes(B, S, H, D, G, nsplit);
  if (noalloc) {
    if (need > sa_internal_scratch_bytes()) return SA_ERR_WORKSPACE;
    workspace = nullptr;
    if (need > 0 && sa_internal_scratch_ptr(&workspace) != 0) return SA_ERR_HIP;
  } else if (need > 0) {
    if (!workspace || workspace_bytes < need) return SA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255u) return SA_ERR_ALIGN;
  }
  const int rc = sa_internal_launch_sparse(q, kv, attn_sink, topk_idxs, out, B, S, H, D, T, K, scale, nsplit,
                                           need > 0 ? workspace : nullptr, phases, fp8, G, stream);
  return rc == 0 ? SA_OK : SA_ERR_HIP;
}

int masked_run(const void* q, const void* k, const void* v, const uint32_t* mask, void* out, float* lse, int64_t B,
               int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv, int64_t padded_q, int64_t words, float scale,
               int mask_load_bits, int offset, void* stream) {
  if (B < 0 || Q < 0 || KV < 0 || H < 0 || Dqk < 0 || Dv < 0 || padded_q < 0 || words < 0) return SA_ERR_SHAPE;
  if (B * Q * H == 0) return SA_OK;
  if (Dqk != 192 || Dv != 128) return SA_ERR_UNSUPPORTED;
  if (H > kMaskedMaxHeads) return SA_ERR_UNSUPPORTED;
  if (mask && (padded_q < Q || words % 4 != 0 || words > kMaskedMaxWords)) return SA_ERR_SHAPE;
  if (Q > kInt32Max || padded_q > kInt32Max || words > kMaskedMaxWords) return SA_ERR_SHAPE;
  if (B * H * cdiv(Q, 128) > kInt32Max || KV > ((int64_t)1 << 30)) return SA_ERR_SHAPE;
  if (!q || !out || (KV > 0 && (!k || !v))) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (k && !aligned16(k)) || (v && !aligned16(v)) || (mask && !aligned16(mask)) ||
      ((uintptr_t)lse & 3) != 0)
    return SA_ERR_ALIGN;
  const int rc = sa_internal_launch_masked(q, k, v, mask, out, lse, B, Q, KV, H, Dqk, Dv, padded_q, words, scale,
                                           mask_load_bits, offset, stream);
  return rc == 0 ? SA_OK : (rc == 2 ? SA_ERR_UNSUPPORTED : SA_ERR_HIP);
}

}  // namespace

extern "C" {

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "a required pointer is NULL";
    case SA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case SA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SA_ERR_UNSUPPORTED: return "unsupported head dimension or head count";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int sparse_attn_head_groups(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K, int fp8) {
  if (!sparse_sizes_ok(B, S, H, D, K)) return 1;
  return head_groups(B * S, H, D, K, fp8 != 0);
}

int sparse_attn_fp8_num_splits(int64_t B, int64_t S, int64_t H, int64_t K) {
  if (!sparse_sizes_ok(B, S, H, 512, K)) return 1;
  return choose_splits(B * head_groups(B * S, H, 512, K, 1), S, K, 0);
}

int sparse_attn_num_splits(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K) {
  if (!sparse_sizes_ok(B, S, H, D, K)) return 1;
  return choose_splits(B * head_groups(B * S, H, D, K, 0), S, K, 0);
}

size_t sparse_attn_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D, int64_t K, int num_splits) {
  if (!sparse_sizes_ok(B, S, H, D, K) || num_splits < 0) return 0;
  if (H < 1 || H > 128) return 0;
  return sparse_ws_bytes_any(B, S, H, D, K, num_splits);
}

int sparse_attn_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* out,
                    int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_run(q, kv, attn_sink, topk_idxs, out, B, S, H, D, T, K, scale, num_splits, workspace,
                         workspace_bytes, stream, 3);
}

int sparse_attn_fwd_noalloc(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs,
                            void* out, int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale,
                            int num_splits, void* stream) {
  return sparse_attn_run(q, kv, attn_sink, topk_idxs, out, B, S, H, D, T, K, scale, num_splits, nullptr, 0, stream, 3,
                         0, 1);
}

int sparse_attn_split_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* out,
                          int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_run(q, kv, attn_sink, topk_idxs, out, B, S, H, D, T, K, scale, num_splits, workspace,
                         workspace_bytes, stream, 1);
}

int sparse_attn_merge_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* out,
                          int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_run(q, kv, attn_sink, topk_idxs, out, B, S, H, D, T, K, scale, num_splits, workspace,
                         workspace_bytes, stream, 2);
}

int sparse_attn_fp8_fwd(const void* q, const void* kv8, const float* attn_sink, const int32_t* topk_idxs, void* out,
                        int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, float scale, int num_splits,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_run(q, kv8, attn_sink, topk_idxs, out, B, S, H, 512, T, K, scale, num_splits, workspace,
                         workspace_bytes, stream, 3, 1);
}

int sparse_attn_fp8_split_fwd(const void* q, const void* kv8, const float* attn_sink, const int32_t* topk_idxs,
                              void* out, int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, float scale,
                              int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_run(q, kv8, attn_sink, topk_idxs, out, B, S, H, 512, T, K, scale, num_splits, workspace,
                         workspace_bytes, stream, 1, 1);
}

int sparse_attn_fp8_merge_fwd(const void* q, const void* kv8, const float* attn_sink, const int32_t* topk_idxs,
                              void* out, int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, float scale,
                              int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_run(q, kv8, attn_sink, topk_idxs, out, B, S, H, 512, T, K, scale, num_splits, workspace,
                         workspace_bytes, stream, 2, 1);
}

int topk_bitmask_shape(int64_t B, int64_t max_q_len, int64_t max_key_len, int reserve_key_start_word,
                       int64_t* out_shape) {
  if (!out_shape) return SA_ERR_NULL;
  if (B < 0 || max_q_len < 0 || max_key_len < 0) return SA_ERR_SHAPE;
  const int64_t tile_m = max_q_len <= 128 ? 128 : 256;
  const int64_t words = cdiv(cdiv(max_key_len, 32) + (reserve_key_start_word ? 1 : 0), 4) * 4;
  out_shape[0] = B;
  out_shape[1] = cdiv(max_q_len, tile_m) * tile_m;
  out_shape[2] = words;
  return SA_OK;
}

int topk_bitmask_build(const int32_t* topk_idxs, const int32_t* q_lens, const int32_t* key_starts, uint32_t* mask,
                       int64_t B, int64_t Q, int64_t topk, int64_t key_len, int64_t padded_q, int64_t words,
                       void* stream) {
  if (B < 0 || Q < 0 || topk < 0 || key_len < 0 || padded_q < 0 || words < 0) return SA_ERR_SHAPE;
  if (padded_q < Q || words % 4 != 0 || 32 * words < key_len) return SA_ERR_SHAPE;
  if (key_starts && (words < cdiv(key_len, 32) + 1 || padded_q < 1)) return SA_ERR_SHAPE;
  if (B * padded_q == 0 || words == 0) return SA_OK;
  if (words > sa_internal_bitmask_max_words()) return SA_ERR_UNSUPPORTED;
  if (B * padded_q > kInt32Max || topk > kInt32Max || B * Q * topk > ((int64_t)1 << 40)) return SA_ERR_SHAPE;
  if (!mask || (Q > 0 && topk > 0 && !topk_idxs)) return SA_ERR_NULL;
  if (!aligned16(mask)) return SA_ERR_ALIGN;
  if ((topk_idxs && ((uintptr_t)topk_idxs & 3u)) || (q_lens && ((uintptr_t)q_lens & 3u)) ||
      (key_starts && ((uintptr_t)key_starts & 3u)))
    return SA_ERR_ALIGN;
  const int rc = sa_internal_launch_bitmask(topk_idxs, q_lens, key_starts, mask, B, Q, topk, key_len, padded_q,
                                            words, stream);
  return rc == 0 ? SA_OK : SA_ERR_HIP;
}

int masked_attn_fwd(const void* q, const void* k, const void* v, const uint32_t* mask, void* out, int64_t B,
                    int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv, int64_t padded_q, int64_t words,
                    float scale, int mask_load_bits, void* stream) {
  if (mask_load_bits != 128 && mask_load_bits != 32) return SA_ERR_SHAPE;
  if (mask && KV > 32 * words) return SA_ERR_SHAPE;
  return masked_run(q, k, v, mask, out, nullptr, B, Q, KV, H, Dqk, Dv, padded_q, words, scale, mask_load_bits, 0,
                    stream);
}

int masked_attn_offset_fwd(const void* q, const void* k, const void* v, const uint32_t* mask, void* out, float* lse,
                           int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv, int64_t padded_q,
                           int64_t words, float scale, void* stream) {
  if (words < 0) return SA_ERR_SHAPE;
  if (B * Q * H > 0 && !mask) return SA_ERR_NULL;
  if (B * Q * H > 0 && words < 4) return SA_ERR_SHAPE;
  return masked_run(q, k, v, mask, out, lse, B, Q, KV, H, Dqk, Dv, padded_q, words, scale, 128, 1, stream);
}

int candidate_mask_apply(float* logits, const int32_t* starts, const int32_t* ends, const uint8_t* flags,
                         int64_t rows, int64_t width, int64_t stride_row, int64_t stride_col, int64_t stride_start,
                         int64_t stride_end, int64_t block_size, int64_t row_repeat, void* stream) {
  if (rows < 0 || width < 0 || block_size < 1 || row_repeat < 1) return SA_ERR_SHAPE;
  if (stride_row < 0 || stride_col < 1 || stride_start < 0 || stride_end < 0) return SA_ERR_SHAPE;
  if (rows == 0 || width == 0) return SA_OK;
  if (width > ((int64_t)1 << 31) - 1 - 4096 || rows > ((int64_t)1 << 31) - 1) return SA_ERR_SHAPE;
  if (rows * (int64_t)sa_internal_candidate_gcols(rows, width) > ((int64_t)1 << 31) - 1) return SA_ERR_SHAPE;
  if (!logits || !ends || !flags) return SA_ERR_NULL;
  if (((uintptr_t)logits & 3u) || ((uintptr_t)ends & 3u) || (starts && ((uintptr_t)starts & 3u))) return SA_ERR_ALIGN;
  const int rc = sa_internal_launch_candidate_mask(logits, starts, ends, flags, rows, width, stride_row, stride_col,
                                                   stride_start, stride_end, block_size, row_repeat, stream);
  return rc == 0 ? SA_OK : SA_ERR_HIP;
}

int candidate_mask_grid(int64_t rows, int64_t width) {
  if (rows <= 0 || width <= 0) return 0;
  return (int)(rows * sa_internal_candidate_gcols(rows, width));
}

}  // extern "C"
