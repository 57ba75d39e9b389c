/*
 * CPU oracle for top-k sparse attention and its bit-packed-mask form.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * reference that the GPU library is checked against. Only the test suite, the
 * package's smoke check and the benchmark's CPU-baseline leg may load it. It
 * shares no code, header, table or helper with the GPU library, and the GPU
 * library never calls it.
 *
 * Arithmetic is IEEE double throughout. bf16 inputs are widened exactly
 * (a bf16 value is the top 16 bits of an IEEE single). Loops run in the order
 * the definitions state; OpenMP only splits independent outputs across threads.
 *
 * Sources (web pages the method is described on):
 *  [DSV4-5]  "DeepSeek V4 源码剖析", chapter 5 "sparse_attn 与 FlashMLA":
 *            section 5.1 (argument shapes, -1 marks an invalid slot),
 *            section 5.2 (loop semantics of sparse_attn),
 *            section 5.4 (invalid slots contribute a zero row),
 *            section 5.5 (sink enters the softmax denominator only; +inf and
 *            -inf sinks are boundary cases of the split-KV combine).
 *  [PR52217] prhub summary of vLLM PR #52217 "Sparse MLA mask 128-bit loads":
 *            key-source section (_topk_mask_shape shape rule, word rows padded
 *            to a multiple of 4) and its test (129 keys -> 8 words, bits 0 and
 *            128 land in words 0 and 4, padding kept and zero).
 *  [PR48770] prhub summary of vLLM PR #48770 "masked MHA for sparse MLA
 *            prefill": key-source section (dense_mask_mod: word = kv >> 5,
 *            bit = kv & 31, LSB first; offset_dense_mask_mod reads key_start
 *            from the last word of query row 0 and adds it to the key index).
 *            section 5.7 (FlashMLA's MODEL1 FP8 row: 448 e4m3 bytes, 64 bf16
 *            RoPE dims, 8 scale bytes for 64-dim quantisation tiles).
 *  [PR56628] prhub summary of vLLM PR #56628 "ROCm DSA decode mask strides to
 *            each row's end": the candidate-mask rule (live columns
 *            [start, end), per-block keep flags relative to start, the edge
 *            flag for the last column, -inf elsewhere) and its tests.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0 /* >0 plants a known mistake; used only by the mutation test */
#endif

/* Exact widening of a bf16 bit pattern: the value is the IEEE single whose
 * high half is `bits` and low half is zero. */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 holds the subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; there is no infinity. */
static double e4m3_to_double(uint8_t x) {
  const int sgn = x >> 7, e = (x >> 3) & 15, m = x & 7;
  double v;
#if ORACLE_MUTANT == 19
  v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 8); /* mutant: bias 8 */
#else
  if (e == 15 && m == 7) return NAN;
  v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
#endif
  return sgn ? -v : v;
}

/* Unsigned power-of-two scale byte (UE8M0): 2^(s - 127); 255 is NaN. */
static double ue8m0_to_double(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* FP8 row layout (MODEL1 row of [DSV4-5] section 5.7, 584 bytes for D = 512): bytes 0..447
 * e4m3 values of dims 0..447, bytes 448..575 the bf16 (little-endian) dims 448..511,
 * bytes 576..582 one scale byte per 64-dim tile of the e4m3 part, byte 583 padding.
 * Dim d < 448 is e4m3(byte d) * 2^(scale[d / 64] - 127). The scale byte encoding is not
 * printed on the page; UE8M0 is this oracle's reading. */
#define FP8_ROW_BYTES 584
#define FP8_NOPE 448
static double fp8_row_value(const uint8_t* row, int64_t d) {
  if (d < FP8_NOPE) {
#if ORACLE_MUTANT == 18
    const int64_t tile = d / 64 + (d >= 64); /* mutant: tile index off by one past the first tile */
#else
    const int64_t tile = d / 64;
#endif
    return e4m3_to_double(row[d]) * ue8m0_to_double(row[FP8_NOPE + 128 + tile]);
  }
  const uint8_t* p = row + FP8_NOPE + 2 * (d - FP8_NOPE);
  return bf16_bits_to_double((uint16_t)(p[0] | (p[1] << 8)));
}

/* ------------------------------------------------------------------------ */
/* sparse_attn  ([DSV4-5] sections 5.1, 5.2, 5.4, 5.5)                       */
/* ------------------------------------------------------------------------ */
/*
 * q    [B][S][H][D] bf16 bits      kv [B][T][D] bf16 bits (row = key = value)
 * sink [H] float                   idx [B][S][K] int32, slot valid iff 0 <= idx < T
 * tokens: list of ntok flat token ids t = b*S + s to evaluate.
 * out  [ntok][H][D] double
 *
 * For one (b, s, h), with V the multiset of valid slots:
 *   x_k = scale * sum_d q[b,s,h,d] * kv[b,idx_k,d]             (k in V)
 *   weights = softmax over the logits {x_k : k in V} plus one extra logit sink[h]
 *   o[d]    = sum_{k in V} weight_k * kv[b,idx_k,d]            (the sink has no row)
 * computed with m = max(sink, max_k x_k) subtracted before exponentiation.
 * Boundary readings: sink NaN -> NaN row; sink +inf -> every real weight is 0,
 * o = 0; no valid slot and sink -inf -> o = 0 (empty softmax taken as zero).
 * Returns 0, or -1 on a bad argument.
 */
/* kv row element: bf16 rows [B][T][D] (fp8 == 0) or FP8 rows [B][T][584] (fp8 != 0, D = 512) */
static double kv_value(const void* kv, int fp8, int64_t b, int64_t T, int64_t D, int64_t j, int64_t d) {
  if (fp8) return fp8_row_value((const uint8_t*)kv + (b * T + j) * FP8_ROW_BYTES, d);
  return bf16_bits_to_double(((const uint16_t*)kv)[(b * T + j) * D + d]);
}

static int sparse_attn_impl(const uint16_t* q, const void* kv, int fp8, const float* sink, const int32_t* idx,
                            double* out, int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K,
                            double scale, const int64_t* tokens, int64_t ntok) {
  if (!q || !kv || !sink || !idx || !out || !tokens) return -1;
  if (B < 0 || S < 0 || H < 0 || D < 0 || T < 0 || K < 0 || ntok < 0) return -1;
  if (fp8 && D != 512) return -1;
  for (int64_t i = 0; i < ntok; i++)
    if (tokens[i] < 0 || tokens[i] >= B * S) return -1;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ti = 0; ti < ntok; ti++) {
    const int64_t t = tokens[ti];
    const int64_t b = t / S;
    const int32_t* slots = idx + t * K;
    double* x = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    for (int64_t h = 0; h < H; h++) {
#if ORACLE_MUTANT == 11
      const uint16_t* qv = q + (t * H + 0) * D; /* mutant: every head uses head 0's query */
#else
      const uint16_t* qv = q + (t * H + h) * D;
#endif
      double* o = out + (ti * H + h) * D;
      const double s_h = (double)sink[h];
      for (int64_t d = 0; d < D; d++) o[d] = 0.0;

      /* logits of the valid slots; an invalid slot gets no logit at all */
      double m = s_h;
      for (int64_t k = 0; k < K; k++) {
        int64_t j = slots[k];
#if ORACLE_MUTANT == 2
        if (j == -1) j = T - 1; /* mutant: -1 read as the last row (python negative index) */
#endif
        if (j < 0 || j >= T) continue;
        double dot = 0.0;
        for (int64_t d = 0; d < D; d++) dot += bf16_bits_to_double(qv[d]) * kv_value(kv, fp8, b, T, D, j, d);
#if ORACLE_MUTANT == 3
        x[k] = dot; /* mutant: scale dropped */
#else
        x[k] = scale * dot;
#endif
        if (x[k] > m) m = x[k];
      }

      if (isnan(s_h)) {
        for (int64_t d = 0; d < D; d++) o[d] = NAN;
        continue;
      }
      if (s_h == INFINITY) continue; /* all weight on the sink, which carries no row */
      if (m == -INFINITY) continue;  /* nothing valid and no sink */

      double l = exp(s_h - m);
#if ORACLE_MUTANT == 1
      l = 0.0; /* mutant: sink left out of the denominator */
#endif
      for (int64_t k = 0; k < K; k++) {
        int64_t j = slots[k];
#if ORACLE_MUTANT == 2
        if (j == -1) j = T - 1;
#endif
        if (j < 0 || j >= T) continue;
#if ORACLE_MUTANT == 5
        /* mutant: duplicate slots collapsed to one occurrence */
        int dup = 0;
        for (int64_t k2 = 0; k2 < k; k2++) dup |= (slots[k2] == j);
        if (dup) continue;
#endif
        const double p = exp(x[k] - m);
        l += p;
        for (int64_t d = 0; d < D; d++) o[d] += p * kv_value(kv, fp8, b, T, D, j, d);
      }
      for (int64_t d = 0; d < D; d++) o[d] /= l;
    }
    free(x);
  }
  return 0;
}

int oracle_sparse_attn(const uint16_t* q, const uint16_t* kv, const float* sink, const int32_t* idx, double* out,
                       int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K, double scale,
                       const int64_t* tokens, int64_t ntok) {
  return sparse_attn_impl(q, kv, 0, sink, idx, out, B, S, H, D, T, K, scale, tokens, ntok);
}

/*
 * The same computation over FP8 rows: kv8 [B][T][584] bytes in the row layout above
 * (D = 512), each row dequantized exactly before use.
 */
int oracle_sparse_attn_fp8(const uint16_t* q, const uint8_t* kv8, const float* sink, const int32_t* idx, double* out,
                           int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, double scale,
                           const int64_t* tokens, int64_t ntok) {
  return sparse_attn_impl(q, kv8, 1, sink, idx, out, B, S, H, 512, T, K, scale, tokens, ntok);
}

/* Dequantized FP8 rows (for checks): out [n][512] double for rows kv8 [n][584]. */
int oracle_fp8_dequant(const uint8_t* kv8, double* out, int64_t n) {
  if (!kv8 || !out || n < 0) return -1;
  for (int64_t j = 0; j < n; j++)
    for (int64_t d = 0; d < 512; d++) out[j * 512 + d] = fp8_row_value(kv8 + j * FP8_ROW_BYTES, d);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* top-k bit mask  ([PR52217] key source + test; [PR48770] dense_mask_mod)   */
/* ------------------------------------------------------------------------ */
static int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

/*
 * Shape of the bit-packed mask for a batch: query rows are padded to a tile of
 * 128 rows when the longest query fits in 128, else to 256; a row holds one bit
 * per key in 32-bit words, plus one reserved word when key starts are stored,
 * and the word count is rounded up to a multiple of 4 so every row is a whole
 * number of 16-byte chunks.
 */
int oracle_topk_mask_shape(int64_t B, int64_t max_q, int64_t max_key, int reserve_key_start_word, int64_t* out3) {
  if (!out3 || B < 0 || max_q < 0 || max_key < 0) return -1;
  const int64_t tile_m = max_q <= 128 ? 128 : 256;
  const int64_t padded_q = cdiv64(max_q, tile_m) * tile_m;
  int64_t words = cdiv64(max_key, 32) + (reserve_key_start_word ? 1 : 0);
  words = cdiv64(words, 4) * 4;
  out3[0] = B;
  out3[1] = padded_q;
  out3[2] = words;
  return 0;
}

/*
 * idx [B][Q][topk] int32; q_lens [B] (NULL = every row is live); key_starts [B]
 * (NULL = none). mask [B][padded_q][W] uint32 is written in full:
 *   mask[b][q][j >> 5] has bit (j & 31) set  iff  q < q_len[b] and some slot of
 *   idx[b][q] equals j with 0 <= j < key_len;
 *   mask[b][0][W-1] = key_starts[b] when key starts are given (the reserved word);
 *   every other word (padding words, rows q >= q_len[b]) is 0.
 * Returns 0, or -1 on a bad argument (including a reserved word that would
 * overlap a bit word).
 */
int oracle_topk_mask_build(const int32_t* idx, const int32_t* q_lens, const int32_t* key_starts, uint32_t* mask,
                           int64_t B, int64_t Q, int64_t topk, int64_t key_len, int64_t padded_q, int64_t W) {
  if (!mask || B < 0 || Q < 0 || topk < 0 || key_len < 0 || padded_q < Q || W < 0) return -1;
  if (Q > 0 && topk > 0 && !idx) return -1;
  if (W * 32 < key_len) return -1;
  if (key_starts && (W < cdiv64(key_len, 32) + 1 || padded_q < 1)) return -1;

  for (int64_t e = 0; e < B * padded_q * W; e++) mask[e] = 0u;
  for (int64_t b = 0; b < B; b++) {
    int64_t live = Q;
    if (q_lens) {
      live = q_lens[b];
      if (live < 0) live = 0;
      if (live > Q) live = Q;
    }
    for (int64_t qi = 0; qi < live; qi++) {
      uint32_t* row = mask + (b * padded_q + qi) * W;
      const int32_t* slots = idx + (b * Q + qi) * topk;
      for (int64_t k = 0; k < topk; k++) {
        const int64_t j = slots[k];
        if (j < 0 || j >= key_len) continue;
#if ORACLE_MUTANT == 6
        row[(j >> 5) + ((j >> 5) + 1 < W ? 1 : 0)] |= 1u << (j & 31); /* mutant: word index off by one */
#elif ORACLE_MUTANT == 7
        row[j >> 5] |= 1u << (31 - (j & 31)); /* mutant: MSB-first bit order */
#else
        row[j >> 5] |= 1u << (j & 31);
#endif
      }
    }
    if (key_starts) {
#if ORACLE_MUTANT == 8
      mask[(b * padded_q + 0) * W + 0] = (uint32_t)key_starts[b]; /* mutant: key start in word 0 */
#else
      mask[(b * padded_q + 0) * W + (W - 1)] = (uint32_t)key_starts[b];
#endif
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* masked attention  ([PR48770] masked-MHA path + dense_mask_mod;            */
/*                    [PR52217] 128-bit mask loads leave the result unchanged) */
/* ------------------------------------------------------------------------ */
/*
 * q [B][Q][H][Dqk], k [B][KV][H][Dqk], v [B][KV][H][Dv] bf16 bits;
 * mask [B][padded_q][W] uint32 or NULL (NULL = every key is visible).
 * rows: list of nrows flat query rows r = b*Q + qi to evaluate.
 * out [nrows][H][Dv] double.
 *   J = { j < KV : mask is NULL or bit (j & 31) of mask[b][qi][j >> 5] is set }
 *   x_j = scale * q.k_j;  o = sum_{j in J} softmax(x)_j v_j   (max subtracted first)
 *   J empty -> o = 0.  No sink, one mask shared by every head.
 *
 * Chunked-context form ([PR48770] offset_dense_mask_mod), offset != 0: k and v are
 * one chunk of a longer context and chunk key j is key p = key_start + j of the mask
 * row, with key_start[b] = mask[b][0][W-1] (the reserved word, read as an unsigned
 * 32-bit value):
 *   J = { j < KV : p < 32 (W - 1) and bit (p & 31) of mask[b][qi][p >> 5] is set }.
 * Positions at or past the reserved word are never visible (that word holds the
 * start, not bits).
 */
static int masked_attn_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* mask,
                            double* out, int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv,
                            int64_t padded_q, int64_t W, double scale, const int64_t* rows, int64_t nrows,
                            int offset) {
  if (!q || !k || !v || !out || !rows) return -1;
  if (B < 0 || Q < 0 || KV < 0 || H < 0 || Dqk < 0 || Dv < 0 || nrows < 0) return -1;
  if (mask && (padded_q < Q || (!offset && W * 32 < KV))) return -1;
  if (offset && (!mask || W < 1)) return -1;
  for (int64_t i = 0; i < nrows; i++)
    if (rows[i] < 0 || rows[i] >= B * Q) return -1;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ri = 0; ri < nrows; ri++) {
    const int64_t r = rows[ri];
    const int64_t b = r / Q, qi = r % Q;
    const uint32_t* mrow = mask ? mask + (b * padded_q + qi) * W : NULL;
    double* x = (double*)malloc(sizeof(double) * (size_t)(KV > 0 ? KV : 1));
    char* vis = (char*)malloc((size_t)(KV > 0 ? KV : 1));
    if (offset) {
#if ORACLE_MUTANT == 14
      const uint64_t key_start = mrow[W - 1]; /* mutant: start read from the query's own row */
#else
      const uint64_t key_start = mask[(b * padded_q + 0) * W + (W - 1)];
#endif
      const uint64_t limit = 32u * (uint64_t)(W - 1);
      for (int64_t j = 0; j < KV; j++) {
#if ORACLE_MUTANT == 13
        const uint64_t p = (uint64_t)j; /* mutant: start ignored */
#else
        const uint64_t p = key_start + (uint64_t)j;
#endif
#if ORACLE_MUTANT == 15
        vis[j] = p < 32u * (uint64_t)W ? (char)((mrow[p >> 5] >> (p & 31)) & 1u) : 0; /* mutant: reserved word read as bits */
#else
        vis[j] = p < limit ? (char)((mrow[p >> 5] >> (p & 31)) & 1u) : 0;
#endif
      }
    } else {
      for (int64_t j = 0; j < KV; j++) {
#if ORACLE_MUTANT == 9
        vis[j] = 1; /* mutant: mask ignored */
#else
        vis[j] = mrow ? (char)((mrow[j >> 5] >> (j & 31)) & 1u) : 1;
#endif
      }
    }
    for (int64_t h = 0; h < H; h++) {
      const uint16_t* qv = q + ((b * Q + qi) * H + h) * Dqk;
      double* o = out + (ri * H + h) * Dv;
      for (int64_t d = 0; d < Dv; d++) o[d] = 0.0;
      double m = -INFINITY;
      for (int64_t j = 0; j < KV; j++) {
        if (!vis[j]) continue;
        const uint16_t* kr = k + ((b * KV + j) * H + h) * Dqk;
        double dot = 0.0;
        for (int64_t d = 0; d < Dqk; d++) dot += bf16_bits_to_double(qv[d]) * bf16_bits_to_double(kr[d]);
#if ORACLE_MUTANT == 12
        x[j] = scale * scale * dot; /* mutant: scale applied twice */
#else
        x[j] = scale * dot;
#endif
        if (x[j] > m) m = x[j];
      }
      if (m == -INFINITY) continue; /* no visible key */
      double l = 0.0;
      for (int64_t j = 0; j < KV; j++) {
        if (!vis[j]) continue;
        const double p = exp(x[j] - m);
        l += p;
#if ORACLE_MUTANT == 10
        const uint16_t* vr = k + ((b * KV + j) * H + h) * Dqk; /* mutant: keys used as values */
#else
        const uint16_t* vr = v + ((b * KV + j) * H + h) * Dv;
#endif
        for (int64_t d = 0; d < Dv; d++) o[d] += p * bf16_bits_to_double(vr[d]);
      }
      for (int64_t d = 0; d < Dv; d++) o[d] /= l;
    }
    free(x);
    free(vis);
  }
  return 0;
}

int oracle_masked_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* mask, double* out,
                       int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv, int64_t padded_q, int64_t W,
                       double scale, const int64_t* rows, int64_t nrows) {
  return masked_attn_impl(q, k, v, mask, out, B, Q, KV, H, Dqk, Dv, padded_q, W, scale, rows, nrows, 0);
}

int oracle_masked_attn_offset(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* mask,
                              double* out, int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv,
                              int64_t padded_q, int64_t W, double scale, const int64_t* rows, int64_t nrows) {
  return masked_attn_impl(q, k, v, mask, out, B, Q, KV, H, Dqk, Dv, padded_q, W, scale, rows, nrows, 1);
}

/* ------------------------------------------------------------------------ */
/* candidate mask  ([PR56628] the indexer's candidate-mask rule)            */
/* ------------------------------------------------------------------------ */
/*
 * The rule of the shared whole-row kernel that the strided MI355X variant must
 * match on [0, end) ([PR56628], key source: the strided kernel's mask rule and
 * its tests' contract). logits [rows] x [width] float, element (r, c) at
 * logits[r * stride_row + c * stride_col], modified in place. For row r, with
 * i = r / row_repeat, s = starts ? starts[i * stride_start] : 0,
 * e = ends[i * stride_end], nblocks = ceil(width / block_size):
 *   column c is live iff s <= c < e;
 *   a live column is kept iff flags[r][(c - s) / block_size] != 0 (a block
 *   index outside [0, nblocks) keeps nothing) or c == width - 1 and the edge
 *   flag flags[r][nblocks] != 0;
 *   every column that is not kept, live or not, becomes -inf; kept columns are
 *   left as they are.
 * flags is uint8 [rows][nblocks + 1]. Returns 0, or -1 on a bad argument.
 */
int oracle_candidate_mask(float* logits, const int32_t* starts, const int32_t* ends, const uint8_t* flags,
                          int64_t rows, int64_t width, int64_t stride_row, int64_t stride_col, int64_t stride_start,
                          int64_t stride_end, int64_t block_size, int64_t row_repeat) {
  if (!logits || !ends || !flags || rows < 0 || width < 0 || block_size < 1 || row_repeat < 1) return -1;
  const int64_t nblocks = (width + block_size - 1) / block_size;
  for (int64_t r = 0; r < rows; r++) {
    const int64_t i = r / row_repeat;
    const int64_t s = starts ? starts[i * stride_start] : 0;
    const int64_t e = ends[i * stride_end];
    const uint8_t* fr = flags + r * (nblocks + 1);
    for (int64_t c = 0; c < width; c++) {
      const int live = (s <= c) && (c < e);
      int keep = 0;
      if (live) {
#if ORACLE_MUTANT == 16
        const int64_t blk = c / block_size; /* mutant: block counted from column 0, not from the start */
#else
        const int64_t blk = (c - s) / block_size;
#endif
        if (blk >= 0 && blk < nblocks && fr[blk] != 0) keep = 1;
#if ORACLE_MUTANT != 17
        if (c == width - 1 && fr[nblocks] != 0) keep = 1; /* mutant 17: edge flag ignored */
#endif
      }
      if (!keep) logits[r * stride_row + c * stride_col] = -INFINITY;
    }
  }
  return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads later calls use (for timing on fewer cores; no effect
   without OpenMP). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
