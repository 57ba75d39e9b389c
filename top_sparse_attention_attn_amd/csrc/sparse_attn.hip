// Top-k sparse attention on gfx950.
//
// What is computed ("DeepSeek V4 源码剖析", ch. 5, sections 5.2, 5.4, 5.5): for every
// token and head, a softmax over the scaled dot products with the K gathered rows
// kv[b, idx] (empty slots excluded) plus one sink logit, applied to the same rows; the
// sink takes part in the normalisation only.
//
// Work decomposition (MI355X-specific; the pages' kernels are prior art only):
//  * One workgroup per (token, slot range) covering ALL heads of the token, so every
//    gathered row is pulled from HBM into LDS once and used by all heads. When there
//    are too few tokens to fill the 256 CUs a token's slots are cut into `nsplit`
//    ranges, merged afterwards by a small kernel that adds the sink exactly once.
//  * Rows arrive in 32-row tiles through a 4-deep ring of LDS buffers, written by
//    buffer loads into LDS (16 bytes per lane, one 1 KB row per wave instruction) straight
//    from memory, two tiles ahead of the tile whose scores are being computed.
//  * 12 waves, 3 per SIMD, in two roles that run one tile apart:
//      score waves (0-3) keep the queries of two 16-head blocks in registers, compute
//        S^T = K Q^T for tile t with MFMA 16x16x32 bf16 (the K operand of the next
//        step is read while the current one multiplies) and the online softmax, and
//        write the bf16 weights P to LDS;
//      value waves (4-11) gather the rows and add P V for tile t-1, each owning a
//        slice of the head dimension of the output for all heads; V is read with the
//        transposing LDS read (ds_read_b64_tr_b16).
//    One barrier per tile. Score waves hold queries, value waves the accumulators, so
//    neither runs short of registers for keeping LDS reads in flight.
//  * Online softmax in base 2 with a lazily moved reference maximum: the output is
//    rescaled only when a head's maximum grows by more than 2^8 (rare after the first
//    tile); weights stay <= 2^8, so nothing overflows.
//  * FP8 rows (the MODEL1 row of section 5.7: 448 e4m3 bytes, 64 bf16 RoPE dims, one scale
//    byte per 64-dim tile, 584 bytes for D = 512): the value waves copy each row's bytes into
//    its ring slot with buffer loads that write LDS, and one tile before the tile is used
//    they expand it in place to the bf16 row (v_cvt_scalef32_pk_bf16_fp8, scale 2^(s-127)),
//    so the scores and P V run unchanged on bf16 rows while HBM moves 584 bytes per row.
#include <stddef.h>

#include <mutex>

#include "common.h"

namespace sa {

constexpr int kTile = 32;       // rows per tile
constexpr int kBufs = 4;        // LDS ring depth (tiles t-1 .. t+2)
constexpr float kLazy = 8.0f;   // reference-max slack, log2 units
constexpr int kMaxSplits = 16;
constexpr int kThreads = 768;   // 4 score waves + 8 value waves
constexpr int kValueWaves = 8;
constexpr int kPStride = kTile + 8;  // bf16 elements per P row in LDS (80 bytes)
constexpr int kF8Row = 584;         // FP8 row: 448 e4m3 + 128 bytes of bf16 RoPE + 8 scale bytes
constexpr int kF8Nope = 448;

template <int D>
struct Geo {
  // Padded LDS row (D*2 + 32 bytes, 8 banks of skew per row): the K operand reads (16 bytes of
  // 16 rows) and the transposed V reads (8 bytes of 4 rows per 16 lanes, rows 4g..4g+3) are
  // then free of bank conflicts on the 64-bank LDS.
  static constexpr int kRowStride = D * 2 + 32;
  static constexpr int kBufBytes = kTile * kRowStride;
  static constexpr int kDSteps = D / 32;         // QK MFMA steps over the head dimension
  static constexpr int kLanesPerRow = D / 8;     // 16-byte chunks per row
  static constexpr int kNDB = D / 16;            // 16-column output blocks
  static constexpr int kDBV = kNDB >= kValueWaves ? kNDB / kValueWaves : 1;  // blocks per value wave
  static constexpr int kRowSeg = 32 - (D == 512 ? 10 : 7);  // rows per 4 GB: 2^kRowSeg (row bytes 2^10 or 2^7)
  static_assert(D == 512 || D == 64, "row segments assume D = 512 or 64");
  static_assert(kNDB % 4 == 0 && (kNDB < kValueWaves || kNDB % kValueWaves == 0),
                "head dimension must be a multiple of 64");
};

template <int D, int HB>
struct Smem {
  unsigned char kv[kBufs][Geo<D>::kBufBytes];
  __bf16 p[2][HB * 16 * kPStride];
  // per-head softmax state, contiguous in this order (the score waves address all of it
  // from one base): reference maximum (log2 units), running weight sum, and the rescale
  // factor of the last two tiles for the value waves
  float mref[HB * 16];
  float lsum[HB * 16];
  float alpha[2][HB * 16];
  float fin[HB * 16];
  unsigned char vmb[kBufs][8];  // per value wave: validity of its 4 rows of the tile (one byte each)
  int flag[2][4];
  int idx[2][64];  // bf16 rows: slot indices of a tile two or three ahead (by tile parity; 32 used)
};

// 32-bit validity mask of a tile's rows (bit j = row j holds a gathered row).
template <int D, int HB>
__device__ __forceinline__ unsigned tile_mask(const Smem<D, HB>& sm, int bi) {
  const uint2 v = *(const uint2*)(&sm.vmb[bi][0]);
  auto nib = [](unsigned x) {
    return (x & 0xFu) | ((x >> 4) & 0xF0u) | ((x >> 8) & 0xF00u) | ((x >> 12) & 0xF000u);
  };
  return nib(v.x) | (nib(v.y) << 16);
}

// Output slice of one wave: NB column blocks starting at block DB0.
template <int D, int HB, int NB>
__device__ __forceinline__ void pv_step(Smem<D, HB>& sm, f32x4 (&oacc)[HB][NB > 0 ? NB : 1], int db0, int tp, int bi,
                                        int lane, int g, int l16) {
  using G = Geo<D>;
  if constexpr (NB > 0) {
    const int par = tp & 1;
    if (sm.flag[par][0] | sm.flag[par][1] | sm.flag[par][2] | sm.flag[par][3]) {
#pragma unroll
      for (int hb = 0; hb < HB; hb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float a = sm.alpha[par][hb * 16 + 4 * g + i];
#pragma unroll
          for (int db = 0; db < NB; db++) oacc[hb][db][i] *= a;
        }
    }
    // V operands of this wave's column blocks (transposed reads), then one P operand per
    // head block: keeps at most one P operand live. The MFMA's k index 8g+i stands for tile
    // row 4g+i (i < 4) or 16+4g+i-4 (i >= 4); P is stored in LDS in the same order.
    const int r4 = (lane >> 2) & 3, c4 = lane & 3;
    const unsigned char* vbase = &sm.kv[bi][(4 * g + r4) * G::kRowStride + (db0 * 16 + 4 * c4) * 2];
    bf16x8 bv[NB];
#pragma unroll
    for (int db = 0; db < NB; db++) {
      const unsigned char* p0 = vbase + db * 32;
      bv[db] = concat_tr(lds_read_tr16(p0), lds_read_tr16(p0 + 16 * G::kRowStride));
    }
#pragma unroll
    for (int hb = 0; hb < HB; hb++) {
      const bf16x8 pa = *(const bf16x8*)(&sm.p[par][(hb * 16 + l16) * kPStride + 8 * g]);
#pragma unroll
      for (int db = 0; db < NB; db++) oacc[hb][db] = mfma16x16x32(pa, bv[db], oacc[hb][db]);
    }
  }
}

template <int D, int HB, bool SCORE, bool F8, bool NT>
__device__ __forceinline__ void run_split(Smem<D, HB>& sm, const __bf16* __restrict__ q, const void* __restrict__ kv,
                                          const float* __restrict__ sink, const int* __restrict__ idx,
                                          __bf16* __restrict__ out, __bf16* __restrict__ ws_o,
                                          float* __restrict__ ws_ml, int S, int H, int T, int K, int nsplit,
                                          int ngrp, int nxcc, int tok_mul, float scale_log2) {
  using G = Geo<D>;
  constexpr int HP = HB * 16;
  constexpr int NB = SCORE ? 0 : G::kDBV;  // output column blocks of this wave
  constexpr int NBX = NB > 0 ? NB : 1;
  using SM = Smem<D, HB>;
  static_assert(offsetof(SM, lsum) == offsetof(SM, mref) + HP * 4 &&
                    offsetof(SM, alpha) == offsetof(SM, mref) + 2 * HP * 4,
                "per-head state must be contiguous");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int sw = SCORE ? wave : wave - 4;  // index within the role
  const int db0 = SCORE ? 0 : sw * G::kDBV;
  const bool pv_active = !SCORE && db0 < G::kNDB;
  // Ring slot of tile t. One token per batch (decode): tiles start at slot 2, so that slots 0-1 can
  // stage the queries while the first two tiles land.
  auto slot = [](int t) { return (t + (NT ? 2 : 0)) % kBufs; };

  int pair = xcd_local_id(blockIdx.x, gridDim.x, nxcc);
  // One split per token: tokens in a scrambled order (pair * tok_mul mod the token count, tok_mul
  // coprime with it), so each round of workgroups mixes tokens from the whole sequence (early
  // tokens have fewer causally valid slots) and the rounds do not load queries and store outputs
  // all at the same time.
  if (nsplit == 1) pair = (int)(((long)pair * tok_mul) % (long)gridDim.x);
  // tok is a (token, head group) pair: token rtok's heads hg*H .. hg*H+H-1 (H is the group's head
  // count), so the q and out rows of tok sit at (tok * H + h) * D as for a token of H heads
  const int tok = pair / nsplit, split = pair % nsplit;
  const int rtok = tok / ngrp, hg = tok - rtok * ngrp;
  const int b = rtok / S;
  const int ntiles_all = (K + kTile - 1) / kTile;
  const int t0 = (int)(((long)split * ntiles_all) / nsplit);
  const int ntl = (int)(((long)(split + 1) * ntiles_all) / nsplit) - t0;
  const int* __restrict__ idx_tok = idx + (size_t)rtok * K;
  const __bf16* __restrict__ kv_b = (const __bf16*)kv + (size_t)(F8 ? 0 : b) * T * D;
  static_assert(!F8 || D == 512, "FP8 rows hold D = 512");
  u32x4 kv8rs = {};  // FP8: the batch's rows as a buffer resource
  // the token's slot indices as a buffer resource (score wave 0 copies them into LDS for bf16 rows)
  const u32x4 idxrs = buffer_rsrc(idx_tok, (uint32_t)((long)K * 4 < 0xFFFFFFFFl ? (long)K * 4 : 0xFFFFFFFFl));
  u32x4 kvrs = {};   // bf16: the batch's rows from the start, 4 GB reach per resource base (no range check)
  if constexpr (!F8) kvrs = buffer_rsrc(kv_b, 0xFFFFFFFFu);
  if constexpr (F8) kv8rs = buffer_rsrc((const uint8_t*)kv + (size_t)b * T * kF8Row, (uint32_t)T * kF8Row);

  // ---- score waves: queries of head blocks sw and sw+4 (B operand of S^T = K Q^T)
  constexpr int QB = SCORE ? (HB > 4 ? 2 : 1) : 1;
  const int nq = SCORE ? ((sw + 4 < HB) ? 2 : ((sw < HB) ? 1 : 0)) : 0;
  bf16x8 qreg[QB][SCORE ? G::kDSteps : 1];
  if constexpr (NT) {
    // One token per batch (decode): each score wave copies the query rows of one of its head blocks
    // at a time as whole rows (1 KB per wave instruction at D = 512) into its own 16 rows of ring
    // slots 0-1, waits for its own copies (no workgroup barrier) and reads its B operands from
    // there. Meanwhile the value waves' first two tiles land in slots 2-3. Loaded straight into the
    // operand layout (16 rows x 64 bytes per wave instruction) the queries landed 4.2 us after the
    // workgroup's start at the decode shape; staged by all waves over the whole ring, 2.6 us, but the
    // row copies then had to wait for them (FP8 decode calls 2.7 % slower than with this form).
    static_assert(64 * G::kRowStride <= 2 * G::kBufBytes, "query staging exceeds ring slots 0-1");
    if constexpr (SCORE) {
      unsigned char* const qst = &sm.kv[0][0] + sw * 16 * G::kRowStride;  // this wave's 16 staging rows
#pragma unroll
      for (int qi = 0; qi < QB; qi++) {
        const int hb = sw + 4 * qi;
        if (qi < nq) {
          for (int r = 0; r < 16; r++) {
            const int h = hb * 16 + r;
            unsigned char* dst = qst + r * G::kRowStride;
            if (h < H) {
              if (lane < G::kLanesPerRow)
                __builtin_amdgcn_global_load_lds((const void*)(q + ((size_t)tok * H + h) * D + lane * 8), (lds_void_t*)dst,
                                                 16, 0, 0);
            } else if (lane < G::kLanesPerRow) {
              *(uint4*)(dst + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
            }
          }
          wait_vm_lgkm0<0>();
        }
#pragma unroll
        for (int s = 0; s < G::kDSteps; s++) {
          bf16x8 v = {};
          if (qi < nq) v = *(const bf16x8*)(qst + l16 * G::kRowStride + 64 * s + 16 * g);
          qreg[qi][s] = v;
        }
        if (g == 0 && qi < nq) {
          sm.mref[hb * 16 + l16] = kNegInf;
          sm.lsum[hb * 16 + l16] = 0.f;
        }
        wait_lgkm0();  // operands in registers before the rows are staged again
      }
    }
  } else if constexpr (SCORE) {
    // Several tokens per batch (prefill): the queries go straight into the operand layout, beside
    // the first row copies (staging them in the ring delays those copies: prefill 1.4 % slower).
#pragma unroll
    for (int qi = 0; qi < QB; qi++) {
      const int h = (sw + 4 * qi) * 16 + l16;
#pragma unroll
      for (int s = 0; s < G::kDSteps; s++) {
        bf16x8 v = {};
        if (qi < nq && h < H) v = *(const bf16x8*)(q + ((size_t)tok * H + h) * D + 32 * s + 8 * g);
        qreg[qi][s] = v;
      }
      if (g == 0 && qi < nq) {
        sm.mref[(sw + 4 * qi) * 16 + l16] = kNegInf;
        sm.lsum[(sw + 4 * qi) * 16 + l16] = 0.f;
      }
    }
    // Let the query loads land before any row DMA is issued, so that no wait for them is
    // left inside the tile loop (it would also drain the DMA queue).
    wait_vm_lgkm0<0>();
  }

  f32x4 oacc[HB][NBX];
#pragma unroll
  for (int hb = 0; hb < HB; hb++)
#pragma unroll
    for (int db = 0; db < NBX; db++) oacc[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- row gather (value waves): value wave v owns rows 4v .. 4v+3 of every tile
  auto load_rows = [&](int tt, int (&rows)[4]) {
    const int slot0 = (t0 + tt) * kTile + sw * 4;
    if (slot0 + 4 <= K) {
#pragma unroll
      for (int r = 0; r < 4; r++) rows[r] = idx_tok[slot0 + r];
    } else {
#pragma unroll
      for (int r = 0; r < 4; r++) rows[r] = (slot0 + r < K) ? idx_tok[slot0 + r] : -1;
    }
  };
  auto issue = [&](int tt, const int (&rows)[4]) -> int {  // returns DMA instructions issued
    const int bi = slot(tt);
    unsigned vbits = 0;
    int n = 0;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int row = rows[r];
      unsigned char* dst = &sm.kv[bi][(sw * 4 + r) * G::kRowStride];
      if constexpr (F8) {
        // one instruction per row: lanes 0-35 copy its first 576 bytes (16 each); lane 36 copies
        // bytes 568-583 (the last 8 RoPE bytes once more, then the 8 scale bytes), which land
        // at slot offset 576, so the scales sit at 584-591 (a separate 4-byte copy of the scales
        // made FP8 decode calls 3 % slower). The row's start is only 8-byte aligned (584-byte
        // rows), which 16-byte buffer loads allow. The other lanes are inactive, so nothing else
        // in the slot is written. An invalid row is zero-filled when the tile is expanded.
        if (row >= 0 && row < T) {
          vbits |= 1u << r;
          n += 1;
          const uint32_t base = (uint32_t)row * kF8Row;
          const uint32_t ldst = lds_addr(dst);
          if (lane < 37) {
            const uint32_t off = base + (lane < 36 ? 16u * lane : 568u);
            if constexpr (NT) dma_lds16_nt(kv8rs, off, ldst);
            else dma_lds16(kv8rs, off, ldst);
          }
        }
      } else if (row >= 0 && row < T) {
        vbits |= 1u << r;
        n++;
        // NT (one token per batch, decode): a row serves one token only, so it is streamed (nt) and
        // does not push the queries and the split partials out of L2. Otherwise neighbouring tokens
        // share rows through L2. The copy is a raw buffer load into LDS: with the row copies in the
        // compiler's global_load_lds form, its wait-count pass no longer took LDS reads as returning
        // in order and made the score and value waves wait for every LDS read in flight before each
        // MFMA group (decode 2 %, ragged decode 4 %, prefill 1-3 % slower). The batch's rows are
        // one resource whose base moves by 4 GB per 2^kRowSeg rows (a scalar add on the high
        // address word; the row index is wave-uniform), so the 32-bit offsets never overflow.
        if (lane < G::kLanesPerRow) {
          u32x4 rs = kvrs;
          rs.y += (uint32_t)row >> G::kRowSeg;
          const uint32_t off = ((uint32_t)row & ((1u << G::kRowSeg) - 1u)) * (uint32_t)(D * 2) + 16u * (uint32_t)lane;
          if constexpr (NT) dma_lds16_nt(rs, off, lds_addr(dst));
          else dma_lds16(rs, off, lds_addr(dst));
        }
      } else if (lane < G::kLanesPerRow) {
        *(uint4*)(dst + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (lane == 0) sm.vmb[bi][sw] = (unsigned char)vbits;  // own byte: no clearing needed
    return n;
  };

  // FP8: expand this wave's 4 rows of tile tt in place from the copied bytes to bf16 rows
  // (lanes 0-55: 8 e4m3 values of dims 8l .. 8l+7 with their tile's scale; lanes 56-63: 8 RoPE
  // dims), invalid rows to zeros. All reads land before any write: the bf16 row overlaps the
  // bytes it is made from. Branch-free across lanes: every lane reads 16 bytes and its tile's
  // scale byte and converts; the RoPE lanes keep the raw bytes. Called once the tile's copies
  // have landed (this wave's own rows).
  auto expand = [&](int tt) {
    const int bi = slot(tt);
    const unsigned vbits = __builtin_amdgcn_readfirstlane((unsigned)sm.vmb[bi][sw]);
    const bool nope = lane < 56;
    const int roff = nope ? 8 * lane : kF8Nope + 16 * (lane - 56);         // source bytes in the slot
    const int woff = nope ? 16 * lane : 2 * kF8Nope + 16 * (lane - 56);    // bf16 destination
    const int soff = 584 + (nope ? (lane >> 3) : 0);                       // scale byte
    uint2 lo[4], hi[4];
    unsigned sb[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const unsigned char* slot = &sm.kv[bi][(sw * 4 + r) * G::kRowStride];
      lo[r] = *(const uint2*)(slot + roff);
      hi[r] = *(const uint2*)(slot + roff + 8);
      sb[r] = slot[soff];
    }
    wait_lgkm0();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < 4; r++) {
      unsigned char* slot = &sm.kv[bi][(sw * 4 + r) * G::kRowStride];
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (vbits & (1u << r)) {  // wave-uniform
        // 2^(s-127) as an fp32 bit pattern, in plain integer steps (no branches): s = 0 gives the
        // subnormal 2^-127 (0x00400000 is the larger of the two), s = 255 sets the quiet bit of
        // the infinity pattern (NaN)
        const unsigned bits = __builtin_elementwise_max(sb[r] << 23, 0x00400000u) | (((sb[r] + 1u) >> 8) << 22);
        const float sc = __uint_as_float(bits);
        const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo[r].x, sc, false);
        const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo[r].x, sc, true);
        const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo[r].y, sc, false);
        const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo[r].y, sc, true);
        const bf16x8 v = bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
        const uint4 cv = __builtin_bit_cast(uint4, v);
        w = nope ? cv : make_uint4(lo[r].x, lo[r].y, hi[r].x, hi[r].y);
      }
      *(uint4*)(slot + woff) = w;
    }
  };

  int rows_next[4];
  int dma_last = 0;  // DMA count of the most recently issued tile
  // Value waves start the gather of tiles 0 and 1 at once: it overlaps the query loads of the
  // score waves (each wave waits only on its own memory counter).
  if constexpr (!SCORE) {
    for (int tt = 0; tt < 2 && tt < ntl; tt++) {
      int rows[4];
      load_rows(tt, rows);
      dma_last = issue(tt, rows);
    }
    if constexpr (F8) {
      if (0 < ntl) {
        wait_vm_lgkm0_dyn(1 < ntl ? dma_last : 0);  // tile 0's copies have landed
        expand(0);
      }
    }
    if (2 < ntl) load_rows(2, rows_next);
  } else {
    // Score waves win MFMA issue arbitration over the value waves of their SIMD, so the
    // scores of a tile are ready early and the softmax runs beside the value waves' PV.
    __builtin_amdgcn_s_setprio(2);
  }

  for (int tt = 0; tt <= ntl; tt++) {
    // Tile tt's rows have landed once only the younger tile's DMAs may still be pending.
    if constexpr (SCORE && !F8) wait_vm_lgkm0<0>();  // score wave 0's index copy has landed
    else if constexpr (SCORE || F8) wait_lgkm0();  // FP8: the tile was expanded (and waited for) before
    else wait_vm_lgkm0_dyn(tt + 1 < ntl ? dma_last : 0);
    wg_barrier();  // tile tt and P(tt-1) visible; everyone is done with tile tt-2 and P(tt-2)
    // bf16 rows: score wave 0 copies tile tt+3's 32 slot indices into LDS (4 bytes per lane, waited for
    // before the next barrier), where the value waves read theirs after that barrier. With the
    // indices as scalar loads after P V, the value waves waited ~400 cycles for them every tile
    // (prefill 3 %, ragged decode 1.7 % slower; FP8 rows keep the scalar loads: their value waves
    // reach the barrier later and measured no gain).
    if constexpr (SCORE && !F8) {
      if (sw == 0 && tt + 3 < ntl && lane < 32)
        dma_lds4(idxrs, (uint32_t)((t0 + tt + 3) * kTile + lane) * 4u, lds_addr(&sm.idx[(tt + 3) & 1][0]));
    }
    // ---- prefetch tile tt+2 into the buffer freed by tile tt-2
    int dma_new = 0;  // copies issued in this iteration (tile tt+2)
    if constexpr (!SCORE) {
      if (tt + 2 < ntl) {
        if (!F8 && tt > 0) {  // tile 2's indices came in with scalar loads before the loop
          const int4 v = *(const int4*)&sm.idx[(tt + 2) & 1][4 * sw];
          const int slot0 = (t0 + tt + 2) * kTile + sw * 4;  // slots at or past K are empty
          rows_next[0] = slot0 + 0 < K ? __builtin_amdgcn_readfirstlane(v.x) : -1;
          rows_next[1] = slot0 + 1 < K ? __builtin_amdgcn_readfirstlane(v.y) : -1;
          rows_next[2] = slot0 + 2 < K ? __builtin_amdgcn_readfirstlane(v.z) : -1;
          rows_next[3] = slot0 + 3 < K ? __builtin_amdgcn_readfirstlane(v.w) : -1;
        }
        dma_last = dma_new = issue(tt + 2, rows_next);
      }
    }
    // ---- scores of tile tt (score waves)
    f32x4 sacc[QB][2];
    unsigned vm = 0u;
    if constexpr (SCORE) {
      if (tt < ntl) vm = tile_mask(sm, slot(tt));
      if (vm != 0u && nq > 0) {
        const unsigned char* buf = sm.kv[slot(tt)];
#pragma unroll
        for (int qi = 0; qi < QB; qi++) sacc[qi][0] = sacc[qi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        // K operands in the order k = 2s + jb (step s over the head dimension, 16-row block jb),
        // each feeding the MFMAs of both head blocks; four registers rotate so every LDS read
        // is issued four operands (eight MFMAs) ahead of its use. The schedule groups keep
        // the compiler from collapsing the rotation.
        const unsigned char* kb = buf + l16 * G::kRowStride + 16 * g;
        constexpr int NK = 2 * G::kDSteps;
        constexpr int KR = NK < 4 ? NK : 4;
        auto kop = [&](int k) { return *(const bf16x8*)(kb + (k & 1) * 16 * G::kRowStride + 64 * (k >> 1)); };
        bf16x8 ka[KR];
#pragma unroll
        for (int k = 0; k < KR; k++) ka[k] = kop(k);
        __builtin_amdgcn_sched_group_barrier(0x100, KR, 0);
#pragma unroll
        for (int k = 0; k < NK; k++) {
          const int st = k >> 1, jb = k & 1;
          sacc[0][jb] = mfma16x16x32(ka[k % KR], qreg[0][st], sacc[0][jb]);
          if (QB > 1) sacc[QB - 1][jb] = mfma16x16x32(ka[k % KR], qreg[QB - 1][st], sacc[QB - 1][jb]);
          __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
          if (k + KR < NK) {
            ka[k % KR] = kop(k + KR);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- online softmax of tile tt (score waves)
    if constexpr (SCORE) {
      if (tt < ntl) {
        const int par = tt & 1;
        bool any_resc = false;
        if (vm != 0u && nq > 0) {
          // Lane-dependent LDS offsets are rebuilt here from the lane id (kept opaque so the
          // compiler cannot carry them, or spill them, across the QK loop); every access
          // below is one of these two offsets plus a constant.
          unsigned ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
          asm volatile("" : "+v"(ln));
          const int lg = (int)(ln >> 4), ll = (int)(ln & 15u);
          const int off_h = (sw * 16 + ll) * 4;                       // per-head state, bytes
          const int off_p = (sw * 16 + ll) * (kPStride * 2) + 16 * lg;  // P row, bytes
          unsigned char* const hst = (unsigned char*)&sm.mref[0] + off_h;
          unsigned char* const pst = (unsigned char*)&sm.p[par][0] + off_p;
          constexpr int kHB = HP * 4;  // bytes of one per-head array
          // softmax state of this lane's heads, read first so the LDS latency overlaps the
          // masking and maximum below
          float mst[QB], lst[QB];
#pragma unroll
          for (int qi = 0; qi < QB; qi++) {
            mst[qi] = *(const float*)(hst + qi * 256);
            lst[qi] = *(const float*)(hst + kHB + qi * 256);
          }
          // validity of this lane's rows 4g+i and 16+4g+i: bits i and 16+i of vg (one shift per
          // tile, immediate masks after it)
          const unsigned vg = vm >> (4 * lg);
          // logits in log2 units, computed in place in the accumulators; empty rows masked to -inf,
          // skipped when all 32 rows hold a gathered row (every tile at the decode shape)
#pragma unroll
          for (int qi = 0; qi < QB; qi++)
#pragma unroll
            for (int jb = 0; jb < 2; jb++)
#pragma unroll
              for (int i = 0; i < 4; i++) sacc[qi][jb][i] *= scale_log2;
          if (vm != 0xFFFFFFFFu) {
#pragma unroll
            for (int qi = 0; qi < QB; qi++)
#pragma unroll
              for (int jb = 0; jb < 2; jb++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                  if (!(vg & (1u << (16 * jb + i)))) sacc[qi][jb][i] = kNegInf;
          }
#pragma unroll
          for (int qi = 0; qi < QB; qi++) {
            float tmax = kNegInf;
#pragma unroll
            for (int jb = 0; jb < 2; jb++)
#pragma unroll
              for (int i = 0; i < 4; i++) tmax = __builtin_elementwise_maximum(tmax, sacc[qi][jb][i]);
            tmax = max4_x16_x32(tmax);
            const float mold = mst[qi];
            const bool move = tmax > mold + kLazy;  // also true for the first finite maximum
            const float mnew = move ? tmax : mold;
            const float alpha = move ? exp2_fast(mold - mnew) : 1.f;  // 0 when mold = -inf
            const bool resc = move && (mold > kNegInf);
            any_resc |= resc;
            const float msub = (mnew > kNegInf) ? mnew : 0.f;  // no finite logit yet: all weights 0
            float lsum;
            // this lane's weights for rows 4g+i and 16+4g+i go to P columns 8g .. 8g+7
            bf16x2 pk[4];
#pragma unroll
            for (int jb = 0; jb < 2; jb++) {
              float pw[4];
#pragma unroll
              for (int i = 0; i < 4; i++) {
                pw[i] = exp2_fast(sacc[qi][jb][i] - msub);
                lsum = (jb == 0 && i == 0) ? pw[0] : lsum + pw[i];  // no 0 + x to start the sum
              }
              pk[2 * jb] = __builtin_convertvector((f32x2){pw[0], pw[1]}, bf16x2);
              pk[2 * jb + 1] = __builtin_convertvector((f32x2){pw[2], pw[3]}, bf16x2);
            }
            *(bf16x8*)(pst + qi * (64 * kPStride * 2)) =
                bf16x8{pk[0][0], pk[0][1], pk[1][0], pk[1][1], pk[2][0], pk[2][1], pk[3][0], pk[3][1]};
            // the row sum uses the fp32 weights; the MFMA operand is their bf16 rounding
            lsum = sum4_x16_x32(lsum);
            if (lg == 0) {
              *(float*)(hst + qi * 256) = mnew;
              *(float*)(hst + kHB + qi * 256) = lst[qi] * alpha + lsum;
              *(float*)(hst + (2 + par) * kHB + qi * 256) = resc ? alpha : 1.f;
            }
          }
        }
        // Every score wave publishes its own rescale flag for this tile (no shared writes). The
        // vote is taken with every lane active: a vote inside the lane-0 branch would see lane 0
        // (the heads of lane column 0) only.
        const bool resc_wave = __any(any_resc);
        if (lane == 0) sm.flag[par][sw] = resc_wave ? 1 : 0;
      }
    }
    // ---- P V for the previous tile (value waves)
    if constexpr (!SCORE) {
      if (tt >= 1 && pv_active) {
        const int tp = tt - 1;
        if (tile_mask(sm, slot(tp)) != 0u) pv_step<D, HB, NB>(sm, oacc, db0, tp, slot(tp), lane, g, l16);
      }
      if constexpr (F8) {
        // expand tile tt+1 for the next barrier, after P V (its copies, issued one tile ago, have
        // landed by then, once at most this iteration's copies are outstanding; before P V the
        // wait for them measured 0.5 % slower)
        if (tt + 1 < ntl) {
          wait_vm_lgkm0_dyn(dma_new);
          // the expansion is on this wave's path to the next barrier: it outranks the score
          // waves' softmax for issue while it runs
          __builtin_amdgcn_s_setprio(3);
          expand(tt + 1);
          __builtin_amdgcn_s_setprio(0);
        }
      }
      // FP8 rows: index loads of tile tt+3 go out after PV (scalar loads share the LDS wait counter,
      // so issued earlier they would hold up every LDS wait of PV).
      if constexpr (F8) {
        if (tt + 3 < ntl) load_rows(tt + 3, rows_next);
      }
    }
  }

  // Lane-dependent values of the epilogue are rebuilt from the lane id (kept opaque), so none
  // of them is carried, or spilled, across the tile loop.
  unsigned lne = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(lne));
  const int lanee = (int)lne, ge = lanee >> 4, l16e = lanee & 15;
  // Per-head output factor f of the no-split path (score waves own the heads): the sink is
  // folded in, o = O 2^(m-M) / (l 2^(m-M) + 2^(sink-M)). With splits, each split's unnormalised
  // O and its (m, l) are merged with the sink afterwards.
  if constexpr (SCORE) {
#pragma unroll
    for (int qi = 0; qi < QB; qi++) {
      if (qi >= nq) break;
      const int h = (sw + 4 * qi) * 16 + l16e;
      const float m = sm.mref[h];
      const float l = sm.lsum[h];
      float f = 0.f;
      if (nsplit == 1) {
        if (h < H) {
          const float sk = sink[hg * H + h];
          if (__builtin_isnan(sk)) {
            f = __builtin_nanf("");
          } else if (sk == __builtin_huge_valf()) {
            f = 0.f;
          } else {
            const float s2 = sk * kLog2e;
            const float M = fmaxf(m, s2);
            if (M > kNegInf) {
              const float c = (m > kNegInf) ? exp2_fast(m - M) : 0.f;
              const float L = l * c + ((s2 > kNegInf) ? exp2_fast(s2 - M) : 0.f);
              f = c / L;
            }
          }
        }
      }
      if (ge == 0) sm.fin[h] = f;
    }
  }
  wait_lgkm0();
  wg_barrier();  // every wave is past its last tile: the row ring is free for staging

  const int tid = threadIdx.x;
  if (nsplit > 1) {
    // split partial for sparse_attn_combine_kernel: the unnormalised block O in the MFMA layout
    // straight from the accumulators, and (m, l) per head. A wave owning an even number of d
    // blocks (D = 512) stores two of them per lane, [head block][d block pair][lane][4 heads of
    // block 2p, then of block 2p+1] (16 bytes per lane, 1 KB per wave store: ragged decode calls
    // 2.6 %, decode 0.3 %, FP8 decode 0.9 % faster than 8 bytes per lane); otherwise
    // [head block][d block][lane][4 heads] (8 bytes per lane).
    if constexpr (NB > 0) {
      if (pv_active) {
        __bf16* const wpart = ws_o + (size_t)pair * HP * D;
        // device-scope (sc1) stores: the partials are read by the merge kernel, possibly on another XCD
        // (decode and FP8 decode calls 0.6-1 % faster than write-back stores; nontemporal plus sc1 7 %
        // slower)
        const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc((void*)wpart, (short)0, HP * D * 2, 0x00020000);
        constexpr int kSc1 = 16;  // cache-policy bits of the store: sc1
#pragma unroll
        for (int hb = 0; hb < HB; hb++) {
          if constexpr (NB % 2 == 0) {
#pragma unroll
            for (int db = 0; db < NB; db += 2) {
              bf16x8 v;
#pragma unroll
              for (int i = 0; i < 4; i++) {
                v[i] = (__bf16)oacc[hb][db][i];
                v[4 + i] = (__bf16)oacc[hb][(db + 1) % NBX][i];
              }
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), prs,
                                                     ((hb * G::kNDB + db0 + db) * 64 + 2 * lanee) * 8, 0, kSc1);
            }
          } else {
#pragma unroll
            for (int db = 0; db < NB; db++) {
              bf16x4 v;
#pragma unroll
              for (int i = 0; i < 4; i++) v[i] = (__bf16)oacc[hb][db][i];
              *(bf16x4*)(wpart + ((hb * G::kNDB + db0 + db) * 64 + lanee) * 4) = v;
            }
          }
        }
      }
    }
    if (tid < HP) *(float2*)(ws_ml + ((size_t)pair * HP + tid) * 2) = make_float2(sm.mref[tid], sm.lsum[tid]);
    return;
  }

  // ---- no split: stage the final rows [h][D + 16] in the row ring as bf16 with the factor
  // applied, then store them with 16-byte writes
  __bf16* const stg = (__bf16*)&sm.kv[0][0];
  constexpr int kOS = D + 16;  // staged row stride (bf16): 8 banks of skew per row
  static_assert(HP * kOS * 2 <= (int)sizeof(sm.kv), "staging exceeds the ring");
  if constexpr (NB > 0) {
    if (pv_active) {
#pragma unroll
      for (int hb = 0; hb < HB; hb++) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; i++) f[i] = sm.fin[hb * 16 + 4 * ge + i];
#pragma unroll
        for (int db = 0; db < NB; db++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            stg[(hb * 16 + 4 * ge + i) * kOS + (db0 + db) * 16 + l16e] = (__bf16)(oacc[hb][db][i] * f[i]);
      }
    }
  }
  wait_lgkm0();
  wg_barrier();
  constexpr int kRC = D / 8;
  for (int c = tid; c < HP * kRC; c += kThreads) {
    const int r = c / kRC, k = c % kRC;
    // the output is not read again by the call: streamed past the caches (prefill 0.5 % faster)
    if (r < H)
      __builtin_nontemporal_store(*(const u32x4*)(&stg[r * kOS + 8 * k]), (u32x4*)(out + ((size_t)tok * H + r) * D + 8 * k));
  }
}

template <int D, int HB, bool F8, bool NT>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_kernel(
    const __bf16* __restrict__ q, const void* __restrict__ kv, const float* __restrict__ sink,
    const int* __restrict__ idx, __bf16* __restrict__ out, __bf16* __restrict__ ws_o, float* __restrict__ ws_ml,
    int S, int H, int T, int K, int nsplit, int G, int nxcc, int tok_mul, float scale_log2) {
  __shared__ __attribute__((aligned(16))) Smem<D, HB> sm;
  if (threadIdx.x < 256)  // waves 0-3
    run_split<D, HB, true, F8, NT>(sm, q, kv, sink, idx, out, ws_o, ws_ml, S, H, T, K, nsplit, G, nxcc, tok_mul,
                               scale_log2);
  else
    run_split<D, HB, false, F8, NT>(sm, q, kv, sink, idx, out, ws_o, ws_ml, S, H, T, K, nsplit, G, nxcc, tok_mul,
                                scale_log2);
}

// Merge the split partials of one (token, 16-head block) and add the sink once:
// o = sum_p 2^(m_p - M) O_p / (sum_p 2^(m_p - M) l_p + 2^(sink - M)), M the largest term, where
// split p left its unnormalised output O_p (bf16) and its reference maximum m_p (log2 units)
// and weight sum l_p.
// Grid: tokens x head blocks x DS column ranges (mapped so a token's workgroups run on the XCD
// that wrote its partials). The block's partials are 16-byte chunks of the MFMA output layout
// [d block][lane][4 heads]; every thread issues all its chunk loads of a group of up to four
// splits before it waits, then the merged block is staged in LDS and stored row by row.
// With DS = 1, 512 threads (two chunks per thread at D = 512) measured faster than 128, 256 or 1024.
// With few (token, head block) pairs (at most 320: up to 40 tokens of 128 heads) each block's 512
// columns are split over DS = 4 workgroups of 128 threads, so that more CUs pull the partials:
// decode calls 6 % faster at 8 tokens, 3-4.5 % at 12-16, 1-2 % at 20-40; at 96-128 tokens the extra
// workgroups cost 1.5-3.5 %, and DS = 2 (256 threads) measured 6-9 % slower at 24-32 tokens.
constexpr int kCombineThreads = 512;
template <int D, int HB, int DS>
__global__ __launch_bounds__(kCombineThreads) void sparse_attn_combine_kernel(const __bf16* __restrict__ ws_o,
                                                                   const float* __restrict__ ws_ml,
                                                                   const float* __restrict__ sink,
                                                                   __bf16* __restrict__ out, int H, int nsplit,
                                                                   int ngrp, int nxcc) {
  using G = Geo<D>;
  constexpr int HP = HB * 16;
  constexpr int NT = kCombineThreads / DS;             // threads of this workgroup
  constexpr int kChunks = G::kNDB * 64 * 8 / 16;       // 16-byte chunks of one partial block
  constexpr int kChunksW = kChunks / DS;               // ... of this workgroup's column range
  constexpr int kPerThread = (kChunksW + NT - 1) / NT;  // chunks per thread
  constexpr int kOutStride = D + 8;                    // bf16 per staged output row
  constexpr bool PAIR = G::kDBV % 2 == 0;              // partials stored two d blocks per lane
  static_assert(DS == 1 || (PAIR && kChunksW % 64 == 0), "column split needs whole d-block pairs");
  __shared__ float wgt[kMaxSplits * 16];
  __shared__ __attribute__((aligned(16))) __bf16 stage[16 * kOutStride];
  const int blk = xcd_local_id(blockIdx.x, gridDim.x, nxcc);
  const int tok = blk / (HB * DS), hb = (blk / DS) % HB, ds = blk % DS;
  const int t = threadIdx.x;
  const int c0 = ds * kChunksW;                        // first chunk of this workgroup's columns

  // PAIR: chunk c of a block is lane c%64 of d-block pair c/64: heads 4*(lane/16)+i, columns
  // (c/64)*32 + lane%16 and 16 more. Otherwise chunk c holds lanes 2(c%32), 2(c%32)+1 of d block
  // c/32: heads 4*(lane/16)+i, columns (c/32)*16 + lane%16 (+1 for the odd lane).
  f32x4 acc[kPerThread][2];
#pragma unroll
  for (int j = 0; j < kPerThread; j++) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weights: thread t < 16 owns head hb*16+t; its (m, l) values are loaded in one round
  float mp[kMaxSplits], lp[kMaxSplits];
  float sk = kNegInf;
  if (t < 16) {
    const int h = hb * 16 + t;
    sk = h < H ? sink[(tok % ngrp) * H + h] : kNegInf;  // head group tok % ngrp of its token
#pragma unroll
    for (int p = 0; p < kMaxSplits; p++) {
      const float2 v = p < nsplit ? *(const float2*)(ws_ml + (((size_t)tok * nsplit + p) * HP + h) * 2)
                                  : make_float2(kNegInf, 0.f);
      mp[p] = v.x;
      lp[p] = v.y;
    }
  }
  for (int p0 = 0; p0 < nsplit; p0 += 4) {
    const int np = nsplit - p0 < 4 ? nsplit - p0 : 4;
    uint4 v[4][kPerThread];
#pragma unroll
    for (int pp = 0; pp < 4; pp++) {
      if (pp < np) {
        const uint4* src = (const uint4*)(ws_o + ((size_t)(tok * nsplit + p0 + pp) * HP + hb * 16) * D);
#pragma unroll
        for (int j = 0; j < kPerThread; j++) {
          const int c = c0 + t + NT * j;
          if (c < c0 + kChunksW) v[pp][j] = src[c];
        }
      }
    }
    if (p0 == 0) {
      if (t < 16) {
        const float s2 = sk * kLog2e;
        float M = s2;
#pragma unroll
        for (int p = 0; p < kMaxSplits; p++) M = fmaxf(M, mp[p]);
        float c[kMaxSplits], L = (s2 > kNegInf && M > kNegInf) ? exp2_fast(s2 - M) : 0.f;
#pragma unroll
        for (int p = 0; p < kMaxSplits; p++) {
          c[p] = (mp[p] > kNegInf && M > kNegInf) ? exp2_fast(mp[p] - M) : 0.f;
          L += c[p] * lp[p];
        }
#pragma unroll
        for (int p = 0; p < kMaxSplits; p++) {
          if (p >= nsplit) break;
          float w = L > 0.f ? c[p] / L : 0.f;
          if (__builtin_isnan(sk)) w = __builtin_nanf("");
          else if (sk == __builtin_huge_valf()) w = 0.f;
          wgt[p * 16 + t] = w;
        }
      }
      __syncthreads();  // weights ready; the chunk loads above are already in flight
    }
#pragma unroll
    for (int pp = 0; pp < 4; pp++) {
      if (pp < np) {
#pragma unroll
        for (int j = 0; j < kPerThread; j++) {
          const int c = c0 + t + NT * j;
          if (c >= c0 + kChunksW) continue;
          const int hq = PAIR ? 4 * ((c & 63) >> 4) : 4 * ((2 * (c & 31)) >> 4);
          const bf16x8 x = __builtin_bit_cast(bf16x8, v[pp][j]);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float w = wgt[(p0 + pp) * 16 + hq + i];
            acc[j][0][i] += (float)x[i] * w;
            acc[j][1][i] += (float)x[4 + i] * w;
          }
        }
      }
    }
  }
  // stage the merged 16 x D block as bf16 rows, then store each row with 16-byte writes
#pragma unroll
  for (int j = 0; j < kPerThread; j++) {
    const int c = c0 + t + NT * j;
    if (c >= c0 + kChunksW) continue;
    if constexpr (PAIR) {
      const int ln = c & 63, col = (c >> 6) * 32 + (ln & 15), hq = 4 * (ln >> 4);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        stage[(hq + i) * kOutStride + col] = (__bf16)acc[j][0][i];
        stage[(hq + i) * kOutStride + col + 16] = (__bf16)acc[j][1][i];
      }
    } else {
      const int lane0 = 2 * (c & 31), col = (c >> 5) * 16 + (lane0 & 15), hq = 4 * (lane0 >> 4);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const bf16x2 pr = __builtin_convertvector((f32x2){acc[j][0][i], acc[j][1][i]}, bf16x2);
        *(bf16x2*)(&stage[(hq + i) * kOutStride + col]) = pr;
      }
    }
  }
  __syncthreads();
  // The output is not read again by this call, so it is stored nontemporally (streamed past the
  // caches): decode calls 0.7-2 % and FP8 decode calls 1.6 % faster. Marking the partial loads
  // the same way made ragged decode calls 5 % slower.
  constexpr int kRowChunks = D / 8 / DS;  // 16-byte chunks per output row (this workgroup's columns)
  for (int c = t; c < 16 * kRowChunks; c += NT) {
    const int r = c / kRowChunks, k = ds * kRowChunks + c % kRowChunks;
    const int h = hb * 16 + r;
    if (h < H)
      __builtin_nontemporal_store(*(const u32x4*)(&stage[r * kOutStride + 8 * k]),
                                  (u32x4*)(out + ((size_t)tok * H + h) * D + 8 * k));
  }
}

// Workspace of a split call: unnormalised bf16 partials [pair][HP*D] (MFMA layout), then fp32
// (m, l) [pair][HP][2] (256-byte aligned parts). Pure scratch: contents on entry do not matter.
struct WsLayout {
  size_t ml, total;
};
static inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
static WsLayout ws_layout(int64_t ntok, int64_t HB, int64_t D, int nsplit) {
  WsLayout w{};
  if (nsplit <= 1) return w;
  const size_t pairs = (size_t)ntok * nsplit, hp = (size_t)HB * 16;
  w.ml = round256(pairs * hp * D * 2);
  w.total = w.ml + round256(pairs * hp * 8);
  return w;
}

// XCDs of the current device (workgroups are dispatched round-robin over them).
static int device_xccs() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (cache[dev] == 0) {
    int v = 1;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || v < 1) v = 1;
    cache[dev] = v;
  }
  return cache[dev];
}

// A multiplier near 0.618 n that is coprime with n (so pair -> pair * m mod n is a bijection).
static int token_multiplier(int64_t n) {
  if (n <= 2) return 1;
  auto gcd = [](int64_t a, int64_t b) { while (b) { const int64_t t = a % b; a = b; b = t; } return a; };
  for (int64_t m = (int64_t)(0.6180339887 * (double)n) | 1; m < n; m += 2)
    if (gcd(m, n) == 1) return (int)m;
  return 1;
}

template <int D, int HB, bool F8>
static hipError_t launch_sparse(const void* q, const void* kv, const float* sink, const int32_t* idx, void* out,
                                int64_t B, int64_t S, int64_t H, int64_t T, int64_t K, float scale, int nsplit,
                                void* ws, int phases, int G, hipStream_t stream) {
  // G head groups: each token is G (token, head group) pairs of H / G heads, all of them "tokens" below
  const int64_t ntok = B * S * G;
  H /= G;
  const int64_t n = ntok * nsplit;
  const WsLayout L = ws_layout(ntok, HB, D, nsplit);
  __bf16* ws_o = nsplit > 1 ? (__bf16*)ws : nullptr;
  float* ws_ml = nsplit > 1 ? (float*)((char*)ws + L.ml) : nullptr;
  const int nxcc = device_xccs();
  if (phases & 1) {
    // one token per batch: the gathered rows are streamed (see run_split)
    auto kern = S == 1 ? sparse_attn_kernel<D, HB, F8, true> : sparse_attn_kernel<D, HB, F8, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)n), dim3(kThreads), 0, stream, (const __bf16*)q, kv, sink, idx,
                       (__bf16*)out, ws_o, ws_ml, (int)S, (int)H, (int)T, (int)K, nsplit, G, nxcc,
                       token_multiplier(n), scale * kLog2e);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nsplit == 1 || !(phases & 2)) return hipSuccess;
  // column split of the merge: more workgroups when there are few (token, head block) pairs
  const int64_t pairs = ntok * HB;
  if constexpr (D == 512) {
    if (pairs <= 320) {
      hipLaunchKernelGGL((sparse_attn_combine_kernel<D, HB, 4>), dim3((unsigned)(pairs * 4)), dim3(kCombineThreads / 4),
                         0, stream, ws_o, ws_ml, sink, (__bf16*)out, (int)H, nsplit, G, nxcc);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((sparse_attn_combine_kernel<D, HB, 1>), dim3((unsigned)pairs), dim3(kCombineThreads), 0, stream,
                     ws_o, ws_ml, sink, (__bf16*)out, (int)H, nsplit, G, nxcc);
  return hipGetLastError();
}

}  // namespace sa

// Head blocks (16 heads each) instantiated for H heads.
extern "C" int sa_internal_head_blocks(int64_t H) {
  const int hb = (int)((H + 15) / 16);
  return hb <= 2 ? hb : (hb <= 4 ? 4 : 8);
}

// phases: bit 0 = the main kernel, bit 1 = the merge of the split partials (if any)
// fp8: kv holds FP8 rows of 584 bytes (D = 512)
extern "C" int sa_internal_launch_sparse(const void* q, const void* kv, const float* sink, const int32_t* idx,
                                         void* out, int64_t B, int64_t S, int64_t H, int64_t D, int64_t T, int64_t K,
                                         float scale, int nsplit, void* ws, int phases, int fp8, int G,
                                         void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (G < 1 || H % G != 0) return 1;
  const int hb = sa_internal_head_blocks(H / G);
  hipError_t e;
#define SA_CASE(DD, HBB) \
  e = sa::launch_sparse<DD, HBB, false>(q, kv, sink, idx, out, B, S, H, T, K, scale, nsplit, ws, phases, G, st)
#define SA_CASE8(HBB) \
  e = sa::launch_sparse<512, HBB, true>(q, kv, sink, idx, out, B, S, H, T, K, scale, nsplit, ws, phases, G, st)
  if (fp8) {
    if (D != 512) return 2;
    if (hb == 1) SA_CASE8(1); else if (hb == 2) SA_CASE8(2); else if (hb == 4) SA_CASE8(4); else SA_CASE8(8);
  } else if (D == 512) {
    if (hb == 1) SA_CASE(512, 1); else if (hb == 2) SA_CASE(512, 2); else if (hb == 4) SA_CASE(512, 4); else SA_CASE(512, 8);
  } else {
    if (hb == 1) SA_CASE(64, 1); else if (hb == 2) SA_CASE(64, 2); else if (hb == 4) SA_CASE(64, 4); else SA_CASE(64, 8);
  }
#undef SA_CASE
#undef SA_CASE8
  return e == hipSuccess ? 0 : 1;
}

// Workspace bytes of a split call (see WsLayout).
extern "C" size_t sa_internal_sparse_ws_bytes(int64_t ntok, int64_t H, int64_t D, int nsplit) {
  return sa::ws_layout(ntok, sa_internal_head_blocks(H), D, nsplit).total;
}

// ---- Scratch of the allocation-free entry point (sparse_attn_fwd_noalloc): the split partials of
// one call live in this file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it only stands in for the
// symbol): each device's address is looked up once, with that device current, and cached.
namespace {
constexpr size_t kScratchBytes = (size_t)40 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];
}  // namespace

extern "C" size_t sa_internal_scratch_bytes(void) { return kScratchBytes; }

// Device address of the current device's scratch array (0 on success).
extern "C" int sa_internal_scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return 1;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}
