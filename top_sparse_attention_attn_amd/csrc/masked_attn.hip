// Dense attention restricted by a bit-packed key mask (the masked-MHA form), on gfx950.
//
// What is computed (prhub summaries of vLLM PR #48770 and PR #52217): for each query
// row, softmax over the scaled dot products with the keys whose mask bit is set, applied
// to the values; the mask row (b, q) is shared by all heads; no sink. The mask is read
// four words (128 keys) per query and 16-byte load; a 4-byte-load variant exists only as
// the control for measuring what the wide load saves, and gives identical results.
// Chunked-context form (offset_dense_mask_mod in the PR #48770 summary): k and v are one
// chunk of a longer context, and chunk key j is mask key key_start + j, key_start being the
// reserved last word of query row 0 of the batch; keys at or past that word are not
// visible. A chunk tile then straddles up to three mask words at any bit offset: the value
// waves copy three words per query with 4-byte loads and the score waves funnel-shift them
// (v_alignbit) into the tile's 64 bits.
//
// Decomposition: one workgroup of 8 waves per (batch, head, 128 queries), 64-key tiles. All waves
// do the same work: wave w owns 32 queries (quarter w & 3) and one 32-key half (w >> 2) of every
// tile, and computes S^T = K Q^T with its queries in registers (MFMA 16x16x32 bf16), the mask,
// an online softmax over its key half (own lazily moved reference maximum and row sum), and
// O += P V with the weights kept in registers (a lane's 8 logits of a query are exactly its P
// operand of the P V MFMA) and V read with the transposing LDS read. With two such waves per
// SIMD, one wave's softmax (VALU work) runs beside the other's MFMAs. The two key halves are two
// independent softmax splits of the keys, merged once per query through LDS after the last tile
// (o = (2^(m0-M) O0 + 2^(m1-M) O1) / (2^(m0-M) l0 + 2^(m1-M) l1), M = max(m0, m1)).
// The waves share the copies of the next key/value tile and its mask words from HBM into LDS:
// buffer loads that write LDS directly, the padded LDS tile filled as one contiguous byte range,
// 64 lanes x 16 bytes per load: a lane whose 16 bytes fall in a row's padding, or in a row past
// KV, gets an offset beyond the buffer's range, so the hardware reads nothing for it (44 loads
// per tile). They are waited for only at the next tile's barrier. Issuing such a load holds the
// issuing wave, so the key-half-1 waves issue the K copies (and the mask words) while the
// key-half-0 wave of each SIMD starts its MFMAs, and issues the V copies after them: the two waves
// of a SIMD then run out of phase.
// An L2 prefetch of later tiles cost more in issue than it saved.
// The row strides (416 and 288 bytes) and the row order of the transposed reads were chosen
// with the LDS bank-conflict counter. One barrier per tile.
#include "common.h"

namespace sa {

namespace masked {

constexpr int kQT = 128;  // queries per workgroup
constexpr int kKT = 64;   // keys per tile
constexpr int kThreads = 512;
constexpr uint32_t kOob = 0x80000000u;  // buffer offset beyond every range used here

template <int DQK, int DV>
struct Smem {
  static constexpr int KS = DQK * 2 + 32;  // K row stride (bytes)
  static constexpr int VS = DV * 2 + 32;   // V row stride (bytes)
  unsigned char k[2][kKT * KS];            // K tiles t (in use), t+1 (being copied)
  unsigned char v[2][kKT * VS];            // V tiles t (in use), t+1 (being copied)
  uint32_t mw[2][kQT * 4];                 // mask words: [chunk parity][query][4], or [tile parity][query][2]
  float alpha[8][2][16];                   // per wave: rescale factor per query of a moved reference
  float mref[2][kQT];                      // per key half: final reference maximum per query
  float lsum[2][kQT];                      // per key half: final weight sum per query
  float fin[2][kQT];                       // per key half: output factor per query
};

}  // namespace masked

// POS: the scale (scale_log2) is positive and finite. Then a query's tile maximum is taken over
// the raw scores (masked to -inf) and scaled once, and each weight is exp2(fma(s, scale_log2, -m)):
// no per-score multiply and subtract. Otherwise every score is scaled first.
// DENSE: no mask (every key visible); the scores of a tile inside the keys need no select.
template <int DQK, int DV, int MASKBITS, bool OFFSET, bool POS, bool DENSE>
__global__ __launch_bounds__(masked::kThreads, 1) void masked_attn_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const uint32_t* __restrict__ mask, __bf16* __restrict__ out, float* __restrict__ lse, int Q, int KV, int H,
    int padded_q, int words, int nxcc, float scale_log2) {
  using namespace masked;
  using SM = Smem<DQK, DV>;
  constexpr int KS = SM::KS, VS = SM::VS;
  constexpr int DSTEPS = DQK / 32;  // QK steps over the head dimension
  constexpr int NDB = DV / 16;      // PV output column blocks
  constexpr int KLANES = DQK / 8, VLANES = DV / 8;  // 16-byte chunks per row
  constexpr int QB = 2;             // 16-query blocks per wave (32 queries)
  static_assert(KLANES <= 64 && VLANES <= 64 && DQK % 32 == 0 && DV % 16 == 0, "head dims");
  __shared__ __attribute__((aligned(16))) SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int qq = wave & 3, kh = wave >> 2;  // query quarter (32 queries) and key half (32 keys of a tile)

  const int nqt = (Q + kQT - 1) / kQT;
  const int wg = xcd_local_id(blockIdx.x, gridDim.x, nxcc);
  const int qt = wg % nqt;
  const int bh = wg / nqt;
  const int h = bh % H, b = bh / H;
  const int qbase = qt * kQT + qq * 32;  // first query of this wave's quarter
  const int nkt = (KV + kKT - 1) / kKT;

  // chunked-context form: the clamped start and the first position past the bit words
  uint32_t ksc = 0, pmax = 0;
  if constexpr (OFFSET) {
    pmax = 32u * (uint32_t)(words - 1);
    const uint32_t ks = mask[(size_t)b * padded_q * words + (words - 1)];
    ksc = ks < pmax ? ks : pmax;
  }

  // ---- queries (B operand of QK), softmax state of this key half, output accumulators
  // O[query 4g+i of block qb][column 16 db + l16] of this key half
  bf16x8 qreg[QB][DSTEPS];
  bool qlive[QB];
  float m_ref[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int qr = qbase + 16 * qb + l16;
    qlive[qb] = qr < Q;
    m_ref[qb] = kNegInf;
    l_part[qb] = 0.f;
#pragma unroll
    for (int s = 0; s < DSTEPS; s++) {
      bf16x8 z = {};
      qreg[qb][s] = qlive[qb] ? *(const bf16x8*)(q + (((size_t)b * Q + qr) * H + h) * DQK + 32 * s + 8 * g) : z;
    }
  }
  f32x4 oacc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++)
#pragma unroll
    for (int db = 0; db < NDB; db++) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tile copies, shared by all 8 waves: the K tile in LDS is KCH 16-byte chunks per row (KLANES
  // of data, then padding), 64 rows: KCH loads of 64 chunks each; V likewise with VCH. Each load
  // belongs to one wave (below); a lane's byte offset is taken relative to row 0 of the tile (head
  // h), kOob for a padding chunk. The offsets do not depend on the tile: each wave computes its
  // own once and the tile only moves the buffer's base.
  constexpr int KCH = KS / 16, VCH = VS / 16, KM = (KCH + 3) / 4, VM = (VCH + 3) / 4;
  // The key-half-1 waves (4-7) issue the K copies and the mask words right after the barrier (load n
  // of K on wave 4 + n % 4); the key-half-0 waves, which have issue priority, start their MFMAs at
  // once and issue the V copies after their QK (load n of V on wave n % 4). Issuing an LDS-DMA load
  // holds the issuing wave, so the two waves of a SIMD then run out of phase. Measured per call:
  // copies spread over all 8 waves at the barrier (at most 6 per wave) 3 % slower, all copies on
  // key half 1 at the barrier 0.8 % slower, K on one half and V on the other both at the barrier
  // 2 % slower, the V copies after key half 0's softmax 1 % slower.
  const int wk = wave & 3, wvv = wave & 3;  // this wave's first K / V load
  uint32_t koffs[KM], voffs[VM];
#pragma unroll
  for (int m = 0; m < KM; m++) {
    const int c = 64 * (wk + 4 * m) + lane, r = c / KCH, col = c % KCH;
    koffs[m] = col < KLANES ? (uint32_t)(r * H * DQK * 2 + col * 16) : kOob;
  }
#pragma unroll
  for (int m = 0; m < VM; m++) {
    const int c = 64 * (wvv + 4 * m) + lane, r = c / VCH, col = c % VCH;
    voffs[m] = col < VLANES ? (uint32_t)(r * H * DV * 2 + col * 16) : kOob;
  }
  auto gather = [&](int t, int part) {
    // rows t*kKT + r with r < nv are in range; the range ends inside row nv's first byte
    const int nv = min(KV - t * kKT, kKT);
    const size_t row0 = ((size_t)b * KV + (size_t)t * kKT) * H + h;
    const u32x4 kr = buffer_rsrc(k + row0 * DQK, (uint32_t)(((nv - 1) * H + 1) * DQK * 2));
    const u32x4 vr = buffer_rsrc(v + row0 * DV, (uint32_t)(((nv - 1) * H + 1) * DV * 2));
    const uint32_t kd = lds_addr(sm.k[t & 1]), vd = lds_addr(sm.v[t & 1]);
#pragma unroll
    for (int m = 0; m < KM; m++)
      if (part == 0 && wk + 4 * m < KCH) dma_lds16(kr, koffs[m], kd + 1024 * (wk + 4 * m));
#pragma unroll
    for (int m = 0; m < VM; m++)
      if (part == 1 && wvv + 4 * m < VCH) dma_lds16(vr, voffs[m], vd + 1024 * (wvv + 4 * m));
  };

  // Mask copy for tile t, by waves 4-7 (pw = 0..3): the wide form copies the 4 words of keys
  // [128 c, 128 c + 128) of all kQT queries at the even tile t = 2c (two 16-byte loads, by waves
  // 4 and 5), into sm.mw[c & 1][query][4]; the control form copies the 2 words of tile t (four
  // 4-byte loads) into sm.mw[t & 1][query][2]; the chunked form copies words w0 .. w0 + 3 of mask
  // position 64 t + key_start (eight 4-byte loads) into sm.mw[t & 1][query][4]. Rows past
  // padded_q read nothing.
  const int q0 = qt * kQT;
  // the mask copy's lane offsets, tile independent (waves 4-7; the chunked form copies two
  // groups of 64 words per wave, i = pw and pw + 4)
  uint32_t moff[2] = {0u, 0u};
  if (wave >= 4) {
    const int pw = wave - 4;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      if constexpr (OFFSET) {
        const int d = 64 * (pw + 4 * u) + lane;
        moff[u] = (uint32_t)((d >> 2) * words + (d & 3)) * 4u;
      } else if constexpr (MASKBITS == 128) {
        moff[u] = (uint32_t)((64 * pw + lane) * words * 4);
      } else {
        const int d = 64 * pw + lane;
        moff[u] = (uint32_t)((d >> 1) * words * 4 + (d & 1) * 4);
      }
    }
  }
  auto mask_copy = [&](int t) {
    if (mask == nullptr || wave < 4) return;
    const int pw = wave - 4;
    const u32x4 mr = buffer_rsrc(mask + ((size_t)b * padded_q + q0) * words,
                                 (uint32_t)(min(kQT, padded_q - q0) * words * 4));
    if constexpr (OFFSET) {
      const uint32_t w0 = (64u * (uint32_t)t + ksc) >> 5;
#pragma unroll
      for (int u = 0; u < 2; u++) dma_lds4(mr, moff[u] + w0 * 4u, lds_addr(sm.mw[t & 1]) + 256 * (pw + 4 * u));
    } else if constexpr (MASKBITS == 128) {
      if ((t & 1) == 0 && pw < 2)
        dma_lds16(mr, moff[0] + (uint32_t)(t >> 1) * 16u, lds_addr(sm.mw[(t >> 1) & 1]) + 1024 * pw);
    } else {
      dma_lds4(mr, moff[0] + (uint32_t)t * 8u, lds_addr(sm.mw[t & 1]) + 256 * pw);
    }
  };

  // The tiles start zeroed: if a skipped (out-of-range) chunk leaves LDS untouched, the rows past
  // KV still hold finite values, which the zero weights of their masked keys then cancel.
  {
    uint4* z = (uint4*)&sm.k[0][0];
    constexpr int NZ = (int)((sizeof(sm.k) + sizeof(sm.v)) / 16);
    static_assert(offsetof(SM, v) == sizeof(SM::k), "k and v tiles are contiguous");
    for (int i = tid; i < NZ; i += kThreads) z[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  wait_lgkm0();
  wg_barrier();
  if (nkt > 0) {
    gather(0, kh == 1 ? 0 : 1);  // K by key half 1, V by key half 0
    mask_copy(0);
  }
  // The two waves of a SIMD (the key halves of one query quarter) would otherwise run each phase
  // (QK MFMAs, softmax VALU work, P V MFMAs) at the same time; the key-half-0 wave gets issue
  // priority, so it runs ahead and each wave's softmax lands beside the other's MFMAs.
  if (kh == 0) __builtin_amdgcn_s_setprio(2);

  for (int t = 0; t < nkt; t++) {
    wait_vm_lgkm0<0>();  // this wave's copies of tile t have landed
    wg_barrier();        // tile t visible; everyone is done with tile t-1's buffers
    if (t + 1 < nkt) {
      if (kh == 1) gather(t + 1, 0);
      mask_copy(t + 1);
    }
    const int par = t & 1;
    // this tile's mask word (32 keys of this key half) per query block
    uint32_t mwd[QB];
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      const int ql = qq * 32 + 16 * qb + l16;
      uint32_t wv;
      if constexpr (OFFSET) {
        // bits of positions p0 + 32 kh .. p0 + 32 kh + 31, none at or past pmax
        const uint4 x = *(const uint4*)&sm.mw[par][ql * 4];
        const uint32_t p0 = 64u * (uint32_t)t + ksc, sh = p0 & 31u;
        const int rem = (int)pmax - (int)p0 - 32 * kh;
        const uint32_t lim = rem >= 32 ? ~0u : (rem > 0 ? (1u << rem) - 1u : 0u);
        wv = (kh == 0 ? __builtin_amdgcn_alignbit(x.y, x.x, sh) : __builtin_amdgcn_alignbit(x.z, x.y, sh)) & lim;
      } else if (mask == nullptr) {
        wv = ~0u;
      } else {
        wv = MASKBITS == 128 ? sm.mw[(t >> 1) & 1][ql * 4 + 2 * (t & 1) + kh] : sm.mw[par][ql * 2 + kh];
      }
      mwd[qb] = qlive[qb] ? wv : 0u;
    }
    // keys past KV (last tile only)
    const int nvalid = KV - t * kKT - 32 * kh;
    const uint32_t kvm = nvalid >= 32 ? ~0u : (nvalid > 0 ? ((1u << nvalid) - 1u) : 0u);

    // ---- S^T = K Q^T of this key half: 2 key blocks x 2 query blocks, each K operand feeding both
    const unsigned char* kb = sm.k[par] + (32 * kh + l16) * KS + 16 * g;
    f32x4 sacc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; qb++) sacc[qb][0] = sacc[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NK = 2 * DSTEPS;  // K operands: (key block, step) pairs
    constexpr int KR = 4;           // K operands in flight
    auto kop = [&](int n) { return *(const bf16x8*)(kb + (n % 2) * 16 * KS + 64 * (n / 2)); };
    bf16x8 ka[KR];
#pragma unroll
    for (int n = 0; n < KR; n++) ka[n] = kop(n);
    __builtin_amdgcn_sched_group_barrier(0x100, KR, 0);
#pragma unroll
    for (int n = 0; n < NK; n++) {
      const int jb = n % 2, st = n / 2;
#pragma unroll
      for (int qb = 0; qb < QB; qb++) sacc[qb][jb] = mfma16x16x32(ka[n % KR], qreg[qb][st], sacc[qb][jb]);
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      if (n + KR < NK) {
        ka[n % KR] = kop(n + KR);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kh == 0 && t + 1 < nkt) gather(t + 1, 1);

    // ---- online softmax per query block over this key half; lane holds keys 16 jb + 4 g + i of
    // query l16, and packs its 8 weights as its own P operand of the P V MFMA (k index 8g+i =
    // key 4g + i for i < 4, 16 + 4g + i - 4 for i >= 4), so P never goes through LDS
    bf16x8 pop[QB];
    bool any_resc = false;
    // No mask and a tile inside the keys: every key of the tile is visible (queries past Q are
    // never stored), so the scores need no select.
    const bool all_vis = DENSE && nvalid >= 32;
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      const uint32_t vg = (mwd[qb] & kvm) >> (4 * g);
      float tmax = kNegInf;
      if (all_vis) {
#pragma unroll
        for (int jb = 0; jb < 2; jb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            if constexpr (!POS) sacc[qb][jb][i] *= scale_log2;
            tmax = __builtin_elementwise_maximum(tmax, sacc[qb][jb][i]);
          }
      } else {
#pragma unroll
        for (int jb = 0; jb < 2; jb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            // all ones if the key is visible, else zero: the score (raw if POS, else scaled) or
            // -inf by one bit select
            const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)vg, 16 * jb + i, 1);
            const float sv = POS ? sacc[qb][jb][i] : sacc[qb][jb][i] * scale_log2;
            const float x = __uint_as_float((sel & __float_as_uint(sv)) | (~sel & 0xff800000u));
            sacc[qb][jb][i] = x;
            tmax = __builtin_elementwise_maximum(tmax, x);
          }
      }
      tmax = max4_x16_x32(tmax);
      if constexpr (POS) tmax *= scale_log2;  // the maximum of the scaled scores
      const float mold = m_ref[qb];
      const bool move = tmax > mold + 8.0f;  // also true for the first finite maximum
      const float mnew = move ? tmax : mold;
      const float alpha = move ? exp2_fast(mold - mnew) : 1.f;  // 0 when mold = -inf
      const bool resc = move && (mold > kNegInf);
      any_resc |= resc;
      m_ref[qb] = mnew;
      const float msub = (mnew > kNegInf) ? mnew : 0.f;  // no visible key yet: all weights 0
      float lsum;
      bf16x2 pk[4];
#pragma unroll
      for (int hf = 0; hf < 2; hf++) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          pv[i] = exp2_fast(POS ? __builtin_fmaf(sacc[qb][hf][i], scale_log2, -msub) : sacc[qb][hf][i] - msub);
          lsum = (hf == 0 && i == 0) ? pv[0] : lsum + pv[i];
        }
        pk[2 * hf] = __builtin_convertvector((f32x2){pv[0], pv[1]}, bf16x2);
        pk[2 * hf + 1] = __builtin_convertvector((f32x2){pv[2], pv[3]}, bf16x2);
      }
      pop[qb] = bf16x8{pk[0][0], pk[0][1], pk[1][0], pk[1][1], pk[2][0], pk[2][1], pk[3][0], pk[3][1]};
      l_part[qb] = l_part[qb] * alpha + lsum;
      sm.alpha[wave][qb][l16] = resc ? alpha : 1.f;  // the 4 lanes of a query agree
    }
    // a moved reference rescales this wave's accumulators; the accumulator lane of query 4g+i
    // reads that query's factor back from LDS (this wave's own area: no barrier needed)
    if (__any(any_resc)) {
      wait_lgkm0();
#pragma unroll
      for (int qb = 0; qb < QB; qb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float a = sm.alpha[wave][qb][4 * g + i];
#pragma unroll
          for (int db = 0; db < NDB; db++) oacc[qb][db][i] *= a;
        }
    }

    // ---- O += P V of this key half: V operands with the transposing read, each feeding both
    // query blocks
    const int r4 = (lane >> 2) & 3, c4 = lane & 3;
    const unsigned char* vk = sm.v[par] + (32 * kh + 4 * g + r4) * VS + 8 * c4;
#pragma unroll
    for (int db = 0; db < NDB; db++) {
      const bf16x8 bv = concat_tr(lds_read_tr16(vk + 32 * db), lds_read_tr16(vk + 16 * VS + 32 * db));
#pragma unroll
      for (int qb = 0; qb < QB; qb++) oacc[qb][db] = mfma16x16x32(pop[qb], bv, oacc[qb][db]);
    }
  }

  // ---- merge the two key halves and store. Every wave publishes each query's reference maximum
  // and weight sum of its key half; each query's factors f_kh = 2^(m_kh - M) / L follow,
  // L = sum over the halves of 2^(m_kh - M) l_kh, M = max(m_0, m_1) (f = 0 without any visible
  // key). Waves of key half 1 leave f_1 O_1 in LDS, those of key half 0 add f_0 O_0, round once
  // and store (queries past Q are not written).
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const float l = sum4_x16_x32(l_part[qb]);
    sm.mref[kh][qq * 32 + 16 * qb + l16] = m_ref[qb];  // the 4 lanes of a query agree
    sm.lsum[kh][qq * 32 + 16 * qb + l16] = l;
  }
  wait_vm_lgkm0<0>();
  wg_barrier();
  if (tid < kQT) {
    const float m0 = sm.mref[0][tid], m1 = sm.mref[1][tid];
    const float M = __builtin_elementwise_maximum(m0, m1);
    const float c0 = m0 > kNegInf ? exp2_fast(m0 - M) : 0.f, c1 = m1 > kNegInf ? exp2_fast(m1 - M) : 0.f;
    const float L = c0 * sm.lsum[0][tid] + c1 * sm.lsum[1][tid];
    sm.fin[0][tid] = L > 0.f ? c0 / L : 0.f;
    sm.fin[1][tid] = L > 0.f ? c1 / L : 0.f;
    // log-sum-exp of the query's scaled logits (natural log; -inf without any visible key):
    // sum_j 2^(y_j) = L 2^M with y in log2 units
    const int qo = qt * kQT + tid;
    if (lse != nullptr && qo < Q) lse[((size_t)b * Q + qo) * H + h] = L > 0.f ? (M + __builtin_log2f(L)) * kLn2 : kNegInf;
  }
  wait_lgkm0();
  wg_barrier();  // factors ready; every wave is past its last tile, so the tile buffers are free
  // f_1 O_1 of query quarter qq, in the accumulator layout [qb][db][lane] (fp32), over the tile buffers
  f32x4* const xch = (f32x4*)&sm.k[0][0];
  static_assert(4 * QB * NDB * 64 * 16 <= (int)(sizeof(SM::k) + sizeof(SM::v)), "merge exceeds the tile buffers");
  if (kh == 1) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float f = sm.fin[1][qq * 32 + 16 * qb + 4 * g + i];
#pragma unroll
        for (int db = 0; db < NDB; db++) oacc[qb][db][i] *= f;
      }
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
#pragma unroll
      for (int db = 0; db < NDB; db++) xch[((qq * QB + qb) * NDB + db) * 64 + lane] = oacc[qb][db];
  }
  wait_lgkm0();
  wg_barrier();
  if (kh == 0) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int ql = 16 * qb + 4 * g + i;
        const int qo = qbase + ql;
        const float f = sm.fin[0][qq * 32 + ql];
        __bf16* orow = out + (((size_t)b * Q + qo) * H + h) * DV + l16;
#pragma unroll
        for (int db = 0; db < NDB; db++) {
          const float o = __builtin_fmaf(oacc[qb][db][i], f, xch[((qq * QB + qb) * NDB + db) * 64 + lane][i]);
          if (qo < Q) orow[db * 16] = (__bf16)o;
        }
      }
  }
}

// XCDs of the current device (workgroups are dispatched round-robin over them).
static int masked_device_xccs() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (cache[dev] == 0) {
    int x = 1;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x < 1) x = 1;
    cache[dev] = x;
  }
  return cache[dev];
}

}  // namespace sa

extern "C" int sa_internal_launch_masked(const void* q, const void* k, const void* v, const uint32_t* mask, void* out,
                                         float* lse, int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk,
                                         int64_t Dv, int64_t padded_q, int64_t words, float scale, int mask_load_bits,
                                         int offset, void* stream) {
  const int64_t nqt = (Q + sa::masked::kQT - 1) / sa::masked::kQT;
  const dim3 grid((unsigned)(B * H * nqt));
  const float sl2 = scale * sa::kLog2e;
  if (Dqk != 192 || Dv != 128) return 2;
  const int nxcc = sa::masked_device_xccs();
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(sa::masked::kThreads), 0, (hipStream_t)stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, mask, (__bf16*)out, lse, (int)Q, (int)KV, (int)H, (int)padded_q,
                       (int)words, nxcc, sl2);
  };
  const bool pos = sl2 > 0.f && sl2 < __builtin_huge_valf();
  if (offset) {
    if (pos) launch(sa::masked_attn_kernel<192, 128, 128, true, true, false>);
    else launch(sa::masked_attn_kernel<192, 128, 128, true, false, false>);
  } else if (mask == nullptr) {
    if (pos) launch(sa::masked_attn_kernel<192, 128, 128, false, true, true>);
    else launch(sa::masked_attn_kernel<192, 128, 128, false, false, true>);
  } else if (mask_load_bits == 32) {
    if (pos) launch(sa::masked_attn_kernel<192, 128, 32, false, true, false>);
    else launch(sa::masked_attn_kernel<192, 128, 32, false, false, false>);
  } else {
    if (pos) launch(sa::masked_attn_kernel<192, 128, 128, false, true, false>);
    else launch(sa::masked_attn_kernel<192, 128, 128, false, false, false>);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
