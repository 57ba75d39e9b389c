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
// Decomposition: one workgroup of 8 waves per (batch, head, 128 queries), in two roles that
// run one 64-key tile apart, as in the sparse kernel. Each wave owns 64 queries (one query half)
// and one 32-key half of every tile, so each K and V element is read from LDS twice per 128
// queries (once per query half), and every K or V operand read feeds four MFMAs:
//  * score waves 0-3 (query half w & 1, key half w >> 1): S^T = K Q^T with the 64 queries in
//    registers (MFMA 16x16x32 bf16), the mask, and an online softmax over their key half only
//    (its own lazily moved reference maximum and row sum); the weights go to LDS in exactly the
//    layout the PV MFMA reads them (one 16-byte chunk per lane), rare reference moves as
//    per-query factors;
//  * value waves 4-7 (the same query and key halves): they copy the next key/value tile and the
//    mask words it needs from HBM into LDS, and add P V of their key half for the previous
//    tile, V read with the transposing LDS read. The copies are buffer loads that write LDS
//    directly, the padded LDS tile filled as one contiguous byte range, 64 lanes x 16 bytes per
//    load: a lane whose 16 bytes fall in a row's padding, or in a row past KV, gets an offset
//    beyond the buffer's range, so the hardware reads nothing for it (44 loads per tile). They
//    are waited for only at the next tile's barrier, so the P V work overlaps their latency.
// The two key halves are two independent softmax splits of the keys; after the last tile they
// are merged once per query through LDS (o = (2^(m0-M) O0 + 2^(m1-M) O1) / (2^(m0-M) l0 +
// 2^(m1-M) l1), M = max(m0, m1)).
// The workgroups of one (batch, head) walk the same tiles at about the same time, so without
// help each of them would wait for the first one's HBM misses on every tile: the score waves
// therefore touch the tile kPrefetch tiles ahead (4 bytes per 128-byte line, each workgroup
// a 1/nqt share of the lines) to bring it into L2 early. Those loads write a scratch LDS
// word and are waited for only at the end, so they never stall a wave.
// The row strides (416 and 288 bytes) and the row order of the transposed reads were chosen
// with the LDS bank-conflict counter. One barrier per tile.
#include "common.h"

namespace sa {

namespace masked {

constexpr int kQT = 128;  // queries per workgroup
constexpr int kKT = 64;   // keys per tile
constexpr int kThreads = 512;
constexpr uint32_t kOob = 0x80000000u;  // buffer offset beyond every range used here
constexpr int kPrefetch = 3;            // L2 prefetch distance in tiles

template <int DQK, int DV>
struct Smem {
  static constexpr int KS = DQK * 2 + 32;  // K row stride (bytes)
  static constexpr int VS = DV * 2 + 32;   // V row stride (bytes)
  unsigned char k[2][kKT * KS];            // K tiles t (QK), t+1 (being copied)
  unsigned char v[2][kKT * VS];            // V tiles t-2 (P V), t-1 (being copied)
  bf16x8 p[2][4][4][64];                   // weights: [tile parity][score wave][query block][lane]
  uint32_t mw[2][kQT * 4];                 // mask words: [chunk parity][query][4], or [tile parity][query][2]
  uint32_t sink[2][64];                    // destination of the L2 prefetch loads (never read)
  float alpha[2][4][64];                   // rescale factor per query of the tile (if moved)
  float mref[2][kQT];                      // per key half: final reference maximum per query
  float lsum[2][kQT];                      // per key half: final weight sum per query
  float fin[2][kQT];                       // per key half: output factor per query
  int flag[2][4];                          // any rescale in this score wave's queries
};

}  // namespace masked

// One role's side of the workgroup (score waves: SCORE; value waves: !SCORE). The roles share the
// barrier sequence; each keeps only its own registers (queries or accumulators).
template <int DQK, int DV, int MASKBITS, bool OFFSET, bool SCORE>
__device__ __forceinline__ void masked_role(masked::Smem<DQK, DV>& sm, const __bf16* __restrict__ q,
                                            const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                            const uint32_t* __restrict__ mask, __bf16* __restrict__ out, int Q,
                                            int KV, int H, int padded_q, int words, int nxcc, float scale_log2) {
  using namespace masked;
  using SM = Smem<DQK, DV>;
  constexpr int KS = SM::KS, VS = SM::VS;
  constexpr int DSTEPS = DQK / 32;  // QK steps over the head dimension
  constexpr int NDB = DV / 16;      // PV output column blocks
  constexpr int KLANES = DQK / 8, VLANES = DV / 8;  // 16-byte chunks per row
  constexpr int QB = 4;             // 16-query blocks per wave (64 queries)
  static_assert(KLANES <= 64 && VLANES <= 64 && DQK % 32 == 0 && DV % 16 == 0, "head dims");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  constexpr bool score = SCORE;
  const int pw = score ? wave : wave - 4;  // index within the role
  const int qh = pw & 1, kh = pw >> 1;     // query half (64 queries) and key half (32 keys of a tile)

  const int nqt = (Q + kQT - 1) / kQT;
  const int wg = xcd_local_id(blockIdx.x, gridDim.x, nxcc);
  const int qt = wg % nqt;
  const int bh = wg / nqt;
  const int h = bh % H, b = bh / H;
  const int qbase = qt * kQT + qh * 64;  // first query of this wave's half
  const int nkt = (KV + kKT - 1) / kKT;

  // chunked-context form: the clamped start and the first position past the bit words
  uint32_t ksc = 0, pmax = 0;
  if constexpr (OFFSET) {
    pmax = 32u * (uint32_t)(words - 1);
    const uint32_t ks = mask[(size_t)b * padded_q * words + (words - 1)];
    ksc = ks < pmax ? ks : pmax;
  }

  // ---- score waves: queries (B operand), softmax state of this key half
  bf16x8 qreg[QB][SCORE ? DSTEPS : 1];
  bool qlive[QB];
  float m_ref[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int qr = qbase + 16 * qb + l16;
    qlive[qb] = qr < Q;
    m_ref[qb] = kNegInf;
    l_part[qb] = 0.f;
  }
  if constexpr (SCORE) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      const int qr = qbase + 16 * qb + l16;
#pragma unroll
      for (int s = 0; s < DSTEPS; s++) {
        bf16x8 z = {};
        qreg[qb][s] = qlive[qb] ? *(const bf16x8*)(q + (((size_t)b * Q + qr) * H + h) * DQK + 32 * s + 8 * g) : z;
      }
    }
  }

  // ---- value waves: output accumulators O[query 4g+i of block qb][column 16 db + l16] of this
  // key half
  constexpr int NDBX = SCORE ? 1 : NDB;
  f32x4 oacc[QB][NDBX];
#pragma unroll
  for (int qb = 0; qb < QB; qb++)
#pragma unroll
    for (int db = 0; db < NDBX; db++) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tile copies by the value waves: K of tile t one tile before its QK, V of tile t one tile
  // before its P V (which runs two tiles after its QK). The K tile in LDS is KCH 16-byte chunks
  // per row (KLANES of data, then padding), 64 rows: KCH loads of 64 chunks each; V likewise
  // with VCH. Load n belongs to wave 4 + n % 4; a lane's byte offset is taken relative to row 0
  // of the tile (head h), kOob for a padding chunk. The offsets do not depend on the tile: the
  // value waves compute theirs once (12 registers) and the tile only moves the buffer's base.
  constexpr int KCH = KS / 16, VCH = VS / 16, KM = (KCH + 3) / 4, VM = (VCH + 3) / 4;
  uint32_t koffs[SCORE ? 1 : KM], voffs[SCORE ? 1 : VM];
  if constexpr (!SCORE) {
#pragma unroll
    for (int m = 0; m < KM; m++) {
      const int c = 64 * (pw + 4 * m) + lane, r = c / KCH, col = c % KCH;
      koffs[m] = col < KLANES ? (uint32_t)(r * H * DQK * 2 + col * 16) : kOob;
    }
#pragma unroll
    for (int m = 0; m < VM; m++) {
      const int c = 64 * (pw + 4 * m) + lane, r = c / VCH, col = c % VCH;
      voffs[m] = col < VLANES ? (uint32_t)(r * H * DV * 2 + col * 16) : kOob;
    }
  }
  auto gather_k = [&](int t) {
    // rows t*kKT + r with r < nv are in range; the range ends inside row nv's first byte
    const int nv = min(KV - t * kKT, kKT);
    const size_t row0 = ((size_t)b * KV + (size_t)t * kKT) * H + h;
    const u32x4 kr = buffer_rsrc(k + row0 * DQK, (uint32_t)(((nv - 1) * H + 1) * DQK * 2));
    const uint32_t kd = lds_addr(sm.k[t & 1]);
#pragma unroll
    for (int m = 0; m < KM; m++)
      if (pw + 4 * m < KCH) dma_lds16(kr, koffs[m % (SCORE ? 1 : KM)], kd + 1024 * (pw + 4 * m));
  };
  auto gather_v = [&](int t) {
    const int nv = min(KV - t * kKT, kKT);
    const size_t row0 = ((size_t)b * KV + (size_t)t * kKT) * H + h;
    const u32x4 vr = buffer_rsrc(v + row0 * DV, (uint32_t)(((nv - 1) * H + 1) * DV * 2));
    const uint32_t vd = lds_addr(sm.v[t & 1]);
#pragma unroll
    for (int m = 0; m < VM; m++)
      if (pw + 4 * m < VCH) dma_lds16(vr, voffs[m % (SCORE ? 1 : VM)], vd + 1024 * (pw + 4 * m));
  };

  // Mask copy by the value waves, for tile t: the wide form copies the 4 words of keys
  // [128 c, 128 c + 128) of all kQT queries at the even tile t = 2c (two 16-byte loads, by waves
  // 4 and 5), into sm.mw[c & 1][query][4]; the control form copies the 2 words of tile t (four
  // 4-byte loads, by waves 4-7) into sm.mw[t & 1][query][2]; the chunked form copies words
  // w0 .. w0 + 3 of mask position 64 t + key_start (eight 4-byte loads) into
  // sm.mw[t & 1][query][4]. Rows past padded_q read nothing.
  const int q0 = qt * kQT;
  auto mask_copy = [&](int t) {
    if (mask == nullptr) return;
    const u32x4 mr = buffer_rsrc(mask + ((size_t)b * padded_q + q0) * words,
                                 (uint32_t)(min(kQT, padded_q - q0) * words * 4));
    if constexpr (OFFSET) {
      const uint32_t w0 = (64u * (uint32_t)t + ksc) >> 5;
      for (int i = pw; i < 8; i += 4) {
        const int d = 64 * i + lane, ql = d >> 2;
        dma_lds4(mr, (uint32_t)(ql * words + (int)w0 + (d & 3)) * 4u, lds_addr(sm.mw[t & 1]) + 256 * i);
      }
    } else if constexpr (MASKBITS == 128) {
      if ((t & 1) == 0 && pw < 2) {
        const int ql = 64 * pw + lane;
        dma_lds16(mr, (uint32_t)(ql * words * 4 + (t >> 1) * 16), lds_addr(sm.mw[(t >> 1) & 1]) + 1024 * pw);
      }
    } else {
      const int d = 64 * pw + lane, ql = d >> 1;
      dma_lds4(mr, (uint32_t)(ql * words * 4 + (2 * t + (d & 1)) * 4), lds_addr(sm.mw[t & 1]) + 256 * pw);
    }
  };

  // L2 prefetch of tile t by the score waves: 128-byte line L of the K tile (row L / LK, part
  // L % LK) is touched by the workgroup with qt = L % nqt, by score wave 0; the V tile's lines
  // by score wave 1. Rows past KV are out of the buffer's range and read nothing.
  constexpr int LK = DQK * 2 / 128, LV = DV * 2 / 128;
  static_assert(DQK * 2 % 128 == 0 && DV * 2 % 128 == 0, "rows are whole 128-byte lines");
  auto prefetch = [&](int t) {
    if (pw >= 2) return;
    const int nv = min(KV - t * kKT, kKT);
    const size_t row0 = ((size_t)b * KV + (size_t)t * kKT) * H + h;
    const int LR = pw == 0 ? LK : LV, nlines = kKT * LR;
    const u32x4 rs = pw == 0 ? buffer_rsrc(k + row0 * DQK, (uint32_t)(((nv - 1) * H + 1) * DQK * 2))
                             : buffer_rsrc(v + row0 * DV, (uint32_t)(((nv - 1) * H + 1) * DV * 2));
    const int rowb = pw == 0 ? H * DQK * 2 : H * DV * 2;
    for (int j0 = 0; qt + nqt * j0 < nlines; j0 += 64) {
      const int L = qt + nqt * (j0 + lane);
      const uint32_t off = L < nlines ? (uint32_t)((L / LR) * rowb + (L % LR) * 128) : kOob;
      dma_lds4(rs, off, lds_addr(sm.sink[pw]));
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
  if (!SCORE && nkt > 0) gather_k(0);
  if (SCORE)
    for (int t = 1; t < kPrefetch && t < nkt; t++) prefetch(t);

  // Software pipeline over the tiles, one barrier per step: at step t the score waves compute
  // QK of tile t and, interleaved with its MFMAs, the softmax of tile t-1 (its logits kept in
  // registers from the previous step), while the value waves copy K of tile t+1, V of tile t-1
  // and the mask words of tile t, and add P V of tile t-2. Steps run t = 0 .. nkt + 1 (rounded
  // up to an even count; the work of a step outside the tiles is skipped or, in the score waves,
  // masked to nothing), unrolled by two so each step's buffer parity is a constant.
  f32x4 sacc[2][QB][2];  // score waves: logits of tiles t (parity t & 1) and t - 1
  auto step = [&](const int t, const int par) __attribute__((always_inline)) {  // par == (t & 1)
    if (SCORE) wait_lgkm0();
    else wait_vm_lgkm0<0>();  // this wave's copies of the previous step have landed
    // K(t), V(t-2), P(t-2), the mask words of tile t-1 and the softmax factors of tile t-2 are
    // visible; everyone is done with K(t-1), V(t-3), P(t-3) and the mask words of tile t-2
    wg_barrier();
    if constexpr (!SCORE) {
      if (t + 1 < nkt) gather_k(t + 1);
      if (t >= 1 && t - 1 < nkt) gather_v(t - 1);
      if (t < nkt) mask_copy(t);
      if (t >= 2 && t - 2 < nkt) {  // O += P V of this key half for tile t-2
        const int pp = par;         // parity of tile t-2
        if (sm.flag[pp][pw]) {
#pragma unroll
          for (int qb = 0; qb < QB; qb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const float a = sm.alpha[pp][pw][16 * qb + 4 * g + i];
#pragma unroll
              for (int db = 0; db < NDBX; db++) oacc[qb][db][i] *= a;
            }
        }
        const int r4 = (lane >> 2) & 3, c4 = lane & 3;
        const unsigned char* vk = sm.v[pp] + (32 * kh + 4 * g + r4) * VS + 8 * c4;
        bf16x8 pa[QB];
#pragma unroll
        for (int qb = 0; qb < QB; qb++) pa[qb] = sm.p[pp][pw][qb][lane];
#pragma unroll
        for (int db = 0; db < NDB; db++) {
          const bf16x8 bv = concat_tr(lds_read_tr16(vk + 32 * db), lds_read_tr16(vk + 16 * VS + 32 * db));
#pragma unroll
          for (int qb = 0; qb < QB; qb++) oacc[qb][db % NDBX] = mfma16x16x32(pa[qb], bv, oacc[qb][db % NDBX]);
        }
      }
    } else {
      const int ts = t - 1;  // tile of this step's softmax (parity par ^ 1)
      const bool ts_live = ts >= 0 && ts < nkt;
      // the softmax tile's mask word (32 keys of this key half) per query block
      uint32_t mwd[QB];
#pragma unroll
      for (int qb = 0; qb < QB; qb++) {
        const int ql = qh * 64 + 16 * qb + l16;
        uint32_t wv;
        if constexpr (OFFSET) {
          // bits of positions p0 + 32 kh .. p0 + 32 kh + 31, none at or past pmax
          const uint4 x = *(const uint4*)&sm.mw[par ^ 1][ql * 4];
          const uint32_t p0 = 64u * (uint32_t)ts + ksc, sh = p0 & 31u;
          const int rem = (int)pmax - (int)p0 - 32 * kh;
          const uint32_t lim = rem >= 32 ? ~0u : (rem > 0 ? (1u << rem) - 1u : 0u);
          wv = (kh == 0 ? __builtin_amdgcn_alignbit(x.y, x.x, sh) : __builtin_amdgcn_alignbit(x.z, x.y, sh)) & lim;
        } else if (mask == nullptr) {
          wv = ~0u;
        } else {
          wv = MASKBITS == 128 ? sm.mw[(ts >> 1) & 1][ql * 4 + 2 * (ts & 1) + kh] : sm.mw[par ^ 1][ql * 2 + kh];
        }
        mwd[qb] = (qlive[qb] && ts_live) ? wv : 0u;
      }
      // keys past KV (last tile only)
      const int nvalid = KV - ts * kKT - 32 * kh;
      const uint32_t kvm = nvalid >= 32 ? ~0u : (nvalid > 0 ? ((1u << nvalid) - 1u) : 0u);

      // ---- S^T = K Q^T of tile t: 2 key blocks x 4 query blocks, each K operand feeding all
      // four (on stale K when t >= nkt: those logits are masked out at the next step)
      const unsigned char* kb = sm.k[par] + (32 * kh + l16) * KS + 16 * g;
#pragma unroll
      for (int qb = 0; qb < QB; qb++) sacc[par][qb][0] = sacc[par][qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      constexpr int NK = 2 * DSTEPS;  // K operands: (key block, step) pairs
      constexpr int KR = 4;           // K operands in flight
      auto kop = [&](int n) { return *(const bf16x8*)(kb + (n % 2) * 16 * KS + 64 * (n / 2)); };
      bf16x8 ka[KR];
#pragma unroll
      for (int n = 0; n < KR; n++) ka[n] = kop(n);
#pragma unroll
      for (int n = 0; n < NK; n++) {
        const int jb = n % 2, st = n / 2;
#pragma unroll
        for (int qb = 0; qb < QB; qb++)
          sacc[par][qb][jb] = mfma16x16x32(ka[n % KR], qreg[qb][st % (SCORE ? DSTEPS : 1)], sacc[par][qb][jb]);
        if (n + KR < NK) ka[n % KR] = kop(n + KR);
      }

      // ---- online softmax of tile t-1 per query block over this key half; lane holds keys
      // 16 jb + 4 g + i of query l16. Branch free (stores by all lanes of a query), so that it
      // interleaves with the MFMAs above.
      const int sp = par ^ 1;
      bool any_resc = false;
#pragma unroll
      for (int qb = 0; qb < QB; qb++) {
        const uint32_t vg = (mwd[qb] & kvm) >> (4 * g);
        float tmax = kNegInf;
#pragma unroll
        for (int jb = 0; jb < 2; jb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const bool vis = (vg >> (16 * jb + i)) & 1u;
            const float x = vis ? sacc[sp][qb][jb][i] * scale_log2 : kNegInf;
            sacc[sp][qb][jb][i] = x;  // in place: tile t-1's logits are dead after this step
            tmax = __builtin_elementwise_maximum(tmax, x);
          }
        tmax = max4_x16_x32(tmax);
        const float mold = m_ref[qb];
        const bool move = tmax > mold + 8.0f;  // also true for the first finite maximum
        const float mnew = move ? tmax : mold;
        const float alpha = move ? exp2_fast(mold - mnew) : 1.f;  // 0 when mold = -inf
        const bool resc = move && (mold > kNegInf);
        any_resc |= resc;
        m_ref[qb] = mnew;
        const float msub = (mnew > kNegInf) ? mnew : 0.f;  // no visible key yet: all weights 0
        // MFMA k index 8g+i = key 4g + i (i < 4) or 16 + 4g + i - 4 of this key half
        float lsum;
        bf16x2 pk[4];
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            pv[i] = exp2_fast(sacc[sp][qb][hf][i] - msub);
            lsum = (hf == 0 && i == 0) ? pv[0] : lsum + pv[i];
          }
          pk[2 * hf] = __builtin_convertvector((f32x2){pv[0], pv[1]}, bf16x2);
          pk[2 * hf + 1] = __builtin_convertvector((f32x2){pv[2], pv[3]}, bf16x2);
        }
        sm.p[sp][pw][qb][lane] = bf16x8{pk[0][0], pk[0][1], pk[1][0], pk[1][1], pk[2][0], pk[2][1], pk[3][0], pk[3][1]};
        l_part[qb] = l_part[qb] * alpha + lsum;
        sm.alpha[sp][pw][16 * qb + l16] = resc ? alpha : 1.f;  // the 4 lanes of a query agree
      }
      sm.flag[sp][pw] = __any(any_resc) ? 1 : 0;  // every lane stores the same value
      __builtin_amdgcn_sched_barrier(0);
      if (t + kPrefetch < nkt) prefetch(t + kPrefetch);
    }
  };
  const int nsteps = (nkt + 3) & ~1;  // t = 0 .. nkt + 1, rounded up to an even count
  for (int t = 0; t < nsteps; t += 2) {
    step(t, 0);
    step(t + 1, 1);
  }

  // ---- merge the two key halves and store. Score waves publish each query's reference maximum
  // and weight sum of their key half; each query's factors f_kh = 2^(m_kh - M) / L follow,
  // L = sum over the halves of 2^(m_kh - M) l_kh, M = max(m_0, m_1) (f = 0 without any visible
  // key). Value waves of key half 1 leave f_1 O_1 in LDS, those of key half 0 add f_0 O_0,
  // round once and store (queries past Q are not written).
  if (score) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      const float l = sum4_x16_x32(l_part[qb]);
      if (g == 0) {
        sm.mref[kh][qh * 64 + 16 * qb + l16] = m_ref[qb];
        sm.lsum[kh][qh * 64 + 16 * qb + l16] = l;
      }
    }
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
  }
  wait_lgkm0();
  wg_barrier();  // factors ready; every wave is past its last tile, so the tile buffers are free
  // f_1 O_1 of query half qh, in the accumulator layout [qb][db][lane] (fp32), over the tile buffers
  f32x4* const xch = (f32x4*)&sm.k[0][0];
  static_assert(2 * QB * NDB * 64 * 16 <= (int)(sizeof(SM::k) + sizeof(SM::v)), "merge exceeds the tile buffers");
  if (!SCORE && kh == 1) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float f = sm.fin[1][qh * 64 + 16 * qb + 4 * g + i];
#pragma unroll
        for (int db = 0; db < NDBX; db++) oacc[qb][db][i] *= f;
      }
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
#pragma unroll
      for (int db = 0; db < NDBX; db++) xch[((qh * QB + qb) * NDB + db) * 64 + lane] = oacc[qb][db];
  }
  wait_lgkm0();
  wg_barrier();
  if (!SCORE && kh == 0) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int ql = 16 * qb + 4 * g + i;
        const int qo = qbase + ql;
        const float f = sm.fin[0][qh * 64 + ql];
        __bf16* orow = out + (((size_t)b * Q + qo) * H + h) * DV + l16;
#pragma unroll
        for (int db = 0; db < NDBX; db++) {
          const float o = __builtin_fmaf(oacc[qb][db][i], f, xch[((qh * QB + qb) * NDB + db) * 64 + lane][i]);
          if (qo < Q) orow[db * 16] = (__bf16)o;
        }
      }
  }
}

template <int DQK, int DV, int MASKBITS, bool OFFSET>
__global__ __launch_bounds__(masked::kThreads, 1) void masked_attn_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const uint32_t* __restrict__ mask, __bf16* __restrict__ out, int Q, int KV, int H, int padded_q, int words,
    int nxcc, float scale_log2) {
  __shared__ __attribute__((aligned(16))) masked::Smem<DQK, DV> sm;
  if (threadIdx.x < 256)  // waves 0-3
    masked_role<DQK, DV, MASKBITS, OFFSET, true>(sm, q, k, v, mask, out, Q, KV, H, padded_q, words, nxcc, scale_log2);
  else
    masked_role<DQK, DV, MASKBITS, OFFSET, false>(sm, q, k, v, mask, out, Q, KV, H, padded_q, words, nxcc, scale_log2);
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
                                         int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv,
                                         int64_t padded_q, int64_t words, float scale, int mask_load_bits, int offset,
                                         void* stream) {
  const int64_t nqt = (Q + sa::masked::kQT - 1) / sa::masked::kQT;
  const dim3 grid((unsigned)(B * H * nqt));
  const float sl2 = scale * sa::kLog2e;
  if (Dqk != 192 || Dv != 128) return 2;
  const int nxcc = sa::masked_device_xccs();
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(sa::masked::kThreads), 0, (hipStream_t)stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, mask, (__bf16*)out, (int)Q, (int)KV, (int)H, (int)padded_q,
                       (int)words, nxcc, sl2);
  };
  if (offset)
    launch(sa::masked_attn_kernel<192, 128, 128, true>);
  else if (mask_load_bits == 32)
    launch(sa::masked_attn_kernel<192, 128, 32, false>);
  else
    launch(sa::masked_attn_kernel<192, 128, 128, false>);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
