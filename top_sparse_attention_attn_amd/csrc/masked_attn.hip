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
// run one 64-key tile apart, as in the sparse kernel:
//  * score waves 0-3 each own 32 queries: S^T = K Q^T with the queries in registers (MFMA
//    16x16x32 bf16), the mask, and the online softmax; the weights go to LDS in exactly the
//    layout the PV MFMA reads them (one 16-byte chunk per lane), with a lazily moved
//    reference maximum whose rare moves are passed on as per-query factors;
//  * value waves 4-7 own the same 32 queries each: they copy the next key/value tile and the
//    mask words it needs from HBM into LDS, and add P V for the previous tile, V read with
//    the transposing LDS read. The copies are buffer loads that write LDS directly, the
//    padded LDS tile filled as one contiguous byte range, 64 lanes x 16 bytes per load: a
//    lane whose 16 bytes fall in a row's padding, or in a row past KV, gets an offset beyond
//    the buffer's range, so the hardware reads nothing for it (44 loads per tile). They are
//    waited for only at the next tile's barrier, so the P V work overlaps their latency.
// The workgroups of one (batch, head) walk the same tiles at about the same time, so without
// help each of them would wait for the first one's HBM misses on every tile: the score waves
// therefore touch the tile kPrefetch tiles ahead (4 bytes per 128-byte line, each workgroup
// a 1/nqt share of the lines) to bring it into L2 early. Those loads write a scratch LDS
// word and are waited for only at the end, so they never stall a wave.
// Each K and V element is read from LDS once per 32 queries. The row strides (416 and 288
// bytes) and the row order of the transposed reads were chosen with the LDS bank-conflict
// counter. One barrier per tile.
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
  unsigned char k[2][kKT * KS];            // K tiles t, t+1
  unsigned char v[3][kKT * VS];            // V tiles t-1, t, t+1
  bf16x8 p[2][4][2][2][64];                // weights: [tile parity][score wave][query block][32-key step][lane]
  uint32_t mw[2][kQT * 4];                 // mask words: [chunk parity][query][4], or [tile parity][query][2]
  uint32_t sink[2][64];                    // destination of the L2 prefetch loads (never read)
  float alpha[2][4][32];                   // rescale factor per query of the tile (if moved)
  float fin[kQT];                          // 1 / row sum per query
  int flag[2][4];                          // any rescale in this score wave's queries
};

}  // namespace masked

template <int DQK, int DV, int MASKBITS, bool OFFSET>
__global__ __launch_bounds__(masked::kThreads, 1) void masked_attn_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const uint32_t* __restrict__ mask, __bf16* __restrict__ out, int Q, int KV, int H, int padded_q, int words,
    int nxcc, float scale_log2) {
  using namespace masked;
  using SM = Smem<DQK, DV>;
  constexpr int KS = SM::KS, VS = SM::VS;
  constexpr int DSTEPS = DQK / 32;  // QK steps over the head dimension
  constexpr int NDB = DV / 16;      // PV output column blocks
  constexpr int KLANES = DQK / 8, VLANES = DV / 8;  // 16-byte chunks per row
  static_assert(KLANES <= 64 && VLANES <= 64 && DQK % 32 == 0 && DV % 16 == 0, "head dims");
  __shared__ __attribute__((aligned(16))) SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const bool score = wave < 4;
  const int pw = score ? wave : wave - 4;  // index of the query group (32 queries) of this wave

  const int nqt = (Q + kQT - 1) / kQT;
  const int wg = xcd_local_id(blockIdx.x, gridDim.x, nxcc);
  const int qt = wg % nqt;
  const int bh = wg / nqt;
  const int h = bh % H, b = bh / H;
  const int qbase = qt * kQT + pw * 32;  // first query of this wave's group
  const int nkt = (KV + kKT - 1) / kKT;

  // chunked-context form: the clamped start and the first position past the bit words
  uint32_t ksc = 0, pmax = 0;
  if constexpr (OFFSET) {
    pmax = 32u * (uint32_t)(words - 1);
    const uint32_t ks = mask[(size_t)b * padded_q * words + (words - 1)];
    ksc = ks < pmax ? ks : pmax;
  }

  // ---- score waves: queries (B operand), mask rows, softmax state
  bf16x8 qreg[2][DSTEPS];
  bool qlive[2] = {false, false};
  float m_ref[2] = {kNegInf, kNegInf}, l_part[2] = {0.f, 0.f};
  if (score) {
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      const int qr = qbase + 16 * qb + l16;
      qlive[qb] = qr < Q;
#pragma unroll
      for (int s = 0; s < DSTEPS; s++) {
        bf16x8 z = {};
        qreg[qb][s] = qlive[qb] ? *(const bf16x8*)(q + (((size_t)b * Q + qr) * H + h) * DQK + 32 * s + 8 * g) : z;
      }
    }
  }

  // ---- value waves: output accumulators O[query 4g+i of block qb][column 16 db + l16]
  f32x4 oacc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; qb++)
#pragma unroll
    for (int db = 0; db < NDB; db++) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tile copy by the value waves. The K tile in LDS is KCH 16-byte chunks per row (KLANES of
  // data, then padding), 64 rows: KCH loads of 64 chunks each; V likewise with VCH. Load n of
  // the NGI per tile belongs to wave 4 + n % 4; a lane's byte offset is taken relative to row 0
  // of the tile (head h), kOob for a padding chunk. The offsets are recomputed per tile rather
  // than kept, to leave the registers to the score path.
  constexpr int KCH = KS / 16, VCH = VS / 16, NGI = KCH + VCH, GPW = (NGI + 3) / 4;
  auto chunk_off = [&](int n, int ln) -> uint32_t {
    if (n < KCH) {
      const int c = 64 * n + ln, r = c / KCH, col = c % KCH;
      return col < KLANES ? (uint32_t)(r * H * DQK * 2 + col * 16) : kOob;
    }
    const int c = 64 * (n - KCH) + ln, r = c / VCH, col = c % VCH;
    return col < VLANES ? (uint32_t)(r * H * DV * 2 + col * 16) : kOob;
  };
  auto gather = [&](int t) {
    // rows t*kKT + r with r < nv are in range; the range ends inside row nv's first byte
    const int nv = min(KV - t * kKT, kKT);
    const size_t row0 = ((size_t)b * KV + (size_t)t * kKT) * H + h;
    const u32x4 kr = buffer_rsrc(k + row0 * DQK, (uint32_t)(((nv - 1) * H + 1) * DQK * 2));
    const u32x4 vr = buffer_rsrc(v + row0 * DV, (uint32_t)(((nv - 1) * H + 1) * DV * 2));
    const uint32_t kd = lds_addr(sm.k[t & 1]), vd = lds_addr(sm.v[t % 3]);
    int ln = lane;
    asm volatile("" : "+v"(ln));  // keeps the offsets inside the loop (not hoisted into registers)
#pragma unroll
    for (int m = 0; m < GPW; m++) {
      const int n = pw + 4 * m;
      if (n < KCH)
        dma_lds16(kr, chunk_off(n, ln), kd + 1024 * n);
      else if (n < NGI)
        dma_lds16(vr, chunk_off(n, ln), vd + 1024 * (n - KCH));
    }
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
  if (!score && nkt > 0) {
    gather(0);
    mask_copy(0);
  }
  if (score)
    for (int t = 1; t < kPrefetch && t < nkt; t++) prefetch(t);

  for (int t = 0; t <= nkt; t++) {
    if (score) wait_lgkm0();
    else wait_vm_lgkm0<0>();  // this wave's rows of tile t have landed
    wg_barrier();             // tile t and P(t-1) visible; everyone is done with tile t-2 and P(t-2)
    if (!score && t + 1 < nkt) {
      gather(t + 1);
      mask_copy(t + 1);
    }

    if (score && t < nkt) {
      const int par = t & 1;
      // this tile's two mask words per query block (copied in by the value waves)
      uint32_t mwd[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        const int ql = pw * 32 + 16 * qb + l16;
        if constexpr (OFFSET) {
          // bits of positions p0 .. p0 + 63, none at or past pmax
          const uint4 x = *(const uint4*)&sm.mw[t & 1][ql * 4];
          const uint32_t p0 = 64u * (uint32_t)t + ksc, sh = p0 & 31u;
          const int rem = (int)pmax - (int)p0;
          const uint32_t lim0 = rem >= 32 ? ~0u : (rem > 0 ? (1u << rem) - 1u : 0u);
          const uint32_t lim1 = rem >= 64 ? ~0u : (rem > 32 ? (1u << (rem - 32)) - 1u : 0u);
          mwd[qb][0] = qlive[qb] ? __builtin_amdgcn_alignbit(x.y, x.x, sh) & lim0 : 0u;
          mwd[qb][1] = qlive[qb] ? __builtin_amdgcn_alignbit(x.z, x.y, sh) & lim1 : 0u;
        } else if (mask == nullptr) {
          mwd[qb][0] = mwd[qb][1] = qlive[qb] ? ~0u : 0u;
        } else {
          const uint2 x = MASKBITS == 128 ? *(const uint2*)&sm.mw[(t >> 1) & 1][ql * 4 + 2 * (t & 1)]
                                          : *(const uint2*)&sm.mw[t & 1][ql * 2];
          mwd[qb][0] = qlive[qb] ? x.x : 0u;
          mwd[qb][1] = qlive[qb] ? x.y : 0u;
        }
      }
      // keys past KV (last tile only)
      const int nvalid = KV - t * kKT;
      const uint32_t kv0 = nvalid >= 32 ? ~0u : ((1u << nvalid) - 1u);
      const uint32_t kv1 = nvalid >= 64 ? ~0u : (nvalid > 32 ? ((1u << (nvalid - 32)) - 1u) : 0u);

      // ---- S^T = K Q^T: 4 key blocks x 2 query blocks, each K operand feeding both
      const unsigned char* kb = sm.k[t & 1] + l16 * KS + 16 * g;
      f32x4 sacc[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; qb++)
#pragma unroll
        for (int j = 0; j < 4; j++) sacc[qb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      constexpr int NK = 4 * DSTEPS;  // K operands: (key block, step) pairs
      auto kop = [&](int n) { return *(const bf16x8*)(kb + (n % 4) * 16 * KS + 64 * (n / 4)); };
      bf16x8 ka[4];
#pragma unroll
      for (int n = 0; n < 4; n++) ka[n] = kop(n);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int n = 0; n < NK; n++) {
        const int jb = n % 4, st = n / 4;
        sacc[0][jb] = mfma16x16x32(ka[n % 4], qreg[0][st], sacc[0][jb]);
        sacc[1][jb] = mfma16x16x32(ka[n % 4], qreg[1][st], sacc[1][jb]);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (n + 4 < NK) {
          ka[n % 4] = kop(n + 4);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- online softmax per query block; lane holds keys 16 jb + 4 g + i of query l16
      bool any_resc = false;
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        const uint32_t w0 = mwd[qb][0] & kv0, w1 = mwd[qb][1] & kv1;
        const uint32_t vg0 = w0 >> (4 * g), vg1 = w1 >> (4 * g);
        float tmax = kNegInf;
#pragma unroll
        for (int jb = 0; jb < 4; jb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint32_t vgw = (jb < 2) ? vg0 : vg1;
            const bool vis = (vgw >> (16 * (jb & 1) + i)) & 1u;
            const float x = vis ? sacc[qb][jb][i] * scale_log2 : kNegInf;
            sacc[qb][jb][i] = x;
            tmax = fmaxf(tmax, x);
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
        float lsum = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          // MFMA k index 8g+i = key 32 ks + 4g + i (i < 4) or 32 ks + 16 + 4g + i - 4
          bf16x2 pk[4];
#pragma unroll
          for (int hf = 0; hf < 2; hf++) {
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
              pv[i] = exp2_fast(sacc[qb][2 * ks + hf][i] - msub);
              lsum += pv[i];
            }
            pk[2 * hf] = __builtin_convertvector((f32x2){pv[0], pv[1]}, bf16x2);
            pk[2 * hf + 1] = __builtin_convertvector((f32x2){pv[2], pv[3]}, bf16x2);
          }
          sm.p[par][pw][qb][ks][lane] =
              bf16x8{pk[0][0], pk[0][1], pk[1][0], pk[1][1], pk[2][0], pk[2][1], pk[3][0], pk[3][1]};
        }
        l_part[qb] = l_part[qb] * alpha + lsum;
        if (g == 0) sm.alpha[par][pw][16 * qb + l16] = resc ? alpha : 1.f;
      }
      if (lane == 0) sm.flag[par][pw] = __any(any_resc) ? 1 : 0;
      if (t + kPrefetch < nkt) prefetch(t + kPrefetch);
    }

    // ---- value waves: O += P V for tile t-1
    if (!score && t >= 1) {
      const int tp = t - 1, par = tp & 1;
      if (sm.flag[par][pw]) {
#pragma unroll
        for (int qb = 0; qb < 2; qb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float a = sm.alpha[par][pw][16 * qb + 4 * g + i];
#pragma unroll
            for (int db = 0; db < NDB; db++) oacc[qb][db][i] *= a;
          }
      }
      const int r4 = (lane >> 2) & 3, c4 = lane & 3;
      const unsigned char* vb = sm.v[tp % 3] + (4 * g + r4) * VS + 8 * c4;
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const bf16x8 pa0 = sm.p[par][pw][0][ks][lane];
        const bf16x8 pa1 = sm.p[par][pw][1][ks][lane];
        const unsigned char* vk = vb + 32 * ks * VS;
#pragma unroll
        for (int db = 0; db < NDB; db++) {
          const bf16x8 bv = concat_tr(lds_read_tr16(vk + 32 * db), lds_read_tr16(vk + 16 * VS + 32 * db));
          oacc[0][db] = mfma16x16x32(pa0, bv, oacc[0][db]);
          oacc[1][db] = mfma16x16x32(pa1, bv, oacc[1][db]);
        }
      }
    }
  }

  // ---- normalise: row sums per query (score waves), 1/l to LDS, then the value waves
  // scale and store (queries past Q are not written)
  if (score) {
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      const float l = sum4_x16_x32(l_part[qb]);
      if (g == 0) sm.fin[pw * 32 + 16 * qb + l16] = l > 0.f ? 1.f / l : 0.f;
    }
  }
  wait_vm_lgkm0<0>();
  wg_barrier();
  if (!score) {
#pragma unroll
    for (int qb = 0; qb < 2; qb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int ql = 16 * qb + 4 * g + i;
        const int qo = qbase + ql;
        if (qo >= Q) continue;
        const float f = sm.fin[pw * 32 + ql];
        __bf16* orow = out + (((size_t)b * Q + qo) * H + h) * DV + l16;
#pragma unroll
        for (int db = 0; db < NDB; db++) orow[db * 16] = (__bf16)(oacc[qb][db][i] * f);
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
