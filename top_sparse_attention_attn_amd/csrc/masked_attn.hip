// Dense attention restricted by a bit-packed key mask (the masked-MHA form), on gfx950.
//
// What is computed (prhub summaries of vLLM PR #48770 and PR #52217): for each query
// row, softmax over the scaled dot products with the keys whose mask bit is set, applied
// to the values; the mask row (b, q) is shared by all heads; no sink. The mask is read
// four words (128 keys) per aligned 16-byte load; a 32-bit-load variant exists only as
// the control for measuring what the wide load saves, and gives identical results.
//
// Decomposition: one workgroup of 8 waves per (batch, head, 128 queries); each wave owns
// 16 queries and runs its own online softmax (no cross-wave reduction). Keys/values come
// in 64-row tiles, staged through registers into padded LDS rows (double buffered).
// QK is computed as S^T = K Q^T so that each lane ends up holding the weights of one
// query for 8 keys: exactly the A operand of the PV MFMA, so P never touches LDS. V is
// read with the transposing LDS read.
#include "common.h"

namespace sa {

template <int DQK, int DV, int MASKBITS>
__global__ __launch_bounds__(512, 1) void masked_attn_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                             const __bf16* __restrict__ v,
                                                             const uint32_t* __restrict__ mask,
                                                             __bf16* __restrict__ out, int Q, int KV, int H,
                                                             int padded_q, int words, float scale_log2) {
  constexpr int QT = 128, KT = 64;
  constexpr int KS = DQK * 2 + 16, VS = DV * 2 + 16;  // padded LDS row strides in bytes
  constexpr int DS = DQK / 32;                        // QK steps over the head dimension
  constexpr int NDB = DV / 16;                        // PV output column blocks
  constexpr int KCH = DQK / 8, VCH = DV / 8;          // 16-byte chunks per row
  constexpr int KLOADS = (KT * KCH + 511) / 512, VLOADS = (KT * VCH + 511) / 512;
  static_assert((KT * KCH) % 512 == 0 && (KT * VCH) % 512 == 0, "tile must split evenly over 512 threads");

  __shared__ __attribute__((aligned(16))) unsigned char ks_[2][KT * KS];
  __shared__ __attribute__((aligned(16))) unsigned char vs_[2][KT * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;

  const int nqt = (Q + QT - 1) / QT;
  const int wg = xcd_local_id(blockIdx.x, gridDim.x);
  const int qt = wg % nqt;
  const int bh = wg / nqt;
  const int h = bh % H, b = bh / H;
  const int qrow = qt * QT + wave * 16 + l16;  // this lane's query (softmax side)
  const bool qlive = qrow < Q;

  bf16x8 qreg[DS];
#pragma unroll
  for (int s = 0; s < DS; s++) {
    bf16x8 z = {};
    qreg[s] = qlive ? *(const bf16x8*)(q + (((size_t)b * Q + qrow) * H + h) * DQK + 32 * s + 8 * g) : z;
  }
  const uint32_t* mrow = (mask != nullptr && qlive) ? mask + ((size_t)b * padded_q + qrow) * words : nullptr;

  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_part = 0.f;

  // staged copy of the next tile (16-byte chunks)
  uint4 kst[KLOADS], vst[VLOADS];
  auto stage = [&](int kt) {
#pragma unroll
    for (int n = 0; n < KLOADS; n++) {
      const int c = tid + 512 * n;
      const int row = c / KCH, ch = c % KCH;
      const int j = kt * KT + row;
      kst[n] = j < KV ? *(const uint4*)(k + (((size_t)b * KV + j) * H + h) * DQK + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int n = 0; n < VLOADS; n++) {
      const int c = tid + 512 * n;
      const int row = c / VCH, ch = c % VCH;
      const int j = kt * KT + row;
      vst[n] = j < KV ? *(const uint4*)(v + (((size_t)b * KV + j) * H + h) * DV + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto commit = [&](int bi) {
#pragma unroll
    for (int n = 0; n < KLOADS; n++) {
      const int c = tid + 512 * n;
      *(uint4*)(&ks_[bi][(c / KCH) * KS + (c % KCH) * 16]) = kst[n];
    }
#pragma unroll
    for (int n = 0; n < VLOADS; n++) {
      const int c = tid + 512 * n;
      *(uint4*)(&vs_[bi][(c / VCH) * VS + (c % VCH) * 16]) = vst[n];
    }
  };

  const int nkt = (KV + KT - 1) / KT;
  stage(0);
  commit(0);
  __syncthreads();
  uint32_t mw[4] = {~0u, ~0u, ~0u, ~0u};  // mask words of the current 128-key chunk
  for (int kt = 0; kt < nkt; kt++) {
    const int bi = kt & 1;
    if (kt + 1 < nkt) stage(kt + 1);
    // ---- mask words for this tile's keys
    if (mrow != nullptr) {
      if (MASKBITS == 128) {
        if ((kt & 1) == 0) {
          const uint4 c = *(const uint4*)(mrow + (kt >> 1) * 4);
          mw[0] = c.x; mw[1] = c.y; mw[2] = c.z; mw[3] = c.w;
        }
      } else {
        const int w0 = kt * 2;
        mw[(kt & 1) * 2 + 0] = mrow[w0];
        mw[(kt & 1) * 2 + 1] = mrow[w0 + 1];
      }
    } else if (mask != nullptr) {
      mw[0] = mw[1] = mw[2] = mw[3] = 0u;  // query row past Q: nothing visible
    }
    // ---- S^T = K Q^T for 64 keys x this wave's 16 queries
    const unsigned char* kb = ks_[bi];
    f32x4 sacc[4];
#pragma unroll
    for (int jb = 0; jb < 4; jb++) sacc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DS; s++)
#pragma unroll
      for (int jb = 0; jb < 4; jb++) {
        const bf16x8 a = *(const bf16x8*)(kb + (16 * jb + l16) * KS + (32 * s + 8 * g) * 2);
        sacc[jb] = mfma16x16x32(a, qreg[s], sacc[jb]);
      }
    float x[4][4];
    float tmax = kNegInf;
#pragma unroll
    for (int jb = 0; jb < 4; jb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int jl = 16 * jb + 4 * g + i;         // key within the tile
        const int jc = (kt & 1) * 64 + jl;          // key within the 128-key chunk
        const bool vis = ((mw[jc >> 5] >> (jc & 31)) & 1u) && (kt * KT + jl < KV);
        const float val = vis ? sacc[jb][i] * scale_log2 : kNegInf;
        x[jb][i] = val;
        tmax = fmaxf(tmax, val);
      }
    tmax = fmaxf(tmax, xor_shuffle(tmax, 16));
    tmax = fmaxf(tmax, xor_shuffle(tmax, 32));
    const bool move = tmax > m_ref + 8.0f;
    const float mnew = move ? tmax : m_ref;
    const float alpha = move ? exp2_fast(m_ref - mnew) : 1.f;
    const bool resc = move && (m_ref > kNegInf);
    m_ref = mnew;
    l_part *= alpha;
    bf16x8 pa[2];
#pragma unroll
    for (int jb = 0; jb < 4; jb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float p = (mnew > kNegInf) ? exp2_fast(x[jb][i] - mnew) : 0.f;
        const __bf16 pb = (__bf16)p;
        l_part += (float)pb;
        pa[jb >> 1][(jb & 1) * 4 + i] = pb;
      }
    if (__any(resc)) {
      // O rows are queries 4g+i; their factors live in lanes whose l16 is that query.
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float a = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((4 * g + i) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
        for (int db = 0; db < NDB; db++) oacc[db][i] *= a;
      }
    }
    // ---- O += P V; k ordering within a 32-key step: lanes of group g hold keys
    // 4g..4g+3 and 16+4g..16+4g+3, matched by the two transposed reads below.
    const unsigned char* vb = vs_[bi];
    const int r4 = (lane >> 2) & 3, c4 = lane & 3;
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const unsigned char* p0 = vb + (32 * ks + 4 * g + r4) * VS + 4 * c4 * 2;
#pragma unroll
      for (int db = 0; db < NDB; db++) {
        const bf16x8 bv = concat_tr(lds_read_tr16(p0 + db * 32), lds_read_tr16(p0 + 16 * VS + db * 32));
        oacc[db] = mfma16x16x32(pa[ks], bv, oacc[db]);
      }
    }
    if (kt + 1 < nkt) {
      __syncthreads();  // everyone is done reading buffer bi^1 (tile kt-1)
      commit(bi ^ 1);
      __syncthreads();
    }
  }

  // ---- normalise: row sums per query, then 1/l for the O rows (queries 4g+i)
  l_part += xor_shuffle(l_part, 16);
  l_part += xor_shuffle(l_part, 32);
  const float inv = l_part > 0.f ? 1.f / l_part : 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float f = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((4 * g + i) << 2, __builtin_bit_cast(int, inv)));
    const int qo = qt * QT + wave * 16 + 4 * g + i;
    if (qo >= Q) continue;
    __bf16* orow = out + (((size_t)b * Q + qo) * H + h) * DV + l16;
#pragma unroll
    for (int db = 0; db < NDB; db++) orow[db * 16] = (__bf16)(oacc[db][i] * f);
  }
}

}  // namespace sa

extern "C" int sa_internal_launch_masked(const void* q, const void* k, const void* v, const uint32_t* mask, void* out,
                                         int64_t B, int64_t Q, int64_t KV, int64_t H, int64_t Dqk, int64_t Dv,
                                         int64_t padded_q, int64_t words, float scale, int mask_load_bits,
                                         void* stream) {
  const int64_t nqt = (Q + 127) / 128;
  const dim3 grid((unsigned)(B * H * nqt));
  const float sl2 = scale * sa::kLog2e;
  if (Dqk != 192 || Dv != 128) return 2;
  if (mask_load_bits == 32)
    hipLaunchKernelGGL((sa::masked_attn_kernel<192, 128, 32>), grid, dim3(512), 0, (hipStream_t)stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, mask, (__bf16*)out, (int)Q, (int)KV,
                       (int)H, (int)padded_q, (int)words, sl2);
  else
    hipLaunchKernelGGL((sa::masked_attn_kernel<192, 128, 128>), grid, dim3(512), 0, (hipStream_t)stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, mask, (__bf16*)out, (int)Q, (int)KV,
                       (int)H, (int)padded_q, (int)words, sl2);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
