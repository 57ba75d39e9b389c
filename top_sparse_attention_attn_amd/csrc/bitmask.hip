// Top-k index lists -> bit-packed mask, on gfx950.
//
// Layout (prhub summary of vLLM PR #52217, key source and tests; bit order from the
// prhub summary of vLLM PR #48770, dense_mask_mod): row (b, q) of the mask holds one bit
// per key, key j in word j >> 5 at bit j & 31; rows are a whole number of 16-byte
// chunks; word words-1 of query row 0 holds the batch's key start when key starts are
// stored.
//
// One workgroup of two waves builds one mask row in LDS (zeroed, then LDS atomic OR of
// every index of the row), then writes the whole row, padding included, with 16-byte
// stores, so the output needs no pre-zeroing. Rows past q_len and padded query rows are
// written as zeros. When topk is a multiple of 4 and the index list starts 16-byte aligned
// (the interface asks for 4-byte alignment only), the indices come in with 16-byte loads,
// all of a thread's loads in flight before its first atomic (small workgroups keep many
// rows' loads in flight per CU).
#include "common.h"

namespace sa {

constexpr int kMaskThreads = 128;
constexpr int kMaskMaxWords = 32768;  // 128 KB of LDS per row

__global__ __launch_bounds__(kMaskThreads) void topk_bitmask_kernel(const int* __restrict__ idx,
                                                                    const int* __restrict__ q_lens,
                                                                    const int* __restrict__ key_starts,
                                                                    uint32_t* __restrict__ mask, int Q, int topk,
                                                                    int key_len, int padded_q, int words) {
  extern __shared__ __attribute__((aligned(16))) uint32_t row_s[];
  const int rowid = blockIdx.x;  // b * padded_q + q
  const int b = rowid / padded_q, qi = rowid % padded_q;
  const int t = threadIdx.x;
  for (int w = t * 4; w < words; w += kMaskThreads * 4) *(uint4*)(row_s + w) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  int live = Q;
  if (q_lens != nullptr) {
    live = q_lens[b];
    live = live < 0 ? 0 : (live > Q ? Q : live);
  }
  if (qi < live) {
    const int* r = idx + ((size_t)b * Q + qi) * topk;
    if ((topk & 3) == 0 && ((uintptr_t)idx & 15u) == 0) {
      // 16-byte index loads (every row starts 16-byte aligned), up to eight per thread in flight
      // before the first atomic
      constexpr int kV = 8;
      for (int k0 = 4 * t; k0 < topk; k0 += 4 * kMaskThreads * kV) {
        int4 v[kV];
#pragma unroll
        for (int u = 0; u < kV; u++) {
          const int k = k0 + u * 4 * kMaskThreads;
          v[u] = k < topk ? *(const int4*)(r + k) : make_int4(-1, -1, -1, -1);
        }
#pragma unroll
        for (int u = 0; u < kV; u++) {
          const int jj[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (jj[e] >= 0 && jj[e] < key_len) atomicOr(row_s + (jj[e] >> 5), 1u << (jj[e] & 31));
        }
      }
    } else {
      for (int k = t; k < topk; k += kMaskThreads) {
        const int j = r[k];
        if (j >= 0 && j < key_len) atomicOr(row_s + (j >> 5), 1u << (j & 31));
      }
    }
  }
  __syncthreads();
  if (key_starts != nullptr && qi == 0 && t == 0) row_s[words - 1] = (uint32_t)key_starts[b];
  __syncthreads();
  uint32_t* dst = mask + (size_t)rowid * words;
  for (int w = t * 4; w < words; w += kMaskThreads * 4) *(uint4*)(dst + w) = *(const uint4*)(row_s + w);
}

}  // namespace sa

extern "C" int sa_internal_launch_bitmask(const int32_t* idx, const int32_t* q_lens, const int32_t* key_starts,
                                          uint32_t* mask, int64_t B, int64_t Q, int64_t topk, int64_t key_len,
                                          int64_t padded_q, int64_t words, void* stream) {
  const size_t lds = (size_t)words * 4;
  if (lds > 65536) {
    if (hipFuncSetAttribute((const void*)sa::topk_bitmask_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return 1;
  }
  hipLaunchKernelGGL(sa::topk_bitmask_kernel, dim3((unsigned)(B * padded_q)), dim3(sa::kMaskThreads), lds,
                     (hipStream_t)stream, idx, q_lens, key_starts, mask, (int)Q, (int)topk, (int)key_len,
                     (int)padded_q, (int)words);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int64_t sa_internal_bitmask_max_words(void) { return sa::kMaskMaxWords; }
