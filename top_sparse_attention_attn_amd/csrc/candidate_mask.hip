// Candidate mask of the DSA indexer's decode path, on gfx950 (prhub summary of vLLM
// PR #56628: the ROCm decode mask strides only up to each row's live end).
//
// The logits workspace is [rows] x [width] fp32 with width = the longest context the
// engine allows, while a decode row holds live logits only in [start, end). For row r
// (row_repeat rows share one start/end), a live column c keeps its logit iff the keep
// flag of its block (c - start) / block_size is set, or c is the last column and the
// row's edge flag is set; every other column is set to -inf. Columns at or past end
// are never written: no consumer reads them, and leaving them is what makes the cost
// follow the live length instead of the workspace width.
//
// Launch shape: rows x gcols workgroups of 256 threads, gcols fixed by (rows, width)
// alone (enough workgroups to cover the GPU, never more tiles than the row has), so a
// captured graph stays valid when only the ends change. Workgroup (r, p) handles the
// 1024-column tiles p, p + gcols, ... below min(end, width). The kernel only writes
// -inf and reads keep flags (a block's columns share one byte through the cache);
// logits are never read.
//  * Vector form (unit column stride, 16-byte aligned rows, block size a multiple of 4,
//    row start a multiple of 4): thread t takes the four adjacent columns 4t .. 4t+3 of
//    the tile. They fall in one block, so one flag byte decides them and one 16-byte
//    store writes them; a wave store covers 1 KB. Only the chunk holding the end, the
//    last column (edge flag) or a partial chunk goes column by column.
//  * Scalar form (any strides): each thread four columns, consecutive threads on
//    consecutive columns, one 4-byte store per masked column.
#include "common.h"

namespace sa {

namespace cand {
constexpr int kThreads = 256;
constexpr int kTile = 4 * kThreads;  // columns per workgroup iteration
}  // namespace cand

// Keep flag of column c of a row (start s, flags fr): its block's flag, or the edge flag for
// the last column; columns below the start are never kept.
__device__ __forceinline__ bool cand_keep(int c, int64_t s, const uint8_t* fr, int nblocks, int block_size,
                                          int bs_shift, int width, bool edge) {
  if ((int64_t)c < s) return false;
  const int64_t off = (int64_t)c - s;
  const int64_t blk = bs_shift >= 0 ? (off >> bs_shift) : off / block_size;
  return (blk < nblocks && fr[blk] != 0) || (c == width - 1 && edge);
}

// bs_shift >= 0: block_size = 1 << bs_shift (a shift instead of a division).
// VEC: the launch meets the vector form's stride, alignment and block-size conditions.
template <bool HAS_STARTS, bool VEC>
__global__ __launch_bounds__(cand::kThreads) void candidate_mask_kernel(
    float* __restrict__ logits, const int32_t* __restrict__ starts, const int32_t* __restrict__ ends,
    const uint8_t* __restrict__ flags, int64_t stride_row, int64_t stride_col, int64_t stride_start,
    int64_t stride_end, int width, int nblocks, int block_size, int bs_shift, int row_repeat, int gcols) {
  using namespace cand;
  const int row = blockIdx.x / gcols, prog = blockIdx.x % gcols;
  const int64_t i = row / row_repeat;
  const int64_t s = HAS_STARTS ? (int64_t)starts[i * stride_start] : 0;
  const int e = ends[i * stride_end];
  const int lim = min(e, width);
  const uint8_t* fr = flags + (size_t)row * (size_t)(nblocks + 1);
  const bool edge = fr[nblocks] != 0;
  float* lr = logits + (int64_t)row * stride_row;
  constexpr float kMasked = -__builtin_huge_valf();
  if (VEC && (s & 3) == 0) {
    // a chunk of four columns starting at a multiple of 4 lies in one block (the start and the
    // block size are multiples of 4) and on one side of the start
    for (int t0 = prog * kTile; t0 < lim; t0 += gcols * kTile) {
      const int c0 = t0 + 4 * (int)threadIdx.x;
      if (c0 >= lim) continue;
      if (c0 + 3 < lim && c0 + 3 != width - 1) {
        if (!cand_keep(c0, s, fr, nblocks, block_size, bs_shift, width, edge))
          *(float4*)(lr + c0) = make_float4(kMasked, kMasked, kMasked, kMasked);
      } else {
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const int c = c0 + k;
          if (c < lim && !cand_keep(c, s, fr, nblocks, block_size, bs_shift, width, edge)) lr[c] = kMasked;
        }
      }
    }
    return;
  }
  for (int t0 = prog * kTile; t0 < lim; t0 += gcols * kTile) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int c = t0 + k * kThreads + (int)threadIdx.x;
      if (c >= lim) continue;
      if (!cand_keep(c, s, fr, nblocks, block_size, bs_shift, width, edge))
        lr[(int64_t)c * stride_col] = kMasked;
    }
  }
}

}  // namespace sa

// Workgroups per row: enough to give ~4096 workgroups in all, at most one per tile (more
// evens out rows of very different live lengths; many more makes short rows pay for the
// launch of workgroups that have nothing to do).
extern "C" int sa_internal_candidate_gcols(int64_t rows, int64_t width) {
  const int64_t tiles = (width + sa::cand::kTile - 1) / sa::cand::kTile;
  int64_t g = rows > 0 ? 4096 / rows : 1;
  if (g < 1) g = 1;
  if (g > tiles) g = tiles;
  return (int)(g < 1 ? 1 : g);
}

extern "C" int sa_internal_launch_candidate_mask(float* logits, const int32_t* starts, const int32_t* ends,
                                                 const uint8_t* flags, int64_t rows, int64_t width,
                                                 int64_t stride_row, int64_t stride_col, int64_t stride_start,
                                                 int64_t stride_end, int64_t block_size, int64_t row_repeat,
                                                 void* stream) {
  const int gcols = sa_internal_candidate_gcols(rows, width);
  const int nblocks = (int)((width + block_size - 1) / block_size);
  int shift = -1;
  if ((block_size & (block_size - 1)) == 0) {
    shift = 0;
    while (((int64_t)1 << shift) < block_size) shift++;
  }
  const dim3 grid((unsigned)(rows * gcols));
  // vector form: unit column stride, every row 16-byte aligned, blocks of a multiple of 4 columns
  const bool vec = stride_col == 1 && ((uintptr_t)logits & 15u) == 0 && (stride_row & 3) == 0 &&
                   (block_size & 3) == 0;
#define SA_CAND(HS, V)                                                                                     \
  hipLaunchKernelGGL((sa::candidate_mask_kernel<HS, V>), grid, dim3(sa::cand::kThreads), 0, (hipStream_t)stream, \
                     logits, starts, ends, flags, stride_row, stride_col, stride_start, stride_end, (int)width,     \
                     nblocks, (int)block_size, shift, (int)row_repeat, gcols)
  if (starts) {
    if (vec) SA_CAND(true, true); else SA_CAND(true, false);
  } else {
    if (vec) SA_CAND(false, true); else SA_CAND(false, false);
  }
#undef SA_CAND
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
