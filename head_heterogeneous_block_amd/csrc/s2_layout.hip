// Layout builder: the CSR of active key blocks per (head, query block).
//
// Pattern: HHST context sharding (S2-Attention OpenReview page, Abstract):
// each head keeps a local window and a head-offset strided subset of earlier
// key blocks so that the heads together cover the context; hybrid dense heads
// come from the arXiv abstract (mlsanity page).  See s2_internal.h for the rule.
//
// gfx950 design: no scan pass.  Every row's offset is a closed-form prefix sum
// (row_prefix), so one launch writes row_ptr and col_idx with one wave per row;
// the 64 lanes of the wave write consecutive entries of the row (coalesced
// int32 stores), and entry e of a sparse row is computed directly:
// e < C (strided blocks left of the window) -> first + e * S, otherwise the
// window block start + (e - C).
#include "s2_internal.h"

namespace s2 {
namespace {

constexpr int kWavesPerGroup = 4;

__global__ __launch_bounds__(64 * kWavesPerGroup) void build_layout_kernel(PatternArgs p,
                                                                           int32_t *row_ptr,
                                                                           int32_t *col_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)p.H * p.nqb;
  const int64_t r = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int h = (int)(r / p.nqb);
  const int64_t i = r % p.nqb;

  // offset of head h: whole heads before it, then rows before i within it
  int64_t start = 0;
  for (int hh = 0; hh < h; ++hh) start += row_prefix(p, hh, p.nqb);
  start += row_prefix(p, h, i);
  const int64_t cnt = row_count(p, h, i);

  if (lane == 0) {
    row_ptr[r] = (int32_t)start;
    if (r == rows - 1) row_ptr[rows] = (int32_t)(start + cnt);
  }
  if (pattern_dense(p, h)) {
    for (int64_t e = lane; e < cnt; e += 64) col_idx[start + e] = (int32_t)e;
  } else {
    const int64_t c = strided_left_count(h, i, p.W, p.S);
    const int64_t first = strided_first(h, p.S);
    const int64_t wstart = i + 1 - (cnt - c);  // first block of the window
    for (int64_t e = lane; e < cnt; e += 64)
      col_idx[start + e] = (int32_t)(e < c ? first + e * p.S : wstart + (e - c));
  }
}

}  // namespace

hipError_t launch_build_layout(const PatternArgs &p, int32_t *row_ptr, int32_t *col_idx,
                               hipStream_t stream) {
  const int64_t rows = (int64_t)p.H * p.nqb;  // >= 1: validated by the caller
  const int64_t groups = (rows + kWavesPerGroup - 1) / kWavesPerGroup;
  hipLaunchKernelGGL(build_layout_kernel, dim3((unsigned)groups), dim3(64 * kWavesPerGroup), 0,
                     stream, p, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace s2

// ---------------------------------------------------------------------------
// Column view (query blocks per key block), for the key-side backward pass.
// Column (h, j) of the rule is the contiguous range of query blocks
// [j, j + col_count(h, j)), so only the column offsets need a prefix sum.
// Workgroup (h, chunk) sums the counts of the head's columns before its chunk
// (at most nqb additions), scans its 256 columns in LDS, and then its waves
// write whole columns with consecutive lanes (coalesced int32 stores).
// ---------------------------------------------------------------------------
namespace s2 {
namespace {

constexpr int kColsPerGroup = 256;

__global__ __launch_bounds__(kColsPerGroup) void build_layout_t_kernel(PatternArgs p, int32_t *col_ptr,
                                                                       int32_t *row_idx) {
  __shared__ int64_t s_off[kColsPerGroup];
  __shared__ int64_t s_part[kColsPerGroup / 64];
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * kColsPerGroup;

  // offset of column j0 of head h: whole heads before it (closed form), then
  // the head's columns before the chunk
  int64_t base = 0;
  for (int hh = 0; hh < h; ++hh) base += row_prefix(p, hh, p.nqb);
  int64_t before = 0;
  for (int64_t j = tid; j < j0; j += kColsPerGroup) before += col_count(p, h, j);
  // block-wide sum of `before` and exclusive scan of this chunk's counts
  const int64_t j = j0 + tid;
  const int64_t cnt = j < p.nqb ? col_count(p, h, j) : 0;
  int64_t x = cnt, y = before;
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t xs = __shfl_up(x, d, 64);
    if (lane >= d) x += xs;
    y += __shfl_xor(y, d, 64);
  }
  if (lane == 63) s_part[wave] = x;
  if (lane == 0) s_off[wave] = y;  // reuse as the per-wave sums of `before`
  __syncthreads();
  int64_t wprefix = 0, btotal = 0;
  for (int w = 0; w < kColsPerGroup / 64; ++w) {
    if (w < wave) wprefix += s_part[w];
    btotal += s_off[w];
  }
  __syncthreads();
  const int64_t start = base + btotal + wprefix + x - cnt;
  s_off[tid] = start;
  if (j < p.nqb) {
    const int64_t c = (int64_t)h * p.nqb + j;
    col_ptr[c] = (int32_t)start;
    if (c == (int64_t)p.H * p.nqb - 1) col_ptr[c + 1] = (int32_t)(start + cnt);
  }
  __syncthreads();
  // each wave writes whole columns: entries j, j + 1, ... of column j
  for (int t = wave; t < kColsPerGroup; t += kColsPerGroup / 64) {
    const int64_t jj = j0 + t;
    if (jj >= p.nqb) break;
    const int64_t n = col_count(p, h, jj), off = s_off[t];
    for (int64_t e = lane; e < n; e += 64) row_idx[off + e] = (int32_t)(jj + e);
  }
}

}  // namespace

hipError_t launch_build_layout_t(const PatternArgs &p, int32_t *col_ptr, int32_t *row_idx,
                                 hipStream_t stream) {
  const unsigned chunks = (unsigned)((p.nqb + kColsPerGroup - 1) / kColsPerGroup);
  hipLaunchKernelGGL(build_layout_t_kernel, dim3(chunks, (unsigned)p.H), dim3(kColsPerGroup), 0, stream,
                     p, col_ptr, row_idx);
  return hipGetLastError();
}

}  // namespace s2
