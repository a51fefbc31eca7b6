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
