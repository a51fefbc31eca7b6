// Layout builder: the CSR of active key blocks per (head, query block).
//
// Pattern: HHST context sharding (S2-Attention OpenReview page, Abstract):
// each head keeps a local window and a head-offset strided subset of earlier
// key blocks so that the heads together cover the context; hybrid dense heads
// come from the arXiv abstract (mlsanity page).  See s2_internal.h for the rule.
//
// gfx950 design: one launch, no separate scan pass, and every lane busy.
// Workgroup (chunk, h) owns 64 consecutive rows of head h.  The head's offset
// is the sum of the closed-form sizes of the heads before it (row_prefix over a
// whole head), one head per thread; the chunk's rows start at the head's
// closed-form prefix of the rows before the chunk, and their own offsets come
// from a wave scan of their closed-form counts.  Sparse rows are short (a
// window plus a few strided blocks), so instead of a wave per row the 256
// threads walk the chunk's entries as one flat range: consecutive threads
// write consecutive int32 entries (coalesced) and find their row by binary
// search over the row offsets in LDS.  Entry e of a sparse row with C strided
// blocks left of its window is first + e * S for e < C, else the window's
// first block + (e - C).  Rows of a dense head are long and entry e is e:
// there each wave writes whole rows.
#include "s2_internal.h"

namespace s2 {
namespace {

constexpr int kRowsPerGroup = 64;
constexpr int kLayoutThreads = 256;

__global__ __launch_bounds__(kLayoutThreads) void build_layout_kernel(PatternArgs p, int32_t *row_ptr,
                                                                      int32_t *col_idx) {
  __shared__ int32_t s_off[kRowsPerGroup + 1];  // chunk-relative row offsets, then the chunk's size
  __shared__ int32_t s_left[kRowsPerGroup], s_win[kRowsPerGroup];
  __shared__ int64_t s_part[kLayoutThreads / 64];
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = (int64_t)blockIdx.x * kRowsPerGroup;
  const int rows = (int)(p.nqb - i0 < kRowsPerGroup ? p.nqb - i0 : kRowsPerGroup);
  const bool dense = pattern_dense(p, h);

  // sizes of the heads before h, one head per thread, summed over the group
  int64_t heads = 0;
  for (int hh = tid; hh < h; hh += kLayoutThreads) heads += row_prefix(p, hh, p.nqb);
  for (int d = 1; d < 64; d <<= 1) heads += __shfl_xor(heads, d, 64);
  if (lane == 0) s_part[wave] = heads;
  // wave 0: counts of the chunk's rows and their exclusive scan
  int32_t cnt = 0, x = 0;
  if (wave == 0) {
    const int64_t i = i0 + lane;
    int32_t left = 0;
    if (lane < rows) {
      cnt = (int32_t)row_count(p, h, i);
      left = dense ? 0 : (int32_t)strided_left_count(h, i, p.W, p.S);
    }
    x = cnt;
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t xs = __shfl_up(x, d, 64);
      if (lane >= d) x += xs;
    }
    s_off[lane] = x - cnt;
    if (lane == 63) s_off[kRowsPerGroup] = x;
    s_left[lane] = left;
    s_win[lane] = (int32_t)(i0 + lane + 1) - (cnt - left);  // first block of the window
  }
  __syncthreads();
  int64_t base = row_prefix(p, h, i0);
  for (int w = 0; w < kLayoutThreads / 64; ++w) base += s_part[w];
  if (wave == 0 && lane < rows) {
    const int64_t r = (int64_t)h * p.nqb + i0 + lane;
    row_ptr[r] = (int32_t)(base + x - cnt);
    if (r == (int64_t)p.H * p.nqb - 1) row_ptr[r + 1] = (int32_t)(base + x);
  }
  if (dense) {
    // rows of a dense head are long (row i holds blocks 0..i): a wave per row
    for (int t = wave; t < rows; t += kLayoutThreads / 64) {
      const int32_t off = s_off[t], n = s_off[t + 1] - off;
      for (int32_t e = lane; e < n; e += 64) col_idx[base + off + e] = e;
    }
    return;
  }
  // the chunk's entries as one flat range; a thread's row only moves forward
  const int32_t total = s_off[kRowsPerGroup];
  const int32_t first = (int32_t)strided_first(h, p.S), S = p.S;
  int lo = 0;
  for (int32_t f = tid; f < total; f += kLayoutThreads) {
    // last row t < rows with s_off[t] <= f (offsets strictly increase: every row holds block i)
    int hi = rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= f) lo = mid; else hi = mid - 1;
    }
    const int32_t e = f - s_off[lo];
    col_idx[base + f] = e < s_left[lo] ? first + e * S : s_win[lo] + (e - s_left[lo]);
  }
}

}  // namespace

hipError_t launch_build_layout(const PatternArgs &p, int32_t *row_ptr, int32_t *col_idx,
                               hipStream_t stream) {
  // H >= 1 and nqb >= 1: validated by the caller
  const unsigned chunks = (unsigned)((p.nqb + kRowsPerGroup - 1) / kRowsPerGroup);
  hipLaunchKernelGGL(build_layout_kernel, dim3(chunks, (unsigned)p.H), dim3(kLayoutThreads), 0, stream, p,
                     row_ptr, col_idx);
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
  int64_t before = 0;
  for (int64_t j = tid; j < j0; j += kColsPerGroup) before += col_count(p, h, j);
  // sizes of the heads before h, one head per thread (summed with `before`)
  for (int hh = tid; hh < h; hh += kColsPerGroup) before += row_prefix(p, hh, p.nqb);
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
  const int64_t start = btotal + wprefix + x - cnt;
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
