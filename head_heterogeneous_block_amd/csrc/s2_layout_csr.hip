// Caller-built layouts: validation and the column view of any CSR.
//
// The S2-Attention OpenReview abstract stresses that the sparsity can be
// customised per head and per context range; the built-in pattern is one
// such choice.  A caller may build any block layout (windows and strides
// that change along the context, global blocks, random blocks as in the
// BigBird and Longformer patterns of the arXiv record's "Builds on" list) as
// the same head-major CSR: rows r = h * nqb + i, row_ptr int32 [H * nqb + 1]
// from 0 to nnz, and in each row strictly ascending key blocks j with
// 0 <= j <= i.  Every kernel of this library reads such a CSR; these kernels
// check one, and build its column view (for the backward) when it is not the
// built-in pattern's closed form.
//
// Column view: a bitmap of H * nqb columns by nqb rows (one bit per block).
// Each CSR entry sets its bit; each column then counts its bits, a scan turns
// the counts into column offsets, and each column writes the rows of its set
// bits in ascending order.  Deterministic, no sort, O(nnz + H * nqb^2 / 32).
#include <algorithm>

#include "s2_internal.h"

namespace s2 {
namespace {

// ---------------------------------------------------------------------------
// validation: the first bad row (or row_ptr entry) wins; code packs
// (row << 8) | kind in 64 bits so that atomicMin keeps the lowest row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void validate_kernel(const int32_t *row_ptr, const int32_t *col_idx,
                                                       int64_t rows, int32_t nqb, int64_t nnz,
                                                       unsigned long long *first) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  auto report = [&](int kind) { atomicMin(first, ((unsigned long long)r << 8) | (unsigned)kind); };
  const int64_t a = row_ptr[r], e = row_ptr[r + 1];
  if (r == 0 && a != 0) return report(kLayoutBadStart);
  if (r == rows - 1 && e != nnz) return report(kLayoutBadEnd);
  if (a < 0 || e < a || e > nnz) return report(kLayoutBadPtr);
  const int i = (int)(r % nqb);
  int prev = -1;
  for (int64_t x = a; x < e; ++x) {
    const int j = col_idx[x];
    if (j < 0 || j > i) return report(kLayoutBadBlock);
    if (j <= prev) return report(kLayoutUnsorted);
    prev = j;
  }
}

__global__ void fill_u64_kernel(unsigned long long *p, unsigned long long v) { *p = v; }

// ---------------------------------------------------------------------------
// column view
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x)
    p[x] = 0u;
}

// one thread per CSR row sets bit i of column (h, j) for every entry j (a
// malformed layout cannot make it read or write out of bounds: entries are
// taken from [0, nnz) only and blocks outside [0, nqb) are skipped)
__global__ __launch_bounds__(256) void set_bits_kernel(const int32_t *row_ptr, const int32_t *col_idx,
                                                       int64_t rows, int32_t nqb, int64_t nnz, int32_t words,
                                                       uint32_t *bits) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int64_t h = r / nqb;
  const int i = (int)(r % nqb);
  const int64_t a = max((int64_t)row_ptr[r], (int64_t)0), e = min((int64_t)row_ptr[r + 1], nnz);
  for (int64_t x = a; x < e; ++x) {
    const int j = col_idx[x];
    if ((unsigned)j < (unsigned)nqb) atomicOr(&bits[(h * nqb + j) * words + (i >> 5)], 1u << (i & 31));
  }
}

// one thread per column: its number of rows, stored at col_ptr[c + 1]
__global__ __launch_bounds__(256) void count_kernel(const uint32_t *bits, int64_t cols, int32_t words,
                                                    int32_t *col_ptr) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c == 0) col_ptr[0] = 0;
  if (c >= cols) return;
  int n = 0;
  for (int w = 0; w < words; ++w) n += __popc(bits[c * words + w]);
  col_ptr[c + 1] = n;
}

// inclusive scan of col_ptr[1 .. cols] in place: one workgroup of 1024
// threads, each owning a contiguous run
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *col_ptr, int64_t cols) {
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t per = (cols + 1023) / 1024;
  const int64_t c0 = min(cols, tid * per), c1 = min(cols, c0 + per);
  int sum = 0;
  for (int64_t c = c0; c < c1; ++c) sum += col_ptr[c + 1];
  int x = sum;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wv] = x;
  __syncthreads();
  int run = x - sum;
  for (int w = 0; w < wv; ++w) run += wave_tot[w];
  for (int64_t c = c0; c < c1; ++c) {
    run += col_ptr[c + 1];
    col_ptr[c + 1] = run;
  }
}

// one thread per column writes the rows of its set bits, ascending
__global__ __launch_bounds__(256) void emit_kernel(const uint32_t *bits, int64_t cols, int32_t words,
                                                   const int32_t *col_ptr, int32_t *row_idx) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  int64_t pos = col_ptr[c];
  for (int w = 0; w < words; ++w) {
    uint32_t m = bits[c * words + w];
    while (m) {
      const int b = __ffs(m) - 1;
      row_idx[pos++] = w * 32 + b;
      m &= m - 1;
    }
  }
}

unsigned grid_for(int64_t n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

}  // namespace

hipError_t launch_validate_layout(const int32_t *row_ptr, const int32_t *col_idx, int32_t num_heads,
                                  int32_t nqb, int64_t nnz, unsigned long long *first, hipStream_t stream) {
  const int64_t rows = (int64_t)num_heads * nqb;
  hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(1), 0, stream, first, ~0ull);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(validate_kernel, dim3(grid_for(rows, 256)), dim3(256), 0, stream, row_ptr, col_idx, rows,
                     nqb, nnz, first);
  return hipGetLastError();
}

int64_t transpose_bitmap_words(int32_t num_heads, int32_t nqb) {
  return (int64_t)num_heads * nqb * ((nqb + 31) / 32);
}

hipError_t launch_transpose_layout(const int32_t *row_ptr, const int32_t *col_idx, int32_t num_heads,
                                   int32_t nqb, int64_t nnz, int32_t *col_ptr, int32_t *row_idx, uint32_t *bits,
                                   hipStream_t stream) {
  const int64_t cols = (int64_t)num_heads * nqb;
  const int32_t words = (nqb + 31) / 32;
  const int64_t nbits = transpose_bitmap_words(num_heads, nqb);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<int64_t>(grid_for(nbits, 256), 4096)), dim3(256),
                     0, stream, bits, nbits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(set_bits_kernel, dim3(grid_for(cols, 256)), dim3(256), 0, stream, row_ptr, col_idx, cols,
                     nqb, nnz, words, bits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(count_kernel, dim3(grid_for(cols, 256)), dim3(256), 0, stream, bits, cols, words, col_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, col_ptr, cols);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(emit_kernel, dim3(grid_for(cols, 256)), dim3(256), 0, stream, bits, cols, words, col_ptr,
                     row_idx);
  return hipGetLastError();
}

}  // namespace s2
