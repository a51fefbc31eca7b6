// Query-aware block lists for decode (Quest page, abstract): the smallest and
// largest key value of every 64-token block are kept per channel; a block's
// criticality for the current query is the largest q.k any key inside that
// per-channel box can reach, sum_d max(q_d kmin_d, q_d kmax_d); the block
// holding the query and the budget - 1 highest-ranked earlier blocks form the
// (sequence, head)'s row of a CSR that the decode kernel reads.
//
// block_minmax_kernel: a workgroup (256 threads, 4 waves) takes kMinmaxBlocks
// consecutive blocks of one (sequence, head).  A block is read in NU rounds of
// RPI key rows, LPR lanes per row and 16 bytes per lane (the decode kernel's
// read pattern); minima and maxima are reduced over the rows of a wave across
// lanes, then over the 4 waves through LDS.  It reads every valid key once:
// bound by HBM bandwidth.
//
// select_blocks_kernel: one workgroup per (sequence, head).
//  * Its row's offset in the CSR follows from seq_lens alone (every row of
//    sequence b holds min(budget, i_b + 1) entries), so rows need no scan pass.
//  * The bound of every earlier block goes into LDS as an order-preserving
//    32-bit key; LPR lanes score one block from 16-byte loads of its minima
//    and maxima (the only HBM traffic: 2 D values per block, 1/64 of K+V).
//  * The (budget - 1)-th largest key is found bit by bit from the top (32
//    counting passes over LDS); blocks above it are taken, and of the blocks
//    equal to it the lowest indices fill the remaining places.  Block-wide
//    prefix sums over contiguous index ranges keep the output ascending.
#include "s2_decode_common.h"

namespace s2 {
namespace {

using namespace decode_detail;

constexpr int kMinmaxBlocks = 4;
constexpr int kWaves = kThreads / 64;

// exclusive prefix sum of v over the workgroup in thread order; total = sum
__device__ int block_excl_scan(int v, int *s_red, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_red[wave] = x;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = s_red[w];
    base += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();  // s_red is reused by the next call
  return base + x - v;
}
__device__ int block_sum(int v, int *s_red) {
  int t;
  block_excl_scan(v, s_red, t);
  return t;
}

// float -> uint32 with the same order (negative values reversed below positives)
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void block_minmax_kernel(MinmaxParams p) {
  constexpr int EPV = Vec<T>::N;       // elements per 16-byte load
  constexpr int LPR = D / EPV;         // lanes per key row
  constexpr int RPI = kThreads / LPR;  // key rows per round
  constexpr int NU = 64 / RPI;         // rounds per block
  __shared__ float s_mn[kWaves][D], s_mx[kWaves][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % LPR, rsub = tid / LPR;
  const int ngrp = (p.nblk + kMinmaxBlocks - 1) / kMinmaxBlocks;
  const int64_t bh = blockIdx.x / ngrp;
  const int grp = blockIdx.x % ngrp;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int L = p.seq_lens[b];
  if (L < 1 || L > p.cache_len) return;  // invalid length: no bounds written
  const int nvalid = (L + 63) / 64;
  const T *kb = static_cast<const T *>(p.k) + b * p.ks[0] + h * p.ks[1] + c * EPV;
  T *omin = static_cast<T *>(p.kmin) + bh * p.nblk * D;
  T *omax = static_cast<T *>(p.kmax) + bh * p.nblk * D;

  for (int jj = 0; jj < kMinmaxBlocks; ++jj) {
    const int j = grp * kMinmaxBlocks + jj;
    if (j >= nvalid) break;
    float mn[EPV], mx[EPV];
#pragma unroll
    for (int x = 0; x < EPV; ++x) {
      mn[x] = INFINITY;
      mx[x] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = j * 64 + u * RPI + rsub;
      if (t < L) {  // rows past the sequence do not count (and may lie beyond the cache)
        float f[EPV];
        Vec<T>::to_float(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (int64_t)t * p.ks[2])), f);
#pragma unroll
        for (int x = 0; x < EPV; ++x) {
          mn[x] = fminf(mn[x], f[x]);
          mx[x] = fmaxf(mx[x], f[x]);
        }
      }
    }
    // rows of this wave holding the same slice c sit LPR lanes apart
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int x = 0; x < EPV; ++x) {
        mn[x] = fminf(mn[x], __shfl_xor(mn[x], off));
        mx[x] = fmaxf(mx[x], __shfl_xor(mx[x], off));
      }
    if (lane < LPR) {
#pragma unroll
      for (int x = 0; x < EPV; ++x) {
        s_mn[wave][c * EPV + x] = mn[x];
        s_mx[wave][c * EPV + x] = mx[x];
      }
    }
    __syncthreads();
    if (tid < D) {
      float a = s_mn[0][tid], z = s_mx[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        a = fminf(a, s_mn[w][tid]);
        z = fmaxf(z, s_mx[w][tid]);
      }
      omin[(int64_t)j * D + tid] = (T)a;  // a value of T already: converting it back is exact
      omax[(int64_t)j * D + tid] = (T)z;
    }
    __syncthreads();
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void select_blocks_kernel(SelectParams p) {
  constexpr int EPV = Vec<T>::N;
  constexpr int LPR = D / EPV;         // lanes per block bound
  constexpr int GPR = kThreads / LPR;  // blocks scored per round
  extern __shared__ uint32_t s_key[];  // [nblk]
  __shared__ int s_red[kWaves];

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  auto row_len = [&](int len) {
    return (len < 1 || len > p.cache_len) ? 0 : min(p.budget, (len - 1) / 64 + 1);
  };
  int part = 0;
  for (int x = tid; x < b; x += kThreads) part += row_len(p.seq_lens[x]);
  const int before = block_sum(part, s_red);  // entries of the rows of sequences 0 .. b-1, per head
  const int L = p.seq_lens[b];
  const int nb = row_len(L);
  const int off = p.H * before + h * nb;
  if (tid == 0) {
    p.row_ptr[bh] = off;
    if (bh == (int64_t)p.B * p.H - 1) p.row_ptr[bh + 1] = off + nb;
  }
  if (nb == 0) return;
  int *out = p.col_idx + off;
  const int i = (L - 1) / 64;
  if (i + 1 <= p.budget) {  // every block fits
    for (int j = tid; j <= i; j += kThreads) out[j] = j;
    return;
  }
  const int kk = p.budget - 1;  // places for blocks before i
  if (tid == 0) out[kk] = i;
  if (kk == 0) return;

  // bounds of blocks 0 .. i-1
  {
    const int c = tid % LPR, g = tid / LPR;
    float qf[EPV];
    Vec<T>::to_float(*reinterpret_cast<const u32x4 *>(static_cast<const T *>(p.q) + b * p.qs[0] + h * p.qs[1] + c * EPV), qf);
    const T *mnp = static_cast<const T *>(p.kmin) + bh * p.nblk * D + c * EPV;
    const T *mxp = static_cast<const T *>(p.kmax) + bh * p.nblk * D + c * EPV;
    for (int j = g; j < i; j += GPR) {
      float a[EPV], z[EPV];
      Vec<T>::to_float(*reinterpret_cast<const u32x4 *>(mnp + (int64_t)j * D), a);
      Vec<T>::to_float(*reinterpret_cast<const u32x4 *>(mxp + (int64_t)j * D), z);
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < EPV; ++x) s += fmaxf(qf[x] * a[x], qf[x] * z[x]);
      s = group_sum<LPR>(s);
      if (c == 0) s_key[j] = order_key(s);
    }
  }
  __syncthreads();

  // contiguous index range of this thread
  const int per = (i + kThreads - 1) / kThreads;
  const int j0 = min(i, tid * per), j1 = min(i, j0 + per);
  // the kk-th largest key: the largest t with #(key >= t) >= kk, bit by bit
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += s_key[j] >= cand;
    if (block_sum(cnt, s_red) >= kk) thr = cand;
  }
  int gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = s_key[j];
    gt += key > thr;
    eq += key == thr;
  }
  int eq_total;
  const int eq_before = block_excl_scan(eq, s_red, eq_total);
  const int need_eq = kk - block_sum(gt, s_red);  // >= 1: #(key > thr) < kk <= #(key >= thr)
  int sel = 0;
  for (int j = j0, e = eq_before; j < j1; ++j) {
    const uint32_t key = s_key[j];
    if (key > thr) ++sel;
    else if (key == thr) sel += e++ < need_eq;
  }
  int sel_total;
  int pos = block_excl_scan(sel, s_red, sel_total);
  for (int j = j0, e = eq_before; j < j1; ++j) {
    const uint32_t key = s_key[j];
    bool take = key > thr;
    if (key == thr) take = e++ < need_eq;
    if (take) out[pos++] = j;
  }
}

template <typename T, int D>
hipError_t launch_minmax_t(const MinmaxParams &p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.B * p.H * ((p.nblk + kMinmaxBlocks - 1) / kMinmaxBlocks);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_minmax_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_select_t(const SelectParams &p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.B * p.H;
  if (grid > 0x7fffffff || p.nblk > kMaxSelectBlocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL((select_blocks_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads),
                     (size_t)p.nblk * sizeof(uint32_t), stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_minmax(const MinmaxParams &p, s2_dtype dtype, int D, hipStream_t stream) {
  if (dtype == S2_BF16) {
    if (D == 128) return launch_minmax_t<__bf16, 128>(p, stream);
    if (D == 64) return launch_minmax_t<__bf16, 64>(p, stream);
  } else {
    if (D == 128) return launch_minmax_t<float, 128>(p, stream);
    if (D == 64) return launch_minmax_t<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_select_blocks(const SelectParams &p, s2_dtype dtype, int D, hipStream_t stream) {
  if (dtype == S2_BF16) {
    if (D == 128) return launch_select_t<__bf16, 128>(p, stream);
    if (D == 64) return launch_select_t<__bf16, 64>(p, stream);
  } else {
    if (D == 128) return launch_select_t<float, 128>(p, stream);
    if (D == 64) return launch_select_t<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace s2
