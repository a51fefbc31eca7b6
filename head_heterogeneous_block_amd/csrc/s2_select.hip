// Query-aware block lists for decode (Quest abstract, in the related-papers list
// of the SampleAttention page): the smallest and
// largest key value of every 64-token block are kept per channel; a block's
// criticality for the current query is the largest q.k any key inside that
// per-channel box can reach, sum_d max(q_d kmin_d, q_d kmax_d); the block
// holding the query and the budget - 1 highest-ranked earlier blocks form the
// (sequence, head)'s row of a CSR that the decode kernel reads.
//
// block_minmax_kernel: a workgroup (256 threads, 4 waves) takes NB consecutive
// blocks of one (sequence, head), NB chosen so that each lane has 8 16-byte
// loads in flight (2 blocks for bf16 at D = 128; 32 in flight ran 3% slower,
// with fewer workgroups resident).  A block is read in NU rounds of
// RPI key rows, LPR lanes per row and 16 bytes per lane (the decode kernel's
// read pattern); every load of the workgroup's blocks is issued before the
// first reduction.  Minima and maxima are reduced over the rows of a wave
// across lanes, then over the 4 waves through LDS.  It reads every valid key
// once: bound by HBM bandwidth.
//
// select_blocks_kernel: one workgroup per (sequence, head).
//  * Its row's offset in the CSR follows from seq_lens alone (every row of
//    sequence b holds min(budget, i_b + 1) entries), so rows need no scan pass.
//  * The bound of every earlier block goes into LDS as an order-preserving
//    32-bit key; LPR lanes score one block from 16-byte loads of its minima
//    and maxima (the only HBM traffic: 2 D values per block, 1/64 of K+V).
//  * The (budget - 1)-th largest key is found one 8-bit digit at a time from
//    the top (4 passes, each an LDS histogram of the digit and a prefix sum
//    over its 256 bins); blocks above it are taken, and of the blocks equal to
//    it the lowest indices fill the remaining places.  Block-wide prefix sums
//    over contiguous index ranges keep the output ascending.
#include "s2_decode_common.h"

namespace s2 {
namespace {

using namespace decode_detail;

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

// Running channel minima and maxima of key rows, one 16-byte slice of a row
// per lane.  fp32: fminf / fmaxf.  bf16: the 16 bits of a value, read as a
// signed integer with the low 15 bits flipped when the sign bit is set, order
// the same way as the values (-0 below +0), so the minima and maxima of a
// slice's 8 values are 4 packed 16-bit integer min and 4 max instructions
// (fminf / fmaxf on fp32 would first quiet every input, which made the vector
// ALU, not HBM, the limit).  The map is its own inverse.  A lane that saw no
// row holds +inf / -inf (fp32) or the extreme keys, which read back as NaN and
// lose to any value in the fminf / fmaxf that combines waves.
typedef short s16x2 __attribute__((ext_vector_type(2)));

// the value of the lane `off` away (off = 1, 2, ..., 32), and this lane's own
// value, in either order: the gfx950 row swaps for 16 and 32, else a permute
__device__ __forceinline__ void with_partner(unsigned x, int off, unsigned &a, unsigned &b) {
  if (off == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  } else if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  } else {
    a = x;
    b = (unsigned)__shfl_xor((int)x, off);
  }
}

template <typename T>
struct Bounds;
template <>
struct Bounds<float> {
  float mn[4], mx[4];
  __device__ void init() {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      mn[x] = INFINITY;
      mx[x] = -INFINITY;
    }
  }
  __device__ void add(const u32x4 &v) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      mn[x] = fminf(mn[x], __uint_as_float(v[x]));
      mx[x] = fmaxf(mx[x], __uint_as_float(v[x]));
    }
  }
  // combine with the lane `off` away (off = 1, 2, ..., 32)
  __device__ void combine(int off) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      unsigned a0, a1, z0, z1;
      with_partner(__float_as_uint(mn[x]), off, a0, a1);
      with_partner(__float_as_uint(mx[x]), off, z0, z1);
      mn[x] = fminf(__uint_as_float(a0), __uint_as_float(a1));
      mx[x] = fmaxf(__uint_as_float(z0), __uint_as_float(z1));
    }
  }
  __device__ void get(float *fmn, float *fmx) const {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      fmn[x] = mn[x];
      fmx[x] = mx[x];
    }
  }
};
template <>
struct Bounds<__bf16> {
  s16x2 mn[4], mx[4];
  static __device__ __forceinline__ s16x2 key(s16x2 x) { return x ^ ((x >> (short)15) & (short)0x7fff); }
  __device__ void init() {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      mn[x] = s16x2{(short)0x7fff, (short)0x7fff};
      mx[x] = s16x2{(short)0x8000, (short)0x8000};
    }
  }
  __device__ void add(const u32x4 &v) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const unsigned w = v[x];  // an element of a vector value, not a bit cast of it: that read element 0
      const s16x2 k = key(__builtin_bit_cast(s16x2, w));
      mn[x] = __builtin_elementwise_min(mn[x], k);
      mx[x] = __builtin_elementwise_max(mx[x], k);
    }
  }
  __device__ void combine(int off) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      unsigned a0, a1, z0, z1;
      with_partner(__builtin_bit_cast(unsigned, mn[x]), off, a0, a1);
      with_partner(__builtin_bit_cast(unsigned, mx[x]), off, z0, z1);
      mn[x] = __builtin_elementwise_min(__builtin_bit_cast(s16x2, a0), __builtin_bit_cast(s16x2, a1));
      mx[x] = __builtin_elementwise_max(__builtin_bit_cast(s16x2, z0), __builtin_bit_cast(s16x2, z1));
    }
  }
  __device__ void get(float *fmn, float *fmx) const {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const unsigned a = __builtin_bit_cast(unsigned, key(mn[x]));
      const unsigned z = __builtin_bit_cast(unsigned, key(mx[x]));
      fmn[2 * x] = __uint_as_float(a << 16);
      fmn[2 * x + 1] = __uint_as_float(a & 0xffff0000u);
      fmx[2 * x] = __uint_as_float(z << 16);
      fmx[2 * x + 1] = __uint_as_float(z & 0xffff0000u);
    }
  }
};

template <typename T, int D>
struct MinmaxShape {
  static constexpr int EPV = Vec<T>::N;       // elements per 16-byte load
  static constexpr int LPR = D / EPV;         // lanes per key row
  static constexpr int RPI = kThreads / LPR;  // key rows per round
  static constexpr int NU = 64 / RPI;         // rounds per block
  static constexpr int NB = 8 / NU;          // blocks per workgroup
  // paged: K/V heads per pass of a workgroup (8 loads per lane, as above)
  static constexpr int HG = 8 / NU;
};

// contiguous cache [B, H, cache_len, D]
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void block_minmax_kernel(MinmaxParams p) {
  using S = MinmaxShape<T, D>;
  constexpr int EPV = S::EPV, LPR = S::LPR, RPI = S::RPI, NU = S::NU, NB = S::NB;
  __shared__ float s_mn[kWaves][NB][D], s_mx[kWaves][NB][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % LPR, rsub = tid / LPR;
  const int ngrp = (p.nblk + NB - 1) / NB;
  // XCD x (workgroups x, x + 8, ...) takes the x-th eighth of the cache in
  // address order, so each XCD's address translations cover one range
  const int64_t total = (int64_t)p.B * p.H * ngrp, per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t lw = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (lw >= total) return;
  const int64_t bh = lw / ngrp;
  const int jb = (int)(lw % ngrp) * NB;  // first block of this workgroup
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int L = p.seq_lens[b];
  if (L < 1 || L > p.cache_len) return;  // invalid length: no bounds written
  const int nvalid = (L + 63) / 64;
  if (jb >= nvalid) return;
  const T *kb = static_cast<const T *>(p.k) + b * p.ks[0] + h * p.ks[1] + c * EPV;

  // every load of the NB blocks first, then the reductions
  u32x4 v[NB][NU];
#pragma unroll
  for (int jj = 0; jj < NB; ++jj)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = (jb + jj) * 64 + u * RPI + rsub;
      v[jj][u] = u32x4{};
      if (t < L)  // rows past the sequence do not count (and may lie beyond the cache)
        v[jj][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (int64_t)t * p.ks[2]));
    }
#pragma unroll
  for (int jj = 0; jj < NB; ++jj) {
    Bounds<T> bd;
    bd.init();
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if ((jb + jj) * 64 + u * RPI + rsub < L) bd.add(v[jj][u]);
    // rows of this wave holding the same slice c sit LPR lanes apart
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) bd.combine(off);
    if (lane < LPR) {
      float mn[EPV], mx[EPV];
      bd.get(mn, mx);
#pragma unroll
      for (int x = 0; x < EPV; ++x) {
        s_mn[wave][jj][c * EPV + x] = mn[x];
        s_mx[wave][jj][c * EPV + x] = mx[x];
      }
    }
  }
  __syncthreads();
  T *omin = static_cast<T *>(p.kmin) + (bh * p.nblk + jb) * D;
  T *omax = static_cast<T *>(p.kmax) + (bh * p.nblk + jb) * D;
  const int nout = min(NB, nvalid - jb) * D;
  for (int e = tid; e < nout; e += kThreads) {
    const int jj = e / D, d = e % D;
    float a = s_mn[0][jj][d], z = s_mx[0][jj][d];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      a = fminf(a, s_mn[w][jj][d]);
      z = fmaxf(z, s_mx[w][jj][d]);
    }
    omin[e] = (T)a;  // a value of T already: converting it back is exact
    omax[e] = (T)z;
  }
}

// Paged cache: token t of sequence b is row t % page size of page
// block_table[b][t / page size] of a pool [page, H, row in page, D].  A page
// holds every K/V head of its tokens, so a workgroup takes one 64-token block
// of one sequence for all heads (HG heads per pass, 8 16-byte loads per lane
// in flight): each page it reads is one contiguous H * rows * D run, and the
// block-table entries of the block are read once for all heads.  A page id
// outside the pool is not read and gives the block NaN bounds for every head.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void block_minmax_paged_kernel(MinmaxParams p) {
  using S = MinmaxShape<T, D>;
  constexpr int EPV = S::EPV, LPR = S::LPR, RPI = S::RPI, NU = S::NU, HG = S::HG;
  __shared__ float s_mn[kWaves][HG][D], s_mx[kWaves][HG][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % LPR, rsub = tid / LPR;
  const int b = (int)(blockIdx.x / p.nblk), jb = (int)(blockIdx.x % p.nblk);
  const int L = p.seq_lens[b];
  if (L < 1 || L > p.cache_len) return;  // invalid length: no bounds written
  if (jb * 64 >= L) return;               // block past the sequence
  const int32_t *table = p.block_table + b * p.bt_stride;

  // the pages of this lane's NU tokens (rows past the sequence are not read)
  int64_t rowoff[NU];
  bool live[NU];
  bool bad = false;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int t = jb * 64 + u * RPI + rsub;
    live[u] = false;
    rowoff[u] = 0;
    if (t < L) {
      const int page = table[t >> p.page_shift];
      if ((unsigned)page < (unsigned)p.num_pages) {
        live[u] = true;
        rowoff[u] = page * p.ks[0] + (int64_t)(t & ((1 << p.page_shift) - 1)) * p.ks[2];
      } else {
        bad = true;
      }
    }
  }
  const bool block_bad = __syncthreads_or(bad);
  const T *kb = static_cast<const T *>(p.k) + c * EPV;

  for (int h0 = 0; h0 < p.H; h0 += HG) {
    u32x4 v[HG][NU];
#pragma unroll
    for (int g = 0; g < HG; ++g)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        v[g][u] = u32x4{};
        if (live[u] && h0 + g < p.H)
          v[g][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (h0 + g) * p.ks[1] + rowoff[u]));
      }
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      Bounds<T> bd;
      bd.init();
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (live[u]) bd.add(v[g][u]);
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) bd.combine(off);
      if (lane < LPR) {
        float mn[EPV], mx[EPV];
        bd.get(mn, mx);
#pragma unroll
        for (int x = 0; x < EPV; ++x) {
          s_mn[wave][g][c * EPV + x] = mn[x];
          s_mx[wave][g][c * EPV + x] = mx[x];
        }
      }
    }
    __syncthreads();
    const int nh = min(HG, p.H - h0);
    for (int e = tid; e < nh * D; e += kThreads) {
      const int g = e / D, d = e % D;
      float a = s_mn[0][g][d], z = s_mx[0][g][d];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        a = fminf(a, s_mn[w][g][d]);
        z = fmaxf(z, s_mx[w][g][d]);
      }
      if (block_bad) a = z = NAN;
      const int64_t o = (((int64_t)b * p.H + h0 + g) * p.nblk + jb) * D + d;
      static_cast<T *>(p.kmin)[o] = (T)a;  // a value of T already: converting it back is exact
      static_cast<T *>(p.kmax)[o] = (T)z;
    }
    __syncthreads();  // s_mn / s_mx are written again by the next pass
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void select_blocks_kernel(SelectParams p) {
  constexpr int EPV = Vec<T>::N;
  constexpr int LPR = D / EPV;         // lanes per block bound
  constexpr int GPR = kThreads / LPR;  // blocks scored per round
  extern __shared__ uint32_t s_key[];  // [nblk]
  __shared__ int s_red[kWaves + 2];
  __shared__ int s_hist[256];
  static_assert(kThreads == 256, "one histogram bin per thread");

  const int tid = threadIdx.x;
  // the query heads sharing a K/V head's bounds run on one XCD and read them through its L2
  int64_t bk;
  int r;
  xcd_group(blockIdx.x, (int64_t)p.B * p.Hkv, p.group, bk, r);
  const int b = (int)(bk / p.Hkv), h = (int)(bk % p.Hkv) * p.group + r;
  const int64_t bh = (int64_t)b * p.H + h;
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

  // bounds of blocks 0 .. i-1, UB rounds of loads in flight per lane
  {
    constexpr int UB = 2;
    const int c = tid % LPR, g = tid / LPR;
    float qf[EPV];
    Vec<T>::to_float(*reinterpret_cast<const u32x4 *>(static_cast<const T *>(p.q) + b * p.qs[0] + h * p.qs[1] + c * EPV), qf);
    const int64_t bk = (int64_t)b * p.Hkv + h / p.group;  // the K/V head whose bounds this head ranks
    const T *mnp = static_cast<const T *>(p.kmin) + bk * p.nblk * D + c * EPV;
    const T *mxp = static_cast<const T *>(p.kmax) + bk * p.nblk * D + c * EPV;
    for (int j0 = g; j0 < i; j0 += UB * GPR) {
      u32x4 va[UB], vz[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int j = min(j0 + u * GPR, i - 1);  // a lane past the end re-reads block i - 1; its score is not stored
        va[u] = *reinterpret_cast<const u32x4 *>(mnp + (int64_t)j * D);
        vz[u] = *reinterpret_cast<const u32x4 *>(mxp + (int64_t)j * D);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        float a[EPV], z[EPV];
        Vec<T>::to_float(va[u], a);
        Vec<T>::to_float(vz[u], z);
        float sc = 0.f;
#pragma unroll
        for (int x = 0; x < EPV; ++x) sc += fmaxf(qf[x] * a[x], qf[x] * z[x]);
        sc = group_sum<LPR>(sc);
        const int j = j0 + u * GPR;
        if (c == 0 && j < i) s_key[j] = order_key(sc);
      }
    }
  }
  __syncthreads();

  // contiguous index range of this thread
  const int per = (i + kThreads - 1) / kThreads;
  const int j0 = min(i, tid * per), j1 = min(i, j0 + per);
  // the kk-th largest key, one 8-bit digit at a time from the top: a histogram of
  // the digit over the keys that match the digits found so far, then the digit at
  // which the count from the top reaches the places still to fill
  uint32_t thr = 0, mask = 0;
  int need = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    s_hist[tid] = 0;
    __syncthreads();
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = s_key[j];
      if ((key & mask) == thr) atomicAdd(&s_hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    const int cnt = s_hist[255 - tid];  // thread t holds digit 255 - t: a prefix sum counts from the top
    int tot;
    const int above = block_excl_scan(cnt, s_red, tot);
    if (above < need && above + cnt >= need) {  // exactly one thread
      s_red[kWaves] = 255 - tid;
      s_red[kWaves + 1] = above;
    }
    __syncthreads();
    thr |= (uint32_t)s_red[kWaves] << shift;
    mask |= 255u << shift;
    need -= s_red[kWaves + 1];
    __syncthreads();  // s_red is written again by the next scan
  }
  int eq = 0;
  for (int j = j0; j < j1; ++j) eq += s_key[j] == thr;
  int eq_total;
  const int eq_before = block_excl_scan(eq, s_red, eq_total);
  const int need_eq = need;  // >= 1: #(key > thr) < kk <= #(key >= thr)
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
  constexpr int NB = MinmaxShape<T, D>::NB;
  if (p.block_table) {
    const int64_t grid = (int64_t)p.B * p.nblk;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((block_minmax_paged_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  } else {
    const int64_t total = (int64_t)p.B * p.H * ((p.nblk + NB - 1) / NB);
    const int64_t grid = (total + kXcds - 1) / kXcds * kXcds;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((block_minmax_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  }
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
