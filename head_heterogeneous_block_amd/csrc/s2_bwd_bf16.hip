// Block-sparse causal attention backward, bf16 in / bf16 out, fp32 accumulate,
// for gfx950 (CDNA4) MFMA.
//
// Method: the gradients of the forward's exact masked softmax attention with
// respect to Q, K and V (the pages' kernels serve training as well as
// inference: S2-Attention OpenReview page, Abstract), computed tile by tile
// over the same active 64x64 tiles, with the probabilities recomputed from the
// forward's logsumexp instead of stored:
//     P = exp(S * scale - LSE),  dV = P^T dO,  dP = dO V^T,
//     dS = P * (dP - delta),     delta = rowsum(dO * O),
//     dQ = dS K * scale,         dK = dS^T Q * scale.
// Three launches: delta, then dQ by query block (walking the layout's rows),
// then dK and dV by key block (walking its column view), so every output
// element is written by one workgroup and nothing needs atomics.
//
// Mapping onto CDNA4 (v_mfma_f32_32x32x16_bf16, the forward's conventions):
//  * dQ: per wave 32 query rows.  S^T = K Q^T and dP^T = V dO^T with Q and dO
//    in registers, so each lane owns one query and its LSE and delta are
//    per-lane scalars; dQ^T += K^T dS^T with K^T read transposed from LDS.
//  * dK, dV: per wave 32 keys.  S = Q K^T and dP = dO V^T with K and V in
//    registers, so each lane owns one key; the P and dS registers then are, as
//    bf16, exactly the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose
//    A operands are transposed reads of the staged dO and Q blocks.
//  * Blocks read both as rows (ds_read_b128) and transposed
//    (ds_read_b64_tr_b16) are stored with a swizzle that keeps both reads free
//    of bank conflicts; K/V (dQ kernel) and Q/dO/LSE/delta (dK/dV kernel) go
//    from global memory straight into LDS (global_load_lds) through a
//    2-stage ring.
#include <algorithm>
#include <type_traits>

#include "s2_internal.h"

namespace s2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int sload(const int32_t *base, int64_t idx) {
  return ((const __attribute__((address_space(4))) int32_t *)(base))[idx];
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(p);
}

// Direct global -> LDS loads: lane L reads base + voff and writes LDS bytes
// [lds + 16L, +16) (dwordx4) or [lds + 4L, +4) (dword).  Inline asm without
// register outputs; the kernels order them with s_waitcnt vmcnt and barriers.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds)
      : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds)
      : "memory", "m0");
}

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// XOR swizzle of the 16-byte chunks of LDS row r for blocks read both as rows
// and transposed.  Row reads: 16 consecutive rows at one logical chunk reach 16
// distinct chunk positions of the 256-byte bank window.  Transposed reads (4
// rows x 64 bytes per 32 lanes): the 4 rows fall in 4 distinct 64-byte bank
// groups.  D = 64 rows are 128 bytes, two per bank window.
template <int D>
__device__ __forceinline__ int swz_rt(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
// row reads only (the forward's K swizzle)
template <int D>
__device__ __forceinline__ int swz_r(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}

template <int D>
struct BwdCfg {
  static constexpr int ROWB = 2 * D;       // bytes of a row
  static constexpr int TILEB = 64 * ROWB;  // one 64-row block
  static constexpr int DC = D / 16;        // k-steps of a product over D
  static constexpr int DT = D / 32;        // 32-wide tiles of D
};

// ---------------------------------------------------------------------------
// Work plans of the dK/dV and dQ kernels, written by a launch of two
// workgroups before them.
//
// Plan: the order in which a kernel's workgroups take their work items (a
// column of the layout for dK/dV, a pair of rows for dQ).  Every (b, h) lists
// its items in one fixed order c (key blocks ascending, query-block pairs
// descending: longest first in a causal layout).  The plan holds first every
// item at least `thresh` blocks long, (b, h) by (b, h) in that order, then the
// shorter ones in the same order.  Going (b, h) by (b, h) keeps few (b, h)
// active at once, and their items, started together and walked in the same
// direction, read the same blocks at about the same time, which L2 then
// serves; putting the long items first lets the short ones fill in the end of
// the launch instead of a long item of the last (b, h) trailing alone (the
// hardware hands workgroups out in index order).  Entry = b * ncol + c, with
// ncol items per (b, h).
// ---------------------------------------------------------------------------
constexpr int kLongCol = 16;  // dK/dV: query blocks in a column
constexpr int kLongRow = 32;  // dQ: key blocks in the later row of a pair

template <class Len>
__device__ void write_plan(int B, int64_t ncol, int thresh, Len item_len, int32_t *plan) {  // 256 threads
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // thread tid owns the items [c0, c1) of the per-(b, h) sequence
  const int64_t per = (ncol + 255) / 256;
  const int64_t c0 = min(ncol, tid * per), c1 = min(ncol, c0 + per);
  int cnt = 0;
  for (int64_t c = c0; c < c1; ++c) cnt += item_len(c) >= thresh;
  // exclusive scan of the long-item counts over the threads
  int x = cnt;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wv] = x;
  __syncthreads();
  int64_t r1 = x - cnt, tot1 = 0;
  for (int w = 0; w < 4; ++w) {
    r1 += w < wv ? wave_tot[w] : 0;
    tot1 += wave_tot[w];
  }
  const int64_t tot2 = ncol - tot1;
  for (int64_t c = c0; c < c1; ++c) {
    const bool lg = item_len(c) >= thresh;
    const int64_t r = lg ? r1 : c - r1;  // rank among the long (or the short) items
    for (int b = 0; b < B; ++b) plan[lg ? b * tot1 + r : B * tot1 + b * tot2 + r] = (int32_t)(b * ncol + c);
    r1 += lg;
  }
}

__device__ void write_plans(const BwdParams &p) {
  const int nqb = p.nqb, ngrp = (nqb + 1) / 2;
  if (blockIdx.x == 0)  // dK/dV: c = h * nqb + j
    write_plan(p.B, (int64_t)p.H * nqb, kLongCol,
               [&](int64_t c) { return p.col_ptr[c + 1] - p.col_ptr[c]; }, p.plan_kv);
  if (blockIdx.x == (gridDim.x > 1 ? 1 : 0)) {  // dQ: c = h * ngrp + (ngrp - 1 - g)
    if (gridDim.x == 1) __syncthreads();
    write_plan(p.B, (int64_t)p.H * ngrp, kLongRow,
               [&](int64_t c) {
                 const int64_t h = c / ngrp;
                 const int i = min(2 * (ngrp - 1 - (int)(c % ngrp)) + 1, nqb - 1);
                 return p.row_ptr[h * nqb + i + 1] - p.row_ptr[h * nqb + i];
               },
               p.plan_q);
  }
}

// the two work plans: workgroup 0 the dK/dV plan, workgroup 1 the dQ plan
__global__ __launch_bounds__(256) void bwd_plan_kernel(BwdParams p) { write_plans(p); }

// ---------------------------------------------------------------------------
// dQ: workgroup = 2 query blocks of one (b, h), 4 waves of 32 query rows;
// walks the union of the two CSR rows, K and V of each block staged in LDS.
// Workgroup w takes the w-th pair of rows of the plan written by the plan
// kernel.  It also computes delta = rowsum(dO * O) and -LSE * log2(e) of its
// rows, which it uses and stores for the dK/dV kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int QB = 2, NW = 4, DC = C::DC, DT = C::DT;
  constexpr int STAGEB = 2 * C::TILEB;          // K then V
  constexpr int LOADS = C::TILEB / (1024 * NW);  // dwordx4 loads per wave per block
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGEB];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = uni(tid >> 6);
  const int ngrp = (p.nqb + QB - 1) / QB;
  const int item = p.plan_q[blockIdx.x];
  const int64_t bh = item / ngrp;
  const int grp = ngrp - 1 - item % ngrp;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int my_qb = wave >> 1, my_i = grp * QB + my_qb;
  const int row_in_blk = (wave & 1) * 32 + l32;
  const bool wave_on = my_i < p.nqb;

  // direct-load offsets: this wave fills LDS bytes [(wave*LOADS + n) * 1024, +1024)
  // of a block; position (r, pos) receives global chunk pos ^ swizzle(r)
  uint32_t gk[LOADS], gv[LOADS];
#pragma unroll
  for (int n = 0; n < LOADS; ++n) {
    const int o = (wave * LOADS + n) * 1024 + lane * 16;
    const int r = o / C::ROWB, pos = (o % C::ROWB) / 16;
    gk[n] = (uint32_t)(r * p.ks[2] * 2 + (pos ^ swz_rt<D>(r)) * 16);
    gv[n] = (uint32_t)(r * p.vs[2] * 2 + (pos ^ swz_r<D>(r)) * 16);
  }
  const char *kbase = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.k) + b * p.ks[0] + h * p.ks[1]);
  const char *vbase = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.v) + b * p.vs[0] + h * p.vs[1]);
  const int64_t kblk = 64 * p.ks[2] * 2, vblk = 64 * p.vs[2] * 2;
  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int j, int stage) {
    const char *kt = kbase + j * kblk;
    const char *vt = vbase + j * vblk;
    const uint32_t kl = uni(smem_lds + stage * STAGEB + wave * LOADS * 1024);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) dma16(kt, gk[n], kl + n * 1024);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) dma16(vt, gv[n], kl + C::TILEB + n * 1024);
  };

  // Q^T and dO^T operands (lane: query l32 of this wave, d = 16dc + 8hh + 0..7),
  // and the query's LSE (base 2) and delta
  bf16x8 qreg[DC], greg[DC];
  float nl2 = 0.f, dlt = 0.f;
  if (wave_on) {
    const int64_t n = (int64_t)my_i * 64 + row_in_blk;
    const __bf16 *qrow = static_cast<const __bf16 *>(p.q) + b * p.qs[0] + h * p.qs[1] + n * p.qs[2] + hh * 8;
    const __bf16 *grow = static_cast<const __bf16 *>(p.dout) + b * p.dos[0] + h * p.dos[1] + n * p.dos[2] + hh * 8;
    const __bf16 *orow = static_cast<const __bf16 *>(p.o) + b * p.os[0] + h * p.os[1] + n * p.os[2] + hh * 8;
    bf16x8 oreg[DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      qreg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + dc * 16));
      greg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(grow + dc * 16));
      oreg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(orow + dc * 16));
    }
    // delta = rowsum(dO * O): this lane's half of the row, then its partner's
    // (lane l ^ 32 holds the other 8 of every 16 channels of the same query)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = fmaf((float)oreg[dc][e], (float)greg[dc][e], dlt);
    dlt += __shfl_xor(dlt, 32);
    const int64_t r = ((int64_t)b * p.H + h) * p.N + n;
    nl2 = -p.lse[r] * kLog2e;
    // both for the dK/dV kernel, which runs next
    if (hh == 0) {
      p.delta[r] = dlt;
      p.nlse2[r] = nl2;
    }
  } else {
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qreg[dc] = greg[dc] = bf16x8{};
  }
  // these loads must land before the block loads start: a compiler wait placed
  // later would also wait for the block loads it cannot see
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) asm volatile("" ::"v"(qreg[dc]), "v"(greg[dc]));
  asm volatile("" ::"v"(nl2), "v"(dlt));

  // row-read operand offsets (K and V as A operands of S^T and dP^T): row
  // kh*32 + l32, chunk 2dc + hh
  uint32_t koff[DC], voffr[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    koff[dc] = (uint32_t)(l32 * C::ROWB + (((2 * dc + hh) ^ swz_rt<D>(l32)) << 4));
    voffr[dc] = (uint32_t)(l32 * C::ROWB + (((2 * dc + hh) ^ swz_r<D>(l32)) << 4));
  }
  // transposed reads of K (K^T operand of dQ^T): lane (gg, kk, q) reads row
  // 16c + 8s + 4(gg>>1) + kk, logical chunk 4dt + 2(gg&1) + (q>>1), half q&1;
  // the swizzle depends on s through bit 2 of the row
  uint32_t ktoff[DT][2];
  {
    const int gg = lane >> 4, kk = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = 8 * s + 4 * (gg >> 1) + kk;
      const int x = 2 * (gg & 1) + (q >> 1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        ktoff[dt][s] = (uint32_t)(r * C::ROWB + (((4 * dt + x) ^ swz_rt<D>(r)) << 4) + (q & 1) * 8);
    }
  }

  // CSR rows of the two query blocks, merged in ascending order
  int rp[QB], re[QB], rc[QB];
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    const int i = grp * QB + r;
    if (i < p.nqb) {
      rp[r] = sload(p.row_ptr, (int64_t)h * p.nqb + i);
      re[r] = sload(p.row_ptr, (int64_t)h * p.nqb + i + 1);
    } else {
      rp[r] = re[r] = 0;
    }
    rc[r] = rp[r] < re[r] ? sload(p.col_idx, rp[r]) : 0x7fffffff;
  }
  auto next_block = [&](int &j, int &mask) -> bool {
    const int jm = min(rc[0], rc[1]);
    if (jm == 0x7fffffff) return false;
    int m = 0;
#pragma unroll
    for (int r = 0; r < QB; ++r)
      if (rc[r] == jm) {
        m |= 1 << r;
        ++rp[r];
        rc[r] = rp[r] < re[r] ? sload(p.col_idx, rp[r]) : 0x7fffffff;
      }
    j = jm;
    mask = m;
    return true;
  };

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};

  auto compute = [&](int stage, int j) {
    const char *kl = smem + stage * STAGEB;
    const char *vl = kl + C::TILEB;
    const bool diag = j == my_i;
    // dS^T as bf16 B operands: chunk c = 2*kh + gg covers keys
    // 16c + {4hh..4hh+3, 8+4hh..8+4hh+3}
    bf16x8 dsk[4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // S^T = K Q^T and dP^T = V dO^T for keys 32kh .. 32kh+31, one half at a
      // time (half the accumulators live); the K and V row reads run RS - 1
      // k-steps ahead of the products through a ring of operand registers
      constexpr int RS = 3;
      f32x16 s = f32x16{}, dp = f32x16{};
      bf16x8 ka[RS], va[RS];
      auto rowread = [&](int dc, bf16x8 &kv, bf16x8 &vv) {
        kv = *reinterpret_cast<const bf16x8 *>(kl + kh * 32 * C::ROWB + koff[dc]);
        vv = *reinterpret_cast<const bf16x8 *>(vl + kh * 32 * C::ROWB + voffr[dc]);
      };
      static_for<0, RS - 1>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        rowread(i, ka[i], va[i]);
      });
      static_for<0, DC>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u + RS - 1 < DC) rowread(u + RS - 1, ka[(u + RS - 1) % RS], va[(u + RS - 1) % RS]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[u % RS], qreg[u], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[u % RS], greg[u], dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      // the diagonal block masks key > query (scores to -inf, probability 0)
      if (diag) {
        int lim = row_in_blk - 4 * hh;  // opaque: the compares stay in this branch
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kh * 32 + 8 * (e >> 2) + (e & 3);
          s[e] = key > lim ? -INFINITY : s[e];
        }
      }
      // P^T = exp2(S^T * scale*log2e - LSE*log2e), dS^T = P^T (dP^T - delta)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        f32x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ee = 8 * gg + e;
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[ee], p.scale_log2, nl2));
          f[e] = pv * (dp[ee] - dlt);
        }
        dsk[2 * kh + gg] = __builtin_convertvector(f, bf16x8);
      }
      // keep the first half's vector work here: moved down to its use it would
      // keep both halves' accumulators live across the second half's products
      if (kh == 0) asm volatile("" ::"v"(dsk[0]), "v"(dsk[1]));
    }
    // dQ^T += K^T dS^T; u = c*DT + dt, the transposed K reads RT - 1 products ahead
    constexpr int NU = 4 * DT, RT = 3;
    bf16x8 kt[RT];
    auto trread = [&](int u, bf16x8 &kv) {
      const char *a0 = kl + (16 * (u / DT)) * C::ROWB;
      const int dt = u % DT;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(a0 + ktoff[dt][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(a0 + ktoff[dt][1]));
      kv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    static_for<0, RT - 1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      trread(i, kt[i]);
    });
    static_for<0, NU>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u + RT - 1 < NU) trread(u + RT - 1, kt[(u + RT - 1) % RT]);
      dq[u % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[u % RT], dsk[u / DT], dq[u % DT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // 2-stage ring: block t+1 loads while block t is computed.  The loop is
  // unrolled over the two stages, so a step's stage is a constant and the LDS
  // operand addresses fold into the read instructions' offsets.
  int j0 = -1, m0 = 0;
  if (next_block(j0, m0)) issue(j0, 0);
  const int my_bit = 1 << my_qb;
  auto step = [&](auto stage_c) -> bool {
    constexpr int stage = decltype(stage_c)::value;
    wait_vm<0>();
    __syncthreads();  // block t landed for every wave; every wave is past block t-1
    int j1 = -1, m1 = 0;
    if (next_block(j1, m1)) issue(j1, stage ^ 1);
    if (wave_on && (m0 & my_bit)) compute(stage, j0);
    j0 = j1;
    m0 = m1;
    return j0 >= 0;
  };
  while (j0 >= 0) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
  }

  if (wave_on) {
    const int64_t n = (int64_t)my_i * 64 + row_in_blk;
    __bf16 *orow = static_cast<__bf16 *>(p.dq) + b * p.dqs[0] + h * p.dqs[1] + n * p.dqs[2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = dq[dt][4 * gi + e] * p.scale;
        *reinterpret_cast<bf16x4 *>(orow + dt * 32 + 8 * gi + 4 * hh) = __builtin_convertvector(f, bf16x4);
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = one key block of one (b, h), 2 waves of 32 keys; walks
// the block's column, Q, dO, -LSE*log2e and delta of each query block staged
// in LDS.  A wave holds its keys' K and V operands and the dK and dV
// accumulators (192 registers) for the whole walk, so it runs one wave per
// SIMD and a CU holds two workgroups; the file is built with the VGPR form of
// the MFMA instructions, which keeps S and dP in the registers the
// exponentials read.  One column per workgroup: a workgroup spanning two
// columns would idle half its waves wherever only one column is active (a
// strided column next to a local one).  Workgroup w takes the w-th column
// of the plan written by the plan kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int NW = 2, DC = C::DC, DT = C::DT;
  constexpr int STAGEB = 2 * C::TILEB + 512;    // Q, dO, then -LSE*log2e and delta (64 floats each)
  constexpr int LOADS = C::TILEB / (1024 * NW);  // dwordx4 loads per wave per block and tensor
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGEB];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = uni(tid >> 6);
  const int item = p.plan_kv[blockIdx.x];
  const int64_t bh = item / p.nqb;
  const int my_j = item % p.nqb;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int key_in_blk = wave * 32 + l32;

  // direct-load source offset of load n of this wave (row r, position pos of
  // the LDS block receives global chunk pos ^ swizzle(r)); computed at each
  // issue rather than held in registers
  auto src_off = [&](int n, int64_t rstride) {
    const int o = (wave * LOADS + n) * 1024 + lane * 16;
    const int r = o / C::ROWB, pos = (o % C::ROWB) / 16;
    return (uint32_t)(r * rstride * 2 + (pos ^ swz_rt<D>(r)) * 16);
  };
  const char *qbase = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.q) + b * p.qs[0] + h * p.qs[1]);
  const char *gbase = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.dout) + b * p.dos[0] + h * p.dos[1]);
  const int64_t qblk = 64 * p.qs[2] * 2, gblk = 64 * p.dos[2] * 2;
  const int64_t rowbase = ((int64_t)b * p.H + h) * p.N;
  // -LSE*log2(e) (wave 0) or delta (wave 1) of the block's 64 queries: one
  // 4-byte load per lane
  const float *sbase = wave ? p.delta + rowbase : p.nlse2 + rowbase;
  const uint32_t soff = (uint32_t)(lane * 4);
  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int i, int stage) {
    const char *qt = qbase + i * qblk;
    const char *gt = gbase + i * gblk;
    const uint32_t ql = uni(smem_lds + stage * STAGEB + wave * LOADS * 1024);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) dma16(qt, src_off(n, p.qs[2]), ql + n * 1024);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) dma16(gt, src_off(n, p.dos[2]), ql + C::TILEB + n * 1024);
    dma4(sbase + (int64_t)i * 64, soff, uni(smem_lds + stage * STAGEB + 2 * C::TILEB + wave * 256));
  };

  // K^T and V^T operands (lane: key l32 of this wave, d = 16dc + 8hh + 0..7)
  bf16x8 kreg[DC], vreg[DC];
  {
    const int64_t n = (int64_t)my_j * 64 + key_in_blk;
    const __bf16 *krow = static_cast<const __bf16 *>(p.k) + b * p.ks[0] + h * p.ks[1] + n * p.ks[2] + hh * 8;
    const __bf16 *vrow = static_cast<const __bf16 *>(p.v) + b * p.vs[0] + h * p.vs[1] + n * p.vs[2] + hh * 8;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      kreg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(krow + dc * 16));
      vreg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(vrow + dc * 16));
    }
  }
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) asm volatile("" ::"v"(kreg[dc]), "v"(vreg[dc]));

  // row reads of Q and dO (A operands of S and dP): row 32qh + l32, chunk 2dc + hh
  uint32_t roff[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) roff[dc] = (uint32_t)(l32 * C::ROWB + (((2 * dc + hh) ^ swz_rt<D>(l32)) << 4));
  // transposed reads of dO and Q (A operands of dV^T and dK^T)
  uint32_t toff[DT][2];
  {
    const int gg = lane >> 4, kk = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = 8 * s + 4 * (gg >> 1) + kk;
      const int x = 2 * (gg & 1) + (q >> 1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        toff[dt][s] = (uint32_t)(r * C::ROWB + (((4 * dt + x) ^ swz_rt<D>(r)) << 4) + (q & 1) * 8);
    }
  }

  // the key block's column of the layout: query blocks row_idx[c0 .. c1)
  const int c0 = sload(p.col_ptr, (int64_t)h * p.nqb + my_j);
  const int c1 = sload(p.col_ptr, (int64_t)h * p.nqb + my_j + 1);

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16{};

  auto compute = [&](int stage, int i) {
    const char *ql = smem + stage * STAGEB;
    const char *gl = ql + C::TILEB;
    const float *sl = reinterpret_cast<const float *>(ql + 2 * C::TILEB);  // -LSE*log2e [64], delta [64]
    const bool diag = i == my_j;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      // S = Q K^T and dP = dO V^T for queries 32qh .. 32qh+31: lane owns key
      // l32; entry e is query 32qh + 8(e>>2) + 4hh + (e&3).  A ring of RS
      // operand pairs keeps RS - 1 row reads ahead of the products.
      constexpr int RS = 2;
      f32x16 s = f32x16{}, dp = f32x16{};
      bf16x8 qa[RS], ga[RS];
      auto rowread = [&](int dc, bf16x8 &qv, bf16x8 &gv) {
        qv = *reinterpret_cast<const bf16x8 *>(ql + qh * 32 * C::ROWB + roff[dc]);
        gv = *reinterpret_cast<const bf16x8 *>(gl + qh * 32 * C::ROWB + roff[dc]);
      };
      static_for<0, RS - 1>([&](auto ic) { rowread(decltype(ic)::value, qa[decltype(ic)::value], ga[decltype(ic)::value]); });
      static_for<0, DC>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u + RS - 1 < DC) rowread(u + RS - 1, qa[(u + RS - 1) % RS], ga[(u + RS - 1) % RS]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[u % RS], kreg[u], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[u % RS], vreg[u], dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      if (diag) {  // key > query is masked (score -inf, probability 0)
        int klim = key_in_blk - 32 * qh - 4 * hh;  // opaque: the compares stay in this branch
        asm volatile("" : "+v"(klim));
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = klim > 8 * (e >> 2) + (e & 3) ? -INFINITY : s[e];
      }
      // P and dS, then as bf16 B operands: chunk c (16 queries) = entries
      // 8c .. 8c+7, the row order of the transposed reads below
      bf16x8 pk[2], dsk[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 nl4 = *reinterpret_cast<const f32x4 *>(sl + 32 * qh + 8 * g + 4 * hh);
        const f32x4 dl4 = *reinterpret_cast<const f32x4 *>(sl + 64 + 32 * qh + 8 * g + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ee = 4 * g + e;
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[ee], p.scale_log2, nl4[e]));
          s[ee] = pv;
          dp[ee] = pv * (dp[ee] - dl4[e]);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x8 fp, fd;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          fp[e] = s[8 * c + e];
          fd[e] = dp[8 * c + e];
        }
        pk[c] = __builtin_convertvector(fp, bf16x8);
        dsk[c] = __builtin_convertvector(fd, bf16x8);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries; u = c*DT + dt
      constexpr int NU = 2 * DT, RT = 2;
      bf16x8 gt[RT], qt[RT];
      auto trread = [&](int u, bf16x8 &gv, bf16x8 &qv) {
        const int rb = (32 * qh + 16 * (u / DT)) * C::ROWB;
        const int dt = u % DT;
        const i16x4 glo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(gl + rb + toff[dt][0]));
        const i16x4 ghi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(gl + rb + toff[dt][1]));
        const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(ql + rb + toff[dt][0]));
        const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(ql + rb + toff[dt][1]));
        gv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7));
        qv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      static_for<0, RT - 1>([&](auto ic) { trread(decltype(ic)::value, gt[decltype(ic)::value], qt[decltype(ic)::value]); });
      static_for<0, NU>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u + RT - 1 < NU) trread(u + RT - 1, gt[(u + RT - 1) % RT], qt[(u + RT - 1) % RT]);
        dv[u % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gt[u % RT], pk[u / DT], dv[u % DT], 0, 0, 0);
        dk[u % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[u % RT], dsk[u / DT], dk[u % DT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };

  // Walk the column from its last query block down (the sum's order does not
  // matter): the columns of one (b, h) start together and then read the same
  // query block at about the same time, so a block fetched into L2 serves them
  // all (ascending walks start at different blocks and re-fetch each block
  // once per column, about 3x the traffic).  2-stage ring: the next block
  // loads while this one is computed.
  int i0 = c0 < c1 ? sload(p.row_idx, c1 - 1) : -1;
  if (i0 >= 0) issue(i0, 0);
  for (int c = c1 - 1; c >= c0; --c) {
    wait_vm<0>();
    __syncthreads();  // block c landed for both waves; both are past block c+1
    const int i1 = c - 1 >= c0 ? sload(p.row_idx, c - 1) : -1;
    if (i1 >= 0) issue(i1, (c1 - c) & 1);
    compute((c1 - 1 - c) & 1, i0);
    i0 = i1;
  }

  {
    const int64_t n = (int64_t)my_j * 64 + key_in_blk;
    __bf16 *krow = static_cast<__bf16 *>(p.dk) + b * p.dks[0] + h * p.dks[1] + n * p.dks[2];
    __bf16 *vrow = static_cast<__bf16 *>(p.dv) + b * p.dvs[0] + h * p.dvs[1] + n * p.dvs[2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4 fk, fv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          fk[e] = dk[dt][4 * gi + e] * p.scale;
          fv[e] = dv[dt][4 * gi + e];
        }
        *reinterpret_cast<bf16x4 *>(krow + dt * 32 + 8 * gi + 4 * hh) = __builtin_convertvector(fk, bf16x4);
        *reinterpret_cast<bf16x4 *>(vrow + dt * 32 + 8 * gi + 4 * hh) = __builtin_convertvector(fv, bf16x4);
      }
  }
}

template <int D>
hipError_t launch_bwd_t(const BwdParams &p, hipStream_t stream) {
  const int64_t groups = (int64_t)p.B * p.H * ((p.nqb + 1) / 2);
  const int64_t cols = (int64_t)p.B * p.H * p.nqb;
  if (cols > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_plan_kernel, dim3(2), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dQ also writes delta and -LSE*log2(e) of its rows, which dK/dV reads
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)groups), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)cols), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams &p, int D, hipStream_t stream) {
  if (D == 128) return launch_bwd_t<128>(p, stream);
  if (D == 64) return launch_bwd_t<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace s2
