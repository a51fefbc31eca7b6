// Block-sparse causal attention forward, bf16 in / bf16 out, fp32 accumulate,
// for gfx950 (CDNA4) MFMA.
//
// Method: exact softmax attention over the active 64x64 tiles of the CSR
// layout with an online (running max / running sum) softmax, the tiling idea
// that S2-Attention credits to FlashAttention for turning sparse FLOP savings
// into wall-clock gains (S2-Attention OpenReview page, Abstract).  Per-row
// logsumexp (natural log) is written for the backward pass / split merging.
//
// Mapping onto CDNA4:
//  * A workgroup owns QB consecutive query blocks of one (batch, head), two
//    waves of 32 query rows per block.  It walks the union of their CSR rows
//    in ascending order; every K/V block of the union is staged once in LDS
//    and consumed by the waves whose own row contains it.
//  * K and V blocks go from HBM/L2 straight into LDS (global_load_lds, 16
//    bytes per lane) through an NSTAGE-deep ring, so NSTAGE - 1 blocks are in
//    flight while one is computed and no staging registers or LDS store
//    instructions are spent.  The per-lane source address places every
//    16-byte chunk at an XOR-swizzled LDS position, which keeps the operand
//    reads below free of bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns ONE query column (lane%32)
//    and 32 of its keys, so the row max needs one cross-half swap
//    (v_permlane32_swap) instead of a 32-lane reduction.
//  * The output is accumulated transposed as well, O^T += V^T P^T: the
//    probabilities stay in the registers the scores came out of (bf16 B
//    operand), and all accumulators of a lane belong to its own query, so the
//    running-max rescale is a per-lane multiply.  V^T operands are read from
//    the row-major V block with ds_read_b64_tr_b16, whose 16-lane transpose
//    delivers 4 consecutive keys of one column per lane.
//  * The launch is persistent (as many workgroups as fit on the chip at
//    once) and workgroups are dispatched round-robin over the 8 XCDs
//    (blockIdx % 8).  Each XCD has its own work queue holding whole (batch,
//    head) pairs, so the blocks a head's rows share (its strided blocks, the
//    overlapping windows, all of a dense head) are fetched from HBM by one
//    XCD and re-read from that XCD's L2; idle workgroups take items from the
//    other queues at the end.
//  * An alternative schedule, selected with S2ATTN_FWD_PIPELINED=1, pipelines
//    the blocks inside each wave: the score products of block t+1 are issued
//    between the vector instructions of block t's softmax (K and V in
//    separate 2-stage rings of the same 64 KB, K loaded two blocks ahead).
//    It computes the same result; on MI355X it is slower than the two-wave
//    overlap above (its per-step row max and masking add vector work), and
//    it is kept selectable so that the comparison can be measured again.
#include <algorithm>
#include <cstdlib>
#include <atomic>
#include <type_traits>

#include "s2_internal.h"

namespace s2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kSumCap = 4294967296.f;  // 2^32: a lane sum above it moves the running max
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// value known to be equal in every lane: keep it in a scalar register
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Scalar load of a wave-uniform int.  Read through the constant address
// space it becomes s_load_dword, counted by lgkmcnt, so it never waits for
// the direct-to-LDS block loads in flight (counted by vmcnt).
__device__ __forceinline__ int sload(const int32_t *base, int64_t idx) {
  return ((const __attribute__((address_space(4))) int32_t *)(base))[idx];
}

// 32-bit LDS address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(p);
}

// One direct global -> LDS load of 16 bytes per lane: lane L reads
// base + voff and writes LDS bytes [lds + 16L, +16).  Written as inline asm so
// that the compiler does not track it as an LDS-DMA store (it would then wait
// for all of them before every LDS read it cannot disambiguate); the kernel
// orders these loads itself with s_waitcnt vmcnt and a barrier.  The asm has
// no register outputs, so no register is left in flight.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds)
      : "memory", "m0");
}

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Next index of work queue `q`, from the caller's workspace.  Each queue is a
// 64-bit word on its own 128-byte line holding (launch tag << 32 | count).  A
// word whose tag is not this launch's is left over from an earlier launch (or
// is any other content): the first workgroup to find it so installs
// (tag << 32 | 1) with a compare-and-swap and takes index 0; every other
// workgroup then counts on from there.  So the workspace needs no clearing
// between launches and any initial content is valid; only two launches that
// share one workspace at the same time would race.
__device__ __forceinline__ int queue_take(unsigned long long *ws, int q, unsigned tag) {
  unsigned long long *c = ws + q * (kFwdQueueStride / 8);
  unsigned long long v = atomicAdd(c, 1ull);
  while ((unsigned)(v >> 32) != tag) {
    const unsigned long long expect = v + 1;  // the stale word, our increment included
    const unsigned long long seen = atomicCAS(c, expect, ((unsigned long long)tag << 32) | 1ull);
    if (seen == expect) return 0;
    if ((unsigned)(seen >> 32) == tag) {
      v = atomicAdd(c, 1ull);  // another workgroup installed the tag: count on
    } else {
      v = seen - 1;  // still stale but moved on: try again against its current value
    }
  }
  return (int)(unsigned)v;
}

template <int D, int QB_, int NSTAGE_>
struct FwdCfg {
  static constexpr int QB = QB_;               // query blocks per workgroup
  static constexpr int NW = 2 * QB;            // waves, 32 query rows each
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int NSTAGE = NSTAGE_;       // LDS ring depth
  static constexpr int ROWB = 2 * D;           // bytes of a K or V row
  static constexpr int TILEB = 64 * ROWB;      // one K or V block
  static constexpr int STAGEB = 2 * TILEB;     // K block then V block
  static constexpr int LOADS = TILEB / (1024 * NW);  // 1 KB direct loads per wave per tensor
  static constexpr int LPT = 2 * LOADS;        // direct loads per wave per block
  static_assert(LOADS >= 1 && TILEB % (1024 * NW) == 0, "block must split over the waves");
  static constexpr int WGS_PER_CU = (160 * 1024) / (NSTAGE * STAGEB + 1024) >= 2 ? 2 : 1;  // persistent grid
};

// XOR swizzles of the 16-byte chunk index of LDS row r.  K: 16 consecutive
// rows read at one logical chunk land in 16 distinct bank groups.  V: the
// 4-row x 64-byte footprint of one transposed read covers all bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128) return (r & 3) << 2;
  else return ((r >> 1) & 1) << 2;
}

// The launch parameters, read from the kernel-argument segment where they are
// needed (scalar loads) instead of being held in scalar registers for the
// whole kernel: the opaque pointer stops the compiler from hoisting the loads.
typedef const __attribute__((address_space(4))) FwdParams *KernargParams;
__device__ __forceinline__ KernargParams kernarg_params() {
  KernargParams q = (KernargParams)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return q;
}

// VL: packed variable-length batch (FwdParams::cu_seqlens); the fixed-length
// instantiation has none of its code
template <int D, int QB_, int NSTAGE_, bool VL, bool PIPE>
__global__ __launch_bounds__(128 * QB_) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_bf16_kernel(FwdParams p_arg) {
  (void)p_arg;  // read through kernarg_params()
  using C = FwdCfg<D, QB_, NSTAGE_>;
  constexpr int QB = C::QB;
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGEB];
  // the item of fetch number t sits in s_item[t & 1]: a slot is written again
  // only two fetches later, after a barrier every wave passes once it has read
  // the slot, even when an item has no block (no barrier of the ring runs)
  __shared__ int s_item[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wave = uni(tid >> 6);

  // ---------------- per-lane constants (the same for every item) ----------
  // Direct-load sources: load n of this wave fills LDS bytes
  // [(wave*LOADS + n) * 1024, +1024) of a block; lane L writes 16 bytes at
  // +16L.  That LDS position is (row r, chunk pos); it receives the global
  // chunk pos ^ swizzle(r) of row r.
  uint32_t gk[C::LOADS], gv[C::LOADS];
#pragma unroll
  for (int n = 0; n < C::LOADS; ++n) {
    const int o = (wave * C::LOADS + n) * 1024 + lane * 16;
    const int r = o / C::ROWB, pos = (o % C::ROWB) / 16;
    gk[n] = (uint32_t)(r * kernarg_params()->ks[2] * 2 + (pos ^ swz_k<D>(r)) * 16);
    gv[n] = (uint32_t)(r * kernarg_params()->vs[2] * 2 + (pos ^ swz_v<D>(r)) * 16);
  }
  const int64_t kblk = 64 * kernarg_params()->ks[2] * 2, vblk = 64 * kernarg_params()->vs[2] * 2;  // bytes per 64-row block
  const uint32_t smem_lds = lds_addr(smem);

  // K operand of S^T (dc = 16-wide slice of D): row kh*32 + l32, chunk 2dc+hh
  uint32_t koff[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    koff[dc] = (uint32_t)(l32 * C::ROWB + (((2 * dc + hh) ^ swz_k<D>(l32)) << 4));
  // V^T operand by transposed reads: lane (gg, kk, q) = (lane>>4, (lane>>2)&3,
  // lane&3) points at V[row 16c + 8s + 4(gg>>1) + kk][32dt + 16(gg&1) + 4q];
  // output lane l then holds V[16c + 8s + 4(l>>5) + k][32dt + l%32], k = 0..3
  uint32_t voff[D / 32];
  {
    const int gg = lane >> 4, kk = (lane >> 2) & 3, q = lane & 3;
    const int r = 4 * (gg >> 1) + kk;
    const int x = 2 * (gg & 1) + (q >> 1);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      voff[dt] = (uint32_t)(r * C::ROWB + (((4 * dt + x) ^ swz_v<D>(r)) << 4) + (q & 1) * 8);
  }
  const float c2 = kernarg_params()->scale_log2;
  const int my_qb = wave >> 1;
  const int row_in_blk = (wave & 1) * 32 + l32;  // query row within its 64-row block

  // ---------------- work items ---------------------------------------------
  // Item = (batch, head, group of QB consecutive query blocks).  Every XCD
  // has its own queue and owns whole (batch, head) pairs: the pairs, ranked
  // by their active block count, are dealt to the XCDs in snake order (ranks
  // 0..7 to XCDs 0..7, ranks 8..15 to XCDs 7..0, ...), and a queue walks its
  // pairs one after the other, the groups of a pair longest rows first.  The
  // workgroups of one XCD then share the K/V blocks of one head through that
  // XCD's L2, and every block is fetched from HBM by one XCD only.  A
  // workgroup whose queue is empty takes items from the other queues (in the
  // order given at `fetch` below).
  const int BH = kernarg_params()->B * kernarg_params()->H;
  const int ngrp = (kernarg_params()->nqb + QB - 1) / QB;
  const int per_queue = (BH + kXcds - 1) / kXcds * ngrp;
  unsigned long long *const queue = kernarg_params()->queue;
  const unsigned tag = kernarg_params()->tag;
  // head ranking: lane r of `order` holds the head of rank r (by decreasing
  // active block count, ties by index); more than 64 heads keep index order
  int order = lane;
  if (kernarg_params()->H <= 64) {
    const int cnt = lane < kernarg_params()->H ? kernarg_params()->row_ptr[(int64_t)(lane + 1) * kernarg_params()->nqb] - kernarg_params()->row_ptr[(int64_t)lane * kernarg_params()->nqb] : -1;
    int rank = 0;
    for (int h2 = 0; h2 < kernarg_params()->H; ++h2) {
      const int c2v = __builtin_amdgcn_readlane(cnt, h2);
      rank += (c2v > cnt || (c2v == cnt && h2 < lane)) ? 1 : 0;
    }
    for (int h2 = 0; h2 < kernarg_params()->H; ++h2)
      if (__builtin_amdgcn_readlane(rank, h2) == lane) order = h2;
  }
  // Varlen: the pairs' work differs with their sequence's length, so the
  // ranking is over (b, h) pairs by their active block count (heaviest
  // first, ties by pair index) rather than over heads; s_pair[rank] = h*B + b.
  // Up to kVlPairs pairs; beyond that the head ranking above is kept.
  constexpr int kVlPairs = 1024;
  __shared__ int s_pair[VL ? 2 * kVlPairs : 1];
  bool by_pair = false;
  if constexpr (VL) {
    const int B = kernarg_params()->B, P = BH;
    by_pair = P <= kVlPairs;
    if (by_pair) {
      int *w = s_pair + kVlPairs;  // weights, then ranks into s_pair
      for (int pp = tid; pp < P; pp += C::NT) {
        const int bb = pp % B, hh2 = pp / B;
        const int c0 = kernarg_params()->cu_seqlens[bb], c1 = kernarg_params()->cu_seqlens[bb + 1];
        const bool ok = 0 <= c0 && c0 <= c1 && c1 <= kernarg_params()->T_total &&
                        c1 - c0 <= kernarg_params()->nqb * 64;
        const int nb = ok ? (c1 - c0 + 63) >> 6 : 0;
        const int64_t r0 = (int64_t)hh2 * kernarg_params()->nqb;
        w[pp] = kernarg_params()->row_ptr[r0 + nb] - kernarg_params()->row_ptr[r0];
      }
      __syncthreads();
      int rk[kVlPairs / 256 + 1];
      int nr = 0;
      for (int pp = tid; pp < P; pp += C::NT) {
        const int wp = w[pp];
        int rank = 0;
        for (int q2 = 0; q2 < P; ++q2) {
          const int wq = w[q2];
          rank += (wq > wp || (wq == wp && q2 < pp)) ? 1 : 0;
        }
        rk[nr++] = rank;
      }
      __syncthreads();  // every weight read before s_pair is written
      nr = 0;
      for (int pp = tid; pp < P; pp += C::NT) s_pair[rk[nr++]] = pp;
      __syncthreads();
    }
  }
  // pair rank of item k of queue q
  auto pair_of = [&](int q, int k) {
    const int pr = k / ngrp;
    return kXcds * pr + ((pr & 1) ? kXcds - 1 - q : q);
  };
  // Next item (queue << 24 | index) or -1 once every queue is empty (tid 0).
  // A workgroup takes its own XCD's queue, then the others in the order
  // q^4, q^1, q^5, q^2, q^6, q^3, q^7: the snake deal puts the heaviest pairs
  // on XCDs 0-3, so a workgroup of XCD x + 4 that runs out helps XCD x first
  // (one helper per heavy queue, each reading its blocks through one more L2,
  // instead of every idle XCD crowding onto the same queue).
  const int q_own = blockIdx.x % kXcds;
  int q_cur = q_own, q_left = kXcds;
  auto fetch = [&]() -> int {
    for (;;) {
      const int k = queue_take(queue, q_cur, tag);
      if (k < per_queue) {
        if (pair_of(q_cur, k) < BH) return (q_cur << 24) | k;
        continue;
      }
      if (--q_left == 0) return -1;
      const int vi = kXcds - q_left;  // queues visited so far
      q_cur = q_own ^ (((vi & 1) << 2) | (vi >> 1));
    }
  };
  for (int it = 0;; ++it) {
    if (tid == 0) s_item[it & 1] = fetch();
    // also orders every wave's last use of the ring before the next item's loads
    __syncthreads();
    const int item = uni(s_item[it & 1]);
    if (item < 0) break;
    const int k_item = item & 0xffffff;
    const int r = pair_of(item >> 24, k_item);
    const int grp = ngrp - 1 - k_item % ngrp;
    int h, b;
    if (VL && by_pair) {
      const int pp = uni(s_pair[r]);
      h = pp / kernarg_params()->B;
      b = pp % kernarg_params()->B;
    } else {
      const int hr = r / kernarg_params()->B;
      h = kernarg_params()->H <= 64 ? __builtin_amdgcn_readlane(order, hr) : hr;
      b = r % kernarg_params()->B;
    }
    const int i_first = grp * QB;

    // this item's sequence: token offset and length (fixed-length: 0 and N).
    // A varlen sequence whose range is malformed or longer than the layout
    // counts as empty: nothing of it is read or written.
    int tok0 = 0, seq_len = kernarg_params()->N, nqb_s = kernarg_params()->nqb;
    if constexpr (VL) {
      const int c0 = sload(kernarg_params()->cu_seqlens, b), c1 = sload(kernarg_params()->cu_seqlens, b + 1);
      const bool ok = 0 <= c0 && c0 <= c1 && c1 <= kernarg_params()->T_total &&
                      c1 - c0 <= kernarg_params()->nqb * 64;
      tok0 = ok ? c0 : 0;
      seq_len = ok ? c1 - c0 : 0;
      nqb_s = (seq_len + 63) >> 6;
      if (i_first >= nqb_s) continue;  // uniform: the whole workgroup skips the item
    }

    // ---------------- this wave's query rows ------------------------------
    const int my_i = i_first + my_qb;
    const bool wave_on = my_i < nqb_s;

    const __bf16 *qbase = static_cast<const __bf16 *>(kernarg_params()->q) + b * kernarg_params()->qs[0] + h * kernarg_params()->qs[1];
    const char *kbase =
        reinterpret_cast<const char *>(static_cast<const __bf16 *>(kernarg_params()->k) + b * kernarg_params()->ks[0] + h * kernarg_params()->ks[1]);
    const char *vbase =
        reinterpret_cast<const char *>(static_cast<const __bf16 *>(kernarg_params()->v) + b * kernarg_params()->vs[0] + h * kernarg_params()->vs[1]);
    if constexpr (VL) {
      qbase += (int64_t)tok0 * kernarg_params()->qs[2];
      kbase += (int64_t)tok0 * kernarg_params()->ks[2] * 2;
      vbase += (int64_t)tok0 * kernarg_params()->vs[2] * 2;
    }

    // Q^T operand: lane holds Q[query][16*dc + 8*hh .. +7]
    bf16x8 qreg[D / 16];
    if (wave_on) {
      int qr = my_i * 64 + row_in_blk;
      if constexpr (VL) qr = min(qr, seq_len - 1);  // rows past the sequence: any finite row, not stored
      const __bf16 *qrow = qbase + (int64_t)qr * kernarg_params()->qs[2] + hh * 8;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
        qreg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + dc * 16));
    } else {
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) qreg[dc] = bf16x8{};
    }
    // Q must have landed before the block loads start: the compiler cannot see
    // those loads, and a wait for Q placed later would also wait for them
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) asm volatile("" ::"v"(qreg[dc]));

    // ---------------- CSR rows of the QB query blocks (uniform) -----------
    const int32_t *const col_idx = kernarg_params()->col_idx;
    int rp[QB], re[QB], rc[QB];
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      if (i_first + r < nqb_s) {
        const int64_t row = (int64_t)h * kernarg_params()->nqb + i_first + r;
        rp[r] = sload(kernarg_params()->row_ptr, row);
        re[r] = sload(kernarg_params()->row_ptr, row + 1);
      } else {
        rp[r] = re[r] = 0;
      }
      rc[r] = rp[r] < re[r] ? sload(col_idx, rp[r]) : 0x7fffffff;
    }
    // next block of the union and the mask of query blocks that contain it
    auto next_block = [&](int &j, int &mask) -> bool {
      int jm = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < QB; ++r) jm = min(jm, rc[r]);
      if (jm == 0x7fffffff) return false;
      int m = 0;
#pragma unroll
      for (int r = 0; r < QB; ++r) {
        if (rc[r] == jm) {
          m |= 1 << r;
          ++rp[r];
          rc[r] = rp[r] < re[r] ? sload(col_idx, rp[r]) : 0x7fffffff;
        }
      }
      j = jm;
      mask = m;
      return true;
    };

    // ---------------- accumulators -----------------------------------------
    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
    float m_run = -INFINITY;  // running max of scaled scores (base 2)
    float l_run = 0.f;        // this lane's share of the running sum

    if constexpr (!PIPE) {
      auto issue = [&](int j, int stage) {
        const char *kt = kbase + j * kblk;
        const char *vt = vbase + j * vblk;
        const uint32_t kl = uni(smem_lds + stage * C::STAGEB + wave * C::LOADS * 1024);
        const uint32_t vl = kl + C::TILEB;
        if constexpr (VL) {
          if ((j + 1) * 64 > seq_len) {
            // the sequence's last, partial block: rows past its end read the
            // last row instead (finite, in bounds; their keys are masked for
            // every query of the sequence and their queries are not stored)
            const int last = seq_len - 1 - j * 64;
#pragma unroll
            for (int n = 0; n < C::LOADS; ++n) {
              const int rr = ((wave * C::LOADS + n) * 1024 + lane * 16) / C::ROWB;
              const int back = max(rr - last, 0);
              dma16(kt, gk[n] - (uint32_t)(back * kernarg_params()->ks[2] * 2), kl + n * 1024);
            }
#pragma unroll
            for (int n = 0; n < C::LOADS; ++n) {
              const int rr = ((wave * C::LOADS + n) * 1024 + lane * 16) / C::ROWB;
              const int back = max(rr - last, 0);
              dma16(vt, gv[n] - (uint32_t)(back * kernarg_params()->vs[2] * 2), vl + n * 1024);
            }
            return;
          }
        }
#pragma unroll
        for (int n = 0; n < C::LOADS; ++n) dma16(kt, gk[n], kl + n * 1024);
#pragma unroll
        for (int n = 0; n < C::LOADS; ++n) dma16(vt, gv[n], vl + n * 1024);
      };


      auto compute = [&](int stage, int j) {
        const char *kl = smem + stage * C::STAGEB;
        const char *vl = kl + C::TILEB;
        // S^T = K Q^T; the first half's reads go first, then one read of the
        // second half behind every MFMA
        f32x16 s[2];
        bf16x8 ka[2][D / 16];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int dc = 0; dc < D / 16; ++dc)
            ka[kh][dc] = *reinterpret_cast<const bf16x8 *>(kl + kh * 32 * C::ROWB + koff[dc]);

#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          s[kh] = f32x16{};
#pragma unroll
          for (int dc = 0; dc < D / 16; ++dc)
            s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kh][dc], qreg[dc], s[kh], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, D / 16, 0);
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, D / 16, 0);


        // causal mask inside the diagonal block: key index > query index
        if (j == my_i) {
          // row - 4*hh, opaque so that the 32 compares stay in this branch
          // instead of being hoisted out of the loop as scalar lane masks
          int lim = row_in_blk - 4 * hh;
          asm volatile("" : "+v"(lim));
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = kh * 32 + 8 * (e >> 2) + (e & 3);
              s[kh][e] = key > lim ? -INFINITY : s[kh][e];
            }
        }
        // Probabilities against the running max as it stands.  The max is kept
        // lazily: it moves only when the lane's sum of the block's
        // probabilities exceeds kSumCap (2^32) or is not a number (an infinite
        // sum on the first block of every row, where the max is still -inf, or
        // a NaN score).  Then the block's row max is taken, the output and
        // the sum are rescaled to it and the probabilities are taken again.  The
        // result is unchanged because the final normalisation uses the same max
        // as the exponentials, and the sums stay far inside fp32 range.
        float neg_m = -m_run;
        float rs = 0.f;
        f32x16 p[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            p[kh][e] = __builtin_amdgcn_exp2f(fmaf(s[kh][e], c2, neg_m));
            rs += p[kh][e];
          }
        if (__any(!(rs <= kSumCap))) {
          float mx = -INFINITY;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kh][e]);
          mx = swap_halves_max(mx) * c2;
          const float m_new = mx > m_run ? mx : m_run;
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
          neg_m = -m_run;
          rs = 0.f;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              p[kh][e] = __builtin_amdgcn_exp2f(fmaf(s[kh][e], c2, neg_m));
              rs += p[kh][e];
            }
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) s[kh] = p[kh];
        l_run += rs;
        // P^T as bf16 B operands: chunk c = 2*kh + gg covers keys
        // 16c + {4hh..4hh+3, 8+4hh..8+4hh+3}
        bf16x8 pk[4];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            f32x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = s[kh][8 * gg + e];
            pk[2 * kh + gg] = __builtin_convertvector(f, bf16x8);
          }

        // O^T += V^T P^T; V^T operands come from two transposed reads each
        bf16x8 va[D / 32][4];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const char *a0 = vl + (16 * c) * C::ROWB + voff[dt];
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4 *)(a0));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4 *)(a0 + 8 * C::ROWB));
            va[dt][c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }

#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][c], pk[c], oacc[dt], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
        for (int n = 0; n < D / 8 - 4; ++n) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);

      };

      // ---------------- pipelined walk over the union of the rows ------------
      // ring of the blocks in flight: jr[k] is block t+k, k < NS-1 (-1: none)
      constexpr int NS = C::NSTAGE;
      static_assert(NS >= 2 && NS <= 4, "ring depth");
      int jr[NS - 1], mr[NS - 1];
#pragma unroll
      for (int k = 0; k < NS - 1; ++k) {
        jr[k] = -1;
        mr[k] = 0;
        int j, m;
        if (next_block(j, m)) {
          jr[k] = j;
          mr[k] = m;
          issue(j, k);
        }
      }
      const int my_bit = 1 << my_qb;
      // One step per block.  The loop is unrolled over the ring's NS stages, so
      // each step's stage is a constant and the LDS operand addresses fold into
      // the instructions' immediate offsets.
      auto step = [&](auto stage_c) -> bool {
        constexpr int stage = decltype(stage_c)::value;
        // block t has landed once at most the loads of the blocks after it remain
        int later = 0;
#pragma unroll
        for (int k = 1; k < NS - 1; ++k) later += jr[k] >= 0;
        if (later == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::LPT) : "memory");
        else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::LPT) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // every wave is past block t-1: its stage takes block t + NS - 1
        int jn = -1, mn = 0;
        if (next_block(jn, mn)) issue(jn, (stage + NS - 1) % NS);
        if (wave_on && (mr[0] & my_bit)) compute(stage, jr[0]);
#pragma unroll
        for (int k = 0; k < NS - 2; ++k) {
          jr[k] = jr[k + 1];
          mr[k] = mr[k + 1];
        }
        jr[NS - 2] = jn;
        mr[NS - 2] = mn;
        return jr[0] >= 0;
      };
      static_assert(NS == 2 || NS == 3, "unrolled ring depth");
      while (jr[0] >= 0) {
        if (!step(std::integral_constant<int, 0>{})) break;
        if (!step(std::integral_constant<int, 1>{})) break;
        if constexpr (NS == 3) {
          if (!step(std::integral_constant<int, 2>{})) break;
        }
      }
    } else {
      // K and V blocks go to separate rings: LDS holds two K stages, then two V
      // stages.  Block t's K is needed one step before its V (its scores are
      // computed during step t - 1), so K is loaded two blocks ahead and V one.
      auto issue_one = [&](const char *tbase, int64_t tblk, const uint32_t (&goff)[C::LOADS], int64_t rstride, int j,
                           uint32_t lds) {
        const char *t = tbase + j * tblk;
        const uint32_t l = uni(lds + wave * C::LOADS * 1024);
        if constexpr (VL) {
          if ((j + 1) * 64 > seq_len) {
            // the sequence's last, partial block: rows past its end read the
            // last row instead (finite, in bounds; their keys are masked for
            // every query of the sequence and their queries are not stored)
            const int last = seq_len - 1 - j * 64;
#pragma unroll
            for (int n = 0; n < C::LOADS; ++n) {
              const int rr = ((wave * C::LOADS + n) * 1024 + lane * 16) / C::ROWB;
              const int back = max(rr - last, 0);
              dma16(t, goff[n] - (uint32_t)(back * rstride * 2), l + n * 1024);
            }
            return;
          }
        }
#pragma unroll
        for (int n = 0; n < C::LOADS; ++n) dma16(t, goff[n], l + n * 1024);
      };
      auto issue_k = [&](int j, int stage) {
        issue_one(kbase, kblk, gk, kernarg_params()->ks[2], j, smem_lds + stage * C::TILEB);
      };
      auto issue_v = [&](int j, int stage) {
        issue_one(vbase, vblk, gv, kernarg_params()->vs[2], j, smem_lds + (2 + stage) * C::TILEB);
      };

      // scores of the block being finished (sacc[P]) and of the next (sacc[P^1])
      f32x16 sacc[2][2];

      // S^T = K Q^T of the block in K stage kst into s.  MFMA n takes key half
      // n & 1 and D slice n >> 1 (consecutive products are independent); its K
      // operand is read kRead products ahead from a small ring of registers.
      // `slot(n)` is issued after MFMA n: the caller's vector work to overlap.
      constexpr int kRead = 3;
      auto scores_with = [&](int kst, f32x16 (&s)[2], auto &&slot) {
        const char *kl = smem + kst * C::TILEB;
        constexpr int NM = 2 * (D / 16);
        bf16x8 kr[kRead];
        auto rd = [&](int n) {
          return *reinterpret_cast<const bf16x8 *>(kl + (n & 1) * 32 * C::ROWB + koff[n >> 1]);
        };
        s[0] = f32x16{};
        s[1] = f32x16{};
        static_for<0, kRead>([&](auto ic) { kr[decltype(ic)::value] = rd(decltype(ic)::value); });
        static_for<0, NM>([&](auto nc) {
          constexpr int n = decltype(nc)::value;
          s[n & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[n % kRead], qreg[n >> 1], s[n & 1], 0, 0, 0);
          if constexpr (n + kRead < NM) kr[n % kRead] = rd(n + kRead);
          slot(nc);
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      auto scores = [&](int kst, f32x16 (&s)[2]) { scores_with(kst, s, [](auto) {}); };
      auto rescale = [&](float m_new, float rs) {
        if (__any(m_new != m_run)) {
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
        }
        m_run = m_new;
        l_run += rs;
      };
      // O^T += V^T P^T with the block's V in V stage vst
      auto pv = [&](int vst, f32x16 (&s)[2]) {
        const char *vl = smem + (2 + vst) * C::TILEB;
        // P^T as bf16 B operands: chunk c = 2*kh + gg covers keys
        // 16c + {4hh..4hh+3, 8+4hh..8+4hh+3}
        bf16x8 pk[4];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            f32x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = s[kh][8 * gg + e];
            pk[2 * kh + gg] = __builtin_convertvector(f, bf16x8);
          }
        // V^T operands come from two transposed reads each; product n takes D
        // tile n % (D / 32) and key chunk n / (D / 32) (consecutive products
        // are independent), its operand read kRead products ahead
        constexpr int NT = D / 32, NM = 4 * NT;
        auto rd = [&](int n) {
          const char *a0 = vl + (16 * (n / NT)) * C::ROWB + voff[n % NT];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(a0));
          const i16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(a0 + 8 * C::ROWB));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 vr[kRead];
        static_for<0, kRead>([&](auto ic) { vr[decltype(ic)::value] = rd(decltype(ic)::value); });
        static_for<0, NM>([&](auto nc) {
          constexpr int n = decltype(nc)::value;
          oacc[n % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[n % kRead], pk[n / NT], oacc[n % NT], 0, 0, 0);
          if constexpr (n + kRead < NM) vr[n % kRead] = rd(n + kRead);
          __builtin_amdgcn_sched_barrier(0);
        });
      };

      // ---------------- pipelined walk over the union of the rows ------------
      // jr[k], mr[k]: block t+k of the union and the mask of the query blocks
      // holding it (-1: none), k = 0, 1, 2.  At step t, with both landed, block
      // t+1's scores are computed from K stage (t+1)%2 while block t's
      // probabilities and output products use its scores (computed at step
      // t-1) and V stage t%2; K of block t+2 and V of block t+1 load meanwhile.
      int jr[3], mr[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        jr[k] = -1;
        mr[k] = 0;
      }
      if (next_block(jr[0], mr[0])) {
        issue_k(jr[0], 0);
        issue_v(jr[0], 0);
        if (next_block(jr[1], mr[1])) issue_k(jr[1], 1);
      }
      const int my_bit = 1 << my_qb;
      if (jr[0] >= 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (wave_on && (mr[0] & my_bit)) scores(0, sacc[0]);
      }
      // One step per block, unrolled over the two stage parities so that the
      // LDS operand addresses fold into the instructions' immediate offsets.
      auto step = [&](auto par_c) -> bool {
        constexpr int P = decltype(par_c)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K of t+1 and V of t
        __syncthreads();  // every wave is past step t-1: K stage P and V stage P^1 are free
        if (next_block(jr[2], mr[2])) issue_k(jr[2], P);
        if (jr[1] >= 0) issue_v(jr[1], P ^ 1);
        // This wave's work on block t exists when its row holds block t; the
        // next block's scores are computed whatever (from stale LDS when there
        // is none, then unused), so that the step is one block of code in which
        // the score products and this block's exponentials interleave.
        const bool cur = wave_on && (mr[0] & my_bit);
        // keys above lim are masked (the diagonal block only; 64 masks none)
        const int lim = jr[0] == my_i ? row_in_blk - 4 * hh : 64;
        f32x16 (&sc)[2] = sacc[P];
        constexpr int kMaxSlots = 6, kPerMax = 6, kPerExp = 4;
        float mx = -INFINITY, m_new = 0.f, neg_m = 0.f, rs = 0.f;
        scores_with(P ^ 1, sacc[P ^ 1], [&](auto nc) {
          constexpr int n = decltype(nc)::value;
          if constexpr (n < kMaxSlots) {
#pragma unroll
            for (int x = n * kPerMax; x < (n + 1) * kPerMax && x < 32; ++x) {
              const int key = (x >> 4) * 32 + 8 * ((x & 15) >> 2) + (x & 3);
              sc[x >> 4][x & 15] = key > lim ? -INFINITY : sc[x >> 4][x & 15];
              mx = fmaxf(mx, sc[x >> 4][x & 15]);
            }
          } else if constexpr (n == kMaxSlots) {
            mx = swap_halves_max(mx) * c2;
            m_new = mx > m_run ? mx : m_run;
            neg_m = -m_new;
          } else {
            constexpr int x0 = (n - kMaxSlots - 1) * kPerExp;
#pragma unroll
            for (int x = x0; x < x0 + kPerExp && x < 32; ++x) {
              sc[x >> 4][x & 15] = __builtin_amdgcn_exp2f(fmaf(sc[x >> 4][x & 15], c2, neg_m));
              rs += sc[x >> 4][x & 15];
            }
          }
        });
        if constexpr (2 * (D / 16) - kMaxSlots - 1 < 32 / kPerExp) {
          // D = 64 has fewer score products than the exponentials need slots:
          // the elements left over
#pragma unroll
          for (int x = (2 * (D / 16) - kMaxSlots - 1) * kPerExp; x < 32; ++x) {
            sc[x >> 4][x & 15] = __builtin_amdgcn_exp2f(fmaf(sc[x >> 4][x & 15], c2, neg_m));
            rs += sc[x >> 4][x & 15];
          }
        }
        if (cur) {
          rescale(m_new, rs);
          pv(P, sc);
        }
        jr[0] = jr[1];
        mr[0] = mr[1];
        jr[1] = jr[2];
        mr[1] = mr[2];
        jr[2] = -1;
        mr[2] = 0;
        return jr[0] >= 0;
      };
      while (jr[0] >= 0) {
        if (!step(std::integral_constant<int, 0>{})) break;
        if (!step(std::integral_constant<int, 1>{})) break;
      }
    }

    // ---------------- epilogue ---------------------------------------------
    if (wave_on) {
      const float l_tot = swap_halves_sum(l_run);
      const int64_t qrow = (int64_t)my_i * 64 + row_in_blk;
      const bool store = !VL || qrow < seq_len;
      // a row with no active block (possible in a caller-built layout) has
      // l = 0 and m = -inf: output 0, logsumexp -inf
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      __bf16 *orow = static_cast<__bf16 *>(kernarg_params()->o) + b * kernarg_params()->os[0] + h * kernarg_params()->os[1] + (tok0 + qrow) * kernarg_params()->os[2];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          f32x4 f;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = oacc[dt][4 * gi + e] * inv;
          const bf16x4 ob = __builtin_convertvector(f, bf16x4);
          if (store) *reinterpret_cast<bf16x4 *>(orow + dt * 32 + 8 * gi + 4 * hh) = ob;
        }
      if (kernarg_params()->lse && hh == 0 && store) {
        const int64_t li = VL ? (int64_t)h * kernarg_params()->T_total + tok0 + qrow
                              : ((int64_t)b * kernarg_params()->H + h) * kernarg_params()->N + qrow;
        kernarg_params()->lse[li] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
      }
    }
  }  // item loop
}



// launch tags of the work queues: distinct for 2^32 consecutive launches of the process
std::atomic<unsigned> g_launch_tag{0x5a17u};

template <int D, int QB, int NS, bool VL, bool PIPE>
hipError_t launch_fwd_bf16_t(FwdParams p, hipStream_t stream) {
  const int64_t ngrp = (p.nqb + QB - 1) / QB;
  const int64_t items = ngrp * p.B * p.H;
  if ((int64_t)(p.B * p.H + kXcds - 1) / kXcds * ngrp >= (1 << 24)) return hipErrorInvalidValue;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  // persistent: as many workgroups per CU as the LDS ring allows, each taking
  // items until every queue is empty
  const int64_t grid = std::min<int64_t>(items, (int64_t)FwdCfg<D, QB, NS>::WGS_PER_CU * cus);
  p.tag = g_launch_tag.fetch_add(1, std::memory_order_relaxed);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NS, VL, PIPE>), dim3((unsigned)grid), dim3(128 * QB), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// compute units of the current device (cached per device)
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Shapes: 2 query blocks (4 waves, one per SIMD) per workgroup and a 2-stage
// ring (64 KB of LDS) at D = 128, so two workgroups share a CU.  Their
// barriers are independent, so the two waves of a SIMD drift apart and the
// matrix phase of one overlaps the softmax of the other; the union of two
// rows wastes fewer wave steps than a wider group.  D = 64 blocks are half
// the size: a 3-stage ring, still two workgroups per CU.
//
// S2ATTN_FWD_PIPELINED=1 in the environment selects the software-pipelined
// schedule instead (the next block's scores under this block's softmax, split
// K and V rings in the same LDS); it computes the same result and is slower
// on MI355X, kept selectable so that the comparison can be measured again.
template <bool VL, bool PIPE>
hipError_t launch_fwd_bf16_d(const FwdParams &p, int D, hipStream_t stream) {
  if (D == 128) return launch_fwd_bf16_t<128, 2, 2, VL, PIPE>(p, stream);
  if (D == 64) return launch_fwd_bf16_t<64, 2, PIPE ? 2 : 3, VL, PIPE>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const FwdParams &p, int D, hipStream_t stream) {
  const char *e = getenv("S2ATTN_FWD_PIPELINED");
  const bool pipe = e && e[0] == '1' && e[1] == 0;
  if (p.cu_seqlens) return pipe ? launch_fwd_bf16_d<true, true>(p, D, stream) : launch_fwd_bf16_d<true, false>(p, D, stream);
  return pipe ? launch_fwd_bf16_d<false, true>(p, D, stream) : launch_fwd_bf16_d<false, false>(p, D, stream);
}

}  // namespace s2
