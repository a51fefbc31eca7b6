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
//  * A workgroup owns QB consecutive query blocks of one (batch, head)
//    (QB = 2: 128 query rows, 4 waves of 32 rows).  It walks the union of
//    their CSR rows in ascending order; every K/V block of the union is
//    staged once in LDS and consumed by the waves whose own row contains it.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns ONE query column (lane%32)
//    and 32 of its keys, so the row max / row sum need one cross-half swap
//    (v_permlane32_swap) instead of a 32-lane reduction.
//  * The output is accumulated transposed as well, O^T += V^T P^T: the
//    probabilities stay in the registers the scores came out of (bf16 B
//    operand), and every accumulator a lane holds belongs to its own query,
//    so the running-max rescale is a per-lane multiply.
//  * K is staged row-major, V transposed (V^T, keys contiguous) in LDS; both
//    use XOR swizzles at 16-byte granularity so the MFMA operand reads
//    (16 consecutive rows, same column) hit distinct banks.  Two LDS stages:
//    the global loads of block t+1 are in flight while block t is computed.
//  * Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8).
//    Query-block pairs of a head are dealt to XCDs round-robin as well, and
//    every XCD walks the heads in the same order (most active blocks first),
//    so the strided blocks of a head, shared by all its query blocks, are
//    re-read from the XCD's own L2 and the work per XCD is balanced.
#include "s2_internal.h"

namespace s2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;

// swizzle of a 16-byte chunk index for a 128-byte LDS row r: distinct banks for
// 16 consecutive rows at the same logical chunk
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 128) return r & 15;  // 256-byte rows: 16 chunks
  else return swz128(r);                   // 128-byte rows
}

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int QB>
struct FwdCfg {
  static constexpr int NW = 2 * QB;        // waves, 32 query rows each
  static constexpr int NT = 64 * NW;       // threads
  static constexpr int KROW = D * 2;       // bytes of one K row in LDS
  static constexpr int KBYTES = 64 * KROW; // K tile
  static constexpr int VBYTES = D * 128;   // V^T tile: D rows of 64 keys
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KCHUNKS = 64 * D / 8;            // 16-byte chunks of a K tile
  static constexpr int KPT = KCHUNKS / NT;              // per thread
  static constexpr int VMICRO = 16 * (D / 8);           // 4-key x 8-d micro tiles of V
  static constexpr int VPT = VMICRO >= NT ? VMICRO / NT : 1;
  static_assert(KCHUNKS % NT == 0, "K tile must split evenly over the threads");
};

template <int D, int QB>
__global__ __launch_bounds__(128 * QB) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_bf16_kernel(FwdParams p) {
  using C = FwdCfg<D, QB>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wave = tid >> 6;

  // ---------------- work item -------------------------------------------
  const int BH = p.B * p.H;
  const int npair = (p.nqb + QB - 1) / QB;
  const int ppx = (npair + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int g = slot / ppx;
  const int pair = xcd + kXcds * (ppx - 1 - slot % ppx);  // longest query blocks first
  if (pair >= npair || g >= BH) return;

  // heads in order of decreasing active-block count (ties: lower index first);
  // slot g -> (rank g / B, batch g % B)
  int *s_cnt = reinterpret_cast<int *>(smem);
  __shared__ int s_head;
  {
    const int want = g / p.B;
    for (int h = tid; h < p.H; h += C::NT)
      s_cnt[h] = p.row_ptr[(int64_t)(h + 1) * p.nqb] - p.row_ptr[(int64_t)h * p.nqb];
    __syncthreads();
    for (int h = tid; h < p.H; h += C::NT) {
      const int ch = s_cnt[h];
      int rank = 0;
      for (int h2 = 0; h2 < p.H; ++h2) {
        const int c2 = s_cnt[h2];
        rank += (c2 > ch) || (c2 == ch && h2 < h);
      }
      if (rank == want) s_head = h;
    }
    __syncthreads();
  }
  const int b = g % p.B;
  const int h = s_head;
  const int i_first = pair * QB;

  // ---------------- this wave's query rows ------------------------------
  const int my_qb = wave >> 1;
  const int my_i = i_first + my_qb;
  const bool wave_on = my_i < p.nqb;
  const int row_in_blk = (wave & 1) * 32 + l32;  // query row within its 64-row block

  const __bf16 *qbase = static_cast<const __bf16 *>(p.q) + b * p.qs[0] + h * p.qs[1];
  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + b * p.ks[0] + h * p.ks[1];
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + b * p.vs[0] + h * p.vs[1];

  // Q^T operand: lane holds Q[query][16*dc + 8*hh .. +7]
  bf16x8 qreg[D / 16];
  if (wave_on) {
    const __bf16 *qrow = qbase + (int64_t)(my_i * 64 + row_in_blk) * p.qs[2] + hh * 8;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      qreg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + dc * 16));
  } else {
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) qreg[dc] = bf16x8{};
  }

  // ---------------- CSR rows of the QB query blocks (uniform) -----------
  int rp[QB], re[QB], rc[QB];
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    if (i_first + r < p.nqb) {
      const int64_t row = (int64_t)h * p.nqb + i_first + r;
      rp[r] = p.row_ptr[row];
      re[r] = p.row_ptr[row + 1];
    } else {
      rp[r] = re[r] = 0;
    }
    rc[r] = rp[r] < re[r] ? p.col_idx[rp[r]] : 0x7fffffff;
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
        rc[r] = rp[r] < re[r] ? p.col_idx[rp[r]] : 0x7fffffff;
      }
    }
    j = jm;
    mask = m;
    return true;
  };

  // ---------------- staging: global -> registers -> LDS ------------------
  u32x4 kst[C::KPT];
  u32x4 vst[C::VPT][4];
  const bool v_loader = tid < C::VMICRO;

  auto load_tile = [&](int j) {
#pragma unroll
    for (int u = 0; u < C::KPT; ++u) {
      const int id = u * C::NT + tid;
      const int row = id / (D / 8), c = id % (D / 8);
      kst[u] = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)(j * 64 + row) * p.ks[2] + c * 8);
    }
    if (v_loader) {
#pragma unroll
      for (int u = 0; u < C::VPT; ++u) {
        const int mt = u * C::NT + tid;
        const int kg = mt & 15, dcv = mt >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vst[u][r] = *reinterpret_cast<const u32x4 *>(
              vbase + (int64_t)(j * 64 + kg * 4 + r) * p.vs[2] + dcv * 8);
      }
    }
  };

  auto store_tile = [&](int buf) {
    char *kl = smem + buf * C::STAGE;
    char *vl = kl + C::KBYTES;
#pragma unroll
    for (int u = 0; u < C::KPT; ++u) {
      const int id = u * C::NT + tid;
      const int row = id / (D / 8), c = id % (D / 8);
      *reinterpret_cast<u32x4 *>(kl + row * C::KROW + ((c ^ k_swz<D>(row)) << 4)) = kst[u];
    }
    if (v_loader) {
#pragma unroll
      for (int u = 0; u < C::VPT; ++u) {
        const int mt = u * C::NT + tid;
        const int kg = mt & 15, dcv = mt >> 4;
        // keys 4kg..4kg+3 sit in 16-key group kg/4; inside the group the key
        // order is [0-3, 8-11 | 4-7, 12-15] so that each lane half of the PV
        // MFMA reads its 8 keys as one 16-byte chunk (see the P^T layout)
        const int kw = (kg & 3) * 4;
        const int c8 = 2 * (kg >> 2) + ((kw >> 2) & 1);
        const int off8 = ((kw >> 3) & 1) * 8;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int odd = 0; odd < 2; ++odd) {
            const unsigned sel = odd ? 0x07060302u : 0x05040100u;
            u32x2 val;
            val[0] = __builtin_amdgcn_perm(vst[u][1][m], vst[u][0][m], sel);
            val[1] = __builtin_amdgcn_perm(vst[u][3][m], vst[u][2][m], sel);
            const int d = dcv * 8 + 2 * m + odd;
            *reinterpret_cast<u32x2 *>(vl + d * 128 + ((c8 ^ swz128(d)) << 4) + off8) = val;
          }
        }
      }
    }
  };

  // ---------------- accumulators -----------------------------------------
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled scores (base 2)
  float l_run = 0.f;        // this lane's share of the running sum
  const float c2 = p.scale_log2;

  auto compute = [&](int buf, int j) {
    const char *kl = smem + buf * C::STAGE;
    const char *vl = kl + C::KBYTES;
    f32x16 s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      s[kh] = f32x16{};
      const int row = kh * 32 + l32;
      const char *krow = kl + row * C::KROW;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + (((2 * dc + hh) ^ k_swz<D>(row)) << 4));
        s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[dc], s[kh], 0, 0, 0);
      }
    }
    // causal mask inside the diagonal block: key index > query index
    if (j == my_i) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kh * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key > row_in_blk) s[kh][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kh][e]);
    mx = swap_halves_max(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = exp2f(fmaf(s[kh][e], c2, -m_new));
        s[kh][e] = pe;
        rs += pe;
      }
    l_run = fmaf(l_run, alpha, rs);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    // P^T as bf16 B operands: chunk c = 2*kh + g covers keys 16c + {4hh..4hh+3, 8+4hh..8+4hh+3}
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
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int d = dt * 32 + l32;
      const char *vrow = vl + d * 128;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vrow + (((2 * c + hh) ^ swz128(d)) << 4));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[c], oacc[dt], 0, 0, 0);
      }
    }
  };

  // ---------------- main loop over the union of the rows -----------------
  int j_cur = 0, mask_cur = 0;
  next_block(j_cur, mask_cur);  // every valid row holds its diagonal block
  load_tile(j_cur);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  const int my_bit = 1 << my_qb;
  while (true) {
    int j_nxt = 0, mask_nxt = 0;
    const bool more = next_block(j_nxt, mask_nxt);
    if (more) load_tile(j_nxt);
    if (wave_on && (mask_cur & my_bit)) compute(buf, j_cur);
    if (!more) break;
    store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    j_cur = j_nxt;
    mask_cur = mask_nxt;
  }

  // ---------------- epilogue ---------------------------------------------
  if (!wave_on) return;
  const float l_tot = swap_halves_sum(l_run);
  const float inv = 1.f / l_tot;
  const int64_t qrow = (int64_t)my_i * 64 + row_in_blk;
  __bf16 *orow = static_cast<__bf16 *>(p.o) + b * p.os[0] + h * p.os[1] + qrow * p.os[2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      f32x4 f;
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = oacc[dt][4 * gi + e] * inv;
      const bf16x4 ob = __builtin_convertvector(f, bf16x4);
      *reinterpret_cast<bf16x4 *>(orow + dt * 32 + 8 * gi + 4 * hh) = ob;
    }
  if (p.lse && hh == 0)
    p.lse[((int64_t)b * p.H + h) * p.N + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

template <int D, int QB>
hipError_t launch_fwd_bf16_t(const FwdParams &p, hipStream_t stream) {
  const int npair = (p.nqb + QB - 1) / QB;
  const int ppx = (npair + kXcds - 1) / kXcds;
  const int64_t grid = (int64_t)kXcds * ppx * p.B * p.H;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB>), dim3((unsigned)grid), dim3(FwdCfg<D, QB>::NT), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams &p, int D, hipStream_t stream) {
  if (D == 128) return launch_fwd_bf16_t<128, 2>(p, stream);
  if (D == 64) return launch_fwd_bf16_t<64, 2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace s2
