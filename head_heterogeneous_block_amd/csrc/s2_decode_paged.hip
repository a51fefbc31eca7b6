// Serving decode: one query token per sequence against a paged K/V cache,
// with several query heads sharing one K/V head.
//
// The S2-Attention OpenReview abstract reports serving with the method in
// vLLM; vLLM keeps the K/V cache in fixed-size pages addressed through a
// per-sequence block table (PagedAttention, in the "Builds on" list of the
// S2-Attention arXiv record, mlsanity page).  Token t of sequence b is row
// t mod P of page block_table[b][t / P]; query head h reads K/V head
// h / (H / H_kv) (grouped-query attention; one K/V head is multi-query
// attention).  The attention itself is the decode of the contiguous path:
// keys t <= p (p = seq_len - 1) of the blocks active for (h, p / 64).
//
// Mapping onto the GPU:
//  * A workgroup serves GQ query heads of one K/V head (a "unit": sequence,
//    K/V head, chunk of GQ heads of its group) and walks the union of their
//    CSR rows in ascending block order.  A block several of them select (the
//    shared local window; every block when one is dense) is read from HBM once
//    and scored for each head that selects it.
//  * Within a block, the lanes read 16-byte slices of key rows as in the
//    contiguous kernel (LPR lanes per row, RPI rows per round); every lane
//    looks up the page of its own row in the block table (the table row of a
//    sequence is a few cached bytes).  A page id outside [0, num_pages) reads
//    as NaN, so a corrupt table poisons exactly the heads that use that block
//    and never reads out of bounds.
//  * The vector ALU does the products: scores of bf16 keys are v_dot2_f32_bf16
//    on the packed query and key slices (no conversion of K), the output a
//    multiply-add per key and channel, plus the reductions and exponentials.
//    Over the layout's rows a workgroup serves two heads (the heads' strided
//    blocks differ, so the union of four rows is long and four heads are bound
//    by the vector ALU); over query-aware lists it serves four, so that each
//    (sequence, K/V head)'s union of kept blocks is read once.
//  * Splits: each head's CSR row is cut into `splits` contiguous runs and a
//    workgroup walks run s of each of its heads; a second launch merges the
//    partial results by logsumexp (Lean Attention abstract, on the
//    SampleAttention page).  Merging in the last workgroup to finish instead
//    needs a device-scope fence per workgroup, which on this GPU writes back
//    and invalidates the XCD's L2 and made the launch several times slower.
#include "s2_decode_common.h"

namespace s2 {
namespace {

using namespace decode_detail;

constexpr int kNoBlock = 0x7fffffff;

template <typename T>
struct NanBits;
template <>
struct NanBits<__bf16> {
  static constexpr unsigned v = 0x7fc07fc0u;
};
template <>
struct NanBits<float> {
  static constexpr unsigned v = 0x7fc00000u;
};

template <typename T, int D, int GQ, bool DIRECT>
__global__ __launch_bounds__(kThreads) void decode_paged_kernel(PagedParams p) {
  constexpr int EPV = Vec<T>::N;       // elements per 16-byte load
  constexpr int LPR = D / EPV;         // lanes per key row
  constexpr int RPI = kThreads / LPR;  // key rows per load round (workgroup)
  constexpr int NU = 64 / RPI;         // load rounds per block
  static_assert(LPR <= 64 && 64 % LPR == 0 && 64 % RPI == 0, "unsupported D");

  __shared__ float s_m[4][GQ], s_l[4][GQ];
  __shared__ float s_acc[4][GQ][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the workgroups of one (sequence, K/V head) run on one XCD: the blocks their
  // heads' rows share are fetched once into its L2
  int64_t bk;
  int r;
  xcd_group(blockIdx.x, (int64_t)p.B * p.Hkv, p.nchunk * p.splits, bk, r);
  const int chunk = r / p.splits, split = r % p.splits;
  const int kvh = (int)(bk % p.Hkv);
  const int b = (int)(bk / p.Hkv);
  const int h0 = kvh * p.group + chunk * GQ;  // first query head of the unit
  const int64_t bh0 = (int64_t)b * p.H + h0;

  const int L = p.seq_lens[b];
  if (L < 1 || (int64_t)L > ((int64_t)p.max_pages << p.page_shift)) {
    // invalid length: poison the unit's rows and read nothing
    if (split == 0) {
      for (int x = tid; x < GQ * D; x += kThreads) {
        T *out = static_cast<T *>(p.o) + b * p.os[0] + (h0 + x / D) * p.os[1];
        out[x % D] = (T)NAN;
      }
      if (tid < GQ && p.lse) p.lse[bh0 + tid] = NAN;
    }
    return;
  }
  const int pos = L - 1;
  const int qb = pos >> 6;

  // run `split` of each head's CSR row
  int cur[GQ], end[GQ], nxt[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const int64_t row = p.per_seq ? bh0 + g : (int64_t)(h0 + g) * p.nqb + qb;
    const int rs = p.row_ptr[row], re = p.row_ptr[row + 1];
    const int per = (re - rs + p.splits - 1) / p.splits;
    cur[g] = min(re, rs + split * per);
    end[g] = min(re, cur[g] + per);
    nxt[g] = cur[g] < end[g] ? p.col_idx[cur[g]] : kNoBlock;
  }

  const int c = tid % LPR;     // which 16-byte slice of a row this lane reads
  const int rsub = tid / LPR;  // row within a load round
  // bf16: the query stays as packed pairs and a score is 4 v_dot2_f32_bf16 on
  // the packed key slice (no conversion of K), scaled after the cross-lane
  // sum; fp32: converted, pre-scaled and multiplied out
  constexpr bool kDot = std::is_same<T, __bf16>::value;
  u32x4 qpk[GQ];
  float qf[GQ][EPV];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const T *qp = static_cast<const T *>(p.q) + b * p.qs[0] + (h0 + g) * p.qs[1] + c * EPV;
    qpk[g] = *reinterpret_cast<const u32x4 *>(qp);
    if constexpr (!kDot) {
      Vec<T>::to_float(qpk[g], qf[g]);
#pragma unroll
      for (int e = 0; e < EPV; ++e) qf[g][e] *= p.scale_log2;
    }
  }
  const T *kb = static_cast<const T *>(p.kp) + kvh * p.kps[1] + c * EPV;
  const T *vb = static_cast<const T *>(p.vp) + kvh * p.vps[1] + c * EPV;
  const int32_t *table = p.block_table + b * p.bt_stride;
  const int pmask = (1 << p.page_shift) - 1;

  float m_run[GQ], l_run[GQ], acc[GQ][EPV];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[g][e] = 0.f;
  }

  // next block of the union of the runs and the heads that select it
  // (kNoBlock when the runs are done)
  auto advance = [&](unsigned &sel) -> int {
    int j = kNoBlock;
#pragma unroll
    for (int g = 0; g < GQ; ++g) j = min(j, nxt[g]);
    sel = 0;
    if (j == kNoBlock) return j;
#pragma unroll
    for (int g = 0; g < GQ; ++g)
      if (nxt[g] == j) {
        sel |= 1u << g;
        ++cur[g];
        nxt[g] = cur[g] < end[g] ? p.col_idx[cur[g]] : kNoBlock;
      }
    return j;
  };
  // pages of this lane's rows of block j (-1: past the query, never read);
  // looked up one block ahead so that the table read is off the load path
  auto lookup = [&](int j, int *pg) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = j * 64 + u * RPI + rsub;
      pg[u] = (j != kNoBlock && j >= 0 && t <= pos) ? table[t >> p.page_shift] : -1;
    }
  };
  unsigned sel_cur;
  int j_cur = advance(sel_cur);
  int pg_cur[NU];
  lookup(j_cur, pg_cur);

  while (j_cur != kNoBlock) {
    const int j = j_cur;
    const unsigned sel = sel_cur;
    u32x4 kv[NU], vv[NU];
    bool ok[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = j * 64 + u * RPI + rsub;
      ok[u] = t <= pos && j >= 0;  // tokens past the query (or before token 0) are never looked up
      const u32x4 nanv = {NanBits<T>::v, NanBits<T>::v, NanBits<T>::v, NanBits<T>::v};
      kv[u] = vv[u] = u32x4{};
      if (ok[u]) {
        const int page = pg_cur[u];
        if ((unsigned)page < (unsigned)p.num_pages) {
          const int64_t r = t & pmask;
          kv[u] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4 *>(kb + page * p.kps[0] + r * p.kps[2]));
          vv[u] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4 *>(vb + page * p.vps[0] + r * p.vps[2]));
        } else {
          kv[u] = vv[u] = nanv;
        }
      }
    }
    j_cur = advance(sel_cur);
    lookup(j_cur, pg_cur);
    float kf[NU][EPV], vf[NU][EPV];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if constexpr (!kDot) Vec<T>::to_float(kv[u], kf[u]);
      Vec<T>::to_float(vv[u], vf[u]);
    }

#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      if (!((sel >> g) & 1u)) continue;
      float s[NU];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float a = 0.f;
        if constexpr (kDot) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const unsigned qw = qpk[g][x], kw = kv[u][x];  // scalars: a bit cast of a vector element read element 0
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw), __builtin_bit_cast(bf16x2, kw), a, false);
          }
          a = group_sum<LPR>(a) * p.scale_log2;
        } else {
#pragma unroll
          for (int x = 0; x < EPV; ++x) a = fmaf(qf[g][x], kf[u][x], a);
          a = group_sum<LPR>(a);
        }
        s[u] = ok[u] ? a : -INFINITY;
        mx = nan_max(mx, s[u]);
      }
      mx = across_groups_max<LPR>(mx);
      const float m_new = nan_max(m_run[g], mx);
      if (m_new == -INFINITY) continue;  // no visible key for this wave yet (NaN stays NaN)
      const float alpha = exp2f(m_run[g] - m_new);
      m_run[g] = m_new;
      l_run[g] *= alpha;
#pragma unroll
      for (int x = 0; x < EPV; ++x) acc[g][x] *= alpha;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float pu = exp2f(s[u] - m_new);
        l_run[g] += pu;
#pragma unroll
        for (int x = 0; x < EPV; ++x) acc[g][x] = fmaf(pu, vf[u][x], acc[g][x]);
      }
    }
  }

  // combine the rows of each wave (lanes with the same slice c), then the waves
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const float l = across_groups_sum<LPR>(l_run[g]);
#pragma unroll
    for (int x = 0; x < EPV; ++x) acc[g][x] = across_groups_sum<LPR>(acc[g][x]);
    if (lane < LPR) {
#pragma unroll
      for (int x = 0; x < EPV; ++x) s_acc[wave][g][c * EPV + x] = acc[g][x];
      if (lane == 0) {
        s_m[wave][g] = m_run[g];
        s_l[wave][g] = l;
      }
    }
  }
  __syncthreads();
  for (int x = tid; x < GQ * D; x += kThreads) {
    const int g = x / D, d = x % D;
    const float mw = fmaxf(fmaxf(s_m[0][g], s_m[1][g]), fmaxf(s_m[2][g], s_m[3][g]));
    float wsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // a wave that saw no visible key has m = -inf and weight 0
      const float wgt = s_m[w][g] == -INFINITY ? 0.f : exp2f(s_m[w][g] - mw);
      wsum = fmaf(s_l[w][g], wgt, wsum);
      o = fmaf(s_acc[w][g][d], wgt, o);
    }
    const int64_t bh = bh0 + g;
    if constexpr (DIRECT) {
      T *out = static_cast<T *>(p.o) + b * p.os[0] + (h0 + g) * p.os[1];
      // wsum is 0 only for an empty row (output 0, logsumexp -inf); a NaN
      // from a bad page or a NaN input reaches both o and wsum and stays NaN
      out[d] = (T)(wsum == 0.f ? 0.f : o / wsum);
      if (d == 0 && p.lse) p.lse[bh] = (mw + __log2f(wsum)) * 0.69314718055994531f;
    } else {
      // an empty run leaves m = -inf, l = 0: partial 0 with weight 0 in the
      // merge (a NaN max, from a NaN score, passes through to the merge)
      p.part_o[(bh * p.splits + split) * D + d] = mw == -INFINITY ? 0.f : o / wsum;
      if (d == 0) p.part_lse[bh * p.splits + split] = mw == -INFINITY ? -INFINITY : mw + __log2f(wsum);
    }
  }
}

// merge: one workgroup of D threads per (sequence, query head)
template <typename T, int D>
__global__ __launch_bounds__(D) void paged_merge_kernel(PagedParams p) {
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % p.H);
  const int b = (int)(bh / p.H);
  const int L = p.seq_lens[b];
  if (L < 1 || (int64_t)L > ((int64_t)p.max_pages << p.page_shift)) return;  // written by the split kernel
  const int d = threadIdx.x;
  const float *pl = p.part_lse + bh * p.splits;
  const float *po = p.part_o + bh * p.splits * D;
  float mx = -INFINITY;
  bool bad = false;
  for (int s = 0; s < p.splits; ++s) {
    const float y = pl[s];
    bad |= y != y;
    mx = fmaxf(mx, y);
  }
  float wsum = 0.f, o = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float y = pl[s];
    const float w = y == -INFINITY ? 0.f : exp2f(y - mx);
    wsum += w;
    o = fmaf(w, po[s * D + d], o);
  }
  T *out = static_cast<T *>(p.o) + b * p.os[0] + h * p.os[1];
  out[d] = (T)(bad ? NAN : (wsum > 0.f ? o / wsum : 0.f));
  if (d == 0 && p.lse) p.lse[bh] = bad ? NAN : (mx + __log2f(wsum)) * 0.69314718055994531f;
}

template <typename T, int D, int GQ>
hipError_t launch_gq(const PagedParams &p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.B * p.Hkv * p.nchunk * p.splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (p.splits == 1) {
    hipLaunchKernelGGL((decode_paged_kernel<T, D, GQ, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_paged_kernel<T, D, GQ, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((paged_merge_kernel<T, D>), dim3((unsigned)((int64_t)p.B * p.H)), dim3(D), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const PagedParams &p, hipStream_t stream) {
  switch (p.group / p.nchunk) {
    case 1: return launch_gq<T, D, 1>(p, stream);
    case 2: return launch_gq<T, D, 2>(p, stream);
    case 4: return launch_gq<T, D, 4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Query heads per workgroup.  Over the layout's rows two (four would be bound
// by the vector ALU: the heads' strided blocks differ, so the union of four
// rows is long); over query-aware lists four, so that each (sequence, K/V
// head)'s union is read once.
int paged_heads_per_group(int group, bool per_seq) {
  if (per_seq && group % 4 == 0) return 4;
  return group % 2 == 0 ? 2 : 1;
}

hipError_t launch_decode_paged(const PagedParams &p, s2_dtype dtype, int D, hipStream_t stream) {
  if (dtype == S2_BF16) {
    if (D == 128) return launch_t<__bf16, 128>(p, stream);
    if (D == 64) return launch_t<__bf16, 64>(p, stream);
  } else {
    if (D == 128) return launch_t<float, 128>(p, stream);
    if (D == 64) return launch_t<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace s2
