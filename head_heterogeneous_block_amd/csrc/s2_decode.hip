// Single-token decode over the active KV blocks, split-KV + logsumexp merge.
//
// Decode reads every active K/V byte once and does ~1 flop per byte, so it is
// bound by HBM bandwidth; the pages stress that KV-cache reads dominate decode
// and that scattered, non-contiguous access wastes bandwidth (Double Sparsity
// page, sections 1 and 3.2; Quest abstract on the SampleAttention page).  The
// block-sparse layout keeps every read a contiguous 64-token block (16 KiB of
// K and of V at D = 128, bf16), so the kernel streams whole blocks with
// 16-byte loads.  A (sequence, head) row is cut into `splits` contiguous runs
// of its CSR row; each run produces a partial (output, logsumexp) and a second
// kernel merges them, using the associativity of online softmax (Lean
// Attention abstract, listed on the SampleAttention page).
//
// Split kernel, per workgroup of 256 threads (4 waves): a 64-token block is
// read as NU load rounds; in each round the whole workgroup covers RPI
// consecutive key rows, LPR lanes per row, 16 bytes per lane.  A lane keeps
// the q slice matching its 16 bytes; row scores are reduced over the LPR
// lanes of the row.  Every wave keeps its own running max / sum / output
// slice, combined across the 4 waves once at the end through LDS.
#include <mutex>

#include "s2_decode_common.h"

namespace s2 {
namespace {

using namespace decode_detail;

// DIRECT: a single split per (sequence, head); the kernel then writes the
// final output and logsumexp itself and no merge pass is needed
template <typename T, int D, bool DIRECT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  constexpr int EPV = Vec<T>::N;        // elements per 16-byte load
  constexpr int LPR = D / EPV;          // lanes per key row
  constexpr int RPI = kThreads / LPR;   // key rows per load round (workgroup)
  constexpr int NU = 64 / RPI;          // load rounds per block
  static_assert(LPR <= 64 && 64 % LPR == 0 && 64 % RPI == 0, "unsupported D");

  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x % p.splits;
  const int64_t bh = blockIdx.x / p.splits;
  const int h = (int)(bh % p.H);
  const int b = (int)(bh / p.H);
  float *po = p.part_o + (bh * p.splits + split) * D;
  float *pl = p.part_lse + bh * p.splits + split;

  T *out = static_cast<T *>(p.o) + b * p.os[0] + h * p.os[1];
  const int L = p.seq_lens[b];
  if (L < 1 || L > p.cache_len) {  // invalid length: poison this row, read nothing
    if constexpr (DIRECT) {
      for (int d = tid; d < D; d += kThreads) out[d] = (T)NAN;
      if (tid == 0 && p.lse) p.lse[bh] = NAN;
    } else {
      for (int d = tid; d < D; d += kThreads) po[d] = NAN;
      if (tid == 0) *pl = NAN;
    }
    return;
  }
  const int pos = L - 1;
  const int64_t row = p.per_seq ? bh : (int64_t)h * p.nqb + pos / 64;
  const int rs = p.row_ptr[row], re = p.row_ptr[row + 1];
  const int per = (re - rs + p.splits - 1) / p.splits;
  const int beg = rs + split * per;
  const int end = min(re, beg + per);
  if (!DIRECT && beg >= end) {  // empty split: weight zero in the merge
    for (int d = tid; d < D; d += kThreads) po[d] = 0.f;
    if (tid == 0) *pl = -INFINITY;
    return;
  }

  const int c = tid % LPR;        // which 16-byte slice of a row this lane reads
  const int rsub = tid / LPR;     // row within a load round
  // bf16: the query stays as packed pairs and a score is 4 v_dot2_f32_bf16 on
  // the packed key slice (no conversion of K), scaled after the cross-lane
  // sum; fp32: converted, pre-scaled and multiplied out
  constexpr bool kDot = std::is_same<T, __bf16>::value;
  float qf[EPV];
  const u32x4 qpk = *reinterpret_cast<const u32x4 *>(static_cast<const T *>(p.q) + b * p.qs[0] + h * p.qs[1] + c * EPV);
  if constexpr (!kDot) {
    Vec<T>::to_float(qpk, qf);
#pragma unroll
    for (int e = 0; e < EPV; ++e) qf[e] *= p.scale_log2;
  }
  const T *kb = static_cast<const T *>(p.kc) + b * p.ks[0] + h * p.ks[1] + c * EPV;
  const T *vb = static_cast<const T *>(p.vc) + b * p.vs[0] + h * p.vs[1] + c * EPV;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;

  for (int e = beg; e < end; ++e) {
    const int j = p.col_idx[e];
    if (j < 0 || j > pos / 64) continue;  // no key of such a block is visible (and it may lie outside the cache)
    u32x4 kv[NU], vv[NU];
    bool ok[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = j * 64 + u * RPI + rsub;
      ok[u] = t <= pos;  // never touch tokens past the query (they may lie beyond the cache)
      if (ok[u]) {
        // each active K/V byte is read exactly once: stream it past the caches
        kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (int64_t)t * p.ks[2]));
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vb + (int64_t)t * p.vs[2]));
      } else {
        kv[u] = u32x4{};
        vv[u] = u32x4{};
      }
    }
    float s[NU];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float a = 0.f;
      if constexpr (kDot) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const unsigned qw = qpk[x], kw = kv[u][x];  // scalars: a bit cast of a vector element read element 0
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw), __builtin_bit_cast(bf16x2, kw), a, false);
        }
        a = group_sum<LPR>(a) * p.scale_log2;
      } else {
        float kf[EPV];
        Vec<T>::to_float(kv[u], kf);
#pragma unroll
        for (int x = 0; x < EPV; ++x) a = fmaf(qf[x], kf[x], a);
        a = group_sum<LPR>(a);
      }
      s[u] = ok[u] ? a : -INFINITY;
      mx = nan_max(mx, s[u]);
    }
    mx = across_groups_max<LPR>(mx);
    const float m_new = nan_max(m_run, mx);
    if (m_new == -INFINITY) continue;  // no visible key for this wave yet (NaN stays NaN)
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int x = 0; x < EPV; ++x) acc[x] *= alpha;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const float pu = exp2f(s[u] - m_new);
      l_run += pu;
      float vf[EPV];
      Vec<T>::to_float(vv[u], vf);
#pragma unroll
      for (int x = 0; x < EPV; ++x) acc[x] = fmaf(pu, vf[x], acc[x]);
    }
  }

  // combine the rows of this wave: lanes with the same slice c
  l_run = across_groups_sum<LPR>(l_run);
#pragma unroll
  for (int x = 0; x < EPV; ++x) acc[x] = across_groups_sum<LPR>(acc[x]);
  if (lane < LPR) {
#pragma unroll
    for (int x = 0; x < EPV; ++x) s_acc[wave][c * EPV + x] = acc[x];
    if (lane == 0) {
      s_m[wave] = m_run;
      s_l[wave] = l_run;
    }
  }
  __syncthreads();
  // combine the 4 waves (a wave that saw no visible key has m = -inf, weight 0)
  float mw = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float wsum = 0.f;
  float wgt[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = s_m[w] == -INFINITY ? 0.f : exp2f(s_m[w] - mw);
    wsum = fmaf(s_l[w], wgt[w], wsum);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;  // empty row: output 0, logsumexp -inf
  for (int d = tid; d < D; d += kThreads) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o = fmaf(s_acc[w][d], wgt[w], o);
    if constexpr (DIRECT) out[d] = (T)(o * inv);
    else po[d] = o * inv;
  }
  if (tid == 0) {
    if constexpr (DIRECT) {
      if (p.lse) p.lse[bh] = (mw + __log2f(wsum)) * 0.69314718055994531f;
    } else {
      *pl = mw + __log2f(wsum);
    }
  }
}

// merge: one workgroup of D threads per (sequence, head)
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % p.H);
  const int b = (int)(bh / p.H);
  const int d = threadIdx.x;
  const float *pl = p.part_lse + bh * p.splits;
  const float *po = p.part_o + bh * p.splits * D;
  float mx = -INFINITY;
  bool bad = false;
  for (int s = 0; s < p.splits; ++s) {
    const float x = pl[s];
    bad |= x != x;
    mx = fmaxf(mx, x);
  }
  float wsum = 0.f, o = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float x = pl[s];
    const float w = x == -INFINITY ? 0.f : exp2f(x - mx);
    wsum += w;
    o = fmaf(w, po[s * D + d], o);
  }
  o = bad ? NAN : (wsum > 0.f ? o / wsum : 0.f);
  T *out = static_cast<T *>(p.o) + b * p.os[0] + h * p.os[1];
  out[d] = (T)o;
  if (p.lse && d == 0) p.lse[bh] = bad ? NAN : (mx + __log2f(wsum)) * 0.69314718055994531f;
}

template <typename T, int D>
hipError_t launch_t(const DecodeParams &p, hipStream_t stream) {
  const int64_t bhs = (int64_t)p.B * p.H;
  if (bhs * p.splits > 0x7fffffff) return hipErrorInvalidValue;
  if (p.splits == 1) {
    hipLaunchKernelGGL((decode_split_kernel<T, D, true>), dim3((unsigned)bhs), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_split_kernel<T, D, false>), dim3((unsigned)(bhs * p.splits)),
                     dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)bhs), dim3(D), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Scratch of the allocation-free decode entry point (s2_attn_decode_noalloc):
// the split partials live in this static array of the library's code object,
// so that the call needs no device allocation.  Each GPU holds its own copy,
// at its own address, from the library's load until the process ends.  In host
// code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) char scratch[S2_NOALLOC_SCRATCH_BYTES];

hipError_t decode_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));  // on the current device
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams &p, s2_dtype dtype, int D, hipStream_t stream) {
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
