// Block-sparse causal attention forward in fp32 (fp32 in, fp32 out).
//
// The fp32 path exists for full-precision checks (max-abs error 1e-4 against
// an fp64 reference rules out rounding products to bf16).  It is a plain
// vector-ALU kernel: one workgroup of 4 waves per (batch, head, query block),
// one query row per lane with its q vector and output accumulator in
// registers.  The 4 waves stage each active K/V block of the CSR row in LDS
// together, and wave w then takes keys 16w .. 16w+15 of it, read as LDS
// broadcasts, with its own running max, sum and output; at the end the 4
// partial results of every query are merged by their maxima (the same rule as
// the split decode's merge).  The online softmax is the same as in the bf16
// MFMA kernel (running max and sum in base 2, one exp per score), so the two
// paths compute the same quantity.
#include "s2_internal.h"

namespace s2 {
namespace {

constexpr int kWavesF32 = 4;
constexpr int kKeysPerWave = 64 / kWavesF32;

template <int D>
__global__ __launch_bounds__(64 * kWavesF32) void fwd_f32_kernel(FwdParams p) {
  // K and V of the current block; after the walk, the merge's exchange space
  __shared__ __attribute__((aligned(16))) float ks[64][D];
  __shared__ __attribute__((aligned(16))) float vs[64][D];
  __shared__ float s_m[kWavesF32][64], s_l[kWavesF32][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t item = blockIdx.x;
  const int i = (int)(item % p.nqb);
  const int64_t bh = item / p.nqb;
  const int h = (int)(bh % p.H);
  const int b = (int)(bh / p.H);

  const float *qbase = static_cast<const float *>(p.q) + b * p.qs[0] + h * p.qs[1];
  const float *kbase = static_cast<const float *>(p.k) + b * p.ks[0] + h * p.ks[1];
  const float *vbase = static_cast<const float *>(p.v) + b * p.vs[0] + h * p.vs[1];
  const int64_t qpos = (int64_t)i * 64 + lane;

  float q[D], acc[D];
  const float *qrow = qbase + qpos * p.qs[2];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qrow[d] * p.scale_log2;  // scores come out scaled, in base 2
    acc[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t row = (int64_t)h * p.nqb + i;
  const int beg = p.row_ptr[row], end = p.row_ptr[row + 1];
  const int t0 = wave * kKeysPerWave;  // this wave's keys of every block
  for (int e = beg; e < end; ++e) {
    const int j = p.col_idx[e];
    __syncthreads();  // every wave is done with the previous block
    for (int idx = tid; idx < 64 * D / 4; idx += 64 * kWavesF32) {
      const int r = idx / (D / 4), c = idx % (D / 4);
      *reinterpret_cast<float4 *>(&ks[r][c * 4]) =
          *reinterpret_cast<const float4 *>(kbase + ((int64_t)j * 64 + r) * p.ks[2] + c * 4);
      *reinterpret_cast<float4 *>(&vs[r][c * 4]) =
          *reinterpret_cast<const float4 *>(vbase + ((int64_t)j * 64 + r) * p.vs[2] + c * 4);
    }
    __syncthreads();
    // keys beyond the query (diagonal block only) are skipped
    const int nkeys = (j == i) ? lane + 1 : 64;
    float s[kKeysPerWave];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kKeysPerWave; ++u) {
      float acc_s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc_s = fmaf(q[d], ks[t0 + u][d], acc_s);
      s[u] = (t0 + u < nkeys) ? acc_s : -INFINITY;
      mx = nan_max(mx, s[u]);
    }
    const float m_new = nan_max(m_run, mx);
    if (m_new == -INFINITY) continue;  // none of this wave's keys is visible yet (a NaN goes on)
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int u = 0; u < kKeysPerWave; ++u) {
      const float pu = exp2f(s[u] - m_new);
      l_run += pu;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(pu, vs[t0 + u][d], acc[d]);
    }
  }

  // merge the waves' partial results of each query: weights 2^(m_w - m) with
  // m the largest m_w; a wave that saw no visible key (m_w = -inf) weighs 0,
  // and a query with none at all gets output 0 and logsumexp -inf
  s_m[wave][lane] = m_run;
  s_l[wave][lane] = l_run;
  __syncthreads();  // also: every wave is done with the last K/V block
  float m = -INFINITY;
  bool nan_seen = false;
#pragma unroll
  for (int w = 0; w < kWavesF32; ++w) {
    m = fmaxf(m, s_m[w][lane]);
    nan_seen |= s_m[w][lane] != s_m[w][lane];
  }
  if (nan_seen) m = NAN;
  const float wt = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m);
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWavesF32; ++w) {
    const float mw = s_m[w][lane];
    lsum += (mw == -INFINITY) ? 0.f : exp2f(mw - m) * s_l[w][lane];
  }
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] *= wt;
  // waves 2 and 3 hand their weighted outputs to waves 0 and 1 (through the
  // K and V buffers), then wave 1 hands the sum to wave 0
  float(*xch)[D] = ks;
  if (wave >= 2) {
    float(*dst)[D] = wave == 2 ? ks : vs;
#pragma unroll
    for (int d = 0; d < D; d += 4) *reinterpret_cast<float4 *>(&dst[lane][d]) = make_float4(acc[d], acc[d + 1], acc[d + 2], acc[d + 3]);
  }
  __syncthreads();
  if (wave < 2) {
    float(*src)[D] = wave == 0 ? ks : vs;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] += src[lane][d];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int d = 0; d < D; d += 4) *reinterpret_cast<float4 *>(&xch[lane][d]) = make_float4(acc[d], acc[d + 1], acc[d + 2], acc[d + 3]);
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] += xch[lane][d];

  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // empty row: output 0, logsumexp -inf
  float *orow = static_cast<float *>(p.o) + b * p.os[0] + h * p.os[1] + qpos * p.os[2];
#pragma unroll
  for (int d = 0; d < D; d += 4)
    *reinterpret_cast<float4 *>(orow + d) =
        make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
  if (p.lse) p.lse[((int64_t)b * p.H + h) * p.N + qpos] = (m + log2f(lsum)) * 0.69314718055994531f;
}

template <int D>
hipError_t launch_t(const FwdParams &p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.B * p.H * p.nqb;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)grid), dim3(64 * kWavesF32), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams &p, int D, hipStream_t stream) {
  if (D == 128) return launch_t<128>(p, stream);
  if (D == 64) return launch_t<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace s2
