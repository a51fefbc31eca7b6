// Internal declarations shared by the HIP translation units of libs2attn.
// Not part of the public ABI (include/s2attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/s2attn.h"

namespace s2 {

constexpr int kBlock = S2_BLOCK;
constexpr int kMaxDenseHeads = 1024;  // dense flags travel as a bitmask in kernel arguments

// ---------------------------------------------------------------------------
// HHST layout in closed form.  Head h, query block i, window W, stride S:
//   active(j) = dense[h] or i - j < W or (j + h) % S == 0,   0 <= j <= i
// A sparse row is the strided blocks left of the window followed by the
// window itself; every quantity below follows from counting those two parts.
// ---------------------------------------------------------------------------
struct PatternArgs {
  int32_t H, nqb, W, S;
  uint32_t dense_bits[kMaxDenseHeads / 32];
};

__host__ __device__ inline bool pattern_dense(const PatternArgs &p, int h) {
  return (p.dense_bits[h >> 5] >> (h & 31)) & 1u;
}

// first block of head h's strided residue class: smallest j >= 0 with (j + h) % S == 0
__host__ __device__ inline int64_t strided_first(int64_t h, int64_t S) { return (S - h % S) % S; }

// number of strided blocks strictly left of the window of query block i
__host__ __device__ inline int64_t strided_left_count(int64_t h, int64_t i, int64_t W, int64_t S) {
  int64_t m = i - W;  // strided blocks outside the window satisfy j <= i - W
  int64_t rho = strided_first(h, S);
  return m < rho ? 0 : (m - rho) / S + 1;
}

__host__ __device__ inline int64_t row_count(const PatternArgs &p, int64_t h, int64_t i) {
  if (pattern_dense(p, (int)h)) return i + 1;
  int64_t win = i + 1 < p.W ? i + 1 : p.W;
  return win + strided_left_count(h, i, p.W, p.S);
}

// sum of row_count(h, i) over i in [0, i0)
__host__ __device__ inline int64_t row_prefix(const PatternArgs &p, int64_t h, int64_t i0) {
  if (i0 <= 0) return 0;
  if (pattern_dense(p, (int)h)) return i0 * (i0 + 1) / 2;
  const int64_t W = p.W, S = p.S;
  int64_t win = i0 <= W ? i0 * (i0 + 1) / 2 : W * (W + 1) / 2 + (i0 - W) * W;
  // rows i >= W + rho contribute floor((i - W - rho) / S) + 1 strided blocks
  int64_t n = i0 - W - strided_first(h, S);  // number of such rows
  int64_t str = 0;
  if (n > 0) {
    int64_t q = n / S, r = n % S;
    str = n + S * q * (q - 1) / 2 + q * r;
  }
  return win + str;
}

// Column view of the same rule: the query blocks i >= j whose row holds key
// block j are i in [j, nqb) when the head is dense or j is on the head's
// stride, else the W blocks whose window reaches j: i in [j, j + W).
__host__ __device__ inline bool strided_block(int64_t h, int64_t j, int64_t S) { return (j + h) % S == 0; }
__host__ __device__ inline int64_t col_count(const PatternArgs &p, int64_t h, int64_t j) {
  const int64_t rest = p.nqb - j;
  if (pattern_dense(p, (int)h) || strided_block(h, j, p.S)) return rest;
  return rest < p.W ? rest : p.W;
}

// max that propagates NaN (fmaxf drops it): NaN inputs must give NaN outputs
__device__ inline float nan_max(float a, float b) { return (a != a || a > b) ? a : b; }

// ---------------------------------------------------------------------------
// launch parameter blocks
// ---------------------------------------------------------------------------
struct FwdParams {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int64_t qs[4], ks[4], vs[4], os[4];
  const int32_t *row_ptr, *col_idx;
  int32_t B, H, N, nqb;
  float scale_log2;  // softmax scale * log2(e): the kernels work in base 2
  // work queues of the persistent launch (caller workspace, kFwdWorkspaceBytes)
  // and this launch's tag in them (set by the launcher)
  unsigned long long *queue;
  uint32_t tag;
  // packed variable-length batches: sequence b is tokens [cu_seqlens[b],
  // cu_seqlens[b + 1]) of a [T_total, H, D] tensor (strides [0, head, token, 1]);
  // LSE is [H, T_total].  NULL for fixed-length batches.
  const int32_t *cu_seqlens;
  int32_t T_total;
};

struct DecodeParams {
  const void *q, *kc, *vc;
  void *o;
  float *lse;
  int64_t qs[3], ks[4], vs[4], os[3];
  const int32_t *row_ptr, *col_idx, *seq_lens;
  int32_t B, H, nqb, cache_len, splits;
  int32_t per_seq;  // 1: row b * H + h of the CSR lists the blocks of (b, h); 0: row h * nqb + p / 64
  float scale_log2;
  float *part_o;    // [B, H, splits, D] fp32
  float *part_lse;  // [B, H, splits] fp32, base-2 logsumexp
};

// Per-block channel minima and maxima of the keys (query-aware block lists).
struct MinmaxParams {
  const void *k;
  int64_t ks[4];  // contiguous cache [B, H, cache_len, D], or pages [page, H, row in page, D]
  const int32_t *seq_lens;
  void *kmin, *kmax;  // [B, H, nblk, D] contiguous, the keys' dtype
  int32_t B, H, nblk, cache_len;  // paged: cache_len = max_pages * page size
  const int32_t *block_table;  // paged only: [B, bt_stride], entry t >> page_shift = page of token t
  int64_t bt_stride;
  int32_t num_pages, page_shift;
};

// Top-budget block lists per (sequence, head) from the block bounds.
constexpr int kMaxSelectBlocks = 16000;  // one 32-bit key per block in LDS, with the kernel's own 1 KiB under 64 KiB
struct SelectParams {
  const void *q;
  int64_t qs[3];
  const void *kmin, *kmax;  // [B, H, nblk, D] contiguous
  const int32_t *seq_lens;
  int32_t *row_ptr, *col_idx;  // [B * H + 1], [B * H * min(budget, ...)]
  int32_t B, H, nblk, cache_len, budget;
  int32_t Hkv, group;  // bounds of K/V head h / group serve query head h (kmin: [B, Hkv, nblk, D])
};

// Serving decode: paged K/V cache, query heads grouped over fewer KV heads.
struct PagedParams {
  const void *q, *kp, *vp;
  void *o;
  float *lse;
  int64_t qs[3], kps[4], vps[4], os[3];  // pages: [page, kv head, row in page, d]
  const int32_t *row_ptr, *col_idx, *seq_lens;
  const int32_t *block_table;  // [B, bt_stride], entry t >> page_shift = page of token t
  int64_t bt_stride;
  int32_t B, H, Hkv, group, nchunk, nqb, splits, num_pages, max_pages, page_shift;
  int32_t per_seq;  // 1: row b * H + h of the CSR lists the blocks of (b, h); 0: row h * nqb + p / 64
  float scale_log2;
  float *part_o;    // [B, H, splits, D] fp32
  float *part_lse;  // [B, H, splits] fp32, base-2 logsumexp
};

struct BwdParams {
  const void *q, *k, *v, *o, *dout;
  void *dq, *dk, *dv;
  const float *lse;  // [B, H, N] natural-log logsumexp of the forward
  float *delta;      // [B, H, N] workspace: rowsum(dO * O)
  float *nlse2;      // [B, H, N] workspace: -LSE * log2(e)
  int32_t *plan_kv;  // [B * H * nqb] workspace: dK/dV work items in launch order
  int32_t *plan_q;   // [B * H * ceil(nqb / 2)] workspace: dQ work items in launch order
  int64_t qs[4], ks[4], vs[4], os[4], dos[4], dqs[4], dks[4], dvs[4];
  const int32_t *row_ptr, *col_idx;  // layout: key blocks per query block
  const int32_t *col_ptr, *row_idx;  // column view: query blocks per key block
  int32_t B, H, N, nqb;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
};

// XCDs of the GPU, each with its own L2; workgroups go to them round-robin.
constexpr int kXcds = 8;

// The forward's workspace: one work-queue word per XCD, each on its own
// 128-byte line.
constexpr int kFwdQueueStride = 128;
constexpr size_t kFwdWorkspaceBytes = (size_t)kXcds * kFwdQueueStride;

// Workgroup n of a launch of units * m workgroups -> (unit, member).  Workgroups
// reach XCD n % kXcds; when units is a multiple of kXcds every member of a unit
// lands on the same XCD (and so shares its L2), otherwise the plain order
// n = unit * m + member is used.  Either way the map is one-to-one.
__device__ __forceinline__ void xcd_group(int64_t n, int64_t units, int m, int64_t &unit, int &member) {
  if (m == 1 || units % kXcds != 0) {
    unit = n / m;
    member = (int)(n % m);
    return;
  }
  const int64_t slot = n / kXcds;
  unit = (slot / m) * kXcds + n % kXcds;
  member = (int)(slot % m);
}
// The backward's workspace: delta and -LSE*log2(e) ([B, H, N] fp32 each), then
// the work plans of the dK/dV and dQ kernels (one int32 per key block and per
// pair of query blocks of every (b, h)).
inline size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) {
  const int64_t nqb = N / 64;
  return 2 * (size_t)(B * H * N) * sizeof(float) + (size_t)(B * H * (nqb + (nqb + 1) / 2)) * sizeof(int32_t);
}

// compute units of the current device (0 if none is visible); cached per device
int device_cus();

// devices whose per-device lookups the library caches
constexpr int kMaxDevices = 64;

// device address of the allocation-free decode's static scratch
// (S2_NOALLOC_SCRATCH_BYTES) on the current device
hipError_t decode_scratch(void **ptr);

hipError_t launch_build_layout(const PatternArgs &p, int32_t *row_ptr, int32_t *col_idx,
                               hipStream_t stream);
hipError_t launch_build_layout_t(const PatternArgs &p, int32_t *col_ptr, int32_t *row_idx,
                                 hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams &p, int D, hipStream_t stream);

// caller-built layouts
enum LayoutFault { kLayoutBadStart = 1, kLayoutBadEnd, kLayoutBadPtr, kLayoutBadBlock, kLayoutUnsorted };
hipError_t launch_validate_layout(const int32_t *row_ptr, const int32_t *col_idx, int32_t num_heads,
                                  int32_t nqb, int64_t nnz, unsigned long long *first, hipStream_t stream);
int64_t transpose_bitmap_words(int32_t num_heads, int32_t nqb);
hipError_t launch_transpose_layout(const int32_t *row_ptr, const int32_t *col_idx, int32_t num_heads,
                                   int32_t nqb, int64_t nnz, int32_t *col_ptr, int32_t *row_idx, uint32_t *bits,
                                   hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams &p, int D, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams &p, int D, hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, s2_dtype dtype, int D, hipStream_t stream);
hipError_t launch_block_minmax(const MinmaxParams &p, s2_dtype dtype, int D, hipStream_t stream);
hipError_t launch_select_blocks(const SelectParams &p, s2_dtype dtype, int D, hipStream_t stream);
int paged_heads_per_group(int group, bool per_seq);  // query heads one paged-decode workgroup serves
hipError_t launch_decode_paged(const PagedParams &p, s2_dtype dtype, int D, hipStream_t stream);

}  // namespace s2
