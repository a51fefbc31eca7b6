// Host side of the C ABI declared in include/s2attn.h: argument validation,
// launch configuration, workspace sizing and error reporting.  Nothing here
// allocates device memory or synchronises.
#include <math.h>
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "s2_internal.h"

namespace {

thread_local char g_err[512];

s2_status fail(s2_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

s2_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return S2_OK;
  return fail(S2_EHIP, "%s: %s", what, hipGetErrorString(e));
}

s2_status check_pattern(const s2_pattern *pt, int32_t nqb, s2::PatternArgs *out) {
  if (!pt) return fail(S2_EINVAL, "pattern is NULL");
  if (pt->num_heads < 1) return fail(S2_EINVAL, "num_heads must be >= 1 (got %d)", pt->num_heads);
  if (pt->block_size != S2_BLOCK)
    return fail(S2_EUNSUPPORTED, "block_size must be %d (got %d)", S2_BLOCK, pt->block_size);
  if (pt->local_blocks < 1)
    return fail(S2_EINVAL, "local_blocks must be >= 1 (got %d)", pt->local_blocks);
  if (pt->stride < 1) return fail(S2_EINVAL, "stride must be >= 1 (got %d)", pt->stride);
  if (nqb < 1) return fail(S2_EINVAL, "num_q_blocks must be >= 1 (got %d)", nqb);
  if (pt->num_heads > s2::kMaxDenseHeads)
    return fail(S2_EUNSUPPORTED, "num_heads > %d is not supported", s2::kMaxDenseHeads);
  memset(out, 0, sizeof(*out));
  out->H = pt->num_heads;
  out->nqb = nqb;
  out->W = pt->local_blocks;
  out->S = pt->stride;
  if (pt->dense)
    for (int h = 0; h < pt->num_heads; ++h)
      if (pt->dense[h]) out->dense_bits[h >> 5] |= 1u << (h & 31);
  return S2_OK;
}

int64_t total_nnz(const s2::PatternArgs &p) {
  int64_t n = 0;
  for (int h = 0; h < p.H; ++h) n += s2::row_prefix(p, h, p.nqb);
  return n;
}

s2_status check_layout(const s2_layout *ly) {
  if (!ly) return fail(S2_EINVAL, "layout is NULL");
  if (!ly->row_ptr || !ly->col_idx) return fail(S2_EINVAL, "layout row_ptr/col_idx is NULL");
  if (ly->block_size != S2_BLOCK)
    return fail(S2_EUNSUPPORTED, "layout block_size must be %d (got %d)", S2_BLOCK, ly->block_size);
  if (ly->num_heads < 1 || ly->num_q_blocks < 1)
    return fail(S2_EINVAL, "layout needs num_heads >= 1 and num_q_blocks >= 1");
  if (ly->nnz < 1 || ly->nnz >= (int64_t(1) << 31))
    return fail(S2_EUNSUPPORTED, "layout nnz must be in [1, 2^31) (got %lld)", (long long)ly->nnz);
  if ((int64_t)ly->num_heads * ly->num_q_blocks >= (int64_t(1) << 31))
    return fail(S2_EUNSUPPORTED, "too many layout rows");
  return S2_OK;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// strides: last one must be 1, others multiples of `mult` (16-byte vector loads)
s2_status check_tensor(const char *name, const void *ptr, const int64_t *st, int ndim,
                       int64_t mult) {
  if (!ptr) return fail(S2_EINVAL, "%s is NULL", name);
  if (!st) return fail(S2_EINVAL, "%s strides are NULL", name);
  if (!aligned16(ptr)) return fail(S2_EINVAL, "%s must be 16-byte aligned", name);
  if (st[ndim - 1] != 1) return fail(S2_EINVAL, "%s: stride of the last dimension must be 1", name);
  for (int i = 0; i < ndim - 1; ++i)
    if (st[i] < 0 || st[i] % mult != 0)
      return fail(S2_EINVAL, "%s: stride %d (= %lld) must be a non-negative multiple of %lld", name,
                  i, (long long)st[i], (long long)mult);
  return S2_OK;
}

float scale_log2(float sm_scale, int D) {
  const float s = sm_scale > 0.f ? sm_scale : 1.f / sqrtf((float)D);
  return s * 1.4426950408889634f;
}

// Workgroups that fill the current device at `per_cu` per compute unit.  The
// count comes from the device (hipDeviceAttributeMultiprocessorCount); with no
// device visible (host-only sizing queries) the MI355X's 256 CUs are assumed.
int64_t fill_target(int per_cu) {
  const int cus = s2::device_cus();
  return (int64_t)(cus > 0 ? cus : 256) * per_cu;
}

int32_t auto_splits(const s2_layout *ly, int32_t B) {
  // aim at >= 8 workgroups of split work per CU, never more splits than blocks
  // in a decode row could use
  const int64_t bh = (int64_t)B * ly->num_heads;
  const int64_t target = fill_target(8);
  int64_t s = (target + bh - 1) / bh;
  const int64_t max_row = ly->num_q_blocks;
  if (s > max_row) s = max_row;
  if (s < 1) s = 1;
  return (int32_t)s;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

s2_status check_fwd_workspace(const void *ws, size_t bytes) {
  if (!ws) return fail(S2_EINVAL, "workspace is NULL (s2_attn_fwd_workspace gives its size)");
  if ((reinterpret_cast<uintptr_t>(ws) & 7) != 0) return fail(S2_EINVAL, "workspace must be 8-byte aligned");
  if (bytes < s2::kFwdWorkspaceBytes)
    return fail(S2_ECAPACITY, "workspace holds %zu bytes, the forward needs %zu", bytes, s2::kFwdWorkspaceBytes);
  return S2_OK;
}

size_t decode_ws_bytes(int64_t bh, int32_t splits, int32_t D) {
  return align256((size_t)bh * splits * D * sizeof(float)) + align256((size_t)bh * splits * sizeof(float));
}

struct PagedShape {  // the paged decode's launch shape
  int32_t group, nchunk, splits;
  int64_t units;
};

// H query heads; rows hold at most row_cap blocks (the automatic split count's cap)
s2_status paged_shape(int32_t H, int32_t row_cap, int32_t B, int32_t num_kv_heads, int32_t splits,
                      bool per_seq, PagedShape *ps) {
  if (B < 1 || H < 1) return fail(S2_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (num_kv_heads < 1 || H % num_kv_heads != 0)
    return fail(S2_EINVAL, "num_kv_heads (%d) must divide the %d query heads", num_kv_heads, H);
  ps->group = H / num_kv_heads;
  ps->nchunk = ps->group / s2::paged_heads_per_group(ps->group, per_seq);
  ps->units = (int64_t)B * num_kv_heads * ps->nchunk;
  int64_t s = splits;
  if (s <= 0) {
    // >= 4 workgroups per CU (what the register use of a two- or four-head workgroup
    // lets a CU hold), never more splits than a row has blocks; a split count
    // above 1 costs a merge launch
    const int64_t target = fill_target(4);
    s = (target + ps->units - 1) / ps->units;
    if (s > row_cap) s = row_cap;
    if (s < 1) s = 1;
  }
  if (s > 65536) return fail(S2_EUNSUPPORTED, "splits must be <= 65536 (got %lld)", (long long)s);
  ps->splits = (int32_t)s;
  return S2_OK;
}

size_t paged_ws_bytes(int64_t bh, const PagedShape &ps, int32_t D) {
  return ps.splits == 1 ? 0 : decode_ws_bytes(bh, ps.splits, D);
}

}  // namespace

extern "C" {

int32_t s2_abi_version(void) { return S2_ABI_VERSION; }

const char *s2_last_error(void) { return g_err; }

s2_status s2_layout_nnz(const s2_pattern *pattern, int32_t num_q_blocks, int64_t *nnz) {
  g_err[0] = 0;
  if (!nnz) return fail(S2_EINVAL, "nnz is NULL");
  s2::PatternArgs pa;
  s2_status st = check_pattern(pattern, num_q_blocks, &pa);
  if (st != S2_OK) return st;
  *nnz = total_nnz(pa);
  return S2_OK;
}

s2_status s2_build_layout(const s2_pattern *pattern, int32_t num_q_blocks, int32_t *row_ptr,
                          int32_t *col_idx, int64_t col_capacity, void *stream) {
  g_err[0] = 0;
  s2::PatternArgs pa;
  s2_status st = check_pattern(pattern, num_q_blocks, &pa);
  if (st != S2_OK) return st;
  if (!row_ptr || !col_idx) return fail(S2_EINVAL, "row_ptr/col_idx is NULL");
  if ((int64_t)pa.H * pa.nqb >= (int64_t(1) << 31)) return fail(S2_EUNSUPPORTED, "too many rows");
  const int64_t nnz = total_nnz(pa);
  if (nnz >= (int64_t(1) << 31))
    return fail(S2_EUNSUPPORTED, "layout has %lld entries; int32 CSR holds < 2^31", (long long)nnz);
  if (col_capacity < nnz)
    return fail(S2_ECAPACITY, "col_idx holds %lld entries, layout needs %lld", (long long)col_capacity,
                (long long)nnz);
  return hip_status(s2::launch_build_layout(pa, row_ptr, col_idx, static_cast<hipStream_t>(stream)),
                    "s2_build_layout launch");
}

s2_status s2_attn_fwd_workspace(size_t *bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(S2_EINVAL, "bytes is NULL");
  *bytes = s2::kFwdWorkspaceBytes;
  return S2_OK;
}

s2_status s2_attn_fwd(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t N, int32_t D,
                      const void *q, const int64_t qs[4], const void *k, const int64_t ks[4],
                      const void *v, const int64_t vs[4], void *o, const int64_t os[4], float *lse,
                      void *workspace, size_t workspace_bytes, float sm_scale, void *stream) {
  g_err[0] = 0;
  s2_status st0 = check_fwd_workspace(workspace, workspace_bytes);
  if (st0 != S2_OK) return st0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (B < 1) return fail(S2_EINVAL, "B must be >= 1 (got %d)", B);
  if (N < 1 || N % S2_BLOCK != 0)
    return fail(S2_EINVAL, "N must be a positive multiple of %d (got %d)", S2_BLOCK, N);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (layout->num_q_blocks != N / S2_BLOCK)
    return fail(S2_EINVAL, "layout has %d query blocks, N / 64 = %d", layout->num_q_blocks,
                N / S2_BLOCK);
  if ((int64_t)B * layout->num_heads * N >= (int64_t(1) << 40))
    return fail(S2_EUNSUPPORTED, "problem too large");
  const int64_t mult = dtype == S2_BF16 ? 8 : 4;
  if ((st = check_tensor("q", q, qs, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("k", k, ks, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("v", v, vs, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("o", o, os, 4, mult)) != S2_OK) return st;
  s2::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  for (int i = 0; i < 4; ++i) {
    p.qs[i] = qs[i];
    p.ks[i] = ks[i];
    p.vs[i] = vs[i];
    p.os[i] = os[i];
  }
  p.row_ptr = layout->row_ptr;
  p.col_idx = layout->col_idx;
  p.B = B;
  p.H = layout->num_heads;
  p.N = N;
  p.nqb = layout->num_q_blocks;
  p.scale_log2 = scale_log2(sm_scale, D);
  p.queue = static_cast<unsigned long long *>(workspace);
  p.tag = 0;
  p.cu_seqlens = nullptr;
  p.T_total = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == S2_BF16 ? s2::launch_fwd_bf16(p, D, s) : s2::launch_fwd_f32(p, D, s);
  return hip_status(e, "s2_attn_fwd launch");
}

s2_status s2_attn_fwd_varlen(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t T_total, int32_t D,
                             const int32_t *cu_seqlens, const void *q, const int64_t qs[3], const void *k,
                             const int64_t ks[3], const void *v, const int64_t vs[3], void *o,
                             const int64_t os[3], float *lse, void *workspace, size_t workspace_bytes,
                             float sm_scale, void *stream) {
  g_err[0] = 0;
  s2_status st0 = check_fwd_workspace(workspace, workspace_bytes);
  if (st0 != S2_OK) return st0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (dtype != S2_BF16) return fail(S2_EUNSUPPORTED, "variable-length batches support bf16 only");
  if (B < 1) return fail(S2_EINVAL, "B must be >= 1 (got %d)", B);
  if (T_total < 1) return fail(S2_EINVAL, "T_total must be >= 1 (got %d)", T_total);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (!cu_seqlens) return fail(S2_EINVAL, "cu_seqlens is NULL");
  if ((int64_t)B * layout->num_heads * ((layout->num_q_blocks + 1) / 2) >= (int64_t(1) << 31))
    return fail(S2_EUNSUPPORTED, "problem too large");
  if ((st = check_tensor("q", q, qs, 3, 8)) != S2_OK) return st;
  if ((st = check_tensor("k", k, ks, 3, 8)) != S2_OK) return st;
  if ((st = check_tensor("v", v, vs, 3, 8)) != S2_OK) return st;
  if ((st = check_tensor("o", o, os, 3, 8)) != S2_OK) return st;
  s2::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  // [T, H, D] as [B, H, N, D] with batch stride 0: the kernel adds the
  // sequence's token offset
  const int64_t *src[4] = {qs, ks, vs, os};
  int64_t *dst[4] = {p.qs, p.ks, p.vs, p.os};
  for (int t = 0; t < 4; ++t) {
    dst[t][0] = 0;
    dst[t][1] = src[t][1];
    dst[t][2] = src[t][0];
    dst[t][3] = 1;
  }
  p.row_ptr = layout->row_ptr;
  p.col_idx = layout->col_idx;
  p.B = B;
  p.H = layout->num_heads;
  p.N = layout->num_q_blocks * S2_BLOCK;
  p.nqb = layout->num_q_blocks;
  p.scale_log2 = scale_log2(sm_scale, D);
  p.queue = static_cast<unsigned long long *>(workspace);
  p.tag = 0;
  p.cu_seqlens = cu_seqlens;
  p.T_total = T_total;
  return hip_status(s2::launch_fwd_bf16(p, D, static_cast<hipStream_t>(stream)), "s2_attn_fwd_varlen launch");
}

s2_status s2_build_layout_t(const s2_pattern *pattern, int32_t num_q_blocks, int32_t *col_ptr,
                            int32_t *row_idx, int64_t capacity, void *stream) {
  g_err[0] = 0;
  s2::PatternArgs pa;
  s2_status st = check_pattern(pattern, num_q_blocks, &pa);
  if (st != S2_OK) return st;
  if (!col_ptr || !row_idx) return fail(S2_EINVAL, "col_ptr/row_idx is NULL");
  if ((int64_t)pa.H * pa.nqb >= (int64_t(1) << 31)) return fail(S2_EUNSUPPORTED, "too many columns");
  const int64_t nnz = total_nnz(pa);
  if (nnz >= (int64_t(1) << 31))
    return fail(S2_EUNSUPPORTED, "layout has %lld entries; int32 CSR holds < 2^31", (long long)nnz);
  if (capacity < nnz)
    return fail(S2_ECAPACITY, "row_idx holds %lld entries, layout needs %lld", (long long)capacity,
                (long long)nnz);
  return hip_status(s2::launch_build_layout_t(pa, col_ptr, row_idx, static_cast<hipStream_t>(stream)),
                    "s2_build_layout_t launch");
}

s2_status s2_attn_bwd_workspace(int32_t B, int32_t H, int32_t N, size_t *bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(S2_EINVAL, "bytes is NULL");
  if (B < 1 || H < 1 || N < 1) return fail(S2_EINVAL, "B, H and N must be >= 1");
  *bytes = s2::bwd_workspace_bytes(B, H, N);
  return S2_OK;
}

s2_status s2_attn_bwd(const s2_layout *layout, const s2_layout *layout_t, s2_dtype dtype, int32_t B,
                      int32_t N, int32_t D, const void *q, const int64_t qs[4], const void *k,
                      const int64_t ks[4], const void *v, const int64_t vs[4], const void *o,
                      const int64_t os[4], const void *dout, const int64_t dos[4], const float *lse,
                      void *dq, const int64_t dqs[4], void *dk, const int64_t dks[4], void *dv,
                      const int64_t dvs[4], void *workspace, size_t workspace_bytes, float sm_scale,
                      void *stream) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (!layout_t) return fail(S2_EINVAL, "layout_t is NULL");
  if ((st = check_layout(layout_t)) != S2_OK) return st;
  if (layout_t->num_heads != layout->num_heads || layout_t->num_q_blocks != layout->num_q_blocks ||
      layout_t->nnz != layout->nnz)
    return fail(S2_EINVAL, "layout_t is not the column view of layout (heads, blocks or nnz differ)");
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (dtype != S2_BF16) return fail(S2_EUNSUPPORTED, "the backward pass supports bf16 only");
  if (B < 1) return fail(S2_EINVAL, "B must be >= 1 (got %d)", B);
  if (N < 1 || N % S2_BLOCK != 0)
    return fail(S2_EINVAL, "N must be a positive multiple of %d (got %d)", S2_BLOCK, N);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (layout->num_q_blocks != N / S2_BLOCK)
    return fail(S2_EINVAL, "layout has %d query blocks, N / 64 = %d", layout->num_q_blocks,
                N / S2_BLOCK);
  if ((int64_t)B * layout->num_heads * N >= (int64_t(1) << 40))
    return fail(S2_EUNSUPPORTED, "problem too large");
  if (!lse) return fail(S2_EINVAL, "lse is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 15) != 0) return fail(S2_EINVAL, "lse must be 16-byte aligned");
  if ((st = check_tensor("q", q, qs, 4, 8)) != S2_OK) return st;
  if ((st = check_tensor("k", k, ks, 4, 8)) != S2_OK) return st;
  if ((st = check_tensor("v", v, vs, 4, 8)) != S2_OK) return st;
  if ((st = check_tensor("o", o, os, 4, 8)) != S2_OK) return st;
  if ((st = check_tensor("dout", dout, dos, 4, 8)) != S2_OK) return st;
  if ((st = check_tensor("dq", dq, dqs, 4, 8)) != S2_OK) return st;
  if ((st = check_tensor("dk", dk, dks, 4, 8)) != S2_OK) return st;
  if ((st = check_tensor("dv", dv, dvs, 4, 8)) != S2_OK) return st;
  const size_t need = s2::bwd_workspace_bytes(B, layout->num_heads, N);
  if (!workspace) return fail(S2_EINVAL, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(S2_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(S2_ECAPACITY, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  s2::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.lse = lse;
  p.delta = static_cast<float *>(workspace);
  p.nlse2 = p.delta + (int64_t)B * layout->num_heads * N;
  p.plan_kv = reinterpret_cast<int32_t *>(p.nlse2 + (int64_t)B * layout->num_heads * N);
  p.plan_q = p.plan_kv + (int64_t)B * layout->num_heads * layout->num_q_blocks;
  for (int i = 0; i < 4; ++i) {
    p.qs[i] = qs[i];
    p.ks[i] = ks[i];
    p.vs[i] = vs[i];
    p.os[i] = os[i];
    p.dos[i] = dos[i];
    p.dqs[i] = dqs[i];
    p.dks[i] = dks[i];
    p.dvs[i] = dvs[i];
  }
  p.row_ptr = layout->row_ptr;
  p.col_idx = layout->col_idx;
  p.col_ptr = layout_t->row_ptr;
  p.row_idx = layout_t->col_idx;
  p.B = B;
  p.H = layout->num_heads;
  p.N = N;
  p.nqb = layout->num_q_blocks;
  p.scale_log2 = scale_log2(sm_scale, D);
  p.scale = sm_scale > 0.f ? sm_scale : 1.f / sqrtf((float)D);
  return hip_status(s2::launch_bwd_bf16(p, D, static_cast<hipStream_t>(stream)), "s2_attn_bwd launch");
}

s2_status s2_attn_decode_workspace(const s2_layout *layout, int32_t B, int32_t D, int32_t splits,
                                   size_t *bytes) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (!bytes) return fail(S2_EINVAL, "bytes is NULL");
  if (B < 1) return fail(S2_EINVAL, "B must be >= 1 (got %d)", B);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  const int32_t sp = splits > 0 ? splits : auto_splits(layout, B);
  *bytes = decode_ws_bytes((int64_t)B * layout->num_heads, sp, D);
  return S2_OK;
}

s2_status s2_attn_decode(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t D,
                         const void *q, const int64_t qs[3], const void *k_cache,
                         const int64_t ks[4], const void *v_cache, const int64_t vs[4],
                         const int32_t *seq_lens, int32_t cache_len, void *o, const int64_t os[3],
                         float *lse, int32_t splits, void *workspace, size_t workspace_bytes,
                         float sm_scale, void *stream) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (B < 1) return fail(S2_EINVAL, "B must be >= 1 (got %d)", B);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (!seq_lens) return fail(S2_EINVAL, "seq_lens is NULL");
  if (cache_len < 1) return fail(S2_EINVAL, "cache_len must be >= 1 (got %d)", cache_len);
  if ((int64_t)layout->num_q_blocks * S2_BLOCK < cache_len)
    return fail(S2_EINVAL, "layout covers %lld tokens, cache_len is %d",
                (long long)layout->num_q_blocks * S2_BLOCK, cache_len);
  const int64_t mult = dtype == S2_BF16 ? 8 : 4;
  if ((st = check_tensor("q", q, qs, 3, mult)) != S2_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, ks, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, vs, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("o", o, os, 3, dtype == S2_BF16 ? 1 : 1)) != S2_OK) return st;
  const int32_t sp = splits > 0 ? splits : auto_splits(layout, B);
  if (sp > 65536) return fail(S2_EUNSUPPORTED, "splits must be <= 65536 (got %d)", sp);
  const int64_t bh = (int64_t)B * layout->num_heads;
  const size_t need = decode_ws_bytes(bh, sp, D);
  if (!workspace) return fail(S2_EINVAL, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(S2_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(S2_ECAPACITY, "workspace holds %zu bytes, %zu needed for %d splits", workspace_bytes,
                need, sp);
  s2::DecodeParams p;
  p.q = q;
  p.kc = k_cache;
  p.vc = v_cache;
  p.o = o;
  p.lse = lse;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = qs[i];
    p.os[i] = os[i];
  }
  for (int i = 0; i < 4; ++i) {
    p.ks[i] = ks[i];
    p.vs[i] = vs[i];
  }
  p.row_ptr = layout->row_ptr;
  p.col_idx = layout->col_idx;
  p.seq_lens = seq_lens;
  p.B = B;
  p.H = layout->num_heads;
  p.nqb = layout->num_q_blocks;
  p.cache_len = cache_len;
  p.splits = sp;
  p.per_seq = 0;
  p.scale_log2 = scale_log2(sm_scale, D);
  p.part_o = static_cast<float *>(workspace);
  p.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                         align256((size_t)bh * sp * D * sizeof(float)));
  return hip_status(s2::launch_decode(p, dtype, D, static_cast<hipStream_t>(stream)),
                    "s2_attn_decode launch");
}

s2_status s2_attn_decode_noalloc(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t D,
                                 const void *q, const int64_t qs[3], const void *k_cache,
                                 const int64_t ks[4], const void *v_cache, const int64_t vs[4],
                                 const int32_t *seq_lens, int32_t cache_len, void *o, const int64_t os[3],
                                 float *lse, int32_t splits, float sm_scale, void *stream) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (B < 1) return fail(S2_EINVAL, "B must be >= 1 (got %d)", B);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  const int32_t sp = splits > 0 ? splits : auto_splits(layout, B);
  if (sp > 65536) return fail(S2_EUNSUPPORTED, "splits must be <= 65536 (got %d)", sp);
  const size_t need = decode_ws_bytes((int64_t)B * layout->num_heads, sp, D);
  if (need > (size_t)S2_NOALLOC_SCRATCH_BYTES)
    return fail(S2_ECAPACITY,
                "s2_attn_decode_noalloc: %d splits over %lld (sequence, head) rows need %zu bytes of "
                "scratch, the static scratch holds %zu; use fewer splits, a smaller batch, or "
                "s2_attn_decode with a workspace",
                sp, (long long)B * layout->num_heads, need, (size_t)S2_NOALLOC_SCRATCH_BYTES);
  void *scratch = nullptr;
  hipError_t e = s2::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "s2_attn_decode_noalloc: scratch address");
  return s2_attn_decode(layout, dtype, B, D, q, qs, k_cache, ks, v_cache, vs, seq_lens, cache_len, o, os, lse,
                        sp, scratch, (size_t)S2_NOALLOC_SCRATCH_BYTES, sm_scale, stream);
}

/* ---- query-aware block lists ---- */

s2_status s2_block_minmax(s2_dtype dtype, int32_t B, int32_t H, int32_t D, const void *k_cache,
                          const int64_t ks[4], const int32_t *seq_lens, int32_t cache_len, void *kmin,
                          void *kmax, int32_t num_blocks, void *stream) {
  g_err[0] = 0;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (B < 1 || H < 1) return fail(S2_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (!seq_lens) return fail(S2_EINVAL, "seq_lens is NULL");
  if (cache_len < 1) return fail(S2_EINVAL, "cache_len must be >= 1 (got %d)", cache_len);
  if ((int64_t)num_blocks * S2_BLOCK < cache_len)
    return fail(S2_EINVAL, "num_blocks (%d) must cover cache_len (%d)", num_blocks, cache_len);
  s2_status st;
  if ((st = check_tensor("k_cache", k_cache, ks, 4, dtype == S2_BF16 ? 8 : 4)) != S2_OK) return st;
  if (!kmin || !kmax) return fail(S2_EINVAL, "kmin / kmax is NULL");
  if (((reinterpret_cast<uintptr_t>(kmin) | reinterpret_cast<uintptr_t>(kmax)) & 15) != 0)
    return fail(S2_EINVAL, "kmin and kmax must be 16-byte aligned");
  s2::MinmaxParams p;
  p.k = k_cache;
  for (int i = 0; i < 4; ++i) p.ks[i] = ks[i];
  p.seq_lens = seq_lens;
  p.kmin = kmin;
  p.kmax = kmax;
  p.B = B;
  p.H = H;
  p.nblk = num_blocks;
  p.cache_len = cache_len;
  p.block_table = nullptr;
  p.bt_stride = 0;
  p.num_pages = 0;
  p.page_shift = 0;
  return hip_status(s2::launch_block_minmax(p, dtype, D, static_cast<hipStream_t>(stream)),
                    "s2_block_minmax launch");
}

s2_status s2_block_minmax_paged(s2_dtype dtype, int32_t B, int32_t num_kv_heads, int32_t D,
                                const void *k_pages, const int64_t kps[4], int32_t num_pages, int32_t page_size,
                                const int32_t *block_table, int64_t bt_stride, int32_t max_pages_per_seq,
                                const int32_t *seq_lens, void *kmin, void *kmax, int32_t num_blocks,
                                void *stream) {
  g_err[0] = 0;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (B < 1 || num_kv_heads < 1)
    return fail(S2_EINVAL, "B and num_kv_heads must be >= 1 (got %d, %d)", B, num_kv_heads);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0)
    return fail(S2_EINVAL, "page_size must be a power of two in [1, 65536] (got %d)", page_size);
  if (num_pages < 1) return fail(S2_EINVAL, "num_pages must be >= 1 (got %d)", num_pages);
  if (!block_table) return fail(S2_EINVAL, "block_table is NULL");
  if (max_pages_per_seq < 1) return fail(S2_EINVAL, "max_pages_per_seq must be >= 1");
  if (bt_stride < max_pages_per_seq)
    return fail(S2_EINVAL, "bt_stride (%lld) must be >= max_pages_per_seq (%d)", (long long)bt_stride,
                max_pages_per_seq);
  const int64_t max_len = (int64_t)max_pages_per_seq * page_size;
  if (max_len >= (int64_t(1) << 31)) return fail(S2_EUNSUPPORTED, "sequences must hold < 2^31 tokens");
  if ((int64_t)num_blocks * S2_BLOCK < max_len)
    return fail(S2_EINVAL, "num_blocks (%d) must cover the block tables' %lld tokens", num_blocks,
                (long long)max_len);
  if (!seq_lens) return fail(S2_EINVAL, "seq_lens is NULL");
  s2_status st;
  if ((st = check_tensor("k_pages", k_pages, kps, 4, dtype == S2_BF16 ? 8 : 4)) != S2_OK) return st;
  if (!kmin || !kmax) return fail(S2_EINVAL, "kmin / kmax is NULL");
  if (((reinterpret_cast<uintptr_t>(kmin) | reinterpret_cast<uintptr_t>(kmax)) & 15) != 0)
    return fail(S2_EINVAL, "kmin and kmax must be 16-byte aligned");
  s2::MinmaxParams p;
  p.k = k_pages;
  for (int i = 0; i < 4; ++i) p.ks[i] = kps[i];
  p.seq_lens = seq_lens;
  p.kmin = kmin;
  p.kmax = kmax;
  p.B = B;
  p.H = num_kv_heads;
  p.nblk = num_blocks;
  p.cache_len = (int32_t)max_len;
  p.block_table = block_table;
  p.bt_stride = bt_stride;
  p.num_pages = num_pages;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  p.page_shift = shift;
  return hip_status(s2::launch_block_minmax(p, dtype, D, static_cast<hipStream_t>(stream)),
                    "s2_block_minmax_paged launch");
}

s2_status s2_select_blocks(s2_dtype dtype, int32_t B, int32_t H, int32_t num_kv_heads, int32_t D, const void *q,
                           const int64_t qs[3], const void *kmin, const void *kmax, int32_t num_blocks,
                           const int32_t *seq_lens, int32_t cache_len, int32_t budget, int32_t *row_ptr,
                           int32_t *col_idx, int64_t col_capacity, void *stream) {
  g_err[0] = 0;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (B < 1 || H < 1) return fail(S2_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (!seq_lens) return fail(S2_EINVAL, "seq_lens is NULL");
  if (cache_len < 1) return fail(S2_EINVAL, "cache_len must be >= 1 (got %d)", cache_len);
  if (budget < 1) return fail(S2_EINVAL, "budget must be >= 1 (got %d)", budget);
  if (num_kv_heads < 1 || H % num_kv_heads != 0)
    return fail(S2_EINVAL, "num_kv_heads (%d) must divide the %d query heads", num_kv_heads, H);
  if ((int64_t)num_blocks * S2_BLOCK < cache_len)
    return fail(S2_EINVAL, "num_blocks (%d) must cover cache_len (%d)", num_blocks, cache_len);
  if (num_blocks > s2::kMaxSelectBlocks)
    return fail(S2_EUNSUPPORTED, "num_blocks must be <= %d (got %d)", s2::kMaxSelectBlocks, num_blocks);
  s2_status st;
  if ((st = check_tensor("q", q, qs, 3, dtype == S2_BF16 ? 8 : 4)) != S2_OK) return st;
  if (!kmin || !kmax) return fail(S2_EINVAL, "kmin / kmax is NULL");
  if (((reinterpret_cast<uintptr_t>(kmin) | reinterpret_cast<uintptr_t>(kmax)) & 15) != 0)
    return fail(S2_EINVAL, "kmin and kmax must be 16-byte aligned");
  if (!row_ptr || !col_idx) return fail(S2_EINVAL, "row_ptr / col_idx is NULL");
  const int64_t longest = std::min<int64_t>(budget, (cache_len + S2_BLOCK - 1) / S2_BLOCK);
  const int64_t most = (int64_t)B * H * longest;
  if (most > 0x7fffffff) return fail(S2_EUNSUPPORTED, "B * H * row length (%lld) must fit int32", (long long)most);
  if (col_capacity < most)
    return fail(S2_ECAPACITY, "col_idx holds %lld entries, up to %lld needed", (long long)col_capacity,
                (long long)most);
  s2::SelectParams p;
  p.q = q;
  for (int i = 0; i < 3; ++i) p.qs[i] = qs[i];
  p.kmin = kmin;
  p.kmax = kmax;
  p.seq_lens = seq_lens;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.B = B;
  p.H = H;
  p.nblk = num_blocks;
  p.cache_len = cache_len;
  p.budget = budget;
  p.Hkv = num_kv_heads;
  p.group = H / num_kv_heads;
  return hip_status(s2::launch_select_blocks(p, dtype, D, static_cast<hipStream_t>(stream)),
                    "s2_select_blocks launch");
}

static int32_t rows_auto_splits(int64_t bh, int32_t max_row_blocks) {
  const int64_t target = fill_target(8);  // >= 8 workgroups of split work per CU, as for layout rows
  int64_t s = (target + bh - 1) / bh;
  if (s > max_row_blocks) s = max_row_blocks;
  return (int32_t)(s < 1 ? 1 : s);
}

s2_status s2_attn_decode_rows_workspace(int32_t B, int32_t H, int32_t D, int32_t max_row_blocks,
                                        int32_t splits, size_t *bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(S2_EINVAL, "bytes is NULL");
  if (B < 1 || H < 1) return fail(S2_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (max_row_blocks < 1) return fail(S2_EINVAL, "max_row_blocks must be >= 1 (got %d)", max_row_blocks);
  const int64_t bh = (int64_t)B * H;
  *bytes = decode_ws_bytes(bh, splits > 0 ? splits : rows_auto_splits(bh, max_row_blocks), D);
  return S2_OK;
}

s2_status s2_attn_decode_rows(s2_dtype dtype, int32_t B, int32_t H, int32_t D, const int32_t *row_ptr,
                              const int32_t *col_idx, int32_t max_row_blocks, const void *q,
                              const int64_t qs[3], const void *k_cache, const int64_t ks[4],
                              const void *v_cache, const int64_t vs[4], const int32_t *seq_lens,
                              int32_t cache_len, void *o, const int64_t os[3], float *lse, int32_t splits,
                              void *workspace, size_t workspace_bytes, float sm_scale, void *stream) {
  g_err[0] = 0;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (B < 1 || H < 1) return fail(S2_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (!row_ptr || !col_idx) return fail(S2_EINVAL, "row_ptr / col_idx is NULL");
  if (max_row_blocks < 1) return fail(S2_EINVAL, "max_row_blocks must be >= 1 (got %d)", max_row_blocks);
  if (!seq_lens) return fail(S2_EINVAL, "seq_lens is NULL");
  if (cache_len < 1) return fail(S2_EINVAL, "cache_len must be >= 1 (got %d)", cache_len);
  const int64_t mult = dtype == S2_BF16 ? 8 : 4;
  s2_status st;
  if ((st = check_tensor("q", q, qs, 3, mult)) != S2_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, ks, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, vs, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("o", o, os, 3, 1)) != S2_OK) return st;
  const int64_t bh = (int64_t)B * H;
  const int32_t sp = splits > 0 ? splits : rows_auto_splits(bh, max_row_blocks);
  if (sp > 65536) return fail(S2_EUNSUPPORTED, "splits must be <= 65536 (got %d)", sp);
  const size_t need = decode_ws_bytes(bh, sp, D);
  if (!workspace) return fail(S2_EINVAL, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(S2_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(S2_ECAPACITY, "workspace holds %zu bytes, %zu needed for %d splits", workspace_bytes,
                need, sp);
  s2::DecodeParams p;
  p.q = q;
  p.kc = k_cache;
  p.vc = v_cache;
  p.o = o;
  p.lse = lse;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = qs[i];
    p.os[i] = os[i];
  }
  for (int i = 0; i < 4; ++i) {
    p.ks[i] = ks[i];
    p.vs[i] = vs[i];
  }
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.seq_lens = seq_lens;
  p.B = B;
  p.H = H;
  p.nqb = 0;
  p.cache_len = cache_len;
  p.splits = sp;
  p.per_seq = 1;
  p.scale_log2 = scale_log2(sm_scale, D);
  p.part_o = static_cast<float *>(workspace);
  p.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                         align256((size_t)bh * sp * D * sizeof(float)));
  return hip_status(s2::launch_decode(p, dtype, D, static_cast<hipStream_t>(stream)),
                    "s2_attn_decode_rows launch");
}

}  // extern "C"

extern "C" {

s2_status s2_attn_decode_paged_workspace(const s2_layout *layout, int32_t B, int32_t num_kv_heads,
                                         int32_t D, int32_t splits, size_t *bytes) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (!bytes) return fail(S2_EINVAL, "bytes is NULL");
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  PagedShape ps;
  if ((st = paged_shape(layout->num_heads, layout->num_q_blocks, B, num_kv_heads, splits, false, &ps)) != S2_OK)
    return st;
  *bytes = paged_ws_bytes((int64_t)B * layout->num_heads, ps, D);
  return S2_OK;
}

}  // extern "C"

namespace {
// the paged decode over the layout's rows (row h * nqb + p / 64, per_seq = 0) or
// over per-(sequence, head) rows (row b * H + h, per_seq = 1)
s2_status paged_run(s2_dtype dtype, int32_t B, int32_t H, int32_t num_kv_heads, int32_t D,
                    const int32_t *row_ptr, const int32_t *col_idx, int32_t nqb, int32_t per_seq,
                    int32_t row_cap, int64_t cover, const void *q, const int64_t qs[3], const void *k_pages,
                    const int64_t kps[4], const void *v_pages, const int64_t vps[4], int32_t num_pages,
                    int32_t page_size, const int32_t *block_table, int64_t bt_stride,
                    int32_t max_pages_per_seq, const int32_t *seq_lens, void *o, const int64_t os[3],
                    float *lse, int32_t splits, void *workspace, size_t workspace_bytes, float sm_scale,
                    void *stream, const char *what) {
  s2_status st;
  if (dtype != S2_BF16 && dtype != S2_F32) return fail(S2_EINVAL, "unknown dtype %d", (int)dtype);
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  PagedShape ps;
  if ((st = paged_shape(H, row_cap, B, num_kv_heads, splits, per_seq != 0, &ps)) != S2_OK) return st;
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0)
    return fail(S2_EINVAL, "page_size must be a power of two in [1, 65536] (got %d)", page_size);
  if (num_pages < 1) return fail(S2_EINVAL, "num_pages must be >= 1 (got %d)", num_pages);
  if (!block_table) return fail(S2_EINVAL, "block_table is NULL");
  if (max_pages_per_seq < 1) return fail(S2_EINVAL, "max_pages_per_seq must be >= 1");
  if (bt_stride < max_pages_per_seq)
    return fail(S2_EINVAL, "bt_stride (%lld) must be >= max_pages_per_seq (%d)", (long long)bt_stride,
                max_pages_per_seq);
  const int64_t max_len = (int64_t)max_pages_per_seq * page_size;
  if (max_len > cover)
    return fail(S2_EINVAL, "block tables reach %lld tokens, the layout covers %lld", (long long)max_len,
                (long long)cover);
  if (max_len >= (int64_t(1) << 31)) return fail(S2_EUNSUPPORTED, "sequences must hold < 2^31 tokens");
  if (!seq_lens) return fail(S2_EINVAL, "seq_lens is NULL");
  const int64_t mult = dtype == S2_BF16 ? 8 : 4;
  if ((st = check_tensor("q", q, qs, 3, mult)) != S2_OK) return st;
  if ((st = check_tensor("k_pages", k_pages, kps, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("v_pages", v_pages, vps, 4, mult)) != S2_OK) return st;
  if ((st = check_tensor("o", o, os, 3, 1)) != S2_OK) return st;
  const int64_t bh = (int64_t)B * H;
  const size_t need = paged_ws_bytes(bh, ps, D);
  if (need > 0) {
    if (!workspace) return fail(S2_EINVAL, "workspace is NULL (%d splits need one)", ps.splits);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
      return fail(S2_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(S2_ECAPACITY, "workspace holds %zu bytes, %zu needed for %d splits", workspace_bytes,
                  need, ps.splits);
  }
  if (ps.units * ps.splits > 0x7fffffff) return fail(S2_EUNSUPPORTED, "problem too large");
  s2::PagedParams p;
  p.q = q;
  p.kp = k_pages;
  p.vp = v_pages;
  p.o = o;
  p.lse = lse;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = qs[i];
    p.os[i] = os[i];
  }
  for (int i = 0; i < 4; ++i) {
    p.kps[i] = kps[i];
    p.vps[i] = vps[i];
  }
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.bt_stride = bt_stride;
  p.B = B;
  p.H = H;
  p.Hkv = num_kv_heads;
  p.group = ps.group;
  p.nchunk = ps.nchunk;
  p.nqb = nqb;
  p.per_seq = per_seq;
  p.splits = ps.splits;
  p.num_pages = num_pages;
  p.max_pages = max_pages_per_seq;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  p.page_shift = shift;
  p.scale_log2 = scale_log2(sm_scale, D);
  p.part_o = nullptr;
  p.part_lse = nullptr;
  if (need > 0) {
    p.part_o = static_cast<float *>(workspace);
    p.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                           align256((size_t)bh * ps.splits * D * sizeof(float)));
  }
  return hip_status(s2::launch_decode_paged(p, dtype, D, static_cast<hipStream_t>(stream)), what);
}
}  // namespace

extern "C" {

s2_status s2_attn_decode_paged(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t num_kv_heads,
                               int32_t D, const void *q, const int64_t qs[3], const void *k_pages,
                               const int64_t kps[4], const void *v_pages, const int64_t vps[4],
                               int32_t num_pages, int32_t page_size, const int32_t *block_table,
                               int64_t bt_stride, int32_t max_pages_per_seq, const int32_t *seq_lens,
                               void *o, const int64_t os[3], float *lse, int32_t splits, void *workspace,
                               size_t workspace_bytes, float sm_scale, void *stream) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  return paged_run(dtype, B, layout->num_heads, num_kv_heads, D, layout->row_ptr, layout->col_idx,
                   layout->num_q_blocks, 0, layout->num_q_blocks, (int64_t)layout->num_q_blocks * S2_BLOCK,
                   q, qs, k_pages, kps, v_pages, vps, num_pages, page_size, block_table, bt_stride,
                   max_pages_per_seq, seq_lens, o, os, lse, splits, workspace, workspace_bytes, sm_scale,
                   stream, "s2_attn_decode_paged launch");
}

s2_status s2_attn_decode_paged_rows_workspace(int32_t B, int32_t H, int32_t num_kv_heads, int32_t D,
                                              int32_t max_row_blocks, int32_t splits, size_t *bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(S2_EINVAL, "bytes is NULL");
  if (D != 64 && D != 128) return fail(S2_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (max_row_blocks < 1) return fail(S2_EINVAL, "max_row_blocks must be >= 1 (got %d)", max_row_blocks);
  PagedShape ps;
  s2_status st;
  if ((st = paged_shape(H, max_row_blocks, B, num_kv_heads, splits, true, &ps)) != S2_OK) return st;
  *bytes = paged_ws_bytes((int64_t)B * H, ps, D);
  return S2_OK;
}

s2_status s2_attn_decode_paged_rows(s2_dtype dtype, int32_t B, int32_t H, int32_t num_kv_heads, int32_t D,
                                    const int32_t *row_ptr, const int32_t *col_idx, int32_t max_row_blocks,
                                    const void *q, const int64_t qs[3], const void *k_pages,
                                    const int64_t kps[4], const void *v_pages, const int64_t vps[4],
                                    int32_t num_pages, int32_t page_size, const int32_t *block_table,
                                    int64_t bt_stride, int32_t max_pages_per_seq, const int32_t *seq_lens,
                                    void *o, const int64_t os[3], float *lse, int32_t splits,
                                    void *workspace, size_t workspace_bytes, float sm_scale, void *stream) {
  g_err[0] = 0;
  if (!row_ptr || !col_idx) return fail(S2_EINVAL, "row_ptr / col_idx is NULL");
  if (max_row_blocks < 1) return fail(S2_EINVAL, "max_row_blocks must be >= 1 (got %d)", max_row_blocks);
  return paged_run(dtype, B, H, num_kv_heads, D, row_ptr, col_idx, 0, 1, max_row_blocks, INT64_MAX, q, qs,
                   k_pages, kps, v_pages, vps, num_pages, page_size, block_table, bt_stride,
                   max_pages_per_seq, seq_lens, o, os, lse, splits, workspace, workspace_bytes, sm_scale,
                   stream, "s2_attn_decode_paged_rows launch");
}

}  // extern "C"

extern "C" {

s2_status s2_validate_layout(const s2_layout *layout, void *scratch, void *stream) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (!scratch || (reinterpret_cast<uintptr_t>(scratch) & 7) != 0)
    return fail(S2_EINVAL, "scratch must be 8 bytes of 8-byte aligned device memory");
  auto *first = static_cast<unsigned long long *>(scratch);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = s2::launch_validate_layout(layout->row_ptr, layout->col_idx, layout->num_heads,
                                            layout->num_q_blocks, layout->nnz, first, s);
  unsigned long long code = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&code, first, sizeof(code), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "s2_validate_layout");
  if (code == ~0ull) return S2_OK;
  const long long row = (long long)(code >> 8);
  const int h = (int)(row / layout->num_q_blocks), i = (int)(row % layout->num_q_blocks);
  switch ((int)(code & 255)) {
    case s2::kLayoutBadStart: return fail(S2_EINVAL, "layout row_ptr[0] must be 0");
    case s2::kLayoutBadEnd:
      return fail(S2_EINVAL, "layout row_ptr[%lld] must equal nnz = %lld", row + 1, (long long)layout->nnz);
    case s2::kLayoutBadPtr:
      return fail(S2_EINVAL, "layout row %lld (head %d, query block %d): row_ptr decreases or leaves [0, nnz]", row,
                  h, i);
    case s2::kLayoutBadBlock:
      return fail(S2_EINVAL, "layout row %lld (head %d, query block %d): a key block outside [0, %d]", row, h, i, i);
    default:
      return fail(S2_EINVAL, "layout row %lld (head %d, query block %d): key blocks not strictly ascending", row,
                  h, i);
  }
}

s2_status s2_transpose_layout_workspace(const s2_layout *layout, size_t *bytes) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (!bytes) return fail(S2_EINVAL, "bytes is NULL");
  *bytes = align256((size_t)s2::transpose_bitmap_words(layout->num_heads, layout->num_q_blocks) * 4);
  return S2_OK;
}

s2_status s2_transpose_layout(const s2_layout *layout, int32_t *col_ptr, int32_t *row_idx, int64_t capacity,
                              void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  s2_status st = check_layout(layout);
  if (st != S2_OK) return st;
  if (!col_ptr || !row_idx) return fail(S2_EINVAL, "col_ptr / row_idx is NULL");
  if (capacity < layout->nnz)
    return fail(S2_ECAPACITY, "row_idx holds %lld entries, layout needs %lld", (long long)capacity,
                (long long)layout->nnz);
  const size_t need = align256((size_t)s2::transpose_bitmap_words(layout->num_heads, layout->num_q_blocks) * 4);
  if (!workspace) return fail(S2_EINVAL, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return fail(S2_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(S2_ECAPACITY, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  return hip_status(s2::launch_transpose_layout(layout->row_ptr, layout->col_idx, layout->num_heads,
                                                layout->num_q_blocks, layout->nnz, col_ptr, row_idx,
                                                static_cast<uint32_t *>(workspace), static_cast<hipStream_t>(stream)),
                    "s2_transpose_layout launch");
}

}  // extern "C"
