/*
 * s2attn.h -- C ABI of the MI355X (gfx950) head-heterogeneous block-sparse
 * causal attention library (S2-Attention / HHST pattern).
 *
 * What the library computes.  "S2-ATTENTION: Hardware-Aware Context Sharding
 * Among Attention Heads" (OpenReview page, Abstract) describes sparse attention
 * whose pattern is chosen per head and per context range, and the HHST
 * architecture in which every head attends to a different subset of the context
 * while the heads together cover all of it; its arXiv abstract (mlsanity page,
 * "Abstract (arXiv)") adds hybrid models with some fully dense heads.  The pages
 * give no formula for the subsets; this library uses 64-token blocks and, for
 * head h and query block i, the key blocks j <= i with
 *     dense[h]  or  i - j < W   or   (j + h) mod S == 0
 * (W = local window in blocks, diagonal included; S = stride).  Within the
 * active blocks attention is exact causal softmax attention (key t visible to
 * query q iff t <= q), scale 1/sqrt(D) unless given, logsumexp in natural log.
 * Every attention entry point also accepts a caller-built layout in the same
 * CSR form (any per-head, per-context-range block pattern; see
 * s2_validate_layout).  Decode can also read per-(sequence, head) block lists
 * chosen at run time from the keys' per-block bounds and the query
 * (s2_select_blocks, s2_attn_decode_rows).
 *
 * Conventions for every entry point:
 *  - Tensors are in device memory owned by the caller; the library never
 *    allocates, frees or keeps device memory and keeps no device state between
 *    calls: scratch (work queues, split partials, gradient plans) comes in
 *    caller-owned workspace arguments.
 *  - Strides are in elements, int64, one per dimension; the last dimension
 *    (D) must have stride 1.  Base pointers must be 16-byte aligned and every
 *    other stride a multiple of 8 elements (bf16) or 4 elements (fp32).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t, NULL = the
 *    default stream).  Nothing synchronises except s2_validate_layout, which
 *    waits for its own result; kernel faults surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated on the host before any launch.  On error the
 *    call returns a non-zero s2_status, enqueues nothing, and s2_last_error()
 *    describes the problem.  Nothing throws or aborts across the ABI.
 *  - Entry points are thread-safe; the error message is per thread.
 */
#ifndef S2ATTN_H
#define S2ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S2_ABI_VERSION 2
#define S2_BLOCK 64 /* tokens per query block and per key block */

typedef enum {
  S2_OK = 0,
  S2_EINVAL = 1,       /* null pointer, bad size, bad stride, bad pattern */
  S2_EUNSUPPORTED = 2, /* valid request this build does not implement */
  S2_ECAPACITY = 3,    /* caller buffer (col_idx, workspace) too small */
  S2_EHIP = 4          /* the HIP runtime reported an error at launch */
} s2_status;

typedef enum { S2_F32 = 0, S2_BF16 = 1 } s2_dtype;

/* The HHST pattern (S2-Attention OpenReview page, Abstract; hybrid dense heads:
 * arXiv abstract).  `dense` is a HOST array of num_heads bytes (non-zero = the
 * head attends to every causal block) or NULL for no dense heads; it is read
 * during the call only. */
typedef struct {
  int32_t num_heads;    /* H >= 1 */
  int32_t block_size;   /* must be S2_BLOCK */
  int32_t local_blocks; /* W >= 1, window of key blocks ending at the diagonal */
  int32_t stride;       /* S >= 1, head h keeps blocks j with (j + h) % S == 0 */
  const uint8_t *dense; /* host [num_heads] or NULL */
} s2_pattern;

/* Block-sparse layout in CSR form: row r = h * num_q_blocks + i lists the
 * active key blocks j of head h, query block i, strictly ascending with
 * 0 <= j <= i.  s2_build_layout's rows always end with i; a caller-built row
 * may lack its diagonal block or be empty (see "Caller-built layouts" below).
 * row_ptr: device int32 [num_heads * num_q_blocks + 1], row_ptr[0] = 0;
 * col_idx: device int32 [nnz].  Any CSR obeying these rules is accepted by the
 * attention entry points (per head, per context range patterns); the kernels
 * trust its contents. */
typedef struct {
  int32_t num_heads;
  int32_t num_q_blocks;
  int32_t block_size; /* must be S2_BLOCK */
  int64_t nnz;        /* row_ptr[last]; must be < 2^31 */
  const int32_t *row_ptr;
  const int32_t *col_idx;
} s2_layout;

/* Version of this ABI (S2_ABI_VERSION). */
int32_t s2_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next s2_* call on the same thread. */
const char *s2_last_error(void);

/* Number of active blocks of `pattern` over num_q_blocks query blocks (host
 * only, closed form).  Writes *nnz.  S2_EINVAL on a bad pattern or NULL. */
s2_status s2_layout_nnz(const s2_pattern *pattern, int32_t num_q_blocks, int64_t *nnz);

/* Build the CSR layout of `pattern` on the device (one kernel on `stream`).
 * row_ptr: device int32 [H * num_q_blocks + 1]; col_idx: device int32 with room
 * for col_capacity entries (S2_ECAPACITY if fewer than s2_layout_nnz).
 * The result is bit-identical to the rule stated at the top of this file. */
s2_status s2_build_layout(const s2_pattern *pattern, int32_t num_q_blocks, int32_t *row_ptr,
                          int32_t *col_idx, int64_t col_capacity, void *stream);

/* Column view of the pattern's layout, for the key side of the backward pass:
 * entry c = h * num_q_blocks + j lists, ascending, the query blocks i whose
 * row (h, i) holds key block j (the transpose of s2_build_layout's CSR).
 * col_ptr: device int32 [H * num_q_blocks + 1]; row_idx: device int32 with room
 * for `capacity` entries (S2_ECAPACITY if fewer than s2_layout_nnz).  One
 * kernel on `stream`.  Pass the result to s2_attn_bwd as an s2_layout whose
 * row_ptr/col_idx are col_ptr/row_idx. */
s2_status s2_build_layout_t(const s2_pattern *pattern, int32_t num_q_blocks, int32_t *col_ptr,
                            int32_t *row_idx, int64_t capacity, void *stream);

/* Bytes of device workspace s2_attn_fwd and s2_attn_fwd_varlen need (the
 * persistent launch's work queues: one 64-bit counter per XCD, each on its own
 * 128-byte line; 1 KiB).  Writes *bytes; fails only on NULL. */
s2_status s2_attn_fwd_workspace(size_t *bytes);

/* Block-sparse causal attention forward (prefill / training forward), the
 * S2-Attention kernels' exact attention over the active tiles (OpenReview page,
 * Abstract).
 *   q, k, v, o : [B, H, N, D] with strides qs/ks/vs/os, dtype `dtype`
 *                (o is written in the same dtype; accumulation is fp32)
 *   lse        : device fp32 [B, H, N] contiguous, natural-log logsumexp of
 *                each query row's scaled scores, or NULL to skip
 *   layout     : num_heads = H, num_q_blocks = N / 64, block_size = 64
 *   workspace  : device memory of at least s2_attn_fwd_workspace() bytes,
 *                8-byte aligned, for the work queues of the bf16 launch (the
 *                fp32 path does not touch it but it must still be given).  Any
 *                content is valid: each launch tags the queue words with its
 *                own launch number, so nothing needs clearing between calls.
 *                Two launches in flight at the same time (on different
 *                streams) must use different workspaces; one workspace may
 *                serve any number of launches in stream order.
 *   sm_scale   : softmax scale; <= 0 selects 1/sqrt(D)
 * N must be a positive multiple of 64; D must be 64 or 128.  S2_ECAPACITY if
 * the workspace is smaller than s2_attn_fwd_workspace().
 * Each output row depends only on the active key blocks of its CSR row.
 * The environment variable S2ATTN_FWD_PIPELINED=1, read at each call, selects
 * an alternative schedule of the bf16 kernel (same result within rounding,
 * slower on MI355X; kept for comparison). */
s2_status s2_attn_fwd(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t N, int32_t D,
                      const void *q, const int64_t qs[4], const void *k, const int64_t ks[4],
                      const void *v, const int64_t vs[4], void *o, const int64_t os[4], float *lse,
                      void *workspace, size_t workspace_bytes, float sm_scale, void *stream);

/* Forward over a packed batch of sequences of different lengths (varlen
 * prefill): sequence b is tokens cu_seqlens[b] .. cu_seqlens[b + 1] - 1 of
 * [T_total, H, D] tensors, and attends within itself with the layout's rows
 * 0 .. ceil(len / 64) - 1 (every sequence starts at block 0).  Lengths need not
 * be multiples of 64: the last block of a sequence is partial, and no token of
 * another sequence is read.
 *   cu_seqlens : device int32 [B + 1], non-decreasing from 0 to at most
 *                T_total; a sequence with a malformed range or longer than
 *                num_q_blocks * 64 tokens is skipped (its outputs are not
 *                written)
 *   q, k, v, o : [T_total, H, D] bf16 with strides (token, head, 1) in
 *                elements, multiples of 8
 *   lse        : device fp32 [H, T_total] contiguous (natural log) or NULL
 *   workspace  : as for s2_attn_fwd (s2_attn_fwd_workspace() bytes, any
 *                content, not shared by launches in flight together)
 * dtype must be S2_BF16 (S2_EUNSUPPORTED otherwise); D 64 or 128.  One
 * persistent launch on `stream`. */
s2_status s2_attn_fwd_varlen(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t T_total, int32_t D,
                             const int32_t *cu_seqlens, const void *q, const int64_t qs[3], const void *k,
                             const int64_t ks[3], const void *v, const int64_t vs[3], void *o,
                             const int64_t os[3], float *lse, void *workspace, size_t workspace_bytes,
                             float sm_scale, void *stream);

/* Bytes of the s2_attn_bwd workspace: 2 * B * H * N floats, then
 * B * H * (nqb + ceil(nqb / 2)) int32 with nqb = N / 64 (the order of the
 * kernels' work). */
s2_status s2_attn_bwd_workspace(int32_t B, int32_t H, int32_t N, size_t *bytes);

/* Block-sparse causal attention backward (training): the gradients dQ, dK, dV
 * of the forward's output with respect to q, k, v, given dout = dL/dO.
 *   layout     : the forward's layout (key blocks per query block)
 *   layout_t   : its column view (s2_build_layout_t): same num_heads,
 *                num_q_blocks and nnz, row_ptr/col_idx = col_ptr/row_idx
 *   q, k, v, o, dout, dq, dk, dv : [B, H, N, D] bf16 with strides in
 *                elements; o is the forward's output
 *   lse        : device fp32 [B, H, N] contiguous, the forward's logsumexp
 *   workspace  : device memory of s2_attn_bwd_workspace bytes, 256-byte
 *                aligned (holds rowsum(dout * o) and -lse * log2(e), fp32,
 *                and the order in which the kernels take their work);
 *                overwritten by every call
 *   sm_scale   : the forward's softmax scale; <= 0 selects 1/sqrt(D)
 * The probabilities are recomputed from lse (not stored); accumulation is
 * fp32 and dq/dk/dv are written in bf16.  dtype must be S2_BF16
 * (S2_EUNSUPPORTED otherwise); D must be 64 or 128.  Every element of dq, dk
 * and dv is written (key blocks no row holds get zero gradients).  Three
 * kernels on `stream`. */
s2_status s2_attn_bwd(const s2_layout *layout, const s2_layout *layout_t, s2_dtype dtype, int32_t B,
                      int32_t N, int32_t D, const void *q, const int64_t qs[4], const void *k,
                      const int64_t ks[4], const void *v, const int64_t vs[4], const void *o,
                      const int64_t os[4], const void *dout, const int64_t dos[4], const float *lse,
                      void *dq, const int64_t dqs[4], void *dk, const int64_t dks[4], void *dv,
                      const int64_t dvs[4], void *workspace, size_t workspace_bytes, float sm_scale,
                      void *stream);

/* Bytes of device workspace s2_attn_decode needs for `splits` key splits per
 * (sequence, head) (splits <= 0: the automatic choice for this layout and B). */
s2_status s2_attn_decode_workspace(const s2_layout *layout, int32_t B, int32_t D, int32_t splits,
                                   size_t *bytes);

/* Single-token decode against a contiguous KV cache, split over the active key
 * blocks and merged by logsumexp (online softmax is associative: Lean Attention
 * abstract, listed on the SampleAttention page).
 *   q          : [B, H, D] (strides qs), the query of the token at position
 *                p = seq_lens[b] - 1 of sequence b
 *   k_cache,
 *   v_cache    : [B, H, cache_len, D] (strides ks / vs); tokens 0..p of sequence
 *                b are valid, including the query token's own key/value
 *   seq_lens   : device int32 [B]; entries outside [1, cache_len] give a NaN
 *                output row and are never used to address the cache
 *   o          : [B, H, D] (strides os), same dtype as q
 *   lse        : device fp32 [B, H] contiguous or NULL
 *   layout     : num_heads = H, num_q_blocks >= ceil(cache_len / 64); row
 *                (h, p / 64) selects the key blocks, restricted to t <= p
 *   splits     : key-block splits per (b, h); <= 0 = automatic
 *   workspace  : device buffer of at least s2_attn_decode_workspace() bytes,
 *                256-byte aligned; its contents need no initialisation
 * D must be 64 or 128. */
s2_status s2_attn_decode(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t D,
                         const void *q, const int64_t qs[3], const void *k_cache,
                         const int64_t ks[4], const void *v_cache, const int64_t vs[4],
                         const int32_t *seq_lens, int32_t cache_len, void *o, const int64_t os[3],
                         float *lse, int32_t splits, void *workspace, size_t workspace_bytes,
                         float sm_scale, void *stream);

/* Bytes of the static device scratch behind s2_attn_decode_noalloc (16 MiB per
 * GPU, held from the library's load until the process ends). */
#define S2_NOALLOC_SCRATCH_BYTES (16u << 20)

/* s2_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * s2_attn_decode with the same `splits` (bit-identical outputs).  The split
 * partials go to a static scratch array of S2_NOALLOC_SCRATCH_BYTES in the
 * library's code object, one per GPU; its address on the current device is
 * looked up once (hipGetSymbolAddress) on the first call there.  No call
 * allocates or frees anything.  Requests whose partials, B * H * splits * (D + 1)
 * floats (each part rounded up to 256 bytes), exceed the scratch return
 * S2_ECAPACITY before any launch.  Nothing in the scratch needs clearing: every
 * partial is written before it is read.  Every call on a GPU shares that GPU's
 * scratch, which keeps the last call's partials: calls of one process that
 * overlap in time on one GPU (on different streams or from different threads,
 * kernels in flight together) race and must not be issued; calls in stream
 * order are safe. */
s2_status s2_attn_decode_noalloc(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t D,
                                 const void *q, const int64_t qs[3], const void *k_cache,
                                 const int64_t ks[4], const void *v_cache, const int64_t vs[4],
                                 const int32_t *seq_lens, int32_t cache_len, void *o, const int64_t os[3],
                                 float *lse, int32_t splits, float sm_scale, void *stream);

/* Caller-built layouts.  The S2-Attention OpenReview abstract stresses that
 * the sparsity may be customised per head and per context range; any block
 * layout in this CSR form is accepted by every s2_attn_* entry point:
 * rows r = h * num_q_blocks + i (head-major), row_ptr int32 [H * num_q_blocks + 1]
 * non-decreasing from 0 to nnz, and in each row strictly ascending key blocks j
 * with 0 <= j <= i.  A row may be empty: its queries attend to nothing and get
 * output 0 and lse -inf.  On the diagonal block the token-level mask t <= q
 * applies as for the built-in pattern.
 *
 * s2_validate_layout checks those rules on the device and returns S2_OK or
 * S2_EINVAL naming the first bad row.  scratch: 8 bytes of 8-byte aligned
 * device memory (overwritten).  Synchronous: it waits for `stream`.  The
 * attention entry points do not re-check a layout; one that breaks the rules
 * gives unspecified results (blocks outside [0, num_q_blocks) are never read
 * by the column-view builder, which only trusts row_ptr within [0, nnz]). */
s2_status s2_validate_layout(const s2_layout *layout, void *scratch, void *stream);

/* Bytes of device workspace s2_transpose_layout needs: one bit per block of
 * every head's num_q_blocks x num_q_blocks grid, rounded up to 256. */
s2_status s2_transpose_layout_workspace(const s2_layout *layout, size_t *bytes);

/* Column view of any valid layout (the input s2_attn_bwd needs as layout_t):
 * col_ptr int32 [H * num_q_blocks + 1] and row_idx int32 [capacity >= nnz],
 * column c = h * num_q_blocks + j listing, ascending, the query blocks i whose
 * row holds j.  workspace: s2_transpose_layout_workspace bytes, 256-byte
 * aligned, no initialisation needed.  Five kernels on `stream`. */
s2_status s2_transpose_layout(const s2_layout *layout, int32_t *col_ptr, int32_t *row_idx, int64_t capacity,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace s2_attn_decode_paged needs (0 when the split
 * count, given or automatic, is 1).  num_kv_heads must divide the layout's
 * num_heads. */
s2_status s2_attn_decode_paged_workspace(const s2_layout *layout, int32_t B, int32_t num_kv_heads,
                                         int32_t D, int32_t splits, size_t *bytes);

/* Serving decode: one query token per sequence against a paged K/V cache with
 * grouped K/V heads.  The S2-Attention OpenReview abstract reports serving in
 * vLLM, whose cache is paged through block tables (PagedAttention, in the
 * "Builds on" list of the S2-Attention arXiv record, mlsanity page).
 *   layout     : num_heads = H query heads; row (h, p / 64) selects the key
 *                blocks of query head h, restricted to t <= p
 *   q          : [B, H, D] (strides qs), the query of the token at position
 *                p = seq_lens[b] - 1 of sequence b
 *   k_pages,
 *   v_pages    : page pools [num_pages, num_kv_heads, page_size, D] (strides
 *                kps / vps, D contiguous); query head h reads K/V head
 *                h / (H / num_kv_heads)
 *   page_size  : tokens per page, a power of two in [1, 65536]
 *   block_table: device int32 [B, bt_stride]; token t of sequence b is row
 *                t mod page_size of page block_table[b * bt_stride + t / page_size];
 *                entries 0 .. ceil(seq_lens[b] / page_size) - 1 are read.  A
 *                page id outside [0, num_pages) reads as NaN: the heads whose
 *                active blocks use it get NaN output and lse, nothing is read
 *                out of bounds
 *   max_pages_per_seq : table entries per sequence; seq_lens[b] may be at
 *                most max_pages_per_seq * page_size, which must be within the
 *                layout (num_q_blocks * 64)
 *   seq_lens   : device int32 [B]; entries outside [1, max_pages_per_seq *
 *                page_size] give a NaN output row and are never used to address
 *                the cache
 *   o          : [B, H, D] (strides os), same dtype as q
 *   lse        : device fp32 [B, H] contiguous (natural log) or NULL
 *   splits     : runs each head's row is cut into; <= 0 = automatic
 *   workspace  : with more than one split, device memory of
 *                s2_attn_decode_paged_workspace bytes, 256-byte aligned, for
 *                the partial results (no initialisation needed); a call with
 *                one split may pass NULL
 * One launch on `stream`, two with several splits (the second merges them by
 * logsumexp).  dtype S2_BF16 or S2_F32; D 64 or 128. */
s2_status s2_attn_decode_paged(const s2_layout *layout, s2_dtype dtype, int32_t B, int32_t num_kv_heads,
                               int32_t D, const void *q, const int64_t qs[3], const void *k_pages,
                               const int64_t kps[4], const void *v_pages, const int64_t vps[4],
                               int32_t num_pages, int32_t page_size, const int32_t *block_table,
                               int64_t bt_stride, int32_t max_pages_per_seq, const int32_t *seq_lens,
                               void *o, const int64_t os[3], float *lse, int32_t splits, void *workspace,
                               size_t workspace_bytes, float sm_scale, void *stream);

/* ---- query-aware block lists for decode (Quest abstract, in the related-papers
 * list of the SampleAttention page) ----
 * The smallest and largest key value of every 64-token block are kept per
 * channel; a block's criticality for a query q is the largest q.k any key in
 * that per-channel box can reach, sum_d max(q_d * kmin_d, q_d * kmax_d) (an
 * upper bound on the block's true scores); decode then attends only to the
 * block holding the query and the budget - 1 earlier blocks ranked highest. */

/* Channel-wise minima and maxima of the keys of every 64-token block.
 *   k_cache    : [B, H, cache_len, D] (strides ks), dtype S2_BF16 or S2_F32
 *   seq_lens   : device int32 [B]; only tokens t < seq_lens[b] count.  Blocks
 *                j < ceil(seq_lens[b] / 64) are written; other blocks, and every
 *                block of a sequence whose length is outside [1, cache_len],
 *                are left untouched
 *   kmin, kmax : device [B, H, num_blocks, D] contiguous, the keys' dtype,
 *                16-byte aligned, caller-owned; num_blocks * 64 >= cache_len
 * Minima and maxima of bf16 keys are exact (-0 counts as below +0); keys must
 * be finite: a NaN key leaves its channel's bounds unspecified.  One launch on
 * `stream`; it reads each valid key once (a serving system calls it when
 * blocks fill). */
s2_status s2_block_minmax(s2_dtype dtype, int32_t B, int32_t H, int32_t D, const void *k_cache,
                          const int64_t ks[4], const int32_t *seq_lens, int32_t cache_len, void *kmin,
                          void *kmax, int32_t num_blocks, void *stream);

/* s2_block_minmax over a paged cache (the s2_attn_decode_paged layout):
 *   k_pages    : [num_pages, num_kv_heads, page_size, D] (strides kps)
 *   block_table, bt_stride, max_pages_per_seq, page_size, num_pages : as in
 *                s2_attn_decode_paged; token t of sequence b is row
 *                t % page_size of page block_table[b * bt_stride + t / page_size]
 *   seq_lens   : device int32 [B]; lengths outside [1, max_pages_per_seq *
 *                page_size] write nothing
 *   kmin, kmax : device [B, num_kv_heads, num_blocks, D] contiguous, 16-byte
 *                aligned; num_blocks * 64 >= max_pages_per_seq * page_size
 * A block with a row whose page id lies outside [0, num_pages) gets NaN bounds
 * (that page is not read).  Otherwise as s2_block_minmax.  One launch on
 * `stream`, one workgroup per (sequence, 64-token block) for all K/V heads. */
s2_status s2_block_minmax_paged(s2_dtype dtype, int32_t B, int32_t num_kv_heads, int32_t D,
                                const void *k_pages, const int64_t kps[4], int32_t num_pages, int32_t page_size,
                                const int32_t *block_table, int64_t bt_stride, int32_t max_pages_per_seq,
                                const int32_t *seq_lens, void *kmin, void *kmax, int32_t num_blocks,
                                void *stream);

/* Per-(sequence, head) block lists from the block bounds, as a CSR that
 * s2_attn_decode_rows and s2_attn_decode_paged_rows read.
 *   q          : [B, H, D] (strides qs), the decode queries
 *   num_kv_heads : K/V heads of the bounds (divides H); query head h ranks
 *                the bounds of K/V head h / (H / num_kv_heads) with its own query
 *   kmin, kmax : s2_block_minmax (num_kv_heads = H) or s2_block_minmax_paged
 *                output, [B, num_kv_heads, num_blocks, D], for the same seq_lens
 *   cache_len  : the longest sequence the bounds cover: the cache length, or
 *                max_pages_per_seq * page_size for a paged cache
 *   num_blocks : their block dimension; num_blocks * 64 >= cache_len and
 *                num_blocks <= 16000 (a 1,024,000-token context)
 *   seq_lens   : device int32 [B]; the query of sequence b is token
 *                p = seq_lens[b] - 1, in block i = p / 64
 *   budget     : blocks per row, >= 1
 *   row_ptr    : device int32 [B * H + 1], written: row r = b * H + h
 *   col_idx    : device int32, capacity col_capacity >= B * H *
 *                min(budget, ceil(cache_len / 64)); written
 * Row (b, h) holds min(budget, i + 1) ascending block indices: all of 0..i when
 * they fit, else block i and the budget - 1 blocks j < i with the largest
 * bounds (equal bounds: the lower j first).  A sequence whose length is
 * outside [1, cache_len] gets empty rows.  The bounds are computed in fp32
 * from the q and box values (exact products; the sum's rounding can order
 * near-equal bounds either way).  One launch on `stream`, one workgroup per
 * (sequence, head). */
s2_status s2_select_blocks(s2_dtype dtype, int32_t B, int32_t H, int32_t num_kv_heads, int32_t D, const void *q,
                           const int64_t qs[3], const void *kmin, const void *kmax, int32_t num_blocks,
                           const int32_t *seq_lens, int32_t cache_len, int32_t budget, int32_t *row_ptr,
                           int32_t *col_idx, int64_t col_capacity, void *stream);

/* Bytes of device workspace s2_attn_decode_rows needs (splits <= 0: the
 * automatic choice for B * H rows of at most max_row_blocks blocks). */
s2_status s2_attn_decode_rows_workspace(int32_t B, int32_t H, int32_t D, int32_t max_row_blocks,
                                        int32_t splits, size_t *bytes);

/* Single-token decode over per-(sequence, head) block lists (s2_select_blocks
 * output, or any CSR of that shape): the same arguments, outputs and error
 * behaviour as s2_attn_decode, with the layout replaced by
 *   row_ptr, col_idx : device int32 CSR of B * H rows; row b * H + h lists the
 *                key blocks of sequence b, head h (keys t <= p of them are
 *                attended to; entries outside [0, p / 64] are skipped)
 *   max_row_blocks   : the longest row (>= 1), for the automatic split count
 * An empty row gives output 0 and lse -inf.  One launch on `stream`, two with
 * several splits. */
s2_status s2_attn_decode_rows(s2_dtype dtype, int32_t B, int32_t H, int32_t D, const int32_t *row_ptr,
                              const int32_t *col_idx, int32_t max_row_blocks, const void *q,
                              const int64_t qs[3], const void *k_cache, const int64_t ks[4],
                              const void *v_cache, const int64_t vs[4], const int32_t *seq_lens,
                              int32_t cache_len, void *o, const int64_t os[3], float *lse, int32_t splits,
                              void *workspace, size_t workspace_bytes, float sm_scale, void *stream);

/* Bytes of device workspace s2_attn_decode_paged_rows needs (0 with one split;
 * splits <= 0: the automatic choice for rows of at most max_row_blocks blocks). */
s2_status s2_attn_decode_paged_rows_workspace(int32_t B, int32_t H, int32_t num_kv_heads, int32_t D,
                                              int32_t max_row_blocks, int32_t splits, size_t *bytes);

/* Serving decode (s2_attn_decode_paged) over per-(sequence, head) block lists:
 * the same arguments, outputs and error behaviour, with the layout replaced by
 *   H                : query heads (num_kv_heads divides it)
 *   row_ptr, col_idx : device int32 CSR of B * H rows, row b * H + h listing the
 *                      ascending key blocks of sequence b, query head h (keys
 *                      t <= p of them are attended to; entries outside
 *                      [0, p / 64] are skipped)
 *   max_row_blocks   : the longest row (>= 1), for the automatic split count
 * A workgroup walks the union of the rows of the query heads that share a K/V
 * head, so a block several of them list is read once. */
s2_status s2_attn_decode_paged_rows(s2_dtype dtype, int32_t B, int32_t H, int32_t num_kv_heads, int32_t D,
                                    const int32_t *row_ptr, const int32_t *col_idx, int32_t max_row_blocks,
                                    const void *q, const int64_t qs[3], const void *k_pages,
                                    const int64_t kps[4], const void *v_pages, const int64_t vps[4],
                                    int32_t num_pages, int32_t page_size, const int32_t *block_table,
                                    int64_t bt_stride, int32_t max_pages_per_seq, const int32_t *seq_lens,
                                    void *o, const int64_t os[3], float *lse, int32_t splits,
                                    void *workspace, size_t workspace_bytes, float sm_scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* S2ATTN_H */
