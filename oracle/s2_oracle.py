"""CPU oracle (numpy, float64) for head-heterogeneous block-sparse causal attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in ``oracle/``.
The HIP product path never does, and this module imports nothing from it.

What is computed (S2-Attention / HHST):
  * S2-Attention OpenReview page, Abstract: attention patterns are customised
    per head and per context range; HHST shards the context across heads so that
    each head attends to a different subset of tokens while the heads together
    cover all of it.  The arXiv abstract (mlsanity page, "Abstract (arXiv)") adds
    that hybrids mixing sparse and dense heads work well.
  * The pages give no formula for the subsets.  The reading taken here: with
    64-token blocks, head h, query block i keeps key block j (j <= i) when
        dense[h]  or  i - j < W  (local window of W blocks, diagonal included)
                  or  (j + h) mod S == 0   (head-offset strided blocks).
  * The attention itself is exact softmax attention restricted to that mask,
    with inclusive token causality (key t visible to query q iff t <= q),
    scale 1/sqrt(D) and a natural-log logsumexp per query row.  The kernels
    reach this result by skipping inactive tiles ("hardware-aware" tiling in
    the manner of FlashAttention, S2-Attention page, Abstract), so the oracle is
    the plain definition, not the tiled algorithm.
  * Backward (the pages' kernels serve training as well as inference: S2-Attention
    OpenReview page, Abstract): gradients of the same masked attention with
    respect to Q, K and V, from the textbook softmax backward on the full masked
    score matrix; the column view of the CSR (query blocks per key block) is the
    plain transpose of the layout.
  * Decode: one query at position p = L - 1 per sequence, keys t <= p of the
    blocks active for (h, p // 64).  Splitting the keys and merging partial
    results is a GPU-side reorganisation (online softmax is associative: Lean
    Attention abstract, on the SampleAttention page's related-papers list) and
    is not done here.
  * Variable-length packed batches: each sequence of a packed batch is an
    independent batch of one, starting at block 0 (``attn_fwd_varlen``).
  * Serving decode: the same decode over a paged cache (block tables, after
    PagedAttention, in the "Builds on" list of the S2-Attention arXiv record on
    the mlsanity page; the OpenReview abstract reports serving in vLLM) with fewer KV heads
    than query heads (grouped- or multi-query attention); ``paged_kv_blocks``
    is the gather that maps (sequence, query head, token) to a cache row.
  * Query-aware block lists (Quest abstract, in the related-papers list of the
    SampleAttention page): the smallest and largest key
    value of every cache page are kept per channel, each page's criticality for
    the current query is estimated from them and the query alone, and only the
    top-K pages are attended to.  Reading taken here: a page is a 64-token block;
    the estimate is the largest q.k that any key inside the per-channel box
    [kmin, kmax] can reach, sum_d max(q_d kmin_d, q_d kmax_d), an upper bound on
    every key of the block; the block holding the query is always kept (the
    query attends to itself, as the diagonal block of the static pattern), the
    other budget - 1 places go to the highest estimates (equal estimates: the
    lower block index first), and the list is ascending.  Attention over the
    list is the ordinary decode over per-(sequence, head) rows.

Parity pins for every function live in tests/test_oracle_*.py.  The only part
with no pin beyond the stated tolerance is the exact bf16 rounding of a given
output element (parity unpinned at the bit level; tolerance only).
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 64


# --------------------------------------------------------------------------
# layout
# --------------------------------------------------------------------------
def active_blocks(h: int, i: int, local_blocks: int, stride: int, dense: bool) -> list[int]:
    """Sorted active key blocks of head h, query block i (set definition)."""
    if dense:
        return list(range(i + 1))
    window = set(range(max(0, i - local_blocks + 1), i + 1))
    first = (-h) % stride                      # smallest j >= 0 with (j + h) % stride == 0
    strided = set(range(first, i + 1, stride))
    return sorted(window | strided)


def build_layout(num_heads: int, num_q_blocks: int, local_blocks: int, stride: int,
                 dense_flags=None):
    """CSR of active key blocks, rows r = h * num_q_blocks + i (head-major).

    Returns (row_ptr int32 [H*nqb+1], col_idx int32 [nnz]); columns ascending.
    """
    if local_blocks < 1 or stride < 1 or num_heads < 1 or num_q_blocks < 0:
        raise ValueError("invalid pattern")
    if dense_flags is None:
        dense_flags = [0] * num_heads
    row_ptr = [0]
    cols: list[int] = []
    for h in range(num_heads):
        for i in range(num_q_blocks):
            a = active_blocks(h, i, local_blocks, stride, bool(dense_flags[h]))
            cols.extend(a)
            row_ptr.append(len(cols))
    return np.asarray(row_ptr, dtype=np.int32), np.asarray(cols, dtype=np.int32)


def row_blocks(row_ptr, col_idx, num_q_blocks: int, h: int, i: int) -> np.ndarray:
    r = h * num_q_blocks + i
    return col_idx[row_ptr[r]:row_ptr[r + 1]]


def token_mask(row_ptr, col_idx, num_q_blocks: int, h: int, N: int) -> np.ndarray:
    """Boolean [N, N] mask of head h: M[q, t] = (t <= q) and block(t) active for block(q)."""
    block_on = np.zeros((num_q_blocks, num_q_blocks), dtype=bool)
    for i in range(num_q_blocks):
        block_on[i, row_blocks(row_ptr, col_idx, num_q_blocks, h, i)] = True
    qb = np.arange(N) // BLOCK
    m = block_on[qb[:, None], qb[None, :]]
    return m & (np.arange(N)[None, :] <= np.arange(N)[:, None])


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def _softmax_rows(s: np.ndarray, v: np.ndarray):
    """Row softmax of scores s (with -inf for masked entries) applied to v.

    A row with no visible key (only in a caller-built layout with an empty row)
    attends to nothing: output 0 and logsumexp -inf, the limit of the empty sum."""
    o = np.zeros((s.shape[0], v.shape[1]))
    lse = np.full(s.shape[0], -np.inf)
    live = np.isfinite(s).any(axis=1) | np.isnan(s).any(axis=1)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1)
        p = np.exp(sl - m[:, None])
        l = p.sum(axis=1)
        o[live] = (p @ v) / l[:, None]
        lse[live] = m + np.log(l)
    return o, lse


def attn_fwd_dense(q, k, v, row_ptr, col_idx, num_q_blocks: int, scale: float | None = None):
    """Mode "dense-mask": full N x N masked scores per (b, h).  For N up to a few thousand.

    q, k, v: arrays [B, H, N, D] (converted to float64).  Returns (O [B,H,N,D], LSE [B,H,N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.empty((B, H, N, D))
    lse = np.empty((B, H, N))
    for h in range(H):
        mask = token_mask(row_ptr, col_idx, num_q_blocks, h, N)
        for b in range(B):
            s = (q[b, h] @ k[b, h].T) * scale
            s[~mask] = -np.inf
            o[b, h], lse[b, h] = _softmax_rows(s, v[b, h])
    return o, lse


def attn_fwd_blocks(q, k, v, row_ptr, col_idx, num_q_blocks: int, scale: float | None = None,
                    heads=None, q_blocks=None, batches=None):
    """Mode "block-gather": per (b, h, i) gather the active key blocks and softmax.

    Same result as ``attn_fwd_dense``; memory per step is 64 x (64 * |row|).
    ``heads`` / ``q_blocks`` / ``batches`` restrict the work to a subset (other
    rows of the result are left NaN), so large problems can be sampled.
    """
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.full((B, H, N, D), np.nan)
    lse = np.full((B, H, N), np.nan)
    heads = range(H) if heads is None else heads
    q_blocks = range(num_q_blocks) if q_blocks is None else q_blocks
    batches = range(B) if batches is None else batches
    for b in batches:
        for h in heads:
            kk = np.asarray(k[b, h], dtype=np.float64)
            vv = np.asarray(v[b, h], dtype=np.float64)
            for i in q_blocks:
                cols = row_blocks(row_ptr, col_idx, num_q_blocks, h, i)
                qpos = np.arange(i * BLOCK, (i + 1) * BLOCK)
                if len(cols) == 0:  # empty row: attends to nothing
                    o[b, h, qpos], lse[b, h, qpos] = 0.0, -np.inf
                    continue
                keys = np.concatenate([np.arange(j * BLOCK, (j + 1) * BLOCK) for j in cols])
                qi = np.asarray(q[b, h, i * BLOCK:(i + 1) * BLOCK], dtype=np.float64)
                s = (qi @ kk[keys].T) * scale
                s[keys[None, :] > qpos[:, None]] = -np.inf
                o[b, h, qpos], lse[b, h, qpos] = _softmax_rows(s, vv[keys])
    return o, lse


def attn_fwd_varlen(q, k, v, cu_seqlens, row_ptr, col_idx, num_q_blocks: int,
                    scale: float | None = None, seqs=None, q_blocks=None):
    """Packed variable-length batch: sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1
    of q, k, v [T, H, D] and attends within itself with the layout's rows
    0 .. ceil(len / 64) - 1, exactly as a batch of one sequence of that length.

    Each sequence is taken out, padded with zero rows to whole blocks (a padded
    key comes after every real query, so the causal mask hides it), passed to
    ``attn_fwd_blocks`` and cut back.  Returns (O [T, H, D], LSE [H, T]); tokens
    of sequences not computed (``seqs`` restricts them, ``q_blocks`` restricts the
    query blocks of each) stay NaN.  A sequence whose range is malformed (it
    starts before 0, ends before it starts or past T) or is longer than the
    layout's 64 * num_q_blocks tokens has no defined result and is skipped: its
    tokens stay NaN ("not written").
    """
    T, H, D = q.shape
    o = np.full((T, H, D), np.nan)
    lse = np.full((H, T), np.nan)
    seqs = range(len(cu_seqlens) - 1) if seqs is None else seqs
    for b in seqs:
        t0, t1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        n = t1 - t0
        if t0 < 0 or t1 > T or n > num_q_blocks * BLOCK:
            continue  # malformed or longer than the layout: skipped
        if n <= 0:
            continue
        nb = -(-n // BLOCK)
        def take(x):
            y = np.zeros((1, H, nb * BLOCK, D))
            y[0, :, :n] = np.asarray(x[t0:t1], dtype=np.float64).transpose(1, 0, 2)
            return y
        blocks = range(nb) if q_blocks is None else [i for i in q_blocks if i < nb]
        ob, lb = attn_fwd_blocks(take(q), take(k), take(v), row_ptr, col_idx, num_q_blocks, scale,
                                 q_blocks=blocks)
        o[t0:t1] = ob[0, :, :n].transpose(1, 0, 2)
        lse[:, t0:t1] = lb[0, :, :n]
    return o, lse


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
def attend_keys(qvec, keys, values, scale: float):
    """Softmax attention of one query vector over explicit key/value rows: (o [D], lse)."""
    qvec = np.asarray(qvec, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:  # no key at all: output 0, logsumexp -inf
        return np.zeros(qvec.shape[0]), -np.inf
    s = (keys @ qvec) * scale
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ values) / l, m + math.log(l)


def _valid_length(n: int, cache_len: int | None) -> bool:
    """A decode length is meaningful for 1 <= n <= cache_len: the query sits at
    position n - 1 of a cache that holds cache_len tokens.  Any other value has no
    query position, and the API's reading for it is a NaN row (output and
    logsumexp), so that a corrupt length cannot pass as a plausible result."""
    return n >= 1 and (cache_len is None or n <= cache_len)


def attn_decode(q, kv_block, seq_lens, row_ptr, col_idx, num_q_blocks: int,
                scale: float | None = None, pairs=None, cache_len: int | None = None):
    """One query per sequence at position p = seq_lens[b] - 1.

    q: [B, H, D].  kv_block(b, h, j) -> (K rows, V rows) of 64-token block j of
    sequence b, head h (arrays [64, D]); only the active blocks are requested.
    A length outside [1, cache_len] (cache_len defaults to the 64 * num_q_blocks
    tokens the layout covers) gives a NaN row and requests no block.
    Returns (O [B, H, D], LSE [B, H]); with ``pairs`` (an iterable of (b, h)) only
    those entries are computed and the rest stay NaN.
    """
    B, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if cache_len is None:
        cache_len = num_q_blocks * BLOCK
    o = np.full((B, H, D), np.nan)
    lse = np.full((B, H), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        if not _valid_length(int(seq_lens[b]), cache_len):
            continue  # stays NaN
        p = int(seq_lens[b]) - 1
        i = p // BLOCK
        ks, vs = [np.zeros((0, D))], [np.zeros((0, D))]
        for j in row_blocks(row_ptr, col_idx, num_q_blocks, h, i):
            kb, vb = kv_block(b, h, int(j))
            t = np.arange(j * BLOCK, (j + 1) * BLOCK)
            keep = t <= p
            ks.append(np.asarray(kb, dtype=np.float64)[keep])
            vs.append(np.asarray(vb, dtype=np.float64)[keep])
        o[b, h], lse[b, h] = attend_keys(q[b, h], np.concatenate(ks), np.concatenate(vs), scale)
    return o, lse


def dense_kv_blocks(k_cache, v_cache):
    """kv_block callable over whole caches [B, H, L, D] (L padded with NaN to a block multiple)."""
    def get(b, h, j):
        kb = np.asarray(k_cache[b, h, j * BLOCK:(j + 1) * BLOCK], dtype=np.float64)
        vb = np.asarray(v_cache[b, h, j * BLOCK:(j + 1) * BLOCK], dtype=np.float64)
        if kb.shape[0] < BLOCK:
            pad = np.full((BLOCK - kb.shape[0], kb.shape[1]), np.nan)
            kb, vb = np.concatenate([kb, pad]), np.concatenate([vb, pad])
        return kb, vb
    return get


def paged_kv_blocks(k_pages, v_pages, block_table, page_size: int, group: int, num_pages=None):
    """kv_block callable over a paged cache with grouped KV heads (serving decode).

    k_pages, v_pages: [num_pages, H_kv, page_size, D]; block_table: [B, max_pages]
    int; query head h reads KV head h // group (consecutive query heads share one
    KV head, as in grouped-query attention; group = H gives multi-query attention,
    group = 1 one KV head per query head).  Token t of sequence b is row t % page_size
    of page block_table[b, t // page_size].  Tokens whose page index falls outside the
    table, or whose page id is outside [0, num_pages), read as NaN.  PagedAttention
    (in the "Builds on" list of the S2-Attention arXiv record, mlsanity page)
    introduced this layout; the result of attention does not depend on where the
    pages lie, which is what makes it a pure gather.
    """
    npg = k_pages.shape[0] if num_pages is None else num_pages
    D = k_pages.shape[3]

    def get(b, h, j):
        kvh = h // group
        kb = np.full((BLOCK, D), np.nan)
        vb = np.full((BLOCK, D), np.nan)
        for r in range(BLOCK):
            t = j * BLOCK + r
            slot = t // page_size
            if slot >= block_table.shape[1]:
                continue
            page = int(block_table[b, slot])
            if 0 <= page < npg:
                kb[r] = np.asarray(k_pages[page, kvh, t % page_size], dtype=np.float64)
                vb[r] = np.asarray(v_pages[page, kvh, t % page_size], dtype=np.float64)
        return kb, vb
    return get


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def transpose_layout(row_ptr, col_idx, num_heads: int, num_q_blocks: int):
    """Column view of the CSR: entry r = h * num_q_blocks + j lists, ascending,
    the query blocks i whose row (h, i) holds key block j.

    Returns (col_ptr int32 [H*nqb+1], row_idx int32 [nnz]).  Plain definition:
    one list per (h, j), filled by scanning the rows in order.
    """
    lists = [[] for _ in range(num_heads * num_q_blocks)]
    for h in range(num_heads):
        for i in range(num_q_blocks):
            for j in row_blocks(row_ptr, col_idx, num_q_blocks, h, i):
                lists[h * num_q_blocks + int(j)].append(i)
    col_ptr = [0]
    rows: list[int] = []
    for lst in lists:
        rows.extend(lst)
        col_ptr.append(len(rows))
    return np.asarray(col_ptr, dtype=np.int32), np.asarray(rows, dtype=np.int32)


def attn_bwd_dense(q, k, v, do, row_ptr, col_idx, num_q_blocks: int, scale: float | None = None,
                   pairs=None):
    """Gradients of O = softmax(masked(Q K^T * scale)) V with respect to Q, K, V,
    given dO, per (b, h) on the full N x N masked score matrix.

    Softmax backward written from its definition: with P the row softmax,
    dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)) (masked entries
    have P = 0), dQ = dS K * scale, dK = dS^T Q * scale.  Everything in float64;
    O is recomputed here, nothing is taken from a forward pass on the GPU.
    Returns (dQ, dK, dV), each [B, H, N, D]; with ``pairs`` (an iterable of
    (b, h)) only those slices are computed and the rest stay NaN.  Inputs may
    be any objects whose [b, h] slices convert to [N, D] arrays.
    """
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    fill = 0.0 if pairs is None else np.nan
    dq, dk, dv = (np.full((B, H, N, D), fill) for _ in range(3))
    if pairs is None:
        pairs = [(b, h) for h in range(H) for b in range(B)]
    masks = {}
    for b, h in pairs:
        if h not in masks:
            masks[h] = token_mask(row_ptr, col_idx, num_q_blocks, h, N)
        mask = masks[h]
        qq, kk, vv, gg = (np.asarray(t[b, h], dtype=np.float64) for t in (q, k, v, do))
        s = (qq @ kk.T) * scale
        s[~mask] = -np.inf
        live = mask.any(axis=1)  # a query with no visible key has P = 0, O = 0
        p = np.zeros_like(s)
        p[live] = np.exp(s[live] - s[live].max(axis=1, keepdims=True))
        p[live] /= p[live].sum(axis=1, keepdims=True)
        o = p @ vv
        dv[b, h] = p.T @ gg
        dp = gg @ vv.T
        delta = (gg * o).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[b, h] = ds @ kk * scale
        dk[b, h] = ds.T @ qq * scale
    return dq, dk, dv


# --------------------------------------------------------------------------
# query-aware block selection (per-block key bounds, top-K by upper bound)
# --------------------------------------------------------------------------
def block_minmax(k_cache, seq_lens):
    """Channel-wise minimum and maximum of the keys of every 64-token block
    (Quest abstract, on the SampleAttention page: the minimal and maximal key
    values of each page).

    k_cache: [B, H, L, D]; only tokens t < seq_lens[b] count.  Returns
    (kmin, kmax), float64 [B, H, ceil(L / 64), D]; blocks without a valid token
    (and every block of a sequence whose length is outside [1, L]) are NaN.
    """
    k = np.asarray(k_cache, dtype=np.float64)
    B, H, L, D = k.shape
    nblk = -(-L // BLOCK)
    kmin = np.full((B, H, nblk, D), np.nan)
    kmax = np.full((B, H, nblk, D), np.nan)
    for b in range(B):
        n = int(seq_lens[b])
        if n < 1 or n > L:
            continue
        for j in range(-(-n // BLOCK)):
            rows = k[b, :, j * BLOCK:min(n, (j + 1) * BLOCK)]  # [H, rows, D]
            kmin[b, :, j] = rows.min(axis=1)
            kmax[b, :, j] = rows.max(axis=1)
    return kmin, kmax


def block_minmax_paged(k_pages, block_table, page_size: int, seq_lens, num_blocks: int):
    """block_minmax over a paged cache: token t of sequence b, K/V head g is row
    t % page_size of page block_table[b, t // page_size] (as paged_kv_blocks).

    k_pages: [num_pages, H_kv, page_size, D].  Returns (kmin, kmax), float64
    [B, H_kv, num_blocks, D]; a sequence is valid when 1 <= seq_lens[b] <=
    min(64 * num_blocks, page_size * table width), else its bounds are NaN."""
    kp = np.asarray(k_pages, dtype=np.float64)
    _, Hkv, P, D = kp.shape
    B = len(seq_lens)
    width = np.asarray(block_table).shape[1]
    kmin = np.full((B, Hkv, num_blocks, D), np.nan)
    kmax = np.full((B, Hkv, num_blocks, D), np.nan)
    for b in range(B):
        n = int(seq_lens[b])
        if n < 1 or n > min(num_blocks * BLOCK, P * width):
            continue
        t = np.arange(n)
        rows = kp[np.asarray(block_table)[b, t // P], :, t % P]  # [n, H_kv, D]
        for j in range(-(-n // BLOCK)):
            blk = rows[j * BLOCK:(j + 1) * BLOCK]
            kmin[b, :, j] = blk.min(axis=0)
            kmax[b, :, j] = blk.max(axis=0)
    return kmin, kmax


def block_scores(q, kmin, kmax):
    """Upper bound of q.k over the box [kmin, kmax] of each block:
    sum over channels of max(q_d kmin_d, q_d kmax_d) (a positive channel of q
    takes the largest key value, a negative one the smallest).

    q: [..., D]; kmin, kmax: [..., nblk, D] -> [..., nblk].
    """
    q = np.asarray(q, dtype=np.float64)[..., None, :]
    return np.maximum(q * np.asarray(kmin, dtype=np.float64), q * np.asarray(kmax, dtype=np.float64)).sum(axis=-1)


def select_blocks(q, kmin, kmax, seq_lens, budget: int, group: int = 1):
    """Per-(sequence, head) block lists for decode at position p = seq_lens[b] - 1.

    Row r = b * H + h holds min(budget, i + 1) ascending block indices, i = p // 64:
    all of 0 .. i when they fit, else block i and the budget - 1 blocks j < i with
    the largest block_scores (equal scores: lower j first).  A sequence whose
    length is outside [1, 64 * nblk] gets an empty row.  With grouped K/V heads
    (kmin, kmax: [B, H / group, nblk, D]) query head h ranks the bounds of K/V head
    h // group with its own query.  Returns (row_ptr [B * H + 1], col_idx) as int32
    arrays.
    """
    B, H, D = np.asarray(q).shape
    nblk = np.asarray(kmin).shape[2]
    rows = []
    for b in range(B):
        n = int(seq_lens[b])
        for h in range(H):
            if n < 1 or n > nblk * BLOCK:
                rows.append([])
                continue
            i = (n - 1) // BLOCK
            if i + 1 <= budget:
                rows.append(list(range(i + 1)))
                continue
            sc = block_scores(q[b, h], kmin[b, h // group, :i], kmax[b, h // group, :i])
            order = sorted(range(i), key=lambda j: (-sc[j], j))
            rows.append(sorted(order[:budget - 1]) + [i])
    row_ptr = np.zeros(B * H + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.array([j for r in rows for j in r], dtype=np.int32)
    return row_ptr, col_idx


def attn_decode_rows(q, kv_block, seq_lens, row_ptr, col_idx, scale: float | None = None, pairs=None,
                     cache_len: int | None = None):
    """Decode over per-(sequence, head) block lists: row b * H + h of the CSR
    lists the key blocks of sequence b, head h; keys t <= p = seq_lens[b] - 1 of
    those blocks are attended to.  Same outputs and conventions as attn_decode;
    a length below 1, or above cache_len when it is given, gives a NaN row."""
    B, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.full((B, H, D), np.nan)
    lse = np.full((B, H), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        if not _valid_length(int(seq_lens[b]), cache_len):
            continue  # stays NaN
        p = int(seq_lens[b]) - 1
        r = b * H + h
        ks, vs = [np.zeros((0, D))], [np.zeros((0, D))]
        for j in col_idx[row_ptr[r]:row_ptr[r + 1]]:
            kb, vb = kv_block(b, h, int(j))
            t = np.arange(j * BLOCK, (j + 1) * BLOCK)
            keep = t <= p
            ks.append(np.asarray(kb, dtype=np.float64)[keep])
            vs.append(np.asarray(vb, dtype=np.float64)[keep])
        o[b, h], lse[b, h] = attend_keys(q[b, h], np.concatenate(ks), np.concatenate(vs), scale)
    return o, lse
