"""Pins of the oracle's packed variable-length forward.

Each sequence must behave as a batch of one: a single sequence whose length is a
multiple of 64 reduces to the fixed-length forward; every row of a ragged
sequence equals single-query attention over that sequence's own keys (the decode
definition, pinned on its own); and no sequence sees another."""
import numpy as np
import pytest

import oracle

BLOCK = oracle.BLOCK


def _setup(lens, H=3, D=8, W=2, S=3, dense=(1,), seed=0):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    nqb = -(-max(lens) // BLOCK)
    rp, ci = oracle.build_layout(H, nqb, W, S, [1 if h in dense else 0 for h in range(H)])
    q, k, v = (rng.standard_normal((T, H, D)) for _ in range(3))
    return rng, cu, nqb, rp, ci, q, k, v


def test_single_aligned_sequence_equals_fixed_length():
    rng, cu, nqb, rp, ci, q, k, v = _setup([256])
    o, lse = oracle.attn_fwd_varlen(q, k, v, cu, rp, ci, nqb)
    of, lf = oracle.attn_fwd_blocks(q.transpose(1, 0, 2)[None], k.transpose(1, 0, 2)[None],
                                    v.transpose(1, 0, 2)[None], rp, ci, nqb)
    assert np.array_equal(o, of[0].transpose(1, 0, 2)) and np.array_equal(lse, lf[0])


@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 130], [200, 7, 129]])
def test_ragged_rows_equal_single_query_attention(lens):
    rng, cu, nqb, rp, ci, q, k, v = _setup(lens)
    o, lse = oracle.attn_fwd_varlen(q, k, v, cu, rp, ci, nqb)
    H = q.shape[1]
    for b, n in enumerate(lens):
        t0 = int(cu[b])
        cache_k = k[t0:t0 + n].transpose(1, 0, 2)[None]
        cache_v = v[t0:t0 + n].transpose(1, 0, 2)[None]
        kv = oracle.dense_kv_blocks(cache_k, cache_v)
        for t in sorted({0, n // 2, n - 1}):
            od, ld = oracle.attn_decode(q[t0 + t][None], kv, [t + 1], rp, ci, nqb)
            assert np.max(np.abs(od[0] - o[t0 + t])) < 1e-12
            assert np.max(np.abs(ld[0] - lse[:, t0 + t])) < 1e-12


def test_sequences_do_not_see_each_other():
    rng, cu, nqb, rp, ci, q, k, v = _setup([100, 150, 70])
    o, lse = oracle.attn_fwd_varlen(q, k, v, cu, rp, ci, nqb)
    k2, v2 = k.copy(), v.copy()
    k2[:100] += 5.0       # sequence 0's keys and values change
    v2[:100] -= 3.0
    o2, lse2 = oracle.attn_fwd_varlen(q, k2, v2, cu, rp, ci, nqb)
    assert np.array_equal(o[100:], o2[100:]) and np.array_equal(lse[:, 100:], lse2[:, 100:])
    assert not np.allclose(o[:100], o2[:100])


def test_planted_offset_mistake_is_caught():
    # a packing read one token late breaks the single-query-attention pin
    rng, cu, nqb, rp, ci, q, k, v = _setup([90, 90])
    shifted = np.roll(k, -1, axis=0)
    o, _ = oracle.attn_fwd_varlen(q, shifted, v, cu, rp, ci, nqb)
    t0, n = 90, 90
    kv = oracle.dense_kv_blocks(k[t0:t0 + n].transpose(1, 0, 2)[None], v[t0:t0 + n].transpose(1, 0, 2)[None])
    od, _ = oracle.attn_decode(q[t0 + 50][None], kv, [51], rp, ci, nqb)
    assert np.max(np.abs(od[0] - o[t0 + 50])) > 1e-6


def test_malformed_sequences_are_skipped():
    """A sequence whose range is malformed or longer than the layout has no defined
    result: its tokens stay NaN, and the well-formed sequences equal their result in
    a batch of their own."""
    rng, cu, nqb, rp, ci, q, k, v = _setup([100, 60, 20])
    T = q.shape[0]
    bad = np.array([0, 100, 90, 200, T], dtype=np.int32)   # seq 1 ends before it starts, seq 2 past T
    o, lse = oracle.attn_fwd_varlen(q, k, v, bad, rp, ci, nqb)
    ok, lok = oracle.attn_fwd_varlen(q[:100], k[:100], v[:100], np.array([0, 100], dtype=np.int32), rp, ci, nqb)
    assert np.array_equal(o[:100], ok) and np.array_equal(lse[:, :100], lok)
    assert np.isnan(o[100:]).all() and np.isnan(lse[:, 100:]).all()
    # one sequence longer than the 64 * nqb tokens the layout covers
    long_cu = np.array([0, nqb * BLOCK + 1], dtype=np.int32)
    qq = rng.standard_normal((nqb * BLOCK + 1, q.shape[1], q.shape[2]))
    o2, l2 = oracle.attn_fwd_varlen(qq, qq, qq, long_cu, rp, ci, nqb)
    assert np.isnan(o2).all() and np.isnan(l2).all()
    # a negative start
    o3, _ = oracle.attn_fwd_varlen(q, k, v, np.array([-1, 50], dtype=np.int32), rp, ci, nqb)
    assert np.isnan(o3).all()
