"""Pins of the oracle's query-aware block selection (Quest abstract, on the
SampleAttention page's related-papers list: keep the
smallest and largest key value of every page, estimate each page's criticality from
them and the query, attend to the top-K pages).

Each pin reaches the oracle's result by another route: the key bounds by the
property that defines them (every key inside, every bound reached), the estimate
by brute force over the corners of the box and by a worked example, the selection
by a rank definition and by exhaustive search over subsets, and decode over the
lists by the dense decode it reduces to."""
import itertools

import numpy as np
import pytest

import oracle

BLOCK = oracle.BLOCK


def _keys(seed, B, H, L, D, lens):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, H, L, D))
    for b, n in enumerate(lens):
        if 0 <= n < L:
            k[b, :, n:] = 1e6 * np.sign(rng.standard_normal((H, L - n, D)))  # must never count
    return k


def test_minmax_bounds_hold_and_are_reached():
    lens = [200, 70, 64, 1]
    k = _keys(1, 4, 3, 200, 8, lens)
    kmin, kmax = oracle.block_minmax(k, lens)
    assert kmin.shape == (4, 3, 4, 8)
    for b, n in enumerate(lens):
        for j in range(4):
            if j * BLOCK >= n:
                assert np.isnan(kmin[b, :, j]).all() and np.isnan(kmax[b, :, j]).all()
                continue
            rows = k[b, :, j * BLOCK:min(n, (j + 1) * BLOCK)]
            assert (rows >= kmin[b, :, j][:, None]).all() and (rows <= kmax[b, :, j][:, None]).all()
            assert (rows == kmin[b, :, j][:, None]).any(axis=1).all()
            assert (rows == kmax[b, :, j][:, None]).any(axis=1).all()
            assert np.abs(kmax[b, :, j]).max() < 100  # the padding never leaks in


def test_minmax_invalid_lengths_give_no_bounds():
    k = _keys(2, 3, 2, 128, 4, [0, 129, 128])
    kmin, kmax = oracle.block_minmax(k, [0, 129, 128])
    assert np.isnan(kmin[:2]).all() and np.isnan(kmax[:2]).all()
    assert not np.isnan(kmin[2]).any()


def test_score_worked_example():
    # q = (1, -2), box [0, 3] x [-1, 1]: channel 0 is positive and takes 3 * 1,
    # channel 1 is negative and takes (-2) * (-1); the corner (3, -1) gives 3 + 2 = 5
    s = oracle.block_scores(np.array([1.0, -2.0]), np.array([[0.0, -1.0]]), np.array([[3.0, 1.0]]))
    assert s.shape == (1,) and s[0] == 5.0


def test_score_is_the_maximum_over_the_box_corners():
    rng = np.random.default_rng(3)
    D = 6
    for _ in range(20):
        q = rng.standard_normal(D)
        a, c = rng.standard_normal((2, 5, D))
        lo, hi = np.minimum(a, c), np.maximum(a, c)
        s = oracle.block_scores(q, lo, hi)
        for j in range(5):
            corners = np.array(list(itertools.product(*zip(lo[j], hi[j]))))  # 2^D corners
            assert abs(s[j] - (corners @ q).max()) < 1e-12


def test_score_bounds_every_key_and_is_tight_on_a_constant_block():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((1, 2, 256, 16))
    k[0, 1, 64:128] = k[0, 1, 70]  # block 1 of head 1: one key repeated
    kmin, kmax = oracle.block_minmax(k, [256])
    q = rng.standard_normal((1, 2, 16))
    s = oracle.block_scores(q, kmin, kmax)  # [1, 2, 4]
    for h in range(2):
        for j in range(4):
            dots = k[0, h, j * BLOCK:(j + 1) * BLOCK] @ q[0, h]
            assert (dots <= s[0, h, j] + 1e-12).all()
    assert abs(s[0, 1, 1] - k[0, 1, 70] @ q[0, 1]) < 1e-12


def _rank_selected(sc, budget):
    """Blocks j < i whose rank (higher score first, equal scores lower j first) is below budget - 1."""
    i = len(sc)
    out = []
    for j in range(i):
        rank = sum(1 for x in range(i) if sc[x] > sc[j]) + sum(1 for x in range(j) if sc[x] == sc[j])
        if rank < budget - 1:
            out.append(j)
    return out


@pytest.mark.parametrize("budget", [1, 2, 5, 9])
def test_select_follows_the_rank_definition(budget):
    rng = np.random.default_rng(5 + budget)
    lens = [1, 64, 65, 300, 511, 512]
    B, H, D = len(lens), 3, 8
    k = _keys(6, B, H, 512, D, lens)
    kmin, kmax = oracle.block_minmax(k, lens)
    q = rng.standard_normal((B, H, D))
    rp, ci = oracle.select_blocks(q, kmin, kmax, lens, budget)
    assert rp[0] == 0 and (np.diff(rp) >= 0).all() and rp[-1] == len(ci)
    for b, n in enumerate(lens):
        i = (n - 1) // BLOCK
        for h in range(H):
            row = list(ci[rp[b * H + h]:rp[b * H + h + 1]])
            if i + 1 <= budget:
                assert row == list(range(i + 1))
                continue
            sc = oracle.block_scores(q[b, h], kmin[b, h, :i], kmax[b, h, :i])
            assert row == _rank_selected(sc, budget) + [i]


def test_select_is_the_best_subset():
    # exhaustive search: with distinct scores, the chosen budget - 1 earlier blocks
    # are the subset with the largest total score
    rng = np.random.default_rng(7)
    D = 4
    for trial in range(10):
        n = 64 * 9 - trial  # i = 8: blocks 0 .. 7 compete
        k = rng.standard_normal((1, 1, n, D))
        kmin, kmax = oracle.block_minmax(k, [n])
        q = rng.standard_normal((1, 1, D))
        sc = oracle.block_scores(q[0, 0], kmin[0, 0, :8], kmax[0, 0, :8])
        for budget in (2, 4, 7):
            rp, ci = oracle.select_blocks(q, kmin, kmax, [n], budget)
            best = max(itertools.combinations(range(8), budget - 1), key=lambda c: sc[list(c)].sum())
            assert list(ci) == sorted(best) + [8]


def test_select_ties_go_to_the_lower_block():
    D = 4
    kmin = np.zeros((1, 1, 6, D))
    kmax = np.ones((1, 1, 6, D))
    kmax[0, 0, 4] = 2.0  # block 4 scores highest, blocks 0 .. 3 tie
    q = np.ones((1, 1, D))
    rp, ci = oracle.select_blocks(q, kmin, kmax, [6 * 64], 4)
    assert list(ci) == [0, 1, 4, 5]


def test_select_invalid_lengths_give_empty_rows():
    kmin = np.zeros((3, 2, 2, 4))
    kmax = np.ones((3, 2, 2, 4))
    rp, ci = oracle.select_blocks(np.ones((3, 2, 4)), kmin, kmax, [0, 129, 100], 1)
    assert list(rp) == [0, 0, 0, 0, 0, 1, 2] and list(ci) == [1, 1]


def test_decode_rows_with_every_block_is_dense_decode():
    rng = np.random.default_rng(8)
    lens = [300, 1, 129]
    B, H, D, L = 3, 2, 8, 320
    k = rng.standard_normal((B, H, L, D))
    v = rng.standard_normal((B, H, L, D))
    q = rng.standard_normal((B, H, D))
    kmin, kmax = oracle.block_minmax(k, lens)
    rp, ci = oracle.select_blocks(q, kmin, kmax, lens, 100)
    o, lse = oracle.attn_decode_rows(q, oracle.dense_kv_blocks(k, v), lens, rp, ci)
    for b, n in enumerate(lens):
        for h in range(H):
            s = k[b, h, :n] @ q[b, h] / np.sqrt(D)
            p = np.exp(s - s.max())
            assert np.abs(o[b, h] - (p / p.sum()) @ v[b, h, :n]).max() < 1e-12
            assert abs(lse[b, h] - (s.max() + np.log(p.sum()))) < 1e-12


def test_decode_rows_copied_from_a_static_layout_match_attn_decode():
    rng = np.random.default_rng(9)
    H, nqb, D = 4, 6, 8
    lens = [384, 200, 65]
    rp_s, ci_s = oracle.build_layout(H, nqb, 2, 3, [False, True, False, False])
    k = rng.standard_normal((3, H, nqb * BLOCK, D))
    v = rng.standard_normal((3, H, nqb * BLOCK, D))
    q = rng.standard_normal((3, H, D))
    rows = []
    for b, n in enumerate(lens):
        for h in range(H):
            rows.append(oracle.row_blocks(rp_s, ci_s, nqb, h, (n - 1) // BLOCK))
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    kv = oracle.dense_kv_blocks(k, v)
    o1, l1 = oracle.attn_decode_rows(q, kv, lens, rp, ci)
    o2, l2 = oracle.attn_decode(q, kv, lens, rp_s, ci_s, nqb)
    assert np.abs(o1 - o2).max() == 0 and np.abs(l1 - l2).max() == 0


def _paged(k, P, rng):
    """Scatter a contiguous cache [B, Hkv, L, D] into shuffled pages of P tokens."""
    B, Hkv, L, D = k.shape
    npb = -(-L // P)
    perm = rng.permutation(B * npb + 3)[:B * npb]  # a few pages stay unused
    pages = np.full((B * npb + 3, Hkv, P, D), np.nan)
    table = perm.reshape(B, npb).astype(np.int32)
    for b in range(B):
        for s in range(npb):
            rows = k[b, :, s * P:(s + 1) * P]
            pages[table[b, s], :, :rows.shape[1]] = rows
    return pages, table


@pytest.mark.parametrize("P", [16, 64])
def test_paged_bounds_equal_contiguous_bounds(P):
    rng = np.random.default_rng(20 + P)
    B, Hkv, L, D = 3, 2, 320, 8
    k = rng.standard_normal((B, Hkv, L, D))
    lens = [320, 100, 1]
    pages, table = _paged(k, P, rng)
    km, kx = oracle.block_minmax_paged(pages, table, P, lens, L // BLOCK)
    cm, cx = oracle.block_minmax(k, lens)
    assert np.array_equal(np.isnan(km), np.isnan(cm))
    ok = ~np.isnan(cm)
    assert np.array_equal(km[ok], cm[ok]) and np.array_equal(kx[ok], cx[ok])
    # a length past the table's reach gives no bounds
    km, _ = oracle.block_minmax_paged(pages, table, P, [320, L + 1, 0], L // BLOCK)
    assert np.isnan(km[1:]).all() and not np.isnan(km[0, :, :5]).any()


def test_grouped_selection_equals_repeated_heads():
    rng = np.random.default_rng(24)
    B, Hkv, g, L, D = 2, 2, 4, 1024, 8
    k = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hkv * g, D))
    lens = [1024, 700]
    km, kx = oracle.block_minmax(k, lens)
    rp, ci = oracle.select_blocks(q, km, kx, lens, 5, group=g)
    rp2, ci2 = oracle.select_blocks(q, np.repeat(km, g, axis=1), np.repeat(kx, g, axis=1), lens, 5)
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
    # query heads of one group rank the same bounds with their own queries: lists differ
    rows = [tuple(ci[rp[r]:rp[r + 1]]) for r in range(B * Hkv * g)]
    assert len(set(rows[:g])) > 1


def test_paged_grouped_decode_rows_equal_repeated_contiguous():
    rng = np.random.default_rng(25)
    B, Hkv, g, L, D, P = 2, 2, 2, 512, 8, 16
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hkv * g, D))
    lens = [512, 333]
    kp, table = _paged(k, P, rng)
    vp = np.full_like(kp, np.nan)
    for b in range(B):
        for s in range(L // P):
            vp[table[b, s]] = v[b, :, s * P:(s + 1) * P].transpose(0, 1, 2)
    km, kx = oracle.block_minmax_paged(kp, table, P, lens, L // BLOCK)
    rp, ci = oracle.select_blocks(q, km, kx, lens, 4, group=g)
    o1, l1 = oracle.attn_decode_rows(q, oracle.paged_kv_blocks(kp, vp, table, P, g), lens, rp, ci)
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    o2, l2 = oracle.attn_decode_rows(q, oracle.dense_kv_blocks(kr, vr), lens, rp, ci)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12
