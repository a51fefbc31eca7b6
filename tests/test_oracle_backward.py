"""Pins of the oracle's backward pass and column layout (CPU only).

The gradients are checked against things the oracle's own formulas do not
produce: central finite differences of the (separately pinned) forward oracle,
torch.autograd in float64 on the all-blocks layout (dense causal attention),
and exact invariants of softmax attention: the key-gradient rows of one
(b, h) sum to zero, the value-gradient rows sum to the sum of the output
gradient rows, a constant V has zero query and key gradients, and blocks no
query row uses get zero key and value gradients.  The column layout is
checked against a brute-force block mask and by a double transpose.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _block_mask(rp, ci, H, nqb):
    m = np.zeros((H, nqb, nqb), dtype=bool)
    for h in range(H):
        for i in range(nqb):
            m[h, i, oracle.row_blocks(rp, ci, nqb, h, i)] = True
    return m


@pytest.mark.parametrize("H,nqb,W,S,dense", [(4, 8, 2, 4, None), (5, 15, 3, 7, [0, 0, 1, 0, 0]),
                                             (3, 1, 1, 1, None), (2, 33, 4, 8, [1, 0])])
def test_transpose_matches_block_mask(H, nqb, W, S, dense):
    rp, ci = oracle.build_layout(H, nqb, W, S, dense)
    cp, ri = oracle.transpose_layout(rp, ci, H, nqb)
    assert cp.dtype == np.int32 and ri.dtype == np.int32
    assert cp[-1] == len(ci) == len(ri)
    m = _block_mask(rp, ci, H, nqb)
    for h in range(H):
        for j in range(nqb):
            r = h * nqb + j
            col = ri[cp[r]:cp[r + 1]]
            assert list(col) == list(np.nonzero(m[h, :, j])[0])   # ascending, exact set
    # transposing the column view again gives the original rows
    rp2, ci2 = oracle.transpose_layout(cp, ri, H, nqb)
    assert np.array_equal(rp2, rp) and np.array_equal(ci2, ci)


def _loss(q, k, v, do, rp, ci, nqb):
    o, _ = oracle.attn_fwd_dense(q, k, v, rp, ci, nqb)
    return float((o * do).sum())


def test_gradients_match_finite_differences():
    B, H, N, D = 1, 3, 192, 8
    nqb = N // 64
    rp, ci = oracle.build_layout(H, nqb, 1, 2, [0, 1, 0])   # sparse heads and one dense head
    q, k, v, do = (_rand((B, H, N, D), s) for s in (11, 12, 13, 14))
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, rp, ci, nqb)
    rng = np.random.default_rng(5)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = (0, rng.integers(H), rng.integers(N), rng.integers(D))
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            lp = _loss(*[xp if n == name else args[n] for n in ("q", "k", "v")], do, rp, ci, nqb)
            lm = _loss(*[xm if n == name else args[n] for n in ("q", "k", "v")], do, rp, ci, nqb)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def test_all_blocks_equals_autograd_causal():
    B, H, N, D = 2, 2, 256, 32
    q, k, v, do = (_rand((B, H, N, D), s) for s in (21, 22, 23, 24))
    rp, ci = oracle.build_layout(H, N // 64, 1, 1, None)   # stride 1: every causal block
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, rp, ci, N // 64)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    s = tq @ tk.transpose(-1, -2) / math.sqrt(D)
    causal = torch.ones(N, N, dtype=torch.bool).tril()
    o = torch.softmax(s.masked_fill(~causal, float("-inf")), dim=-1) @ tv
    o.backward(torch.from_numpy(do))
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(ours - ref.numpy())) < 1e-11


def test_gradient_invariants():
    B, H, N, D = 2, 5, 320, 16
    nqb = N // 64
    rp, ci = oracle.build_layout(H, nqb, 2, 3, [1, 0, 0, 0, 0])
    q, k, v, do = (_rand((B, H, N, D), s) for s in (31, 32, 33, 34))
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, rp, ci, nqb)
    # every query row's softmax sums to one: the key gradients of a (b, h)
    # sum to zero, and the value gradients sum to the output gradients
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-10
    assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) < 1e-10
    # a constant V makes the output independent of Q and K
    vc = np.full_like(v, 0.75)
    dq0, dk0, _ = oracle.attn_bwd_dense(q, k, vc, do, rp, ci, nqb)
    assert np.max(np.abs(dq0)) < 1e-12 and np.max(np.abs(dk0)) < 1e-12


def test_unused_blocks_get_no_gradient():
    # a hand-made single-head CSR in which no row holds key block 1 (rows need
    # not contain their diagonal block): rows 0..3 = [0], [0], [0, 2], [2, 3]
    B, H, N, D = 1, 1, 256, 16
    nqb = N // 64
    rp = np.array([0, 1, 2, 4, 6], dtype=np.int32)
    ci = np.array([0, 0, 0, 2, 2, 3], dtype=np.int32)
    q, k, v, do = (_rand((B, H, N, D), s) for s in (41, 42, 43, 44))
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, rp, ci, nqb)
    assert not dk[:, :, 64:128].any() and not dv[:, :, 64:128].any()
    assert dk[:, :, 128:192].any() and dv[:, :, 192:256].any()
    # changing K/V of key block 2 leaves the query blocks that do not hold it unchanged
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 128:192] += 1.0
    v2[:, :, 128:192] -= 2.0
    dq2, _, _ = oracle.attn_bwd_dense(q, k2, v2, do, rp, ci, nqb)
    assert np.array_equal(dq[:, :, :128], dq2[:, :, :128])
    assert not np.array_equal(dq[:, :, 128:], dq2[:, :, 128:])
