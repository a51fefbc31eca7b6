"""Pins of the oracle on caller-built layouts (any head-major CSR of causal blocks).

Caller-built layouts may hold empty rows and rows without their diagonal block.
A row with no key is given output 0 and logsumexp -inf (the limit of the empty
softmax sum); the pins check that both forward modes and decode agree on that,
that the other rows are untouched by it, and that the backward stays the exact
gradient (finite differences) on such layouts."""
import numpy as np
import pytest

import oracle

BLOCK = oracle.BLOCK


def random_layout(rng, H, nqb, density=0.3, empty_rows=(), drop_diag=()):
    """Random causal CSR; rows listed in empty_rows have no block, rows in drop_diag
    lack their diagonal block (and keep at least block 0)."""
    rp, ci = [0], []
    for h in range(H):
        for i in range(nqb):
            if (h, i) in empty_rows:
                cols = []
            else:
                cols = sorted(set(np.nonzero(rng.random(i + 1) < density)[0].tolist()) | {i})
                if (h, i) in drop_diag:
                    cols = [j for j in cols if j != i] or [0] if i > 0 else cols
            ci += cols
            rp.append(len(ci))
    return np.array(rp, dtype=np.int32), np.array(ci, dtype=np.int32)


def test_empty_rows_give_zero_and_minus_inf():
    rng = np.random.default_rng(1)
    H, nqb, D = 2, 5, 8
    N = nqb * BLOCK
    rp, ci = random_layout(rng, H, nqb, empty_rows={(0, 2), (1, 0), (1, 4)}, drop_diag={(0, 3)})
    q, k, v = (rng.standard_normal((1, H, N, D)) for _ in range(3))
    od, ld = oracle.attn_fwd_dense(q, k, v, rp, ci, nqb)
    ob, lb = oracle.attn_fwd_blocks(q, k, v, rp, ci, nqb)
    assert np.max(np.abs(od - ob)) < 1e-12 and np.array_equal(np.isinf(ld), np.isinf(lb))
    fin = np.isfinite(ld)
    assert np.max(np.abs(ld[fin] - lb[fin])) < 1e-12
    for h, i in ((0, 2), (1, 0), (1, 4)):
        rows = slice(i * BLOCK, (i + 1) * BLOCK)
        assert not od[0, h, rows].any() and np.all(ld[0, h, rows] == -np.inf)
    # every other row still attends to something: finite logsumexp
    assert fin.sum() == H * N - 3 * BLOCK
    # decode on an empty row: the same convention
    kv = oracle.dense_kv_blocks(k, v)
    o1, l1 = oracle.attn_decode(q[:, :, 0 + 2 * BLOCK], kv, [2 * BLOCK + 1], rp, ci, nqb)
    assert not o1[0, 0].any() and l1[0, 0] == -np.inf
    assert np.max(np.abs(o1[0, 1] - od[0, 1, 2 * BLOCK])) < 1e-12


def test_row_without_diagonal_has_no_token_mask():
    # keys of a block strictly before the query block are all visible
    rng = np.random.default_rng(2)
    H, nqb, D = 1, 3, 4
    rp = np.array([0, 1, 2, 3], dtype=np.int32)
    ci = np.array([0, 0, 1], dtype=np.int32)  # row 1 reads block 0 only, row 2 reads block 1 only
    q, k, v = (rng.standard_normal((1, H, nqb * BLOCK, D)) for _ in range(3))
    o, lse = oracle.attn_fwd_blocks(q, k, v, rp, ci, nqb)
    qv = q[0, 0, 2 * BLOCK + 5]
    s = k[0, 0, BLOCK:2 * BLOCK] @ qv / np.sqrt(D)
    p = np.exp(s - s.max())
    assert np.max(np.abs(o[0, 0, 2 * BLOCK + 5] - (p / p.sum()) @ v[0, 0, BLOCK:2 * BLOCK])) < 1e-12


def test_backward_finite_differences_on_user_layout():
    rng = np.random.default_rng(3)
    H, nqb, D = 2, 3, 4
    N = nqb * BLOCK
    rp, ci = random_layout(rng, H, nqb, density=0.5, empty_rows={(1, 1)}, drop_diag={(0, 2)})
    q, k, v, do = (rng.standard_normal((1, H, N, D)) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, rp, ci, nqb)

    def loss(q_, k_, v_):
        return float((oracle.attn_fwd_dense(q_, k_, v_, rp, ci, nqb)[0] * do).sum())
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 5, 1), (0, 1, 70, 2), (0, 1, N - 1, 3), (0, 0, 130, 0), (0, 1, 100, 0)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])
    # the empty row's queries get no gradient and pass none on
    assert not dq[0, 1, BLOCK:2 * BLOCK].any()


@pytest.mark.parametrize("seed,H,nqb", [(4, 3, 7), (5, 2, 40), (6, 1, 33)])
def test_transpose_of_random_layouts(seed, H, nqb):
    rng = np.random.default_rng(seed)
    rp, ci = random_layout(rng, H, nqb, density=0.2, empty_rows={(0, 1)})
    cp, ri = oracle.transpose_layout(rp, ci, H, nqb)
    m = np.zeros((H, nqb, nqb), dtype=bool)
    for h in range(H):
        for i in range(nqb):
            m[h, i, ci[rp[h * nqb + i]:rp[h * nqb + i + 1]]] = True
    for h in range(H):
        for j in range(nqb):
            assert list(ri[cp[h * nqb + j]:cp[h * nqb + j + 1]]) == list(np.nonzero(m[h, :, j])[0])
