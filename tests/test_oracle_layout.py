"""Pins of the oracle's layout builder (CPU only).

The oracle builds each row as a set union (window set | strided residue set).
It is pinned against: a hand-worked fixture, a per-block brute-force predicate,
a closed-form row count derived by counting, the coverage invariant stated by
the S2-Attention pages (heads together cover the whole context), and the
structural invariants of a causal CSR.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_tiny.txt")


def _pattern(w):
    c = synth.WORKLOADS[w]
    return c["H"], c["N"] // 64, c["W"], c["S"], synth.dense_flags(c["H"], c["dense"])


def _closed_form_count(h, i, W, S, dense):
    """Row length by counting: window min(W, i+1) plus strided blocks strictly left of it."""
    if dense:
        return i + 1
    rho = (-h) % S                 # first block index of head h's residue class
    m = i - W                      # strided blocks must lie in [0, i - W] to be outside the window
    extra = 0 if m < rho else (m - rho) // S + 1
    return min(W, i + 1) + extra


def _brute_force_row(h, i, W, S, dense):
    return [j for j in range(i + 1) if dense or (i - j) < W or (j + h) % S == 0]


def test_golden_tiny_layout():
    H, nqb, W, S, dense = _pattern(1)
    row_ptr, col_idx = oracle.build_layout(H, nqb, W, S, dense)
    seen = 0
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            head, rest = line.split(":")
            h, i = (int(x) for x in head.split())
            want = [int(x) for x in rest.split()]
            got = oracle.row_blocks(row_ptr, col_idx, nqb, h, i).tolist()
            assert got == want, (h, i, got, want)
            seen += 1
    assert seen == H * nqb
    assert row_ptr[-1] == 81


@pytest.mark.parametrize("H,nqb,W,S,dense", [
    (4, 8, 2, 4, [0, 0, 0, 0]),
    (5, 37, 3, 7, [0, 1, 0, 0, 1]),
    (8, 64, 1, 1, [0] * 8),
    (3, 50, 60, 5, [0, 0, 0]),
    (6, 40, 4, 9, [0] * 6),
])
def test_brute_force_and_closed_form(H, nqb, W, S, dense):
    row_ptr, col_idx = oracle.build_layout(H, nqb, W, S, dense)
    for h in range(H):
        for i in range(nqb):
            got = oracle.row_blocks(row_ptr, col_idx, nqb, h, i).tolist()
            assert got == _brute_force_row(h, i, W, S, dense[h])
            assert len(got) == _closed_form_count(h, i, W, S, dense[h])


# nnz per batch of each workload, by the closed-form count summed over rows.
EXPECTED_NNZ = {1: 81, 2: 37157, 3: 384696, 4: 11115950, 5: 384696}


@pytest.mark.parametrize("w", [1, 2, 3, 4, 5])
def test_workload_layouts(w):
    H, nqb, W, S, dense = _pattern(w)
    row_ptr, col_idx = oracle.build_layout(H, nqb, W, S, dense)
    assert row_ptr.dtype == np.int32 and col_idx.dtype == np.int32
    assert row_ptr.shape == (H * nqb + 1,) and row_ptr[0] == 0
    assert int(row_ptr[-1]) == EXPECTED_NNZ[w] == col_idx.shape[0]
    lens = np.diff(row_ptr)
    want = np.array([_closed_form_count(h, i, W, S, dense[h]) for h in range(H) for i in range(nqb)])
    assert np.array_equal(lens, want)
    # every row ends on its diagonal block and is strictly ascending
    i_of_row = np.tile(np.arange(nqb), H)
    assert np.array_equal(col_idx[row_ptr[1:] - 1], i_of_row)
    d = np.diff(col_idx)
    starts = set(row_ptr[1:-1].tolist())
    inner = np.array([k + 1 not in starts for k in range(len(d))], dtype=bool)
    assert np.all(d[inner] > 0)
    assert col_idx.min() >= 0


@pytest.mark.parametrize("w", [1, 2, 3, 4, 5])
def test_heads_cover_context(w):
    """Heads together cover every causal key block of every query block."""
    H, nqb, W, S, dense = _pattern(w)
    row_ptr, col_idx = oracle.build_layout(H, nqb, W, S, dense)
    covered = np.zeros((nqb, nqb), dtype=bool)
    for h in range(H):
        for i in range(nqb):
            covered[i, oracle.row_blocks(row_ptr, col_idx, nqb, h, i)] = True
    assert np.array_equal(covered, np.tril(np.ones((nqb, nqb), dtype=bool)))


def test_128k_sparse_heads_alone_miss_residues():
    """Without its 4 dense heads the 128K pattern leaves residues {0, 29, 30, 31} uncovered."""
    H, nqb, W, S, _ = _pattern(4)
    covered = set()
    for h in range(4, H):
        covered |= {(-h) % S}
    assert set(range(S)) - covered == {0, 29, 30, 31}
    i = nqb - 1
    union = set()
    for h in range(4, H):
        union |= set(oracle.active_blocks(h, i, W, S, False))
    missing = set(range(i + 1)) - union
    assert missing and all(j % S in {0, 29, 30, 31} for j in missing)


def test_decode_row_lengths():
    """Decode at position 32767 reads row i=511: 40 blocks for h mod 16 in {0, 9..15}, else 39."""
    H, nqb, W, S, dense = _pattern(5)
    row_ptr, col_idx = oracle.build_layout(H, nqb, W, S, dense)
    for h in range(H):
        n = len(oracle.row_blocks(row_ptr, col_idx, nqb, h, nqb - 1))
        assert n == (40 if (h % 16 == 0 or h % 16 >= 9) else 39)


def test_planted_window_off_by_one_is_caught(monkeypatch):
    """A window read as 'diagonal plus W previous blocks' must fail the fixture."""
    def wrong(h, i, W, S, dense):
        if dense:
            return list(range(i + 1))
        return sorted(set(range(max(0, i - W), i + 1)) | set(range((-h) % S, i + 1, S)))
    monkeypatch.setattr(oracle.s2_oracle, "active_blocks", wrong)
    with pytest.raises(AssertionError):
        test_golden_tiny_layout()


def test_planted_stride_sign_is_caught(monkeypatch):
    """Strided blocks anchored at (j - h) instead of (j + h) must fail the fixture."""
    def wrong(h, i, W, S, dense):
        if dense:
            return list(range(i + 1))
        return sorted(set(range(max(0, i - W + 1), i + 1)) | set(range(h % S, i + 1, S)))
    monkeypatch.setattr(oracle.s2_oracle, "active_blocks", wrong)
    with pytest.raises(AssertionError):
        test_golden_tiny_layout()
