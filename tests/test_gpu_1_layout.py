"""GPU layout builder: bit-exact against the oracle's set construction."""
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import device

pytestmark = pytest.mark.gpu


def _check(H, nqb, W, S, dense_heads):
    import head_heterogeneous_block_amd as s2
    dev = device()
    print(f"layout H={H} nqb={nqb} W={W} S={S} dense={dense_heads}", flush=True)
    lay = s2.s2_build_layout(s2.Pattern(H, W, S, tuple(dense_heads)), nqb, dev)
    torch.cuda.synchronize()
    rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, dense_heads))
    got_rp = lay.row_ptr.cpu().numpy()
    got_ci = lay.col_idx[:lay.nnz].cpu().numpy()
    assert lay.nnz == int(rp[-1])
    assert got_rp.dtype == np.int32 and got_ci.dtype == np.int32
    assert np.array_equal(got_rp, rp)
    assert np.array_equal(got_ci, ci)
    # the column view: bit-exact against the transpose of the oracle's rows
    lt = s2.s2_build_layout_t(s2.Pattern(H, W, S, tuple(dense_heads)), nqb, dev)
    torch.cuda.synchronize()
    cp, ri = _transpose(rp, ci, H, nqb)
    assert lt.nnz == int(rp[-1])
    assert np.array_equal(lt.row_ptr.cpu().numpy(), cp)
    assert np.array_equal(lt.col_idx[:lt.nnz].cpu().numpy(), ri)


def _transpose(rp, ci, H, nqb):
    """Column view of a row CSR: the oracle's list-based transpose for small
    layouts; above a million entries a stable sort of the same entries by
    (head, key block), which keeps the query blocks ascending."""
    if len(ci) <= 1_000_000:
        return oracle.transpose_layout(rp, ci, H, nqb)
    rows = np.repeat(np.arange(H * nqb, dtype=np.int64), np.diff(rp))
    h, i = rows // nqb, rows % nqb
    key = h * nqb + ci.astype(np.int64)
    order = np.argsort(key, kind="stable")
    cp = np.zeros(H * nqb + 1, dtype=np.int32)
    cp[1:] = np.cumsum(np.bincount(key, minlength=H * nqb))
    return cp, i[order].astype(np.int32)


@pytest.mark.parametrize("w", [1, 2, 3, 4, 5])
def test_layout_workloads(w):
    c = synth.WORKLOADS[w]
    _check(c["H"], c["N"] // 64, c["W"], c["S"], c["dense"])


def test_layout_random_patterns():
    rng = random.Random(11)
    for _ in range(25):
        H = rng.randint(1, 40)
        nqb = rng.randint(1, 300)
        W = rng.randint(1, 20)
        S = rng.randint(1, 40)
        dense = [h for h in range(H) if rng.random() < 0.15]
        _check(H, nqb, W, S, dense)


def test_layout_edge_cases():
    _check(1, 1, 1, 1, [])          # one row, one block
    _check(3, 5, 100, 1000, [])     # window wider than the context
    _check(2, 64, 1, 1, [])         # stride 1: every block active
    _check(4, 33, 1, 7, [0, 1, 2, 3])  # all heads dense


@pytest.mark.parametrize("H,nqb,W,S,dense", [
    (1, 65535, 16, 32, (0,)),    # one dense head: nnz = 2,147,450,880, just under 2^31
    (16, 65536, 16, 32, ()),     # sixteen sparse heads of 4M tokens: nnz about 1.1e9
])
def test_layout_maximum_size(H, nqb, W, S, dense):
    """Layouts at the int32 CSR limit (nnz < 2^31, col_idx of up to 8.6 GB).
    Sampled rows of every head (the first, the last, random ones) are bit-exact
    against the oracle's set definition, including the row that ends at nnz;
    the column view's last columns of every head likewise (rows i >= j whose
    oracle row holds j).  Over the whole arrays: the row pointers ascend from 0
    to nnz, and the two views hold the same (row, column) pairs (equal sums of
    the block indices each one stores against the other's counts)."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    pat = s2.Pattern(H, W, S, tuple(dense))
    nnz = s2.s2_layout_nnz(pat, nqb)
    print(f"layout max H={H} nqb={nqb} W={W} S={S} dense={dense} nnz={nnz}", flush=True)
    assert nnz < 2 ** 31
    lay = s2.s2_build_layout(pat, nqb, dev)
    torch.cuda.synchronize()
    rp = lay.row_ptr.cpu().numpy().astype(np.int64)
    assert lay.nnz == nnz and rp[0] == 0 and rp[-1] == nnz and np.all(np.diff(rp) >= 1)
    rng = np.random.default_rng(2 ** 31 - 1)
    for h in range(H):
        rows = sorted({0, 1, nqb - 2, nqb - 1, *(int(x) for x in rng.integers(0, nqb, 6))})
        for i in rows:
            want = oracle.active_blocks(h, i, W, S, h in dense)
            r = h * nqb + i
            assert rp[r + 1] - rp[r] == len(want), (h, i)
            got = lay.col_idx[int(rp[r]):int(rp[r + 1])].cpu().numpy()
            assert np.array_equal(got, np.asarray(want, dtype=np.int32)), (h, i)
    # row view: sum over rows of the stored blocks, and of row index x row length
    ci_sum = sum(int(c.to(torch.int64).sum()) for c in lay.col_idx[:nnz].split(1 << 28))
    row_len = torch.from_numpy(np.diff(rp)).to(dev)
    i_of_row = torch.arange(H * nqb, device=dev, dtype=torch.int64) % nqb
    row_weighted = int((i_of_row * row_len).sum())
    del lay
    torch.cuda.empty_cache()

    lt = s2.s2_build_layout_t(pat, nqb, dev)
    torch.cuda.synchronize()
    cp = lt.row_ptr.cpu().numpy().astype(np.int64)
    assert lt.nnz == nnz and cp[0] == 0 and cp[-1] == nnz and np.all(np.diff(cp) >= 1)
    for h in range(H):
        for j in (nqb - 64, nqb - 33, nqb - 2, nqb - 1):
            want = [i for i in range(j, nqb) if j in set(oracle.active_blocks(h, i, W, S, h in dense))]
            c = h * nqb + j
            got = lt.col_idx[int(cp[c]):int(cp[c + 1])].cpu().numpy()
            assert np.array_equal(got, np.asarray(want, dtype=np.int32)), (h, j)
    # the same (row, column) pairs: sum of stored query blocks = sum of i x row
    # length, and sum of j x column length = sum of the row view's stored blocks
    ri_sum = sum(int(c.to(torch.int64).sum()) for c in lt.col_idx[:nnz].split(1 << 28))
    col_len = torch.from_numpy(np.diff(cp)).to(dev)
    col_weighted = int((i_of_row * col_len).sum())
    assert ri_sum == row_weighted
    assert col_weighted == ci_sum
