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
