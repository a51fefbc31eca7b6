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
