"""Seeded random shapes and patterns (forward, decode, backward) against the fp64
oracle: the number of query blocks, heads, batch, head dim, window, stride and
dense heads drawn at random, so that pairs of rows, ragged group ends, windows
wider than the sequence, strides of 1 and all-dense or all-sparse heads meet
in combinations the fixed cases do not list."""
import numpy as np
import pytest
import torch

import oracle
import synth
import test_gpu_2_fwd as F
import test_gpu_3_decode as Dd
import test_gpu_4_bwd as Bw
from gpu_common import assert_lse_close, assert_out_close, f64

pytestmark = pytest.mark.gpu


def _draw(seed, n, max_nqb):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(rng.integers(1, 6))
        dense = tuple(int(h) for h in range(H) if rng.random() < 0.25)
        out.append(dict(B=int(rng.integers(1, 3)), H=H, nqb=int(rng.integers(1, max_nqb + 1)),
                        D=int(rng.choice([64, 128])), W=int(rng.integers(1, 7)), S=int(rng.integers(1, 10)),
                        dense=dense, seed=int(rng.integers(1 << 30))))
    return out


FWD = _draw(9101, 24, 24)
DEC = _draw(9102, 12, 20)
BWD = _draw(9103, 8, 12)


def _ids(cases):
    return [f"B{c['B']}H{c['H']}n{c['nqb']}D{c['D']}W{c['W']}S{c['S']}d{''.join(map(str, c['dense']))}" for c in cases]


@pytest.mark.parametrize("pipelined", [False, True])
@pytest.mark.parametrize("c", FWD, ids=_ids(FWD))
def test_random_forward(c, pipelined, monkeypatch):
    monkeypatch.setenv("S2ATTN_FWD_PIPELINED", "1" if pipelined else "0")
    B, H, D, N = c["B"], c["H"], c["D"], 64 * c["nqb"]
    dtype = "f32" if c["seed"] % 5 == 0 else "bf16"
    print(f"random fwd {dtype} pipelined={pipelined} {c}", flush=True)
    q, k, v = synth.fwd_inputs(c["seed"] % 100000, B, H, N, D, dtype)
    o, lse, _ = F._run(q, k, v, H, N, c["W"], c["S"], c["dense"])
    rp, ci = oracle.build_layout(H, c["nqb"], c["W"], c["S"], synth.dense_flags(H, c["dense"]))
    oo, ol = oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, c["nqb"])
    assert_out_close(f64(o), oo, dtype)
    assert_lse_close(f64(lse), ol, dtype)


@pytest.mark.parametrize("c", DEC, ids=_ids(DEC))
def test_random_decode(c):
    rng = np.random.default_rng(c["seed"])
    L = 64 * c["nqb"] - int(rng.integers(0, 64))
    lens = [int(x) for x in rng.integers(1, L + 1, size=c["B"])]
    lens[0] = L if c["B"] > 1 else lens[0]
    splits = int(rng.choice([0, 1, 2, 5]))
    o, lse, oo, ol = Dd._small("bf16", c["B"], c["H"], c["D"], L, c["W"], c["S"], c["dense"], lens, splits)
    assert_out_close(f64(o), oo, "bf16")
    assert_lse_close(f64(lse), ol, "bf16")


@pytest.mark.parametrize("c", BWD, ids=_ids(BWD))
def test_random_backward(c):
    B, H, D, N = c["B"], c["H"], c["D"], 64 * c["nqb"]
    print(f"random bwd {c}", flush=True)
    q, k, v, do = Bw._inputs(c["seed"] % 100000, B, H, N, D)
    dq, dk, dv = Bw._gpu_bwd(q, k, v, do, H, N, c["W"], c["S"], c["dense"])
    rp, ci = oracle.build_layout(H, c["nqb"], c["W"], c["S"], synth.dense_flags(H, c["dense"]))
    rq, rk, rv = oracle.attn_bwd_dense(f64(q), f64(k), f64(v), f64(do), rp, ci, c["nqb"])
    Bw.assert_grad_close(f64(dq), rq, "dq")
    Bw.assert_grad_close(f64(dk), rk, "dk")
    Bw.assert_grad_close(f64(dv), rv, "dv")


PAGED = _draw(9104, 10, 16)


@pytest.mark.parametrize("c", PAGED, ids=_ids(PAGED))
def test_random_paged_decode(c):
    import test_gpu_5_paged as Pg
    rng = np.random.default_rng(c["seed"])
    group = int(rng.choice([1, 2, 3, 4, 8]))
    Hkv = int(rng.integers(1, 4))
    H = Hkv * group
    dense = tuple(h for h in c["dense"] if h < H)
    P = int(rng.choice([16, 32, 64, 128]))
    # the tables' capacity (whole pages) must lie within the layout: a cache of
    # whole pages, the sequences ragged inside it
    L = max(1, 64 * c["nqb"] // P) * P
    B = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(1, L + 1, size=B)]
    splits = int(rng.choice([0, 1, 2, 3]))
    o, lse, oo, ol, _ = Pg._case("bf16", B, H, Hkv, c["D"], L, c["W"], c["S"], dense, lens, P, splits,
                                 seed=c["seed"] % 1000)
    assert_out_close(f64(o), oo, "bf16")
    assert_lse_close(f64(lse), ol, "bf16")


VARLEN = _draw(9105, 8, 12)


@pytest.mark.parametrize("pipelined", [False, True])
@pytest.mark.parametrize("c", VARLEN, ids=_ids(VARLEN))
def test_random_varlen(c, pipelined, monkeypatch):
    import test_gpu_7_varlen as V
    monkeypatch.setenv("S2ATTN_FWD_PIPELINED", "1" if pipelined else "0")
    rng = np.random.default_rng(c["seed"])
    lens = [int(x) for x in rng.integers(1, 64 * c["nqb"] + 1, size=int(rng.integers(1, 6)))]
    cu, q, k, v, rp, ci, nqb, o, lse = V._run(lens, H=c["H"], D=c["D"], W=c["W"], S=c["S"], dense=c["dense"],
                                              seed=c["seed"] % 1000)
    oo, ol = oracle.attn_fwd_varlen(f64(q), f64(k), f64(v), cu, rp, ci, nqb)
    assert_out_close(o, oo, "bf16")
    assert_lse_close(lse, ol, "bf16")
