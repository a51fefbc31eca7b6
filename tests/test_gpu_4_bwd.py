"""GPU backward kernels (bf16 MFMA) against the fp64 oracle.

Tolerance: the gradients are compared on the scale of the reference tensor,
max-abs error <= 2e-2 * max|ref| and mean-abs error <= 2e-3 * max|ref| (the
forward's bf16 bounds, which are stated for outputs of unit scale, applied
relative to each gradient's own scale; the derivation is in the design notes).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import LazyF64, device, f64

pytestmark = pytest.mark.gpu

GRAD_MAX_REL, GRAD_MEAN_REL = 2e-2, 2e-3


def assert_grad_close(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape
    keep = np.isfinite(want)
    assert keep.any()
    g, w = got[keep], want[keep]
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the GPU result"
    scale = float(np.abs(w).max())
    err = np.abs(g - w)
    print(f"  {what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} (max|ref| {scale:.3e})", flush=True)
    assert err.max() <= GRAD_MAX_REL * scale, f"{what}: max-abs {err.max():.3e} > {GRAD_MAX_REL} * {scale:.3e}"
    assert err.mean() <= GRAD_MEAN_REL * scale, f"{what}: mean-abs {err.mean():.3e} > {GRAD_MEAN_REL} * {scale:.3e}"


def _inputs(seed, B, H, N, D):
    q, k, v, do = synth.fwd_inputs(seed, B, H, N, D, "bf16",
                                   which=(synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V, synth.TENSOR_DO))
    return q, k, v, do


def _gpu_bwd(q, k, v, do, H, N, W, S, dense, sm_scale=0.0):
    import head_heterogeneous_block_amd as s2
    dev = device()
    pat = s2.Pattern(H, W, S, tuple(dense))
    lay = s2.s2_build_layout(pat, N // 64, dev)
    lt = s2.s2_build_layout_t(pat, N // 64, dev)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = s2.s2_attn_fwd(qd, kd, vd, lay, sm_scale=sm_scale)
    dq, dk, dv = s2.s2_attn_bwd(qd, kd, vd, o, dod, lse, lay, lt, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    # B, H, N, D, W, S, dense
    (1, 2, 256, 128, 2, 4, ()),
    (2, 4, 512, 128, 2, 4, (1,)),       # a dense head
    (1, 3, 448, 128, 3, 5, ()),         # odd number of blocks: ragged query and key pairs
    (1, 4, 512, 64, 4, 8, (0,)),        # D = 64
    (1, 2, 64, 128, 1, 1, ()),          # a single block
    (1, 2, 1024, 128, 1, 1, ()),        # stride 1: dense causal
    (2, 5, 960, 128, 3, 7, (4,)),       # 15 blocks, several tiles and a ragged tail
    (1, 3, 576, 64, 2, 3, ()),
]


@pytest.mark.parametrize("B,H,N,D,W,S,dense", CASES)
def test_bwd_small_cases(B, H, N, D, W, S, dense):
    print(f"bwd bf16 B={B} H={H} N={N} D={D} W={W} S={S} dense={dense}", flush=True)
    q, k, v, do = _inputs(17, B, H, N, D)
    dq, dk, dv = _gpu_bwd(q, k, v, do, H, N, W, S, dense)
    rp, ci = oracle.build_layout(H, N // 64, W, S, synth.dense_flags(H, dense))
    rq, rk, rv = oracle.attn_bwd_dense(f64(q), f64(k), f64(v), f64(do), rp, ci, N // 64)
    assert_grad_close(f64(dq), rq, "dq")
    assert_grad_close(f64(dk), rk, "dk")
    assert_grad_close(f64(dv), rv, "dv")


def test_bwd_custom_scale():
    B, H, N, D = 1, 2, 384, 128
    print("bwd bf16 custom scale 0.3", flush=True)
    q, k, v, do = _inputs(18, B, H, N, D)
    dq, dk, dv = _gpu_bwd(q, k, v, do, H, N, 2, 3, (), sm_scale=0.3)
    rp, ci = oracle.build_layout(H, N // 64, 2, 3)
    rq, rk, rv = oracle.attn_bwd_dense(f64(q), f64(k), f64(v), f64(do), rp, ci, N // 64, scale=0.3)
    assert_grad_close(f64(dq), rq, "dq")
    assert_grad_close(f64(dk), rk, "dk")
    assert_grad_close(f64(dv), rv, "dv")


def test_bwd_constant_v_and_sums():
    # V constant: the output does not depend on Q or K, so dQ = dK = 0; and at
    # any V the value-gradient rows of a (b, h) sum to the output-gradient rows
    B, H, N, D = 1, 4, 1024, 128
    print("bwd bf16 properties", flush=True)
    q, k, _, do = _inputs(19, B, H, N, D)
    v = torch.full_like(q, 0.5)
    dq, dk, dv = _gpu_bwd(q, k, v, do, H, N, 3, 4, (2,))
    assert float(dq.float().abs().max()) < 1e-2 and float(dk.float().abs().max()) < 1e-2
    colsum = dv.float().sum(dim=2).cpu().numpy()
    ref = do.float().sum(dim=2).numpy()
    assert np.max(np.abs(colsum - ref)) <= 2e-2 * np.abs(ref).max() + 0.05


def test_bwd_full_size_sampled():
    # the 1.3B-shaped workload at full size; the oracle computes two (b, h) slices
    c = synth.WORKLOADS[2]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    print("bwd bf16 1.3B-shaped full size, sampled", flush=True)
    q, k, v, do = _inputs(2, B, H, N, D)
    dq, dk, dv = _gpu_bwd(q, k, v, do, H, N, c["W"], c["S"], c["dense"])
    rp, ci = oracle.build_layout(H, N // 64, c["W"], c["S"], synth.dense_flags(H, c["dense"]))
    pairs = [(3, 1), (1, 6)]  # a dense head and a sparse one
    rq, rk, rv = oracle.attn_bwd_dense(LazyF64(q), LazyF64(k), LazyF64(v), LazyF64(do), rp, ci, N // 64,
                                       pairs=pairs)
    for b, h in pairs:
        assert_grad_close(f64(dq[b, h]), rq[b, h], f"dq[{b},{h}]")
        assert_grad_close(f64(dk[b, h]), rk[b, h], f"dk[{b},{h}]")
        assert_grad_close(f64(dv[b, h]), rv[b, h], f"dv[{b},{h}]")
