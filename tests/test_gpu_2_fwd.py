"""GPU forward kernels (bf16 MFMA and fp32) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import LazyF64, assert_lse_close, assert_out_close, device, f64

pytestmark = pytest.mark.gpu


def _run(q, k, v, H, N, W, S, dense, **kw):
    import head_heterogeneous_block_amd as s2
    dev = device()
    lay = s2.s2_build_layout(s2.Pattern(H, W, S, tuple(dense)), N // 64, dev)
    o, lse = s2.s2_attn_fwd(q.to(dev), k.to(dev), v.to(dev), lay, **kw)
    torch.cuda.synchronize()
    return o, lse, lay


def _case(seed, B, H, N, D, dtype):
    return synth.fwd_inputs(seed, B, H, N, D, dtype)


def test_tiny_workload_f32_full():
    c = synth.WORKLOADS[1]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    print("fwd tiny f32 workload", flush=True)
    q, k, v = _case(1, B, H, N, D, "f32")
    o, lse, _ = _run(q, k, v, H, N, c["W"], c["S"], c["dense"])
    rp, ci = oracle.build_layout(H, N // 64, c["W"], c["S"], synth.dense_flags(H, c["dense"]))
    oo, ol = oracle.attn_fwd_dense(f64(q), f64(k), f64(v), rp, ci, N // 64)
    assert_out_close(f64(o), oo, "f32")
    assert_lse_close(f64(lse), ol, "f32")


SMALL = [
    # B, H, N, D, W, S, dense
    (2, 4, 512, 128, 2, 4, (1,)),
    (1, 3, 448, 128, 3, 5, ()),         # odd number of query blocks (ragged pair)
    (1, 4, 1024, 64, 4, 8, (0,)),       # D = 64
    (1, 2, 64, 128, 1, 1, ()),          # a single block
    (1, 2, 2048, 128, 1, 1, ()),        # stride 1: dense causal
    (2, 5, 960, 128, 3, 7, (4,)),       # 15 query blocks, several tiles and a ragged tail
    (1, 3, 576, 64, 2, 3, ()),
    (1, 80, 256, 64, 2, 3, (0, 79)),   # more than 64 heads: the queues keep head order
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,N,D,W,S,dense", SMALL)
def test_small_cases(dtype, B, H, N, D, W, S, dense):
    print(f"fwd {dtype} B={B} H={H} N={N} D={D} W={W} S={S} dense={dense}", flush=True)
    q, k, v = _case(7, B, H, N, D, dtype)
    o, lse, _ = _run(q, k, v, H, N, W, S, dense)
    rp, ci = oracle.build_layout(H, N // 64, W, S, synth.dense_flags(H, dense))
    oo, ol = oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, N // 64)
    assert_out_close(f64(o), oo, dtype)
    assert_lse_close(f64(lse), ol, dtype)


def test_custom_scale_and_no_lse():
    B, H, N, D = 1, 2, 256, 128
    q, k, v = _case(8, B, H, N, D, "bf16")
    o, lse, _ = _run(q, k, v, H, N, 2, 3, (), sm_scale=0.3, want_lse=False)
    assert lse is None
    rp, ci = oracle.build_layout(H, N // 64, 2, 3)
    oo, _ = oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, N // 64, scale=0.3)
    assert_out_close(f64(o), oo, "bf16")


def test_v_ones_gives_ones():
    B, H, N, D = 1, 4, 1024, 128
    q, k, _ = _case(9, B, H, N, D, "bf16")
    v = torch.ones_like(q)
    o, _, _ = _run(q, k, v, H, N, 3, 4, (2,))
    assert float((o.float() - 1).abs().max()) <= 2 ** -7


def test_strided_bshd_equals_contiguous():
    import head_heterogeneous_block_amd as s2
    B, H, N, D = 2, 4, 512, 128
    dev = device()
    q, k, v = (t.to(dev) for t in _case(10, B, H, N, D, "bf16"))
    lay = s2.s2_build_layout(s2.Pattern(H, 2, 4, (0,)), N // 64, dev)
    o1, l1 = s2.s2_attn_fwd(q, k, v, lay)
    # the same values stored as [B, N, H, D], passed as [B, H, N, D] views
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    assert not qs.is_contiguous()
    o2, l2 = s2.s2_attn_fwd(qs, ks, vs, lay, out=torch.empty_like(qs))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic():
    B, H, N, D = 2, 4, 1024, 128
    q, k, v = _case(11, B, H, N, D, "bf16")
    o1, l1, _ = _run(q, k, v, H, N, 4, 4, (1,))
    o2, l2, _ = _run(q, k, v, H, N, 4, 4, (1,))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_poisoned_block_only_reaches_rows_that_use_it(dtype):
    """NaN in one key block must reach exactly the query blocks whose CSR row lists it."""
    B, H, N, D, W, S = 1, 4, 1024, 128, 2, 4
    q, k, v = _case(12, B, H, N, D, dtype)
    clean, _, _ = _run(q, k, v, H, N, W, S, ())
    nqb = N // 64
    rp, ci = oracle.build_layout(H, nqb, W, S)
    for h, j in [(1, 3), (2, 6), (0, 0)]:
        kp, vp = k.clone(), v.clone()
        kp[0, h, j * 64:(j + 1) * 64] = float("nan")
        vp[0, h, j * 64:(j + 1) * 64] = float("nan")
        o, _, _ = _run(q, kp, vp, H, N, W, S, ())
        for hh in range(H):
            for i in range(nqb):
                rows = slice(i * 64, (i + 1) * 64)
                uses = hh == h and j in oracle.row_blocks(rp, ci, nqb, h, i)
                blk = o[0, hh, rows]
                if uses:
                    assert torch.isnan(blk).any(), (h, j, hh, i)
                else:
                    assert torch.equal(blk, clean[0, hh, rows]), (h, j, hh, i)


def _sampled_full(w):
    c = synth.WORKLOADS[w]
    B, H, N, D, W, S, dense = c["B"], c["H"], c["N"], c["D"], c["W"], c["S"], c["dense"]
    nqb = N // 64
    print(f"fwd full workload {w}: generating inputs", flush=True)
    q, k, v = synth.fwd_inputs(w, B, H, N, D, c["dtype"])
    print("fwd full: running kernel", flush=True)
    o, lse, lay = _run(q, k, v, H, N, W, S, dense)
    rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, dense))
    assert np.array_equal(lay.row_ptr.cpu().numpy(), rp)
    rng = np.random.default_rng(w)
    heads = sorted(set([0, H - 1, *[int(x) for x in dense[:1]], *rng.integers(0, H, 2).tolist()]))
    blocks = sorted(set([0, 1, nqb // 2, nqb - 2, nqb - 1, int(rng.integers(0, nqb))]))
    print(f"fwd full: oracle on heads {heads} blocks {blocks}", flush=True)
    ob = int(rng.integers(0, B))
    oo, ol = oracle.attn_fwd_blocks(LazyF64(q[ob:ob + 1]), LazyF64(k[ob:ob + 1]),
                                    LazyF64(v[ob:ob + 1]), rp, ci, nqb, heads=heads, q_blocks=blocks)
    got_o, got_l = f64(o[ob]), f64(lse[ob])
    for h in heads:
        for i in blocks:
            rows = slice(i * 64, (i + 1) * 64)
            assert_out_close(got_o[h, rows], oo[0, h, rows], "bf16", f"head {h} block {i}")
            assert_lse_close(got_l[h, rows], ol[0, h, rows], "bf16")
    # properties at full size: every output finite, |o| bounded by max |v|
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert float(o.float().abs().max()) <= float(v.float().abs().max()) + 1e-2


@pytest.mark.parametrize("w", [2, 3, 4])
def test_full_size_sampled(w):
    _sampled_full(w)


def test_workspace_content_does_not_matter():
    """The work queues tag their words with the launch: a workspace holding zeros,
    all ones, random bytes or the words of earlier launches gives the same result."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, N, D, W, S, dense = 2, 4, 1024, 128, 3, 4, (1,)
    print("fwd workspace contents", flush=True)
    q, k, v = _case(13, B, H, N, D, "bf16")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lay = s2.s2_build_layout(s2.Pattern(H, W, S, dense), N // 64, dev)
    nbytes = s2.s2_attn_fwd_workspace()
    g = torch.Generator(device=dev).manual_seed(5)
    fills = [torch.zeros(nbytes, dtype=torch.uint8, device=dev),
             torch.full((nbytes,), 255, dtype=torch.uint8, device=dev),
             torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=g)]
    outs = []
    for ws in fills:
        for _ in range(3):   # the same workspace again: its words now hold the previous launch's tag
            outs.append(s2.s2_attn_fwd(qd, kd, vd, lay, workspace=ws))
    torch.cuda.synchronize()
    rp, ci = oracle.build_layout(H, N // 64, W, S, synth.dense_flags(H, dense))
    oo, ol = oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, N // 64)
    assert_out_close(f64(outs[0][0]), oo, "bf16")
    assert_lse_close(f64(outs[0][1]), ol, "bf16")
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_two_streams_concurrently():
    """Two forwards enqueued on two streams with nothing ordering them, each with its
    own workspace (and a varlen forward on a third), all equal to the oracle."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    H, N, D, W, S, dense = 8, 2048, 128, 4, 8, (0,)
    print("fwd two streams", flush=True)
    lay = s2.s2_build_layout(s2.Pattern(H, W, S, dense), N // 64, dev)
    cases = [_case(14 + c, 1, H, N, D, "bf16") for c in range(2)]
    dev_in = [[t.to(dev) for t in c] for c in cases]
    cu = torch.tensor([0, 700, 2048], dtype=torch.int32, device=dev)
    qv = dev_in[0][0][0].transpose(0, 1).contiguous()
    kv, vv = (dev_in[0][i][0].transpose(0, 1).contiguous() for i in (1, 2))
    streams = [torch.cuda.Stream(device=dev) for _ in range(3)]
    main = torch.cuda.current_stream(dev)
    for st in streams:
        st.wait_stream(main)
    results = []
    for rep in range(3):
        for c, st in enumerate(streams[:2]):
            with torch.cuda.stream(st):
                results.append((c, s2.s2_attn_fwd(*dev_in[c], lay)))
        with torch.cuda.stream(streams[2]):
            results.append(("varlen", s2.s2_attn_fwd_varlen(qv, kv, vv, cu, lay)))
    for st in streams:
        main.wait_stream(st)
    torch.cuda.synchronize()
    rp, ci = oracle.build_layout(H, N // 64, W, S, synth.dense_flags(H, dense))
    refs = [oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, N // 64) for q, k, v in cases]
    q0, k0, v0 = (f64(t[0].transpose(0, 1)) for t in cases[0])
    ref_vl = oracle.attn_fwd_varlen(q0, k0, v0, cu.cpu().numpy(), rp, ci, N // 64)
    for c, (o, l) in results:
        if c == "varlen":
            assert_out_close(f64(o), ref_vl[0], "bf16", "varlen")
            assert_lse_close(f64(l), ref_vl[1], "bf16")
        else:
            assert_out_close(f64(o), refs[c][0], "bf16", f"stream {c}")
            assert_lse_close(f64(l), refs[c][1], "bf16")
