"""GPU packed variable-length forward against the fp64 oracle.

Sequences are packed back to back in [T_total, H, D] tensors; a sentinel fills
the output first, so a write outside a sequence's own tokens shows up."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import assert_lse_close, assert_out_close, device, f64

pytestmark = pytest.mark.gpu

BLOCK = 64


def _packed(seed, T, H, D):
    q, k, v = synth.fwd_inputs(seed, 1, H, T, D, "bf16")
    return tuple(x[0].transpose(0, 1).contiguous() for x in (q, k, v))  # [T, H, D]


def _run(lens, H=3, D=128, W=2, S=3, dense=(1,), layout=None, seed=71, cu=None, T=None):
    import head_heterogeneous_block_amd as s2
    dev = device()
    if cu is None:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1]) if T is None else T
    nqb = -(-max(lens) // BLOCK)
    if layout is None:
        rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, dense))
        ly = s2.s2_build_layout(s2.Pattern(H, W, S, dense), nqb, dev)
    else:
        rp, ci = layout
        ly = s2.layout_from_csr(torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), H, nqb)
    print(f"varlen lens={list(lens)} H={H} D={D} T={T}", flush=True)
    q, k, v = _packed(seed, T, H, D)
    out = torch.full((T, H, D), 7.0, dtype=torch.bfloat16, device=dev)   # sentinel
    lse = torch.full((H, T), 7.0, dtype=torch.float32, device=dev)
    s2.s2_attn_fwd_varlen(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(cu).to(dev), ly, out=out, lse=lse)
    torch.cuda.synchronize()
    return cu, q, k, v, rp, ci, nqb, f64(out), f64(lse)


@pytest.mark.parametrize("D", [128, 64])
def test_varlen_ragged(D):
    lens = [1, 63, 64, 65, 130, 700, 1000]
    cu, q, k, v, rp, ci, nqb, o, lse = _run(lens, D=D)
    oo, ol = oracle.attn_fwd_varlen(f64(q), f64(k), f64(v), cu, rp, ci, nqb)
    assert_out_close(o, oo, "bf16")
    assert_lse_close(lse, ol, "bf16")


def test_varlen_single_sequence_equals_fixed_length():
    import head_heterogeneous_block_amd as s2
    dev = device()
    cu, q, k, v, rp, ci, nqb, o, lse = _run([1024], H=4, W=3, S=4, dense=())
    ly = s2.s2_build_layout(s2.Pattern(4, 3, 4), nqb, dev)
    of, lf = s2.s2_attn_fwd(*(x.transpose(0, 1)[None].contiguous().to(dev) for x in (q, k, v)), ly)
    torch.cuda.synchronize()
    assert np.array_equal(o, f64(of[0].transpose(0, 1))) and np.array_equal(lse, f64(lf[0]))


def test_varlen_user_layout_with_empty_rows():
    rng = np.random.default_rng(72)
    H, nqb = 3, 12
    rp, ci = [0], []
    for h in range(H):
        for i in range(nqb):
            cols = [] if rng.random() < 0.15 else sorted(set(np.nonzero(rng.random(i + 1) < 0.4)[0].tolist()) | {i})
            ci += cols
            rp.append(len(ci))
    rp, ci = np.array(rp, dtype=np.int32), np.array(ci, dtype=np.int32)
    lens = [700, 33, 768, 129]
    cu, q, k, v, rp, ci, nqb, o, lse = _run(lens, H=H, layout=(rp, ci))
    oo, ol = oracle.attn_fwd_varlen(f64(q), f64(k), f64(v), cu, rp, ci, nqb)
    empty = np.isinf(ol)
    assert np.array_equal(np.isinf(lse), empty) and not o.transpose(1, 0, 2)[empty].any()
    assert_out_close(o, oo, "bf16")
    assert_lse_close(lse[~empty], ol[~empty], "bf16")


def test_varlen_malformed_sequences_are_skipped():
    # sequence 1 ends past T_total, sequence 2 starts after it ends, sequence 3
    # is longer than the layout: only sequence 0 is computed, the rest untouched
    T = 900
    cu = np.array([0, 300, 5000, 400, 900], dtype=np.int32)
    cu_ok, q, k, v, rp, ci, nqb, o, lse = _run([300], cu=cu, T=T)   # the layout covers 320 tokens
    oo, ol = oracle.attn_fwd_varlen(f64(q), f64(k), f64(v), cu, rp, ci, nqb)
    skipped = np.isnan(ol).all(axis=0)        # tokens of the sequences the oracle skips
    assert skipped[300:].all() and not skipped[:300].any()
    assert_out_close(o[:300], oo[:300], "bf16")
    assert_lse_close(lse[:, :300], ol[:, :300], "bf16")
    assert np.all(o[skipped] == 7.0) and np.all(lse[:, skipped] == 7.0)   # not written


def test_varlen_full_size_sampled():
    """32768 tokens (the 1.3B-shaped prefill's batch) in seven ragged sequences,
    16 heads, D = 128, the 1.3B pattern; sampled sequences and blocks."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    c = synth.WORKLOADS[2]
    H, D = c["H"], c["D"]
    lens = [8192, 5000, 3000, 1, 12000, 4511, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    nqb = -(-max(lens) // BLOCK)
    ly = s2.s2_build_layout(s2.Pattern(H, c["W"], c["S"], c["dense"]), nqb, dev)
    rp, ci = oracle.build_layout(H, nqb, c["W"], c["S"], synth.dense_flags(H, c["dense"]))
    q = synth.randn_device(731, (T, H, D), "bf16", dev)
    k = synth.randn_device(732, (T, H, D), "bf16", dev)
    v = synth.randn_device(733, (T, H, D), "bf16", dev)
    print("varlen full: running kernel", flush=True)
    o, lse = s2.s2_attn_fwd_varlen(q, k, v, torch.from_numpy(cu).to(dev), ly)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    for b in (0, 1, 3, 4, 6):
        n = lens[b]
        blocks = sorted({0, (n - 1) // 128, (n - 1) // 64})
        t0 = int(cu[b])
        sub = slice(t0, t0 + n)
        cu_b = np.array([0, n], dtype=np.int32)
        oo, ol = oracle.attn_fwd_varlen(f64(q[sub]), f64(k[sub]), f64(v[sub]), cu_b, rp, ci, nqb, q_blocks=blocks)
        for i in blocks:
            rows = slice(i * BLOCK, min(n, (i + 1) * BLOCK))
            assert_out_close(f64(o[sub][rows]), oo[rows], "bf16", f"seq {b} block {i}")
            assert_lse_close(f64(lse[:, sub][:, rows]), ol[:, rows], "bf16")


@pytest.mark.parametrize("pipelined", [False, True])
@pytest.mark.parametrize("n_seq", [256, 300])
def test_varlen_many_sequences(n_seq, pipelined, monkeypatch):
    """Many short sequences: with 4 heads, 256 sequences are 1,024 (sequence,
    head) pairs, the most the kernel ranks pair by pair; 300 are 1,200, past
    it, where the queues fall back to ranking by head.  Lengths 1..200 tokens,
    ragged block tails everywhere."""
    monkeypatch.setenv("S2ATTN_FWD_PIPELINED", "1" if pipelined else "0")
    rng = np.random.default_rng(n_seq)
    lens = [int(x) for x in rng.integers(1, 201, size=n_seq)]
    cu, q, k, v, rp, ci, nqb, o, lse = _run(lens, H=4, W=2, S=2, dense=(3,), seed=n_seq)
    oo, ol = oracle.attn_fwd_varlen(f64(q), f64(k), f64(v), cu, rp, ci, nqb)
    assert_out_close(o, oo, "bf16")
    assert_lse_close(lse, ol, "bf16")
