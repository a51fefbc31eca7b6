"""s2_attn_decode_noalloc (split partials in the library's static per-GPU scratch)
against s2_attn_decode with a caller workspace: the same kernels with the same split
count, so the outputs must be bit-identical; both also within the tolerance of the
fp64 oracle.  Two calls in a row, the second smaller, so the second reads scratch the
first left behind."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import assert_rows_match_oracle, device, f64

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, D, L, W, S, dense, dtype):
    import head_heterogeneous_block_amd as s2
    dev = device()
    q = synth.decode_query(seed, B, H, D, dtype)
    kc = synth.full_cache(seed, synth.TENSOR_K, B, H, L, D, dtype)
    vc = synth.full_cache(seed, synth.TENSOR_V, B, H, L, D, dtype)
    nqb = -(-L // 64)
    lay = s2.s2_build_layout(s2.Pattern(H, W, S, dense), nqb, dev)
    return q, kc, vc, lay, nqb


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_workspace_decode_twice(dtype):
    import head_heterogeneous_block_amd as s2
    dev = device()
    cases = [
        # seed, B, H, D, L, W, S, dense, seq_lens, splits
        (61, 6, 8, 128, 3000, 4, 8, (1,), [3000, 1, 2999, 64, 65, 1700], 5),
        (62, 2, 4, 64, 700, 2, 4, (), [700, 333], 3),          # smaller: reads the first call's leftovers
    ]
    for seed, B, H, D, L, W, S, dense, seq, splits in cases:
        print(f"noalloc {dtype} B={B} H={H} D={D} L={L} splits={splits}", flush=True)
        q, kc, vc, lay, nqb = _inputs(seed, B, H, D, L, W, S, dense, dtype)
        qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
        sl = torch.tensor(seq, dtype=torch.int32, device=dev)
        o_ref, l_ref = s2.s2_attn_decode(qd, kd, vd, sl, lay, splits=splits)
        o = torch.empty_like(o_ref)
        lse = torch.empty_like(l_ref)
        s2.s2_attn_decode_noalloc(qd, kd, vd, sl, lay, o, lse, splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, dense))
        oo, ol = oracle.attn_decode(f64(q), oracle.dense_kv_blocks(f64(kc), f64(vc)), seq, rp, ci, nqb,
                                    cache_len=L)
        assert_rows_match_oracle(f64(o), f64(lse), oo, ol, dtype)


def test_noalloc_automatic_splits_and_invalid_lengths():
    """Automatic split count (several splits for a small batch: the scratch is used),
    NaN rows for invalid lengths, as the workspace entry point."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 3, 2, 128, 1024
    q, kc, vc, lay, nqb = _inputs(63, B, H, D, L, 2, 4, (), "bf16")
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    seq = [1024, 0, 517]
    sl = torch.tensor(seq, dtype=torch.int32, device=dev)
    assert s2.s2_attn_decode_workspace(lay, B, D, 0) > 0
    o_ref, l_ref = s2.s2_attn_decode(qd, kd, vd, sl, lay)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    for _ in range(2):
        s2.s2_attn_decode_noalloc(qd, kd, vd, sl, lay, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(o[[0, 2]], o_ref[[0, 2]]) and torch.equal(lse[[0, 2]], l_ref[[0, 2]])
        assert torch.isnan(o[1]).all() and torch.isnan(lse[1]).all()
    rp, ci = oracle.build_layout(H, nqb, 2, 4)
    oo, ol = oracle.attn_decode(f64(q), oracle.dense_kv_blocks(f64(kc), f64(vc)), seq, rp, ci, nqb, cache_len=L)
    assert_rows_match_oracle(f64(o), f64(lse), oo, ol, "bf16")


def test_noalloc_rejects_oversize_before_launch():
    """Partials beyond the static scratch: S2_ECAPACITY, nothing launched (the output
    keeps its sentinel)."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 64, 32, 128, 128
    q = torch.zeros((B, H, D), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((B, H, L, D), dtype=torch.bfloat16, device=dev)
    lay = s2.s2_build_layout(s2.Pattern(H, 1, 1), L // 64, dev)
    sl = torch.full((B,), L, dtype=torch.int32, device=dev)
    o = torch.full((B, H, D), 7.0, dtype=torch.bfloat16, device=dev)
    # 64 * 32 * 2 splits * 129 floats = 2.1 MB fits; 64 splits would need 67.6 MB
    s2.s2_attn_decode_noalloc(q, kc, kc, sl, lay, o, splits=2)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    o.fill_(7.0)
    with pytest.raises(s2.S2Error) as ei:
        s2.s2_attn_decode_noalloc(q, kc, kc, sl, lay, o, splits=64)
    assert ei.value.status == 3 and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
