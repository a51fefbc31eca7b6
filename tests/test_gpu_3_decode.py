"""GPU split-KV decode against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import assert_lse_close, assert_out_close, assert_rows_match_oracle, device, f64

pytestmark = pytest.mark.gpu


def _small(dtype, B, H, D, cache_len, W, S, dense, seq_lens, splits):
    import head_heterogeneous_block_amd as s2
    dev = device()
    nqb = (cache_len + 63) // 64
    print(f"decode {dtype} B={B} H={H} D={D} L={cache_len} seq={seq_lens} splits={splits}", flush=True)
    q = synth.decode_query(21, B, H, D, dtype)
    kc = synth.full_cache(21, synth.TENSOR_K, B, H, cache_len, D, dtype)
    vc = synth.full_cache(21, synth.TENSOR_V, B, H, cache_len, D, dtype)
    lay = s2.s2_build_layout(s2.Pattern(H, W, S, tuple(dense)), nqb, dev)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=dev)
    o, lse = s2.s2_attn_decode(q.to(dev), kc.to(dev), vc.to(dev), sl, lay, splits=splits)
    torch.cuda.synchronize()
    rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, dense))
    oo, ol = oracle.attn_decode(f64(q), oracle.dense_kv_blocks(f64(kc), f64(vc)), seq_lens, rp, ci, nqb)
    return o, lse, oo, ol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [1, 2, 3, 0, 16])
def test_small_ragged(dtype, splits):
    o, lse, oo, ol = _small(dtype, 3, 4, 128, 1000, 2, 4, (2,), [1000, 1, 517], splits)
    assert_out_close(f64(o), oo, dtype)
    assert_lse_close(f64(lse), ol, dtype)


@pytest.mark.parametrize("D", [64, 128])
def test_head_dims(D):
    o, lse, oo, ol = _small("bf16", 2, 3, D, 640, 3, 5, (), [640, 130], 0)
    assert_out_close(f64(o), oo, "bf16")
    assert_lse_close(f64(lse), ol, "bf16")


def test_split_invariance():
    outs = []
    for sp in (1, 2, 5, 40):
        o, lse, oo, ol = _small("f32", 2, 4, 128, 2560, 8, 16, (), [2560, 2000], sp)
        outs.append((f64(o), f64(lse)))
    for o, l in outs[1:]:
        assert np.max(np.abs(o - outs[0][0])) <= 1e-6
        assert np.max(np.abs(l - outs[0][1])) <= 1e-6


def test_invalid_lengths_give_nan_rows():
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 3, 2, 128, 256
    q = synth.decode_query(22, B, H, D, "bf16").to(dev)
    kc = synth.full_cache(22, synth.TENSOR_K, B, H, L, D, "bf16").to(dev)
    vc = synth.full_cache(22, synth.TENSOR_V, B, H, L, D, "bf16").to(dev)
    lay = s2.s2_build_layout(s2.Pattern(H, 2, 2), L // 64, dev)
    seq = [0, 100, L + 1]
    sl = torch.tensor(seq, dtype=torch.int32, device=dev)
    rp, ci = oracle.build_layout(H, L // 64, 2, 2)
    oo, ol = oracle.attn_decode(f64(q), oracle.dense_kv_blocks(f64(kc), f64(vc)), seq, rp, ci, L // 64,
                                cache_len=L)
    assert np.isnan(ol[0]).all() and np.isnan(ol[2]).all() and np.isfinite(ol[1]).all()
    for splits in (1, 2, 0):
        print(f"decode invalid lengths splits={splits}", flush=True)
        o, lse = s2.s2_attn_decode(q, kc, vc, sl, lay, splits=splits)
        torch.cuda.synchronize()
        assert_rows_match_oracle(f64(o), f64(lse), oo, ol, "bf16", f"splits={splits}")


def test_decode_equals_forward_last_row():
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, N, D, W, S = 2, 4, 2048, 128, 8, 16
    q, k, v = synth.fwd_inputs(23, B, H, N, D, "bf16")
    lay = s2.s2_build_layout(s2.Pattern(H, W, S), N // 64, dev)
    sl = torch.full((B,), N, dtype=torch.int32, device=dev)
    od, ld = s2.s2_attn_decode(q[:, :, -1].contiguous().to(dev), k.to(dev), v.to(dev), sl, lay)
    torch.cuda.synchronize()
    rp, ci = oracle.build_layout(H, N // 64, W, S)
    of, lf = oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, N // 64, q_blocks=[N // 64 - 1])
    assert_out_close(f64(od), of[:, :, -1], "bf16")
    assert_lse_close(f64(ld), lf[:, :, -1], "bf16")


def test_full_size_decode_sampled():
    """64 sequences x 32 heads x 32768 context: only active blocks hold data, the
    rest of the 34 GB cache is NaN, so any read outside the CSR row shows up."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    c = synth.WORKLOADS[5]
    B, H, L, D = c["B"], c["H"], c["N"], c["D"]
    nqb = L // 64
    lay = s2.s2_build_layout(s2.Pattern(H, c["W"], c["S"], c["dense"]), nqb, dev)
    rp, ci = oracle.build_layout(H, nqb, c["W"], c["S"], synth.dense_flags(H, c["dense"]))
    print("decode full: allocating 2 x 17 GB caches", flush=True)
    kc = torch.full((B, H, L, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full((B, H, L, D), float("nan"), dtype=torch.bfloat16, device=dev)
    print("decode full: writing the active blocks", flush=True)
    for h in range(H):
        cols = oracle.row_blocks(rp, ci, nqb, h, nqb - 1).tolist()
        idx = torch.tensor(cols, device=dev)
        for b in range(B):
            kb = torch.stack([synth.cache_block(5, synth.TENSOR_K, b, h, j, D, "bf16") for j in cols])
            vb = torch.stack([synth.cache_block(5, synth.TENSOR_V, b, h, j, D, "bf16") for j in cols])
            kc[b, h].view(nqb, 64, D).index_copy_(0, idx, kb.to(dev))
            vc[b, h].view(nqb, 64, D).index_copy_(0, idx, vb.to(dev))
    q = synth.decode_query(5, B, H, D, "bf16")
    sl = torch.full((B,), L, dtype=torch.int32, device=dev)
    print("decode full: running kernel", flush=True)
    o, lse = s2.s2_attn_decode(q.to(dev), kc, vc, sl, lay)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(5)
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 48), rng.integers(0, H, 48))]
    pairs += [(0, 0), (B - 1, H - 1), (0, 1), (1, 9)]

    def kv_block(b, h, j):
        return (f64(synth.cache_block(5, synth.TENSOR_K, b, h, j, D, "bf16")),
                f64(synth.cache_block(5, synth.TENSOR_V, b, h, j, D, "bf16")))
    oo, ol = oracle.attn_decode(f64(q), kv_block, [L] * B, rp, ci, nqb, pairs=pairs)
    got_o, got_l = f64(o), f64(lse)
    for b, h in pairs:
        assert_out_close(got_o[b, h], oo[b, h], "bf16", f"seq {b} head {h}")
        assert_lse_close(got_l[b, h], ol[b, h], "bf16")
    del kc, vc
    torch.cuda.empty_cache()
