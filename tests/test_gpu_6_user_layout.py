"""GPU path on caller-built layouts (any head-major CSR of causal blocks) against
the fp64 oracle: device validation, the general column view, and the forward,
decode, paged decode and backward kernels on layouts that are not the built-in
pattern (windows and strides changing along the context, global blocks, random
blocks, empty rows, rows without their diagonal block)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import LazyF64, assert_lse_close, assert_out_close, device, f64

pytestmark = pytest.mark.gpu

BLOCK = 64


def ranged_layout(H, nqb, ranges):
    """Per head and per query-block range its own window and stride: ranges[h] is a
    list of (first query block, W, S, dense) in ascending order of first block."""
    rp, ci = [0], []
    for h in range(H):
        for i in range(nqb):
            first, W, S, dense = [r for r in ranges[h] if r[0] <= i][-1]
            ci += oracle.active_blocks(h, i, W, S, dense)
            rp.append(len(ci))
    return np.array(rp, dtype=np.int32), np.array(ci, dtype=np.int32)


def global_window_layout(H, nqb, globals_, W, rng=None, extra=0):
    """Longformer-like (global blocks + local window), plus `extra` random earlier
    blocks per row as in BigBird when rng is given."""
    rp, ci = [0], []
    for h in range(H):
        for i in range(nqb):
            cols = {j for j in globals_ if j <= i} | set(range(max(0, i - W + 1), i + 1))
            if rng is not None and i > 0:
                cols |= set(rng.integers(0, i, size=extra).tolist())
            ci += sorted(cols)
            rp.append(len(ci))
    return np.array(rp, dtype=np.int32), np.array(ci, dtype=np.int32)


def random_layout(rng, H, nqb, density=0.3, p_empty=0.1, p_nodiag=0.2):
    rp, ci = [0], []
    for h in range(H):
        for i in range(nqb):
            u = rng.random()
            if u < p_empty:
                cols = []
            else:
                cols = set(np.nonzero(rng.random(i + 1) < density)[0].tolist())
                if u >= p_empty + p_nodiag:
                    cols.add(i)
                else:
                    cols.discard(i)
                cols = sorted(cols)
            ci += cols
            rp.append(len(ci))
    return np.array(rp, dtype=np.int32), np.array(ci, dtype=np.int32)


def _dev_layout(rp, ci, H, nqb, validate=True):
    import head_heterogeneous_block_amd as s2
    dev = device()
    return s2.layout_from_csr(torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), H, nqb, validate)


LAYOUTS = {
    "ranged": lambda rng, H, nqb: ranged_layout(
        H, nqb, [[(0, 2, 4, h == 0), (nqb // 3, 4, 8, False), (2 * nqb // 3, 1 + h % 3, 2 + h, h == 1)]
                 for h in range(H)]),
    "longformer": lambda rng, H, nqb: global_window_layout(H, nqb, (0, 1), 3),
    "bigbird": lambda rng, H, nqb: global_window_layout(H, nqb, (0,), 2, rng, 2),
    "random": lambda rng, H, nqb: random_layout(rng, H, nqb),
}


# ---------------------------------------------------------------------------
# validation
# ---------------------------------------------------------------------------
def test_validate_accepts_good_layouts():
    rng = np.random.default_rng(60)
    for name, make in LAYOUTS.items():
        rp, ci = make(rng, 3, 20)
        print("validate", name, flush=True)
        _dev_layout(rp, ci, 3, 20)   # raises if rejected


@pytest.mark.parametrize("fault,row,text", [
    ("start", 0, "row_ptr[0]"), ("end", 59, "must equal nnz"), ("ptr", 12, "row_ptr decreases"),
    ("future", 7, "outside"), ("negative", 30, "outside"), ("unsorted", 44, "ascending"),
    ("duplicate", 51, "ascending")])
def test_validate_rejects(fault, row, text):
    import head_heterogeneous_block_amd as s2
    H, nqb = 3, 20
    rp, ci = random_layout(np.random.default_rng(61), H, nqb, p_empty=0.0, p_nodiag=0.0, density=0.5)
    rp, ci = rp.copy(), ci.copy()
    i = row % nqb
    a, e = rp[row], rp[row + 1]
    if fault == "start":
        rp[0] = 1
    elif fault == "end":
        rp[-1] -= 1
    elif fault == "ptr":
        rp[row + 1] = rp[row] - 1
    elif fault == "future":
        ci[e - 1] = i + 1
    elif fault == "negative":
        ci[a] = -1
    elif fault == "unsorted":
        assert e - a >= 2
        ci[a], ci[a + 1] = ci[a + 1], ci[a]
    elif fault == "duplicate":
        assert e - a >= 2
        ci[a + 1] = ci[a]
    ly = _dev_layout(rp, ci, H, nqb, validate=False)
    with pytest.raises(s2.S2Error) as err:
        s2.s2_validate_layout(ly)
    assert text in str(err.value), str(err.value)
    if fault not in ("start", "end"):
        assert f"row {row} " in str(err.value), str(err.value)


# ---------------------------------------------------------------------------
# column view
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,H,nqb", [("ranged", 3, 40), ("longformer", 2, 33), ("bigbird", 4, 65),
                                        ("random", 5, 31), ("random", 1, 1), ("ranged", 2, 128)])
def test_transpose_matches_oracle(name, H, nqb):
    import head_heterogeneous_block_amd as s2
    rng = np.random.default_rng(62)
    rp, ci = LAYOUTS[name](rng, H, nqb)
    if len(ci) == 0:
        pytest.skip("empty layout")
    print(f"transpose {name} H={H} nqb={nqb} nnz={len(ci)}", flush=True)
    ly = _dev_layout(rp, ci, H, nqb)
    lt = s2.s2_transpose_layout(ly)
    torch.cuda.synchronize()
    cp, ri = oracle.transpose_layout(rp, ci, H, nqb)
    assert np.array_equal(lt.row_ptr.cpu().numpy(), cp)
    assert np.array_equal(lt.col_idx.cpu().numpy()[:len(ri)], ri)


@pytest.mark.parametrize("H,nqb,W,S,dense", [(4, 64, 2, 4, (1,)), (16, 128, 4, 8, (0, 1)), (3, 37, 3, 5, ())])
def test_transpose_equals_closed_form_column_view(H, nqb, W, S, dense):
    import head_heterogeneous_block_amd as s2
    dev = device()
    pat = s2.Pattern(H, W, S, dense)
    lay = s2.s2_build_layout(pat, nqb, dev)
    a = s2.s2_transpose_layout(lay)
    b = s2.s2_build_layout_t(pat, nqb, dev)
    torch.cuda.synchronize()
    assert torch.equal(a.row_ptr, b.row_ptr) and torch.equal(a.col_idx[:lay.nnz], b.col_idx[:lay.nnz])


# ---------------------------------------------------------------------------
# attention on caller-built layouts
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", list(LAYOUTS))
def test_forward_on_user_layouts(dtype, name):
    import head_heterogeneous_block_amd as s2
    B, H, N, D = 2, 3, 1536, 128 if dtype == "bf16" else 64
    nqb = N // BLOCK
    rp, ci = LAYOUTS[name](np.random.default_rng(63), H, nqb)
    print(f"fwd {dtype} on {name} layout: B={B} H={H} N={N} D={D} nnz={len(ci)}", flush=True)
    ly = _dev_layout(rp, ci, H, nqb)
    q, k, v = synth.fwd_inputs(63, B, H, N, D, dtype)
    dev = device()
    o, lse = s2.s2_attn_fwd(q.to(dev), k.to(dev), v.to(dev), ly)
    torch.cuda.synchronize()
    oo, ol = oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, nqb)
    got_o, got_l = f64(o), f64(lse)
    empty = np.isinf(ol)
    assert np.array_equal(np.isinf(got_l), empty) and np.all(got_l[empty] < 0)
    assert not got_o[empty].any()                      # empty rows: output 0
    assert_out_close(got_o, oo, dtype)
    assert_lse_close(got_l[~empty], ol[~empty], dtype)


@pytest.mark.parametrize("name", ["ranged", "random"])
def test_decode_on_user_layouts(name):
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 4, 3, 128, 1200
    nqb = -(-L // BLOCK)
    rp, ci = LAYOUTS[name](np.random.default_rng(64), H, nqb)
    ly = _dev_layout(rp, ci, H, nqb)
    seq = [1200, 1, 700, 64]
    print(f"decode on {name} layout seq={seq}", flush=True)
    q = synth.decode_query(64, B, H, D, "bf16")
    kc = synth.full_cache(64, synth.TENSOR_K, B, H, L, D, "bf16")
    vc = synth.full_cache(64, synth.TENSOR_V, B, H, L, D, "bf16")
    sl = torch.tensor(seq, dtype=torch.int32, device=dev)
    oo, ol = oracle.attn_decode(f64(q), oracle.dense_kv_blocks(f64(kc), f64(vc)), seq, rp, ci, nqb)
    empty = np.isinf(ol)
    for splits in (1, 3):
        o, lse = s2.s2_attn_decode(q.to(dev), kc.to(dev), vc.to(dev), sl, ly, splits=splits)
        torch.cuda.synchronize()
        got_o, got_l = f64(o), f64(lse)
        assert np.array_equal(np.isinf(got_l), empty) and not got_o[empty].any()
        assert_out_close(got_o[~empty], oo[~empty], "bf16")
        assert_lse_close(got_l[~empty], ol[~empty], "bf16")


def test_paged_decode_on_user_layout():
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, Hkv, D, L, P = 3, 4, 2, 128, 1024, 32
    nqb = L // BLOCK
    rp, ci = LAYOUTS["random"](np.random.default_rng(65), H, nqb)
    ly = _dev_layout(rp, ci, H, nqb)
    seq = [1024, 500, 77]
    q = synth.decode_query(65, B, H, D, "bf16")
    kc = synth.full_cache(65, synth.TENSOR_K, B, Hkv, L, D, "bf16")
    vc = synth.full_cache(65, synth.TENSOR_V, B, Hkv, L, D, "bf16")
    perm = np.random.default_rng(66).permutation(B * L // P).astype(np.int32)
    table = perm.reshape(B, L // P)
    kp = torch.empty((B * L // P, Hkv, P, D), dtype=torch.bfloat16)
    vp = torch.empty_like(kp)
    for b in range(B):
        for s in range(L // P):
            kp[table[b, s]] = kc[b, :, s * P:(s + 1) * P]
            vp[table[b, s]] = vc[b, :, s * P:(s + 1) * P]
    o, lse = s2.s2_attn_decode_paged(q.to(dev), kp.to(dev), vp.to(dev), torch.from_numpy(table).to(dev),
                                     torch.tensor(seq, dtype=torch.int32, device=dev), ly, splits=2)
    torch.cuda.synchronize()
    oo, ol = oracle.attn_decode(f64(q), oracle.paged_kv_blocks(f64(kp), f64(vp), table, P, H // Hkv), seq,
                                rp, ci, nqb)
    empty = np.isinf(ol)
    got_o, got_l = f64(o), f64(lse)
    assert np.array_equal(np.isinf(got_l), empty) and not got_o[empty].any()
    assert_out_close(got_o[~empty], oo[~empty], "bf16")
    assert_lse_close(got_l[~empty], ol[~empty], "bf16")


def _rel_check(got, ref, what):
    scale = np.max(np.abs(ref))
    err = np.abs(got - ref)
    print(f"  {what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} (max|ref| {scale:.3e})", flush=True)
    assert err.max() <= 2e-2 * scale and err.mean() <= 2e-3 * scale


@pytest.mark.parametrize("name", ["ranged", "random", "bigbird"])
def test_backward_on_user_layouts(name):
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, N, D = 1, 3, 1024, 128
    nqb = N // BLOCK
    rp, ci = LAYOUTS[name](np.random.default_rng(67), H, nqb)
    print(f"bwd on {name} layout nnz={len(ci)}", flush=True)
    ly = _dev_layout(rp, ci, H, nqb)
    lt = s2.s2_transpose_layout(ly)
    q, k, v = synth.fwd_inputs(67, B, H, N, D, "bf16")
    do = synth.fwd_inputs(68, B, H, N, D, "bf16")[0]
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = s2.s2_attn_fwd(qd, kd, vd, ly)
    dq, dk, dv = s2.s2_attn_bwd(qd, kd, vd, o, dod, lse, ly, lt)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd_dense(f64(q), f64(k), f64(v), f64(do), rp, ci, nqb)
    for got, ref, w in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        _rel_check(f64(got), ref, w)


def test_full_size_ranged_layout_sampled():
    """1.3B-shaped prefill (B=4, H=16, N=8192) on a layout whose window and stride
    change over three context ranges per head; the column view is compared whole,
    the forward on sampled (b, h, query block) rows."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    c = synth.WORKLOADS[2]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    nqb = N // BLOCK
    ranges = [[(0, 2, 4, h == 0), (nqb // 4, 4, 8, False), (nqb // 2, 8, 16 + h, h in (1, 2))]
              for h in range(H)]
    rp, ci = ranged_layout(H, nqb, ranges)
    print(f"full ranged: nnz {len(ci)}", flush=True)
    ly = _dev_layout(rp, ci, H, nqb)
    lt = s2.s2_transpose_layout(ly)
    q, k, v = synth.fwd_inputs(2, B, H, N, D, "bf16")
    o, lse = s2.s2_attn_fwd(q.to(dev), k.to(dev), v.to(dev), ly)
    torch.cuda.synchronize()
    cp, ri = oracle.transpose_layout(rp, ci, H, nqb)
    assert np.array_equal(lt.row_ptr.cpu().numpy(), cp) and np.array_equal(lt.col_idx.cpu().numpy(), ri)
    rng = np.random.default_rng(69)
    blocks = sorted(set(rng.integers(0, nqb, 6).tolist()) | {0, nqb // 4, nqb // 2, nqb - 1})
    for b, h in ((0, 0), (3, 1), (2, 7), (1, 15)):
        oo, ol = oracle.attn_fwd_blocks(LazyF64(q), LazyF64(k), LazyF64(v), rp, ci, nqb, heads=[h],
                                        q_blocks=blocks, batches=[b])
        for i in blocks:
            rows = slice(i * BLOCK, (i + 1) * BLOCK)
            assert_out_close(f64(o[b, h, rows]), oo[b, h, rows], "bf16", f"b {b} h {h} block {i}")
            assert_lse_close(f64(lse[b, h, rows]), ol[b, h, rows], "bf16")
