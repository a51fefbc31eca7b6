"""GPU query-aware block lists (block key bounds, top-budget selection, decode over
per-(sequence, head) rows) against the fp64 oracle.

Block bounds are minima and maxima of the keys: bit-exact.  The selection is an
integer result decided by floating point: the kernel sums the bound in fp32, the
oracle in fp64, so where two blocks' bounds differ by less than the fp32 rounding of
the sum either may be chosen.  Tests whose keys give every block a clearly different
bound require the oracle's lists exactly; the others check that the chosen blocks are
a valid top-budget set within that rounding.  Decode over the rows is compared with
the oracle on the rows the GPU chose."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import assert_lse_close, assert_out_close, assert_rows_match_oracle, device, f64

pytestmark = pytest.mark.gpu

BLOCK = 64


def _keys(seed, B, H, L, D, dtype, spread=3.0):
    """N(0, 1) keys plus one random offset vector per 64-token block (spread > 0), so
    that blocks differ in their bounds; spread = 0 gives iid keys."""
    g = torch.Generator().manual_seed(seed)
    nb = -(-L // BLOCK)
    k = torch.randn((B, H, nb * BLOCK, D), generator=g)
    if spread:
        k += spread * torch.randn((B, H, nb, 1, D), generator=g).expand(B, H, nb, BLOCK, D).reshape(B, H, nb * BLOCK, D)
    return k[:, :, :L].to(synth.torch_dtype(dtype))


def _check_rows(rp, ci, q64, kmin64, kmax64, lens, budget, H, exact=True, group=1):
    """GPU rows against the oracle.  Row offsets must match exactly.  A row whose
    choice is decided (no candidate at all, or a gap at the top-(budget-1) boundary
    wider than twice the fp32 rounding of the bounds) must equal the oracle's list;
    any other row must be a valid top-(budget-1) choice within that rounding.
    exact=True also requires every row with a choice to be decided.  Returns the
    number of rows equal to the oracle's."""
    rp_o, ci_o = oracle.select_blocks(q64, kmin64, kmax64, lens, budget, group=group)
    assert np.array_equal(rp, rp_o), "row offsets"
    same = 0
    for b, n in enumerate(lens):
        for h in range(H):
            r = b * H + h
            got, want = ci[rp[r]:rp[r + 1]], ci_o[rp_o[r]:rp_o[r + 1]]
            i = (n - 1) // BLOCK
            kk = budget - 1
            if len(want) == 0 or i + 1 <= budget or kk == 0:  # nothing to decide
                assert np.array_equal(got, want), f"seq {b} head {h}: {got} != {want}"
                same += 1
                continue
            g = h // group
            sc = oracle.block_scores(q64[b, h], kmin64[b, g, :i], kmax64[b, g, :i])
            mag = np.abs(q64[b, h]) * np.maximum(np.abs(kmin64[b, g, :i]), np.abs(kmax64[b, g, :i]))
            tol = 1e-5 * mag.sum(axis=1).max()  # bound on the fp32 rounding of one block's sum
            srt = np.sort(sc)[::-1]
            decided = srt[kk - 1] - srt[kk] > 2 * tol
            assert decided or not exact, f"seq {b} head {h}: boundary gap {srt[kk - 1] - srt[kk]:.2e} within rounding"
            if decided:
                assert np.array_equal(got, want), f"seq {b} head {h}: {got} != {want}"
                same += 1
                continue
            assert len(got) == len(want) and got[-1] == i and np.all(np.diff(got) > 0) and got[0] >= 0
            chosen, rest = got[:-1], np.setdiff1d(np.arange(i), got[:-1])
            assert sc[chosen].min() >= sc[rest].max() - tol, f"seq {b} head {h}: not a top-{kk} set"
            same += int(np.array_equal(got, want))
    return same


def _run(dtype, B, H, D, L, lens, budget, seed=81, spread=3.0, splits=0):
    import head_heterogeneous_block_amd as s2
    dev = device()
    print(f"select {dtype} B={B} H={H} D={D} L={L} lens={lens} budget={budget} splits={splits}", flush=True)
    k = _keys(seed, B, H, L, D, dtype, spread)
    v = _keys(seed + 1, B, H, L, D, dtype, 0.0)
    q = synth.decode_query(seed, B, H, D, dtype)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    kd, vd, qd = k.to(dev), v.to(dev), q.to(dev)
    nb = -(-L // BLOCK)
    kmin = torch.full((B, H, nb, D), 7.0, dtype=k.dtype, device=dev)  # sentinel: untouched blocks keep it
    kmax = torch.full((B, H, nb, D), 7.0, dtype=k.dtype, device=dev)
    s2.s2_block_minmax(kd, sl, kmin=kmin, kmax=kmax)
    rp, ci = s2.s2_select_blocks(qd, kmin, kmax, sl, budget, L)
    longest = min(budget, nb)
    o, lse = s2.s2_attn_decode_rows(qd, kd, vd, sl, rp, ci, longest, splits=splits)
    torch.cuda.synchronize()
    return dict(k=k, v=v, q=q, kmin=f64(kmin), kmax=f64(kmax), rp=rp.cpu().numpy(), ci=ci.cpu().numpy(),
                o=o, lse=lse)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_block_minmax_exact(dtype, D):
    B, H, L = 6, 3, 700
    lens = [700, 1, 64, 65, 0, 701]  # the last two are invalid: nothing written
    r = _run(dtype, B, H, D, L, lens, 4)
    kmin_o, kmax_o = oracle.block_minmax(f64(r["k"]), lens)
    for b, n in enumerate(lens):
        nv = -(-n // BLOCK) if 1 <= n <= L else 0
        assert np.array_equal(r["kmin"][b, :, :nv], kmin_o[b, :, :nv])
        assert np.array_equal(r["kmax"][b, :, :nv], kmax_o[b, :, :nv])
        assert np.all(r["kmin"][b, :, nv:] == 7.0) and np.all(r["kmax"][b, :, nv:] == 7.0)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("budget", [1, 3, 8, 100])
def test_select_matches_oracle(dtype, D, budget):
    B, H, L = 5, 4, 2000
    lens = [2000, 1, 640, 641, 1234]
    r = _run(dtype, B, H, D, L, lens, budget)
    kmin_o, kmax_o = oracle.block_minmax(f64(r["k"]), lens)
    assert _check_rows(r["rp"], r["ci"], f64(r["q"]), kmin_o, kmax_o, lens, budget, H) == B * H


def test_select_ties_take_the_lower_blocks():
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 2, 3, 128, 1280
    blk = torch.randn((1, 1, BLOCK, D), generator=torch.Generator().manual_seed(5))
    k = blk.repeat(B, H, L // BLOCK, 1).to(torch.bfloat16)  # every block the same keys
    q = synth.decode_query(86, B, H, D, "bf16")
    sl = torch.tensor([1280, 700], dtype=torch.int32, device=dev)
    kmin, kmax = s2.s2_block_minmax(k.to(dev), sl)
    rp, ci = s2.s2_select_blocks(q.to(dev), kmin, kmax, sl, 5, L)
    torch.cuda.synchronize()
    rp, ci = rp.cpu().numpy(), ci.cpu().numpy()
    for b, i in ((0, 19), (1, 10)):
        for h in range(H):
            assert list(ci[rp[b * H + h]:rp[b * H + h + 1]]) == [0, 1, 2, 3, i]


def test_select_iid_keys_is_a_valid_top_set():
    B, H, D, L = 4, 8, 128, 4096
    lens = [4096, 3000, 4000, 2049]
    r = _run("bf16", B, H, D, L, lens, 9, spread=0.0)
    kmin_o, kmax_o = oracle.block_minmax(f64(r["k"]), lens)
    same = _check_rows(r["rp"], r["ci"], f64(r["q"]), kmin_o, kmax_o, lens, 9, H, exact=False)
    print(f"iid keys: {same} of {B * H} rows equal the oracle's exactly", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_decode_rows_matches_oracle(dtype, splits):
    B, H, D, L = 4, 3, 128, 1500
    lens = [1500, 1, 777, 64]
    r = _run(dtype, B, H, D, L, lens, 6, splits=splits)
    oo, ol = oracle.attn_decode_rows(f64(r["q"]), oracle.dense_kv_blocks(f64(r["k"]), f64(r["v"])), lens,
                                     r["rp"], r["ci"])
    assert_out_close(f64(r["o"]), oo, dtype)
    assert_lse_close(f64(r["lse"]), ol, dtype)


def test_decode_rows_with_every_block_equals_layout_decode():
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 3, 4, 128, 1024
    lens = [1024, 333, 960]
    r = _run("bf16", B, H, D, L, lens, 100)
    lay = s2.s2_build_layout(s2.Pattern(H, 1, 1, tuple(range(H))), L // BLOCK, dev)  # every head dense
    o, lse = s2.s2_attn_decode(r["q"].to(dev), r["k"].to(dev), r["v"].to(dev),
                               torch.tensor(lens, dtype=torch.int32, device=dev), lay)
    torch.cuda.synchronize()
    assert np.abs(f64(o) - f64(r["o"])).max() <= 1e-2 and np.abs(f64(lse) - f64(r["lse"])).max() <= 1e-5
    oo, ol = oracle.attn_decode_rows(f64(r["q"]), oracle.dense_kv_blocks(f64(r["k"]), f64(r["v"])), lens,
                                     r["rp"], r["ci"])
    assert_out_close(f64(r["o"]), oo, "bf16")


def test_invalid_lengths_give_empty_rows_and_nan_outputs():
    B, H, D, L = 3, 2, 128, 512
    lens = [0, 513, 100]
    r = _run("bf16", B, H, D, L, lens, 3, splits=2)
    assert list(r["rp"]) == [0, 0, 0, 0, 0, 2, 4]
    oo, ol = oracle.attn_decode_rows(f64(r["q"]), oracle.dense_kv_blocks(f64(r["k"]), f64(r["v"])), lens,
                                     r["rp"], r["ci"], cache_len=L)
    assert np.isnan(oo[:2]).all() and np.isfinite(oo[2]).all()
    assert_rows_match_oracle(f64(r["o"]), f64(r["lse"]), oo, ol, "bf16")


def test_full_size_select_decode_sampled():
    """The 7B-shaped serving step: 64 sequences x 32 heads, context 32768, D = 128,
    budget 40 blocks (the static pattern's mean row), iid bf16 keys as the timing run
    uses; sampled (sequence, head) rows against the oracle."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    c = synth.WORKLOADS[5]
    B, H, L, D = c["B"], c["H"], c["N"], c["D"]
    budget = 40
    print("select full: generating 2 x 17 GB caches", flush=True)
    k = synth.randn_device(851, (B, H, L, D), "bf16", dev)
    v = synth.randn_device(852, (B, H, L, D), "bf16", dev)
    q = synth.randn_device(853, (B, H, D), "bf16", dev)
    lens = [L - 37 * b for b in range(B)]  # ragged, the longest a full context
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    print("select full: running kernels", flush=True)
    kmin, kmax = s2.s2_block_minmax(k, sl)
    rp, ci = s2.s2_select_blocks(q, kmin, kmax, sl, budget, L)
    o, lse = s2.s2_attn_decode_rows(q, k, v, sl, rp, ci, budget)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rp, ci = rp.cpu().numpy(), ci.cpu().numpy()
    assert rp[-1] == B * H * budget and np.all(np.diff(rp) == budget)
    rng = np.random.default_rng(85)
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 24), rng.integers(0, H, 24))] + [(0, 0), (B - 1, H - 1)]
    same = 0
    for b, h in pairs:
        kk = f64(k[b, h])[None, None]
        km, kx = oracle.block_minmax(kk, [lens[b]])
        n = -(-lens[b] // BLOCK)
        assert np.array_equal(f64(kmin[b, h, :n]), km[0, 0, :n]) and np.array_equal(f64(kmax[b, h, :n]), kx[0, 0, :n])
        r = b * H + h
        row = ci[rp[r]:rp[r + 1]]
        same += _check_rows(np.array([0, budget]), row, f64(q[b:b + 1, h:h + 1]), km, kx, [lens[b]], budget, 1,
                            exact=False)
        one = np.array([0, budget], dtype=np.int32)
        oo, ol = oracle.attn_decode_rows(f64(q[b:b + 1, h:h + 1]), oracle.dense_kv_blocks(kk, f64(v[b, h])[None, None]),
                                         [lens[b]], one, row)
        assert_out_close(f64(o[b, h]), oo[0, 0], "bf16", f"seq {b} head {h}")
        assert_lse_close(f64(lse[b, h]), ol[0, 0], "bf16")
    print(f"select full: {same} of {len(pairs)} sampled rows equal the oracle's exactly", flush=True)
    del k, v
    torch.cuda.empty_cache()


def test_decode_rows_skips_blocks_outside_the_visible_range():
    """A caller's CSR with entries below 0 or past the query's block reads nothing
    for them: the result equals decode over the valid entries alone."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 2, 2, 128, 512
    lens = [300, 512]  # query blocks 4 and 7
    k = _keys(91, B, H, L, D, "bf16")
    v = _keys(92, B, H, L, D, "bf16", 0.0)
    q = synth.decode_query(91, B, H, D, "bf16")
    rows = [[-7, 0, 3, 4, 5, 1 << 20], [-1, 2, 4], [0, 6, 7, 8, 12], [1 << 30, 3]]  # rows b * H + h
    valid = [[j for j in r if 0 <= j <= (lens[i // H] - 1) // BLOCK] for i, r in enumerate(rows)]
    def csr(rs):
        rp = np.concatenate([[0], np.cumsum([len(r) for r in rs])]).astype(np.int32)
        return rp, np.array([j for r in rs for j in r], dtype=np.int32)
    rp, ci = csr(rows)
    print(f"decode rows with out-of-range entries {rows}", flush=True)
    o, lse = s2.s2_attn_decode_rows(q.to(dev), k.to(dev), v.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
                                    torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), 6, splits=2)
    torch.cuda.synchronize()
    rpv, civ = csr(valid)
    oo, ol = oracle.attn_decode_rows(f64(q), oracle.dense_kv_blocks(f64(k), f64(v)), lens, rpv, civ)
    assert_out_close(f64(o), oo, "bf16")
    assert_lse_close(f64(lse), ol, "bf16")


def _to_pages(x, P, seed):
    """Contiguous [B, Hkv, L, D] -> shuffled pages [num_pages, Hkv, P, D] (unused pages
    and rows NaN) and an int32 block table [B, ceil(L / P)]."""
    B, Hkv, L, D = x.shape
    npb = -(-L // P)
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(B * npb + 5, generator=g)[:B * npb]
    pages = torch.full((B * npb + 5, Hkv, P, D), float("nan"), dtype=x.dtype)
    table = perm.reshape(B, npb).to(torch.int32)
    for b in range(B):
        for s_ in range(npb):
            rows = x[b, :, s_ * P:(s_ + 1) * P]
            pages[table[b, s_], :, :rows.shape[1]] = rows
    return pages, table


@pytest.mark.parametrize("group,P,lens,dtype,D", [
    (1, 16, [1000, 1, 513], "bf16", 128), (2, 16, [1000, 1, 513], "bf16", 128), (4, 64, [1000, 1, 513], "bf16", 128),
    (2, 64, [1000, 1, 513], "bf16", 128),
    # 4 x 2 (sequence, K/V head) units: the XCD-grouped workgroup order
    (4, 16, [1000, 1, 513, 777], "bf16", 128),
    (2, 16, [1000, 1, 513], "f32", 128), (2, 32, [1000, 1, 513], "bf16", 64), (4, 16, [1000, 1, 513, 777], "f32", 64)])
def test_paged_select_decode_matches_oracle(group, P, lens, dtype, D):
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, Hkv, L, budget = len(lens), 2, 1024, 5
    H = Hkv * group
    print(f"paged select {dtype} D={D} group={group} P={P} lens={lens}", flush=True)
    k = _keys(95, B, Hkv, L, D, dtype)
    v = _keys(96, B, Hkv, L, D, dtype, 0.0)
    q = synth.decode_query(95, B, H, D, dtype)
    kp, table = _to_pages(k, P, 97)
    vp, _ = _to_pages(v, P, 97)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    nb = L // BLOCK
    kmin, kmax = s2.s2_block_minmax_paged(kp.to(dev), table.to(dev), sl, nb)
    rp, ci = s2.s2_select_blocks(q.to(dev), kmin, kmax, sl, budget, table.shape[1] * P)
    o, lse = s2.s2_attn_decode_paged_rows(q.to(dev), kp.to(dev), vp.to(dev), table.to(dev), sl, rp, ci, budget,
                                          splits=2)
    torch.cuda.synchronize()
    km, kx = oracle.block_minmax_paged(f64(kp), table.numpy(), P, lens, nb)
    for b, n in enumerate(lens):
        nv = -(-n // BLOCK)
        assert np.array_equal(f64(kmin[b, :, :nv]), km[b, :, :nv]) and np.array_equal(f64(kmax[b, :, :nv]), kx[b, :, :nv])
    rp, ci = rp.cpu().numpy(), ci.cpu().numpy()
    assert _check_rows(rp, ci, f64(q), km, kx, lens, budget, H, group=group) == B * H
    oo, ol = oracle.attn_decode_rows(f64(q), oracle.paged_kv_blocks(f64(kp), f64(vp), table.numpy(), P, group),
                                     lens, rp, ci)
    assert_out_close(f64(o), oo, dtype)
    assert_lse_close(f64(lse), ol, dtype)


def test_paged_bounds_bad_page_gives_nan_block():
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, Hkv, D, L, P = 2, 2, 128, 512, 16
    k = _keys(98, B, Hkv, L, D, "bf16")
    kp, table = _to_pages(k, P, 99)
    table[1, 9] = kp.shape[0] + 100  # a page id outside the pool: tokens 144 .. 159 of sequence 1, block 2
    sl = torch.tensor([512, 512], dtype=torch.int32, device=dev)
    print("paged bounds with a bad page id", flush=True)
    kmin, kmax = s2.s2_block_minmax_paged(kp.to(dev), table.to(dev), sl, L // BLOCK)
    torch.cuda.synchronize()
    km, kx = f64(kmin), f64(kmax)
    assert np.isnan(km[1, :, 2]).all() and np.isnan(kx[1, :, 2]).all()
    good = np.ones(L // BLOCK, dtype=bool)
    good[2] = False
    assert np.isfinite(km[1, :, good]).all() and np.isfinite(km[0]).all()
    ref, _ = oracle.block_minmax_paged(f64(kp), table.numpy().clip(max=kp.shape[0] - 1), P, [512, 512], L // BLOCK)
    assert np.array_equal(km[0], ref[0]) and np.array_equal(km[1, :, good], ref[1, :, good])


@pytest.mark.parametrize("splits", [1, 0])
def test_paged_rows_four_heads_bad_pages_match_oracle(splits):
    """Decode over per-sequence lists with four query heads per K/V head (one
    workgroup serves a whole group): page ids outside the pool poison exactly the
    heads whose lists hold the affected blocks, as the oracle's gather does.  The
    query's own block is in every list, so sequence 0 is poisoned for every head."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    group, P, lens, D = 4, 16, [1000, 777, 513], 128
    B, Hkv, L, budget = len(lens), 2, 1024, 5
    H = Hkv * group
    print(f"paged rows, 4 heads per group, bad pages, splits={splits}", flush=True)
    k = _keys(98, B, Hkv, L, D, "bf16")
    v = _keys(99, B, Hkv, L, D, "bf16", 0.0)
    q = synth.decode_query(98, B, H, D, "bf16")
    kp, table = _to_pages(k, P, 96)
    vp, _ = _to_pages(v, P, 96)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    kmin, kmax = s2.s2_block_minmax_paged(kp.to(dev), table.to(dev), sl, L // BLOCK)  # bounds of the clean pool
    rp, ci = s2.s2_select_blocks(q.to(dev), kmin, kmax, sl, budget, table.shape[1] * P)
    bad = table.clone()
    bad[0, 999 // P] = kp.shape[0] + 7  # the query's page of sequence 0: outside the pool
    bad[1, 0] = -3                      # tokens 0..15 of sequence 1: block 0, if a list keeps it
    o, lse = s2.s2_attn_decode_paged_rows(q.to(dev), kp.to(dev), vp.to(dev), bad.to(dev), sl, rp, ci, budget,
                                          splits=splits)
    torch.cuda.synchronize()
    oo, ol = oracle.attn_decode_rows(f64(q), oracle.paged_kv_blocks(f64(kp), f64(vp), bad.numpy(), P, group),
                                     lens, rp.cpu().numpy(), ci.cpu().numpy())
    assert np.isnan(oo[0]).all() and np.isfinite(oo[2]).all()
    assert_rows_match_oracle(f64(o), f64(lse), oo, ol, "bf16", f"splits={splits}")
