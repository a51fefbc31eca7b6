"""GPU serving decode (paged K/V cache, grouped K/V heads) against the fp64 oracle.

The page pools are built by scattering a contiguous cache into shuffled pages;
every page and page row no sequence uses holds NaN, so a read outside the
table shows up as a NaN output."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import assert_lse_close, assert_out_close, assert_rows_match_oracle, device, f64

pytestmark = pytest.mark.gpu


def _pool(kc: torch.Tensor, vc: torch.Tensor, seq_lens, P: int, rng, spare: int = 5):
    """Scatter caches [B, Hkv, L, D] into a shuffled page pool [n, Hkv, P, D] (NaN elsewhere)."""
    B, Hkv, L, D = kc.shape
    npb = -(-L // P)
    n = B * npb + spare
    perm = rng.permutation(n)
    kp = torch.full((n, Hkv, P, D), float("nan"), dtype=kc.dtype)
    vp = torch.full((n, Hkv, P, D), float("nan"), dtype=kc.dtype)
    # 3 spare columns: the kernels get a [B, npb] slice whose row stride is npb + 3;
    # entries past a sequence's last page are never read
    table = np.full((B, npb + 3), -1, dtype=np.int32)
    for b in range(B):
        used = -(-int(seq_lens[b]) // P) if 1 <= seq_lens[b] <= L else 0
        for s in range(used):
            page = int(perm[b * npb + s])
            table[b, s] = page
            t0, t1 = s * P, min(int(seq_lens[b]), (s + 1) * P)
            kp[page, :, : t1 - t0] = kc[b, :, t0:t1]
            vp[page, :, : t1 - t0] = vc[b, :, t0:t1]
    return kp, vp, table


def _case(dtype, B, H, Hkv, D, L, W, S, dense, seq_lens, P, splits, seed=31, table_edit=None, all_pairs=False):
    import head_heterogeneous_block_amd as s2
    dev = device()
    nqb = -(-L // 64)
    print(f"paged decode {dtype} B={B} H={H} Hkv={Hkv} D={D} L={L} P={P} seq={seq_lens} splits={splits}",
          flush=True)
    rng = np.random.default_rng(seed)
    q = synth.decode_query(seed, B, H, D, dtype)
    kc = synth.full_cache(seed, synth.TENSOR_K, B, Hkv, L, D, dtype)
    vc = synth.full_cache(seed, synth.TENSOR_V, B, Hkv, L, D, dtype)
    kp, vp, table = _pool(kc, vc, seq_lens, P, rng)
    if table_edit:
        table_edit(table, kp.shape[0])
    lay = s2.s2_build_layout(s2.Pattern(H, W, S, tuple(dense)), nqb, dev)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=dev)
    npb = -(-L // P)
    o, lse = s2.s2_attn_decode_paged(q.to(dev), kp.to(dev), vp.to(dev),
                                     torch.from_numpy(table).to(dev)[:, :npb], sl, lay, splits=splits)
    torch.cuda.synchronize()
    rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, dense))
    gather = oracle.paged_kv_blocks(f64(kp), f64(vp), table, P, H // Hkv)
    valid = [b for b in range(B) if 1 <= seq_lens[b] <= L]
    pairs = [(b, h) for b in (range(B) if all_pairs else valid) for h in range(H)]
    oo, ol = oracle.attn_decode(f64(q), gather, seq_lens, rp, ci, nqb, pairs=pairs, cache_len=L)
    return o, lse, oo, ol, valid


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hkv,P,splits", [(8, 64, 1), (4, 16, 3), (2, 256, 0), (1, 32, 2), (2, 16, 1),
                                          (8, 128, 0)])
def test_paged_small(dtype, Hkv, P, splits):
    o, lse, oo, ol, valid = _case(dtype, 3, 8, Hkv, 128, 1000, 2, 4, (2,), [1000, 1, 517], P, splits)
    assert_out_close(f64(o), oo, dtype)
    assert_lse_close(f64(lse), ol, dtype)


@pytest.mark.parametrize("Hkv", [3, 1])
def test_paged_head_dim_64_and_uneven_groups(Hkv):
    # 12 query heads: groups of 4 or 12, served two heads at a time
    o, lse, oo, ol, _ = _case("bf16", 2, 12, Hkv, 64, 640, 3, 5, (7,), [640, 130], 64, 0)
    assert_out_close(f64(o), oo, "bf16")
    assert_lse_close(f64(lse), ol, "bf16")


def test_paged_odd_group():
    # 12 query heads over 4 K/V heads: groups of 3, served one head at a time
    o, lse, oo, ol, _ = _case("bf16", 2, 12, 4, 128, 700, 2, 3, (), [700, 65], 16, 2)
    assert_out_close(f64(o), oo, "bf16")
    assert_lse_close(f64(lse), ol, "bf16")


def test_paged_matches_contiguous_decode():
    """One K/V head per query head, 64-token pages in order: the contiguous decode's input."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, D, L = 2, 4, 128, 1024
    q = synth.decode_query(32, B, H, D, "f32").to(dev)
    kc = synth.full_cache(32, synth.TENSOR_K, B, H, L, D, "f32").to(dev)
    vc = synth.full_cache(32, synth.TENSOR_V, B, H, L, D, "f32").to(dev)
    lay = s2.s2_build_layout(s2.Pattern(H, 3, 4, (1,)), L // 64, dev)
    sl = torch.tensor([1024, 700], dtype=torch.int32, device=dev)
    # page p = (b, s): the pool is the contiguous cache viewed as [B * 16, H, 64, D]
    kp = kc.view(B, H, L // 64, 64, D).permute(0, 2, 1, 3, 4).reshape(B * L // 64, H, 64, D)
    vp = vc.view(B, H, L // 64, 64, D).permute(0, 2, 1, 3, 4).reshape(B * L // 64, H, 64, D)
    table = torch.arange(B * L // 64, dtype=torch.int32, device=dev).view(B, L // 64)
    o1, l1 = s2.s2_attn_decode(q, kc, vc, sl, lay, splits=3)
    o2, l2 = s2.s2_attn_decode_paged(q, kp, vp, table, sl, lay, splits=3)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 1e-6
    assert (l1 - l2).abs().max().item() <= 1e-6


def test_paged_split_invariance_and_workspace_reuse():
    import head_heterogeneous_block_amd as s2
    dev = device()
    B, H, Hkv, D, L, P = 2, 8, 2, 128, 2560, 32
    rng = np.random.default_rng(33)
    q = synth.decode_query(33, B, H, D, "f32").to(dev)
    kc = synth.full_cache(33, synth.TENSOR_K, B, Hkv, L, D, "f32")
    vc = synth.full_cache(33, synth.TENSOR_V, B, Hkv, L, D, "f32")
    seq = [2560, 2000]
    kp, vp, table = _pool(kc, vc, seq, P, rng)
    kp, vp, table = kp.to(dev), vp.to(dev), torch.from_numpy(table).to(dev)[:, :L // P]
    lay = s2.s2_build_layout(s2.Pattern(H, 8, 16), L // 64, dev)
    sl = torch.tensor(seq, dtype=torch.int32, device=dev)
    ref = s2.s2_attn_decode_paged(q, kp, vp, table, sl, lay, splits=1)
    for sp in (2, 5, 40):
        ws = torch.full((s2.s2_attn_decode_paged_workspace(lay, B, Hkv, D, sp),), 255, dtype=torch.uint8,
                        device=dev)  # garbage: the workspace needs no initialisation
        for rep in range(3):
            o, l = s2.s2_attn_decode_paged(q, kp, vp, table, sl, lay, splits=sp, workspace=ws)
            torch.cuda.synchronize()
            assert (o - ref[0]).abs().max().item() <= 1e-6, (sp, rep)
            assert (l - ref[1]).abs().max().item() <= 1e-6, (sp, rep)


@pytest.mark.parametrize("splits", [1, 2, 0])
def test_paged_invalid_lengths_and_bad_pages(splits):
    """Invalid lengths and page ids outside the pool give NaN rows, as the oracle's
    gather does, with one split (the split kernel writes the result), several (the
    merge launch writes it) and the automatic count."""
    L = 1024

    def corrupt(table, n):
        table[0, 1] = n + 7   # tokens 64..127 of sequence 0: key block 1
        table[1, 0] = -3      # tokens 0..63 of sequence 1: key block 0

    seq = [1024, 1024, 0, L + 1]
    o, lse, oo, ol, valid = _case("bf16", 4, 4, 2, 128, L, 1, 4, (), seq, 64, splits, table_edit=corrupt,
                                  all_pairs=True)
    got, gl = f64(o), f64(lse)
    assert np.isnan(oo[2]).all() and np.isnan(oo[3]).all()             # invalid lengths
    poisoned = sum(int(np.isnan(oo[b, h]).any()) for b in (0, 1) for h in range(4))
    assert 0 < poisoned < 8                   # the bad pages poison some heads, not all
    assert_rows_match_oracle(got, gl, oo, ol, "bf16", f"splits={splits}")


def test_paged_full_size_gqa_sampled():
    """7B-shaped serving decode: 64 sequences of ragged length up to 32768, 32 query
    heads over 8 K/V heads, 16-token pages in a shuffled pool; sampled heads."""
    import head_heterogeneous_block_amd as s2
    dev = device()
    c = synth.WORKLOADS[5]
    B, H, L, D = c["B"], c["H"], c["N"], c["D"]
    Hkv, P = 8, 16
    nqb = L // 64
    rng = np.random.default_rng(34)
    seq = rng.integers(L // 2, L + 1, size=B).astype(np.int32)
    seq[0] = L
    npb = L // P
    n = B * npb
    print("paged full: filling 2 x 4.3 GB page pools", flush=True)
    kp = synth.randn_device(341, (n, Hkv, P, D), "bf16", dev)
    vp = synth.randn_device(342, (n, Hkv, P, D), "bf16", dev)
    table = rng.permutation(n).astype(np.int32).reshape(B, npb)
    lay = s2.s2_build_layout(s2.Pattern(H, c["W"], c["S"], c["dense"]), nqb, dev)
    q = synth.decode_query(34, B, H, D, "bf16")
    print("paged full: running kernel", flush=True)
    o, lse = s2.s2_attn_decode_paged(q.to(dev), kp, vp, torch.from_numpy(table).to(dev),
                                     torch.from_numpy(seq).to(dev), lay)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rp, ci = oracle.build_layout(H, nqb, c["W"], c["S"], synth.dense_flags(H, c["dense"]))
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 24), rng.integers(0, H, 24))]
    pairs += [(0, 0), (B - 1, H - 1)]

    class Pages:
        """The pool pages the sampled pairs read, copied to the host on first use."""

        def __init__(self, pool):
            self.pool, self.cache, self.shape = pool, {}, tuple(pool.shape)

        def __getitem__(self, idx):
            page, kvh, row = idx
            if page not in self.cache:
                self.cache[page] = f64(self.pool[page])
            return self.cache[page][kvh, row]

    gather = oracle.paged_kv_blocks(Pages(kp), Pages(vp), table, P, H // Hkv)
    oo, ol = oracle.attn_decode(f64(q), gather, seq, rp, ci, nqb, pairs=pairs)
    got_o, got_l = f64(o), f64(lse)
    for b, h in pairs:
        assert_out_close(got_o[b, h], oo[b, h], "bf16", f"seq {b} head {h}")
        assert_lse_close(got_l[b, h], ol[b, h], "bf16")
    del kp, vp
    torch.cuda.empty_cache()
