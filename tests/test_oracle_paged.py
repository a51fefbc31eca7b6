"""Pins of the serving-decode gather (paged KV cache, grouped KV heads).

paged_kv_blocks only decides which cache row a (sequence, query head, token)
reads; the attention on top is oracle.attn_decode, pinned elsewhere.  These
tests fix the gather against the contiguous cache it must reproduce, against
the textbook definition of grouped-query attention (every query head of a group
reading the same K/V, i.e. K/V repeated per query head), and against
invariances of paging (page size, page placement, shared pages)."""
import numpy as np
import pytest

import oracle

BLOCK = oracle.BLOCK


def _setup(B=3, H=8, Hkv=2, L=640, D=16, W=2, S=3, dense=(), seed=0):
    rng = np.random.default_rng(seed)
    nqb = -(-L // BLOCK)
    rp, ci = oracle.build_layout(H, nqb, W, S, [1 if h in dense else 0 for h in range(H)])
    kc = rng.standard_normal((B, Hkv, L, D))
    vc = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, H, D))
    lens = rng.integers(1, L + 1, size=B)
    lens[0] = L
    return rng, rp, ci, nqb, kc, vc, q, lens


def _page(kc, vc, P, rng, spare=3):
    """Scatter contiguous caches [B, Hkv, L, D] into a shuffled page pool."""
    B, Hkv, L, D = kc.shape
    npb = -(-L // P)
    n = B * npb + spare
    perm = rng.permutation(n)
    kp = rng.standard_normal((n, Hkv, P, D)) * 100.0  # junk in unused rows
    vp = rng.standard_normal((n, Hkv, P, D)) * 100.0
    table = np.zeros((B, npb), dtype=np.int32)
    for b in range(B):
        for s in range(npb):
            page = perm[b * npb + s]
            table[b, s] = page
            t0, t1 = s * P, min(L, (s + 1) * P)
            kp[page, :, : t1 - t0] = kc[b, :, t0:t1]
            vp[page, :, : t1 - t0] = vc[b, :, t0:t1]
    return kp, vp, table


def _repeat_heads(x, group):
    return np.repeat(x, group, axis=1)


@pytest.mark.parametrize("P", [16, 64, 256])
def test_paged_one_kv_head_per_query_head_equals_contiguous(P):
    rng, rp, ci, nqb, kc, vc, q, lens = _setup(Hkv=8)
    kp, vp, table = _page(kc, vc, P, rng)
    ref = oracle.attn_decode(q, oracle.dense_kv_blocks(kc, vc), lens, rp, ci, nqb)
    got = oracle.attn_decode(q, oracle.paged_kv_blocks(kp, vp, table, P, 1), lens, rp, ci, nqb)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("Hkv", [1, 2, 4])
def test_grouped_kv_equals_kv_repeated_per_query_head(Hkv):
    # grouped-query attention by definition: query head h attends with K/V head
    # h // (H / Hkv); with the K/V heads repeated that many times it is plain
    # multi-head attention (Hkv = 1: multi-query attention)
    H = 8
    rng, rp, ci, nqb, kc, vc, q, lens = _setup(H=H, Hkv=Hkv, dense=(5,))
    kp, vp, table = _page(kc, vc, 64, rng)
    g = H // Hkv
    ref = oracle.attn_decode(q, oracle.dense_kv_blocks(_repeat_heads(kc, g), _repeat_heads(vc, g)),
                             lens, rp, ci, nqb)
    got = oracle.attn_decode(q, oracle.paged_kv_blocks(kp, vp, table, 64, g), lens, rp, ci, nqb)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


def test_page_size_does_not_change_the_result():
    rng, rp, ci, nqb, kc, vc, q, lens = _setup(L=1000)
    outs = []
    for P in (16, 32, 64, 128, 256):
        kp, vp, table = _page(kc, vc, P, np.random.default_rng(P))
        outs.append(oracle.attn_decode(q, oracle.paged_kv_blocks(kp, vp, table, P, 4), lens, rp, ci, nqb))
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])


def test_shared_prefix_pages():
    # two sequences whose tables point at the same pages read the same keys
    rng, rp, ci, nqb, kc, vc, q, lens = _setup(B=2, L=512)
    kp, vp, table = _page(kc, vc, 64, rng)
    table[1] = table[0]
    q[1] = q[0]
    o, lse = oracle.attn_decode(q, oracle.paged_kv_blocks(kp, vp, table, 64, 4), [300, 300], rp, ci, nqb)
    assert np.array_equal(o[0], o[1]) and np.array_equal(lse[0], lse[1])
    o2, _ = oracle.attn_decode(q, oracle.paged_kv_blocks(kp, vp, table, 64, 4), [300, 200], rp, ci, nqb)
    assert not np.array_equal(o2[0], o2[1])


def test_bad_page_poisons_only_rows_that_read_it():
    rng, rp, ci, nqb, kc, vc, q, lens = _setup(B=2, H=4, Hkv=2, L=1024, W=1, S=4)
    kp, vp, table = _page(kc, vc, 64, rng, spare=0)
    n = kp.shape[0]
    lens = np.array([1024, 1024])
    table[0, 1] = n + 5   # block 1 of sequence 0: read only by heads whose stride hits 1
    o, lse = oracle.attn_decode(q, oracle.paged_kv_blocks(kp, vp, table, 64, 2), lens, rp, ci, nqb)
    i = (1024 - 1) // BLOCK
    readers = [1 in oracle.row_blocks(rp, ci, nqb, h, i) for h in range(4)]
    assert any(readers) and not all(readers)
    for h in range(4):
        reads = 1 in oracle.row_blocks(rp, ci, nqb, h, i)
        assert np.isnan(o[0, h]).all() == reads and np.isnan(lse[0, h]) == reads
    assert np.isfinite(o[1]).all()


def test_planted_gather_mistakes_are_caught():
    rng, rp, ci, nqb, kc, vc, q, lens = _setup(H=8, Hkv=2)
    kp, vp, table = _page(kc, vc, 16, rng)
    ref = oracle.attn_decode(q, oracle.dense_kv_blocks(_repeat_heads(kc, 4), _repeat_heads(vc, 4)),
                             lens, rp, ci, nqb)[0]

    def gather(head_of, row_of):
        def get(b, h, j):
            kb = np.full((BLOCK, kc.shape[3]), np.nan)
            vb = kb.copy()
            for r in range(BLOCK):
                t = j * BLOCK + r
                if t // 16 < table.shape[1]:
                    pg = table[b, t // 16]
                    kb[r] = kp[pg, head_of(h), row_of(t)]
                    vb[r] = vp[pg, head_of(h), row_of(t)]
            return kb, vb
        return get
    good = oracle.attn_decode(q, gather(lambda h: h // 4, lambda t: t % 16), lens, rp, ci, nqb)[0]
    assert np.array_equal(good, ref)
    for wrong in (gather(lambda h: h % 2, lambda t: t % 16),         # interleaved head groups
                  gather(lambda h: h // 4, lambda t: (t + 1) % 16)):  # page row off by one
        bad = oracle.attn_decode(q, wrong, lens, rp, ci, nqb)[0]
        assert not np.allclose(bad, ref, atol=1e-6, equal_nan=True)
