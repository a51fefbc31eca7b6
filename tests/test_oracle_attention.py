"""Pins of the oracle's forward and decode attention (CPU only).

Each pin comes from outside the oracle's own code: a library routine
(torch's scaled_dot_product_attention in float64 for the all-blocks special
case), closed forms (V = 1, Q = 0, the first row), invariants (inactive blocks
do not matter, the two forward modes agree, decode equals the forward's last
row) and the associativity of softmax merging (Lean Attention abstract, on the
SampleAttention page's related-papers list).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _layout(H, N, W, S, dense=None):
    return oracle.build_layout(H, N // 64, W, S, dense)


def test_all_blocks_equals_sdpa_causal():
    B, H, N, D = 2, 3, 256, 64
    q, k, v = (_rand((B, H, N, D), s) for s in (1, 2, 3))
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    # three different ways of making every causal block active
    for W, S, dense in [(1, 1, None), (N // 64, 5, None), (1, 7, [1, 1, 1])]:
        rp, ci = _layout(H, N, W, S, dense)
        o, lse = oracle.attn_fwd_dense(q, k, v, rp, ci, N // 64)
        assert np.max(np.abs(o - sdpa)) < 1e-12
        ob, lseb = oracle.attn_fwd_blocks(q, k, v, rp, ci, N // 64)
        assert np.max(np.abs(ob - sdpa)) < 1e-12
        # LSE of the causal softmax, from the library's own scores
        s = np.einsum("bhqd,bhkd->bhqk", q, k) / math.sqrt(D)
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        want = np.log(np.sum(np.exp(s - s.max(-1, keepdims=True)), -1)) + s.max(-1)
        assert np.max(np.abs(lse - want)) < 1e-10


def test_sparse_differs_from_dense():
    """A sparse pattern must not reproduce dense attention (guards a no-op mask)."""
    B, H, N, D = 1, 4, 512, 64
    q, k, v = (_rand((B, H, N, D), s) for s in (4, 5, 6))
    rp, ci = _layout(H, N, 2, 4)
    o, _ = oracle.attn_fwd_dense(q, k, v, rp, ci, N // 64)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    assert np.max(np.abs(o - sdpa)) > 1e-2


@pytest.mark.parametrize("mode", ["dense", "blocks"])
def test_v_ones_gives_ones(mode):
    B, H, N, D = 1, 4, 512, 64
    q, k = _rand((B, H, N, D), 7), _rand((B, H, N, D), 8)
    v = np.ones((B, H, N, D))
    rp, ci = _layout(H, N, 2, 4)
    fn = oracle.attn_fwd_dense if mode == "dense" else oracle.attn_fwd_blocks
    o, _ = fn(q, k, v, rp, ci, N // 64)
    assert np.max(np.abs(o - 1.0)) < 1e-13


def _active_keys_by_counting(rp, ci, nqb, h, qpos):
    """Token positions visible to query qpos, listed from the CSR row directly."""
    i = qpos // 64
    r = h * nqb + i
    keys = []
    for j in ci[rp[r]:rp[r + 1]]:
        keys.extend(t for t in range(j * 64, (j + 1) * 64) if t <= qpos)
    return keys


@pytest.mark.parametrize("mode", ["dense", "blocks"])
def test_q_zero_gives_mean_of_active_values(mode):
    B, H, N, D = 1, 4, 512, 64
    q = np.zeros((B, H, N, D))
    k, v = _rand((B, H, N, D), 9), _rand((B, H, N, D), 10)
    rp, ci = _layout(H, N, 2, 4)
    fn = oracle.attn_fwd_dense if mode == "dense" else oracle.attn_fwd_blocks
    o, lse = fn(q, k, v, rp, ci, N // 64)
    for h in range(H):
        for qpos in list(range(0, N, 37)) + [N - 1, 63, 64, 65]:
            keys = _active_keys_by_counting(rp, ci, N // 64, h, qpos)
            assert np.max(np.abs(o[0, h, qpos] - v[0, h, keys].mean(0))) < 1e-13
            assert abs(lse[0, h, qpos] - math.log(len(keys))) < 1e-13


def test_first_row_is_first_value():
    B, H, N, D = 2, 4, 256, 128
    q, k, v = (_rand((B, H, N, D), s) for s in (11, 12, 13))
    rp, ci = _layout(H, N, 2, 3)
    for fn in (oracle.attn_fwd_dense, oracle.attn_fwd_blocks):
        o, lse = fn(q, k, v, rp, ci, N // 64)
        assert np.array_equal(o[:, :, 0], v[:, :, 0])
        want = np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]) / math.sqrt(D)
        assert np.max(np.abs(lse[:, :, 0] - want)) < 1e-13


@pytest.mark.parametrize("H,N,W,S,dense", [
    (4, 512, 2, 4, None),
    (4, 2048, 8, 16, [1, 0, 0, 0]),
    (3, 1024, 3, 5, [0, 0, 1]),
])
def test_dense_mode_equals_block_mode(H, N, W, S, dense):
    B, D = 1, 64
    q, k, v = (_rand((B, H, N, D), s) for s in (14, 15, 16))
    rp, ci = _layout(H, N, W, S, dense)
    o1, l1 = oracle.attn_fwd_dense(q, k, v, rp, ci, N // 64)
    o2, l2 = oracle.attn_fwd_blocks(q, k, v, rp, ci, N // 64)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


def test_inactive_blocks_do_not_matter():
    B, H, N, D = 1, 4, 512, 64
    q, k, v = (_rand((B, H, N, D), s) for s in (17, 18, 19))
    rp, ci = _layout(H, N, 2, 4)
    o, lse = oracle.attn_fwd_blocks(q, k, v, rp, ci, N // 64)
    k2, v2 = k.copy(), v.copy()
    h = 1
    nqb = N // 64
    inactive_for_last = set(range(nqb)) - set(oracle.row_blocks(rp, ci, nqb, h, nqb - 1).tolist())
    for j in inactive_for_last:
        k2[0, h, j * 64:(j + 1) * 64] = 1e4
        v2[0, h, j * 64:(j + 1) * 64] = -1e4
    o2, lse2 = oracle.attn_fwd_blocks(k=k2, v=v2, q=q, row_ptr=rp, col_idx=ci, num_q_blocks=nqb,
                                      heads=[h], q_blocks=[nqb - 1])
    sl = slice((nqb - 1) * 64, nqb * 64)
    assert np.array_equal(o2[0, h, sl], o[0, h, sl])
    assert np.array_equal(lse2[0, h, sl], lse[0, h, sl])
    # and perturbing an active block does change the result
    j = int(oracle.row_blocks(rp, ci, nqb, h, nqb - 1)[0])
    k2[0, h, j * 64] += 1.0
    o3, _ = oracle.attn_fwd_blocks(q, k2, v2, rp, ci, nqb, heads=[h], q_blocks=[nqb - 1])
    assert not np.array_equal(o3[0, h, sl], o[0, h, sl])


@pytest.mark.parametrize("L", [512, 511, 449, 1, 64, 65])
def test_decode_equals_forward_row(L):
    B, H, D = 2, 4, 64
    N = ((L + 63) // 64) * 64
    q, k, v = (_rand((B, H, N, D), s) for s in (20, 21, 22))
    rp, ci = _layout(H, 512, 2, 4)          # layout for the longest context; rows are prefixes
    nqb = 512 // 64
    of, lf = oracle.attn_fwd_blocks(q, k, v, rp, ci, nqb, q_blocks=[(L - 1) // 64])
    kc = np.concatenate([k, np.full((B, H, 512 - N, D), np.nan)], axis=2)
    vc = np.concatenate([v, np.full((B, H, 512 - N, D), np.nan)], axis=2)
    kc[:, :, L:] = np.nan                    # tokens beyond the context must never be read
    vc[:, :, L:] = np.nan
    od, ld = oracle.attn_decode(q[:, :, L - 1], oracle.dense_kv_blocks(kc, vc), [L] * B, rp, ci, nqb)
    assert np.max(np.abs(od - of[:, :, L - 1])) < 1e-12
    assert np.max(np.abs(ld - lf[:, :, L - 1])) < 1e-12


def test_logsumexp_merge_of_partitions():
    """Partial results over any partition of the keys merge to the unsplit result."""
    rng = np.random.default_rng(23)
    D, n = 128, 700
    qv, K, V = rng.standard_normal(D), rng.standard_normal((n, D)) * 3, rng.standard_normal((n, D))
    o, lse = oracle.attend_keys(qv, K, V, 1 / math.sqrt(D))
    for cuts in ([350], [1, 2, 699], [64, 128, 500, 640]):
        parts = np.split(np.arange(n), cuts)
        po, pl = zip(*(oracle.attend_keys(qv, K[p], V[p], 1 / math.sqrt(D)) for p in parts))
        pl = np.array(pl)
        m = pl.max()
        total = m + math.log(np.exp(pl - m).sum())
        merged = sum(np.exp(li - total) * oi for li, oi in zip(pl, po))
        assert abs(total - lse) < 1e-12
        assert np.max(np.abs(merged - o)) < 1e-12


def test_tiny_workload_inputs_deterministic():
    c = synth.WORKLOADS[1]
    q1, = synth.fwd_inputs(1, c["B"], c["H"], c["N"], c["D"], c["dtype"], which=(synth.TENSOR_Q,))
    q2, = synth.fwd_inputs(1, c["B"], c["H"], c["N"], c["D"], c["dtype"], which=(synth.TENSOR_Q,))
    assert torch.equal(q1, q2)
    assert abs(float(q1.mean())) < 0.02 and abs(float(q1.std()) - 1) < 0.02


def test_planted_scale_error_is_caught(monkeypatch):
    """Dropping the 1/sqrt(D) scale must fail the SDPA pin."""
    orig = oracle.s2_oracle.attn_fwd_dense

    def wrong(q, k, v, rp, ci, nqb, scale=None):
        return orig(q, k, v, rp, ci, nqb, scale=1.0)
    monkeypatch.setattr(oracle, "attn_fwd_dense", wrong)
    with pytest.raises(AssertionError):
        test_all_blocks_equals_sdpa_causal()


def test_planted_strict_causality_is_caught(monkeypatch):
    """Reading causality as t < q (a query not seeing itself) must fail the SDPA pin."""
    orig_mask = oracle.s2_oracle.token_mask

    def wrong(rp, ci, nqb, h, N):
        m = orig_mask(rp, ci, nqb, h, N)
        m[np.arange(1, N), np.arange(1, N)] = False      # row 0 keeps its only key
        return m
    monkeypatch.setattr(oracle.s2_oracle, "token_mask", wrong)
    with pytest.raises(AssertionError):
        test_all_blocks_equals_sdpa_causal()


def test_decode_invalid_lengths_give_nan_rows_and_read_nothing():
    """Reading 18 of the API: a length outside [1, cache length] has no query
    position; its row is NaN (output and logsumexp) and no block is requested, while
    the valid rows are unchanged."""
    B, H, D, L = 4, 3, 16, 256
    nqb = L // 64
    rp, ci = _layout(H, L, 2, 3)
    q = _rand((B, H, D), 30)
    kc, vc = _rand((B, H, L, D), 31), _rand((B, H, L, D), 32)
    seq = [0, 200, L + 1, -5]
    requested = set()
    base = oracle.dense_kv_blocks(kc, vc)

    def gather(b, h, j):
        requested.add(b)
        return base(b, h, j)
    o, lse = oracle.attn_decode(q, gather, seq, rp, ci, nqb)
    assert requested == {1}
    for b in (0, 2, 3):
        assert np.isnan(o[b]).all() and np.isnan(lse[b]).all()
    ref, lref = oracle.attn_decode(q[1:2], oracle.dense_kv_blocks(kc[1:2], vc[1:2]), [200], rp, ci, nqb)
    assert np.array_equal(o[1], ref[0]) and np.array_equal(lse[1], lref[0])
    # a shorter cache than the layout covers: a length past it is invalid too
    o2, _ = oracle.attn_decode(q, base, [200, 200, 201, 1], rp, ci, nqb, cache_len=200)
    assert np.isfinite(o2[[0, 1, 3]]).all() and np.isnan(o2[2]).all()
    # decode over explicit rows follows the same rule
    rows_rp = np.array([0] + [1] * (B * H), dtype=np.int32)
    rows_rp[1:] = np.arange(1, B * H + 1)
    rows_ci = np.zeros(B * H, dtype=np.int32)
    o3, l3 = oracle.attn_decode_rows(q, base, [0, 1, L + 1, 64], rows_rp, rows_ci, cache_len=L)
    assert np.isnan(o3[0]).all() and np.isnan(o3[2]).all() and np.isnan(l3[[0, 2]]).all()
    assert np.isfinite(o3[1]).all() and np.isfinite(o3[3]).all()
    # row of length 1: the only key is token 0, so the output is V[0] exactly
    assert np.allclose(o3[1], vc[1, :, 0], atol=1e-12)
