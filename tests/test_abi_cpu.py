"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, sizes layouts in closed form identically to the oracle, and rejects
bad arguments on the host before any launch (fake device addresses are fine
because validation returns first)."""
import ctypes
import os
import random
import re

import pytest

import oracle
import synth

s2 = pytest.importorskip("head_heterogeneous_block_amd")
from head_heterogeneous_block_amd import s2attn as B  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "s2attn.h")
FAKE = 0x7f0000000000  # 256-byte aligned placeholder address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B._LIB_PATH):
        pytest.skip("libs2attn.so not built")
    return B.library()


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(s2_[a-z_]+)\s*\(", text))
    assert declared == set(B.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.s2_abi_version() == 2


def test_layout_nnz_matches_oracle_random(lib):
    rng = random.Random(5)
    for _ in range(60):
        H = rng.randint(1, 9)
        nqb = rng.randint(1, 70)
        W = rng.randint(1, 12)
        S = rng.randint(1, 20)
        dense = [rng.random() < 0.2 for _ in range(H)]
        rp, ci = oracle.build_layout(H, nqb, W, S, dense)
        pat = B.Pattern(H, W, S, tuple(h for h in range(H) if dense[h]))
        assert B.s2_layout_nnz(pat, nqb) == int(rp[-1])


@pytest.mark.parametrize("w", [1, 2, 3, 4, 5])
def test_layout_nnz_workloads(lib, w):
    c = synth.WORKLOADS[w]
    n = B.s2_layout_nnz(B.Pattern(c["H"], c["W"], c["S"], c["dense"]), c["N"] // 64)
    assert n == {1: 81, 2: 37157, 3: 384696, 4: 11115950, 5: 384696}[w]


def _pat(H=4, bs=64, W=2, S=4):
    return B._Pattern(H, bs, W, S, None)


def _status(fn, *args):
    st = fn(*args)
    return st, B.library().s2_last_error().decode()


@pytest.mark.parametrize("pat,nqb,status", [
    (_pat(W=0), 8, B.S2_EINVAL),
    (_pat(S=0), 8, B.S2_EINVAL),
    (_pat(H=0), 8, B.S2_EINVAL),
    (_pat(bs=32), 8, B.S2_EUNSUPPORTED),
    (_pat(), 0, B.S2_EINVAL),
])
def test_build_layout_rejects(lib, pat, nqb, status):
    st, msg = _status(lib.s2_build_layout, ctypes.byref(pat), nqb, FAKE, FAKE, 1 << 20, None)
    assert st == status and msg


def test_build_layout_capacity(lib):
    pat = _pat()
    st, msg = _status(lib.s2_build_layout, ctypes.byref(pat), 8, FAKE, FAKE, 80, None)
    assert st == B.S2_ECAPACITY and "81" in msg
    st, _ = _status(lib.s2_build_layout, ctypes.byref(pat), 8, None, FAKE, 100, None)
    assert st == B.S2_EINVAL


def _layout(H=4, nqb=8, nnz=81):
    return B._Layout(H, nqb, 64, nnz, FAKE, FAKE)


def _st(*v):
    return (ctypes.c_int64 * len(v))(*v)


def _fwd(lib, layout=None, dtype=B.S2_BF16, Bn=1, N=512, D=128, q=FAKE, qs=None, o=FAKE, ws=FAKE,
         ws_bytes=1024):
    layout = layout or _layout()
    s = _st(4 * N * D, N * D, D, 1)
    return _status(lib.s2_attn_fwd, ctypes.byref(layout), dtype, Bn, N, D, q, qs or s, FAKE, s, FAKE,
                   s, o, s, None, ws, ws_bytes, 0.0, None)


def test_fwd_workspace_size(lib):
    n = ctypes.c_size_t(0)
    assert lib.s2_attn_fwd_workspace(ctypes.byref(n)) == B.S2_OK
    assert n.value == 8 * 128                                       # one 128-byte line per XCD queue
    assert lib.s2_attn_fwd_workspace(None) == B.S2_EINVAL
    assert B.s2_attn_fwd_workspace() == 1024


def test_fwd_rejects(lib):
    assert _fwd(lib, N=500)[0] == B.S2_EINVAL                      # N not a multiple of 64
    assert _fwd(lib, D=96)[0] == B.S2_EUNSUPPORTED                  # head dim
    assert _fwd(lib, N=1024)[0] == B.S2_EINVAL                      # layout has 8 blocks, N/64 = 16
    assert _fwd(lib, q=None)[0] == B.S2_EINVAL
    assert _fwd(lib, q=FAKE + 2)[0] == B.S2_EINVAL                  # misaligned
    assert _fwd(lib, qs=_st(4 * 512 * 128, 512 * 128, 128, 2))[0] == B.S2_EINVAL  # D stride
    assert _fwd(lib, qs=_st(4 * 512 * 128, 512 * 128, 100, 1))[0] == B.S2_EINVAL  # row stride % 8
    assert _fwd(lib, dtype=7)[0] == B.S2_EINVAL
    assert _fwd(lib, Bn=0)[0] == B.S2_EINVAL
    assert _fwd(lib, layout=_layout(nnz=1 << 31))[0] == B.S2_EUNSUPPORTED
    bad = B._Layout(4, 8, 32, 81, FAKE, FAKE)
    assert _fwd(lib, layout=bad)[0] == B.S2_EUNSUPPORTED
    st, msg = _fwd(lib, N=500)
    assert "multiple of 64" in msg
    assert _fwd(lib, ws=None)[0] == B.S2_EINVAL                     # workspace missing
    assert _fwd(lib, ws=FAKE + 4)[0] == B.S2_EINVAL                 # not 8-byte aligned
    st, msg = _fwd(lib, ws_bytes=1023)
    assert st == B.S2_ECAPACITY and "1024" in msg


def _dec(lib, ws_bytes=1 << 30, cache_len=512, seq=FAKE, splits=0, ws=FAKE, D=128):
    ly = _layout()
    q = _st(4 * D, D, 1)
    c = _st(4 * cache_len * D, cache_len * D, D, 1)
    return _status(lib.s2_attn_decode, ctypes.byref(ly), B.S2_BF16, 1, D, FAKE, q, FAKE, c, FAKE, c,
                   seq, cache_len, FAKE, q, None, splits, ws, ws_bytes, 0.0, None)


def test_decode_rejects(lib):
    assert _dec(lib, ws_bytes=16)[0] == B.S2_ECAPACITY
    assert _dec(lib, cache_len=513)[0] == B.S2_EINVAL               # beyond the layout's 512 tokens
    assert _dec(lib, cache_len=0)[0] == B.S2_EINVAL
    assert _dec(lib, seq=None)[0] == B.S2_EINVAL
    assert _dec(lib, ws=None)[0] == B.S2_EINVAL
    assert _dec(lib, ws=FAKE + 16)[0] == B.S2_EINVAL                # workspace alignment
    assert _dec(lib, D=80)[0] == B.S2_EUNSUPPORTED


def test_decode_workspace_size(lib):
    ly = _layout()
    n = ctypes.c_size_t()
    assert lib.s2_attn_decode_workspace(ctypes.byref(ly), 2, 128, 3, ctypes.byref(n)) == 0
    # partial outputs [B*H*splits, D] fp32 and partial lse [B*H*splits], each 256-byte aligned
    assert n.value == 24 * 128 * 4 + 256
    assert lib.s2_attn_decode_workspace(ctypes.byref(ly), 2, 128, 0, ctypes.byref(n)) == 0
    assert n.value > 0


def test_build_layout_t_rejects(lib):
    pat = _pat()
    st, msg = _status(lib.s2_build_layout_t, ctypes.byref(pat), 8, FAKE, FAKE, 80, None)
    assert st == B.S2_ECAPACITY and "81" in msg
    assert _status(lib.s2_build_layout_t, ctypes.byref(pat), 8, None, FAKE, 100, None)[0] == B.S2_EINVAL
    assert _status(lib.s2_build_layout_t, ctypes.byref(_pat(W=0)), 8, FAKE, FAKE, 100, None)[0] == B.S2_EINVAL


def _bwd(lib, layout_t="same", dtype=B.S2_BF16, N=512, D=128, lse=FAKE, ws=FAKE, ws_bytes=1 << 30,
         dq=FAKE):
    ly = _layout()
    lt = _layout() if layout_t == "same" else layout_t
    s = _st(4 * N * D, N * D, D, 1)
    return _status(lib.s2_attn_bwd, ctypes.byref(ly), ctypes.byref(lt) if lt is not None else None,
                   dtype, 1, N, D, FAKE, s, FAKE, s, FAKE, s, FAKE, s, FAKE, s, lse,
                   dq, s, FAKE, s, FAKE, s, ws, ws_bytes, 0.0, None)


def test_bwd_rejects(lib):
    assert _bwd(lib, dtype=B.S2_F32)[0] == B.S2_EUNSUPPORTED         # bf16 only
    assert _bwd(lib, dtype=9)[0] == B.S2_EINVAL
    assert _bwd(lib, layout_t=None)[0] == B.S2_EINVAL
    assert _bwd(lib, layout_t=_layout(nnz=80))[0] == B.S2_EINVAL      # not the column view
    assert _bwd(lib, N=1024)[0] == B.S2_EINVAL
    assert _bwd(lib, D=96)[0] == B.S2_EUNSUPPORTED
    assert _bwd(lib, lse=None)[0] == B.S2_EINVAL
    assert _bwd(lib, ws=None)[0] == B.S2_EINVAL
    assert _bwd(lib, ws=FAKE + 64)[0] == B.S2_EINVAL                  # workspace alignment
    st, msg = _bwd(lib, ws_bytes=2 * 4 * 512 * 4 - 4)
    assert st == B.S2_ECAPACITY and msg
    assert _bwd(lib, dq=None)[0] == B.S2_EINVAL


def test_bwd_workspace_size(lib):
    n = ctypes.c_size_t()
    assert lib.s2_attn_bwd_workspace(2, 3, 256, ctypes.byref(n)) == 0
    # delta and -LSE*log2(e) per row, then one int32 per key block and per pair
    # of query blocks of every (b, h)
    assert n.value == 2 * 2 * 3 * 256 * 4 + 2 * 3 * (4 + 2) * 4
    assert lib.s2_attn_bwd_workspace(4, 16, 8192, ctypes.byref(n)) == 0
    assert n.value == 2 * 4 * 16 * 8192 * 4 + 4 * 16 * (128 + 64) * 4
    assert lib.s2_attn_bwd_workspace(1, 1, 192, ctypes.byref(n)) == 0
    assert n.value == 2 * 192 * 4 + (3 + 2) * 4
    assert lib.s2_attn_bwd_workspace(0, 3, 256, ctypes.byref(n)) == B.S2_EINVAL


def _paged(lib, Hkv=2, D=128, dtype=B.S2_BF16, num_pages=16, P=64, table=FAKE, bt_stride=8, max_pages=8,
           seq=FAKE, splits=2, ws=FAKE, ws_bytes=1 << 30, kps=None):
    ly = _layout()  # 4 heads, 8 query blocks (512 tokens)
    q = _st(4 * D, D, 1)
    pg = _st(Hkv * P * D, P * D, D, 1)
    return _status(lib.s2_attn_decode_paged, ctypes.byref(ly), dtype, 1, Hkv, D, FAKE, q, FAKE, kps or pg,
                   FAKE, pg, num_pages, P, table, bt_stride, max_pages, seq, FAKE, q, None, splits, ws,
                   ws_bytes, 0.0, None)


def test_decode_paged_rejects(lib):
    assert _paged(lib, Hkv=3)[0] == B.S2_EINVAL                      # must divide 4 query heads
    assert _paged(lib, Hkv=0)[0] == B.S2_EINVAL
    for P in (0, 48, 1 << 17):
        assert _paged(lib, P=P)[0] == B.S2_EINVAL                    # power of two in [1, 65536]
    assert _paged(lib, num_pages=0)[0] == B.S2_EINVAL
    assert _paged(lib, table=None)[0] == B.S2_EINVAL
    assert _paged(lib, max_pages=0)[0] == B.S2_EINVAL
    assert _paged(lib, bt_stride=4)[0] == B.S2_EINVAL                # shorter than max_pages
    st, msg = _paged(lib, max_pages=9, bt_stride=9)                  # 576 tokens > the layout's 512
    assert st == B.S2_EINVAL and "layout" in msg
    assert _paged(lib, seq=None)[0] == B.S2_EINVAL
    assert _paged(lib, D=96)[0] == B.S2_EUNSUPPORTED
    assert _paged(lib, dtype=7)[0] == B.S2_EINVAL
    assert _paged(lib, ws=None)[0] == B.S2_EINVAL                    # 2 splits need a workspace
    assert _paged(lib, ws=FAKE + 16)[0] == B.S2_EINVAL
    assert _paged(lib, ws_bytes=64)[0] == B.S2_ECAPACITY
    assert _paged(lib, kps=_st(2 * 64 * 128, 64 * 128, 128, 2))[0] == B.S2_EINVAL  # D stride
    assert _paged(lib, splits=1 << 17)[0] == B.S2_EUNSUPPORTED


def test_decode_paged_workspace_size(lib):
    ly = _layout()
    n = ctypes.c_size_t()
    # partial outputs [B*H*splits, D] fp32 and partial lse [B*H*splits], each
    # 256-byte aligned
    assert lib.s2_attn_decode_paged_workspace(ctypes.byref(ly), 2, 2, 128, 3, ctypes.byref(n)) == 0
    assert n.value == 2 * 4 * 3 * 128 * 4 + 256
    assert lib.s2_attn_decode_paged_workspace(ctypes.byref(ly), 2, 2, 128, 1, ctypes.byref(n)) == 0
    assert n.value == 0                                              # one split: no workspace
    assert lib.s2_attn_decode_paged_workspace(ctypes.byref(ly), 2, 1, 64, 0, ctypes.byref(n)) == 0
    assert n.value > 0                                               # automatic: several splits
    assert lib.s2_attn_decode_paged_workspace(ctypes.byref(ly), 2, 3, 128, 0, ctypes.byref(n)) == B.S2_EINVAL


def test_validate_and_transpose_reject(lib):
    ly = _layout()
    assert _status(lib.s2_validate_layout, ctypes.byref(ly), None, None)[0] == B.S2_EINVAL     # no scratch
    assert _status(lib.s2_validate_layout, ctypes.byref(ly), FAKE + 4, None)[0] == B.S2_EINVAL  # misaligned
    bad = B._Layout(4, 8, 64, 0, FAKE, FAKE)
    assert _status(lib.s2_validate_layout, ctypes.byref(bad), FAKE, None)[0] == B.S2_EUNSUPPORTED  # nnz 0
    n = ctypes.c_size_t()
    assert lib.s2_transpose_layout_workspace(ctypes.byref(ly), ctypes.byref(n)) == 0
    assert n.value == 256                                     # 4 heads x 8 columns x 1 word, rounded to 256
    big = B._Layout(32, 2048, 64, 1000, FAKE, FAKE)
    assert lib.s2_transpose_layout_workspace(ctypes.byref(big), ctypes.byref(n)) == 0
    assert n.value == 32 * 2048 * 64 * 4                      # one bit per block of each head's grid

    def tr(col_ptr=FAKE, row_idx=FAKE, cap=81, ws=FAKE, ws_bytes=1 << 20):
        return _status(lib.s2_transpose_layout, ctypes.byref(ly), col_ptr, row_idx, cap, ws, ws_bytes, None)
    assert tr(col_ptr=None)[0] == B.S2_EINVAL
    assert tr(cap=80)[0] == B.S2_ECAPACITY
    assert tr(ws=None)[0] == B.S2_EINVAL
    assert tr(ws=FAKE + 16)[0] == B.S2_EINVAL
    assert tr(ws_bytes=128)[0] == B.S2_ECAPACITY


def test_fwd_varlen_rejects(lib):
    ly = _layout()

    def vl(dtype=B.S2_BF16, Bn=2, T=700, D=128, cu=FAKE, s=None, ws=FAKE, ws_bytes=1024):
        st = s or _st(4 * D, D, 1)
        return _status(lib.s2_attn_fwd_varlen, ctypes.byref(ly), dtype, Bn, T, D, cu, FAKE, st, FAKE, st, FAKE,
                       st, FAKE, st, None, ws, ws_bytes, 0.0, None)
    assert vl(dtype=B.S2_F32)[0] == B.S2_EUNSUPPORTED      # bf16 only
    assert vl(dtype=5)[0] == B.S2_EINVAL
    assert vl(Bn=0)[0] == B.S2_EINVAL
    assert vl(T=0)[0] == B.S2_EINVAL
    assert vl(D=80)[0] == B.S2_EUNSUPPORTED
    assert vl(cu=None)[0] == B.S2_EINVAL
    assert vl(s=_st(4 * 128, 128, 2))[0] == B.S2_EINVAL       # D stride
    assert vl(s=_st(4 * 128 + 4, 128, 1))[0] == B.S2_EINVAL   # token stride not a multiple of 8
    assert vl(ws=None)[0] == B.S2_EINVAL
    assert vl(ws_bytes=8)[0] == B.S2_ECAPACITY


def _c4(Bn, H, L, D):
    return (ctypes.c_int64 * 4)(H * L * D, L * D, D, 1)


def test_block_minmax_rejects(lib):
    def call(dtype=B.S2_BF16, D=128, seq=FAKE, cache_len=512, kmin=FAKE, nb=8):
        return _status(lib.s2_block_minmax, dtype, 2, 3, D, FAKE, _c4(2, 3, 512, D), seq, cache_len, kmin,
                       FAKE, nb, None)
    assert call(nb=7)[0] == B.S2_EINVAL                  # 7 blocks do not cover 512 tokens
    assert call(kmin=FAKE + 8)[0] == B.S2_EINVAL         # 16-byte alignment of the bounds
    assert call(kmin=None)[0] == B.S2_EINVAL
    assert call(seq=None)[0] == B.S2_EINVAL
    assert call(cache_len=0)[0] == B.S2_EINVAL
    assert call(D=80)[0] == B.S2_EUNSUPPORTED
    assert call(dtype=7)[0] == B.S2_EINVAL


def test_select_blocks_rejects(lib):
    def call(budget=4, nb=8, cache_len=512, cap=2 * 3 * 4, row_ptr=FAKE, D=128, hkv=3):
        q = (ctypes.c_int64 * 3)(3 * D, D, 1)
        return _status(lib.s2_select_blocks, B.S2_BF16, 2, 3, hkv, D, FAKE, q, FAKE, FAKE, nb, FAKE, cache_len,
                       budget, row_ptr, FAKE, cap, None)
    assert call(budget=0)[0] == B.S2_EINVAL
    assert call(nb=7)[0] == B.S2_EINVAL
    assert call(nb=16001, cache_len=16001 * 64)[0] == B.S2_EUNSUPPORTED   # one LDS key per block
    st, msg = call(cap=23)
    assert st == B.S2_ECAPACITY and "24" in msg                            # B * H * min(budget, 8)
    st, msg = call(budget=100, cap=47)
    assert st == B.S2_ECAPACITY and "48" in msg                            # rows never exceed 8 blocks
    assert call(row_ptr=None)[0] == B.S2_EINVAL
    assert call(D=96)[0] == B.S2_EUNSUPPORTED
    assert call(hkv=2)[0] == B.S2_EINVAL                                  # 2 K/V heads cannot serve 3 heads


def test_decode_rows_rejects_and_workspace(lib):
    n = ctypes.c_size_t()
    assert lib.s2_attn_decode_rows_workspace(2, 3, 128, 40, 3, ctypes.byref(n)) == 0
    assert n.value == 6 * 3 * 128 * 4 + 256
    assert lib.s2_attn_decode_rows_workspace(2, 3, 128, 40, 0, ctypes.byref(n)) == 0
    assert n.value == 6 * 40 * 128 * 4 + 1024  # automatic: 2048 / 6 rows, capped at 40 blocks per row
    assert _status(lib.s2_attn_decode_rows_workspace, 2, 3, 128, 0, 0, ctypes.byref(n))[0] == B.S2_EINVAL

    def call(row_ptr=FAKE, max_row=40, ws=FAKE, ws_bytes=1 << 30, seq=FAKE, D=128):
        q = (ctypes.c_int64 * 3)(3 * D, D, 1)
        c = _c4(2, 3, 512, D)
        return _status(lib.s2_attn_decode_rows, B.S2_BF16, 2, 3, D, row_ptr, FAKE, max_row, FAKE, q, FAKE, c,
                       FAKE, c, seq, 512, FAKE, q, None, 0, ws, ws_bytes, 0.0, None)
    assert call(row_ptr=None)[0] == B.S2_EINVAL
    assert call(max_row=0)[0] == B.S2_EINVAL
    assert call(seq=None)[0] == B.S2_EINVAL
    assert call(ws_bytes=1024)[0] == B.S2_ECAPACITY
    assert call(ws=FAKE + 16)[0] == B.S2_EINVAL
    assert call(D=80)[0] == B.S2_EUNSUPPORTED


def test_paged_query_aware_rejects(lib):
    pg = (ctypes.c_int64 * 4)(2 * 16 * 128, 16 * 128, 128, 1)

    def mm(P=16, table=FAKE, bt=8, width=8, nb=2, hkv=2):
        return _status(lib.s2_block_minmax_paged, B.S2_BF16, 2, hkv, 128, FAKE, pg, 64, P, table, bt, width, FAKE,
                       FAKE, FAKE, nb, None)
    assert mm(nb=1)[0] == B.S2_EINVAL       # 8 pages of 16 tokens need 2 blocks
    assert mm(P=24)[0] == B.S2_EINVAL       # page size not a power of two
    assert mm(table=None)[0] == B.S2_EINVAL
    assert mm(bt=4)[0] == B.S2_EINVAL       # stride below the table width
    assert mm(hkv=0)[0] == B.S2_EINVAL
    n = ctypes.c_size_t()
    assert lib.s2_attn_decode_paged_rows_workspace(2, 8, 2, 128, 40, 1, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.s2_attn_decode_paged_rows_workspace(2, 8, 2, 128, 40, 3, ctypes.byref(n)) == 0
    assert n.value == 16 * 3 * 128 * 4 + 256
    assert _status(lib.s2_attn_decode_paged_rows_workspace, 2, 8, 3, 128, 40, 1, ctypes.byref(n))[0] == B.S2_EINVAL

    def dec(row_ptr=FAKE, max_row=40, hkv=2):
        q = (ctypes.c_int64 * 3)(8 * 128, 128, 1)
        return _status(lib.s2_attn_decode_paged_rows, B.S2_BF16, 2, 8, hkv, 128, row_ptr, FAKE, max_row, FAKE, q,
                       FAKE, pg, FAKE, pg, 64, 16, FAKE, 8, 8, FAKE, FAKE, q, None, 1, None, 0, 0.0, None)
    assert dec(row_ptr=None)[0] == B.S2_EINVAL
    assert dec(max_row=0)[0] == B.S2_EINVAL
    assert dec(hkv=3)[0] == B.S2_EINVAL     # 3 K/V heads cannot serve 8 query heads


def test_decode_noalloc_rejects_oversize_on_the_host(lib):
    """Partials beyond the static scratch are refused before any device call."""
    ly = _layout()
    D = 128
    q = _st(4 * D, D, 1)
    c = _st(4 * 512 * D, 512 * D, D, 1)
    # 2048 batch x 4 heads x 64 splits x 129 floats > 16 MiB
    st, msg = _status(lib.s2_attn_decode_noalloc, ctypes.byref(ly), B.S2_BF16, 2048, D, FAKE, q, FAKE, c, FAKE, c,
                      FAKE, 512, FAKE, q, None, 64, 0.0, None)
    assert st == B.S2_ECAPACITY and "scratch" in msg
    st, _ = _status(lib.s2_attn_decode_noalloc, ctypes.byref(ly), B.S2_BF16, 0, D, FAKE, q, FAKE, c, FAKE, c,
                    FAKE, 512, FAKE, q, None, 1, 0.0, None)
    assert st == B.S2_EINVAL
