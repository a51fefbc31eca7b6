"""The forward's alternative software-pipelined schedule (S2ATTN_FWD_PIPELINED=1:
the next block's score products under this block's softmax, K and V in
separate LDS rings) against the fp64 oracle, on the cases the default
schedule is tested on: fixed-length shapes with ragged pairs, a single block,
D = 64, caller layouts with empty rows, packed varlen batches, NaN reach and
a full-size sampled workload."""
import numpy as np
import pytest
import torch

import oracle
import synth
import test_gpu_2_fwd as F
import test_gpu_7_varlen as V
from gpu_common import assert_lse_close, assert_out_close, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _pipelined(monkeypatch):
    monkeypatch.setenv("S2ATTN_FWD_PIPELINED", "1")


@pytest.mark.parametrize("B,H,N,D,W,S,dense", F.SMALL)
def test_pipelined_small_cases(B, H, N, D, W, S, dense):
    print(f"fwd pipelined B={B} H={H} N={N} D={D} W={W} S={S} dense={dense}", flush=True)
    q, k, v = F._case(7, B, H, N, D, "bf16")
    o, lse, _ = F._run(q, k, v, H, N, W, S, dense)
    rp, ci = oracle.build_layout(H, N // 64, W, S, synth.dense_flags(H, dense))
    oo, ol = oracle.attn_fwd_blocks(f64(q), f64(k), f64(v), rp, ci, N // 64)
    assert_out_close(f64(o), oo, "bf16")
    assert_lse_close(f64(lse), ol, "bf16")


def test_pipelined_matches_default_schedule(monkeypatch):
    B, H, N, D = 2, 4, 2048, 128
    q, k, v = F._case(13, B, H, N, D, "bf16")
    o1, l1, _ = F._run(q, k, v, H, N, 4, 8, (1,))
    monkeypatch.setenv("S2ATTN_FWD_PIPELINED", "0")
    o0, l0, _ = F._run(q, k, v, H, N, 4, 8, (1,))
    # the two schedules round P against different maxima: bf16-level agreement
    assert float((o1.float() - o0.float()).abs().max()) <= 2 ** -6
    assert float((l1 - l0).abs().max()) <= 1e-4


def test_pipelined_poisoned_block_only_reaches_rows_that_use_it():
    F.test_poisoned_block_only_reaches_rows_that_use_it("bf16")


@pytest.mark.parametrize("D", [128, 64])
def test_pipelined_varlen_ragged(D):
    V.test_varlen_ragged(D)


def test_pipelined_varlen_user_layout_with_empty_rows():
    V.test_varlen_user_layout_with_empty_rows()


def test_pipelined_varlen_malformed_sequences_are_skipped():
    V.test_varlen_malformed_sequences_are_skipped()


def test_pipelined_full_size_sampled():
    print("fwd pipelined full-size sampled: 7B 32K", flush=True)
    F._sampled_full(3)
