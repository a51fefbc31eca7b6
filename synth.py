"""Seeded synthetic inputs for head-heterogeneous block-sparse attention.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.
It holds workload definitions (shapes, dtypes, pattern parameters) and random
numbers only: no attention arithmetic, no layout arithmetic.  The CPU oracle and
the HIP path both receive the exact tensors produced here.

Workloads mirror the settings the S2-Attention pages evaluate (1.3B- and
7B-sized models, a 128K context, 7B inference; S2-Attention OpenReview page,
Abstract).  The pages publish no dataset-independent input, so every tensor is
iid N(0, 1), drawn in fp32 with ``torch.Generator`` and rounded to the working
dtype with round-to-nearest-even.

Seeding recipe (reproducible, device independent, bounded host memory):
  * fwd tensors Q, K, V of shape [B, H, N, D]: one ``randn((N, D))`` chunk per
    (tensor, b, h), seed ``seed_of(workload, tensor, b, h)``.
  * decode query [B, H, D]: one ``randn((D,))`` per (b, h).
  * decode KV cache [B, H, L, D]: one ``randn((64, D))`` chunk per 64-token block
    (tensor, b, h, j), seed ``seed_of(workload, tensor, b, h, j + 1)``, so that a
    caller can materialise only the blocks an attention row reads.
Tensor ids: Q = 1, K = 2, V = 3.
"""
from __future__ import annotations

import torch

BLOCK = 64
TENSOR_Q, TENSOR_K, TENSOR_V = 1, 2, 3
TENSOR_DO = 4  # output gradient of the backward pass

# Workloads 1-4 are forward (prefill) problems, workload 5 is decode.
# W = local window in 64-token blocks (diagonal included), S = stride of the
# head-offset strided blocks, dense = heads that attend to every causal block.
WORKLOADS = {
    1: dict(name="tiny-fwd-f32", kind="fwd", B=1, H=4, N=512, D=64, dtype="f32",
            W=2, S=4, dense=()),
    2: dict(name="1.3B-fwd-bf16", kind="fwd", B=4, H=16, N=8192, D=128, dtype="bf16",
            W=4, S=8, dense=(0, 1)),
    3: dict(name="7B-fwd-bf16", kind="fwd", B=1, H=32, N=32768, D=128, dtype="bf16",
            W=8, S=16, dense=()),
    4: dict(name="7B-128K-fwd-bf16", kind="fwd", B=1, H=32, N=131072, D=128, dtype="bf16",
            W=16, S=32, dense=(0, 1, 2, 3)),
    5: dict(name="7B-decode-bf16", kind="decode", B=64, H=32, N=32768, D=128, dtype="bf16",
            W=8, S=16, dense=()),
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def dense_flags(num_heads: int, dense_heads) -> list[int]:
    """Per-head 0/1 flags from a collection of dense head indices."""
    s = set(int(h) for h in dense_heads)
    return [1 if h in s else 0 for h in range(num_heads)]


def seed_of(workload: int, tensor: int, b: int, h: int, j: int = 0) -> int:
    """Deterministic 63-bit seed of one generated chunk."""
    assert 0 <= tensor < 10 and 0 <= b < 1000 and 0 <= h < 1000 and 0 <= j < 10**6
    return ((((workload * 10 + tensor) * 1000 + b) * 1000 + h) * 10**6) + j


def randn(seed: int, shape) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32)


def fwd_inputs(workload: int, B: int, H: int, N: int, D: int, dtype: str,
               which=(TENSOR_Q, TENSOR_K, TENSOR_V)):
    """Q, K, V as CPU tensors [B, H, N, D] in ``dtype`` (iid N(0,1), RNE-rounded)."""
    td = torch_dtype(dtype)
    out = []
    for t in which:
        x = torch.empty((B, H, N, D), dtype=td)
        for b in range(B):
            for h in range(H):
                x[b, h] = randn(seed_of(workload, t, b, h), (N, D)).to(td)
        out.append(x)
    return out


def decode_query(workload: int, B: int, H: int, D: int, dtype: str) -> torch.Tensor:
    td = torch_dtype(dtype)
    q = torch.empty((B, H, D), dtype=td)
    for b in range(B):
        for h in range(H):
            q[b, h] = randn(seed_of(workload, TENSOR_Q, b, h), (D,)).to(td)
    return q


def cache_block(workload: int, tensor: int, b: int, h: int, j: int, D: int,
                dtype: str) -> torch.Tensor:
    """One 64-token block [64, D] of the K (tensor=2) or V (tensor=3) cache."""
    return randn(seed_of(workload, tensor, b, h, j + 1), (BLOCK, D)).to(torch_dtype(dtype))


def full_cache(workload: int, tensor: int, B: int, H: int, L: int, D: int,
               dtype: str) -> torch.Tensor:
    """Whole cache [B, H, L, D] assembled from per-block chunks (small cases only)."""
    nb = (L + BLOCK - 1) // BLOCK
    x = torch.empty((B, H, nb * BLOCK, D), dtype=torch_dtype(dtype))
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                x[b, h, j * BLOCK:(j + 1) * BLOCK] = cache_block(workload, tensor, b, h, j, D, dtype)
    return x[:, :, :L].contiguous()


def randn_device(seed: int, shape, dtype: str, device) -> torch.Tensor:
    """Seeded iid N(0,1) generated on the device (bulk inputs of the timing runs)."""
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.empty(shape, dtype=torch_dtype(dtype), device=device)
    # fill in slices so that the fp32 staging buffer stays small
    flat = x.view(-1)
    step = 1 << 28
    for s in range(0, flat.numel(), step):
        n = min(step, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(x.dtype)
    return x
