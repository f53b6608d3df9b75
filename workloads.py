"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds the workload sizes and the random-number recipes only; it
contains none of the exchange's arithmetic (callers pass the shape they
want), so the CPU oracle and the HIP path can both be fed from it without
sharing any computation.

Recipe (the pages publish no dataset; these video-DiT-shaped tensors stand
in for the FastVideo sequence-parallel attention activations):
  * "normal":  torch.Generator("cpu").manual_seed(seed); torch.randn in fp32,
               then rounded to the target dtype (round-to-nearest-even).
  * "uniform": same generator; torch.rand * 2 - 1 in fp32, then rounded.
  * "index":   the flat element index over the whole rank-stacked tensor,
               int64 -> fp32 (exact below 2**24, neighbours collide above).
  * "index_bits": the flat index as an int32 bit pattern reinterpreted as the
               4-byte dtype, so every element is unique at any size.
  * "bytes":   uniform random bit patterns of the element width (integer view).
"""
from __future__ import annotations

import torch

# name -> (w, B, S_local, H, D, dtype, value recipe, seed for mode 0, seed for mode 1, chunked)
CONFIGS = {
    "tiny": dict(w=2, B=1, S_local=8, H=4, D=16, dtype="bf16", dist="normal",
                 seed0=0, seed1=1, chunked=False),
    "mid": dict(w=4, B=1, S_local=1024, H=24, D=128, dtype="bf16", dist="normal",
                seed0=0, seed1=1, chunked=False),
    "video_dit": dict(w=8, B=1, S_local=9450, H=40, D=128, dtype="bf16", dist="normal",
                      seed0=0, seed1=1, chunked=False),
    "chunked": dict(w=4, B=4, S_local=2048, H=16, D=64, dtype="fp16", dist="uniform",
                    seed0=0, seed1=1, chunked=True),
    "awkward": dict(w=3, B=2, S_local=4681, H=12, D=80, dtype="fp32", dist="index",
                    seed0=None, seed1=None, chunked=False),
}

# Measurement-only shapes for the short-run (LDS) and unaligned-run paths,
# sized past the 256 MB on-package cache so they measure HBM.
MEASURE = {
    "short_run": dict(w=8, B=1, S_local=131072, H=8, D=32, dtype="bf16", dist="normal",
                      seed0=0, seed1=1, chunked=False),     # run 64 B, 537 MB per tensor
    "odd_run": dict(w=4, B=1, S_local=2097152, H=4, D=7, dtype="bf16", dist="normal",
                    seed0=0, seed1=1, chunked=False),       # run 14 B, 470 MB per tensor
    # the short-run shape in four batch planes, for the chunked exchange on the LDS path
    # (bench.py --chunked): window of one plane of every rank, 134 MB
    "short_run_b4": dict(w=8, B=4, S_local=32768, H=8, D=32, dtype="bf16", dist="normal",
                         seed0=0, seed1=1, chunked=True),   # run 64 B, 537 MB per tensor
}

# Shapes whose per-rank run (H/w * D elements) is not a multiple of 16 bytes,
# or is shorter than a 128-byte cache line: (w, B, S_local, H, D, dtype).
TAIL_SHAPES = [
    (3, 1, 5, 3, 7, "bf16"),    # run 14 B
    (2, 2, 3, 6, 5, "fp32"),    # run 60 B
    (4, 1, 7, 4, 3, "fp16"),    # run 6 B
    (2, 1, 9, 2, 12, "fp16"),   # run 24 B
    (5, 3, 37, 10, 3, "u8"),    # run 6 B, 1-byte elements
    (3, 2, 11, 6, 5, "f64"),    # run 80 B, 8-byte elements
    (2, 1, 300, 4, 16, "bf16"),  # run 64 B, many rows
    (8, 2, 257, 8, 24, "bf16"),  # run 48 B
    (4, 2, 192, 4, 7, "bf16"),   # run 14 B, tiles of whole 128-byte lines (16-byte chunks only)
    (2, 2, 64, 6, 5, "fp32"),    # run 60 B, the same with 4-byte pieces
    (2, 1, 80, 2, 12, "fp16"),   # run 24 B, the same with 8-byte pieces
]

DTYPES = {
    "bf16": torch.bfloat16,
    "fp16": torch.float16,
    "fp32": torch.float32,
    "f64": torch.float64,
    "u8": torch.uint8,
    "i32": torch.int32,
    "i64": torch.int64,
}

# integer type of the same width, for bit-pattern views and comparisons
BITS_VIEW = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}


def make_tensor(shape, dtype: str, dist: str, seed=None) -> torch.Tensor:
    """A contiguous CPU tensor of `shape` filled by the named recipe."""
    tdt = DTYPES[dtype]
    n = 1
    for s in shape:
        n *= int(s)
    if dist in ("normal", "uniform", "bytes"):
        gen = torch.Generator("cpu")
        gen.manual_seed(int(seed))
    if dist == "normal":
        return torch.randn(n, generator=gen, dtype=torch.float32).to(tdt).reshape(shape)
    if dist == "uniform":
        return (torch.rand(n, generator=gen, dtype=torch.float32) * 2 - 1).to(tdt).reshape(shape)
    if dist == "index":
        return torch.arange(n, dtype=torch.int64).to(tdt).reshape(shape)
    if dist == "index_bits":
        esize = torch.empty((), dtype=tdt).element_size()
        if esize == 4:
            return torch.arange(n, dtype=torch.int32).view(tdt).reshape(shape)
        if esize == 8:
            return torch.arange(n, dtype=torch.int64).view(tdt).reshape(shape)
        raise ValueError("index_bits needs a 4- or 8-byte dtype")
    if dist == "bytes":
        esize = torch.empty((), dtype=tdt).element_size()
        raw = torch.randint(0, 256, (n * esize,), generator=gen, dtype=torch.uint8)
        return raw.view(tdt).reshape(shape)
    raise ValueError(f"unknown value recipe {dist!r}")
