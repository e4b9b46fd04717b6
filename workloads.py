"""Seeded synthetic inputs for sigmoid attention on padded variable-length batches.

This module draws lengths and random tensors and nothing else: it holds none of
the attention arithmetic.  The oracle-based tests, the HIP parity tests and the
bench all take their inputs from here, so both sides see identical bf16 values.

Why synthetic: the workloads of "Better Models, Faster Training: Sigmoid
Attention for single-cell Foundation Models" are single-cell expression
profiles whose cells express from hundreds to thousands of genes and are padded
to the longest cell of the batch (summary, §1 problem statement).  Those
datasets are not available, so lengths are drawn from distributions of that
shape and Q/K/V/dO are iid standard normal, rounded to bf16 (the precision named
in §2C of the same summary).

Recipe (one CPU ``torch.Generator`` per workload, seeded):
  1. draw the valid lengths (per-workload rule below);
  2. draw Q, K, V, dO = randn(B, H, Lmax, d) in float32, in that order;
  3. for the saturation-stress workload multiply Q, K, V (not dO) by 4;
  4. round to bf16 (round-to-nearest-even).
Padded positions keep their random values: they are garbage that every
consumer must ignore.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    Lmax: int
    lengths: str          # rule name, see draw_lengths()
    pad: float = 0.0      # target mean padding fraction for the "stratified" rule
    scale_qkv: float = 1.0
    note: str = ""


# Names say what the workload is and its sizes.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_b2h2d64_l128", 2, 2, 64, 128, "fixed_128_77",
                 note="two sequences, one full and one ragged (77 of 128); the oracle finishes in well under a second"),
        Workload("cells_b8h16d64_l2048", 8, 16, 64, 2048, "uniform_256",
                 note="single-cell-like padded batch: lengths iid uniform integers in [256, 2048]"),
        Workload("sweep_b16h16d64_l4096_pad00", 16, 16, 64, 4096, "stratified", pad=0.0,
                 note="padding sweep, 0% padding (all lengths 4096)"),
        Workload("sweep_b16h16d64_l4096_pad25", 16, 16, 64, 4096, "stratified", pad=0.25,
                 note="padding sweep, mean padding 25%: lengths stratified-uniform in [2048, 4096]"),
        Workload("sweep_b16h16d64_l4096_pad50", 16, 16, 64, 4096, "stratified", pad=0.50,
                 note="padding sweep, mean padding 50%: lengths stratified-uniform in [0, 4096]"),
        Workload("dense_b4h16d128_l8192", 4, 16, 128, 8192, "full",
                 note="dense long context, no padding, head dim 128"),
        Workload("cells8k_b8h12d64_l8192_x4", 8, 12, 64, 8192, "lognormal_2000", scale_qkv=4.0,
                 note="160M-class layer shape (12 heads of 64) at 8K; log-normal lengths (median 2000, sigma 0.8) "
                      "clipped to [200, 8192]; Q/K/V scaled by 4 so sigmoid arguments saturate"),
        # Equal work (sum of n^2 per head) cut three ways: few long sequences,
        # and many short cells as single-cell batches hold them.
        Workload("few_b4h16d64_l4096", 4, 16, 64, 4096, "full",
                 note="4 sequences of 4096 (the long-sequence reference for the two short-cell batches)"),
        Workload("many_b1024h16d64_l256", 1024, 16, 64, 256, "full",
                 note="1024 cells of 256 genes: the same sum of n^2 as 4 x 4096"),
        Workload("many_b4096h16d64_l128", 4096, 16, 64, 128, "full",
                 note="4096 cells of 128 genes: the same sum of n^2 as 4 x 4096"),
    )
}

# The workload the headline throughput is quoted on (single-cell padded batch).
HEADLINE = "cells_b8h16d64_l2048"
TINY = "tiny_b2h2d64_l128"


def draw_lengths(w: Workload, gen: torch.Generator) -> np.ndarray:
    """Valid lengths, right padding: sequence b holds rows 0..n_b-1."""
    B, L = w.B, w.Lmax
    if w.lengths == "fixed_128_77":
        n = torch.tensor([128, 77])
    elif w.lengths == "uniform_256":
        n = torch.randint(256, L + 1, (B,), generator=gen)
    elif w.lengths == "full":
        n = torch.full((B,), L)
    elif w.lengths == "stratified":
        # One draw per stratum of [lo, L] hits the target mean padding exactly in
        # expectation; iid draws at B=16 miss it by several points.
        lo = int(round(L * (1.0 - 2.0 * w.pad)))
        u = torch.rand(B, generator=gen, dtype=torch.float64)
        b = torch.arange(B, dtype=torch.float64)
        n = lo + torch.floor((L - lo + 1) * (b + u) / B).to(torch.int64)
        n = n[torch.randperm(B, generator=gen)]
    elif w.lengths == "lognormal_2000":
        z = torch.randn(B, generator=gen, dtype=torch.float64)
        n = torch.clamp(torch.round(torch.exp(math.log(2000.0) + 0.8 * z)), 200, L).to(torch.int64)
    else:
        raise ValueError(f"unknown length rule {w.lengths!r}")
    n = n.to(torch.int64).numpy().astype(np.int32)
    if n.shape != (B,) or n.min() < 0 or n.max() > L:
        raise AssertionError("length draw out of range")
    return n


def lengths(name: str, seed: int = 0) -> np.ndarray:
    """Only the lengths of a workload (cheap: no tensors drawn)."""
    w = WORKLOADS[name]
    g = torch.Generator().manual_seed(seed)
    return draw_lengths(w, g)


def make(name: str, seed: int = 0, with_dout: bool = True, dtype=torch.bfloat16) -> dict:
    """Draw a workload.  Returns CPU tensors (bf16, or `dtype`) and lengths
    (int32 numpy)."""
    w = WORKLOADS[name]
    g = torch.Generator().manual_seed(seed)
    n = draw_lengths(w, g)
    shape = (w.B, w.H, w.Lmax, w.d)
    out = {"workload": w, "seqlens": n}
    names = ("q", "k", "v", "do") if with_dout else ("q", "k", "v")
    for t in names:
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if t != "do" and w.scale_qkv != 1.0:
            x.mul_(w.scale_qkv)
        out[t] = x.to(dtype)
        del x
    return out


def random_case(B, H, d, Lmax, seqlens, seed=0, scale_qkv=1.0, dtype=torch.bfloat16) -> dict:
    """Same recipe for an ad-hoc shape (parity edge cases); `dtype` is the
    16-bit type the float32 draws are rounded to (bf16, or fp16)."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, Lmax, d)
    out = {"seqlens": np.asarray(seqlens, dtype=np.int32)}
    for t in ("q", "k", "v", "do"):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if t != "do" and scale_qkv != 1.0:
            x.mul_(scale_qkv)
        out[t] = x.to(dtype)
    return out


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 (or any float) tensor to float64 numpy."""
    return t.detach().to("cpu").to(torch.float64).numpy()
