"""Helpers shared by the GPU tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads as W

# Tolerances: bf16 O element-wise |gpu - ref| <= 2e-2 + 2e-2 |ref|; fp32 L max-abs 1e-3.
O_ATOL = 2e-2
O_RTOL = 2e-2
L_ATOL = 1e-3


def torch_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*args):
    """Name the case before a GPU step, so a crash still tells which one ran."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, dtype: str = "bf16"):
    """16-bit patterns -> a device tensor of that type ('bf16' or 'f16')."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def to_f64(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    widen = W.bf16_bits_to_f32 if dtype == "bf16" else W.f16_bits_to_f32
    return widen(bits).astype(np.float64)


def o_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_o_close(o_gpu: np.ndarray, o_ref: np.ndarray, what: str = ""):
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    err = np.abs(o_gpu - o_ref)
    bad = err > O_ATOL + O_RTOL * np.abs(o_ref)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} O elements out of tolerance; first at {tuple(idx)}: "
                             f"gpu {o_gpu[tuple(idx)]} ref {o_ref[tuple(idx)]}; max abs err {err.max()}")
    return float(err.max()) if err.size else 0.0


def assert_l_close(l_gpu: np.ndarray, l_ref: np.ndarray, what: str = ""):
    assert l_gpu.shape == l_ref.shape, (l_gpu.shape, l_ref.shape)
    assert np.all(np.isfinite(l_gpu)), f"{what}: non-finite L"
    err = np.abs(l_gpu - l_ref)
    m = float(err.max()) if err.size else 0.0
    assert m <= L_ATOL, f"{what}: L max abs err {m} > {L_ATOL}"
    return m
