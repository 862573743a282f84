"""Helpers shared by the GPU tests: moving seeded inputs to the device,
parity checks against the FP64 oracle, and bitwise comparisons."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances of the parity gate (GPU vs FP64 oracle).
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2   # bf16 Out: |g - o| <= 2e-2 + 1e-2 |o|
F32_ATOL = 1e-4                     # fp32 Out: |g - o| <= 1e-4
LSE_ATOL = 1e-4                     # LSE (natural log): |g - o| <= 1e-4


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_parity(out_g, lse_g, out_o, lse_o, *, f32_out: bool, what: str):
    """Element-wise parity of GPU results (any shape, flattened per row) with
    the oracle's float64 values.  Returns the max abs errors for reporting."""
    og = np.asarray(out_g, np.float64).reshape(out_o.shape)
    lg = np.asarray(lse_g, np.float64).reshape(lse_o.shape)
    assert np.isfinite(og).all(), f"{what}: non-finite Out"
    err = np.abs(og - out_o)
    if f32_out:
        bad = err > F32_ATOL
        bound = f"{F32_ATOL}"
    else:
        bad = err > BF16_ATOL + BF16_RTOL * np.abs(out_o)
        bound = f"{BF16_ATOL} + {BF16_RTOL}|o|"
    assert not bad.any(), (f"{what}: {int(bad.sum())} Out elements exceed {bound}; "
                           f"max abs err {err.max():.3e}")
    both_inf = np.isneginf(lg) & np.isneginf(lse_o)
    with np.errstate(invalid="ignore"):
        lerr = np.where(both_inf, 0.0, np.abs(lg - lse_o))
    assert not np.isnan(lerr).any(), f"{what}: NaN / mismatched -inf in LSE"
    assert lerr.max(initial=0.0) <= LSE_ATOL, f"{what}: LSE max abs err {lerr.max():.3e} > {LSE_ATOL}"
    denom = np.maximum(np.abs(out_o), 1e-6)
    return {"out_max_abs": float(err.max(initial=0.0)), "out_max_rel": float((err / denom).max(initial=0.0)),
            "lse_max_abs": float(lerr.max(initial=0.0))}


def bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def assert_bitwise(a: torch.Tensor, b: torch.Tensor, what: str):
    """Bitwise equality (max abs difference 0.0 and identical bit patterns)."""
    assert a.shape == b.shape, f"{what}: shape {tuple(a.shape)} vs {tuple(b.shape)}"
    if not torch.equal(bits(a), bits(b)):
        fa, fb = a.float(), b.float()
        both_inf = torch.isinf(fa) & torch.isinf(fb) & (torch.sign(fa) == torch.sign(fb))
        diff = torch.where(both_inf, torch.zeros_like(fa), (fa - fb).abs())
        raise AssertionError(f"{what}: not bitwise identical (max abs diff {diff.max().item():.3e}, "
                             f"{int((bits(a) != bits(b)).sum())} differing elements)")


def sample_rows(S: int, n_random: int, seed: int) -> np.ndarray:
    """Positions to check at full size: ends, tile and block boundaries, plus
    seeded random positions."""
    fixed = [0, 1, 2, 31, 32, 33, 63, 64, 127, 128, 129, 255, 256, S // 2 - 1, S // 2, S - 129, S - 128,
             S - 33, S - 32, S - 2, S - 1]
    rnd = np.random.Generator(np.random.PCG64(seed)).integers(0, S, n_random)
    rows = np.unique(np.array([r for r in fixed if 0 <= r < S] + list(rnd), np.int64))
    return rows
