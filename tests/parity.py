"""Helpers for the GPU parity tests: host<->device transfer and comparisons.

Comparison bar: indices bit-exact; attention outputs and gradients within
max |d| <= 2e-2 and mean |d| <= 2e-3 (bf16 I/O, fp32 accumulation), plus a
relative-L2 bound of 1e-2 so that small-magnitude tensors cannot pass by
being near zero.  LSE within 1e-3.

The max-abs bound is applied to the error in excess of half a bf16 ulp of
the value: rounding a correct result to bf16 alone moves values in [8, 16)
by up to 2^-5 > 2e-2 (accumulated dK/dV of keys that many queries select
reach that range), so no bf16 output could meet a bare 2e-2 there.  Below
|x| = 4 half an ulp is at most 2^-7 and the bare bound dominates.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import synthetic as syn

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2
LSE_ABS = 1e-3


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def dev_i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return syn.bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, max_abs=MAX_ABS, mean_abs=MEAN_ABS,
                 rel=REL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    d = np.abs(got - ref)
    mag = np.maximum(np.abs(got), np.abs(ref))
    half_ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 8), 0.0)
    excess = np.maximum(d - half_ulp, 0.0)
    mx, mn = float(excess.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    raw = float(d.max()) if d.size else 0.0
    nr = float(np.linalg.norm(ref))
    rl = float(np.linalg.norm(got - ref) / nr) if nr > 0 else float(np.linalg.norm(got))
    note(f"  {name}: max|d|={raw:.3e} (beyond bf16 half-ulp {mx:.3e}) mean|d|={mn:.3e} "
         f"relL2={rl:.3e} (|ref|max={np.abs(ref).max():.3e})")
    assert mx <= max_abs, f"{name}: max abs err beyond bf16 rounding {mx} > {max_abs}"
    assert mn <= mean_abs, f"{name}: mean abs err {mn} > {mean_abs}"
    assert rl <= rel, f"{name}: relative L2 err {rl} > {rel}"


def assert_idx_equal(name: str, got: np.ndarray, ref: np.ndarray, rows=None):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    bad = np.nonzero((got != ref).any(axis=1))[0]
    if bad.size:
        r = bad[0]
        rr = rows[r] if rows is not None else r
        diff = np.nonzero(got[r] != ref[r])[0][:8]
        raise AssertionError(
            f"{name}: {bad.size} rows differ; first row {rr}: cols {diff.tolist()} "
            f"got {got[r][diff].tolist()} want {ref[r][diff].tolist()}")
    note(f"  {name}: {got.shape[0]} rows bit-exact")


def sample_rows(Sq: int, topk: int, q_pos=None, n_random: int = 96, seed: int = 0) -> np.ndarray:
    """Rows to check at full size: the first and last rows, the rows around
    the point where a query first has k complete pools, every position mod 4,
    and random rows."""
    pos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    rows = set(range(min(8, Sq))) | set(range(max(0, Sq - 8), Sq))
    edge = 4 * topk
    near = np.nonzero(np.abs(pos - edge) <= 8)[0]
    rows |= set(near.tolist())
    rng = np.random.default_rng([seed, 99])
    rows |= set(rng.integers(0, Sq, size=n_random).tolist())
    for m in range(4):
        cand = np.nonzero(pos % 4 == m)[0]
        if cand.size:
            rows.add(int(cand[-1]))
    return np.array(sorted(rows), dtype=np.int64)
