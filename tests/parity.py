"""Helpers for the GPU parity tests: host<->device transfer and comparisons.

Comparison bar: indices bit-exact; attention outputs and gradients within
max |d| <= 2e-2 and mean |d| <= 2e-3 (bf16 I/O, fp32 accumulation), plus a
relative-L2 bound of 1e-2 so that small-magnitude tensors cannot pass by
being near zero.  LSE within 1e-3.

Where the reference value is at least 4 in magnitude, one bf16 ulp is 2^-5 or
more, wider than the 2e-2 bar itself: a correct fp32 result rounded to bf16
lands up to half an ulp away from the exact value, so there the max-abs bar
applies to the error beyond half a bf16 ulp of the reference value.  The
allowance is taken from |ref| alone (a wrong, large output cannot widen its
own bound) and is zero below |ref| = 4, where the bare 2e-2 applies.

With DSA_PARITY_LOG set to a file name, every comparison appends one JSON
line with the errors it measured (raw max |d|, max |d| where |ref| < 4, max
excess where |ref| >= 4, mean |d|, relative L2), so the margins under the bar
are on record.
"""
from __future__ import annotations

import json
import os
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


HALF_ULP_FROM = 4.0   # |ref| at and above which the half-ulp allowance applies


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp of |ref| where |ref| >= HALF_ULP_FROM, else 0 (float64)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    big = a >= HALF_ULP_FROM
    e = np.floor(np.log2(np.where(big, a, 1.0)))
    return np.where(big, np.exp2(e - 8.0), 0.0)


def _log_errors(rec: dict):
    path = os.environ.get("DSA_PARITY_LOG")
    if path:
        rec["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, max_abs=MAX_ABS, mean_abs=MEAN_ABS,
                 rel=REL_L2, allowance=True):
    """Element-wise comparison at the bar above.  allowance=False applies the bare max_abs
    everywhere (for fp32 outputs such as LSE)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if got.size == 0:
        return
    d = np.abs(got - ref)
    half = bf16_half_ulp(ref) if allowance else np.zeros_like(ref)
    excess = np.maximum(d - half, 0.0)
    big = half > 0
    mx = float(excess.max())
    mn = float(d.mean())
    raw = float(d.max())
    small_max = float(d[~big].max()) if (~big).any() else 0.0
    big_excess = float(excess[big].max()) if big.any() else 0.0
    nr = float(np.linalg.norm(ref))
    rl = float(np.linalg.norm(got - ref) / nr) if nr > 0 else float(np.linalg.norm(got))
    note(f"  {name}: max|d|={raw:.3e} (|ref|<4: {small_max:.3e}; beyond half-ulp where |ref|>=4: "
         f"{big_excess:.3e}) mean|d|={mn:.3e} relL2={rl:.3e} (|ref|max={np.abs(ref).max():.3e})")
    _log_errors({"name": name, "n": int(d.size), "max_abs": raw, "max_abs_ref_lt4": small_max,
                 "max_excess_ref_ge4": big_excess, "n_ref_ge4": int(big.sum()), "mean_abs": mn,
                 "rel_l2": rl, "ref_absmax": float(np.abs(ref).max()), "bar": [max_abs, mean_abs, rel]})
    assert mx <= max_abs, f"{name}: max abs err {mx} > {max_abs} (beyond half a bf16 ulp where |ref| >= 4)"
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
