"""Causal work of a sequence split over N devices (test infrastructure only).

Source: "128K 的序列,激活放在哪?" (context-parallel lesson), section "改进二:Ring
Attention / 上下文并行" and its zig-zag paragraph; the misconceptions list (a
contiguous split tends to 1:3:5:7 for 4 devices).

Counting rule: query i attends keys j <= i, so a token at position i carries
i+1 (query, key) pairs.  A contiguous split gives device c the c-th block of
S/N tokens; a zig-zag split cuts the sequence into 2N segments of a = S/(2N)
tokens and gives device k segments k and 2N-1-k.  The lesson derives that a
zig-zag share carries (2N-1)*a^2 + a*(a+1) pairs for every k.

The pool count does the same for indexer work: a query at position i scores
floor((i+1)/4) complete pools.

Pins: the counts the lesson prints for 16 tokens on 4 devices (10, 26, 42,
58; zig-zag 34 each) and its closed form, checked by brute force in
tests/test_oracle_pins.py; the fixture is tests/golden/zigzag_counts.json.
"""
from __future__ import annotations

import numpy as np


def token_pairs(positions) -> int:
    """Sum over the given query positions of (i + 1)."""
    p = np.asarray(positions, dtype=np.int64)
    return int((p + 1).sum())


def pool_pairs(positions, pool: int = 4) -> int:
    """Sum over the given query positions of floor((i + 1) / pool)."""
    p = np.asarray(positions, dtype=np.int64)
    return int(((p + 1) // pool).sum())


def contiguous_positions(seq: int, n: int, c: int) -> np.ndarray:
    b = seq // n
    return np.arange(c * b, (c + 1) * b, dtype=np.int64)


def zigzag_share(seq: int, n: int, k: int) -> np.ndarray:
    a = seq // (2 * n)
    s2 = 2 * n - 1 - k
    return np.concatenate([np.arange(k * a, (k + 1) * a), np.arange(s2 * a, (s2 + 1) * a)]).astype(np.int64)


def contiguous_pairs(seq: int, n: int) -> list[int]:
    return [token_pairs(contiguous_positions(seq, n, c)) for c in range(n)]


def zigzag_pairs(seq: int, n: int) -> list[int]:
    return [token_pairs(zigzag_share(seq, n, k)) for k in range(n)]


def zigzag_closed_form(seq: int, n: int) -> int:
    """(2N-1) a^2 + a (a+1) with a = S / (2N)."""
    a = seq // (2 * n)
    return (2 * n - 1) * a * a + a * (a + 1)
