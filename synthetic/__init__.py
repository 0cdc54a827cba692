"""Seeded synthetic inputs for one DeepSeek-Sparse-Attention (DSA) layer.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds workload definitions and random-number generation only: none of the
layer's arithmetic (pooling, scoring, selection, softmax) lives here.

Every tensor is drawn from its own NumPy stream ``default_rng([seed, tensor_id,
chunk])`` so that any tensor can be regenerated alone.  Floating-point tensors
are rounded to bfloat16 (round to nearest even) and handed out as raw uint16
bit patterns, which is exactly what the device sees; the indexer inputs are
small integers in [-3, 3] and therefore exact in bfloat16.

Workloads (one DSA layer, multi-query attention with one shared K/V head):

  name      Sq          Sk          H   topk  q_chunk  pass
  s4k       4,096       4,096       4   128   256      fwd
  s32k      32,768      32,768      16  512   512      fwd
  s128k     131,072     131,072     4   128   256      fwd+bwd
  s1m       1,048,576   1,048,576   16  512   256      fwd
  zigzag4   65,536      262,144     4   128   256      fwd+bwd  (one share of a
            4-way zig-zag split: segments 1 and 6 of 8)

Head dim 128, indexer 4 heads x 64 dims, pools of 4 tokens.  Q/K/V/dO are
N(0,1); indexer q/k/w are uniform integers {-3..3}.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os
from dataclasses import dataclass, replace

import numpy as np

HEAD_DIM = 128
IDX_HEADS = 4
IDX_DIM = 64
POOL = 4

# tensor ids: one independent stream per tensor
_TID = {"q": 1, "k": 2, "v": 3, "q_idx": 4, "k_idx": 5, "w_idx": 6, "dout": 7,
        "sel": 8}

_CHUNK = 1 << 24  # elements per generator chunk (parallel, reproducible)


@dataclass(frozen=True)
class Workload:
    name: str
    seq: int            # S: full sequence length (= Sk)
    heads: int          # H
    topk: int           # k, selected pools per query
    q_chunk: int
    backward: bool
    zigzag: tuple | None = None   # (N ranks, rank k) for one zig-zag share
    seed: int = 0

    @property
    def sk(self) -> int:
        return self.seq

    def q_positions(self) -> np.ndarray | None:
        """Global positions of this call's queries; None = identity 0..S-1."""
        if self.zigzag is None:
            return None
        n, k = self.zigzag
        return zigzag_positions(self.seq, n, k)

    @property
    def sq(self) -> int:
        qp = self.q_positions()
        return self.seq if qp is None else int(qp.shape[0])

    def scaled(self, seq: int, **kw) -> "Workload":
        return replace(self, seq=seq, **kw)


WORKLOADS = {
    "s4k": Workload("s4k", 4096, 4, 128, 256, False),
    "s32k": Workload("s32k", 32768, 16, 512, 512, False),
    "s128k": Workload("s128k", 131072, 4, 128, 256, True),
    "s1m": Workload("s1m", 1 << 20, 16, 512, 256, False),
    "zigzag4": Workload("zigzag4", 262144, 4, 128, 256, True, zigzag=(4, 1)),
}


def zigzag_positions(seq: int, n_ranks: int, rank: int) -> np.ndarray:
    """Token positions owned by `rank` under a 2N-segment zig-zag split.

    The sequence is cut into 2N equal segments; rank k owns segment k and
    segment 2N-1-k.  Positions are returned ascending as int32.
    """
    segs = 2 * n_ranks
    if seq % segs:
        raise ValueError("sequence length must divide into 2N segments")
    a = seq // segs
    lo = np.arange(rank * a, (rank + 1) * a, dtype=np.int64)
    hi_seg = segs - 1 - rank
    hi = np.arange(hi_seg * a, (hi_seg + 1) * a, dtype=np.int64)
    return np.concatenate([lo, hi]).astype(np.int32)


# ----------------------------------------------------------------------------
# bit-level helpers (input preparation only)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill(shape, seed: int, tid: int, kind: str) -> np.ndarray:
    """Generate a tensor in independent chunks (parallel and reproducible)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def job(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng([seed, tid, c])
        if kind == "normal":
            out[lo:hi] = f32_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))
        else:  # small integers, exact in bf16
            v = rng.integers(-3, 4, size=hi - lo, dtype=np.int8).astype(np.float32)
            out[lo:hi] = (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)

    if nchunks == 1:
        job(0)
    else:
        with _fut.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(job, range(nchunks)))
    return out.reshape(shape)


def make_inputs(w: Workload, parts=("index", "attn"), seed: int | None = None) -> dict:
    """All host-side inputs of one DSA layer call, as bf16 bit arrays.

    parts: subset of {"index", "attn", "bwd"}.  Returns a dict with keys
    q_idx, k_idx, w_idx (index), q, k, v (attn), dout (bwd), q_pos (int32 or
    None), and the shape constants.
    """
    s = w.seed if seed is None else seed
    qp = w.q_positions()
    sq, sk = w.sq, w.sk
    d = {"q_pos": qp, "Sq": sq, "Sk": sk, "H": w.heads, "topk": w.topk,
         "pool": POOL, "q_chunk": w.q_chunk}
    if "index" in parts:
        d["q_idx"] = _fill((sq, IDX_HEADS, IDX_DIM), s, _TID["q_idx"], "int")
        d["k_idx"] = _fill((sk, IDX_DIM), s, _TID["k_idx"], "int")
        d["w_idx"] = _fill((sq, IDX_HEADS), s, _TID["w_idx"], "int")
    if "attn" in parts:
        d["q"] = _fill((sq, w.heads, HEAD_DIM), s, _TID["q"], "normal")
        d["k"] = _fill((sk, HEAD_DIM), s, _TID["k"], "normal")
        d["v"] = _fill((sk, HEAD_DIM), s, _TID["v"], "normal")
    if "bwd" in parts:
        d["dout"] = _fill((sq, w.heads, HEAD_DIM), s, _TID["dout"], "normal")
    return d


def random_selection(n_candidates: np.ndarray, topk: int, seed: int = 0) -> np.ndarray:
    """A valid pool-index list drawn at random, for attention-only tests.

    Row r gets min(topk, n_candidates[r]) distinct ids drawn uniformly from
    [0, n_candidates[r]), ascending, padded with -1.  The caller states how
    many pools each row may choose from; this is a stand-in for an indexer
    result (any valid selection is a legal input to the attention entry
    points), not an indexer.
    """
    n_candidates = np.asarray(n_candidates, dtype=np.int64)
    out = np.full((n_candidates.shape[0], topk), -1, dtype=np.int32)
    rng = np.random.default_rng([seed, _TID["sel"]])
    for r, nc in enumerate(n_candidates):
        nc = int(nc)
        m = min(topk, nc)
        if m == 0:
            continue
        if nc <= 4 * topk:
            pick = rng.permutation(nc)[:m]
        else:
            pick = np.unique(rng.integers(0, nc, size=2 * m))
            while pick.shape[0] < m:
                pick = np.unique(np.concatenate([pick, rng.integers(0, nc, size=m)]))
            pick = rng.permutation(pick)[:m]
        out[r, :m] = np.sort(pick)
    return out
