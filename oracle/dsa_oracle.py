"""Plain float64 CPU definition of one DSA layer (test infrastructure only).

Sources (web pages; cited by title and section):
  [P1] "SkyRL 将 GLM-5.3-Flash 训练上下文扩至 100 万 token" (news item), sections
       "模型与瓶颈" (model and bottleneck) and "四块优化 1. DSA 真稀疏" (make DSA
       truly sparse), "3. 上下文并行（CP）".
  [P2] "How Lila Sciences and Anyscale Scaled GLM-5.3-Flash Training..." (Anyscale
       blog), section "how we reached 1M tokens", lessons paragraph.
  [P3] "128K 的序列,激活放在哪?" (context-parallel lesson), sections "改进二:Ring
       Attention / 上下文并行" and "证据三问".

What the layer computes, step by step:
  1. pool_keys      -- indexer keys are grouped in pools of 4 consecutive tokens
                       [P1 model-and-bottleneck]; a pool key is the mean of its
                       4 token keys (reading: mean pooling).
  2. scores_row     -- every causal query is scored against every pool [P1, P2].
                       The pages give no formula; the reading used here is the
                       lightning-indexer form s(i,p) = sum_h w[i,h] *
                       max(0, q[i,h].kpool[p]).  A pool competes only once all
                       its 4 tokens are visible: p < floor((i+1)/4).
  3. select_topk    -- the top-k pools by score; ties go to the lower pool id;
                       the ids are returned ascending and padded with -1 when a
                       query has fewer than k complete pools.  Selection is a
                       full stable sort (no partial selection shortcut).
  4. key_positions  -- the selected pools' tokens plus the query's own
                       incomplete pool (1-3 tokens), hence at most 4k+3 keys:
                       2051 for k = 512 [P1 DSA section: 2051 rather than 2048].
  5. attn_fwd_row   -- NoPE softmax attention of every head of the query over
                       that key set [P1 DSA section]; one shared K/V head (MQA).
                       Explicit one-shot softmax; LSE in natural log.
  6. attn_bwd_row   -- its exact gradient (training context [P1]).
  blockwise_fwd_row -- the same forward accumulated over key blocks with the
                       online max/sum rescaling [P3 ring-attention section and
                       evidence table: identical to the one-shot result]; used
                       only to check that identity.

Pins (tests/test_oracle_pins.py): dense causal attention and its autograd
gradient from torch (library routines) when k covers all pools; online-softmax
identity; heapq selection; closed-form score values; closed-form attention
cases (K = 0, V = const); central finite differences; exact integer scoring;
4k+3 key bound.  Parity unpinned: nothing.
"""
from __future__ import annotations

import math
import multiprocessing as _mp
import os

import numpy as np

# ---------------------------------------------------------------------------
# input widening (the oracle's own copy; bf16 -> float64 is exact)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def n_complete_pools(i: int, pool: int = 4) -> int:
    """Pools whose tokens are all visible to a query at global position i."""
    return (int(i) + 1) // pool


# ---------------------------------------------------------------------------
# step 1: pooled indexer keys


def pool_keys(k_idx: np.ndarray, pool: int = 4) -> np.ndarray:
    """kpool[p] = mean of token keys 4p..4p+3, for every complete pool."""
    k_idx = np.asarray(k_idx, dtype=np.float64)
    n = k_idx.shape[0] // pool
    return k_idx[: n * pool].reshape(n, pool, k_idx.shape[1]).mean(axis=1)


# ---------------------------------------------------------------------------
# step 2: indexer scores of one query


def scores_row(q_row: np.ndarray, w_row: np.ndarray, kpool: np.ndarray, n_c: int) -> np.ndarray:
    """s[p] = sum_h w[h] * max(0, q[h] . kpool[p]) for p < n_c (float64)."""
    d = kpool[:n_c] @ np.asarray(q_row, dtype=np.float64).T          # [n_c, heads]
    s = (np.maximum(d, 0.0) * np.asarray(w_row, dtype=np.float64)[None, :]).sum(axis=1)
    return s + 0.0   # -0.0 and +0.0 are the same score


# ---------------------------------------------------------------------------
# step 3: top-k by full stable sort


def select_topk(s: np.ndarray, k: int) -> np.ndarray:
    """Top-k pool ids of one score row: descending score, ties to the lower id.

    Returns k int32 ids, ascending, -1 padded.
    """
    order = np.argsort(-s, kind="stable")
    sel = np.sort(order[: min(k, s.shape[0])])
    out = np.full(k, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


# ---------------------------------------------------------------------------
# step 4: key set of one query


def key_positions(sel: np.ndarray, i: int, pool: int = 4) -> np.ndarray:
    """Token positions attended by a query at position i with pools `sel`."""
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[sel >= 0]
    n_c = n_complete_pools(i, pool)
    toks = (sel[:, None] * pool + np.arange(pool)[None, :]).reshape(-1)
    own = np.arange(n_c * pool, int(i) + 1, dtype=np.int64)
    return np.concatenate([toks, own])


# ---------------------------------------------------------------------------
# steps 5 and 6: attention of one query row


def attn_fwd_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Explicit softmax attention of H heads over n keys.

    q [H, D], K/V [n, D] -> (O [H, D], lse [H], P [H, n]).
    """
    logits = scale * (q @ K.T)
    m = logits.max(axis=1)
    e = np.exp(logits - m[:, None])
    z = e.sum(axis=1)
    P = e / z[:, None]
    return P @ V, m + np.log(z), P


def attn_bwd_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, scale: float):
    """Gradient of sum(dO * O) for one query row.

    Returns dq [H, D], dK [n, D], dV [n, D] (contributions to the selected
    keys of this row only).
    """
    O, _, P = attn_fwd_row(q, K, V, scale)
    delta = (dO * O).sum(axis=1)                  # [H]
    dP = dO @ V.T                                 # [H, n]
    dS = P * (dP - delta[:, None])                # d loss / d logits (unscaled)
    dq = scale * (dS @ K)
    dK = scale * (dS.T @ q)
    dV = P.T @ dO
    return dq, dK, dV


def blockwise_fwd_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, block: int):
    """The forward of attn_fwd_row accumulated over key blocks of `block`.

    Keeps a running max m, running normaliser l and unnormalised output acc;
    each block rescales the old state by exp(m_old - m_new).
    """
    H, D = q.shape
    m = np.full(H, -np.inf)
    l = np.zeros(H)
    acc = np.zeros((H, V.shape[1]))
    for b0 in range(0, K.shape[0], block):
        lg = scale * (q @ K[b0:b0 + block].T)
        m_new = np.maximum(m, lg.max(axis=1))
        alpha = np.exp(m - m_new)
        p = np.exp(lg - m_new[:, None])
        l = l * alpha + p.sum(axis=1)
        acc = acc * alpha[:, None] + p @ V[b0:b0 + block]
        m = m_new
    return acc / l[:, None], m + np.log(l)


# ---------------------------------------------------------------------------
# whole-layer drivers (row-parallel over processes)

_G: dict = {}


def _workers(n_rows: int, workers: int | None) -> int:
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    return max(1, min(int(workers), max(1, n_rows // 8)))


def _single_thread_blas():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass


def _run_rows(fn, rows: np.ndarray, workers: int | None, blocks_per_worker: int = 4):
    """Map fn over row blocks; returns the list of block results in order.

    Worker processes run single-threaded BLAS so that W workers use W cores.
    """
    w = _workers(rows.shape[0], workers)
    blocks = np.array_split(rows, max(w * blocks_per_worker, 1))
    blocks = [b for b in blocks if b.shape[0]]
    if w == 1:
        return [fn(b) for b in blocks]
    ctx = _mp.get_context("fork")
    with ctx.Pool(w, initializer=_single_thread_blas) as pool:
        return pool.map(fn, blocks)


def _positions(q_pos, Sq: int) -> np.ndarray:
    if q_pos is None:
        return np.arange(Sq, dtype=np.int64)
    return np.asarray(q_pos, dtype=np.int64)


def _index_block(rows):
    g = _G
    out = np.empty((rows.shape[0], g["topk"]), dtype=np.int32)
    for j, r in enumerate(rows):
        i = int(g["pos"][r])
        n_c = n_complete_pools(i, g["pool"])
        s = scores_row(widen_bf16(g["q_idx"][r]), widen_bf16(g["w_idx"][r]), g["kpool"], n_c)
        out[j] = select_topk(s, g["topk"])
    return out


def index_topk(q_idx, k_idx, w_idx, q_pos, topk: int, pool: int = 4, rows=None, workers=None):
    """Selected pool ids [len(rows), topk] int32 for bf16-bit inputs.

    q_idx [Sq, HI, DI], k_idx [Sk, DI], w_idx [Sq, HI] are uint16 bf16 bits;
    q_pos is None (identity) or int positions [Sq].
    """
    Sq = q_idx.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    _G.clear()
    _G.update(q_idx=q_idx, w_idx=w_idx, kpool=pool_keys(widen_bf16(k_idx), pool),
              pos=_positions(q_pos, Sq), pool=pool, topk=topk)
    parts = _run_rows(_index_block, rows, workers)
    _G.clear()
    return np.concatenate(parts, axis=0) if parts else np.empty((0, topk), np.int32)


def _fwd_block(rows):
    g = _G
    H, D = g["q"].shape[1], g["q"].shape[2]
    O = np.empty((rows.shape[0], H, D))
    L = np.empty((rows.shape[0], H))
    for j, r in enumerate(rows):
        keys = key_positions(g["idx"][r], int(g["pos"][r]), g["pool"])
        o, lse, _ = attn_fwd_row(widen_bf16(g["q"][r]), widen_bf16(g["k"][keys]),
                                 widen_bf16(g["v"][keys]), g["scale"])
        O[j], L[j] = o, lse
    return O, L


def sparse_attn_fwd(q, k, v, idx, q_pos, scale: float, pool: int = 4, rows=None, workers=None):
    """(O [len(rows), H, D], lse [len(rows), H]) in float64."""
    Sq = q.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    _G.clear()
    _G.update(q=q, k=k, v=v, idx=np.asarray(idx), pos=_positions(q_pos, Sq), pool=pool,
              scale=float(scale))
    parts = _run_rows(_fwd_block, rows, workers)
    _G.clear()
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _bwd_block(rows):
    g = _G
    H, D = g["q"].shape[1], g["q"].shape[2]
    dq = np.empty((rows.shape[0], H, D))
    want = g["key_rows"]
    nk = want.shape[0]
    dk = np.zeros((nk, D))
    dv = np.zeros((nk, D))
    slot = g["key_slot"]
    for j, r in enumerate(rows):
        keys = key_positions(g["idx"][r], int(g["pos"][r]), g["pool"])
        a, b, c = attn_bwd_row(widen_bf16(g["q"][r]), widen_bf16(g["k"][keys]),
                               widen_bf16(g["v"][keys]), widen_bf16(g["dout"][r]), g["scale"])
        dq[j] = a
        if nk:
            s = slot[keys]
            hit = s >= 0
            if hit.any():
                dk[s[hit]] += b[hit]
                dv[s[hit]] += c[hit]
    return dq, dk, dv


def sparse_attn_bwd(q, k, v, dout, idx, q_pos, scale: float, pool: int = 4,
                    rows=None, key_rows=None, workers=None):
    """Gradients of sum(dout * O).

    Returns dq [len(rows), H, D] for the query rows `rows` (default: all) and
    dk, dv [len(key_rows), D] for the key rows `key_rows` (default: all Sk
    keys), summed over every query row of the call (all Sq rows contribute
    to dk/dv, whatever `rows` is).  Keys no query selects get 0.
    """
    Sq, Sk = q.shape[0], k.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    key_rows = np.arange(Sk) if key_rows is None else np.asarray(key_rows, dtype=np.int64)
    key_slot = np.full(Sk, -1, dtype=np.int64)
    key_slot[key_rows] = np.arange(key_rows.shape[0])
    pos = _positions(q_pos, Sq)
    # dk/dv need every row whose key set meets key_rows; dq only `rows`.
    want = np.zeros(Sq, dtype=bool)
    want[rows] = True
    if key_rows.shape[0]:
        idx = np.asarray(idx)
        kp = np.zeros(Sk // pool + 1, dtype=bool)
        kp[key_rows // pool] = True
        sel = idx.astype(np.int64)
        touch = (kp[np.where(sel >= 0, sel, Sk // pool)] & (sel >= 0)).any(axis=1)
        # own partial pool: keys 4*n_c .. i
        n_c = (pos + 1) // pool
        touch |= kp[np.minimum(n_c, Sk // pool)] & (((pos + 1) % pool) > 0)
        want |= touch
    all_rows = np.nonzero(want)[0]
    _G.clear()
    _G.update(q=q, k=k, v=v, dout=dout, idx=np.asarray(idx), pos=pos, pool=pool,
              scale=float(scale), key_rows=key_rows, key_slot=key_slot)
    parts = _run_rows(_bwd_block, all_rows, workers, blocks_per_worker=1)
    _G.clear()
    dq_all = np.concatenate([p[0] for p in parts]) if parts else np.empty((0,) + q.shape[1:])
    dk = sum((p[1] for p in parts), np.zeros((key_rows.shape[0], k.shape[1])))
    dv = sum((p[2] for p in parts), np.zeros((key_rows.shape[0], k.shape[1])))
    loc = np.full(Sq, -1, dtype=np.int64)
    loc[all_rows] = np.arange(all_rows.shape[0])
    return dq_all[loc[rows]], dk, dv


def default_scale(head_dim: int) -> float:
    """Softmax temperature 1/sqrt(D) (the pages state none; a reading)."""
    return 1.0 / math.sqrt(head_dim)
