"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins and where the expected value comes from: a
library routine (torch's dense attention and autograd, heapq), a closed form,
brute force on tiny inputs, or a value printed on the pages (fixtures under
tests/golden/).
"""
import heapq
import json
import math
import os

import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import dsa_oracle as O
from oracle import zigzag as Z
from tests.conftest import GOLDEN


def _bits(x):
    return syn.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------------------
# zig-zag work counts: values printed on the context-parallel lesson


def test_zigzag_counts_match_page():
    g = json.load(open(os.path.join(GOLDEN, "zigzag_counts.json")))
    c = Z.contiguous_pairs(16, 4)
    assert c == g["contiguous_16_tokens_4_devices"]
    assert round(max(c) / (sum(c) / 4), 2) == g["contiguous_16_tokens_4_devices_max_over_mean"]
    assert max(c) == g["ring_total_contiguous"]
    assert Z.zigzag_pairs(16, 4) == g["zigzag_16_tokens_4_devices"]
    assert sum(c) // 4 == g["ring_total_balanced"]
    zz8 = Z.zigzag_pairs(32, 8)
    assert len(set(zz8)) == 1 and g["zigzag_32_tokens_8_devices_all_equal"]


@pytest.mark.parametrize("seq,n", [(16, 4), (32, 8), (64, 2), (4096, 4), (262144, 4), (1 << 20, 8)])
def test_zigzag_closed_form_equals_brute_force(seq, n):
    assert Z.zigzag_pairs(seq, n) == [Z.zigzag_closed_form(seq, n)] * n


def test_contiguous_split_tends_to_1_3_5_7():
    g = json.load(open(os.path.join(GOLDEN, "zigzag_counts.json")))
    c = np.array(Z.contiguous_pairs(1 << 20, 4), dtype=np.float64)
    assert np.allclose(c / c[0], g["contiguous_long_sequence_ratio_4_devices"], rtol=1e-4)


def test_zigzag_share_workload_equal_work():
    # the one-share workload: S = 262,144, N = 4, rank 1 (segments 1 and 6)
    w = syn.WORKLOADS["zigzag4"]
    pos = w.q_positions()
    assert np.array_equal(pos, Z.zigzag_share(262144, 4, 1))
    per_rank = [Z.token_pairs(Z.zigzag_share(262144, 4, k)) for k in range(4)]
    assert per_rank == [8_589_967_360] * 4 == [Z.zigzag_closed_form(262144, 4)] * 4
    pools = [Z.pool_pairs(Z.zigzag_share(262144, 4, k)) for k in range(4)]
    assert len(set(pools)) == 1 and pools[0] == Z.pool_pairs(pos) == 2_147_467_264


# ---------------------------------------------------------------------------
# key budget: 2051 keys for 512 pools (the GLM-5.3-Flash figure on page 1)


def test_key_budget_4k_plus_3():
    g = json.load(open(os.path.join(GOLDEN, "dsa_key_budget.json")))
    k, pool = g["topk_pools"], g["pool"]
    sizes = []
    for i in range(4 * k - 8, 4 * k + 16):
        sel = np.arange(min(k, O.n_complete_pools(i, pool)), dtype=np.int32)
        sizes.append(O.key_positions(sel, i, pool).shape[0])
    assert max(sizes) == g["max_keys_per_query"] == 4 * k + 3
    assert O.key_positions(np.full(k, -1, np.int32), 0, pool).tolist() == [0]  # min: 1 key


def test_key_positions_partial_pool_and_visibility():
    # i = 4m + 2: pool m is incomplete (token 4m+3 is in the future)
    i, m = 4 * 7 + 2, 7
    assert O.n_complete_pools(i) == m
    keys = O.key_positions(np.array([0, 3, -1, -1], np.int32), i)
    assert keys.tolist() == [0, 1, 2, 3, 12, 13, 14, 15, 28, 29, 30]
    # i = 4m + 3: pool m is complete and competes; no partial tokens
    assert O.n_complete_pools(4 * m + 3) == m + 1
    assert O.key_positions(np.array([m], np.int32), 4 * m + 3).tolist() == [28, 29, 30, 31]


# ---------------------------------------------------------------------------
# indexer scores: closed forms and exact integer arithmetic


def _closed_form_inputs(n_pools=12):
    # kpool[p, 0] = p - 5 built from four different token values (mean pool)
    k_idx = np.zeros((4 * n_pools + 3, 64), np.float32)
    for p in range(n_pools):
        base = p - 5
        k_idx[4 * p:4 * p + 4, 0] = [base + 1, base - 1, base + 2, base - 2]
        k_idx[4 * p:4 * p + 4, 1] = [1, 1, 1, 1]
    q = np.zeros((4, 64), np.float32)
    q[0, 0] = 1.0      # head 0 sees  (p - 5)
    q[1, 0] = -1.0     # head 1 sees  (5 - p)
    q[2, 1] = 2.0      # head 2 sees  2 (constant)
    q[3, 0] = 1.0
    q[3, 1] = -3.0     # head 3 sees  (p - 5) - 3
    w = np.array([1.0, 2.0, -1.0, 0.5], np.float32)
    return k_idx, q, w


def test_scores_closed_form():
    k_idx, q, w = _closed_form_inputs()
    kpool = O.pool_keys(O.widen_bf16(_bits(k_idx)))
    assert np.array_equal(kpool[:, 0], np.arange(12) - 5.0)   # mean, not sum
    s = O.scores_row(q.astype(np.float64), w.astype(np.float64), kpool, 12)
    p = np.arange(12, dtype=np.float64)
    expect = (1.0 * np.maximum(p - 5, 0) + 2.0 * np.maximum(5 - p, 0)
              - 1.0 * 2.0 + 0.5 * np.maximum(p - 8, 0))
    assert np.array_equal(s, expect)
    # ranking follows: p=0 (10-2=8), p=1 (6), ... ties resolved to lower id
    sel = O.select_topk(s, 3)
    order = sorted(range(12), key=lambda j: (-expect[j], j))[:3]
    assert sel.tolist() == sorted(order)


def test_scores_exact_against_integer_recomputation():
    rng = np.random.default_rng(7)
    k_idx = rng.integers(-3, 4, size=(203, 64))
    q = rng.integers(-3, 4, size=(4, 64))
    w = rng.integers(-3, 4, size=4)
    kpool = O.pool_keys(k_idx.astype(np.float64))
    n_c = 50
    s = O.scores_row(q.astype(np.float64), w.astype(np.float64), kpool, n_c)
    # integers: 4*s = sum_h w_h * max(0, q_h . ksum_p), ksum = 4 * kpool
    ksum = k_idx[:200].reshape(50, 4, 64).sum(axis=1).astype(np.int64)
    s4 = np.zeros(n_c, dtype=np.int64)
    for p in range(n_c):
        for h in range(4):
            dot = int(sum(int(q[h, d]) * int(ksum[p, d]) for d in range(64)))
            s4[p] += int(w[h]) * max(0, dot)
    assert np.array_equal(s * 4.0, s4.astype(np.float64))
    assert np.abs(s4).max() < (1 << 24)   # every fp32 partial sum is exact


def test_zero_weights_select_first_pools():
    rng = np.random.default_rng(1)
    q_idx = _bits(rng.integers(-3, 4, size=(40, 4, 64)))
    k_idx = _bits(rng.integers(-3, 4, size=(160, 64)))
    w_idx = _bits(np.zeros((40, 4)))
    idx = O.index_topk(q_idx, k_idx, w_idx, np.full(40, 159), topk=7, workers=1)
    assert (idx == np.arange(7)[None, :]).all()


def test_increasing_scores_select_last_pools():
    n = 30
    k_idx = np.zeros((4 * n, 64), np.float32)
    k_idx[:, 0] = np.repeat(np.arange(n) * 0.25, 4)
    q_idx = np.zeros((3, 4, 64), np.float32)
    q_idx[:, :, 0] = 1.0
    w_idx = np.ones((3, 4), np.float32)
    pos = np.array([4 * n - 1, 4 * 20 + 1, 4 * 5])    # 30, 20 and 5 complete pools
    idx = O.index_topk(_bits(q_idx), _bits(k_idx), _bits(w_idx), pos, topk=8, workers=1)
    assert idx[0].tolist() == list(range(22, 30))
    assert idx[1].tolist() == list(range(12, 20))
    assert idx[2].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]


@pytest.mark.parametrize("seed", range(5))
def test_selection_against_heapq(seed):
    rng = np.random.default_rng(seed)
    for n, k in [(1, 1), (5, 8), (64, 16), (300, 128), (1000, 512)]:
        s = rng.integers(-4, 5, size=n).astype(np.float64) * 0.25   # many ties
        if seed % 2:
            s[rng.random(n) < 0.3] = -0.0
        got = O.select_topk(s, k)
        top = heapq.nlargest(min(k, n), range(n), key=lambda p: (s[p], -p))
        want = sorted(top) + [-1] * (k - min(k, n))
        assert got.tolist() == want


def test_causal_visibility_excludes_incomplete_pool():
    # the query's own incomplete pool must not compete even with a huge score
    k_idx = np.zeros((12, 64), np.float32)
    k_idx[8:11, 0] = 3.0                 # pool 2 has tokens 8..11; 11 is future for i=10
    q_idx = np.zeros((1, 4, 64), np.float32)
    q_idx[0, :, 0] = 1.0
    idx = O.index_topk(_bits(q_idx), _bits(k_idx), _bits(np.ones((1, 4))), np.array([10]), topk=1, workers=1)
    assert idx.tolist() == [[0]]         # pools 0, 1 tie at 0 -> lower id; pool 2 invisible
    idx = O.index_topk(_bits(q_idx), _bits(k_idx), _bits(np.ones((1, 4))), np.array([11]), topk=1, workers=1)
    assert idx.tolist() == [[2]]


# ---------------------------------------------------------------------------
# attention: dense equivalence against torch (library routines)


def _dense_torch(q, k, v, dout, scale):
    """torch float64 SDPA, causal, MQA expanded over heads; returns O, dq, dk, dv."""
    H = q.shape[1]
    tq = torch.tensor(q).permute(1, 0, 2).contiguous().requires_grad_(True)      # [H, S, D]
    tk = torch.tensor(k).requires_grad_(True)
    tv = torch.tensor(v).requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.expand(H, -1, -1), tv.expand(H, -1, -1), is_causal=True, scale=scale)
    (o * torch.tensor(dout).permute(1, 0, 2)).sum().backward()
    return (o.detach().permute(1, 0, 2).numpy(), tq.grad.permute(1, 0, 2).numpy(),
            tk.grad.numpy(), tv.grad.numpy())


@pytest.mark.parametrize("S,H", [(1, 1), (2, 3), (3, 2),
                                 (5, 4), (8, 2), (13, 4), (66, 3)])
def test_dense_equivalence_fwd_bwd(S, H):
    rng = np.random.default_rng(S * 10 + H)
    D = 128
    q = _bits(rng.standard_normal((S, H, D)))
    k = _bits(rng.standard_normal((S, D)))
    v = _bits(rng.standard_normal((S, D)))
    do = _bits(rng.standard_normal((S, H, D)))
    kk = max(1, S // 4)
    idx = np.full((S, kk), -1, np.int32)
    for i in range(S):
        nc = (i + 1) // 4
        idx[i, :nc] = np.arange(nc)
    sc = 1.0 / math.sqrt(D)
    Oo, lse = O.sparse_attn_fwd(q, k, v, idx, None, sc, workers=1)
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, None, sc, workers=1)
    qf, kf, vf, df = (O.widen_bf16(x) for x in (q, k, v, do))
    to, tdq, tdk, tdv = _dense_torch(qf, kf, vf, df, sc)
    assert np.allclose(Oo, to, atol=1e-12)
    assert np.allclose(dq, tdq, atol=1e-11)
    assert np.allclose(dk, tdk, atol=1e-11)
    assert np.allclose(dv, tdv, atol=1e-11)
    # lse against torch's logsumexp over the causal row
    lg = sc * np.einsum("shd,td->sht", qf, kf)
    mask = np.tril(np.ones((S, S), bool))[:, None, :]
    ref = torch.logsumexp(torch.tensor(np.where(mask, lg, -np.inf)), dim=-1).numpy()
    assert np.allclose(lse, ref, atol=1e-12)


@pytest.mark.parametrize("block", [1, 3, 64])
def test_online_softmax_equals_one_shot(block):
    rng = np.random.default_rng(block)
    q = rng.standard_normal((4, 128))
    K = rng.standard_normal((515, 128)) * 3.0
    V = rng.standard_normal((515, 128))
    o1, l1, _ = O.attn_fwd_row(q, K, V, 0.1)
    o2, l2 = O.blockwise_fwd_row(q, K, V, 0.1, block)
    assert np.allclose(o1, o2, atol=1e-12, rtol=0)
    assert np.allclose(l1, l2, atol=1e-12, rtol=0)


def test_zero_keys_give_mean_values():
    rng = np.random.default_rng(3)
    S, H, D = 37, 2, 128
    q = _bits(rng.standard_normal((S, H, D)))
    k = _bits(np.zeros((S, D)))
    v = _bits(rng.standard_normal((S, D)))
    idx = syn.random_selection((np.arange(S) + 1) // 4, 3, seed=1)
    Oo, lse = O.sparse_attn_fwd(q, k, v, idx, None, 0.3, workers=1)
    vf = O.widen_bf16(v)
    for i in range(S):
        keys = O.key_positions(idx[i], i)
        assert np.allclose(Oo[i], vf[keys].mean(axis=0)[None, :], atol=1e-13)
        assert np.allclose(lse[i], math.log(keys.shape[0]), atol=1e-13)


def test_constant_values_zero_key_grads():
    rng = np.random.default_rng(4)
    S, H, D = 29, 3, 128
    q = _bits(rng.standard_normal((S, H, D)))
    k = _bits(rng.standard_normal((S, D)))
    v = _bits(np.full((S, D), 1.5))
    do = _bits(rng.standard_normal((S, H, D)))
    idx = syn.random_selection((np.arange(S) + 1) // 4, 2, seed=2)
    Oo, _ = O.sparse_attn_fwd(q, k, v, idx, None, 0.2, workers=1)
    assert np.allclose(Oo, 1.5, atol=1e-13)
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, None, 0.2, workers=1)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # dV sums softmax-weighted upstream grads; total equals sum of dO (rows sum to 1)
    assert np.allclose(dv.sum(axis=0), O.widen_bf16(do).sum(axis=(0, 1)), atol=1e-10)


def test_backward_finite_differences():
    rng = np.random.default_rng(5)
    H, n, D = 3, 11, 128
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    dO = rng.standard_normal((H, D))
    sc = 0.17
    dq, dK, dV = O.attn_bwd_row(q, K, V, dO, sc)

    def loss(q_, K_, V_):
        return float((O.attn_fwd_row(q_, K_, V_, sc)[0] * dO).sum())

    eps = 1e-6
    for (arr, grad) in ((q, dq), (K, dK), (V, dV)):
        for _ in range(6):
            ix = tuple(rng.integers(0, s) for s in arr.shape)
            a1 = arr.copy(); a1[ix] += eps
            a2 = arr.copy(); a2[ix] -= eps
            args1 = [q, K, V]; args2 = [q, K, V]
            j = 0 if arr is q else (1 if arr is K else 2)
            args1[j] = a1; args2[j] = a2
            fd = (loss(*args1) - loss(*args2)) / (2 * eps)
            assert abs(fd - grad[ix]) < 1e-7 * max(1.0, abs(fd))


def test_bwd_key_sampling_matches_full():
    rng = np.random.default_rng(6)
    S, H, D = 61, 2, 128
    q = _bits(rng.standard_normal((S, H, D)))
    k = _bits(rng.standard_normal((S, D)))
    v = _bits(rng.standard_normal((S, D)))
    do = _bits(rng.standard_normal((S, H, D)))
    pos = rng.permutation(S)[:40]
    idx = syn.random_selection((pos + 1) // 4, 3, seed=3)
    dq, dk, dv = O.sparse_attn_bwd(q[:40], k, v, do[:40], idx, pos, 0.2, workers=1)
    kr = np.array([0, 5, 33, 60, 59])
    rr = np.array([3, 17, 39])
    dq2, dk2, dv2 = O.sparse_attn_bwd(q[:40], k, v, do[:40], idx, pos, 0.2, rows=rr, key_rows=kr, workers=1)
    assert np.allclose(dq2, dq[rr], atol=0) and np.allclose(dk2, dk[kr], atol=1e-14)
    assert np.allclose(dv2, dv[kr], atol=1e-14)


def test_query_positions_permute_rows():
    rng = np.random.default_rng(8)
    S = 96
    q_idx = _bits(rng.integers(-3, 4, size=(S, 4, 64)))
    k_idx = _bits(rng.integers(-3, 4, size=(S, 64)))
    w_idx = _bits(rng.integers(-3, 4, size=(S, 4)))
    base = O.index_topk(q_idx, k_idx, w_idx, None, topk=5, workers=1)
    perm = rng.permutation(S)
    got = O.index_topk(q_idx[perm], k_idx, w_idx[perm], perm, topk=5, workers=1)
    assert np.array_equal(got, base[perm])


def test_multiprocess_matches_single():
    w = syn.WORKLOADS["s4k"].scaled(2048)
    d = syn.make_inputs(w, parts=("index",))
    a = O.index_topk(d["q_idx"], d["k_idx"], d["w_idx"], None, 32, rows=np.arange(0, 2048, 7), workers=1)
    b = O.index_topk(d["q_idx"], d["k_idx"], d["w_idx"], None, 32, rows=np.arange(0, 2048, 7), workers=4)
    assert np.array_equal(a, b)


def test_no_complete_pool_rows():
    # S < 4: no pool is complete, every id is padding and the key set is the
    # query's own tokens 0..i (causal attention over the prefix)
    for S in (1, 2, 3):
        q = _bits(np.ones((S, 4, 64)))
        k = _bits(np.ones((S, 64)))
        idx = O.index_topk(q, k, _bits(np.ones((S, 4))), None, topk=2, workers=1)
        assert (idx == -1).all()
        for i in range(S):
            assert O.key_positions(idx[i], i).tolist() == list(range(i + 1))
