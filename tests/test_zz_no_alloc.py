"""GPU: the allocation-free backward entry point against dsa_sparse_attn_bwd and the oracle.

Two calls in a row, the second with a smaller input (fewer rows, positions given, fewer
heads, smaller k), so the second call runs on the scratch the first one left behind.
dq must equal dsa_sparse_attn_bwd's bit for bit (the same kernels on the same inputs);
dk and dv sum each pool's rows in an order that LDS atomics set, so they must agree
within one bf16 ulp; all three must match the oracle's exact backward at the parity bar.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_topk_amd as D
import synthetic as syn
from oracle import dsa_oracle as O
from tests.parity import assert_close, dev_bf16, dev_i32, host_f64, note

pytestmark = pytest.mark.gpu
SCALE = 1.0 / np.sqrt(128.0)


def _bits(x):
    return syn.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _within_one_ulp(name, got, ref):
    g, r = got.float(), ref.float()
    bound = 2.0 ** -7 * torch.maximum(g.abs(), r.abs()) + 1e-5
    bad = int(((g - r).abs() > bound).sum())
    assert bad == 0, f"{name}: {bad} elements differ by more than one bf16 ulp"


def _case(Sq, Sk, H, topk, positions, seed):
    rng = np.random.default_rng([seed, 5])
    pos = np.sort(rng.choice(Sk, size=Sq, replace=False)).astype(np.int32) if positions else None
    n_c = ((np.arange(Sq) if pos is None else pos).astype(np.int64) + 1) // 4
    idx = syn.random_selection(n_c, topk, seed=seed)
    q = _bits(rng.standard_normal((Sq, H, 128)))
    k = _bits(rng.standard_normal((Sk, 128)))
    v = _bits(rng.standard_normal((Sk, 128)))
    do = _bits(rng.standard_normal((Sq, H, 128)))
    return pos, idx, q, k, v, do


def test_noalloc_backward_two_calls():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    D.lib()
    for Sq, Sk, H, topk, positions in ((4096, 4096, 16, 128, False), (1500, 2003, 3, 16, True)):
        note(f"noalloc bwd Sq={Sq} Sk={Sk} H={H} topk={topk} positions={positions}")
        pos, idx, q, k, v, do = _case(Sq, Sk, H, topk, positions, seed=Sq + H)
        tq = None if pos is None else dev_i32(pos)
        ti = dev_i32(idx)
        dq_, dk_, dv_, ddo = (dev_bf16(x) for x in (q, k, v, do))
        out, lse = D.sparse_attn_fwd(dq_, dk_, dv_, ti, q_pos=tq, scale=SCALE)
        ref = D.sparse_attn_bwd(dq_, dk_, dv_, out, ddo, lse, ti, q_pos=tq, scale=SCALE)
        got = D.sparse_attn_bwd_noalloc(dq_, dk_, dv_, out, ddo, lse, ti, q_pos=tq, scale=SCALE)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), "dq differs from dsa_sparse_attn_bwd"
        _within_one_ulp("dk", got[1], ref[1])
        _within_one_ulp("dv", got[2], ref[2])
        dq_r, dk_r, dv_r = O.sparse_attn_bwd(q, k, v, do, idx, pos, SCALE)
        assert_close("noalloc dq", host_f64(got[0]), dq_r)
        assert_close("noalloc dk", host_f64(got[1]), dk_r)
        assert_close("noalloc dv", host_f64(got[2]), dv_r)
