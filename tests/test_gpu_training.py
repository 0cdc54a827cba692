"""GPU: the autograd integration (plain, lean and offload modes) against the oracle.

Every mode's idx must equal the oracle's selection exactly, and its out and the gradients
that reach q, k and v must match the oracle's forward and exact backward element by
element at the parity bar.  The three modes also run the library's kernels on the same
inputs, so out, idx and every gradient must equal, bit for bit, those of
dsa_index_attn_fwd followed by dsa_sparse_attn_bwd (dK and dV sum each pool's rows in
ascending row order, so the backward is bitwise reproducible).
"""
import numpy as np
import pytest
import torch

import long_context_sparse_topk_amd as D
import synthetic as syn
from long_context_sparse_topk_amd import training as T
from oracle import dsa_oracle as O
from tests.parity import assert_close, assert_idx_equal, dev_bf16, dev_i32, host_f64, note

pytestmark = pytest.mark.gpu
SCALE = 1.0 / np.sqrt(128.0)


def _bits(x):
    return syn.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _host_inputs(Sq, Sk, H, seed):
    rng = np.random.default_rng([seed, 77])
    qi = _bits(rng.integers(-3, 4, size=(Sq, 4, 64)))
    ki = _bits(rng.integers(-3, 4, size=(Sk, 64)))
    wi = _bits(rng.integers(-3, 4, size=(Sq, 4)))
    q = _bits(rng.standard_normal((Sq, H, 128)))
    k = _bits(rng.standard_normal((Sk, 128)))
    v = _bits(rng.standard_normal((Sk, 128)))
    do = _bits(rng.standard_normal((Sq, H, 128)))
    return qi, ki, wi, q, k, v, do


def _inputs(Sq, Sk, H, seed):
    return [dev_bf16(x) for x in _host_inputs(Sq, Sk, H, seed)]


_ORACLE = {}


def _oracle(Sq, Sk, H, topk, zigzag, seed, pos):
    """The oracle's selection, forward and exact backward for one shape (cached: every mode
    compares with the same values)."""
    key = (Sq, Sk, H, topk, zigzag, seed)
    if key not in _ORACLE:
        qi, ki, wi, q, k, v, do = _host_inputs(Sq, Sk, H, seed)
        idx = O.index_topk(qi, ki, wi, pos, topk)
        o, lse = O.sparse_attn_fwd(q, k, v, idx, pos, SCALE)
        dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, pos, SCALE)
        _ORACLE[key] = {"idx": idx, "out": o, "dq": dq, "dk": dk, "dv": dv}
    return _ORACLE[key]


@pytest.mark.parametrize("mode", T.MODES)
@pytest.mark.parametrize("Sq,Sk,H,topk,zigzag", [(3001, 3001, 4, 64, False),
                                                 (2048, 8192, 16, 128, True)])
def test_training_modes_against_oracle(mode, Sq, Sk, H, topk, zigzag):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    seed = Sq + H
    qi, ki, wi, q, k, v, do = _inputs(Sq, Sk, H, seed)
    hpos = syn.zigzag_positions(Sk, 2, 1)[:Sq] if zigzag else None
    pos = dev_i32(hpos) if zigzag else None
    note(f"training mode={mode} Sq={Sq} Sk={Sk} H={H} topk={topk} zigzag={zigzag}")
    ref = _oracle(Sq, Sk, H, topk, zigzag, seed, hpos)
    # direct calls
    idx_r, out_r, lse_r = D.index_attn_fwd(qi, ki, wi, q, k, v, topk=topk, q_pos=pos)
    dq_r, dk_r, dv_r = D.sparse_attn_bwd(q, k, v, out_r, do, lse_r, idx_r, q_pos=pos)
    # autograd, twice in a row (the pinned staging buffers and streams are reused)
    for _ in range(2):
        ql, kl, vl = (t.clone().requires_grad_(True) for t in (q, k, v))
        out, idx = T.sparse_attention(qi, ki, wi, ql, kl, vl, topk=topk, q_pos=pos, mode=mode)
        node = out.grad_fn
        if mode == "offload":
            assert node.saved_device_bytes == 0 and node.saved_host_bytes > 0
        elif mode == "lean":
            assert node.saved_device_bytes == lse_r.numel() * 4 + idx_r.numel() * 4
        else:
            assert node.saved_device_bytes == lse_r.numel() * 4 + idx_r.numel() * 4 + out_r.numel() * 2
        assert not idx.requires_grad
        out.backward(do)
        torch.cuda.synchronize()
        # against the oracle: the selection exactly, out and every gradient at the bar
        assert_idx_equal(f"{mode} idx", idx.cpu().numpy(), ref["idx"])
        assert_close(f"{mode} out", host_f64(out), ref["out"])
        assert_close(f"{mode} q.grad", host_f64(ql.grad), ref["dq"])
        assert_close(f"{mode} k.grad", host_f64(kl.grad), ref["dk"])
        assert_close(f"{mode} v.grad", host_f64(vl.grad), ref["dv"])
        # and against the direct calls
        assert torch.equal(idx, idx_r) and torch.equal(out, out_r)
        assert torch.equal(ql.grad, dq_r), "dq differs from dsa_sparse_attn_bwd"
        assert torch.equal(kl.grad, dk_r), "dk differs from dsa_sparse_attn_bwd"
        assert torch.equal(vl.grad, dv_r), "dv differs from dsa_sparse_attn_bwd"


def test_training_inputs_changed_in_place_are_caught():
    # lean keeps q, k, v through save_for_backward: an in-place change before the
    # backward is an autograd error, not a silent wrong gradient
    qi, ki, wi, q, k, v, do = _inputs(512, 512, 2, 5)
    ql = q.clone().requires_grad_(True)
    qq = ql * 1.0
    out, _ = T.sparse_attention(qi, ki, wi, qq, k, v, topk=16, mode="lean")
    qq.add_(1.0)
    with pytest.raises(RuntimeError, match="modified by an inplace operation"):
        out.backward(do)
    torch.cuda.synchronize()
