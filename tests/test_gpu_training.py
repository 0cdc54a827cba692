"""GPU: the autograd integration (plain, lean and offload modes) against the direct calls.

The three modes run the library's kernels on the same inputs, so out, idx and dq must
equal, bit for bit, those of dsa_index_attn_fwd followed by dsa_sparse_attn_bwd (whose
parity with the oracle the other GPU tests establish).  dK and dV sum each pool's rows
in the order of a device-atomic scatter, which is not fixed, so two backward calls may
round a sum differently: they must agree within one bf16 ulp.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_topk_amd as D
import synthetic as syn
from long_context_sparse_topk_amd import training as T
from tests.parity import dev_bf16, dev_i32, note

pytestmark = pytest.mark.gpu


def _bits(x):
    return syn.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _inputs(Sq, Sk, H, seed):
    rng = np.random.default_rng([seed, 77])
    qi = _bits(rng.integers(-3, 4, size=(Sq, 4, 64)))
    ki = _bits(rng.integers(-3, 4, size=(Sk, 64)))
    wi = _bits(rng.integers(-3, 4, size=(Sq, 4)))
    q = _bits(rng.standard_normal((Sq, H, 128)))
    k = _bits(rng.standard_normal((Sk, 128)))
    v = _bits(rng.standard_normal((Sk, 128)))
    do = _bits(rng.standard_normal((Sq, H, 128)))
    return [dev_bf16(x) for x in (qi, ki, wi, q, k, v, do)]


def _within_one_ulp(name, got, ref):
    g, r = got.float(), ref.float()
    bound = 2.0 ** -7 * torch.maximum(g.abs(), r.abs()) + 1e-5
    bad = int(((g - r).abs() > bound).sum())
    assert bad == 0, f"{name}: {bad} elements differ by more than one bf16 ulp"


@pytest.mark.parametrize("mode", T.MODES)
@pytest.mark.parametrize("Sq,Sk,H,topk,zigzag", [(3001, 3001, 4, 64, False),
                                                 (2048, 8192, 16, 128, True)])
def test_training_modes_equal_direct_calls(mode, Sq, Sk, H, topk, zigzag):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    qi, ki, wi, q, k, v, do = _inputs(Sq, Sk, H, Sq + H)
    pos = dev_i32(syn.zigzag_positions(Sk, 2, 1)[:Sq]) if zigzag else None
    note(f"training mode={mode} Sq={Sq} Sk={Sk} H={H} topk={topk} zigzag={zigzag}")
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
        assert torch.equal(idx, idx_r) and torch.equal(out, out_r)
        assert torch.equal(ql.grad, dq_r), "dq differs from dsa_sparse_attn_bwd"
        _within_one_ulp("dk", kl.grad, dk_r)
        _within_one_ulp("dv", vl.grad, dv_r)


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
