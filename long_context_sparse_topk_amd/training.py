"""Training use of the DSA layer: autograd over the C ABI, with a memory-lean mode.

Pages: "SkyRL 将 GLM-5.3-Flash 训练上下文扩至 100 万 token", section "2. 激活重算与
Offload": activations are recomputed in the backward instead of being kept, and the
saved layer inputs wait in pinned host memory between the forward and the backward.
For the sparse-attention layer this module offers three modes:

  plain   keeps q, k, v, O, LSE and idx for the backward;
  lean    keeps q, k, v, LSE and idx; the backward recomputes O with the forward kernel
          (the same kernel on the same inputs, so O is equal bit for bit and so are the
          gradients).  The indexer, the layer's quadratic part, is never recomputed: idx
          is kept;
  offload lean, and the kept tensors are copied to pinned host memory on a side stream
          after the forward and copied back before the backward's kernels, so the layer
          holds no device memory between the two.

Every step still runs in the library's kernels; this module orders calls and copies.
No gradient reaches the indexer inputs (q_idx, k_idx, w_idx): the selection is a
discrete choice.
"""
from __future__ import annotations

import torch

from . import index_attn_fwd, sparse_attn_bwd, sparse_attn_fwd

MODES = ("plain", "lean", "offload")

_copy_streams: dict[int, torch.cuda.Stream] = {}


def _copy_stream(dev: torch.device) -> torch.cuda.Stream:
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _copy_streams:
        _copy_streams[key] = torch.cuda.Stream(device=dev)
    return _copy_streams[key]


def _to_host(tensors, dev):
    """Copy device tensors to new pinned host tensors on the side stream; returns (hosts, event)."""
    side = _copy_stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    hosts = []
    with torch.cuda.stream(side):
        for t in tensors:
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t, non_blocking=True)
            t.record_stream(side)          # the allocator keeps t until the copy is done
            hosts.append(h)
    ev = torch.cuda.Event()
    ev.record(side)
    return hosts, ev


def _to_device(hosts, ev, dev):
    """Copy pinned host tensors back on the current stream, after the offload copies ended."""
    cur = torch.cuda.current_stream(dev)
    cur.wait_event(ev)
    return [h.to(dev, non_blocking=True) for h in hosts]


class SparseAttention(torch.autograd.Function):
    """out = sparse attention over the indexer's top-k pools; also returns idx (no gradient)."""

    @staticmethod
    def forward(ctx, q_idx, k_idx, w_idx, q, k, v, q_pos, topk, q_chunk, scale, mode):
        if mode not in MODES:
            raise ValueError(f"mode must be one of {MODES}, got {mode!r}")
        idx, out, lse = index_attn_fwd(q_idx.detach(), k_idx.detach(), w_idx.detach(), q.detach(),
                                       k.detach(), v.detach(), topk=topk, q_chunk=q_chunk,
                                       q_pos=q_pos, scale=scale)
        ctx.mode, ctx.scale, ctx.q_pos = mode, scale, q_pos
        ctx.dev = q.device
        keep = [q.detach(), k.detach(), v.detach(), lse, idx]
        if mode == "plain":
            keep.append(out)
        if mode == "offload":
            ctx.hosts, ctx.ev = _to_host(keep, q.device)
        else:
            ctx.save_for_backward(*keep)   # also checks that nothing changed them in place
        ctx.saved_device_bytes = 0 if mode == "offload" else sum(
            t.numel() * t.element_size() for t in keep[3:])
        ctx.saved_host_bytes = (sum(t.numel() * t.element_size() for t in ctx.hosts)
                                if mode == "offload" else 0)
        ctx.mark_non_differentiable(idx)
        return out, idx

    @staticmethod
    def backward(ctx, dout, _didx):
        if ctx.mode == "offload":
            keep = _to_device(ctx.hosts, ctx.ev, ctx.dev)
            ctx.hosts = None
        else:
            keep = ctx.saved_tensors
        q, k, v, lse, idx = keep[:5]
        if ctx.mode == "plain":
            out = keep[5]
        else:
            out, _ = sparse_attn_fwd(q, k, v, idx, q_pos=ctx.q_pos, scale=ctx.scale)
        dq, dk, dv = sparse_attn_bwd(q, k, v, out, dout.contiguous(), lse, idx, q_pos=ctx.q_pos,
                                     scale=ctx.scale)
        return None, None, None, dq, dk, dv, None, None, None, None, None


def sparse_attention(q_idx, k_idx, w_idx, q, k, v, *, topk: int, q_pos=None, scale=None,
                     q_chunk: int = 256, mode: str = "lean"):
    """(out [Sq, H, 128] bf16, idx [Sq, topk] int32); gradients flow to q, k and v.

    mode: "plain", "lean" (recompute O in the backward) or "offload" (lean, and the kept
    tensors wait in pinned host memory).  All three give the same out, idx and gradients.
    """
    return SparseAttention.apply(q_idx, k_idx, w_idx, q, k, v, q_pos, topk, q_chunk, scale, mode)
