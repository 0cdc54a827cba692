"""C ABI checks that need no GPU: every declared symbol is exported, the
workspace queries are consistent, and host-side validation rejects bad
arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import long_context_sparse_topk_amd as D
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported_and_bound():
    names = _declared()
    assert names == sorted(D.SIGNATURES), "binding and header disagree"
    L = D.lib()
    for n in names:
        assert hasattr(L, n), n


def test_exported_symbols_are_only_the_abi():
    out = os.popen(f"nm -D --defined-only {D.LIB_PATH}").read()
    exported = sorted(set(re.findall(r" T (dsa_[a-z0-9_]+)", out)))
    assert exported == _declared()


def test_status_strings():
    L = D.lib()
    assert L.dsa_version() >= 100
    for s in range(5):
        assert L.dsa_status_string(s)
    assert L.dsa_status_string(99) == b"unknown status"


def test_workspace_sizes():
    a = D.index_topk_ws_bytes(4096, 4096, 128)
    b = D.index_topk_ws_bytes(1 << 20, 1 << 20, 512)
    assert 0 < a < b < 2 * 2**30          # chunked indexer scratch stays below 2 GiB
    assert D.index_topk_ws_bytes(131072, 131072, 128) < 2**30
    assert D.lib().dsa_index_topk_ws_bytes(10, 10, 4, 64, 4, 0, 1) == 0
    # Delta (Sq x heads), one offset per pool, the inverted lists (Sq x (topk + 1)) and per-chunk
    # pool counts (at most 16 MiB)
    assert D.sparse_attn_bwd_ws_bytes(10, 1000, 4, 8) >= 4 * (10 * 4 + 250 + 10 * 9)
    assert D.sparse_attn_bwd_ws_bytes(131072, 131072, 4, 128) < 2**27
    assert D.lib().dsa_sparse_attn_bwd_ws_bytes(10, 1000, 4, 128, 0) == 0
    # heads 1..64 are supported, 65 is not
    assert D.sparse_attn_bwd_ws_bytes(10, 1000, 64, 8) >= 4 * (10 * 64 * 4)
    assert D.lib().dsa_sparse_attn_bwd_ws_bytes(10, 1000, 65, 128, 8) == 0


P = 1 << 20  # a fake, 16-byte aligned address: validation fails before any use


def _idx(**kw):
    a = dict(q_idx=P, k_idx=P, w_idx=P, q_pos=None, Sq=64, Sk=64, heads=4, dim=64, pool=4,
             topk=8, q_chunk=256, out=P, ws=P, ws_bytes=1 << 40)
    a.update(kw)
    return D.lib().dsa_index_topk(a["q_idx"], a["k_idx"], a["w_idx"], a["q_pos"], a["Sq"], a["Sk"],
                                  a["heads"], a["dim"], a["pool"], a["topk"], a["q_chunk"],
                                  a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q_idx=None), 1, "q_idx is NULL"),
    (dict(k_idx=P + 8), 1, "k_idx is not 16-byte aligned"),
    (dict(out=None), 1, "idx_out is NULL"),
    (dict(Sq=0), 1, "must be >= 1"),
    (dict(Sq=65, Sk=64), 1, "Sq=65 > Sk=64"),
    (dict(q_pos=P + 2), 1, "q_pos is not 4-byte aligned"),
    (dict(Sk=1 << 31), 2, "< 2^31"),
    (dict(dim=128), 2, "idx_dim=128"),
    (dict(heads=9), 2, "idx_heads=9"),
    (dict(heads=0), 2, "idx_heads=0"),
    (dict(pool=8), 2, "pool=8"),
    (dict(topk=0), 2, "topk=0"),
    (dict(topk=4096), 2, "topk=4096"),
    (dict(q_chunk=0), 1, "q_chunk=0"),
    (dict(ws_bytes=100), 3, "ws_bytes=100"),
])
def test_index_validation(kw, status, msg):
    assert _idx(**kw) == status
    assert msg in D.lib().dsa_last_error().decode()


def test_index_fp8_validation():
    # the fp8 indexer validates like dsa_index_topk and takes 1..4 indexer heads
    L = D.lib()
    args = [P, P, P, None, 64, 64, 5, 64, 4, 8, 256, P, P, 1 << 40, None]
    assert L.dsa_index_topk_fp8(*args) == 2 and b"fp8 indexer supports 1..4" in L.dsa_last_error()
    a = list(args); a[6] = 4; a[7] = 32
    assert L.dsa_index_topk_fp8(*a) == 2 and b"idx_dim=32" in L.dsa_last_error()
    a = list(args); a[6] = 4; a[13] = 100
    assert L.dsa_index_topk_fp8(*a) == 3


def test_index_stats_validation():
    # the statistics query checks its arguments before it reads the workspace
    L = D.lib()
    r, e = ctypes.c_uint32(7), ctypes.c_uint32(7)
    ra, ea = ctypes.addressof(r), ctypes.addressof(e)
    need = D.index_topk_ws_bytes(64, 64, 8)
    assert L.dsa_index_topk_stats(None, need, 64, 64, 8, ra, ea, None) == 1
    assert b"ws is NULL" in L.dsa_last_error()
    assert L.dsa_index_topk_stats(P + 4, need, 64, 64, 8, ra, ea, None) == 1
    assert L.dsa_index_topk_stats(P, need, 64, 64, 8, None, ea, None) == 1
    assert L.dsa_index_topk_stats(P, need, 64, 64, 0, ra, ea, None) == 2
    assert L.dsa_index_topk_stats(P, need, 64, 64, 4096, ra, ea, None) == 2
    assert L.dsa_index_topk_stats(P, need - 1, 64, 64, 8, ra, ea, None) == 3
    assert (r.value, e.value) == (7, 7)   # outputs untouched on error


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, idx=P, q_pos=None, Sq=64, Sk=64, H=4, D=128, pool=4, topk=8,
             scale=0.1, out=P, lse=P)
    a.update(kw)
    return D.lib().dsa_sparse_attn_fwd(a["q"], a["k"], a["v"], a["idx"], a["q_pos"], a["Sq"], a["Sk"],
                                       a["H"], a["D"], a["pool"], a["topk"], a["scale"], a["out"],
                                       a["lse"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), 1, "q is NULL"),
    (dict(v=P + 4), 1, "v is not 16-byte aligned"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(D=64), 2, "head_dim=64"),
    (dict(H=0), 2, "heads=0"),
    (dict(H=65), 2, "heads=65"),
    (dict(pool=2), 2, "pool=2"),
    (dict(topk=2049), 2, "topk=2049"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(Sq=100), 1, "Sq=100 > Sk=64"),
])
def test_fwd_validation(kw, status, msg):
    assert _fwd(**kw) == status
    assert msg in D.lib().dsa_last_error().decode()


def test_bwd_validation():
    L = D.lib()
    args = [P, P, P, P, P, P, P, None, 64, 64, 4, 128, 4, 8, 0.1, P, P, P, P, 1 << 40, None]
    a = list(args); a[4] = None
    assert L.dsa_sparse_attn_bwd(*a) == 1 and b"dout is NULL" in L.dsa_last_error()
    a = list(args); a[18] = None
    assert L.dsa_sparse_attn_bwd(*a) == 1 and b"ws is NULL" in L.dsa_last_error()
    a = list(args); a[19] = 1000
    assert L.dsa_sparse_attn_bwd(*a) == 3 and b"ws_bytes=1000" in L.dsa_last_error()
    a = list(args); a[11] = 256
    assert L.dsa_sparse_attn_bwd(*a) == 2
    # the inverted selection lists use 32-bit offsets
    a = list(args); a[8] = 1 << 21; a[9] = 1 << 22; a[13] = 1024
    assert L.dsa_sparse_attn_bwd(*a) == 2 and b"Sq*(topk+1)" in L.dsa_last_error()


def test_bwd_noalloc_validation():
    # the allocation-free backward validates like dsa_sparse_attn_bwd and rejects shapes whose
    # workspace exceeds its 96 MiB scratch, all before any HIP call
    L = D.lib()
    args = [P, P, P, P, P, P, P, None, 64, 64, 4, 128, 4, 8, 0.1, P, P, P, None]
    a = list(args); a[4] = None
    assert L.dsa_sparse_attn_bwd_noalloc(*a) == 1 and b"dout is NULL" in L.dsa_last_error()
    a = list(args); a[10] = 65
    assert L.dsa_sparse_attn_bwd_noalloc(*a) == 2 and b"heads=65" in L.dsa_last_error()
    a = list(args); a[8] = 1 << 18; a[9] = 1 << 18; a[13] = 128
    assert D.sparse_attn_bwd_ws_bytes(1 << 18, 1 << 18, 4, 128) > 96 << 20
    assert L.dsa_sparse_attn_bwd_noalloc(*a) == 2
    assert b"exceeds the allocation-free scratch" in L.dsa_last_error()
    # the largest training workload's backward fits
    assert D.sparse_attn_bwd_ws_bytes(131072, 131072, 4, 128) <= 96 << 20


def test_python_binding_checks_dtypes():
    import torch
    q = torch.zeros(4, 4, 64, dtype=torch.float32)
    with pytest.raises(TypeError):
        D.index_topk(q, q[:, 0], q[:, :, 0], topk=4)


def _pipe(**kw):
    a = dict(q_idx=P, k_idx=P, w_idx=P, q=P, k=P, v=P, q_pos=None, Sq=64, Sk=64, HI=4, DI=64, H=4,
             D=128, pool=4, topk=8, q_chunk=256, scale=0.1, idx=P, out=P, lse=P, ws=P,
             ws_bytes=1 << 40)
    a.update(kw)
    return D.lib().dsa_index_attn_fwd(a["q_idx"], a["k_idx"], a["w_idx"], a["q"], a["k"], a["v"],
                                      a["q_pos"], a["Sq"], a["Sk"], a["HI"], a["DI"], a["H"], a["D"],
                                      a["pool"], a["topk"], a["q_chunk"], a["scale"], a["idx"],
                                      a["out"], a["lse"], a["ws"], a["ws_bytes"], None, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q_idx=None), 1, "q_idx is NULL"),
    (dict(q=None), 1, "q is NULL"),
    (dict(v=P + 4), 1, "v is not 16-byte aligned"),
    (dict(idx=None), 1, "idx_out is NULL"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(ws=None), 1, "ws is NULL"),
    (dict(Sq=65, Sk=64), 1, "Sq=65 > Sk=64"),
    (dict(DI=32), 2, "idx_dim=32"),
    (dict(HI=9), 2, "idx_heads=9"),
    (dict(D=64), 2, "head_dim=64"),
    (dict(H=65), 2, "heads=65"),
    (dict(topk=4096), 2, "topk=4096"),
    (dict(q_chunk=0), 1, "q_chunk=0"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(ws_bytes=100), 3, "ws_bytes=100"),
])
def test_pipelined_validation(kw, status, msg):
    # validation of both stages runs on the host before any HIP call
    assert _pipe(**kw) == status
    assert msg in D.lib().dsa_last_error().decode()


def test_pipelined_workspace_is_the_indexers():
    L = D.lib()
    for Sq, Sk, k in ((4096, 4096, 128), (1 << 20, 1 << 20, 512), (65536, 262144, 128)):
        assert L.dsa_index_attn_fwd_ws_bytes(Sq, Sk, 4, 64, 4, k, 256) == \
            L.dsa_index_topk_ws_bytes(Sq, Sk, 4, 64, 4, k, 256)


def test_python_binding_checks_output_shapes():
    # caller-provided outputs must match exactly, so no kernel write can leave them
    # (the checks raise before any library call)
    import torch
    bf = torch.bfloat16
    qi, ki, wi = torch.zeros(64, 4, 64, dtype=bf), torch.zeros(64, 64, dtype=bf), torch.zeros(64, 4, dtype=bf)
    q, k, v = torch.zeros(64, 2, 128, dtype=bf), torch.zeros(64, 128, dtype=bf), torch.zeros(64, 128, dtype=bf)
    idx = torch.zeros(64, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        D.index_topk(qi, ki, wi, topk=8, out=torch.zeros(63, 8, dtype=torch.int32))
    with pytest.raises(ValueError, match="lse must have shape"):
        D.sparse_attn_fwd(q, k, v, idx, lse=torch.zeros(64, 3, dtype=torch.float32))
    with pytest.raises(ValueError, match="out must have shape"):
        D.sparse_attn_fwd(q, k, v, idx, out=torch.zeros(64, 2, 64, dtype=bf))
    with pytest.raises(ValueError, match="idx must have shape"):
        D.index_attn_fwd(qi, ki, wi, q, k, v, topk=8, idx=torch.zeros(64, 4, dtype=torch.int32))
    with pytest.raises(ValueError, match="dk must have shape"):
        D.sparse_attn_bwd(q, k, v, q, q, torch.zeros(64, 2), idx, dk=torch.zeros(32, 128, dtype=bf))
    with pytest.raises(ValueError, match="attention shapes disagree"):
        D.sparse_attn_bwd(q, k, v, q, q, torch.zeros(64, 3), idx)
    with pytest.raises(TypeError, match="ws must be"):
        D.index_topk(qi, ki, wi, topk=8, ws=torch.zeros(1 << 20, dtype=torch.float32))


@pytest.mark.parametrize("width", [64, 256])
@pytest.mark.parametrize("which", ["k", "v", "both"])
def test_python_binding_checks_kv_width(width, which):
    # K/V rows are read (and dK/dV rows written) at q's head_dim stride: a k or v of
    # another width is rejected before any library call, in all three entry points
    import torch
    bf = torch.bfloat16
    qi, ki, wi = torch.zeros(64, 4, 64, dtype=bf), torch.zeros(64, 64, dtype=bf), torch.zeros(64, 4, dtype=bf)
    q = torch.zeros(64, 2, 128, dtype=bf)
    k = torch.zeros(64, width if which in ("k", "both") else 128, dtype=bf)
    v = torch.zeros(64, width if which in ("v", "both") else 128, dtype=bf)
    idx = torch.zeros(64, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="must both be"):
        D.sparse_attn_fwd(q, k, v, idx)
    with pytest.raises(ValueError, match="must both be"):
        D.index_attn_fwd(qi, ki, wi, q, k, v, topk=8)
    with pytest.raises(ValueError, match="must both be"):
        D.sparse_attn_bwd(q, k, v, q, q, torch.zeros(64, 2), idx)


def test_training_rejects_unknown_mode():
    # the mode is checked before any library call
    import torch
    from long_context_sparse_topk_amd import training as T
    bf = torch.bfloat16
    qi, ki, wi = torch.zeros(8, 4, 64, dtype=bf), torch.zeros(8, 64, dtype=bf), torch.zeros(8, 4, dtype=bf)
    q = torch.zeros(8, 2, 128, dtype=bf, requires_grad=True)
    k, v = torch.zeros(8, 128, dtype=bf), torch.zeros(8, 128, dtype=bf)
    assert T.MODES == ("plain", "lean", "offload")
    with pytest.raises(ValueError, match="mode must be one of"):
        T.sparse_attention(qi, ki, wi, q, k, v, topk=2, mode="recompute-all")
