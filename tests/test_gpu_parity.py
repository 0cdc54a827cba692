"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases are compared element by element over every row; the full-size
workloads run in the launch configuration the benchmark times and are
compared on sampled rows (and sampled keys for dK/dV), which the oracle
computes one by one.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_topk_amd as D
import synthetic as syn
from oracle import dsa_oracle as O
from tests.parity import (LSE_ABS, assert_close, assert_idx_equal, dev_bf16, dev_i32, host_f64,
                          note, sample_rows)

pytestmark = pytest.mark.gpu
SCALE = 1.0 / np.sqrt(128.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    D.lib()
    yield
    torch.cuda.synchronize()


_INDEX_FP8 = [False]   # the variant gpu_index() calls: dsa_index_topk or dsa_index_topk_fp8


@pytest.fixture(params=[4, 8, 16, "fp8"])
def queries_per_wave(request):
    """Run an indexer test with each workgroup sub-tile of the bf16 indexer (16, 32 and 64
    queries; dsa_set_index_queries_per_wave forces one) and with the fp8 indexer
    (dsa_index_topk_fp8), which must give the same ids on these integer inputs."""
    fp8 = request.param == "fp8"
    D.set_index_queries_per_wave(0 if fp8 else request.param)
    _INDEX_FP8[0] = fp8
    yield request.param
    D.set_index_queries_per_wave(0)
    _INDEX_FP8[0] = False


def _bits(x):
    return syn.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _int_inputs(Sq, Sk, seed, heads=4):
    rng = np.random.default_rng([seed, 1234])
    return (_bits(rng.integers(-3, 4, size=(Sq, heads, 64))),
            _bits(rng.integers(-3, 4, size=(Sk, 64))),
            _bits(rng.integers(-3, 4, size=(Sq, heads))))


def gpu_index(q_idx, k_idx, w_idx, topk, q_chunk=256, q_pos=None, fp8=None, stats=False):
    """The selected ids; with stats=True also (retried rows, exact-pass rows) of the call."""
    qp = None if q_pos is None else dev_i32(q_pos)
    Sq, Sk = q_idx.shape[0], k_idx.shape[0]
    ws = torch.empty(D.index_topk_ws_bytes(Sq, Sk, topk, idx_heads=q_idx.shape[1]), dtype=torch.uint8,
                     device="cuda")
    idx = D.index_topk(dev_bf16(q_idx), dev_bf16(k_idx), dev_bf16(w_idx), topk=topk, ws=ws,
                       q_chunk=q_chunk, q_pos=qp, fp8=_INDEX_FP8[0] if fp8 is None else fp8)
    torch.cuda.synchronize()
    if stats:
        return idx.cpu().numpy(), D.index_topk_stats(ws, Sq=Sq, Sk=Sk, topk=topk)
    return idx.cpu().numpy()


# ---------------------------------------------------------------------------
# indexer + top-k: bit-exact


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 7, 8, 63, 64, 65, 127, 200, 511, 515])
@pytest.mark.parametrize("topk", [1, 3, 8, 64])
def test_index_tiny_sweep(S, topk, queries_per_wave):
    q, k, w = _int_inputs(S, S, seed=S * 7 + topk)
    note(f"index tiny S={S} topk={topk} qpw={queries_per_wave}")
    got = gpu_index(q, k, w, topk)
    ref = O.index_topk(q, k, w, None, topk, workers=1)
    assert_idx_equal(f"idx S={S} k={topk}", got, ref)


def test_index_s4k_full(queries_per_wave):
    wl = syn.WORKLOADS["s4k"]
    d = syn.make_inputs(wl, parts=("index",))
    note(f"index s4k full qpw={queries_per_wave}")
    got, (retried, exact) = gpu_index(d["q_idx"], d["k_idx"], d["w_idx"], wl.topk, wl.q_chunk, stats=True)
    ref = O.index_topk(d["q_idx"], d["k_idx"], d["w_idx"], None, wl.topk)
    assert_idx_equal("idx s4k", got, ref)
    # the sampled thresholds hold for nearly every row (margin of 3 spreads) and the
    # wider retry margin for all of them: the fast path ran
    note(f"  rows retried {retried}, exact pass {exact}")
    assert exact == 0 and retried <= wl.sq // 100


@pytest.mark.parametrize("S,topk,heads", [(8192, 512, 4), (6000, 100, 3), (3001, 2048, 4),
                                          (2050, 17, 1)])
def test_index_compaction_and_heads(S, topk, heads, queries_per_wave):
    q, k, w = _int_inputs(S, S, seed=S + topk, heads=heads)
    note(f"index S={S} topk={topk} heads={heads} qpw={queries_per_wave}")
    got = gpu_index(q, k, w, topk, q_chunk=512)
    ref = O.index_topk(q, k, w, None, topk)
    assert_idx_equal("idx", got, ref)


def test_index_all_ties(queries_per_wave):
    S, topk = 2048, 40
    q, k, _ = _int_inputs(S, S, seed=3)
    w = _bits(np.zeros((S, 4)))
    got = gpu_index(q, k, w, topk)
    ref = O.index_topk(q, k, w, None, topk)
    assert_idx_equal("idx all ties", got, ref)
    full = np.arange(topk)[None, :]
    assert (got[4 * topk:] == full).all()


@pytest.mark.parametrize("direction", [1, -1])
def test_index_monotone_scores(direction, queries_per_wave):
    # score(p) = p (or n-1-p): with increasing scores every pool beats the
    # running threshold, so candidate lists fill and compact on every tile
    S, topk = 3072, 64
    n = S // 4
    vals = np.arange(n) if direction > 0 else np.arange(n)[::-1]
    dims = np.arange(64)
    kp = np.clip(0.25 * vals[:, None] - 3.0 * dims[None, :], 0.0, 3.0)   # sum over dims = vals/4
    k_idx = np.repeat(kp, 4, axis=0).astype(np.float32)
    q = np.ones((S, 4, 64), np.float32)
    w = np.ones((S, 4), np.float32)
    q, k_idx, w = _bits(q), _bits(k_idx), _bits(w)
    got = gpu_index(q, k_idx, w, topk)
    ref = O.index_topk(q, k_idx, w, None, topk)
    assert_idx_equal(f"idx monotone {direction}", got, ref)
    last = S - 1
    want = np.arange(n - topk, n) if direction > 0 else np.arange(topk)
    assert got[last].tolist() == want.tolist()


def test_index_chunk_invariance_repeat_and_positions(queries_per_wave):
    S, topk = 4096, 128
    q, k, w = _int_inputs(S, S, seed=11)
    base = gpu_index(q, k, w, topk, q_chunk=256)
    for qc in (1, 64, 4096):
        assert np.array_equal(gpu_index(q, k, w, topk, q_chunk=qc), base)
    assert np.array_equal(gpu_index(q, k, w, topk, q_chunk=256), base)
    perm = np.random.default_rng(5).permutation(S)
    got = gpu_index(q[perm], k, w[perm], topk, q_pos=perm)
    assert np.array_equal(got, base[perm])
    ref = O.index_topk(q, k, w, None, topk)
    assert_idx_equal("idx 4096", base, ref)


def test_index_subset_positions_sk_larger(queries_per_wave):
    # queries are a strided subset of a longer sequence (Sk not a multiple of 4)
    Sk, topk = 5003, 32
    pos = np.arange(0, Sk, 7)[::-1].copy()
    q, k, w = _int_inputs(pos.shape[0], Sk, seed=21)
    got = gpu_index(q, k, w, topk, q_pos=pos)
    ref = O.index_topk(q, k, w, pos, topk)
    assert_idx_equal("idx subset", got, ref)


def _threshold_trap_keys(S, unsampled):
    """Indexer keys for q = w = 1, where the score of pool p is 4 * T(p).

    The indexer estimates each query's threshold from a sample of every 16th
    tile of 64 pools (tiles 0, 16, 32, ...), or of every 8th for query tiles
    whose causal range spans at most 128 pool tiles when k <= 256 (as here).
    Tile 0 holds the best scores, T = 150 - p, the other tiles of either sample
    (every 8th) T = 50, and every pool outside them T = `unsampled`, so the
    sample overstates how good the unsampled pools are.  With `unsampled` = 125
    the small-margin threshold of long queries (about the 23rd best sampled
    score at S = 10240, k = 64) keeps fewer than k pools and the larger-margin
    retry (about the 40th) keeps every unsampled pool; with 10 both keep fewer
    than k and those rows need the exact pass.
    """
    n = S // 4
    T = np.full(n, unsampled)
    tile = np.arange(n) // 64
    T[tile % 8 == 0] = 50
    T[:64] = 150 - np.arange(64)
    kp = np.clip(T[:, None] - 3 * np.arange(64)[None, :], 0, 3)   # row sums = T
    return _bits(np.repeat(kp, 4, axis=0).astype(np.float32))


@pytest.mark.parametrize("unsampled", [125, 10])
@pytest.mark.parametrize("permute", [False, True])
def test_index_sampled_threshold_too_high(unsampled, permute, queries_per_wave):
    # every query row needs its own fallback: a retry, or the exact pass; with
    # permuted positions a workgroup mixes rows that fail with rows that do not
    S, topk = 10240, 64
    k_idx = _threshold_trap_keys(S, unsampled)
    q = _bits(np.ones((S, 4, 64), np.float32))
    w = _bits(np.ones((S, 4), np.float32))
    pos = np.random.default_rng(17).permutation(S) if permute else None
    note(f"index threshold trap unsampled={unsampled} permute={permute} qpw={queries_per_wave}")
    got = gpu_index(q, k_idx, w, topk, q_pos=pos)
    ref = O.index_topk(q, k_idx, w, pos, topk)
    assert_idx_equal(f"idx trap {unsampled}", got, ref)
    if unsampled == 125:   # ties at 4*125: pool 25 first, then the lowest unsampled ids
        last = S - 1 if pos is None else int(np.argmax(pos))
        assert got[last].tolist() == list(range(26)) + list(range(64, 102))


@pytest.mark.parametrize("unsampled", [125, 10])
def test_index_rows_at_one_position_threshold_trap(unsampled, queries_per_wave):
    # 512 query rows, all at the last of 16384 key positions (q_pos constant):
    # every query tile has the same 64-tile causal range, sampled on the trap's
    # tiles 0, 8, 16, ..., so every row retries (unsampled = 125) or needs the
    # exact pass (10); a workgroup's rows all take the same path.
    Sq, Sk, topk = 512, 16384, 64
    k_idx = _threshold_trap_keys(Sk, unsampled)
    q = _bits(np.ones((Sq, 4, 64), np.float32))
    w = _bits(np.ones((Sq, 4), np.float32))
    pos = np.full(Sq, Sk - 1, dtype=np.int64)
    note(f"index rows at one position, threshold trap unsampled={unsampled} qpw={queries_per_wave}")
    got, (retried, exact) = gpu_index(q, k_idx, w, topk, q_pos=pos, stats=True)
    ref = O.index_topk(q, k_idx, w, pos, topk)
    assert_idx_equal(f"idx one-position trap {unsampled}", got, ref)
    # the first threshold (the 23rd best sampled score, that of tile 0's pool 22) keeps
    # tile 0's 23 best pools in every row; the retry's (the 40th) keeps every unsampled
    # pool at T = 125 and only tile 0's 40 at T = 10
    assert retried == Sq and exact == (0 if unsampled == 125 else Sq), (retried, exact)


def _operand_rounding(fp8):
    """(unit roundoff, absolute error floor) of the indexer's operand format:
    bf16 has 8 significant bits and the fp32 exponent range; OCP e4m3 has 4
    significant bits and subnormals spaced 2^-9 below 2^-6."""
    return (2.0 ** -4, 2.0 ** -10) if fp8 else (2.0 ** -8, 0.0)


def _score_error_bound(x, kp, fp8):
    """Bound on |GPU score - exact score| per pool for one query.

    x [H, 64] = w_h * q_h (exact), kp [n, 64] = exact pooled keys.  The GPU
    rounds both operands once (to bf16 or e4m3) and accumulates in fp32; the
    clamp of each head is 1-Lipschitz, so per head the error is at most that of
    the rounded dot product, (2u + u^2) sum|x||k| + a(1 + u) sum(|x| + |k|) +
    64 a^2, plus fp32 accumulation (64 and 3 terms), summed over the heads."""
    u, a = _operand_rounding(fp8)
    ax, ak = np.abs(x), np.abs(kp)
    prod = ak @ ax.T                                       # [n, H] sum_d |x||k|
    per_head = ((2 * u + u * u) * prod + a * (1 + u) * (ax.sum(axis=1)[None, :] + ak.sum(axis=1)[:, None])
                + 64 * a * a)
    fp32 = 2.0 ** -24 * (70 * prod.sum(axis=1) + 3 * prod.sum(axis=1))
    return 1.01 * per_head.sum(axis=1) + fp32 + 1e-12


def test_index_real_valued_inputs_select_a_valid_top_k(queries_per_wave):
    # N(0,1) indexer inputs: the operand rounding (bf16, or e4m3 for the fp8
    # indexer) may reorder pools whose exact scores are close, so the ids are not
    # compared with the oracle's; instead every row must hold min(k, n_c) distinct
    # visible pools, ascending, and no pool left out may beat a selected one by
    # more than the two pools' error bounds: min(s_sel + e_sel) >= max(s_out - e_out).
    # (On a CPU emulation of the rounding the bf16 bound catches a dropped head, a
    # missing ReLU or a flipped weight sign in most rows; the e4m3 bound is 16 times
    # wider and catches only gross errors there: the integer cases grade fp8 exactly.)
    S, topk = 4100, 64
    rng = np.random.default_rng(61)
    q = _bits(rng.standard_normal((S, 4, 64)))
    k = _bits(rng.standard_normal((S, 64)))
    w = _bits(rng.standard_normal((S, 4)))
    fp8 = _INDEX_FP8[0]
    note(f"index real-valued inputs S={S} topk={topk} qpw={queries_per_wave}")
    got = gpu_index(q, k, w, topk)
    qf, wf = O.widen_bf16(q), O.widen_bf16(w)
    kp = O.pool_keys(O.widen_bf16(k))
    worst = np.inf
    for i in range(S):
        n_c = O.n_complete_pools(i)
        m = min(topk, n_c)
        row = got[i]
        assert (row[m:] == -1).all() and (row[:m] >= 0).all() and (row[:m] < n_c).all(), f"row {i}: {row}"
        assert (np.diff(row[:m]) > 0).all(), f"row {i}: ids not strictly ascending"
        if m == 0 or m == n_c:
            continue
        s = O.scores_row(qf[i], wf[i], kp, n_c)
        e = _score_error_bound(qf[i] * wf[i][:, None], kp[:n_c], fp8)
        sel = np.zeros(n_c, dtype=bool)
        sel[row[:m]] = True
        margin = (s[sel] + e[sel]).min() - (s[~sel] - e[~sel]).max()
        worst = min(worst, margin)
        assert margin >= 0, f"row {i}: a left-out pool beats a selected one beyond the error bounds"
    note(f"  smallest margin {worst:.3e}")


@pytest.mark.parametrize("heads", [5, 6, 8])
def test_index_five_to_eight_heads(heads):
    # 5 to 8 indexer heads: two groups of 4 heads per query in the MFMA tile
    S, topk = 3001, 64
    q, k, w = _int_inputs(S, S, seed=40 + heads, heads=heads)
    note(f"index heads={heads} S={S} topk={topk}")
    got = gpu_index(q, k, w, topk)
    ref = O.index_topk(q, k, w, None, topk)
    assert_idx_equal(f"idx heads={heads}", got, ref)


# ---------------------------------------------------------------------------
# attention: forward and backward


def gpu_attn(d, idx, q_pos=None, bwd=True):
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    qp = None if q_pos is None else dev_i32(q_pos)
    ti = dev_i32(idx)
    out, lse = D.sparse_attn_fwd(q, k, v, ti, q_pos=qp, scale=SCALE)
    res = {"out": out, "lse": lse}
    if bwd:
        dq, dk, dv = D.sparse_attn_bwd(q, k, v, out, dev_bf16(d["dout"]), lse, ti, q_pos=qp,
                                       scale=SCALE)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: host_f64(t) for n, t in res.items()}


def _attn_inputs(Sq, Sk, H, seed):
    rng = np.random.default_rng([seed, 77])
    return {"q": _bits(rng.standard_normal((Sq, H, 128))), "k": _bits(rng.standard_normal((Sk, 128))),
            "v": _bits(rng.standard_normal((Sk, 128))), "dout": _bits(rng.standard_normal((Sq, H, 128)))}


def _check_attn(tag, got, d, idx, q_pos, bwd=True):
    o, lse = O.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, q_pos, SCALE)
    assert_close(f"{tag} O", got["out"], o)
    assert_close(f"{tag} lse", got["lse"], lse, max_abs=LSE_ABS, mean_abs=LSE_ABS, rel=1e-4, allowance=False)
    if bwd:
        dq, dk, dv = O.sparse_attn_bwd(d["q"], d["k"], d["v"], d["dout"], idx, q_pos, SCALE)
        assert_close(f"{tag} dq", got["dq"], dq)
        assert_close(f"{tag} dk", got["dk"], dk)
        assert_close(f"{tag} dv", got["dv"], dv)


@pytest.mark.parametrize("S,H,topk", [(2048, 4, 32), (4096, 16, 512), (1031, 3, 16), (9, 1, 1),
                                      (2053, 16, 128), (8400, 2, 2048)])
def test_pipeline_small(S, H, topk):
    # (8400, 2, 2048): the largest k; the last rows attend 4k + 3 = 8195 keys
    note(f"pipeline small S={S} H={H} topk={topk}")
    q_idx, k_idx, w_idx = _int_inputs(S, S, seed=S + H)
    idx = gpu_index(q_idx, k_idx, w_idx, topk)
    ref_idx = O.index_topk(q_idx, k_idx, w_idx, None, topk)
    assert_idx_equal("idx", idx, ref_idx)
    d = _attn_inputs(S, S, H, seed=S * 3 + H)
    got = gpu_attn(d, idx)          # the HIP pipeline runs on its own selection
    _check_attn(f"S={S} H={H} k={topk}", got, d, ref_idx, None)


def test_attention_random_selection_positions():
    # a subset of queries of a longer sequence, shuffled, with a random valid
    # selection; Sk not a multiple of 4
    Sk, H, topk = 3001, 4, 24
    pos = np.random.default_rng(2).permutation(Sk)[:1500]
    idx = syn.random_selection((pos + 1) // 4, topk, seed=4)
    d = _attn_inputs(pos.shape[0], Sk, H, seed=8)
    got = gpu_attn(d, idx, q_pos=pos)
    _check_attn("subset", got, d, idx, pos)


def test_attention_skips_invalid_ids():
    # ids outside [0, n_c) and -1 in the middle are skipped, as documented
    S, H, topk = 400, 2, 8
    pos = np.arange(S)
    idx = syn.random_selection((pos + 1) // 4, topk, seed=5)
    bad = idx.copy()
    bad[::3, 1] = -1
    bad[1::5, 2] = 10 ** 6
    clean = np.full_like(bad, -1)
    for r in range(S):
        nc = (r + 1) // 4
        keep = [p for p in bad[r] if 0 <= p < nc]
        clean[r, :len(keep)] = keep
    d = _attn_inputs(S, S, H, seed=9)
    got = gpu_attn(d, bad)
    _check_attn("invalid ids", got, d, clean, None)


def test_dense_equivalence_against_torch():
    # topk covering every pool gives causal dense attention (torch fp32 SDPA on GPU)
    S, H = 512, 4
    d = _attn_inputs(S, S, H, seed=12)
    topk = S // 4
    idx = np.full((S, topk), -1, np.int32)
    for i in range(S):
        idx[i, :(i + 1) // 4] = np.arange((i + 1) // 4)
    got = gpu_attn(d, idx, bwd=False)
    q = dev_bf16(d["q"]).float().permute(1, 0, 2).contiguous()
    k = dev_bf16(d["k"]).float().unsqueeze(0).expand(H, -1, -1).contiguous()
    v = dev_bf16(d["v"]).float().unsqueeze(0).expand(H, -1, -1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=SCALE)
    assert_close("dense O", got["out"], ref.permute(1, 0, 2).double().cpu().numpy())


@pytest.mark.parametrize("H", [17, 32, 64])
def test_attention_more_than_16_heads(H):
    # heads beyond 16 run in groups of 16, one wave per (row, group); the dK/dV pass
    # takes 16 heads of one row per step.  Forward and backward against the oracle on
    # every element, with the library's own selection (8 indexer heads at H = 64).
    S, topk = 1500, 32
    hi = 8 if H == 64 else 4
    q_idx, k_idx, w_idx = _int_inputs(S, S, seed=H, heads=hi)
    note(f"heads={H} S={S} topk={topk} idx_heads={hi}")
    idx = gpu_index(q_idx, k_idx, w_idx, topk)
    ref_idx = O.index_topk(q_idx, k_idx, w_idx, None, topk)
    assert_idx_equal("idx", idx, ref_idx)
    d = _attn_inputs(S, S, H, seed=7 * H)
    got = gpu_attn(d, idx)
    _check_attn(f"H={H}", got, d, ref_idx, None)


def test_pipelined_wide_heads_8_index_heads():
    # the pipelined entry point over two chunks (so the forward of the first runs beside the
    # indexer of the second) with two groups of heads and 8 indexer heads
    Sq, H, topk = 262_144 + 64, 24, 16
    rng = np.random.default_rng([Sq, H])
    qi, ki, wi = _int_inputs(Sq, Sq, seed=99, heads=8)
    q = _bits(rng.standard_normal((Sq, H, 128), dtype=np.float32))
    k = _bits(rng.standard_normal((Sq, 128), dtype=np.float32))
    v = _bits(rng.standard_normal((Sq, 128), dtype=np.float32))
    dqi, dki, dwi, dq, dk, dv = (dev_bf16(x) for x in (qi, ki, wi, q, k, v))
    note(f"pipelined Sq={Sq} H={H} idx_heads=8 topk={topk}")
    idx_p, out_p, lse_p = D.index_attn_fwd(dqi, dki, dwi, dq, dk, dv, topk=topk, scale=SCALE)
    idx_s = D.index_topk(dqi, dki, dwi, topk=topk)
    out_s, lse_s = D.sparse_attn_fwd(dq, dk, dv, idx_s, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_s) and torch.equal(out_p, out_s) and torch.equal(lse_p, lse_s)
    rows = sample_rows(Sq, topk, None, n_random=24)
    ref_idx = O.index_topk(qi, ki, wi, None, topk, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    assert_idx_equal("pipelined idx", idx_p[sel].cpu().numpy(), ref_idx, rows)
    full_idx = np.zeros((Sq, topk), np.int32)
    full_idx[rows] = ref_idx
    o_ref, lse_ref = O.sparse_attn_fwd(q, k, v, full_idx, None, SCALE, rows=rows)
    assert_close("pipelined O", host_f64(out_p[sel]), o_ref)
    assert_close("pipelined lse", host_f64(lse_p[sel]), lse_ref, max_abs=LSE_ABS, mean_abs=LSE_ABS,
                 rel=1e-4, allowance=False)


@pytest.mark.parametrize("S,H", [(1030, 5), (700, 16)])
def test_backward_dense_selection_long_pool_lists(S, H):
    # every query selects every complete pool, so pool 0 is attended by about
    # S rows: the pool-major dk/dv pass walks lists far longer than one
    # 64-row chunk per wave; H = 5 leaves one (row, head) pair of each step
    # unused, H = 16 gives one row per step
    d = _attn_inputs(S, S, H, seed=S + 31 * H)
    topk = S // 4
    idx = np.full((S, topk), -1, np.int32)
    for i in range(S):
        idx[i, :(i + 1) // 4] = np.arange((i + 1) // 4)
    got = gpu_attn(d, idx)
    _check_attn(f"dense S={S} H={H}", got, d, idx, None)


# ---------------------------------------------------------------------------
# full-size workloads (launch configuration of the benchmark), sampled checks

FULL = ["s32k", "s128k", "zigzag4", "s1m"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_pipeline(name):
    wl = syn.WORKLOADS[name]
    parts = ("index", "attn", "bwd") if wl.backward else ("index", "attn")
    note(f"full {name}: generating inputs")
    d = syn.make_inputs(wl, parts=parts)
    qp = d["q_pos"]
    dev = {k: dev_bf16(d[k]) for k in ("q_idx", "k_idx", "w_idx", "q", "k", "v")}
    tq = None if qp is None else dev_i32(qp)
    note(f"full {name}: GPU pipelined index + fwd{' + bwd' if wl.backward else ''}")
    # the launch configuration the benchmark times: indexer and forward pipelined over query chunks
    idx, out, lse = D.index_attn_fwd(dev["q_idx"], dev["k_idx"], dev["w_idx"], dev["q"], dev["k"],
                                     dev["v"], topk=wl.topk, q_chunk=wl.q_chunk, q_pos=tq, scale=SCALE)
    if wl.backward:
        tdo = dev_bf16(d["dout"])
        dq, dk, dv = D.sparse_attn_bwd(dev["q"], dev["k"], dev["v"], out, tdo, lse, idx, q_pos=tq,
                                       scale=SCALE)
    torch.cuda.synchronize()
    # every row, except at S = 1M: there the edge rows and 4096 random ones
    full_rows = name != "s1m"
    rows = np.arange(wl.sq) if full_rows else sample_rows(wl.sq, wl.topk, qp, n_random=4096)
    note(f"full {name}: oracle on {rows.shape[0]} rows")
    ref_idx = O.index_topk(d["q_idx"], d["k_idx"], d["w_idx"], qp, wl.topk, rows=rows)
    got_idx = idx[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert_idx_equal(f"{name} idx", got_idx, ref_idx, rows)
    # the fp8 indexer on the same integer inputs: the same ids (exact in e4m3)
    idx8 = D.index_topk(dev["q_idx"], dev["k_idx"], dev["w_idx"], topk=wl.topk, q_chunk=wl.q_chunk,
                        q_pos=tq, fp8=True)
    torch.cuda.synchronize()
    assert_idx_equal(f"{name} idx fp8", idx8[torch.from_numpy(rows).cuda()].cpu().numpy(), ref_idx, rows)
    del idx8
    # attention rows: the oracle uses its own selection for those rows
    full_idx = np.zeros((wl.sq, wl.topk), np.int32)
    full_idx[rows] = ref_idx
    o_ref, lse_ref = O.sparse_attn_fwd(d["q"], d["k"], d["v"], full_idx, qp, SCALE, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    assert_close(f"{name} O", host_f64(out[sel]), o_ref)
    assert_close(f"{name} lse", host_f64(lse[sel]), lse_ref, max_abs=LSE_ABS, mean_abs=LSE_ABS, rel=1e-4, allowance=False)
    if wl.backward:
        # every row's dq and every key's dK, dV (the oracle's selection is the whole idx here)
        dq_ref, dk_ref, dv_ref = O.sparse_attn_bwd(d["q"], d["k"], d["v"], d["dout"], full_idx, qp,
                                                   SCALE, rows=rows)
        assert_close(f"{name} dq", host_f64(dq[sel]), dq_ref)
        assert_close(f"{name} dk", host_f64(dk), dk_ref)
        assert_close(f"{name} dv", host_f64(dv), dv_ref)
        # properties that hold at any size: sum_j dV[j] = sum_{r,h} dO[r,h];
        # sum_j dK[j] = scale * sum_{r,h} (sum_j dS) q = 0 up to bf16 rounding of O
        sdv = host_f64(dv).sum(axis=0)
        sdo = host_f64(tdo.float().sum(dim=(0, 1)))
        # every dV[j] is rounded to bf16 once; those independent roundings (variance
        # ulp^2 / 12 each) move the sum over keys by sigma per dim: allow 6 sigma
        a = np.abs(dv_ref)
        ulp = np.where(a > 0, np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7.0), 0.0)
        six_sigma = 6.0 * float(np.sqrt((ulp ** 2).sum(axis=0) / 12.0).max())
        note(f"  {name}: sum dV bar (6 sigma of the bf16 roundings) = {six_sigma:.3e}")
        assert_close(f"{name} sum dV", sdv, sdo, max_abs=six_sigma, mean_abs=six_sigma, rel=1e-3,
                     allowance=False)
        sdk = np.abs(host_f64(dk).sum(axis=0)).max()
        note(f"  {name}: max |sum dK| = {sdk:.3e}")
        assert sdk < 1.0


def test_backward_many_row_chunks_and_pool_slices():
    # 10,000 query rows at scattered positions of a 524,291-key sequence: the
    # inverse selection lists are built over 31 row chunks (the cap on chunk
    # counters binds) and 9 pool slices, the last holding only the partial
    # pool 131,072 (the own pool of the rows at the last 3 positions).  Every
    # row selects 32 of 512 "hot" pools, so each hot pool's rows span every
    # chunk.
    Sk, Sq, H, topk = 524291, 10000, 2, 32
    rng = np.random.default_rng([7, 11])
    pos = rng.choice(np.arange(Sk // 2, Sk - 3), size=Sq - 3, replace=False)
    pos = np.concatenate([pos, [Sk - 3, Sk - 2, Sk - 1]])
    rng.shuffle(pos)
    pos = pos.astype(np.int32)
    hot = rng.choice(Sk // 32, size=512, replace=False)          # below every row's n_c
    idx = np.sort(np.stack([rng.choice(hot, size=topk, replace=False) for _ in range(Sq)]),
                  axis=1).astype(np.int32)
    q = _bits(rng.standard_normal((Sq, H, 128)).astype(np.float32))
    k = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    v = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    dout = _bits(rng.standard_normal((Sq, H, 128)).astype(np.float32))
    note("backward: 31 row chunks x 9 pool slices")
    tq, ti = dev_i32(pos), dev_i32(idx)
    tqq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, lse = D.sparse_attn_fwd(tqq, tk, tv, ti, q_pos=tq, scale=SCALE)
    dq, dk, dv = D.sparse_attn_bwd(tqq, tk, tv, out, dev_bf16(dout), lse, ti, q_pos=tq, scale=SCALE)
    torch.cuda.synchronize()
    hot_keys = (4 * np.sort(hot)[[0, 100, 257, 511]][:, None] + np.arange(4)[None, :]).ravel()
    keys = np.unique(np.concatenate([hot_keys, [Sk - 4, Sk - 3, Sk - 2, Sk - 1, 0],
                                     rng.integers(0, Sk, 6)]))
    rows = np.unique(np.concatenate([rng.integers(0, Sq, 40), np.nonzero(pos >= Sk - 3)[0]]))
    dq_ref, dk_ref, dv_ref = O.sparse_attn_bwd(q, k, v, dout, idx, pos, SCALE, rows=rows, key_rows=keys)
    sel = torch.from_numpy(rows).cuda()
    ks = torch.from_numpy(keys).cuda()
    assert_close("chunked dq", host_f64(dq[sel]), dq_ref)
    assert_close("chunked dk", host_f64(dk[ks]), dk_ref)
    assert_close("chunked dv", host_f64(dv[ks]), dv_ref)
    assert np.abs(dk_ref[np.isin(keys, hot_keys)]).min() > 0   # the hot keys have many rows
    # a pool's rows are summed in ascending row order: a second call gives the same bits
    dq2, dk2, dv2 = D.sparse_attn_bwd(tqq, tk, tv, out, dev_bf16(dout), lse, ti, q_pos=tq, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_backward_repeated_ids_are_safe():
    # The layer requires distinct ids in a row; a row that repeats one is listed once
    # under that pool by the backward's inverse lists (their counts and slots both
    # count rows, not entries), so no list slot is left unwritten: the call completes,
    # the gradients are finite, keys no repeating row touches match the oracle, and a
    # second call gives the same bits.
    Sq, Sk, H, topk = 600, 600, 4, 16
    rng = np.random.default_rng(29)
    pos = np.arange(Sq)
    idx = np.full((Sq, topk), -1, np.int32)
    for r in range(Sq):
        nc = (r + 1) // 4
        m = min(topk, nc)
        if m:
            idx[r, :m] = np.sort(rng.choice(nc, size=m, replace=False))
    rep = [r for r in range(16, 80) if r % 5 == 0]              # rows with 4..20 pools
    idx[rep, 1] = idx[rep, 0]                                   # pool idx[r, 0] twice
    q = _bits(rng.standard_normal((Sq, H, 128)).astype(np.float32))
    k = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    v = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    dout = _bits(rng.standard_normal((Sq, H, 128)).astype(np.float32))
    note(f"backward with {len(rep)} rows repeating an id")
    ti = dev_i32(idx)
    tqq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, lse = D.sparse_attn_fwd(tqq, tk, tv, ti, scale=SCALE)
    grads = [D.sparse_attn_bwd(tqq, tk, tv, out, dev_bf16(dout), lse, ti, scale=SCALE) for _ in range(2)]
    torch.cuda.synchronize()
    for a_, b_ in zip(*grads):
        assert torch.equal(a_, b_) and bool(torch.isfinite(a_.float()).all())
    # keys of pools that no row lists twice and that no repeating row selects
    touched = np.zeros(Sk // 4 + 1, bool)
    for r in rep:
        touched[idx[r][idx[r] >= 0]] = True
        touched[(r + 1) // 4] = True
    clean_pools = np.nonzero(~touched[: Sk // 4])[0]
    keys = (4 * rng.choice(clean_pools, size=12, replace=False)[:, None] + np.arange(4)).ravel()
    _, dk_ref, dv_ref = O.sparse_attn_bwd(q, k, v, dout, idx, pos, SCALE, rows=np.array([Sq - 1]),
                                          key_rows=keys)
    dk1, dv1 = grads[0][1], grads[0][2]
    assert_close("dk, clean keys", host_f64(dk1[torch.from_numpy(keys).cuda()]), dk_ref)
    assert_close("dv, clean keys", host_f64(dv1[torch.from_numpy(keys).cuda()]), dv_ref)


@pytest.mark.parametrize("name", ["s128k", "zigzag4"])
def test_full_size_backward_sampled_keys(name):
    # dK/dV of sampled keys need every query that selected them: use a random
    # valid selection (a legal input of the attention entry points) so the
    # oracle can find those queries without running the indexer on all rows
    wl = syn.WORKLOADS[name]
    d = syn.make_inputs(wl, parts=("attn", "bwd"))
    qp = d["q_pos"]
    pos = np.arange(wl.sq) if qp is None else qp
    note(f"full {name}: random selection")
    idx = syn.random_selection((pos.astype(np.int64) + 1) // 4, wl.topk, seed=1)
    got_t = {}
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    tq = None if qp is None else dev_i32(qp)
    ti = dev_i32(idx)
    out, lse = D.sparse_attn_fwd(q, k, v, ti, q_pos=tq, scale=SCALE)
    dq, dk, dv = D.sparse_attn_bwd(q, k, v, out, dev_bf16(d["dout"]), lse, ti, q_pos=tq, scale=SCALE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    keys = np.unique(np.concatenate([rng.integers(0, wl.sk, 24), [0, 1, 5, int(pos.max()),
                                                                   int(pos.max()) - 3, wl.sk - 1]]))
    rows = sample_rows(wl.sq, wl.topk, qp, n_random=32)
    note(f"full {name}: oracle bwd on {rows.shape[0]} rows, {keys.shape[0]} keys")
    dq_ref, dk_ref, dv_ref = O.sparse_attn_bwd(d["q"], d["k"], d["v"], d["dout"], idx, qp, SCALE,
                                               rows=rows, key_rows=keys)
    sel = torch.from_numpy(rows).cuda()
    ks = torch.from_numpy(keys).cuda()
    assert_close(f"{name} dq", host_f64(dq[sel]), dq_ref)
    assert_close(f"{name} dk", host_f64(dk[ks]), dk_ref)
    assert_close(f"{name} dv", host_f64(dv[ks]), dv_ref)


# ---------------------------------------------------------------------------
# pipelined indexer + forward: equal, bit for bit, to the two separate calls


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("Sq,Sk,H,topk,zigzag,same_stream", [
    (300_001, 300_001, 3, 32, False, False),     # 2 chunks, ragged tail tile
    (262_144, 1 << 20, 2, 16, True, False),      # zig-zag share: q_pos given, 2 chunks
    (1031, 1031, 5, 16, False, False),           # one chunk
    (32_768 * 8, 32_768 * 8, 2, 16, False, False),  # 2 chunks: 32- then 64-query indexer sub-tiles
    (300_001, 300_001, 3, 32, False, True),      # aux stream == stream: sequential
])
def test_pipelined_equals_separate_calls(Sq, Sk, H, topk, zigzag, same_stream, fp8):
    rng = np.random.default_rng([Sq, H, topk])
    qi, ki, wi = _int_inputs(Sq, Sk, seed=Sq + topk)
    q = _bits(rng.standard_normal((Sq, H, 128)).astype(np.float32))
    k = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    v = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    pos = syn.zigzag_positions(Sk, 2, 1)[:Sq] if zigzag else None
    tq = None if pos is None else dev_i32(pos)
    dqi, dki, dwi, dq, dk, dv = (dev_bf16(x) for x in (qi, ki, wi, q, k, v))
    note(f"pipelined Sq={Sq} Sk={Sk} H={H} topk={topk} zigzag={zigzag} same_stream={same_stream} "
         f"fp8={fp8}")
    aux = torch.cuda.current_stream() if same_stream else None
    idx_p, out_p, lse_p = D.index_attn_fwd(dqi, dki, dwi, dq, dk, dv, topk=topk, q_pos=tq,
                                           scale=SCALE, aux_stream=aux, fp8=fp8)
    idx_s = D.index_topk(dqi, dki, dwi, topk=topk, q_pos=tq, fp8=fp8)
    out_s, lse_s = D.sparse_attn_fwd(dq, dk, dv, idx_s, q_pos=tq, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_s), "pipelined idx differs from dsa_index_topk"
    assert torch.equal(out_p, out_s), "pipelined out differs from dsa_sparse_attn_fwd"
    assert torch.equal(lse_p, lse_s), "pipelined lse differs from dsa_sparse_attn_fwd"
    # and the oracle on sampled rows, chunk boundaries included
    # the one inner boundary of 2 chunks: the first takes f/2 of the indexer work
    # (f = 0.75 with the fp8 indexer, 1.05 with the bf16 one)
    bounds = [int(round(Sq * np.sqrt((0.75 if fp8 else 1.05) / 2) / 64)) * 64]
    rows = np.unique(np.concatenate([sample_rows(Sq, topk, pos, n_random=24),
                                     [b + d for b in bounds for d in (-1, 0, 1) if 0 <= b + d < Sq]]))
    ref_idx = O.index_topk(qi, ki, wi, pos, topk, rows=rows)
    assert_idx_equal("pipelined idx", idx_p[torch.from_numpy(rows).cuda()].cpu().numpy(), ref_idx, rows)
    full_idx = np.zeros((Sq, topk), np.int32)
    full_idx[rows] = ref_idx
    o_ref, lse_ref = O.sparse_attn_fwd(q, k, v, full_idx, pos, SCALE, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    assert_close("pipelined O", host_f64(out_p[sel]), o_ref)
    assert_close("pipelined lse", host_f64(lse_p[sel]), lse_ref, max_abs=LSE_ABS, mean_abs=LSE_ABS,
                 rel=1e-4, allowance=False)


@pytest.mark.parametrize("fp8", [False, True])
def test_pipelined_exact_fallback(fp8):
    # the threshold trap at two chunks: nearly every row fails both sampled thresholds, so the
    # exact pass (a small grid while the forward shares the CUs) scores them
    S, topk, H = 262_144 + 100, 64, 1
    k_idx = _threshold_trap_keys(S, 10)
    qi = _bits(np.ones((S, 4, 64), np.float32))
    wi = _bits(np.ones((S, 4), np.float32))
    rng = np.random.default_rng(5)
    q = _bits(rng.standard_normal((S, H, 128)).astype(np.float32))
    k = _bits(rng.standard_normal((S, 128)).astype(np.float32))
    v = _bits(rng.standard_normal((S, 128)).astype(np.float32))
    note(f"pipelined threshold trap, 2 chunks, fp8={fp8}")
    dqi, dki, dwi, dq, dk, dv = (dev_bf16(x) for x in (qi, k_idx, wi, q, k, v))
    ws_p, ws_s = (torch.empty(D.index_topk_ws_bytes(S, S, topk), dtype=torch.uint8, device="cuda")
                  for _ in range(2))
    idx_p, out_p, lse_p = D.index_attn_fwd(dqi, dki, dwi, dq, dk, dv, topk=topk, scale=SCALE, fp8=fp8,
                                           ws=ws_p)
    idx_s = D.index_topk(dqi, dki, dwi, topk=topk, fp8=fp8, ws=ws_s)
    out_s, lse_s = D.sparse_attn_fwd(dq, dk, dv, idx_s, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_s) and torch.equal(out_p, out_s) and torch.equal(lse_p, lse_s)
    # every row with a usable sample fails its first threshold here, and all but a few
    # short rows (whose wider-margin rank exceeds the sample) the retry too: the separate
    # call sends nearly all S rows to the exact pass, and the pipelined call's counters,
    # those of its last chunk (all long rows), every row of that chunk.  The first of the
    # two chunks takes a share f/2 of the indexer work (f = 1.05 with the bf16 indexer,
    # 0.75 with the fp8 one), so the second holds the rows past S * sqrt(f / 2)
    retried_s, exact_s = D.index_topk_stats(ws_s, Sq=S, Sk=S, topk=topk)
    retried_p, exact_p = D.index_topk_stats(ws_p, Sq=S, Sk=S, topk=topk)
    note(f"  separate: retried {retried_s}, exact {exact_s}; pipelined last chunk: {retried_p}, {exact_p}")
    f = 0.75 if fp8 else 1.05
    last = S - int(round(S * np.sqrt(f / 2) / 64)) * 64
    assert exact_s > 0.99 * S and exact_s <= retried_s < exact_s + 0.01 * S
    assert retried_p == exact_p == last
    rows = sample_rows(S, topk, None, n_random=16)
    ref = O.index_topk(qi, k_idx, wi, None, topk, rows=rows)
    assert_idx_equal("pipelined trap idx", idx_p[torch.from_numpy(rows).cuda()].cpu().numpy(), ref, rows)


def test_forward_staged_and_register_k_agree():
    # the forward stages K through LDS for key sets of at most 2^17 keys and loads it into
    # MFMA registers above that; both orders give the same products.  The same 512 queries,
    # at positions below 2^17, against exactly 2^17 keys and against 256 more that no query
    # can select (they lie past every query's causal range): ids, O and LSE equal bit for bit
    Sq, Sk0, H, topk = 512, 1 << 17, 16, 512
    rng = np.random.default_rng([Sk0, 17])
    qi, ki, wi = _int_inputs(Sq, Sk0 + 256, seed=17)
    q = _bits(rng.standard_normal((Sq, H, 128)).astype(np.float32))
    k = _bits(rng.standard_normal((Sk0 + 256, 128)).astype(np.float32))
    v = _bits(rng.standard_normal((Sk0 + 256, 128)).astype(np.float32))
    pos = np.sort(rng.choice(Sk0, size=Sq, replace=False)).astype(np.int32)
    pos[-8:] = np.arange(Sk0 - 8, Sk0, dtype=np.int32)   # rows that reach the last keys
    tq = dev_i32(pos)
    dqi, dwi, dq = dev_bf16(qi), dev_bf16(wi), dev_bf16(q)
    res = []
    for Sk in (Sk0, Sk0 + 256):
        note(f"forward, {Sk} keys ({'K staged' if Sk <= Sk0 else 'K in registers'})")
        dki, dk, dv = dev_bf16(ki[:Sk]), dev_bf16(k[:Sk]), dev_bf16(v[:Sk])
        res.append(D.index_attn_fwd(dqi, dki, dwi, dq, dk, dv, topk=topk, q_pos=tq, scale=SCALE))
    torch.cuda.synchronize()
    for name, a, b in zip(("idx", "out", "lse"), res[0], res[1]):
        assert torch.equal(a, b), f"{name} differs between the staged and the register K forward"
    rows = sample_rows(Sq, topk, pos, n_random=12)
    ref_idx = O.index_topk(qi, ki[:Sk0], wi, pos, topk, rows=rows)
    assert_idx_equal("staged-K idx", res[0][0][torch.from_numpy(rows).cuda()].cpu().numpy(), ref_idx, rows)
    full_idx = np.zeros((Sq, topk), np.int32)
    full_idx[rows] = ref_idx
    o_ref, _ = O.sparse_attn_fwd(q, k[:Sk0], v[:Sk0], full_idx, pos, SCALE, rows=rows)
    assert_close("staged-K O", host_f64(res[0][1][torch.from_numpy(rows).cuda()]), o_ref)


def test_s4k_workload_every_row():
    # the S = 4096 workload (H = 4, top-128, its own seeded inputs) through the benchmark's entry
    # point, compared element by element on every row: idx exactly, O and LSE to tolerance
    wl = syn.WORKLOADS["s4k"]
    d = syn.make_inputs(wl, parts=("index", "attn"))
    note("s4k workload, every row")
    t = {n: dev_bf16(d[n]) for n in ("q_idx", "k_idx", "w_idx", "q", "k", "v")}
    idx, out, lse = D.index_attn_fwd(t["q_idx"], t["k_idx"], t["w_idx"], t["q"], t["k"], t["v"],
                                     topk=wl.topk, q_chunk=wl.q_chunk, scale=SCALE)
    torch.cuda.synchronize()
    ref_idx = O.index_topk(d["q_idx"], d["k_idx"], d["w_idx"], None, wl.topk)
    assert_idx_equal("s4k idx", idx.cpu().numpy(), ref_idx)
    o_ref, lse_ref = O.sparse_attn_fwd(d["q"], d["k"], d["v"], ref_idx, None, SCALE)
    assert_close("s4k O", host_f64(out), o_ref)
    assert_close("s4k lse", host_f64(lse), lse_ref, max_abs=LSE_ABS, mean_abs=LSE_ABS, rel=1e-4, allowance=False)


@pytest.mark.parametrize("Sq,Sk,H,topk,permute", [
    (262_144 + 64, 600_000, 2, 64, True),     # 2 chunks, positions in no order, caller's stream
    (262_144, 262_144, 16, 2048, False),      # 2 chunks at the largest k (up to 8195 keys a row)
])
def test_pipelined_positions_and_largest_k(Sq, Sk, H, topk, permute):
    rng = np.random.default_rng([Sq, topk, 3])
    qi, ki, wi = _int_inputs(Sq, Sk, seed=topk + 5)
    q = _bits(rng.standard_normal((Sq, H, 128)).astype(np.float32))
    k = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    v = _bits(rng.standard_normal((Sk, 128)).astype(np.float32))
    pos = rng.choice(Sk, size=Sq, replace=False).astype(np.int32) if permute else None
    tq = None if pos is None else dev_i32(pos)
    dqi, dki, dwi, dq, dk, dv = (dev_bf16(x) for x in (qi, ki, wi, q, k, v))
    note(f"pipelined Sq={Sq} Sk={Sk} H={H} topk={topk} permute={permute}")
    aux = torch.cuda.Stream()   # a second stream of the caller's own
    idx_p, out_p, lse_p = D.index_attn_fwd(dqi, dki, dwi, dq, dk, dv, topk=topk, q_pos=tq, scale=SCALE,
                                           aux_stream=aux)
    idx_s = D.index_topk(dqi, dki, dwi, topk=topk, q_pos=tq)
    out_s, lse_s = D.sparse_attn_fwd(dq, dk, dv, idx_s, q_pos=tq, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_s) and torch.equal(out_p, out_s) and torch.equal(lse_p, lse_s)
    rows = sample_rows(Sq, topk, pos, n_random=16)
    ref_idx = O.index_topk(qi, ki, wi, pos, topk, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    assert_idx_equal("pipelined idx", idx_p[sel].cpu().numpy(), ref_idx, rows)
    full_idx = np.zeros((Sq, topk), np.int32)
    full_idx[rows] = ref_idx
    o_ref, lse_ref = O.sparse_attn_fwd(q, k, v, full_idx, pos, SCALE, rows=rows)
    assert_close("pipelined O", host_f64(out_p[sel]), o_ref)
    assert_close("pipelined lse", host_f64(lse_p[sel]), lse_ref, max_abs=LSE_ABS, mean_abs=LSE_ABS,
                 rel=1e-4, allowance=False)
