"""bench.py's work accounting against closed forms (CPU).

The roofline figures divide algorithmic flops or bytes per launch by measured
durations; these tests pin the per-launch counts for the identity-position
workloads (S = 4m query rows at positions 0 .. S-1) to sums written out by hand:

  nc(t) = floor((t + 1) / 4) complete pools before query t, part(t) = (t + 1) mod 4
  sum_t nc(t)            = 2 m^2 - m
  sum_t part(t)          = 6 m
  sum_t [part(t) > 0]    = 3 m
  sum_t min(nc(t), k)    = 2 k (k + 1) + 4 k (m - 1 - k) + k      (m > k)

A query scores 4 heads x 64 dims against each complete pool (512 flops a pair),
gathers 4 min(nc, k) + part keys of 512 bytes (a K and a V row), and reads its
Q row and writes its O row (2 H 128 bf16), its LSE (4 H bytes) and its k ids.
"""
import pytest

import bench
import synthetic as syn


def closed_forms(S, H, k):
    assert S % 4 == 0
    m = S // 4
    assert m > k
    sum_nc = 2 * m * m - m
    sum_min = 2 * k * (k + 1) + 4 * k * (m - 1 - k) + k
    keys = 4 * sum_min + 6 * m
    return {
        "index_pairs": sum_nc,
        "index_flop": 512 * sum_nc,
        "keys": keys,
        "entries": sum_min + 3 * m,
        "fwd_bytes": 512 * keys + (2 * H * 128 * 2 + 4 * H + 4 * k) * S,
    }


@pytest.mark.parametrize("name", ["s4k", "s32k", "s128k", "s1m"])
def test_work_matches_closed_forms(name):
    wl = syn.WORKLOADS[name]
    assert wl.q_positions() is None and wl.sq == wl.sk
    got = bench.work(wl)
    want = closed_forms(wl.sq, wl.heads, wl.topk)
    for key, value in want.items():
        assert got[key] == value, (name, key, got[key], value)


def test_s1m_indexer_flops_and_gathered_bytes():
    # the figures the S = 1M roofline is quoted with: 7.04e13 indexer flops per launch
    # (2^38 query-pool pairs, less the incomplete pools) and 1.11e12 forward bytes
    got = bench.work(syn.WORKLOADS["s1m"])
    assert got["index_flop"] == 512 * (2 ** 37 - 2 ** 18)
    assert abs(got["fwd_bytes"] / 1.1102e12 - 1) < 1e-3


def test_zigzag_share_counts_its_own_positions():
    # the zig-zag share's rows sit at positions [S/8, S/4) and [3S/4, 7S/8) of S = 2^18: the
    # pool pairs are the sum of floor((p + 1) / 4) over exactly those positions
    wl = syn.WORKLOADS["zigzag4"]
    pos = syn.zigzag_positions(wl.sk, 4, 1)
    assert len(pos) == wl.sq
    want = int(((pos.astype("int64") + 1) // 4).sum())
    assert bench.work(wl)["index_pairs"] == want
