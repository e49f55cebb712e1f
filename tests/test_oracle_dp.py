"""Pins for the data-parallel shard helpers of the oracle and the host-only
C-ABI functions ([P1] 关键源码片段 _get_dp_gather_slot; [P2] 实现拆解 items 3-4,
TP-major head shards and rank-major row selection)."""
import numpy as np
import pytest

import layer_embedding_lookup_amd as ple
import oracle


def test_dp_gather_slot_worked_examples():
    counts = [5, 9, 2, 7]
    # groups of 2: ranks {0,1} share slot 9, ranks {2,3} share slot 7
    assert [oracle.dp_gather_slot(counts, 2, r) for r in range(4)] == [(9, 0), (9, 9), (7, 0), (7, 7)]
    # one group of 4: slot 9, offsets 0, 9, 18, 27
    assert [oracle.dp_gather_slot(counts, 4, r) for r in range(4)] == [(9, 0), (9, 9), (9, 18), (9, 27)]
    # no sharding across DP: the replica's own count, offset 0 (the page's early return)
    assert [oracle.dp_gather_slot(counts, 1, r) for r in range(4)] == [(5, 0), (9, 0), (2, 0), (7, 0)]


def test_dp_gather_slot_abi_matches_oracle():
    rng = np.random.default_rng(3)
    for _ in range(200):
        g = int(rng.choice([1, 2, 4, 8]))
        dp = g * int(rng.integers(1, 4))
        counts = rng.integers(0, 5000, dp)
        r = int(rng.integers(0, dp))
        assert ple.ple_dp_gather_slot(counts, g, r) == oracle.dp_gather_slot(counts, g, r)


def test_head_shard_tp_major():
    # 8 heads over TP 2 x DP 2: the TP rank is the major index
    got = {(tp, dp): oracle.head_shard(8, 2, tp, 2, dp) for tp in range(2) for dp in range(2)}
    assert got == {(0, 0): (0, 2), (0, 1): (2, 2), (1, 0): (4, 2), (1, 1): (6, 2)}
    assert oracle.head_shard(6, 2, 0, 2, 0) is None   # uneven
    assert oracle.head_shard(2, 2, 0, 2, 0) is None   # empty shards
    for H, tp, dp in [(8, 2, 2), (16, 2, 4), (8, 1, 8), (4, 4, 1)]:
        for a in range(tp):
            for b in range(dp):
                assert ple.ple_head_shard(H, tp, a, dp, b) == oracle.head_shard(H, tp, a, dp, b)
    with pytest.raises(RuntimeError):
        ple.ple_head_shard(6, 2, 0, 2, 0)


def test_select_rows_inverts_the_rank_major_layout():
    """Scatter per-rank rows into the gathered layout (written here from the
    layout's description), then selecting rank r's window gives them back."""
    rng = np.random.default_rng(4)
    E, W = 3, 16
    counts = [5, 2, 4]
    S = max(counts)
    F = [rng.integers(0, 65536, size=(n, E * W), dtype=np.uint16) for n in counts]
    gathered = rng.integers(0, 65536, size=(E, E * S, W), dtype=np.uint16)  # padding rows stay random
    for r in range(E):
        for t in range(counts[r]):
            for k in range(E):
                gathered[k, r * S + t, :] = F[r][t, k * W:(k + 1) * W]
    for r in range(E):
        np.testing.assert_array_equal(oracle.select_rows(gathered, r, counts[r]), F[r])
