"""The structured-mask FLOP count (workloads.visible_pairs_general) against
a pair-by-pair count with the oracle's visibility rule (no GPU)."""

import pytest

from exact_tiled_attention_attn_amd.workloads import (VARLEN_WORKLOADS, visible_pairs_general,
                                                      visible_scores_per_head)
from oracle import visible


@pytest.mark.parametrize("rule", [(False, 0, 0, 0), (True, 0, 0, 0), (True, 9, 0, 0),
                                  (False, 0, 5, 0), (False, 0, 5, 3), (True, 0, 4, 6),
                                  (True, 7, 3, 2), (False, 0, 0, 5), (False, 0, 40, 2)])
@pytest.mark.parametrize("N", [1, 2, 17, 64])
def test_pair_count_matches_brute_force(rule, N):
    causal, window, radius, n_global = rule
    brute = sum(visible(i, j, causal, window, radius, n_global)
                for i in range(N) for j in range(N))
    assert visible_pairs_general(N, causal, window, radius, n_global) == brute


def test_reduces_to_the_forward_count():
    for N in (1, 100, 1000):
        for causal, window in ((False, 0), (True, 0), (True, 33)):
            assert (visible_pairs_general(N, causal, window, 0, 0)
                    == visible_scores_per_head(N, causal, window))


def test_workloads_are_well_formed():
    for w in VARLEN_WORKLOADS.values():
        assert all(L >= 1 for L in w.lens) and w.Hq % w.Hkv == 0
