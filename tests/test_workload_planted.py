"""The planted long-prefill workload is what it claims to be: its planted
blocks stand out from the rest by a clear margin in the oracle's block
scores.  Prints the realised gap (the recipe fixes the per-key mean shift,
not the block-max gap, so the latter is reported as measured)."""
import numpy as np
import pytest

import oracle
import workloads as W


@pytest.mark.slow
def test_planted_gap_is_realised_and_printed():
    w = W.config(2)
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(w.T, size=96, replace=False)).astype(np.int32)
    g = oracle.planted_gap(w, tokens)
    print("planted-vs-unplanted block max gap:", g)
    assert len(w.meta["planted_blocks"]) == 13
    assert g["gap"] > 0 and g["gap_in_unplanted_sd"] > 1.0
    # planted blocks are 5% of the blocks but take far more of the free slots
    assert g["planted_share_of_free_slots"] > 0.15
