"""The shaped caches of the softmax edge tests have the score shapes those
tests rely on (checked with the oracle's scores, on the CPU)."""
import numpy as np
import pytest

import oracle
from edge_inputs import base2_scores, shaped_cache


@pytest.mark.parametrize("layout", [(4, 8, 4), (4, 12, 4), (4, 12, 8), (8, 8, 4), (5, 12, 4)])
def test_sink_dominates_by_the_stated_gap(layout):
    g, kb, sd = layout
    c = shaped_cache("sink_const", g, kb, sd, 4096, seed=1)
    for h in range(g):
        s = base2_scores(c, 0, h)
        assert s[0] - np.max(s[1:]) > 18.0 * (1 + 0.08 * h)
    # every token has the same value row, with entries of magnitude ~30
    v = oracle.vq_decode(oracle.unpack_codes(c.codes_v[0, 0, :4096], c.wl.v_bits, 128 // sd),
                         c.cb_v[0])
    assert np.all(v == v[0]) and np.abs(v[0]).min() > 25.0


def test_sink_tail_values_have_opposite_signs():
    c = shaped_cache("sink_tail", 4, 8, 4, 4096, seed=1)
    v = oracle.vq_decode(oracle.unpack_codes(c.codes_v[0, 0, :4096], 8, 32), c.cb_v[0])
    assert np.all(v[0] < -25.0) and np.all(v[1:] > 25.0)


@pytest.mark.parametrize("layout", [(4, 8, 4), (4, 12, 8)])
def test_climb_exceeds_the_rescale_slack_every_512_tokens(layout):
    g, kb, sd = layout
    c = shaped_cache("climb", g, kb, sd, 16384, seed=1)
    s = base2_scores(c, 0, 0)
    climb = s[512::512] - s[:-512:512]
    assert climb.min() > 10.0


@pytest.mark.parametrize("kind,sign", [("large_pos", 1), ("large_neg", -1)])
def test_large_scores(kind, sign):
    c = shaped_cache(kind, 4, 12, 4, 4096, seed=1)
    s = base2_scores(c, 0, 0)
    assert np.all(sign * s > 600.0)
    assert np.ptp(s) > 5.0
