"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def test_gather_selection_matches_full(orc):
    """Selected-output evaluation equals the full evaluation on those outputs."""
    import numpy as np
    import synth
    inp = synth.make(synth.WORKLOADS["C4"].scaled(N=40, K=64, E=8))
    y, A = orc.gather("cb3", inp.codes, inp.scales, inp.ids, "q8", inp.x, inp.xs, x_per_slot=True)
    outs = np.array([0, 7, 39, 40, 81, 159], np.int64)
    ys, As = orc.gather("cb3", inp.codes, inp.scales, inp.ids, "q8", inp.x, inp.xs,
                        x_per_slot=True, outs=outs)
    assert np.array_equal(ys, y.reshape(-1)[outs])
    assert np.array_equal(As, A.reshape(-1)[outs])
