"""The fp64 oracle against hand-worked examples, exact rational brute force,
special cases with textbook answers and invariants (no GPU)."""
import pytest

import oracle
from oracle_pins import gemv_pins, gemv_q8_pins, markov_pins, markov_q8_pins, probe_pins


def _ids(pins):
    return [p[0] for p in pins]


@pytest.mark.parametrize("suite,fn", [
    (markov_pins, oracle.markov_sample),
    (gemv_pins, oracle.gemv),
    (probe_pins, oracle.conf_probe),
], ids=["markov_sample", "gemv", "conf_probe"])
def test_oracle_meets_every_pin(suite, fn):
    results = suite(fn)
    failed = [(n, d) for n, ok, d in results if not ok]
    assert not failed, failed


def test_q8_oracle_meets_every_pin():
    failed = [(n, d) for n, ok, d in gemv_q8_pins(oracle.gemv_q8, oracle.gemv) if not ok]
    failed += [(n, d) for n, ok, d in markov_q8_pins(oracle.markov_sample_q8, oracle.markov_sample) if not ok]
    assert not failed, failed


def test_markov_step_matches_loop():
    """The single-step function (used for teacher-forced checks) agrees with
    the loop when fed the loop's own previous tokens."""
    import numpy as np
    from gemv_markov_argmax_amd import synth
    base, w1, w2, prev0, _ = synth.markov_inputs(1, 5, 500, 16, seed=3)
    out = oracle.markov_sample(base, w1, w2, prev0, 5)
    prev = int(prev0[0])
    for i in range(5):
        st = oracle.markov_step(base[0, i], w1, w2, prev)
        assert st.tok == out["tok"][0, i] and st.margin == out["margin"][0, i]
        prev = st.tok


def test_oracle_rejects_out_of_range_prev():
    import numpy as np
    w = np.zeros((4, 2), np.uint16)
    with pytest.raises(ValueError):
        oracle.markov_step(np.zeros(4, np.float32), w, w, 4)
