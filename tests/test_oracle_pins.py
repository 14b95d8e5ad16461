"""The CPU oracle against what the method's definition and mathematics fix."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_layer_wrapper_matches_per_head_calls():
    r = np.random.default_rng(3)
    X = [r.standard_normal((2, 3, 20, 8)) for _ in range(4)]
    for kind, fn in (("linear", oracle.linear_attention), ("softmax", oracle.softmax_attention)):
        out = oracle.layer(kind, *X)
        for b in range(2):
            for h in range(3):
                assert np.array_equal(out[b, h], fn(*(x[b, h] for x in X)))
    rows = np.array([1, 7, 19])
    assert np.array_equal(oracle.layer("softmax", *X, rows=rows), oracle.layer("softmax", *X)[:, :, rows])
    with pytest.raises(ValueError):
        oracle.layer("cosine", *X)


def test_group_rejects_wrong_layer_count():
    X = [np.zeros((3, 1, 1, 4, 4)) for _ in range(4)]
    with pytest.raises(ValueError):
        oracle.group(*X)
