"""CPU tests: the fp64 oracle against its pins (hand-worked fixtures, closed forms,
invariants, brute force, library routines)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("name", pins.all_pin_names())
def test_pin(name):
    getattr(pins, name)()


def test_oracle_rejects_bad_arguments():
    X = np.zeros((1, 4), np.float32)
    W = np.zeros((3, 4), np.float16)
    with pytest.raises(ValueError):
        oracle.forward(X, W, W, np.array([0, 3], np.int32))       # index out of range
    with pytest.raises(ValueError):
        oracle.permutation(np.zeros(5, np.int64), 6)               # more hot than neurons
    with pytest.raises(ValueError):
        oracle.compact(np.zeros((65, 4), np.uint8))                # more than 64 tokens


def test_n_hot_rule():
    assert oracle.n_hot_for(16384, 0.20) == 3277
    assert oracle.n_hot_for(3072, 0.20) == 615
    assert oracle.n_hot_for(49152, 0.10) == 4916
    assert oracle.n_hot_for(11008, 0.20) == 2202
    assert oracle.n_hot_for(8, 0.5) == 4
