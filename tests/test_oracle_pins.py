"""The oracle against facts that mathematics fixes (see ``oracle_pins``).

The pages print no worked numerical example, so these pins stand in for one:
high-precision brute force, scipy's softmax/logsumexp, closed forms and
invariants of softmax attention.
"""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.load())


def test_thread_split_is_bitwise_neutral():
    """Splitting rows across host threads does not change a single bit."""
    import numpy as np
    from oracle_pins import rand_bf16
    rng = np.random.default_rng(5)
    q, k, v = (rand_bf16(rng, (2, 3, 50, 16)) for _ in range(3))
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, causal, 0.25, threads=1)
        o4, l4 = oracle.attention(q, k, v, causal, 0.25, threads=4)
        assert np.array_equal(o1, o4) and np.array_equal(l1, l4)


def test_rows_api_matches_full():
    import numpy as np
    from oracle_pins import rand_bf16
    rng = np.random.default_rng(6)
    q, k, v = (rand_bf16(rng, (2, 2, 30, 8)) for _ in range(3))
    o, lse = oracle.attention(q, k, v, True, 0.3)
    rows = np.array([0, 29, 31, 77, 119])
    ro, rl = oracle.attention_rows(q, k, v, True, 0.3, rows, threads=2)
    assert np.array_equal(ro, o.reshape(-1, 8)[rows])
    assert np.array_equal(rl, lse.reshape(-1)[rows])


def test_rejects_bad_rows():
    import numpy as np
    from oracle_pins import rand_bf16
    rng = np.random.default_rng(7)
    q, k, v = (rand_bf16(rng, (1, 1, 4, 2)) for _ in range(3))
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v, False, 1.0, [4])
