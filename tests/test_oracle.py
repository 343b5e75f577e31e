"""The CPU oracle against its pins (see tests/oracle_pins.py)."""
import numpy as np
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_mod, pin):
    pin(None)


def test_oracle_rejects_bad_arguments(oracle_mod):
    q = np.zeros((1, 2, 4, 8))
    k = np.zeros((1, 2, 3, 8))
    with pytest.raises(ValueError):          # Hq % Hkv != 0
        oracle_mod.ref_attention(q, k, k, np.zeros((4, 2)), [2])
    k = np.zeros((1, 2, 2, 8))
    with pytest.raises(ValueError):          # fewer keys than queries
        oracle_mod.ref_attention(q, k, k, np.zeros((4, 2)), [1])
    with pytest.raises(ValueError):          # more keys than the array holds
        oracle_mod.ref_attention(q, k, k, np.zeros((4, 2)), [3])


def test_sampled_rows_equal_full_call(oracle_mod):
    from relative_bias_gqa_amd import synth
    c = synth.make_prefill(3, 2, 40, 70, 4, 2, 16, 9, "bf16")
    out, lse, _ = oracle_mod.ref_prefill(c.q, c.k, c.v, c.bias, c.window)
    rows = [(0, 0), (1, 39), (0, 17), (1, 5)]
    o, l = oracle_mod.ref_prefill_rows(c.q, c.k, c.v, c.bias, c.window, rows)
    for n, (b, t) in enumerate(rows):
        assert np.array_equal(o[n], out[b, t]) and np.array_equal(l[n], lse[b, t])
