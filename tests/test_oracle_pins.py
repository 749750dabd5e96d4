"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

from oracle import wkv7_sequence, wkv7_forward, wkv7_decode_batch
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(wkv7_sequence)


def test_forward_packs_sequences_and_slots():
    """wkv7_forward = per-sequence wkv7_sequence on its own slot's state."""
    rng = np.random.default_rng(5)
    H, N = 2, 8
    lens = [3, 0, 5, 1]
    ids = [7, 2, 4, 0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    x = {n: rng.standard_normal((T, H, N)) for n in P.NAMES}
    x["w"] = np.exp(-np.exp(rng.normal(-0.6, 0.5, (T, H, N))))
    states = {7: rng.standard_normal((H, N, N)), 0: rng.standard_normal((H, N, N))}
    o, out = wkv7_forward(states, ids, cu, x, H, N)
    for s, slot in enumerate(ids):
        lo, hi = cu[s], cu[s + 1]
        S0 = states.get(slot, np.zeros((H, N, N)))
        o_s, S_s = wkv7_sequence(S0, **{n: x[n][lo:hi] for n in P.NAMES})
        assert np.array_equal(o[lo:hi], o_s)
        assert np.array_equal(out[slot], S_s)
    # the zero-length sequence leaves its (zero) slot unchanged
    assert np.array_equal(out[2], np.zeros((H, N, N)))
    with pytest.raises(ValueError):
        wkv7_forward(states, [1, 1], [0, 1, 2], {n: x[n][:2] for n in P.NAMES},
                     H, N)


def test_decode_batch_equals_sequences():
    rng = np.random.default_rng(6)
    B, H, N = 5, 3, 8
    S0 = rng.standard_normal((B, H, N, N))
    x = {n: rng.standard_normal((B, H, N)) for n in P.NAMES}
    o, S1 = wkv7_decode_batch(S0, x)
    for bb in range(B):
        o_s, S_s = wkv7_sequence(S0[bb], **{n: x[n][bb:bb + 1] for n in P.NAMES})
        assert np.array_equal(o[bb], o_s[0])
        assert np.array_equal(S1[bb], S_s)
