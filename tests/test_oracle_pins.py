"""The CPU oracle against its pins (no GPU)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_config1_rate():
    """Config 1 lands at 1.00 % changed (within 0.5 % relative), 64 flips included."""
    import numpy as np
    from bit_exact_xor_amd import synth
    lay = synth.config1_layout()
    old, new, _lr, pos = synth.config1_values(lay, lr=synth.CFG1_LR)
    frac = np.count_nonzero(old != new) / old.size
    assert abs(frac - 0.01) <= 0.01 * 0.005, frac
    assert len(set(pos.tolist())) == 64


def test_generator_rates():
    """Bernoulli thresholds give the configured rate (+-0.5 % relative at 4M draws)."""
    import numpy as np
    from bit_exact_xor_amd import synth
    for rate in (0.01, 0.03, 0.05, 0.00085):
        ch, _up, _h = synth.change_mask(synth.derive_key(1, 2, 1), 0, 1 << 22, synth.rate_thr(rate))
        got = ch.mean()
        tol = 0.005 if rate >= 0.01 else 0.03
        assert abs(got - rate) <= rate * tol, (rate, got)
