"""The oracle against its pins (CPU only).  See tests/oracle_pins.py."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_oracle_refuses_a_bank_its_strides_overrun(oracle_lib):
    """The C oracle trusts its strides; the wrapper checks that the bank
    buffer holds every element they address before calling it."""
    import numpy as np
    import oracle
    T, H, cap = 3, 16, 4
    prefix = np.zeros((T, H), dtype=np.uint16)
    w = np.full(H, 0x3F80, dtype=np.uint16)                  # bf16 1.0
    slot_major = np.zeros(cap * T * H, dtype=np.uint16)      # [cap, T, H]
    r = oracle.attnres_oracle(prefix, None, slot_major, H, T * H, cap, 2, w, w, 1e-6, None, 0.0,
                              -1, lib=oracle_lib)
    assert r.out_bits.shape == (T, H)
    with pytest.raises(ValueError):
        # the first token's slice only: slots 1.. of it lie past its end
        oracle.attnres_oracle(prefix[:1], None, slot_major[:H], H, T * H, cap, 2, w, w, 1e-6,
                              None, 0.0, -1, lib=oracle_lib)
