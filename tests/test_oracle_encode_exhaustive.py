"""The oracle's E4M3 encoder against torch's float8_e4m3fn cast on every finite float32
value v with 2^-12 <= |v| < 464, both signs: 21 binades of 2^23 values each (survey
check P2, done exhaustively).  Below 2^-12 every value encodes to a signed zero (the
smallest code step is 2^-9, so its rounding midpoint is 2^-10); from 464 up torch's cast
gives NaN where the oracle saturates at 448, and [448, 464) rounds to 448 on both sides.
Takes about half a minute on one core."""
import numpy as np
import pytest

import pins


@pytest.mark.slow
@pytest.mark.parametrize("sign", [1.0, -1.0], ids=["pos", "neg"])
def test_encoder_every_float_in_range(orc, sign):
    for e in range(-12, 9):                              # binade [2^e, 2^(e+1))
        v = (np.arange(1 << 23, dtype=np.uint32) | np.uint32((e + 127) << 23)).view(np.float32)
        if e == 8:
            v = v[v < np.float32(464.0)]
        v = (v * np.float32(sign)).astype(np.float32)
        mine = orc.e4m3_encode(v)
        ref = pins.torch_e4m3_encode(v)
        bad = np.nonzero(mine != ref)[0]
        assert bad.size == 0, "binade 2^%d: encoder differs from torch at %r" % (e, v[bad[:5]])


def test_below_range_encodes_to_signed_zero(orc):
    """A sweep below 2^-12 (every 2^13-th pattern of every binade from the smallest
    subnormal up): all codes are 0x00 for +v and 0x80 for -v, as torch's cast gives."""
    pats = np.arange(1, (127 - 12) << 23, 1 << 13, dtype=np.uint32)
    v = pats.view(np.float32)
    assert v.max() < np.float32(2.0 ** -12)
    assert np.all(orc.e4m3_encode(v) == 0x00) and np.all(pins.torch_e4m3_encode(v) == 0x00)
    assert np.all(orc.e4m3_encode(-v) == 0x80) and np.all(pins.torch_e4m3_encode(-v) == 0x80)
