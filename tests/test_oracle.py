"""The CPU oracle against its pins (no GPU).  See tests/oracle_pins.py."""
import os

import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    fails = pin(orc)
    assert not fails, "\n".join(fails[:10])


# Planted mistakes: each is a plausible slip in the oracle; at least one pin
# must catch it (the planted copy is built into a temp dir, never used by the
# product or the other tests).
PLANTS = {
    "nibble": [pins.pin_golden],          # element j / j+16 nibbles swapped
    "offset": [pins.pin_golden],          # the -8 of Q4_0 dropped
    "half": [pins.pin_codec],             # subnormal binary16 decoded as normal
    "round": [pins.pin_golden],           # ties to even instead of away from zero
    "d32": [pins.pin_nearest],            # divide by the fp32 scale, not the stored fp16 one
    "xindex": [pins.pin_exact_gemv],      # activation index slip (k ^ 1)
    "drop": [pins.pin_exact_gemv],        # last block of each row dropped from the sum
    "scaleidx": [pins.pin_prefill],       # scale of the next block used
    "silu": [pins.pin_silu],              # e^v instead of e^-v in silu
    "glu": [pins.pin_swiglu],             # silu applied to the up half, not the gate
    "actround": [pins.pin_act8],          # activation codes rounded half away from zero
    "actscale": [pins.pin_act8],          # the next block's activation scale used
    "q2order": [pins.pin_q2w],            # 2-bit codes read as four consecutive per byte
}


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_planted_mistake_is_caught(plant, tmp_path):
    path = oracle.build(plant=plant, out=str(tmp_path / f"liboracle_{plant}.so"))
    bad = oracle.Oracle(path)
    caught = []
    for pin in PLANTS[plant]:
        caught += pin(bad)
    assert caught, f"planted mistake '{plant}' passed every pin"


def test_sabotaged_bytes_fail_every_check(orc):
    """Corrupting the packed bytes (every code byte XOR 0x11, every scale's sign
    flipped) must fail the acceptance bound on every check; the clean bytes are
    what the reference keeps [volta-kernel-bakeoff, "Making it fair"]."""
    import seeded_inputs as si
    for fmt in (oracle.Q4_0, oracle.Q8_0):
        N, K = 64, 256
        p = orc.quantize(fmt, si.weights(N, K, seed=1))
        x = si.activations(4, K, seed=1)
        y_ref, s = orc.gemv(fmt, p, N, K, x)
        bad = p.copy()
        nb = N * K // 32
        cb = 16 if fmt == oracle.Q4_0 else 32
        bad[:nb * cb] ^= 0x11
        s0 = (nb * cb + 255) // 256 * 256
        bad[s0 + 1:s0 + 2 * nb:2] ^= 0x80
        y_bad, _ = orc.gemv(fmt, bad, N, K, x)
        ok = oracle.within_bound(y_bad, y_ref, s)
        # one check = one call; it fails if any element is outside the bound,
        # and here nearly every element is
        assert ok.mean() < 0.05


def test_quantizer_rejects_non_finite(orc):
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = np.inf
    with pytest.raises(ValueError):
        orc.quantize(oracle.Q4_0, w)
    w[0, 3] = 1e6  # fl32(1e6 / 7) overflows binary16
    with pytest.raises(ValueError):
        orc.quantize(oracle.Q4_0, w)
    assert orc.packed_bytes(oracle.Q4_0, 4, 48) == 0
