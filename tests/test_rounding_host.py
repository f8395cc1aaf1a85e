"""Host check of the rounding the requantisation kernel uses (no GPU).

The kernel rounds x = v * (1/d) half away from zero as trunc(x + c) with c
the largest float32 below one half carrying x's sign.  The quotient never
exceeds 127 in magnitude by more than a rounding, so every float32 with
|x| <= 128 is checked here against the plain definition (floor(|x| + 1/2)
with x's sign, in float64, where that sum is exact)."""
import numpy as np

C = np.float32(np.nextafter(np.float32(0.5), np.float32(0.0)))


def test_constant():
    assert C == np.float32(0.5) - np.float32(2.0 ** -25)


def test_every_float_up_to_128():
    """Every x in [0, 128]; float32 addition rounds to nearest, so
    -x + (-c) = -(x + c) and the negative half mirrors this one (its ties
    are checked below)."""
    top = int(np.array(128.0, dtype=np.float32).view(np.uint32))
    step = 1 << 23
    for lo in range(0, top + 1, step):
        x = np.arange(lo, min(lo + step, top + 1), dtype=np.uint32).view(np.float32)
        got = np.trunc(x + C).astype(np.int32)
        want = np.floor(x.astype(np.float64) + 0.5).astype(np.int32)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (x[bad[:4]], got[bad[:4]], want[bad[:4]])


def test_ties_and_neighbours():
    for k in range(-128, 128):
        t = np.float32(k + 0.5)
        below, above = np.nextafter(t, np.float32(-np.inf)), np.nextafter(t, np.float32(np.inf))
        for x in (below, t, above):
            got = int(np.trunc(x + np.copysign(C, x)))
            xd = float(x)
            want = int(np.sign(xd) * np.floor(abs(xd) + 0.5))
            assert got == want, (x, got, want)
