"""The cache-cold timing plan of bench.py (host logic only)."""
import pytest

import bench


@pytest.mark.parametrize("nbytes", [41120, 8421376, 19169280, 21463040, 38879232, 97419264, 147159040, 233717760])
@pytest.mark.parametrize("steps", [1, 5, 20, 50, 100, 97])
def test_rotation_plan(nbytes, steps):
    R, S = bench.rotation_plan(nbytes, nbytes / 2.5e6, steps)
    assert steps % S == 0, "exactly the requested number of steps is timed"
    assert R % S == 0, "every graph holds S distinct copies"
    # a copy is reused only after R - 1 others have passed: 3x the Infinity Cache,
    # or the cap on copies
    assert R * nbytes >= bench.ROTATE_BYTES or R >= bench.MAX_COPIES
    # no graph much longer than ~400 us of work at 2.5 TB/s
    assert S == 1 or S * nbytes / 2.5e6 <= 400.0
