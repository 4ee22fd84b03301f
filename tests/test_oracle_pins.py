"""The CPU oracle against the pins (worked examples, closed forms, invariants,
library routines, brute force).  CPU only."""
import pytest

from pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(orc, name):
    PINS[name](orc)


def test_oracle_threads_do_not_change_results(orc):
    """Rows are independent: 1 thread and the default thread count agree."""
    import numpy as np
    import workloads as wl
    w = wl.WORKLOADS[1]
    x, gain, eps = wl.gen_rmsnorm(w)
    q, k, pos, inv = wl.gen_rope(w)
    n = orc.threads()
    try:
        orc.set_threads(1)
        y1, _ = orc.rmsnorm(x, gain, eps)
        r1, _ = orc.rope(q, pos, 16, inv, 1.0, 0)
    finally:
        orc.set_threads(n)
    y2, _ = orc.rmsnorm(x, gain, eps)
    r2, _ = orc.rope(q, pos, 16, inv, 1.0, 0)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))
