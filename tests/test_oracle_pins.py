"""The fp64 oracle against closed forms, invariants, library routines and
hand-derived examples (CPU only)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS + oracle_pins.FP8_PINS + oracle_pins.VARLEN_DECODE_PINS, ids=lambda p: p.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_rows_subset_matches_full(oracle_lib):
    """Computing a sample of rows gives the same values as the full computation."""
    import numpy as np
    import torch
    q, k, v = (torch.randn((2, 3, n, 16), generator=torch.Generator().manual_seed(s)).half()
               for n, s in ((9, 1), (12, 2), (12, 3)))
    o, lse = oracle_lib.attention(q, k, v, True, 0.25)
    rows = np.array([0, 5, 17, 53, 26])
    os_, ls_ = oracle_lib.attention(q, k, v, True, 0.25, rows=rows)
    assert np.array_equal(os_, o.reshape(-1, 16)[rows])
    assert np.array_equal(ls_, lse.reshape(-1)[rows])


def test_threads_do_not_change_results(oracle_lib):
    import numpy as np
    import torch
    q, k, v = (torch.randn((1, 4, n, 8), generator=torch.Generator().manual_seed(s)).bfloat16()
               for n, s in ((33, 4), (40, 5), (40, 6)))
    a = oracle_lib.attention(q, k, v, False, 0.3, nthreads=1)
    b = oracle_lib.attention(q, k, v, False, 0.3, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
