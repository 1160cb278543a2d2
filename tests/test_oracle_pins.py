"""The fp64 oracle against closed forms, invariants, an independent library routine and
finite differences (CPU only)."""
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_FORWARD + pins.ALL_BACKWARD,
                         ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_fwd_rows_match_full():
    """The per-row entry point agrees with the full forward."""
    import numpy as np
    from workloads import make_inputs_like
    q, k, v, _ = make_inputs_like(2, 33, 4, 1, 8, "bf16", 5)
    for causal, window in ((True, 0), (True, 5), (False, 7)):
        O, L = oracle.attn_fwd(q, k, v, 0.3, causal, window, row_chunk=8)
        trip = [(1, 3, 0), (0, 0, 32), (1, 2, 17), (0, 1, 5)]
        o, l = oracle.attn_fwd_rows(q, k, v, 0.3, causal, window, trip)
        for n, (b, h, i) in enumerate(trip):
            assert np.allclose(o[n], O[b, i, h], atol=1e-14, rtol=0)
            assert abs(l[n] - L[b, h, i]) < 1e-13


def test_bwd_group_selection_matches_full():
    import numpy as np
    from workloads import make_inputs_like
    q, k, v, do = make_inputs_like(2, 20, 4, 2, 8, "f32", 9)
    full = oracle.attn_bwd(q, k, v, do, 0.4, True, 6, row_chunk=7)
    part = oracle.attn_bwd(q, k, v, do, 0.4, True, 6, groups=[(1, 0)])
    for name in ("dq",):
        assert np.allclose(part[name][1, :, 0:2], full[name][1, :, 0:2], atol=1e-14)
    for name in ("dk", "dv"):
        assert np.allclose(part[name][1, :, 0], full[name][1, :, 0], atol=1e-14)
        assert np.isnan(part[name][0]).all()
