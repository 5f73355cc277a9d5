"""The output bound of the GPU parity tests (CPU only): the stated
max-abs-error bound (fp16 2e-3, bf16 1e-2; fp32 1e-5) applies unchanged
wherever half an output ulp fits in half of it -- bf16 below |x| = 2, fp16
below 4, fp32 below 64 -- and grows by half an
ulp only beyond."""

import numpy as np

from helpers import TOL, out_bound, rounding_bound


def test_stated_bound_below_the_crossover():
    for dt, lim in (("bf16", 2.0), ("f16", 4.0), ("f32", 64.0)):
        x = np.linspace(-lim, lim, 20001)[1:-1]
        assert (out_bound(x, dt) == TOL[dt]).all(), dt


def test_wider_only_where_half_an_ulp_exceeds_half_the_bound():
    x = np.array([2.0, 3.99, 4.0, 7.9, -5.0])
    b = out_bound(x, "bf16")
    assert (b > TOL["bf16"]).all()
    assert np.allclose(b, rounding_bound(x, "bf16") + TOL["bf16"] / 2)
    # half an ulp of bf16 at 4 is 2^-6
    assert out_bound(np.array([4.0]), "bf16")[0] == 2.0 ** -6 + 5e-3
    assert out_bound(np.array([4.0]), "f16")[0] == 2.0 ** -9 + 1e-3
