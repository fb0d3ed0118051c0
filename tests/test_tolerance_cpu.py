"""The parity bound on bf16 outputs (CPU only): the tolerance, widened only on
elements whose exact value is itself farther than the tolerance from every
bf16 number."""

import numpy as np
import torch

from gpu_util import o_max_allowed, rounding_floor


def test_floor_is_the_rounding_of_the_exact_value():
    # 4.1144808 lies between the bf16 numbers 4.09375 and 4.125 (2^-5 apart
    # on [4, 8)); round to nearest gives 4.125, 1.0519e-2 away.
    x = np.array([4.1144808252473695, 1.0, 0.3, -2.7, 4.109375])
    f = rounding_floor(x, torch.bfloat16)
    assert abs(f[0] - (4.125 - 4.1144808252473695)) < 1e-15
    assert f[1] == 0.0
    assert np.all(f[2:4] <= 2.0 ** -8)          # [0.25, 0.5) and [2, 4): half-spacings 2^-10, 2^-7
    assert abs(f[4] - 2.0 ** -6) < 1e-15          # exactly half-way: the largest floor on [4, 8)
    b = o_max_allowed(x, torch.bfloat16)
    assert b[0] == f[0] + 1e-3                  # widened only where the floor passes 1e-2
    assert np.all(b[1:4] == 1e-2)
    # fp32 outputs keep their tolerance everywhere.
    assert np.all(o_max_allowed(x, torch.float32) == 1e-5)


def test_floor_never_exceeds_half_a_spacing():
    r = np.random.default_rng(0).uniform(-8, 8, 100_000)
    f = rounding_floor(r, torch.bfloat16)
    spacing = 2.0 ** (np.floor(np.log2(np.abs(r))) - 7)
    # Rounding goes through fp32 (as a kernel's fp32 result does), which may
    # move a value just past a midpoint onto it: 2^-24 relative at most.
    assert np.all(f <= spacing / 2 + np.abs(r) * 2.0 ** -24)
    # Below |o| = 2.56 the tolerance 1e-2 always covers the rounding.
    assert np.all(o_max_allowed(r[np.abs(r) < 2.56], torch.bfloat16) == 1e-2)
