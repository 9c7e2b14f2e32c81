"""Pins of the oracle's producer-epilogue step (oracle.epilogue / oracle.silu,
the elementwise work [AE] §6.4 gives the post-processing unit), CPU only,
from closed forms that do not restate the oracle's formula:
  - silu(ln 3) = (3/4) ln 3 (the logistic function at ln 3 is 3/4);
  - silu(x) - silu(-x) = x for every x, silu(0) = 0, slope 1/2 at 0;
  - silu(x) -> x for large x and -> 0 for very negative x;
  - the copy takes the first k columns, the residual adds, and SwiGLU gates
    the second half of z with the first (not the other way round).
"""

import math

import numpy as np

import oracle as O


def test_silu_closed_forms():
    assert abs(O.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    x = np.linspace(-20, 20, 401)
    assert np.allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-13)
    assert O.silu(np.array([0.0]))[0] == 0.0
    h = 1e-6
    assert abs((O.silu(np.array([h]))[0] - O.silu(np.array([-h]))[0]) / (2 * h) - 0.5) < 1e-9
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15


def test_epilogue_ops_select_and_combine_the_right_columns():
    z = np.array([[math.log(3.0), 1.0, 2.0, 5.0]])
    assert np.array_equal(O.epilogue("copy", z, 2), z[:, :2])
    r = np.array([[10.0, -1.0]])
    assert np.array_equal(O.epilogue("residual", z, 2, r), np.array([[10.0 + math.log(3.0), 0.0]]))
    v = O.epilogue("swiglu", z, 2)
    # gate = first half (ln 3, 1), up = second half (2, 5)
    assert abs(v[0, 0] - 0.75 * math.log(3.0) * 2.0) < 1e-15
    assert abs(v[0, 1] - 5.0 / (1.0 + math.exp(-1.0))) < 1e-15
