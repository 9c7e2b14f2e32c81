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


def test_rmsnorm_residual_closed_forms():
    """The residual RMSNorm step (oracle.rmsnorm_residual), pinned by facts
    that hold whatever the implementation: a row with squares summing to 25
    over k = 2 has RMS sqrt(12.5); scaling a row by a power of two leaves the
    normalized row unchanged bit for bit when eps = 0 (sqrt and fp32
    rounding commute with it); a zero row stays zero; each row is normalized
    by its own RMS; u is the fp32 residual sum and only the first k columns of
    z count."""
    z = np.array([[1.0, 4.0, 99.0]])
    r = np.array([[2.0, 0.0]])
    v, u = O.rmsnorm_residual(z, 2, r, eps=0.0)            # u = (3, 4)
    assert u.dtype == np.float32 and np.array_equal(u, np.array([[3.0, 4.0]], np.float32))
    c = np.float32(1.0 / math.sqrt(12.5))
    assert np.array_equal(v, np.array([[np.float32(3.0) * c, np.float32(4.0) * c]], np.float32))
    # u is rounded as an fp32 sum: 1 + 2^-30 is 1 in fp32
    _, u2 = O.rmsnorm_residual(np.array([[2.0 ** -30]]), 1, np.array([[1.0]]))
    assert u2[0, 0] == np.float32(1.0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    zero = np.zeros_like(x)
    v1, _ = O.rmsnorm_residual(zero, 64, x, eps=0.0)
    v4, _ = O.rmsnorm_residual(zero, 64, 4.0 * x, eps=0.0)
    v_small, _ = O.rmsnorm_residual(zero, 64, x / 1024.0, eps=0.0)
    assert np.array_equal(v1, v4) and np.array_equal(v1, v_small)
    # each row is normalized by its own RMS: rms(v) = sqrt(m / (m + eps)),
    # m = mean(u^2), for rows of very different scale
    y = np.concatenate([x[:1] * 1e-2, x[1:2] * 1e3, x[2:]], axis=0).astype(np.float32)
    vy, _ = O.rmsnorm_residual(zero, 64, y)
    m = (y.astype(np.float64) ** 2).mean(axis=1)
    rms = np.sqrt((vy.astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(rms - np.sqrt(m / (m + O.RMS_EPS))) < 1e-6), rms
    assert abs(rms[1] - 1.0) < 1e-6 and rms[0] < 0.96
    # eps enters as mean + eps: a row of constant 1e-3 gives 1e-3 / sqrt(1e-6 + 1e-5)
    vc, _ = O.rmsnorm_residual(np.zeros((1, 8)), 8, np.full((1, 8), 1e-3))
    assert abs(float(vc[0, 0]) - 1e-3 / math.sqrt(1e-6 + 1e-5)) < 1e-6
    vz, _ = O.rmsnorm_residual(np.zeros((1, 16)), 16, np.zeros((1, 16)))
    assert not vz.any()
    # the epilogue dispatcher returns the same v
    assert np.array_equal(O.epilogue("residual_rmsnorm", z, 2, r), O.rmsnorm_residual(z, 2, r)[0])
