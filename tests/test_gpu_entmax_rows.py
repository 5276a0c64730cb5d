"""GPU parity of the row-wise alpha-entmax (entmax_rows, through the C ABI)
against the float64 CPU oracle's exact threshold: float32 outputs within 1e-4,
bfloat16 within 2e-2, tau within 1e-4, supports equal except for entries within
1e-4 of tau; rows held by one wavefront and by one workgroup, ragged widths,
the three tau solver specialisations, and the degenerate rows (-inf entries, a
row with no finite entry, a single entry, a constant row, in place). Its
backward (entmax_rows_backward) against the oracle's vector-Jacobian product,
directly and through torch autograd.
"""

import numpy as np
import pytest
import torch

from adaptive_sparse_long_amd import api
from oracle.entmax import entmax, entmax_backward, entmax_threshold_rows

from _helpers import TOL_BF16, TOL_F32, assert_close, assert_sets_match, f64, tau_close

pytestmark = pytest.mark.gpu


def _x(rows, n, seed, scale=1.0, dtype=torch.float32):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy((scale * rng.standard_normal((rows, n))).astype(np.float32))
    return x.to(dtype).to("cuda")


def check_rows(x, alpha, where=""):
    y, tau = api.entmax(x, alpha=alpha, return_tau=True)
    torch.cuda.synchronize()
    Z = f64(x).reshape(-1, x.shape[-1])
    t_ref = entmax_threshold_rows(Z, alpha)
    U = np.where(np.isfinite(Z), (alpha - 1.0) * Z, -np.inf)
    umt = U - np.where(np.isfinite(t_ref), t_ref, np.inf)[:, None]
    p_ref = np.where(umt > 0, np.maximum(umt, 0.0) ** (1.0 / (alpha - 1.0)), 0.0)
    y_ = f64(y).reshape(Z.shape)
    tol = TOL_F32 if x.dtype == torch.float32 else TOL_BF16
    assert_close(y_, p_ref, tol, f"{where} p")
    tau_close(f64(tau).ravel(), t_ref, where)
    if x.dtype == torch.float32:
        assert_sets_match(y_ > 0, p_ref > 0, umt, where)
        has = np.isfinite(t_ref)
        assert np.all(np.abs(y_[has].sum(1) - 1.0) < 1e-5), f"{where}: rows do not sum to 1"
    return y, tau


@pytest.mark.parametrize("n", [1, 2, 37, 64, 100, 256, 1000, 2048, 2049, 5000, 32768])
@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.333])
def test_entmax_rows_f32(n, alpha):
    rows = 6 if n > 4096 else 13
    check_rows(_x(rows, n, 11 + n, scale=2.0), alpha, f"n={n} alpha={alpha}")


@pytest.mark.parametrize("n,alpha,scale", [(256, 1.5, 1.0), (3000, 2.0, 3.0), (700, 3.0, 0.5)])
def test_entmax_rows_bf16(n, alpha, scale):
    check_rows(_x(9, n, 101 + n, scale=scale, dtype=torch.bfloat16), alpha, f"bf16 n={n} alpha={alpha}")


def test_entmax_rows_pages_example_shape():
    """The activation's example shape: 128 rows of 256, alpha 1.5, 10 iterations."""
    check_rows(_x(128, 256, 7), 1.5, "128x256")


def test_entmax_rows_degenerate_rows():
    n = 300
    x = _x(6, n, 5, scale=1.5)
    x[0, 100:] = -float("inf")  # masked tail
    x[1] = -float("inf")  # no candidate: zeros, tau = +inf
    x[2] = 0.75  # constant: uniform over the row
    x[3, 17] = 1.0e3  # one dominant entry: one-hot
    y, tau = check_rows(x, 1.5, "degenerate")
    y_ = f64(y)
    assert np.all(y_[1] == 0.0) and np.isinf(f64(tau)[1])
    assert np.allclose(y_[2], 1.0 / n, atol=1e-6)
    assert y_[3, 17] == 1.0 and np.count_nonzero(y_[3]) == 1
    one = _x(4, 1, 9, scale=5.0)
    assert np.all(f64(api.entmax(one, alpha=2.0)) == 1.0)
    check_rows(x, 2.0, "degenerate sparsemax")


def test_entmax_rows_in_place_and_batched_shape():
    x = _x(2 * 3 * 5, 77, 13).reshape(2, 3, 5, 77)
    ref = api.entmax(x, alpha=1.5)
    y = api.entmax(x, alpha=1.5, out=x)
    torch.cuda.synchronize()
    assert y.data_ptr() == x.data_ptr()
    assert torch.equal(y, ref)


@pytest.mark.parametrize("n", [1, 37, 256, 2048, 2049, 5000])
@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.333])
def test_entmax_rows_backward_f32(n, alpha):
    x = _x(7, n, 200 + n, scale=2.0)
    x[3, : n // 2] = -float("inf")  # a masked part (zeros of y)
    y = api.entmax(x, alpha=alpha)
    dy = _x(7, n, 300 + n)
    dx = api.entmax_backward(y, dy, alpha=alpha)
    torch.cuda.synchronize()
    y_, dy_ = f64(y), f64(dy)
    ref = np.stack([entmax_backward(y_[r], dy_[r], alpha) for r in range(7)])
    assert_close(f64(dx), ref, TOL_F32, f"backward n={n} alpha={alpha}")
    assert np.all(np.abs(f64(dx).sum(1)) < 1e-4)


@pytest.mark.parametrize("n,alpha", [(300, 1.5), (3000, 2.0), (700, 3.0)])
def test_entmax_rows_backward_bf16(n, alpha):
    """bfloat16 gradients: 2e-2 absolute plus the bf16 rounding of the output
    itself (2^-9 of its magnitude, taken twice): dX is not bounded (for alpha > 2
    the factor y^(2-alpha) grows without limit at the edge of the support), so a
    bound on the absolute error alone cannot hold for a bf16 result."""
    x = _x(5, n, 400 + n, scale=1.5, dtype=torch.bfloat16)
    y = api.entmax(x, alpha=alpha)
    dy = _x(5, n, 500 + n, dtype=torch.bfloat16)
    dx = api.entmax_backward(y, dy, alpha=alpha)
    torch.cuda.synchronize()
    y_, dy_ = f64(y), f64(dy)
    ref = np.stack([entmax_backward(y_[r], dy_[r], alpha) for r in range(5)])
    err = np.abs(f64(dx) - ref)
    bound = TOL_BF16 + 2.0 ** -8 * np.abs(ref)
    assert np.all(np.isfinite(f64(dx)))
    assert np.all(err <= bound), f"bf16 backward n={n} alpha={alpha}: worst excess {float(np.max(err - bound)):.3e}"


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_entmax_autograd_matches_oracle(alpha):
    """torch autograd through entmax_fn: the gradient of sum(w * entmax(x)) with
    respect to x, against the oracle's exact forward and its Jacobian."""
    x = _x(6, 500, 71, scale=2.0).requires_grad_(True)
    w = _x(6, 500, 72)
    (api.entmax_fn(x, alpha=alpha) * w).sum().backward()
    x_, w_ = f64(x.detach()), f64(w)
    ref = np.stack([entmax_backward(entmax(x_[r], alpha), w_[r], alpha) for r in range(6)])
    assert_close(f64(x.grad), ref, TOL_F32, f"autograd alpha={alpha}")


def test_entmax_rows_backward_in_place():
    x = _x(4, 129, 81, scale=2.0)
    y = api.entmax(x, alpha=1.5)
    dy = _x(4, 129, 82)
    ref = api.entmax_backward(y, dy, alpha=1.5)
    out = api.entmax_backward(y, dy, alpha=1.5, out=dy)
    torch.cuda.synchronize()
    assert out.data_ptr() == dy.data_ptr() and torch.equal(out, ref)

