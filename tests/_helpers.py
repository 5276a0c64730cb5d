"""Helpers shared by the GPU parity tests (comparison rules, conversions)."""

import numpy as np
import torch

# Tolerances: outputs 2e-2 absolute for bfloat16 and 1e-4 for float32, tau 1e-4;
# routed sets equal except for entries within 1e-4 of tau (in u units).
TOL_BF16 = 2e-2
TOL_F32 = 1e-4
TOL_TAU = 1e-4
MARGIN = 1e-4


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def unpack_bits(words: np.ndarray, n: int) -> np.ndarray:
    """[..., W] uint32 words -> [..., n] bool (bit c % 32 of word c // 32)."""
    w = np.asarray(words).astype(np.uint32)
    c = np.arange(n)
    return ((w[..., c // 32] >> (c % 32).astype(np.uint32)) & 1).astype(bool)


def assert_sets_match(gpu_bits, ref_bits, u_minus_tau, where=""):
    """Routed sets must agree except where the oracle's u - tau is within MARGIN of 0."""
    gpu_bits = np.asarray(gpu_bits, dtype=bool)
    ref_bits = np.asarray(ref_bits, dtype=bool)
    diff = gpu_bits != ref_bits
    if diff.any():
        bad = diff & ~(np.abs(u_minus_tau) < MARGIN)
        assert not bad.any(), f"{where}: {int(bad.sum())} routed-set entries differ away from tau; first at {np.argwhere(bad)[:5]}"


def assert_close(gpu, ref, tol, where=""):
    """|gpu - ref| <= tol elementwise; tol is a number or an array of ref's shape."""
    err = np.abs(np.asarray(gpu, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), err.shape)
    assert np.all(np.isfinite(gpu)), f"{where}: non-finite values"
    if err.size and not np.all(err <= tol):
        at = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{where}: abs error {float(err[at]):.3e} > {float(tol[at]):.2e} at {at} "
                             f"(max abs error {float(np.nanmax(err)):.3e})")


def half_ulp_bf16(x):
    """Half the spacing of bfloat16 numbers at |x| (8 significand bits)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 8)


def tol_bf16_out(ref):
    """Bar for a bfloat16 output: 2e-2, or where bf16 cannot hold a value that
    close (|ref| >= 8: neighbours 0.0625 apart) the correctly rounded neighbour,
    half an ulp, plus 1e-3 of computation error."""
    return np.maximum(TOL_BF16, half_ulp_bf16(ref) + 1e-3)


def tau_close(gpu_tau, ref_tau, where=""):
    g = np.asarray(gpu_tau, dtype=np.float64)
    r = np.asarray(ref_tau, dtype=np.float64)
    inf_r = np.isinf(r)
    assert np.array_equal(np.isinf(g), inf_r), f"{where}: +inf rows differ"
    assert_close(g[~inf_r], r[~inf_r], TOL_TAU, where + " tau")
