"""Comparison of a result with the oracle's (test infrastructure only: used by the
tests, the smoke check and the benchmark's CPU-baseline leg).

The bar for float32 outputs is max|y - y_ref| <= 2e-3 * max|y_ref| and relative L2
<= 1e-4; expert index sets must be equal. A set may differ only where the oracle's
margin between its K-th and (K+1)-th selection key is below NEAR_TIE (the two
implementations round the logits differently there); the oracle then follows the
other set."""
import numpy as np

NEAR_TIE = 1e-5


def parity(y, y_ref, what=""):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - y_ref).max()
    scale = np.abs(y_ref).max()
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert err <= 2e-3 * scale, f"{what}: max|err| {err:.3e} > 2e-3 * {scale:.3e}"
    assert rel <= 1e-4, f"{what}: rel-L2 {rel:.3e} > 1e-4"
    return err / max(scale, 1e-300), rel


def same_set(a, b):
    return sorted(int(v) for v in a) == sorted(int(v) for v in b)
