"""The K rotation: seeded sign flips followed by an orthonormal Hadamard transform.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

R = (1/sqrt(d)) * H_d * diag(s)

* H_d is the Sylvester Hadamard matrix, built by the doubling
  H_2n = [[H, H], [H, -H]] from H_1 = [1] (P1, section "为什么 vLLM 选了
  Hadamard 而不是随机正交矩阵"), so H[i][j] = (-1)^popcount(i & j), H = H^T
  and H H^T = d I (P2, Hadamard section).  d must be a power of two.
* s is a vector of d seeded signs.  vLLM itself uses the pure Hadamard
  (same section: random signs do not change a symmetric Lloyd-Max
  quantiser's distortion); the method as specified here flips signs from a
  seed first, and ``sign_flip = False`` reproduces the pure Hadamard.  The
  pages name no generator; SplitMix64 (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014) is the reading
  taken: sign i is the top bit of the i-th output, 1 -> -1.
* The fast transform (FWHT) applies H in log2(d) butterfly stages instead
  of a d x d product (the same section calls the butterfly the alternative
  vLLM did not take).  The fp32 contract fixes the stage order: h = 1, 2,
  4, ..., d/2, each butterfly (a, b) -> (a + b, a - b).
"""

import numpy as np

MASK64 = (1 << 64) - 1


def sylvester_hadamard(d):
    """Integer Sylvester Hadamard matrix of order d (d a power of two)."""
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError("Sylvester Hadamard needs a power-of-two order")
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def splitmix64_outputs(seed, n):
    """First n outputs of SplitMix64 started from state ``seed``."""
    st = seed & MASK64
    out = []
    for _ in range(n):
        st = (st + 0x9E3779B97F4A7C15) & MASK64
        z = st
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        z = z ^ (z >> 31)
        out.append(z)
    return out


def rotation_signs(seed, d, sign_flip=True):
    """d signs (+1/-1, int8): s_i = -1 iff the top bit of output i is set."""
    if not sign_flip:
        return np.ones(d, dtype=np.int8)
    return np.array([-1 if (z >> 63) else 1 for z in splitmix64_outputs(seed, d)],
                    dtype=np.int8)


def rotation_matrix_f64(signs):
    """Explicit R = H diag(s) / sqrt(d) in float64; a d x d matrix passed in
    place of the signs (the Haar rotation's Q32) is returned as float64."""
    if np.ndim(signs) == 2:
        return np.asarray(signs, dtype=np.float64)
    d = len(signs)
    H = sylvester_hadamard(d).astype(np.float64)
    return H * np.asarray(signs, dtype=np.float64)[None, :] / np.sqrt(d)


def fwht_f64(x):
    """Unnormalised Walsh-Hadamard transform along the last axis, float64."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def fwht_f32_contract(u):
    """Unnormalised FWHT along the last axis in binary32, contract order.

    Stage h pairs index i (bit h clear) with i + h and writes
    (u_i + u_{i+h}, u_i - u_{i+h}); stages run h = 1, 2, ..., d/2.
    Every add and subtract is one rounded binary32 operation.
    """
    y = np.array(u, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b      # float32 + float32 -> float32, one rounding
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    assert y.dtype == np.float32
    return y
