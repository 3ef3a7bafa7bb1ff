"""A Haar (uniformly random) orthogonal rotation, the alternative to the
seeded-sign Hadamard transform.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

P3 (kwkr.cn news 555717) rotates with a random orthogonal matrix Pi drawn by
QR decomposition of a Gaussian matrix, which makes every rotated coordinate
of a unit vector follow the sphere marginal exactly; P1 (section "为什么 vLLM
选了 Hadamard 而不是随机正交矩阵") weighs it against the Hadamard transform
(a dense d x d product instead of d log d butterflies).

Construction from ``rot_seed`` (the pages name no generator; this is the
reading taken):
  * SplitMix64 outputs z_0, z_1, ... from state rot_seed (the generator of the
    sign flips) give uniforms u_k = ((z_k >> 11) + 1/2) / 2^53 in (0, 1);
  * Box-Muller turns each pair into two normals:
    g_2m = sqrt(-2 ln u_2m) cos(2 pi u_2m+1),  g_2m+1 = sqrt(-2 ln u_2m) sin(2 pi u_2m+1);
  * G (d x d) is filled row by row with g_0, g_1, ...;
  * G = Q R (Householder QR, a library routine), and Q diag(sign(diag R)) is
    Haar distributed (Mezzadri, "How to generate random matrices from the
    classical compact groups", Notices AMS 2007);
  * the rotation used is that matrix rounded to float32, Q32: y = Q32 x.

Store contract with this rotation (single binary32 operations, nearest even):
  y_j = (pairwise tree over i of Q32[j, i] * x_i) * (1 / (|x| + 1e-8)),
the tree in index order as for the norm; no 1/sqrt(d) (Q is orthonormal).
"""

import math

import numpy as np

from .rotation import splitmix64_outputs

F32 = np.float32


def gaussian_stream(seed, n):
    """n standard normals from SplitMix64 + Box-Muller (see module docstring)."""
    z = splitmix64_outputs(seed, n + (n & 1))
    u = [((v >> 11) + 0.5) / 9007199254740992.0 for v in z]
    g = []
    for m in range(0, len(u), 2):
        r = math.sqrt(-2.0 * math.log(u[m]))
        g.append(r * math.cos(2.0 * math.pi * u[m + 1]))
        g.append(r * math.sin(2.0 * math.pi * u[m + 1]))
    return np.array(g[:n], dtype=np.float64)


def haar_matrix_f64(seed, d):
    G = gaussian_stream(seed, d * d).reshape(d, d)
    Q, R = np.linalg.qr(G)
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Q * s[None, :]


def haar_matrix_f32(seed, d):
    return haar_matrix_f64(seed, d).astype(F32)


def rotate_contract(x, Q32):
    """Unscaled rotated vectors: pairwise tree over i of Q32[j, i] * x_i, fp32;
    x [..., d] float32 -> [..., d] float32."""
    from .store import pairwise_sum_f32
    x = np.asarray(x, dtype=F32)
    prod = (np.asarray(Q32, dtype=F32)[None, :, :] * x.reshape(-1, 1, x.shape[-1])).astype(F32)
    return pairwise_sum_f32(prod).reshape(x.shape)
