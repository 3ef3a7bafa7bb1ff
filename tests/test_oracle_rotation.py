"""Pins for the oracle's rotation (Sylvester Hadamard, signs, FWHT).

P1, section "为什么 vLLM 选了 Hadamard 而不是随机正交矩阵": H_2n = [[H, H],
[H, -H]], orthonormal after dividing by sqrt(d), symmetric.  P2 (Hadamard
section): H H^T = d I.
"""

import numpy as np
import pytest

from oracle import rotation as rot
from conftest import load_golden

DIMS = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_orthogonal_and_symmetric(d):
    H = rot.sylvester_hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))
    assert np.array_equal(H, H.T)
    assert set(np.unique(H)) <= {-1, 1}


def test_hadamard_entry_formula():
    # closed form of the Sylvester construction: H[i][j] = (-1)^popcount(i & j)
    d = 128
    H = rot.sylvester_hadamard(d)
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(H, np.where(pc % 2 == 0, 1, -1))


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        rot.sylvester_hadamard(96)


@pytest.mark.parametrize("d", [2, 8, 64, 128, 256])
def test_fwht_equals_matrix_product(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((50, d))
    H = rot.sylvester_hadamard(d).astype(np.float64)
    ref = x @ H.T
    got = rot.fwht_f64(x)
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref)) * d


def test_fwht_f32_contract_matches_scalar_loop():
    """The vectorised contract equals a plain scalar loop over the stated
    stage order (h ascending; (u_i, u_{i+h}) <- (u_i + u_{i+h}, u_i - u_{i+h}))."""
    d = 32
    rng = np.random.default_rng(1)
    u = rng.standard_normal(d).astype(np.float32) * np.float32(3.7)
    ref = [np.float32(v) for v in u]
    h = 1
    while h < d:
        for i in range(d):
            if i & h == 0:
                a, b = ref[i], ref[i + h]
                ref[i], ref[i + h] = np.float32(a + b), np.float32(a - b)
        h *= 2
    got = rot.fwht_f32_contract(u[None])[0]
    assert np.array_equal(got.view(np.uint32), np.array(ref, dtype=np.float32).view(np.uint32))


def test_fwht_f32_close_to_f64():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20000, 128)).astype(np.float32)
    x[:, :4] *= 20
    got = rot.fwht_f32_contract(x).astype(np.float64)
    ref = rot.fwht_f64(x.astype(np.float64))
    scale = np.sqrt((x.astype(np.float64) ** 2).sum(axis=1, keepdims=True))
    assert np.max(np.abs(got - ref) / scale) < 1e-6


@pytest.mark.parametrize("seed,flip", [(0, True), (12345, True), (7, False)])
def test_rotation_is_orthonormal(seed, flip):
    s = rot.rotation_signs(seed, 128, flip)
    R = rot.rotation_matrix_f64(s)
    assert np.max(np.abs(R @ R.T - np.eye(128))) < 1e-15 * 128


def test_splitmix64_published_vectors():
    g = load_golden("splitmix64_vectors.json")["vectors"]
    for seed, outs in g.items():
        want = [int(v, 0) for v in outs]
        assert rot.splitmix64_outputs(int(seed), len(want)) == want


def test_signs_from_top_bit_and_pure_hadamard():
    s = rot.rotation_signs(0, 3)
    # 0xe220..: top bit 1 -> -1; 0x6e78..: 0 -> +1; 0x06c4..: 0 -> +1
    assert list(s) == [-1, 1, 1]
    assert np.all(rot.rotation_signs(99, 128, sign_flip=False) == 1)
    s = rot.rotation_signs(2024, 128)
    assert 40 < (s < 0).sum() < 88          # a fair coin, loosely
