"""Pins of the layer-operator oracle (oracle/layer_ops.py) against facts that do not come from
its own formulas: closed forms of RMSNorm, exact integer products, identities, and a brute force
over Python scalars on tiny inputs."""
import math

import numpy as np
import torch

from oracle import layer_ops as lo
from synth import layer_inputs as li


def test_bf16_decode_matches_torch_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = lo.bf16_bits_to_f64(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_rmsnorm_constant_row_closed_form():
    # x = c everywhere: mean(x^2) = c^2, so y = c / sqrt(c^2 + eps) * w.
    H, eps = 64, 1e-5
    w = np.linspace(0.5, 1.5, H)
    for c in (3.0, -0.25, 1e-3):
        y = lo.rmsnorm(np.full((1, H), c), w, eps)
        np.testing.assert_allclose(y[0], c / math.sqrt(c * c + eps) * w, rtol=1e-13)


def test_rmsnorm_one_hot_row():
    # A single nonzero a at j: mean(x^2) = a^2 / H; every other output is exactly 0.
    H, eps, a, j = 32, 1e-6, 2.5, 7
    x = np.zeros((1, H))
    x[0, j] = a
    w = np.arange(1, H + 1, dtype=np.float64)
    y = lo.rmsnorm(x, w, eps)
    assert np.count_nonzero(y) == 1
    assert math.isclose(y[0, j], a / math.sqrt(a * a / H + eps) * w[j], rel_tol=1e-14)


def test_rmsnorm_scale_and_sign_symmetry_and_unit_rms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 128))
    w = np.ones(128)
    y = lo.rmsnorm(x, w, 0.0)
    np.testing.assert_allclose(lo.rmsnorm(7.5 * x, w, 0.0), y, rtol=1e-13)   # scale invariance at eps = 0
    np.testing.assert_allclose(lo.rmsnorm(-x, w, 0.0), -y, rtol=1e-15)        # odd in x
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)       # unit RMS at eps = 0


def test_rmsnorm_brute_force_tiny():
    x = [[1.0, -2.0, 3.0, 0.5], [0.0, 0.0, 4.0, -4.0]]
    w = [1.0, 2.0, 0.5, -1.0]
    eps = 0.25
    y = lo.rmsnorm(np.array(x), np.array(w), eps)
    for i, row in enumerate(x):
        s = 0.0
        for v in row:
            s += v * v
        r = 1.0 / math.sqrt(s / len(row) + eps)
        for j, v in enumerate(row):
            assert math.isclose(y[i][j], v * r * w[j], rel_tol=1e-14, abs_tol=0.0)


def test_gemm_exact_on_small_integers():
    # Integer entries small enough that every product and sum is exact in fp64.
    rng = np.random.default_rng(1)
    a = rng.integers(-8, 9, (7, 33))
    w = rng.integers(-8, 9, (5, 33))
    c = lo.gemm(a, w)
    for m in range(7):
        for n in range(5):
            assert c[m, n] == sum(int(a[m, k]) * int(w[n, k]) for k in range(33))


def test_gemm_identity_and_transpose_convention():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((4, 16))
    np.testing.assert_array_equal(lo.gemm(a, np.eye(16)), a)          # W = I gives A back
    w = rng.standard_normal((3, 16))
    np.testing.assert_allclose(lo.gemm(a, w), (w @ a.T).T, rtol=1e-14)  # C[m][n] = <a_m, w_n>
    v = rng.standard_normal(3)
    np.testing.assert_allclose(lo.gemm(a, w) @ v, a @ (w.T @ v), rtol=1e-12)


def test_gemm_on_bf16_tensors_matches_float64_cast():
    a = li.activations(0, 0, 9, 64)
    w = li.gemm_weight(0, 32, 64)
    c = lo.gemm(a, w)
    ref = a.double().numpy() @ w.double().numpy().T
    np.testing.assert_allclose(c, ref, rtol=1e-13, atol=1e-14)


def test_activation_rows_are_position_keyed():
    whole = li.activations(3, 0, 100, 128)
    part = li.activations(3, 37, 61, 128)
    assert torch.equal(whole[37:61].view(torch.int16), part.view(torch.int16))
