"""Pins for oracle/rotation.py: closed forms, library routines and hand-derived orders."""
import os
from fractions import Fraction

import numpy as np
import scipy.linalg

from oracle import rotation as rot

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_hadamard_matches_scipy():
    assert np.array_equal(rot.hadamard_sylvester(128), scipy.linalg.hadamard(128).astype(np.float64))


def test_hadamard_involution():
    h = rot.hadamard_sylvester(128)
    assert np.array_equal(h @ h, 128 * np.eye(128))


def test_inv_sqrt_constant_is_nearest_fp32():
    c = rot.INV_SQRT_D_F32
    assert int(c.view(np.uint32)) == 0x3DB504F3
    # |c^2 * 128 - 1| is smallest among c and its neighbours (exact rationals)
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(1))]
    err = [abs(Fraction(float(x)) ** 2 * 128 - 1) for x in cands]
    assert err[1] == min(err)


def test_sign_fwht_close_to_closed_form():
    rng = np.random.default_rng(1)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    x = rng.standard_normal((500, 128)).astype(np.float16).astype(np.float32)
    x[:, 5] *= 30
    y = rot.sign_fwht_f32(x, s)
    R = rot.rotation_matrix_f64("sign_fwht", s)
    ref = x.astype(np.float64) @ R.T
    # 7 rounded stages + 1 multiply: error well under 16 ulp of the vector norm
    tol = 16 * 2.0 ** -24 * np.linalg.norm(x, axis=1, keepdims=True)
    assert np.all(np.abs(y - ref) <= tol)
    # norm preserved up to fp32 rounding; orthogonality of the fp64 operator
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    assert np.allclose(R @ R.T, np.eye(128), atol=1e-12)


def test_sign_fwht_unit_vector_is_scaled_first_column():
    s = np.ones(128)
    s[0] = -1
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 1
    y = rot.sign_fwht_f32(x, s)
    assert np.all(y == -rot.INV_SQRT_D_F32)


def test_sign_fwht_integer_inputs_exact():
    # small integers: every butterfly is exact, so y = fl32((H diag(s) x) * c) exactly
    rng = np.random.default_rng(2)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    x = rng.integers(-50, 50, (64, 128)).astype(np.float32)
    hx = (x.astype(np.int64) * s) @ scipy.linalg.hadamard(128).T
    want = hx.astype(np.float32) * rot.INV_SQRT_D_F32
    assert np.array_equal(rot.sign_fwht_f32(x, s), want)


def test_fwht_stage_order_golden():
    x = np.zeros(128, np.float32)
    x[0], x[1], x[2] = 2.0, 3 * 2.0 ** -24, 2.0 ** -23
    assert np.float16(x[1]) == x[1] and np.float16(x[2]) == x[2]  # valid fp16 inputs
    u = rot.fwht_f32(x)
    for idx, bits in _rows("fwht_stage_order.txt"):
        assert int(u[int(idx)].view(np.uint32)) == int(bits, 16)


def test_dense_chain_order_golden():
    x = np.full(128, 2.0 ** -24, np.float32)
    x[0] = 1.0
    r = np.zeros((128, 128), np.float16)
    r[0, :] = 1
    r[1, 1:] = 1
    y = rot.dense_rotate_f32(x[None, :], r)[0]
    for row, bits in _rows("dense_chain_order.txt"):
        assert int(y[int(row)].view(np.uint32)) == int(bits, 16)


def test_dense_rotation_close_to_matvec():
    rng = np.random.default_rng(3)
    q, rr = np.linalg.qr(rng.standard_normal((128, 128)))
    r16 = (q * np.sign(np.diag(rr))).astype(np.float16)
    x = rng.standard_normal((200, 128)).astype(np.float16).astype(np.float32)
    y = rot.dense_rotate_f32(x, r16)
    ref = x.astype(np.float64) @ r16.astype(np.float64).T
    bound = 128 * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(r16.astype(np.float64)).T)
    assert np.all(np.abs(y - ref) <= bound)
    # fp16 rounding of an orthogonal matrix keeps it orthogonal to ~1e-3
    R = rot.rotation_matrix_f64("dense", r16=r16)
    assert np.abs(R @ R.T - np.eye(128)).max() < 2e-3


# ---- SRFT ("When Quantization Is Free", Methodology sections 1 and 2)

def _signs(seed):
    rng = np.random.default_rng(seed)
    return np.where(rng.integers(0, 2, 128) == 1, 1, -1)


def test_srft_matrix_is_orthonormal_and_the_packed_real_dft():
    s = _signs(50)
    R = rot.srft_matrix_f64(s)
    assert np.abs(R @ R.T - np.eye(128)).max() < 1e-13
    # against numpy's real FFT (a library routine): rows are DC, Nyquist, then Re/Im pairs
    x = np.random.default_rng(51).standard_normal((4, 128))
    X = np.fft.rfft(x * s, axis=-1)
    y = x @ R.T
    assert np.allclose(y[:, 0], X[:, 0].real / np.sqrt(128), atol=1e-12)
    assert np.allclose(y[:, 1], X[:, 64].real / np.sqrt(128), atol=1e-12)
    assert np.allclose(y[:, 2::2], X[:, 1:64].real * np.sqrt(2 / 128), atol=1e-12)
    assert np.allclose(y[:, 3::2], X[:, 1:64].imag * np.sqrt(2 / 128), atol=1e-12)


def test_stockham_fft_matches_numpy_fft():
    rng = np.random.default_rng(52)
    re = rng.standard_normal((8, 64)).astype(np.float32)
    im = rng.standard_normal((8, 64)).astype(np.float32)
    zr, zi = rot.stockham_fft64_f32(re, im)
    Z = np.fft.fft(re.astype(np.float64) + 1j * im.astype(np.float64), axis=-1)
    # fp32 butterflies: error grows like log2(64) roundings of values of size sqrt(64)
    assert np.abs(zr - Z.real).max() < 2e-5 and np.abs(zi - Z.imag).max() < 2e-5
    # an impulse at n gives W64^(k n) exactly in magnitude
    e = np.zeros((64,), np.float32)
    e[5] = 1.0
    zr, zi = rot.stockham_fft64_f32(e, np.zeros_like(e))
    assert np.allclose(zr + 1j * zi, np.exp(-2j * np.pi * 5 * np.arange(64) / 64), atol=1e-6)


def test_srft_f32_close_to_the_matrix():
    s = _signs(53)
    x = np.random.default_rng(54).standard_normal((16, 128)).astype(np.float32) * 3
    y = rot.srft_f32(x, s)
    ref = x.astype(np.float64) @ rot.srft_matrix_f64(s).T
    assert np.abs(y - ref).max() < 1e-5 * np.abs(ref).max() + 1e-7
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x.astype(np.float64), axis=-1), rtol=1e-5)


def test_srft_first_unit_vector_closed_form_exact():
    # x = e_0: Z_k = s_0 for every k (only twiddles W^0 = 1 are applied), so X_k = s_0:
    # y = s_0 (c0, c0, 1/8, 0, 1/8, 0, ...) exactly
    s = _signs(55)
    x = np.zeros(128, np.float32)
    x[0] = 1.0
    y = rot.srft_f32(x, s)
    c0 = rot.INV_SQRT_D_F32
    want = np.zeros(128, np.float32)
    want[0] = want[1] = s[0] * c0
    want[2::2] = s[0] * np.float32(0.125)
    assert np.array_equal(y, want)  # +0 == -0


def test_twiddles_are_the_rounded_fp64_values():
    wr, wi = rot.twiddles_f32(128, 65)
    assert wr[0] == 1.0 and wi[0] == 0.0 and wr[64] == -1.0
    assert wr[32] == np.float32(np.cos(np.pi / 2)) and wi[32] == -1.0
    for k in (1, 17, 45):
        ang = 2 * np.pi * k / 128
        assert wr[k] == np.float32(np.cos(ang)) and wi[k] == np.float32(-np.sin(ang))
        assert abs(float(wr[k]) - np.cos(ang)) <= abs(np.spacing(np.float32(wr[k]))) / 2


def test_srft_pass_order_golden():
    # hand-derived bits ("When Quantization Is Free", Methodology sections 1-2): the
    # Stockham passes add points 32 apart first; the other order changes the last bits
    x = np.zeros(128, np.float16)
    outs = {}
    for row in _rows("srft_pass_order.txt"):
        if row[0] == "in":
            x.view(np.uint16)[int(row[1])] = int(row[2], 16)
        else:
            outs[int(row[1])] = int(row[2], 16)
    y = rot.srft_f32(x.astype(np.float32)[None], np.ones(128))[0]
    for idx, bits in outs.items():
        assert int(y[idx].view(np.uint32)) == bits, (idx, hex(int(y[idx].view(np.uint32))), hex(bits))
