"""Rotations applied before quantization (write side) and to the query/output.

Test infrastructure only: see the package docstring for who may import it.

Sign + Walsh-Hadamard form.  "When Quantization Is Free" (Methodology section 1)
rotates each head vector by a fixed random sign vector followed by an orthogonal
transform, and reports the Hadamard variant (SRHT) as statistically
indistinguishable from its Fourier one; "Search Your Block Floating Point
Scales!" (Methodology, incoherence processing) uses the Hadamard transform for
the same purpose.  Here y = (1/sqrt(d)) H diag(s) x with H the Sylvester
(natural-order) Hadamard matrix, d = 128.

The pages do not fix a butterfly order or where the normalisation is applied.
Reading taken (part of the bit-exact contract): the fp32 sign flip, then stages
h = 1, 2, 4, ..., 64, each replacing (u_i, u_{i+h}) by (u_i + u_{i+h},
u_i - u_{i+h}) for every i with i & h == 0, each sum/difference rounded to fp32,
then one fp32 multiply by fl32(1/sqrt(128)).

Dense form.  "OSCAR" (section 2.2A, composite rotation) applies a fixed dense
d x d orthogonal rotation to keys and values before 2-bit quantization.  The
matrix used here is stored as fp16 (R16); the write side computes each output
as a fixed-order fp32 multiply-add chain over k = 0..127 (products of two fp16
numbers are exact in fp32, so each step is one rounding of acc + product).

Fourier form (SRFT).  "When Quantization Is Free" (Methodology section 1) defines
the rotation as SRFT(x) = pack(F diag(s) x), F the unitary DFT and s a fixed
random sign vector; its fused write kernel (section 2) flips the signs, runs
log2(d/2) radix-2 Stockham butterfly passes and unpacks the Hermitian symmetry
into a real representation.  Reading taken (part of the bit-exact contract, all
fp32, round to nearest, no fused operations):
  u = s * x; z_n = u_2n + i u_2n+1 (n = 0..63);
  Z = the 64-point forward FFT of z by Stockham autosort passes: for sub-length
      L = 64, 32, ..., 2 (stride m = 64 / L), every j < L/2 and k < m:
      a = x[j m + k], b = x[(j + L/2) m + k], y[2 j m + k] = a + b,
      y[(2 j + 1) m + k] = (a - b) * W64^(j m), complex products as
      (ar wr - ai wi, ar wi + ai wr);
  X_k (k = 0..64, the real DFT of u; Z_64 = Z_0): with A = Z_k, B = conj(Z_(64-k)),
      E = ((Ar + Br) / 2, (Ai + Bi) / 2), O = ((Ai - Bi) / 2, -(Ar - Br) / 2),
      X_k = E + W128^k * O;
  y_0 = X_0.re c0, y_1 = X_64.re c0, y_2k = X_k.re / 8, y_2k+1 = X_k.im / 8
      (k = 1..63), c0 = fl32(1/sqrt(128)); this packing is orthonormal.
Twiddles W_n^k = (fl32(cos(2 pi k / n)), fl32(-sin(2 pi k / n))), the fp64 values
rounded once.

Queries and outputs are rotated in fp64 by the same operator: q_rot = R q and
o = R^T o_rot, so scores q.k are unchanged by the rotation ("Search Your Block
Floating Point Scales!", incoherence processing: rotating Q and K by the same
orthogonal matrix preserves the attention scores).
"""

import numpy as np

D = 128
INV_SQRT_D_F32 = np.float32(1.0 / np.sqrt(np.float64(D)))  # fl32(1/sqrt(128))


def hadamard_sylvester(n=D):
    """Natural-order (Sylvester) Hadamard matrix, H_n = H_2 kron H_{n/2}."""
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(u):
    """The fp32 butterfly network on the last axis (length 128), stages h=1..64.

    u: float32 array [..., 128].  Each stage is vectorised over i but every
    element sees exactly one fp32 add or subtract per stage, in the stated order.
    """
    u = np.array(u, dtype=np.float32, copy=True)
    lead = u.shape[:-1]
    h = 1
    while h < D:
        v = u.reshape(lead + (D // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b  # float32 + float32 -> rounded fp32
        v[..., 1, :] = a - b
        u = v.reshape(lead + (D,))
        h *= 2
    return u


def sign_fwht_f32(x, signs):
    """Write-side rotation y = fl32(FWHT(s * x) * fl32(1/sqrt(128))), bit-exact fp32.

    x: float32 [..., 128] (exactly widened fp16/bf16); signs: [128] of +-1.
    The sign flip is exact.
    """
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(signs, dtype=np.float32)
    u = x * s
    u = fwht_f32(u)
    return u * INV_SQRT_D_F32


def dense_rotate_f32(x, r16):
    """Write-side dense rotation y_j = sum_k R16[j,k] x_k as a fixed-order fp32 chain.

    acc starts at +0; for k = 0..127: acc = fl32(acc + R16[j,k] * x_k).  The
    product of an fp16 matrix entry and an fp16 input is exact in fp32, so each
    step is a single rounding (what a fused multiply-add gives).
    """
    x = np.asarray(x, dtype=np.float32)
    r = np.asarray(r16, dtype=np.float16).astype(np.float32)
    acc = np.zeros(x.shape[:-1] + (D,), dtype=np.float32)
    for k in range(D):
        prod = r[:, k] * x[..., k:k + 1]  # exact in fp32
        acc = acc + prod
    return acc


def twiddles_f32(n, count):
    """W_n^k = exp(-2 pi i k / n) for k < count as fp32 (cos, -sin), the fp64 values rounded."""
    ang = 2 * np.pi * np.arange(count, dtype=np.float64) / n
    return np.cos(ang).astype(np.float32), (-np.sin(ang)).astype(np.float32)


def stockham_fft64_f32(re, im):
    """The 64-point forward FFT of (re + i im) [..., 64] by the Stockham passes above (fp32)."""
    wr, wi = twiddles_f32(64, 32)
    x_re = np.array(re, dtype=np.float32, copy=True)
    x_im = np.array(im, dtype=np.float32, copy=True)
    L, m = 64, 1
    while L > 1:
        half = L // 2
        y_re = np.empty_like(x_re)
        y_im = np.empty_like(x_im)
        for j in range(half):
            w_r, w_i = wr[j * m], wi[j * m]
            a_re, a_im = x_re[..., j * m:j * m + m], x_im[..., j * m:j * m + m]
            b_re, b_im = x_re[..., (j + half) * m:(j + half) * m + m], x_im[..., (j + half) * m:(j + half) * m + m]
            y_re[..., 2 * j * m:2 * j * m + m] = a_re + b_re
            y_im[..., 2 * j * m:2 * j * m + m] = a_im + b_im
            d_re, d_im = a_re - b_re, a_im - b_im
            y_re[..., (2 * j + 1) * m:(2 * j + 1) * m + m] = d_re * w_r - d_im * w_i
            y_im[..., (2 * j + 1) * m:(2 * j + 1) * m + m] = d_re * w_i + d_im * w_r
        x_re, x_im = y_re, y_im
        L, m = half, 2 * m
    return x_re, x_im


def srft_f32(x, signs):
    """Write-side SRFT rotation, bit-exact fp32 (the reading above).  x: float32 [..., 128]."""
    u = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    z_re, z_im = stockham_fft64_f32(u[..., 0::2], u[..., 1::2])
    idx = np.arange(65) % 64
    ridx = (64 - np.arange(65)) % 64
    a_re, a_im = z_re[..., idx], z_im[..., idx]
    b_re, b_im = z_re[..., ridx], -z_im[..., ridx]  # conj(Z_(64-k))
    half = np.float32(0.5)
    e_re, e_im = half * (a_re + b_re), half * (a_im + b_im)
    o_re, o_im = half * (a_im - b_im), -(half * (a_re - b_re))
    wr, wi = twiddles_f32(128, 65)
    t_re = o_re * wr - o_im * wi
    t_im = o_re * wi + o_im * wr
    X_re, X_im = e_re + t_re, e_im + t_im
    y = np.empty(u.shape, dtype=np.float32)
    y[..., 0] = X_re[..., 0] * INV_SQRT_D_F32
    y[..., 1] = X_re[..., 64] * INV_SQRT_D_F32
    eighth = np.float32(0.125)
    y[..., 2::2] = X_re[..., 1:64] * eighth
    y[..., 3::2] = X_im[..., 1:64] * eighth
    return y


def srft_matrix_f64(signs):
    """The orthonormal real matrix of the SRFT (fp64): row 0 the DC term, row 1 the
    Nyquist term, rows 2k, 2k+1 the real and imaginary parts of X_k (k = 1..63)."""
    n = np.arange(D)
    F = np.zeros((D, D))
    F[0] = 1.0 / np.sqrt(D)
    F[1] = (-1.0) ** n / np.sqrt(D)
    for k in range(1, 64):
        ang = 2 * np.pi * k * n / D
        F[2 * k] = np.sqrt(2.0 / D) * np.cos(ang)
        F[2 * k + 1] = -np.sqrt(2.0 / D) * np.sin(ang)
    return F * np.asarray(signs, dtype=np.float64)[None, :]


def rotate_input_f32(x, kind, signs=None, r16=None):
    """Dispatch the write-side rotation: 'none', 'sign_fwht', 'dense' or 'srft'."""
    if kind == "none":
        return np.asarray(x, dtype=np.float32).copy()
    if kind == "sign_fwht":
        return sign_fwht_f32(x, signs)
    if kind == "dense":
        return dense_rotate_f32(x, r16)
    if kind == "srft":
        return srft_f32(x, signs)
    raise ValueError(kind)


def rotation_matrix_f64(kind, signs=None, r16=None):
    """The operator R (fp64 [128,128]) whose exact action the write side rounds.

    sign_fwht: (1/sqrt(128)) H diag(s).  dense: R16 as fp64.  srft: the packed
    unitary DFT times diag(s).  none: identity.
    """
    if kind == "none":
        return np.eye(D)
    if kind == "sign_fwht":
        s = np.asarray(signs, dtype=np.float64)
        return hadamard_sylvester(D) * s[None, :] / np.sqrt(np.float64(D))
    if kind == "dense":
        return np.asarray(r16, dtype=np.float16).astype(np.float64)
    if kind == "srft":
        return srft_matrix_f64(signs)
    raise ValueError(kind)
