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


def rotate_input_f32(x, kind, signs=None, r16=None):
    """Dispatch the write-side rotation: 'none', 'sign_fwht' or 'dense'."""
    if kind == "none":
        return np.asarray(x, dtype=np.float32).copy()
    if kind == "sign_fwht":
        return sign_fwht_f32(x, signs)
    if kind == "dense":
        return dense_rotate_f32(x, r16)
    raise ValueError(kind)


def rotation_matrix_f64(kind, signs=None, r16=None):
    """The operator R (fp64 [128,128]) whose exact action the write side rounds.

    sign_fwht: (1/sqrt(128)) H diag(s).  dense: R16 as fp64.  none: identity.
    """
    if kind == "none":
        return np.eye(D)
    if kind == "sign_fwht":
        s = np.asarray(signs, dtype=np.float64)
        return hadamard_sylvester(D) * s[None, :] / np.sqrt(np.float64(D))
    if kind == "dense":
        return np.asarray(r16, dtype=np.float16).astype(np.float64)
    raise ValueError(kind)
