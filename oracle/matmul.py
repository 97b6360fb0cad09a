"""Reference for the weight-only dequantizing matmul (GEMV and GEMM).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: page "Huit bits, puis quatre" (smallbard.com), section "Ranger des
entiers dans des f32": the QuantizedMatmul operation takes the codes and the
scales; its generation-time products read the codes and its large
evaluation-time products use the dequantized weights, and both agree up to
the rounding of the summation order.  The mathematical result both must
approximate is therefore the plain product with the dequantized weights:

    y[m, n] = sum_k x[m, k] * w_hat[n, k]

with w_hat from ``oracle.rtn.unpack`` (fp32 values, not rounded further).
The stored weight is [n][k] row-major: each row is one output channel and
the groups run along k.

The reference computes in fp64 with the library matmul (the only step a
library primitive takes).  Every product x * w_hat of two fp32 values is
exact in fp64, and the fp64 sum of K such terms is within K * 2**-53 of the
exact sum relative to ``error_base``, far below the tolerances used.

The tolerance of a GPU result is stated per output element against

    B[m, n] = sum_k |x[m, k] * w_hat[n, k]|

because a weight error hurts an output in proportion to the activation it
meets (page "量化推理：INT8/INT4 的体积、困惑度与速度为什么不同步", the
``checks`` function's equal-weight-error example).

GEMM activations are bf16 (page on floating-point formats, xdnf.cn, section
on the 16-bit "bfloat" type: 1 sign bit, 8 exponent bits, 7 mantissa bits,
i.e. the top half of an fp32).
"""

import numpy as np

from .rtn import unpack


def bf16_bits_to_f32(bits):
    """Exact value of bf16 numbers given as uint16 bit patterns: the pattern
    is the upper 16 bits of an fp32 with the lower 16 bits zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_round(x):
    """fp32 values rounded to the nearest bf16 number, ties to the even bit
    pattern (the rounding the GEMM path applies to fp32 activations), as
    uint16 bit patterns.  Inputs must be finite.

    Written from the definition: below |x| lies the bf16 number whose
    pattern is the top half of |x|'s pattern (truncation), above it the
    next pattern; the one at the smaller exact distance wins (the pattern
    0x7F80 above the largest finite bf16 counts as 2^128, so values past the
    last midpoint go to infinity, as round to nearest does)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    mag = x.view(np.uint32) & np.uint32(0x7FFFFFFF)
    sign = (x.view(np.uint32) >> np.uint32(16)) & np.uint32(0x8000)
    lo = mag >> np.uint32(16)
    hi = lo + np.uint32(1)

    def value(p):                      # exact magnitude of a bf16 pattern
        e = (p >> np.uint32(7)).astype(np.int64)
        f = (p & np.uint32(0x7F)).astype(np.float64)
        normal = np.ldexp(1.0 + f / 128.0, e - 127)
        sub = np.ldexp(f / 128.0, -126)
        return np.where(e == 0, sub, normal)

    a = mag.view(np.float32).astype(np.float64)
    d_lo = a - value(lo)
    d_hi = value(hi) - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == 1))
    return (np.where(up, hi, lo) | sign).astype(np.uint16)


def _as_matrix(rec):
    shape = rec["shape"]
    if len(shape) != 2:
        raise ValueError("the matmul reference needs a 2-D [n][k] weight")
    return unpack(rec).astype(np.float64)


def gemv_ref(rec, x):
    """fp32 activations x [m][k] times the dequantized weight [n][k]^T,
    in fp64.  Returns y [m][n] (float64)."""
    w_hat = _as_matrix(rec)
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] != w_hat.shape[1]:
        raise ValueError(f"x must be [m][{w_hat.shape[1]}], got {x.shape}")
    return x.astype(np.float64) @ w_hat.T


def gemm_ref(rec, x_bf16_bits):
    """bf16 activations (uint16 bit patterns) [m][k] times the dequantized
    weight [n][k]^T, in fp64.  Returns y [m][n] (float64)."""
    x = bf16_bits_to_f32(x_bf16_bits)
    return gemv_ref(rec, x)


def error_base(rec, x):
    """B[m, n] = sum_k |x[m, k] * w_hat[n, k]| in fp64; ``x`` is fp32 values
    (for a GEMM, first decode its bf16 bits with ``bf16_bits_to_f32``)."""
    w_hat = _as_matrix(rec)
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    return np.abs(x) @ np.abs(w_hat).T
