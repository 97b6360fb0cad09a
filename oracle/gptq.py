"""GPTQ: choosing the group codes so that the layer's output, not each
weight, moves as little as possible.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: page "Huit bits, puis quatre" (smallbard.com), section "Arrondir
mieux : GPTQ".  What the section fixes:

* the goal is to keep X . W close to X . W' on typical layer inputs X, not
  each weight close to its rounded value;
* all that is needed from the inputs is the [K, K] matrix H = sum x^T x,
  accumulated over a few calibration batches (each weight matrix adds
  x^T x of its input to an accumulator before its product);
* a damping of 1 % of the mean of H's diagonal is added to H;
* H^-1 is factored as U^T U with U upper triangular (the Cholesky factor of
  the inverse);
* the input components are processed one after the other, in order; the
  component k of every output channel is rounded, its error divided by
  U[k, k] is carried onto every later component j > k with the factor
  U[k, j]; the group scale is fixed when the group's first component is
  reached, from the weights as corrected so far;
* the codes and scales are the same format as the plain round-to-nearest
  ones (same kernels, better chosen codes).

Orientation.  The stored weight is [n][k] (one row per output channel, the
groups and the input components along k), so the page's "row k of W" is
column k of the stored array, and every output channel is processed at once.

Readings taken where the section is silent:

* "Rounding" a component is the same quantizer as the plain path (oracle
  ``rtn``): the corrected weights are fp64, and each one is taken to fp32
  before the scale (fp32 division of the group's max |w| by qmax, zero
  replaced by 1) and the code (fp32 division, round half to even, clip to
  +-qmax) are computed; the rounded weight is fl32(code * scale).  With a
  diagonal H nothing is carried and the result is then bit-identical to the
  plain quantizer, which is what the page's first check asks for.
* The carried error is (w_k - w_hat_k) / U[k, k] in fp64, w_k being the
  corrected fp64 weight and w_hat_k the rounded one.
* H, its damping, its inverse and the factor are fp64 (the page runs the
  whole algorithm on the host in f64).
* A zero mean diagonal (no calibration data) leaves H singular: rejected.

The implementation follows the section's order literally: an explicit
inverse, the library Cholesky of that inverse, and one column at a time
with an immediate update of all later columns (no blocking).
"""

import numpy as np

from .rtn import QMAX, pack_codes


def hessian(batches):
    """H = sum over the calibration batches of x^T x, in fp64.

    ``batches`` is an iterable of fp32 arrays [t_b][k] (one row per token).
    Every product of two fp32 values is exact in fp64."""
    h = None
    for x in batches:
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
        if x.ndim != 2:
            raise ValueError("a calibration batch must be [tokens][k]")
        part = x.T @ x
        h = part if h is None else h + part
    if h is None:
        raise ValueError("no calibration batch")
    return h


def damped(h, frac=0.01):
    """H + frac * mean(diag H) * I (fp64)."""
    h = np.asarray(h, dtype=np.float64)
    lam = frac * np.mean(np.diag(h))
    if not lam > 0.0:
        raise ValueError("H has no positive mean diagonal; it cannot be damped")
    return h + lam * np.eye(h.shape[0])


def inverse_factor(hd):
    """U upper triangular with hd^-1 = U^T U: the inverse by the library
    routine, then the library Cholesky of the inverse (lower L with
    hd^-1 = L L^T), U = L^T."""
    hinv = np.linalg.inv(np.asarray(hd, dtype=np.float64))
    low = np.linalg.cholesky(hinv)
    return np.ascontiguousarray(low.T)


def _fl32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def quantize_pack(w, u, bits, group):
    """GPTQ codes of an fp32 weight [n][k] given the factor U [k][k].

    Returns the same record as ``rtn.quantize_pack`` ({bits, group, shape,
    payload, scales, q}) plus ``w_at_quant`` (fp64 [n][k]): the corrected
    value of every weight at the moment its component was rounded."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("GPTQ needs a 2-D [n][k] weight")
    n, k = w.shape
    u = np.asarray(u, dtype=np.float64)
    if u.shape != (k, k):
        raise ValueError(f"U must be [{k}][{k}], got {u.shape}")
    if bits not in QMAX:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    if group < 1 or k % group != 0:
        raise ValueError(f"group {group} must divide k = {k}")
    if bits == 4 and group % 2 != 0:
        raise ValueError("int4 packing needs an even group")
    qmax = np.float32(QMAX[bits])

    cur = w.astype(np.float64)          # weights as corrected so far
    q = np.zeros((n, k), dtype=np.int8)
    scales = np.zeros((n, k // group), dtype=np.float32)
    at_quant = np.zeros((n, k), dtype=np.float64)
    s = None
    for c in range(k):
        if c % group == 0:
            # the group's scale, from the corrected weights of the whole group
            m = np.abs(_fl32(cur[:, c:c + group])).max(axis=1)
            s = (m / qmax).astype(np.float32)
            s[s == np.float32(0.0)] = np.float32(1.0)
            scales[:, c // group] = s
        at_quant[:, c] = cur[:, c]
        r = (_fl32(cur[:, c]) / s).astype(np.float32)
        code = np.clip(np.rint(r), -qmax, qmax)
        q[:, c] = code.astype(np.int8)
        w_hat = (code.astype(np.float32) * s).astype(np.float32)
        err = (cur[:, c] - w_hat.astype(np.float64)) / u[c, c]
        # carry the error onto every later component of each channel
        cur[:, c + 1:] -= np.outer(err, u[c, c + 1:])

    q = q.reshape(-1)
    return dict(bits=bits, group=group, shape=[n, k],
                payload=pack_codes(q, bits),
                scales=scales.reshape(-1).astype("<f4"), q=q,
                w_at_quant=at_quant)


def gptq(w, h, bits, group, damp=0.01):
    """The whole chain from the accumulated H: damping, factor, codes."""
    return quantize_pack(w, inverse_factor(damped(h, damp)), bits, group)
