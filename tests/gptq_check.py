"""Comparison of GPTQ codes from the GPU with the oracle's (page "Huit bits,
puis quatre", section "Arrondir mieux : GPTQ").

Both sides decide every code in fp32 from an fp64 weight that has been
corrected by the carried errors of all earlier components.  The two fp64
weights are the same sum taken in another order (the GPU adds blocked
updates of d * (U[c][j] / U[c][c]); the oracle adds (d / U[c][c]) * U[c][j]
one component at a time), and when the GPU uses its own factor, with a U
that differs from the oracle's in its last bits.  So a code, or a group's
scale, can differ without a bug when the oracle's weight lies within that
difference of a rounding boundary; after such a case the two rows carry
different errors and their later codes are not comparable.

``compare`` accepts a row when it is identical, or when its first difference
is such a boundary case:

* weight bound.  For weight (i, j) at the moment it is rounded,
      eps[i, j] = (1 + A) * ( tau * (|w[i, j]| + sum_{c<j} |e[i, c] U[c][j]|)
                              + dU * sum_{c<j} |e[i, c]| (1 + |V[c][j]|) )
  with e the oracle's carried errors (w - w_hat) / U[c][c], V[c][j] =
  U[c][j] / U[c][c], tau = 2 (k + 3) 2^-53 (the summation-order bound of
  two fp64 evaluations of the same k-term sum), dU = max |U_gpu - U_oracle|
  (0 when both use the same factor), and 1 + A with
  A = max_j sum_{c<j} |V[c][j]| the first-order amplification of those
  differences through the errors they change;
* a scale is excused when the GPU's value lies in the range of
  fl32(max_j |fl32(v_j)| / qmax) over weights v_j within eps of the
  oracle's group weights at the group's first component;
* a code is excused when the GPU's code lies in the range of
  clip(rint(fl32(fl32(v) / S))) over v within eps of the oracle's weight.

Excused rows must still hold valid codes (|q| <= qmax) and positive finite
scales; the caller asserts that they are few.
"""

import numpy as np

QMAX = {4: 7, 8: 127}


def _codes(payload, bits, n, k):
    b = np.asarray(payload, np.uint8).reshape(-1)
    if bits == 8:
        q = b.view(np.int8).astype(np.int32)
    else:
        q = np.empty(2 * b.size, np.int32)
        q[0::2] = (b & 15).astype(np.int32) - 8
        q[1::2] = (b >> 4).astype(np.int32) - 8
    return q.reshape(n, k)


def _f32(v):
    return np.asarray(v, np.float64).astype(np.float32)


def _code_range(w_lo, w_hi, s, qmax):
    lo = np.clip(np.rint((_f32(w_lo) / np.float32(s)).astype(np.float32)), -qmax, qmax)
    hi = np.clip(np.rint((_f32(w_hi) / np.float32(s)).astype(np.float32)), -qmax, qmax)
    return int(lo), int(hi)


def compare(w, u_ref, want, payload, scales, bits, group, u_gpu=None):
    """Returns (exact_rows, excused_rows, bad) where ``bad`` lists
    (row, component, reason) of differences that no boundary explains.
    ``want`` is the oracle record for (w, u_ref) with its ``w_at_quant``."""
    w = np.asarray(w, np.float32).astype(np.float64)
    n, k = w.shape
    qmax = QMAX[bits]
    u = np.asarray(u_ref, np.float64)
    qo = want["q"].reshape(n, k).astype(np.int32)
    so = want["scales"].reshape(n, k // group)
    qg = _codes(payload, bits, n, k)
    sg = np.asarray(scales, np.float32).reshape(n, k // group)

    diag = np.diag(u)
    vu = np.triu(u / diag[:, None], 1)              # V[c][j] for c < j
    w_hat = (qo.astype(np.float32) * np.repeat(so, group, axis=1)).astype(np.float32)
    e = (want["w_at_quant"] - w_hat.astype(np.float64)) / diag[None, :]
    tau = 2.0 * (k + 3) * 2.0 ** -53
    amp = 1.0 + float(np.max(np.sum(np.abs(vu), axis=0))) if k > 1 else 1.0
    du = 0.0 if u_gpu is None else float(np.max(np.abs(np.asarray(u_gpu) - u)))
    au = np.abs(np.triu(u, 1))

    def eps_row(i, c_end):
        """eps of row i's weights as corrected by components < c_end."""
        ei = np.abs(e[i, :c_end])
        mag = np.abs(w[i]) + ei @ au[:c_end]
        upd = ei @ (np.triu(np.ones((c_end, k)), 1) + np.abs(vu[:c_end])) if du else 0.0
        return amp * (tau * mag + du * upd)

    exact, excused, bad = 0, 0, []
    for i in range(n):
        diff_code = np.nonzero(qg[i] != qo[i])[0]
        diff_scale = np.nonzero(sg[i] != so[i])[0]
        c_code = int(diff_code[0]) if diff_code.size else k
        c_scale = int(diff_scale[0]) * group if diff_scale.size else k
        if c_code == k and c_scale == k:
            exact += 1
            continue
        if c_scale <= c_code:
            c0 = c_scale
            # the group's weights as corrected by the components before c0
            cur = w[i, c0:c0 + group] - e[i, :c0] @ u[:c0, c0:c0 + group]
            eps = eps_row(i, c0)[c0:c0 + group]
            lo = np.maximum(np.abs(cur) - eps, 0.0)
            hi = np.abs(cur) + eps
            m_lo, m_hi = np.max(np.abs(_f32(lo))), np.max(np.abs(_f32(hi)))
            s_lo = np.float32(m_lo) / np.float32(qmax)
            s_hi = np.float32(m_hi) / np.float32(qmax)
            s_lo = np.float32(1.0) if s_lo == 0 else s_lo
            ok = s_lo <= sg[i, c0 // group] <= s_hi
            reason = f"scale {sg[i, c0 // group]!r} outside [{s_lo!r}, {s_hi!r}]"
            c = c0
        else:
            c = c_code
            wq = want["w_at_quant"][i, c]
            eps = eps_row(i, c)[c]
            lo, hi = _code_range(wq - eps, wq + eps, so[i, c // group], qmax)
            ok = lo <= qg[i, c] <= hi
            reason = f"code {qg[i, c]} outside [{lo}, {hi}] (oracle {qo[i, c]})"
        valid = (np.all(np.abs(qg[i]) <= qmax) and np.all(np.isfinite(sg[i]))
                 and np.all(sg[i] > 0))
        if ok and valid:
            excused += 1
        else:
            bad.append((i, c, reason if not ok else "invalid codes or scales"))
    return exact, excused, bad
