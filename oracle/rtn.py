"""Symmetric round-to-nearest (RTN) group quantization, packing and unpacking.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (cited by page title and section):

* "量化推理：INT8/INT4 的体积、困惑度与速度为什么不同步" (zffjzz.top), script
  function ``pack``: the weight array is viewed as consecutive groups of
  ``group`` elements in storage order; each group gets one little-endian fp32
  scale = max|w| / qmax (computed in fp32), a zero scale is replaced by 1; the
  codes are the fp32 quotients w / scale rounded half-to-even and clipped to
  +-qmax; int8 codes are stored as their two's-complement bytes; int4 codes
  are offset by +8 and stored two per byte, element 2i in the low nibble and
  element 2i+1 in the high nibble.  Function ``unpack`` reverses the packing
  and multiplies each code (as fp32) by its group's scale.
* "Huit bits, puis quatre" (smallbard.com), section "Arrondir": the same
  three formulas (scale, code, reconstructed weight) with qmax 127 / 7 and the
  half-step error bound.
* "Quantisation, worked as Chapter 23 works it" (nlp.jcrlabz.com), STEP 2
  ``quantise``: the per-tensor special case (one group = the whole tensor).

Readings taken where the pages are silent or disagree:

* Rounding is half-to-even (numpy ``rint``), clipping is to +-qmax (the
  Chapter 23 script clips the negative side to -qmax-1, which never binds
  because |w / scale| <= qmax up to one ulp and rint maps such a value to
  qmax).
* The quotient w / scale is an IEEE fp32 division, as in the ``pack``
  function, whose arrays are float32.
* int4 needs an even element count (two codes per byte).
* Inputs are finite; NaN / Inf behaviour is not defined here.
"""

import numpy as np

#: largest code magnitude per bit width: 2**(bits-1) - 1
QMAX = {8: 127, 4: 7}


def _check(bits, group, size):
    if bits not in QMAX:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    if group < 1 or size % group != 0:
        raise ValueError(f"group {group} does not divide the element count {size}")
    if bits == 4 and size % 2 != 0:
        raise ValueError("int4 packing needs an even number of elements")


def quantize_pack(w, bits, group):
    """Quantize an fp32 array with one scale per ``group`` consecutive
    elements (storage order) and pack the codes.

    Returns a record ``{bits, group, shape, payload, scales, q}``:
    ``payload`` is a uint8 array of ``size * bits / 8`` bytes, ``scales`` a
    float32 array with one scale per group, ``q`` the int8 codes.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    _check(bits, group, w.size)
    qmax = np.float32(QMAX[bits])

    # step 1: the groups are consecutive runs of `group` elements
    groups = w.reshape(-1, group)

    # step 2: absolute maximum per group (exact in fp32)
    m = np.abs(groups).max(axis=1)

    # step 3: scale = m / qmax, an fp32 division; an all-zero group gets 1
    scales = (m / qmax).astype(np.float32)
    scales[scales == np.float32(0.0)] = np.float32(1.0)

    # step 4: fp32 quotient, round half to even, clip to +-qmax
    r = (groups / scales[:, None]).astype(np.float32)
    q = np.clip(np.rint(r), -qmax, qmax).astype(np.int8).reshape(-1)

    # step 5: packing
    payload = pack_codes(q, bits)

    return dict(bits=bits, group=group, shape=list(w.shape),
                payload=payload, scales=scales.astype("<f4"), q=q)


def pack_codes(q, bits):
    """Pack signed codes (storage order) into the payload: int8 codes as
    their two's-complement bytes; int4 codes offset by +8, element 2i in the
    low nibble and element 2i+1 in the high nibble of byte i."""
    q = np.asarray(q, dtype=np.int8).reshape(-1)
    if bits == 8:
        return q.view(np.uint8).copy()
    if bits != 4:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    u = (q.astype(np.int16) + 8).astype(np.uint8)  # 1..15
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8)


def codes_from_payload(payload, bits, count):
    """Recover the signed integer codes from a payload (int16 array)."""
    b = np.asarray(payload, dtype=np.uint8).reshape(-1)
    if bits == 8:
        q = b.view(np.int8).astype(np.int16)
    elif bits == 4:
        low = (b & 0x0F).astype(np.int16)
        high = (b >> 4).astype(np.int16)
        q = np.stack((low, high), axis=1).reshape(-1) - 8
    else:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    if q.size != count:
        raise ValueError(f"payload holds {q.size} codes, expected {count}")
    return q


def unpack(rec):
    """Dequantize a record: w_hat = fp32(code) * scale of its group, as an
    fp32 array of the original shape."""
    shape = tuple(rec["shape"])
    size = int(np.prod(shape)) if shape else 1
    q = codes_from_payload(rec["payload"], rec["bits"], size)
    scales = np.asarray(rec["scales"], dtype=np.float32)
    w = q.astype(np.float32).reshape(-1, rec["group"]) * scales[:, None]
    return w.astype(np.float32).reshape(shape)


def payload_bytes(bits, n, k):
    """Bytes of packed codes for an n x k matrix."""
    return n * k * bits // 8


def num_scales(group, n, k):
    """Number of fp32 scales for an n x k matrix."""
    return n * k // group


def bits_per_weight(bits, group, scale_bytes=4):
    """Storage cost per weight including the group's scale."""
    return bits + 8.0 * scale_bytes / group
