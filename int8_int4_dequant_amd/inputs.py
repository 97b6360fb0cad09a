"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check.

This module only draws random numbers and lays them out; it holds none of
the quantization or matmul arithmetic, so both the HIP path and the CPU
oracle can be fed from it without sharing any of the method.

Weights are generated directly in the stored layout [n][k] (one row per
output channel, k contiguous), as fp32 draws of N(0, sigma) with numpy's
``default_rng`` (PCG64) seeded per matrix.  A configuration written "A x B"
(in x out) is stored as n = B rows of k = A values.

The five workloads (sizes of the 7B- and 70B-style linear layers the pages
talk about; the pages ship no weights, so seeded Gaussians stand in for
trained ones):

=====  =====================================================================
c1     one 256 x 256 matrix, N(0, 0.05), seed 0; int8 and int4, group 32;
       one activation row N(0, 1)
c2     4096 x 4096, N(0, 0.02) with 0.1 % of the entries (16,777 distinct
       positions) replaced by +-U(0.5, 1.0); int8, one scale per output
       channel (group = k = 4096); M = 1
c3     MLP up (n=11008, k=4096) and down (n=4096, k=11008), N(0, 0.02);
       int4 group 128; M in {1, 4, 8}
c4     32 layers x [q, k, v, o (4096 x 4096), gate, up (n=11008, k=4096),
       down (n=4096, k=11008)] = 224 matrices, N(0, 0.02); int4 group 32;
       one M = 1 activation per k
c5     (n=28672, k=8192), N(0, 0.015); int4 group 128; activations
       M = 2048 x 8192 N(0, 1) rounded to bf16 (round to nearest even)
=====  =====================================================================
"""

import concurrent.futures as _cf
import os

import numpy as np

# ---------------------------------------------------------------- basics


def weight(seed, n, k, sigma):
    """fp32 [n][k] with N(0, sigma) entries from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, k), dtype=np.float32)
    a *= np.float32(sigma)
    return a


def activations(seed, m, k):
    """fp32 [m][k] with N(0, 1) entries from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((m, k), dtype=np.float32)


def bf16_round_bits(a):
    """Round fp32 values to bf16 (round to nearest, ties to even) and return
    the uint16 bit patterns.  Inputs must be finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_activations(seed, m, k):
    """bf16 bit patterns [m][k] of N(0, 1) draws (see ``bf16_round_bits``)."""
    return bf16_round_bits(activations(seed, m, k))


# ---------------------------------------------------------------- configs

C1 = dict(name="c1_tiny_256x256", n=256, k=256, sigma=0.05, group=32,
          w_seed=0, x_seed=1)

C2 = dict(name="c2_gemv_int8_per_channel_4096x4096", n=4096, k=4096,
          sigma=0.02, bits=8, group=4096, outlier_frac=0.001,
          w_seed=[2, 0], x_seed=[2, 0, 100], m=1)

C3 = dict(name="c3_gemv_int4_g128_mlp", bits=4, group=128, sigma=0.02,
          mats=[dict(tag="up", n=11008, k=4096, j=0),
                dict(tag="down", n=4096, k=11008, j=1)],
          ms=[1, 4, 8])

C4_SLOTS = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
            ("o", 4096, 4096), ("gate", 11008, 4096), ("up", 11008, 4096),
            ("down", 4096, 11008)]
C4 = dict(name="c4_7b_stack_int4_g32", layers=32, bits=4, group=32,
          sigma=0.02, slots=C4_SLOTS)

C5 = dict(name="c5_prefill_gemm_int4_g128_28672x8192", n=28672, k=8192,
          m=2048, bits=4, group=128, sigma=0.015, w_seed=[5, 0],
          x_seed=[5, 0, 100])


def c1_weight():
    return weight(C1["w_seed"], C1["n"], C1["k"], C1["sigma"])


def c1_x():
    return activations(C1["x_seed"], 1, C1["k"])


def c2_weight():
    """c2 weight: N(0, 0.02) plus round(0.001 * n * k) outliers at distinct
    positions (uniform without replacement), sign +-1 with probability 1/2
    and magnitude U(0.5, 1.0)."""
    n, k = C2["n"], C2["k"]
    rng = np.random.default_rng(C2["w_seed"])
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(C2["sigma"])
    count = int(round(C2["outlier_frac"] * n * k))
    pos = rng.choice(n * k, size=count, replace=False)
    sign = np.where(rng.integers(0, 2, size=count) == 1, 1.0, -1.0)
    mag = rng.uniform(0.5, 1.0, size=count)
    w.reshape(-1)[pos] = (sign * mag).astype(np.float32)
    return w


def c2_x():
    return activations(C2["x_seed"], C2["m"], C2["k"])


def c3_weight(j):
    mat = C3["mats"][j]
    return weight([3, j], mat["n"], mat["k"], C3["sigma"])


def c3_x(j, m):
    return activations([3, j, 100 + m], m, C3["mats"][j]["k"])


def c4_matrices():
    """List of (layer, slot_name, n, k, seed) for the 224 matrices."""
    out = []
    for layer in range(C4["layers"]):
        for s, (tag, n, k) in enumerate(C4["slots"]):
            out.append((layer, tag, n, k, [4, 7 * layer + s]))
    return out


def c4_weight(layer, slot):
    tag, n, k = C4["slots"][slot]
    return weight([4, 7 * layer + slot], n, k, C4["sigma"])


def c4_x(k):
    """The fixed M = 1 activation used by every matrix of reduction size k."""
    return activations([4, 0 if k == 4096 else 1, 100], 1, k)


def c4_x8(k):
    """8 rows of x of length k for a decode pass through the stack at 8 rows
    (several sequences at once): fp32 N(0, 1)."""
    return activations(808 + k, 8, k)


def c4_weights_parallel(callback, threads=None):
    """Generate the 224 c4 matrices on a thread pool (numpy releases the GIL
    while filling) and call ``callback(index, layer, tag, w)`` for each, in
    order, as soon as it is ready.  Host memory stays bounded to a few
    matrices in flight."""
    mats = c4_matrices()
    threads = threads or min(16, os.cpu_count() or 1)

    def gen(entry):
        layer, tag, n, k, seed = entry
        return weight(seed, n, k, C4["sigma"])

    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        window = []
        it = iter(enumerate(mats))
        for _ in range(threads):
            try:
                i, e = next(it)
            except StopIteration:
                break
            window.append((i, e, ex.submit(gen, e)))
        while window:
            i, e, fut = window.pop(0)
            callback(i, e[0], e[1], fut.result())
            try:
                i2, e2 = next(it)
                window.append((i2, e2, ex.submit(gen, e2)))
            except StopIteration:
                pass


def c5_weight():
    return weight(C5["w_seed"], C5["n"], C5["k"], C5["sigma"])


def c5_x_bf16():
    return bf16_activations(C5["x_seed"], C5["m"], C5["k"])


# ------------------------------------------------------------ GPTQ calibration
#
# One layer of the small model of the GPTQ section (model width 512,
# feed-forward width 1368, so its largest matrix is 1368 x 512), with the
# section's calibration budget of 8 batches of 16 sequences, 65,536 tokens.
# The trained weights and real layer inputs are not available: the weights
# are N(0, 0.02) draws, and the inputs are synthetic activations whose
# components are correlated (a low-rank common part plus independent noise),
# have uneven magnitudes, and include three components 2.5x larger than the
# rest (the section's calibration statistics find three such components,
# 112, 257 and 285, about 2.5 times the median).

SMALLEM_D = 512
SMALLEM_FFN = 1368
CALIB_TOKENS = 65536
#: (name, n, k, calibration input) of the layer's linear maps, stored [n][k]
SMALLEM_LAYER = [
    ("q", SMALLEM_D, SMALLEM_D, "attn_in"),
    ("k", SMALLEM_D, SMALLEM_D, "attn_in"),
    ("v", SMALLEM_D, SMALLEM_D, "attn_in"),
    ("o", SMALLEM_D, SMALLEM_D, "o_in"),
    ("gate", SMALLEM_FFN, SMALLEM_D, "ffn_in"),
    ("up", SMALLEM_FFN, SMALLEM_D, "ffn_in"),
    ("down", SMALLEM_D, SMALLEM_FFN, "down_in"),
]
#: calibration inputs: name -> (k, seed)
SMALLEM_INPUTS = {
    "attn_in": (SMALLEM_D, [6, 100]),
    "o_in": (SMALLEM_D, [6, 101]),
    "ffn_in": (SMALLEM_D, [6, 102]),
    "down_in": (SMALLEM_FFN, [6, 103]),
}
SMALLEM_OUTLIER_COMPONENTS = (112, 257, 285)


def smallem_group(k):
    """int4 group of a map with k inputs: 64, or for the 1368-input down map
    (not a multiple of 64, and a group may not span two output channels)
    72, the smallest divisor of 1368 above 64."""
    return 64 if k % 64 == 0 else 72


def calibration_activations(seed, t, k):
    """fp32 [t][k] correlated activations from ``default_rng(seed)``:
    x = (0.8 * z_c . F + 0.4 * z_i) * c, with z_c [t][r] and z_i [t][k]
    N(0, 1), r = max(1, k // 16) common factors, F [r][k] N(0, 1/r), and
    per-component magnitudes c = exp(0.5 * N(0, 1)), multiplied by 2.5 at
    the components 112, 257 and 285 that exist."""
    rng = np.random.default_rng(seed)
    r = max(1, k // 16)
    f = rng.standard_normal((r, k), dtype=np.float32)
    f *= np.float32(1.0 / np.sqrt(r))
    c = np.exp(0.5 * rng.standard_normal(k)).astype(np.float32)
    for j in SMALLEM_OUTLIER_COMPONENTS:
        if j < k:
            c[j] *= np.float32(2.5)
    zc = rng.standard_normal((t, r), dtype=np.float32)
    x = zc @ f
    x *= np.float32(0.8)
    x += np.float32(0.4) * rng.standard_normal((t, k), dtype=np.float32)
    x *= c[None, :]
    return x


def smallem_weight(slot):
    """fp32 weight [n][k] of the layer's map number ``slot`` (q, k, v, o,
    gate, up, down)."""
    _, n, k, _ = SMALLEM_LAYER[slot]
    return weight([6, slot], n, k, 0.02)


def smallem_calibration(name, t=CALIB_TOKENS):
    k, seed = SMALLEM_INPUTS[name]
    return calibration_activations(seed, t, k)


# ------------------------------------------------------------ edge cases


def tie_vector():
    """Eight values whose group scale is exactly 1 at int4 (max 7), with
    exact half-integers to exercise ties-to-even."""
    return np.array([7.0, 2.5, -2.5, 3.5, -0.5, 0.5, 1.5, 6.5], np.float32)


def near_tie_matrix(seed, bits, rows, group):
    """Rows of ``group`` values, each row with its own random maximum; the
    other entries sit on, or 1-2 ulps either side of, the half-way points
    (j + 1/2) * max / qmax between codes.  Returned as fp32 [rows][group]."""
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(seed)
    out = np.empty((rows, group), np.float32)
    for r in range(rows):
        mx = np.float32(rng.uniform(0.01, 4.0))
        step = np.float64(mx) / qmax
        j = rng.integers(-qmax, qmax, size=group)
        v = ((j + 0.5) * step).astype(np.float32)
        ulps = rng.integers(-2, 3, size=group).astype(np.int32)
        v = (v.view(np.int32) + ulps * np.sign(v).astype(np.int32)).view(np.float32)
        v = np.clip(v, -mx, mx)
        v[0] = mx if rng.integers(0, 2) else -mx
        out[r] = v
    return out


def subnormal_matrix(seed, rows, group):
    """Rows whose values are all fp32 subnormals or tiny normals."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, group), dtype=np.float32)
    a *= np.float32(1e-39)
    return a
