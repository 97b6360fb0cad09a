"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: payload, scales and unpacked weights bit-identical; GEMV outputs within
1e-5 * sum|x * w_hat| and GEMM outputs within 8e-3 * sum|x * w_hat| per
element.  Small cases compare every element; the full-size workloads compare
every byte of the quantization where the oracle is quick enough, otherwise
sampled rows (groups never cross rows there, so a row's payload depends on
that row only), in the same launch configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
from int8_int4_dequant_amd import inputs, qw

pytestmark = pytest.mark.gpu

GEMV_TOL = 1e-5
GEMM_TOL = 8e-3


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bits(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def quant_both(w, bits, group):
    ref = oracle.quantize_pack(w, bits, group)
    rec = qw.quantize_pack(dev(w), bits, group)
    assert same_bits(host(rec["scales"]), ref["scales"]), "scales differ"
    assert same_bits(host(rec["payload"]), ref["payload"]), "payload differs"
    return ref, rec


def check_unpack(ref, rec):
    assert same_bits(host(qw.unpack(rec)), oracle.unpack(ref)), "unpack differs"


def check_gemv(ref, rec, x):
    y = host(qw.gemv(rec, dev(x)))
    yr = oracle.gemv_ref(ref, x)
    B = oracle.error_base(ref, x)
    err = np.abs(y.astype(np.float64) - yr)
    assert np.all(err <= GEMV_TOL * B), f"gemv max err/B = {np.max(err / np.maximum(B, 1e-300))}"
    return y


def check_gemm(ref, rec, xb):
    y = host(qw.gemm(rec, dev(xb.view(np.int16))))
    yr = oracle.gemm_ref(ref, xb)
    B = oracle.error_base(ref, oracle.bf16_bits_to_f32(xb))
    err = np.abs(y.astype(np.float64) - yr)
    assert np.all(err <= GEMM_TOL * B), f"gemm max err/B = {np.max(err / np.maximum(B, 1e-300))}"
    return y


# ------------------------------------------------------------ small cases


@pytest.mark.parametrize("bits", [8, 4])
def test_tiny_config(bits):
    w, x = inputs.c1_weight(), inputs.c1_x()
    ref, rec = quant_both(w, bits, 32)
    check_unpack(ref, rec)
    check_gemv(ref, rec, x)


def test_worked_example_on_gpu():
    w = np.array([[0.12, -0.45, 0.33, -0.08, 0.51, -0.22, 0.07, -0.37]], np.float32)
    for bits, hexp in ((8, "1e9052ec7fc911a4"), (4, "2a7d5f39")):
        ref, rec = quant_both(w, bits, 8)
        assert host(rec["payload"]).tobytes().hex() == hexp
        check_unpack(ref, rec)


def test_ties_on_gpu():
    w = inputs.tie_vector().reshape(1, 8)
    ref, rec = quant_both(w, 4, 8)
    assert host(rec["payload"]).tobytes().hex() == "afc688ea"


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("group", [32, 128])
def test_near_ties(bits, group):
    w = inputs.near_tie_matrix(seed=100 + bits + group, bits=bits, rows=512, group=group)
    ref, rec = quant_both(w.reshape(64, -1), bits, group)
    check_unpack(ref, rec)


@pytest.mark.parametrize("bits", [8, 4])
def test_subnormal_and_zero_groups(bits):
    w = np.concatenate([inputs.subnormal_matrix(3, 16, 64),
                        np.zeros((4, 64), np.float32),
                        inputs.weight(4, 12, 64, 1e-3)], axis=0)
    w[18, 5] = np.float32(1e-45)  # smallest subnormal alone in a group
    w[0, 32:64] = np.linspace(-3.3e38, 3.3e38, 32, dtype=np.float32)  # scale > 2^125 at int4
    for group in (32, 64):
        ref, rec = quant_both(w, bits, group)
        check_unpack(ref, rec)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("group,n,k", [
    (8, 16, 64), (16, 16, 64), (64, 8, 256), (256, 8, 512), (512, 6, 1024),  # subgroup
    (1024, 6, 2048), (4096, 4, 4096), (11008, 3, 11008), (2048, 5, 6144),   # block
    (1, 4, 16), (6, 4, 48), (24, 5, 48), (4 * 64, 4, 64), (3 * 96, 3, 96),   # generic
])
def test_group_families(bits, group, n, k):
    w = inputs.weight(group + n + k, n, k, 0.3)
    ref, rec = quant_both(w, bits, group)
    check_unpack(ref, rec)
    if group % k == 0 or k % group == 0:
        x = inputs.activations(7, 3, k)
        check_gemv(ref, rec, x)


@pytest.mark.parametrize("bits", [8, 4])
def test_per_tensor_group(bits):
    w = inputs.weight(31, 24, 256, 0.2)
    ref, rec = quant_both(w, bits, w.size)
    check_unpack(ref, rec)
    check_gemv(ref, rec, inputs.activations(8, 2, 256))
    check_gemm(ref, rec, inputs.bf16_activations(9, 5, 256))


@pytest.mark.parametrize("bits", [8, 4])
def test_unaligned_pointers_take_generic_kernels(bits):
    n, k, group = 24, 128, 32
    w = inputs.weight(5, n, k, 0.1)
    ref = oracle.quantize_pack(w, bits, group)
    wd = torch.empty(n * k + 1, dtype=torch.float32, device="cuda")
    wd[1:] = dev(w).reshape(-1)
    nb = n * k * bits // 8
    pd = torch.zeros(nb + 1, dtype=torch.uint8, device="cuda")
    sd = torch.zeros(n * k // group + 1, dtype=torch.float32, device="cuda")
    assert qw.qw_debug_path(0, bits, group, n, k, wd[1:], pd[1:]) == 3
    assert qw.qw_quantize_pack(bits, group, n, k, wd[1:], pd[1:], sd[1:]) == 0
    assert same_bits(host(pd[1:]), ref["payload"])
    assert same_bits(host(sd[1:]), ref["scales"])
    out = torch.zeros(n * k + 1, dtype=torch.float32, device="cuda")
    assert qw.qw_unpack(bits, group, n, k, pd[1:], sd[1:], out[1:]) == 0
    assert same_bits(host(out[1:]), oracle.unpack(ref).reshape(-1))
    x = inputs.activations(6, 2, k)
    xd = torch.zeros(2 * k + 1, dtype=torch.float32, device="cuda")
    xd[1:] = dev(x).reshape(-1)
    y = torch.zeros(2 * n, dtype=torch.float32, device="cuda")
    assert qw.qw_gemv(bits, group, n, k, pd[1:], sd[1:], 2, xd[1:], y) == 0
    B = oracle.error_base(ref, x)
    assert np.all(np.abs(host(y).reshape(2, n) - oracle.gemv_ref(ref, x)) <= GEMV_TOL * B)


# ------------------------------------------------------------------- GEMV


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 128), (8, 16), (8, 4096 // 4)])
@pytest.mark.parametrize("n,k", [(13, 4096), (77, 11008), (200, 1024), (8, 32 * 3)])
def test_gemv_shapes_all_m(bits, group, n, k):
    if k % group:
        pytest.skip("group does not divide k")
    w = inputs.weight(n * 7 + k, n, k, 0.02)
    ref, rec = quant_both(w, bits, group)
    for m in range(1, 9):
        check_gemv(ref, rec, inputs.activations(m * 13 + n, m, k))


# A lone matrix with fewer than 32768 rows (M <= 4; 16384 for M > 4) runs the
# split-K kernel (four waves per block share rows, each a quarter of K); a
# taller one the row-streaming kernel.  Short rows (k = 8, 16, 24: some waves
# get no chunk), a row count that is not a multiple of the block's 4 rows,
# and both kernels at every m.
@pytest.mark.parametrize("bits,group,n,k", [
    (4, 8, 9, 8), (8, 16, 6, 16), (4, 24, 7, 24), (4, 32, 4099, 512),
    (4, 32, 32768 + 5, 256), (8, 256, 16384 + 3, 256),
])
def test_gemv_split_and_stream_kernels(bits, group, n, k):
    w = inputs.weight(n + 3 * k, n, k, 0.02)
    ref, rec = quant_both(w, bits, group)
    for m in (1, 2, 5, 8):
        check_gemv(ref, rec, inputs.activations(m + n, m, k))


def test_gemv_k_zero_and_empty():
    rec = dict(bits=4, group=32, shape=[5, 0],
               payload=torch.empty(0, dtype=torch.uint8, device="cuda"),
               scales=torch.empty(0, dtype=torch.float32, device="cuda"))
    y = torch.full((3, 5), 7.0, device="cuda")
    x = torch.empty((3, 0), dtype=torch.float32, device="cuda")
    assert qw.qw_gemv(4, 32, 5, 0, rec["payload"], rec["scales"], 3, x, y) == 0
    assert np.all(host(y) == 0)
    w = np.zeros((0, 64), np.float32)
    rec = qw.quantize_pack(dev(w), 4, 32)
    assert rec["payload"].numel() == 0 and rec["scales"].numel() == 0


def test_gemv_deterministic():
    w = inputs.weight(1, 300, 4096, 0.02)
    rec = qw.quantize_pack(dev(w), 4, 128)
    x = dev(inputs.activations(2, 4, 4096))
    y1 = host(qw.gemv(rec, x))
    y2 = host(qw.gemv(rec, x))
    assert same_bits(y1, y2)


# ------------------------------------------------------------------- GEMM


@pytest.mark.parametrize("bits,group", [(4, 128), (4, 32), (8, 64), (8, 128)])
@pytest.mark.parametrize("m,n,k", [(1, 256, 512), (9, 300, 256), (40, 77, 1024),
                                   (300, 520, 512), (257, 2048, 128)])
def test_gemm_shapes(bits, group, m, n, k):
    w = inputs.weight(m + n + k, n, k, 0.015)
    ref, rec = quant_both(w, bits, group)
    check_gemm(ref, rec, inputs.bf16_activations(m * 3 + 1, m, k))


def test_gemm_generic_shape():
    w = inputs.weight(3, 33, 96, 0.1)
    ref, rec = quant_both(w, 4, 16)
    assert qw.qw_debug_path(3, 4, 16, 33, 96, rec["payload"], rec["payload"]) == 3
    check_gemm(ref, rec, inputs.bf16_activations(4, 7, 96))


def test_codes_path_agrees_with_dequantized_path():
    # rows 1, 9, 40, 300 as in the Smallem tests: the GEMM (dequantized
    # operand) and, at one row, the GEMV (codes) against unpack + fp64.
    w = inputs.weight(77, 256, 1024, 0.02)
    ref, rec = quant_both(w, 4, 32)
    w_hat = host(qw.unpack(rec)).astype(np.float64)
    for m in (1, 9, 40, 300):
        xb = inputs.bf16_activations(500 + m, m, 1024)
        xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
        y = host(qw.gemm(rec, dev(xb.view(np.int16))))
        B = np.abs(xf) @ np.abs(w_hat).T
        assert np.all(np.abs(y - xf @ w_hat.T) <= GEMM_TOL * B)
        if m == 1:
            yv = host(qw.gemv(rec, dev(xf.astype(np.float32))))
            assert np.all(np.abs(yv - xf @ w_hat.T) <= GEMV_TOL * B)


@pytest.mark.parametrize("bits,group,n,k", [(4, 32, 256, 1024), (8, 128, 300, 512),
                                           (4, 128, 520, 256)])
def test_matmul_dispatch_across_m(bits, group, n, k):
    """qw_matmul (QuantizedMatmul) at the Smallem test rows 1, 9, 40, 300 and
    around the crossover: up to MATMUL_GEMV_MAX_M rows it is the codes GEMV
    (bit for bit, and within the GEMV bar); above, the work buffer holds
    exactly the oracle's bf16 rounding of x, the result equals qw_gemm on
    those bits, and it is within the GEMM bar of the fp32-x product."""
    w = inputs.weight(n + k + bits, n, k, 0.02)
    ref, rec = quant_both(w, bits, group)
    for m in (1, 4, 5, 9, 40, 300):
        x = inputs.activations(900 + m, m, k)
        xd = dev(x)
        nb = qw.qw_matmul_work_bytes(m, k)
        assert (nb == 0) == (m <= qw.MATMUL_GEMV_MAX_M)
        work = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        assert qw.qw_matmul(bits, group, n, k, rec["payload"], rec["scales"], m, xd, y,
                            work if nb else None, nb) == 0
        yh = host(y)
        yr = oracle.gemv_ref(ref, x)
        B = oracle.error_base(ref, x)
        err = np.abs(yh.astype(np.float64) - yr)
        if m <= qw.MATMUL_GEMV_MAX_M:
            assert same_bits(yh, host(qw.gemv(rec, xd)))
            assert np.all(err <= GEMV_TOL * B)
        else:
            xb = oracle.bf16_round(x)
            got = host(work)[: m * k * 2].view(np.uint16).reshape(m, k)
            assert np.array_equal(got, xb), "bf16 rounding of x differs"
            assert same_bits(yh, host(qw.gemm(rec, dev(xb.view(np.int16)))))
            assert np.all(err <= GEMM_TOL * B)


@pytest.mark.parametrize("offset", [0, 1])
def test_matmul_rounding_tail_and_unaligned_x(offset):
    """The bf16 rounding of x on its element-wise path: a count that is not a
    multiple of 8 (5 x 100 = 500 values) and, with offset 1, an x that is
    only 4-byte aligned."""
    n, k, m = 40, 100, 5
    w = inputs.weight(61, n, k, 0.05)
    ref, rec = quant_both(w, 4, 4)
    x = inputs.activations(62, m, k)
    buf = torch.zeros(m * k + offset, dtype=torch.float32, device="cuda")
    buf[offset:] = dev(x.reshape(-1))
    xv = buf[offset:].view(m, k)
    nb = qw.qw_matmul_work_bytes(m, k)
    work = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    y = qw.matmul(rec, xv, work=work)
    got = host(work)[: m * k * 2].view(np.uint16).reshape(m, k)
    assert np.array_equal(got, oracle.bf16_round(x))
    yr = oracle.gemv_ref(ref, x)
    B = oracle.error_base(ref, x)
    assert np.all(np.abs(host(y).astype(np.float64) - yr) <= GEMM_TOL * B)


# The tiled kernel runs one 256 x 256 output tile per block.  When the last
# round of tiles would leave at least half the compute units idle, those
# tiles are split in two along K and both halves add into Y (zeroed first).
# Shapes: every tile split (small), every tile whole (140 tiles), and 256
# whole tiles followed by 100 split ones; k = 192 gives halves of one and two
# k-steps.
@pytest.mark.parametrize("bits,group,m,n,k", [
    (4, 64, 300, 520, 192),
    (4, 128, 64, 256 * 140, 128),
    (8, 128, 300, 256 * 178 - 40, 128),
])
def test_gemm_split_tail(bits, group, m, n, k):
    w = inputs.weight(n + k, n, k, 0.02)
    ref, rec = quant_both(w, bits, group)
    check_gemm(ref, rec, inputs.bf16_activations(m + 7, m, k))


# Up to 32 rows of X the small-M kernel runs: a 32-row tile of 32 or 64
# columns per block, K split over the block's four waves (some idle when
# k / 64 < 4), partial tiles added in LDS.  Ragged columns, per-tensor
# groups, int8, and a width that selects 64-column tiles (n >= 16384).
@pytest.mark.parametrize("bits,group,m,n,k", [
    (4, 128, 1, 300, 512), (4, 32, 2, 77, 64), (8, 64, 17, 130, 192), (4, 32, 31, 96, 128),
    (8, 128, 32, 257, 1024), (4, 96 * 2, 5, 40, 96 * 2), (4, 256, 3, 16448, 256),
    (4, 1024 * 3, 7, 3, 1024),
])
def test_gemm_small_m(bits, group, m, n, k):
    w = inputs.weight(m + n + k + 5, n, k, 0.02)
    ref, rec = quant_both(w, bits, group)
    check_gemm(ref, rec, inputs.bf16_activations(m * 5 + 3, m, k))


def test_gemm_ignores_stale_output():
    # the split tiles accumulate into Y: stale contents (NaN) must not leak
    w = inputs.weight(21, 300, 512, 0.02)
    ref, rec = quant_both(w, 4, 32)
    xb = inputs.bf16_activations(22, 40, 512)
    out = torch.full((40, 300), float("nan"), dtype=torch.float32, device="cuda")
    y = host(qw.gemm(rec, dev(xb.view(np.int16)), out=out))
    yr = oracle.gemm_ref(ref, xb)
    B = oracle.error_base(ref, oracle.bf16_bits_to_f32(xb))
    assert np.all(np.abs(y - yr) <= GEMM_TOL * B)


def test_gemm_deterministic():
    w = inputs.weight(9, 512, 1024, 0.02)
    rec = qw.quantize_pack(dev(w), 4, 128)
    xb = dev(inputs.bf16_activations(3, 300, 1024).view(np.int16))
    assert same_bits(host(qw.gemm(rec, xb)), host(qw.gemm(rec, xb)))


# ------------------------------------------------------ full-size configs


def test_config2_int8_per_channel():
    w, x = inputs.c2_weight(), inputs.c2_x()
    ref, rec = quant_both(w, 8, 4096)
    check_unpack(ref, rec)
    check_gemv(ref, rec, x)


@pytest.mark.parametrize("j", [0, 1])
def test_config3_int4_g128(j):
    w = inputs.c3_weight(j)
    ref, rec = quant_both(w, 4, 128)
    for m in (1, 4, 8):
        check_gemv(ref, rec, inputs.c3_x(j, m))


def _rows_check(rec, w, bits, group, rows, x=None, y=None):
    """Oracle on selected rows only (groups lie inside rows)."""
    n, k = w.shape
    ref = oracle.quantize_pack(w[rows], bits, group)
    pb = k * bits // 8
    payload = host(rec["payload"]).reshape(n, pb)[rows]
    scales = host(rec["scales"]).reshape(n, k // group)[rows]
    assert same_bits(payload.reshape(-1), ref["payload"])
    assert same_bits(scales.reshape(-1), ref["scales"])
    if x is not None:
        yr = oracle.gemv_ref(ref, x)
        B = oracle.error_base(ref, x)
        assert np.all(np.abs(y[:, rows] - yr) <= GEMV_TOL * B)


def test_config4_layers_sampled():
    # layers 0 and 31 of the 7B stack: batched quantize, then the decode
    # GEMVs as one batched call (the launch configuration of the benchmark)
    # and as single calls, and the batched unpack; sampled rows against the
    # oracle.
    rng = np.random.default_rng(4)
    ws, xs = [], []
    for layer in (0, 31):
        for slot, (tag, n, k) in enumerate(inputs.C4_SLOTS):
            ws.append(inputs.c4_weight(layer, slot))
            xs.append(dev(inputs.c4_x(k)))
    recs = qw.quantize_pack_batched([dev(w) for w in ws], 4, 32)
    ys = [host(y) for y in qw.gemv_batched(recs, xs)]
    # the batched unpack of the same matrices (also the benchmark's launch)
    w_hats = [host(o) for o in qw.unpack_batched(recs)]
    for w, rec, x, y, w_hat in zip(ws, recs, xs, ys, w_hats):
        n, k = w.shape
        rows = np.sort(rng.choice(n, size=96, replace=False))
        rows[0], rows[-1] = 0, n - 1
        _rows_check(rec, w, 4, 32, rows, host(x), y)
        y1 = host(qw.gemv(rec, x))
        _rows_check(rec, w, 4, 32, rows, host(x), y1)
        ref_rows = oracle.unpack(oracle.quantize_pack(w[rows], 4, 32)).reshape(len(rows), k)
        assert same_bits(w_hat.reshape(n, k)[rows], ref_rows)


@pytest.mark.parametrize("bits", [4, 8])
def test_matrix_beyond_32bit_indexing(bits):
    """One matrix of 65,537 x 32,768 = 2^31 + 32,768 weights (at int8 also
    more than 2^31 payload bytes), drawn on the GPU from a seeded generator:
    quantize, unpack, GEMV (m = 1) and GEMM (m = 16) through the C ABI,
    checked against the oracle on rows at both ends and in the middle, so
    every element index and byte offset past 2^31 is exercised."""
    n, k, group = 65537, 32768, 128
    print("beyond-2^31 matrix", bits, flush=True)
    gen = torch.Generator(device="cuda").manual_seed(77 + bits)
    w = torch.randn((n, k), dtype=torch.float32, device="cuda", generator=gen) * 0.02
    rec = qw.quantize_pack(w, bits, group)
    rows = np.array([0, 1, n // 2, n - 4, n - 3, n - 2, n - 1])
    w_rows = host(w[torch.from_numpy(rows).cuda()])
    ref = oracle.quantize_pack(w_rows, bits, group)
    pb = k * bits // 8
    assert same_bits(host(rec["payload"].view(n, pb)[torch.from_numpy(rows).cuda()]).reshape(-1),
                     ref["payload"])
    assert same_bits(host(rec["scales"].view(n, k // group)[torch.from_numpy(rows).cuda()])
                     .reshape(-1), ref["scales"])
    # unpack of the whole matrix, sampled rows
    w_hat = qw.unpack(rec)
    assert same_bits(host(w_hat[torch.from_numpy(rows).cuda()]),
                     oracle.unpack(ref).reshape(len(rows), k))
    del w_hat, w
    torch.cuda.empty_cache()
    # GEMV and GEMM outputs of the sampled rows
    x = inputs.activations([77, bits], 1, k)
    y = host(qw.gemv(rec, dev(x)))[:, rows]
    B = oracle.error_base(ref, x)
    assert np.all(np.abs(y - oracle.gemv_ref(ref, x)) <= GEMV_TOL * B)
    xb = inputs.bf16_activations([78, bits], 16, k)
    yg = host(qw.gemm(rec, dev(xb.view(np.int16))))[:, rows]
    Bg = oracle.error_base(ref, oracle.bf16_bits_to_f32(xb))
    assert np.all(np.abs(yg - oracle.gemm_ref(ref, xb)) <= GEMM_TOL * Bg)


@pytest.mark.parametrize("m", [1, 3, 8])
def test_gemv_batched_mixed(m):
    # mixed bit widths, groups, shapes, a generic-path matrix, an empty one
    # and one with k == 0; more than one launch's worth of int4 matrices.
    specs = []
    for i in range(40):
        bits = 4 if i % 3 else 8
        n = [5, 64, 300, 1000][i % 4]
        k = [128, 256, 4096, 96][(i // 4) % 4]
        group = [32, k, 32 * k, 16][i % 4] if bits == 4 else [16, k, 64, 32][i % 4]
        if (n * k) % group:
            group = k
        specs.append((bits, group, n, k))
    specs += [(4, 6, 8, 24), (8, 32, 0, 64), (4, 32, 7, 0)]
    # and more matrices than one launch holds (QW_BATCH_PER_LAUNCH)
    specs += [(4, 32, 1 + i % 9, 64) for i in range(qw.BATCH_PER_LAUNCH + 20)]
    refs, recs, xs, xds = [], [], [], []
    for j, (bits, group, n, k) in enumerate(specs):
        w = inputs.weight(900 + j, n, k, 0.05)
        ref = oracle.quantize_pack(w, bits, group)
        rec = qw.quantize_pack(dev(w), bits, group) if n * k else dict(
            bits=bits, group=group, shape=[n, k],
            payload=torch.empty(0, dtype=torch.uint8, device="cuda"),
            scales=torch.empty(0, dtype=torch.float32, device="cuda"))
        x = inputs.activations(950 + j, m, k)
        refs.append(ref); recs.append(rec); xs.append(x); xds.append(dev(x))
    ys = qw.gemv_batched(recs, xds)
    for ref, x, y in zip(refs, xs, ys):
        yr = oracle.gemv_ref(ref, x)
        B = oracle.error_base(ref, x)
        assert np.all(np.abs(host(y) - yr) <= GEMV_TOL * B)


def test_quantize_pack_batched_mixed():
    # several (bits, group) classes, a generic-path group, an empty matrix and
    # more matrices than one launch holds; every output bit-identical
    nmany = qw.BATCH_PER_LAUNCH + 14
    specs = [(4, 32, 16, 256)] * nmany + [(8, 128, 33, 512), (4, 4096, 4, 4096), (8, 6, 5, 12),
                                          (4, 32, 0, 64), (4, 1024, 2, 2048), (8, 8, 3, 8)]
    ws = [inputs.weight(700 + j, n, k, 0.05) for j, (b, g, n, k) in enumerate(specs)]
    recs = []
    for (bits, group, n, k), w in zip(specs, ws):
        nb, ns = n * k * bits // 8, n * k // group
        recs.append(dict(bits=bits, group=group, shape=[n, k],
                         payload=torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda"),
                         scales=torch.full((ns,), -1.0, dtype=torch.float32, device="cuda")))
    wd = [dev(w) for w in ws]
    arr, cnt = qw.make_quant_descs((r["bits"], r["group"], r["shape"][0], r["shape"][1], w,
                                    r["payload"], r["scales"]) for r, w in zip(recs, wd))
    assert qw.qw_quantize_pack_batched(cnt, arr) == 0
    for (bits, group, n, k), w, rec in zip(specs, ws, recs):
        ref = oracle.quantize_pack(w, bits, group)
        assert same_bits(host(rec["payload"]), ref["payload"])
        assert same_bits(host(rec["scales"]), ref["scales"])
    # the convenience wrapper takes the same path
    recs2 = qw.quantize_pack_batched(wd[:nmany], 4, 32)
    for w, rec in zip(ws[:nmany], recs2):
        ref = oracle.quantize_pack(w, 4, 32)
        assert same_bits(host(rec["payload"]), ref["payload"])


def test_unpack_batched_mixed():
    # both bit widths; groups of a power-of-two and of another number of
    # float4 vectors; a group the vector kernel does not take (6); an empty
    # matrix; an output that is only 4-byte aligned (single-call path); and
    # more matrices than one launch holds.  Every output bit-identical to the
    # oracle's unpack.
    nmany = qw.BATCH_PER_LAUNCH + 9
    specs = [(4, 32, 16, 256)] * nmany + [(8, 128, 33, 512), (4, 4096, 4, 4096), (8, 6, 5, 12),
                                          (4, 32, 0, 64), (4, 1024, 2, 2048), (8, 8, 3, 8),
                                          (4, 12, 4, 24), (8, 20, 5, 40), (4, 64, 7, 64)]
    refs, recs = [], []
    for j, (bits, group, n, k) in enumerate(specs):
        ref = oracle.quantize_pack(inputs.weight(800 + j, n, k, 0.05), bits, group)
        refs.append(ref)
        recs.append(dict(bits=bits, group=group, shape=[n, k], payload=dev(ref["payload"]),
                         scales=dev(ref["scales"])))
    outs = [torch.full((n, k), float("nan"), dtype=torch.float32, device="cuda")
            for (_b, _g, n, k) in specs]
    n_last, k_last = specs[-1][2], specs[-1][3]
    buf = torch.full((n_last * k_last + 1,), float("nan"), dtype=torch.float32, device="cuda")
    outs[-1] = buf[1:].view(n_last, k_last)          # 4-byte aligned only
    qw.unpack_batched(recs, outs)
    for ref, out in zip(refs, outs):
        assert same_bits(host(out), oracle.unpack(ref).reshape(out.shape))


def test_quantize_pack_batched_validation():
    arr, cnt = qw.make_quant_descs([(4, 32, 64, 256, None, None, None)])
    assert qw.qw_quantize_pack_batched(cnt, arr) == -5
    arr, cnt = qw.make_quant_descs([(4, 33, 64, 256, None, None, None)])
    assert qw.qw_quantize_pack_batched(cnt, arr) == -2
    assert qw.qw_quantize_pack_batched(-2, arr) == -7


def test_gemv_batched_validation():
    arr, cnt = qw.make_gemv_descs([(4, 32, 64, 128, None, None, None, None)])
    assert qw.qw_gemv_batched(cnt, arr, 1) == -5
    arr, cnt = qw.make_gemv_descs([(5, 32, 64, 128, None, None, None, None)])
    assert qw.qw_gemv_batched(cnt, arr, 1) == -1
    assert qw.qw_gemv_batched(-1, arr, 1) == -7
    assert qw.qw_gemv_batched(1, arr, 9) == -4


def test_config5_gemm_sampled():
    w = inputs.c5_weight()
    n, k = w.shape
    rec = qw.quantize_pack(dev(w), 4, 128)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(n, size=64, replace=False))
    rows[0], rows[-1] = 0, n - 1
    _rows_check(rec, w, 4, 128, rows)
    xb = inputs.c5_x_bf16()
    y = host(qw.gemm(rec, dev(xb.view(np.int16))))
    ms = np.sort(rng.choice(xb.shape[0], size=48, replace=False))
    ms[0], ms[-1] = 0, xb.shape[0] - 1
    ref = oracle.quantize_pack(w[rows], 4, 128)
    yr = oracle.gemm_ref(ref, xb[ms])
    B = oracle.error_base(ref, oracle.bf16_bits_to_f32(xb[ms]))
    got = y[np.ix_(ms, rows)]
    assert np.all(np.abs(got - yr) <= GEMM_TOL * B)
