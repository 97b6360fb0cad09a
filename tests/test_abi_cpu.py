"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, computes sizes, and rejects invalid arguments before it
touches a GPU.  No compute call is made here."""

import ctypes
import os
import re

import pytest

from int8_int4_dequant_amd import qw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "qw.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qw_[a-z_]+)\s*\(", txt)))


def test_header_lists_the_boundary():
    fns = header_functions()
    for name in ("qw_quantize_pack", "qw_unpack", "qw_gemv", "qw_gemm"):
        assert name in fns
    assert sorted(qw.EXPORTS) == fns


def test_library_exports_every_declared_symbol():
    L = qw.lib()
    raw = ctypes.CDLL(qw.LIB_PATH)
    for name in header_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def test_batch_capacity_matches_header():
    txt = open(os.path.join(ROOT, "include", "qw.h")).read()
    m = re.search(r"#define QW_BATCH_PER_LAUNCH (\d+)", txt)
    assert m and int(m.group(1)) == qw.BATCH_PER_LAUNCH


def test_sizes():
    L = qw.lib()
    assert L.qw_payload_bytes(4, 11008, 4096) == 11008 * 4096 // 2
    assert L.qw_payload_bytes(8, 4096, 4096) == 4096 * 4096
    assert L.qw_payload_bytes(4, 3, 3) == -1
    assert L.qw_payload_bytes(5, 4, 4) == -1
    assert L.qw_num_scales(128, 11008, 4096) == 11008 * 32
    assert L.qw_num_scales(3, 4, 4) == -1
    assert L.qw_num_scales(0, 4, 4) == -1
    # the 7B stack of 224 matrices at int4 group 32
    total_p = total_s = 0
    for n, k in [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]:
        total_p += L.qw_payload_bytes(4, n, k)
        total_s += 4 * L.qw_num_scales(32, n, k)
    assert 32 * total_p == 3_238_002_688
    assert 32 * total_s == 809_500_672


def test_status_strings():
    L = qw.lib()
    for st in range(-9, 1):
        assert L.qw_status_string(st)
    assert L.qw_status_string(0) == b"ok"


def _q(bits, group, n, k, w=None, p=None, s=None):
    return qw.lib().qw_quantize_pack(bits, group, n, k, w, p, s, None)


def test_validation_before_any_launch():
    L = qw.lib()
    assert _q(3, 32, 4, 32) == -1
    assert _q(8, 0, 4, 32) == -2
    assert _q(8, 33, 4, 32) == -2
    assert _q(4, 1, 3, 3) == -3
    assert _q(8, 32, -1, 32) == -3
    assert _q(8, 32, 4, 32) == -5          # null pointers with real work
    assert _q(8, 32, 0, 32) == 0           # empty: nothing to do
    assert _q(8, 32, 4, 0) == 0
    assert L.qw_unpack(8, 32, 4, 32, None, None, None, None) == -5
    assert L.qw_gemv(8, 32, 4, 32, None, None, 9, None, None, None) == -4
    assert L.qw_gemv(8, 32, 4, 32, None, None, -1, None, None, None) == -4
    assert L.qw_gemv(8, 32, 4, 32, None, None, 0, None, None, None) == 0
    assert L.qw_gemv(8, 32, 4, 32, None, None, 1, None, None, None) == -5
    assert L.qw_gemm(8, 32, 4, 32, None, None, -1, None, None, None) == -4
    assert L.qw_gemm(4, 32, 4, 32, None, None, 0, None, None, None) == 0
    assert L.qw_gemm(4, 32, 4, 32, None, None, 5, None, None, None) == -5


def test_chain_validation_before_any_launch():
    L = qw.lib()
    arr = (qw.QwGemvDesc * 2)()
    for i in range(2):
        arr[i] = qw.QwGemvDesc(None, None, None, None, 64, 64, 32, 4, 0)
    st = (ctypes.c_int32 * 2)(0, 1)
    assert L.qw_gemv_chain(2, arr, None, 1, None) == -7       # no stage list
    assert L.qw_gemv_chain(2, arr, (ctypes.c_int32 * 2)(1, 0), 1, None) == -7
    assert L.qw_gemv_chain(2, arr, st, 9, None) == -4
    assert L.qw_gemv_chain(2, arr, st, 1, None) == -5         # null pointers
    assert L.qw_gemv_chain(-1, arr, st, 1, None) == -7
    assert L.qw_gemv_chain(0, None, None, 1, None) == 0


def test_unpack_batched_validation():
    L = qw.lib()
    fake = 1 << 20  # never dereferenced: every call below fails validation or is empty
    arr, cnt = qw.make_unpack_descs([(4, 32, 64, 256, None, fake, fake)])
    assert L.qw_unpack_batched(cnt, arr, None) == -5
    arr, cnt = qw.make_unpack_descs([(4, 32, 64, 256, fake, fake, fake),
                                     (4, 33, 64, 256, fake, fake, fake)])
    assert L.qw_unpack_batched(cnt, arr, None) == -2        # nothing enqueued for the first
    arr, cnt = qw.make_unpack_descs([(3, 32, 64, 256, fake, fake, fake)])
    assert L.qw_unpack_batched(cnt, arr, None) == -1
    arr[0].bits, arr[0].reserved = 4, 1
    assert L.qw_unpack_batched(cnt, arr, None) == -7
    assert L.qw_unpack_batched(-1, arr, None) == -7
    assert L.qw_unpack_batched(0, None, None) == 0
    arr, cnt = qw.make_unpack_descs([(4, 32, 0, 256, None, None, None)])
    assert L.qw_unpack_batched(cnt, arr, None) == 0          # empty: nothing to do


def test_matmul_work_size_and_validation():
    L = qw.lib()
    t = qw.MATMUL_GEMV_MAX_M
    assert L.qw_matmul_work_bytes(t, 4096) == 0          # the GEMV side needs none
    assert L.qw_matmul_work_bytes(t + 1, 4096) >= (t + 1) * 4096 * 2
    assert L.qw_matmul_work_bytes(300, 1000) % 256 == 0
    assert L.qw_matmul_work_bytes(-1, 8) == -1
    fake = 1 << 20  # never dereferenced: every call below fails validation or is empty
    need = L.qw_matmul_work_bytes(9, 256)
    assert L.qw_matmul(4, 32, 64, 256, fake, fake, 9, fake, fake, None, need, None) == -8
    assert L.qw_matmul(4, 32, 64, 256, fake, fake, 9, fake, fake, fake, need - 1, None) == -8
    assert L.qw_matmul(3, 32, 64, 256, fake, fake, 9, fake, fake, fake, need, None) == -1
    assert L.qw_matmul(4, 48, 64, 100, fake, fake, 9, fake, fake, fake, need, None) == -2
    assert L.qw_matmul(4, 32, 64, 256, fake, fake, -1, fake, fake, fake, need, None) == -4
    assert L.qw_matmul(4, 32, 64, 256, None, fake, 9, fake, fake, fake, need, None) == -5
    assert L.qw_matmul(4, 32, 64, 256, fake, fake, 9, fake, None, fake, need, None) == -5
    assert L.qw_matmul(4, 32, 0, 256, None, None, 9, None, None, None, 0, None) == 0
    assert L.qw_matmul(4, 32, 64, 256, fake, fake, 0, fake, fake, None, 0, None) == 0
    # the GEMV side keeps qw_gemv's own limits and needs no work buffer
    assert L.qw_matmul(4, 32, 64, 256, None, fake, 3, fake, fake, None, 0, None) == -5


def test_gptq_work_sizes():
    L = qw.lib()
    assert L.qw_gptq_hessian_work_bytes(-1, 5) == -1
    assert L.qw_gptq_hessian_work_bytes(512, 8192) > 0
    # the partial sums cover whole k x k matrices, one per token chunk
    assert L.qw_gptq_hessian_work_bytes(512, 8192) % (512 * 512 * 8) == 0
    # one partial sum per token chunk: 14 chunks for 36 64-wide tiles at k = 512
    # (504 of the 512 work-group slots); at k = 1368, 66 128-wide tiles take
    # 7 full chunks and a short eighth (528 work-groups)
    assert L.qw_gptq_hessian_work_bytes(512, 8192) == 14 * 512 * 512 * 8
    assert L.qw_gptq_hessian_work_bytes(1368, 8192) == 8 * 1368 * 1368 * 8
    # few tokens: chunks of at least 256 tokens
    assert L.qw_gptq_hessian_work_bytes(200, 1000) == 3 * 200 * 200 * 8
    kp = 1408  # 1368 rounded up to the 64-wide blocks of the factorization
    assert L.qw_gptq_factor_work_bytes(1368) >= 2 * kp * kp * 8
    assert L.qw_gptq_factor_work_bytes(-3) == -1
    assert L.qw_gptq_quantize_work_bytes(512, 1368) >= (512 * 1368 + 1368 * 1368) * 8
    assert L.qw_gptq_quantize_work_bytes(-1, 4) == -1


def test_gptq_validation_before_any_launch():
    L = qw.lib()
    fake = 1 << 20  # never dereferenced: every call below fails validation
    # H: shapes, pointers, work buffer
    assert L.qw_gptq_hessian(-1, 4, fake, fake, fake, 1 << 30, None) == -3
    assert L.qw_gptq_hessian(8, 0, None, None, None, 0, None) == 0
    assert L.qw_gptq_hessian(8, 16, None, fake, fake, 1 << 30, None) == -5
    need = L.qw_gptq_hessian_work_bytes(8, 16)
    assert L.qw_gptq_hessian(8, 16, fake, fake, fake, need - 1, None) == -8
    assert L.qw_gptq_hessian(8, 16, fake, fake, None, need, None) == -8
    # factor: damping must be finite and >= 0
    assert L.qw_gptq_factor(8, fake, -0.01, fake, None, fake, 1 << 30, None) == -9
    assert L.qw_gptq_factor(8, fake, float("nan"), fake, None, fake, 1 << 30, None) == -9
    assert L.qw_gptq_factor(8, fake, float("inf"), fake, None, fake, 1 << 30, None) == -9
    assert L.qw_gptq_factor(0, None, 0.01, None, None, None, 0, None) == 0
    assert L.qw_gptq_factor(8, None, 0.01, fake, None, fake, 1 << 30, None) == -5
    assert L.qw_gptq_factor(8, fake, 0.01, fake, None, fake, 16, None) == -8
    # codes: a group lies inside one output channel, even for int4
    big = 1 << 30
    assert L.qw_gptq_quantize_pack(4, 64, 4, 96, fake, fake, fake, fake, fake, big, None) == -2
    assert L.qw_gptq_quantize_pack(4, 3, 4, 96, fake, fake, fake, fake, fake, big, None) == -2
    assert L.qw_gptq_quantize_pack(5, 32, 4, 96, fake, fake, fake, fake, fake, big, None) == -1
    assert L.qw_gptq_quantize_pack(8, 32, 0, 96, None, None, None, None, None, 0, None) == 0
    assert L.qw_gptq_quantize_pack(8, 32, 4, 96, None, fake, fake, fake, fake, big, None) == -5
    assert L.qw_gptq_quantize_pack(8, 32, 4, 96, fake, fake, fake, fake, fake, 8, None) == -8


@pytest.mark.parametrize("bits,group,n,k,al,expect", [
    (4, 32, 64, 256, 16, 1), (8, 128, 64, 256, 16, 1), (8, 512, 4, 512, 16, 1),
    (8, 4096, 8, 4096, 16, 2), (4, 11008, 4, 11008, 16, 2), (4, 1024, 4, 1024, 16, 1),
    (4, 2048, 4, 2048, 16, 2),
    (4, 3, 4, 6, 16, 3), (8, 1, 4, 8, 16, 3), (4, 4096 * 16, 16, 4096, 16, 3),
    (4, 32, 64, 256, 4, 3),
])
def test_quantize_dispatch(bits, group, n, k, al, expect):
    base = 1 << 20
    assert qw.lib().qw_debug_path(0, bits, group, n, k, base + (al % 16), base) == expect


@pytest.mark.parametrize("op,bits,group,n,k,expect", [
    (2, 4, 128, 4096, 11008, 1), (2, 8, 4096, 4096, 4096, 1), (2, 4, 32, 11008, 4096, 1),
    (2, 4, 16, 64, 256, 1), (2, 4, 8, 64, 256, 1), (2, 4, 4, 64, 256, 3), (2, 4, 32, 8, 48, 3), (2, 4, 4096 * 8, 8, 4096, 1),
    (2, 4, 3, 8, 48, 3),
    (3, 4, 128, 28672, 8192, 1), (3, 8, 32, 64, 256, 1), (3, 4, 16, 64, 256, 3),
    (3, 4, 32, 64, 96, 3),
    # 3..8 rows of x: the matrix-core GEMV for rows of whole 128-code steps
    # with groups of whole steps, of 32 or 64 codes or of whole rows, else the
    # fp32 kernels
    (4, 4, 128, 11008, 4096, 4), (4, 4, 128, 4096, 11008, 4), (4, 8, 4096, 4096, 4096, 4),
    (4, 4, 4096 * 8, 8, 4096, 4), (4, 8, 256, 2, 128, 4), (4, 4, 64, 64, 256, 4), (4, 4, 96, 64, 384, 1),
    (4, 4, 32, 11008, 4096, 4), (4, 8, 32, 300, 1024, 4), (4, 4, 128, 64, 384 + 8, 3),
    (4, 4, 8, 64, 96, 1),
    (4, 4, 3, 8, 48, 3), (4, 4, 128, 64, 0, 3),
    # qw_matmul at 5..8 rows: the GEMV (1) for matrices of up to 8192 rows the
    # matrix-core GEMV takes, else the GEMM (2)
    (5, 4, 128, 4096, 11008, 1), (5, 8, 4096, 8192, 4096, 1), (5, 4, 128, 8193, 4096, 2),
    (5, 4, 128, 11008, 4096, 2), (5, 4, 16, 64, 256, 2), (5, 4, 32, 64, 96, 2),
])
def test_product_dispatch(op, bits, group, n, k, expect):
    base = 1 << 20
    assert qw.lib().qw_debug_path(op, bits, group, n, k, base, base) == expect


def test_binding_checks_buffers_before_any_call():
    """The C ABI takes bare pointers, so the Python binding checks every
    buffer a kernel would touch (dtype, contiguity, element count, device)
    and every record's payload and scales against its bits, group and shape
    before calling it; a mismatch raises ValueError and reaches no kernel."""
    import torch

    n, k, m = 8, 64, 2
    good = dict(bits=4, group=32, shape=[n, k],
                payload=torch.zeros(n * k // 2, dtype=torch.uint8),
                scales=torch.ones(n * k // 32, dtype=torch.float32))
    x = torch.zeros((m, k), dtype=torch.float32)
    cases = [
        (lambda: qw.gemv(dict(good, payload=good["payload"][:-1]), x), "payload"),
        (lambda: qw.gemv(dict(good, scales=good["scales"][:-1]), x), "scales"),
        (lambda: qw.gemv(dict(good, scales=good["scales"].double()), x), "scales"),
        (lambda: qw.gemv(dict(good, group=48), x), "group"),
        (lambda: qw.gemv(good, x, out=torch.empty((m, n - 1))), "out"),
        (lambda: qw.gemv(good, x, out=torch.empty((m, n), dtype=torch.float64)), "out"),
        (lambda: qw.gemv(good, x, out=torch.empty((n, m)).t()), "out"),
        (lambda: qw.gemv(good, x[:, :k - 1]), "x"),
        (lambda: qw.unpack(good, out=torch.empty(n * k - 1)), "out"),
        (lambda: qw.unpack_batched([good], [torch.empty(n * k + 1)]), "output"),
        (lambda: qw.gemv_batched([good], [x], [torch.empty((m, n + 1))]), "output"),
        (lambda: qw.gemv_chain([good], [x], [torch.empty((m, n - 1))], [0]), "y"),
        (lambda: qw.gemm(good, torch.zeros((m, k), dtype=torch.int16),
                         out=torch.empty((m + 1, n))), "out"),
        (lambda: qw.gemm(good, torch.zeros((m, k), dtype=torch.float32)), "x"),
        (lambda: qw.matmul(good, torch.zeros((9, k)), out=torch.empty((9, n - 1))), "out"),
        # right sizes everywhere, but host tensors: refused as well
        (lambda: qw.gemv(good, x), "device"),
    ]
    for fn, word in cases:
        with pytest.raises(ValueError, match=word):
            fn()


def test_noalloc_matmul_size_limit_before_any_launch():
    """qw_matmul_noalloc refuses an x whose bf16 copy exceeds its static
    scratch (QW_ESCRATCH) during validation, before it looks up the scratch
    or launches anything (so this runs without a GPU)."""
    L = qw.lib()
    cap = qw.MATMUL_NOALLOC_MAX_BYTES
    k = 4096
    m_ok, m_big = cap // (2 * k), cap // (2 * k) + 1
    assert L.qw_matmul_work_bytes(m_ok, k) <= cap < L.qw_matmul_work_bytes(m_big, k)
    assert L.qw_matmul_noalloc(4, 128, 16, k, None, None, m_big, None, None, None) == -10
    assert L.qw_matmul_noalloc(4, 128, 16, k, None, None, m_ok, None, None, None) == -5
    assert L.qw_matmul_noalloc(4, 100, 16, k, None, None, m_ok, None, None, None) == -2
    assert L.qw_matmul_noalloc(4, 128, 16, k, None, None, -1, None, None, None) == -4
    assert b"scratch" in L.qw_status_string(-10)
    txt = open(os.path.join(ROOT, "include", "qw.h")).read()
    assert re.search(r"#define QW_MATMUL_NOALLOC_MAX_BYTES \(32ll << 20\)", txt)
    assert cap == 32 << 20
