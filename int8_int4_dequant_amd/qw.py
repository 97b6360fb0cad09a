"""Thin Python binding of libqw (include/qw.h).

Argument marshalling only: every step of quantization, unpacking and the
products runs in the HIP kernels of libqw.so.  PyTorch provides device
memory and the current HIP stream.  If the library has not been built this
module raises; there is no CPU fallback.

Low-level functions carry the C names (``qw_quantize_pack``, ``qw_unpack``,
``qw_gemv``, ``qw_gemm``) and take preallocated tensors; the convenience
layer (``quantize_pack``, ``unpack``, ``gemv``, ``gemm``) allocates outputs
and returns a record shaped like the pages' ``pack`` result:
``{bits, group, shape, payload, scales}``.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqw.so")

#: matrices per kernel launch in the batched calls (QW_BATCH_PER_LAUNCH in qw.h)
BATCH_PER_LAUNCH = 256

QW_OK = 0
STATUS_NAMES = {0: "QW_OK", -1: "QW_EBITS", -2: "QW_EGROUP", -3: "QW_ESHAPE", -4: "QW_EM",
                -5: "QW_ENULL", -6: "QW_EHIP", -7: "QW_ECOUNT", -8: "QW_EWORK", -9: "QW_EARG",
                -10: "QW_ESCRATCH"}

#: symbols declared in include/qw.h
EXPORTS = ["qw_payload_bytes", "qw_num_scales", "qw_status_string", "qw_last_error",
           "qw_quantize_pack", "qw_quantize_pack_batched", "qw_unpack", "qw_unpack_batched",
           "qw_gemv",
           "qw_gemv_batched", "qw_gemv_chain", "qw_gemm", "qw_matmul_work_bytes", "qw_matmul",
           "qw_matmul_noalloc",
           "qw_debug_path",
           "qw_gptq_hessian_work_bytes", "qw_gptq_hessian", "qw_gptq_factor_work_bytes",
           "qw_gptq_factor", "qw_gptq_quantize_work_bytes", "qw_gptq_quantize_pack"]


# Rows up to which qw_matmul runs the codes GEMV (QW_MATMUL_GEMV_MAX_M in qw.h).
MATMUL_GEMV_MAX_M = 4
# Bytes of the static scratch of qw_matmul_noalloc (QW_MATMUL_NOALLOC_MAX_BYTES).
MATMUL_NOALLOC_MAX_BYTES = 32 << 20


class QwQuantDesc(ctypes.Structure):
    """Mirror of `qw_quant_desc` in include/qw.h."""
    _fields_ = [("w", ctypes.c_void_p), ("payload", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("group", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class QwUnpackDesc(ctypes.Structure):
    """Mirror of `qw_unpack_desc` in include/qw.h."""
    _fields_ = [("payload", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("w_out", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("group", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class QwGemvDesc(ctypes.Structure):
    """Mirror of `qw_gemv_desc` in include/qw.h."""
    _fields_ = [("payload", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("group", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("reserved", ctypes.c_int32)]

_lib = None


class QwError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = f"{what}: {STATUS_NAMES.get(status, status)} ({_text(status)})"
        if status == -6:
            msg += f": {_lib.qw_last_error().decode()}"
        super().__init__(msg)


def _text(status):
    return _lib.qw_status_string(status).decode() if _lib else str(status)


def lib():
    """Load libqw.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    L.qw_payload_bytes.argtypes = [i32, i64, i64]
    L.qw_payload_bytes.restype = i64
    L.qw_num_scales.argtypes = [i64, i64, i64]
    L.qw_num_scales.restype = i64
    L.qw_status_string.argtypes = [i32]
    L.qw_status_string.restype = ctypes.c_char_p
    L.qw_last_error.argtypes = []
    L.qw_last_error.restype = ctypes.c_char_p
    L.qw_quantize_pack.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp]
    L.qw_quantize_pack.restype = i32
    L.qw_quantize_pack_batched.argtypes = [i32, ctypes.POINTER(QwQuantDesc), vp]
    L.qw_quantize_pack_batched.restype = i32
    L.qw_unpack.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp]
    L.qw_unpack.restype = i32
    L.qw_unpack_batched.argtypes = [i32, ctypes.POINTER(QwUnpackDesc), vp]
    L.qw_unpack_batched.restype = i32
    L.qw_gemv.argtypes = [i32, i64, i64, i64, vp, vp, i64, vp, vp, vp]
    L.qw_gemv.restype = i32
    L.qw_gemv_batched.argtypes = [i32, ctypes.POINTER(QwGemvDesc), i64, vp]
    L.qw_gemv_batched.restype = i32
    L.qw_gemv_chain.argtypes = [i32, ctypes.POINTER(QwGemvDesc), ctypes.POINTER(ctypes.c_int32),
                                i64, vp]
    L.qw_gemv_chain.restype = i32
    L.qw_gemm.argtypes = [i32, i64, i64, i64, vp, vp, i64, vp, vp, vp]
    L.qw_gemm.restype = i32
    L.qw_matmul_work_bytes.argtypes = [i64, i64]
    L.qw_matmul_work_bytes.restype = i64
    L.qw_matmul.argtypes = [i32, i64, i64, i64, vp, vp, i64, vp, vp, vp, i64, vp]
    L.qw_matmul.restype = i32
    L.qw_matmul_noalloc.argtypes = [i32, i64, i64, i64, vp, vp, i64, vp, vp, vp]
    L.qw_matmul_noalloc.restype = i32
    L.qw_debug_path.argtypes = [i32, i32, i64, i64, i64, vp, vp]
    L.qw_debug_path.restype = i32
    L.qw_gptq_hessian_work_bytes.argtypes = [i64, i64]
    L.qw_gptq_hessian_work_bytes.restype = i64
    L.qw_gptq_hessian.argtypes = [i64, i64, vp, vp, vp, i64, vp]
    L.qw_gptq_hessian.restype = i32
    L.qw_gptq_factor_work_bytes.argtypes = [i64]
    L.qw_gptq_factor_work_bytes.restype = i64
    L.qw_gptq_factor.argtypes = [i64, vp, ctypes.c_double, vp, vp, vp, i64, vp]
    L.qw_gptq_factor.restype = i32
    L.qw_gptq_quantize_work_bytes.argtypes = [i64, i64]
    L.qw_gptq_quantize_work_bytes.restype = i64
    L.qw_gptq_quantize_pack.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.qw_gptq_quantize_pack.restype = i32
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return t  # raw integer address
    if t.numel() and not t.is_cuda:
        raise ValueError("libqw takes device tensors")
    return t.data_ptr() if t.numel() else None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(status, what):
    if status != QW_OK:
        raise QwError(status, what)


# ------------------------------------------------------------ C-name layer


def qw_payload_bytes(bits, n, k):
    return lib().qw_payload_bytes(bits, n, k)


def qw_num_scales(group, n, k):
    return lib().qw_num_scales(group, n, k)


def qw_quantize_pack(bits, group, n, k, w, payload, scales, stream=None):
    return lib().qw_quantize_pack(bits, group, n, k, _ptr(w), _ptr(payload), _ptr(scales),
                                  _stream(stream))


def make_quant_descs(items):
    """items: iterable of (bits, group, n, k, w, payload, scales); returns a
    ctypes array for qw_quantize_pack_batched and its length."""
    items = list(items)
    arr = (QwQuantDesc * max(1, len(items)))()
    for i, (bits, group, n, k, w, payload, scales) in enumerate(items):
        arr[i] = QwQuantDesc(_ptr(w), _ptr(payload), _ptr(scales), n, k, group, bits, 0)
    return arr, len(items)


def qw_quantize_pack_batched(count, descs, stream=None):
    return lib().qw_quantize_pack_batched(count, descs, _stream(stream))


def qw_unpack(bits, group, n, k, payload, scales, w_out, stream=None):
    return lib().qw_unpack(bits, group, n, k, _ptr(payload), _ptr(scales), _ptr(w_out),
                           _stream(stream))


def make_unpack_descs(items):
    """items: iterable of (bits, group, n, k, payload, scales, w_out); returns
    a ctypes array for qw_unpack_batched and its length."""
    items = list(items)
    arr = (QwUnpackDesc * max(1, len(items)))()
    for i, (bits, group, n, k, payload, scales, w_out) in enumerate(items):
        arr[i] = QwUnpackDesc(_ptr(payload), _ptr(scales), _ptr(w_out), n, k, group, bits, 0)
    return arr, len(items)


def qw_unpack_batched(count, descs, stream=None):
    return lib().qw_unpack_batched(count, descs, _stream(stream))


def qw_gemv(bits, group, n, k, payload, scales, m, x, y, stream=None):
    return lib().qw_gemv(bits, group, n, k, _ptr(payload), _ptr(scales), m, _ptr(x), _ptr(y),
                         _stream(stream))


def make_gemv_descs(items):
    """items: iterable of (bits, group, n, k, payload, scales, x, y) with
    device tensors (or raw addresses); returns a ctypes array for
    qw_gemv_batched."""
    items = list(items)
    arr = (QwGemvDesc * max(1, len(items)))()
    for i, (bits, group, n, k, payload, scales, x, y) in enumerate(items):
        arr[i] = QwGemvDesc(_ptr(payload), _ptr(scales), _ptr(x), _ptr(y), n, k, group, bits, 0)
    return arr, len(items)


def qw_gemv_batched(count, descs, m, stream=None):
    return lib().qw_gemv_batched(count, descs, m, _stream(stream))


def qw_gemv_chain(count, descs, stages, m, stream=None):
    """``stages``: a ctypes int32 array (or a list) of ``count`` stage numbers."""
    if not isinstance(stages, ctypes.Array):
        stages = (ctypes.c_int32 * max(1, len(stages)))(*stages)
    return lib().qw_gemv_chain(count, descs, stages, m, _stream(stream))


def qw_gemm(bits, group, n, k, payload, scales, m, x_bf16, y, stream=None):
    return lib().qw_gemm(bits, group, n, k, _ptr(payload), _ptr(scales), m, _ptr(x_bf16),
                         _ptr(y), _stream(stream))


def qw_matmul_work_bytes(m, k):
    return lib().qw_matmul_work_bytes(m, k)


def qw_matmul(bits, group, n, k, payload, scales, m, x, y, work, work_bytes, stream=None):
    return lib().qw_matmul(bits, group, n, k, _ptr(payload), _ptr(scales), m, _ptr(x), _ptr(y),
                           _ptr(work), work_bytes, _stream(stream))


def qw_matmul_noalloc(bits, group, n, k, payload, scales, m, x, y, stream=None):
    return lib().qw_matmul_noalloc(bits, group, n, k, _ptr(payload), _ptr(scales), m, _ptr(x),
                                   _ptr(y), _stream(stream))


def qw_debug_path(op, bits, group, n, k, a=None, b=None):
    return lib().qw_debug_path(op, bits, group, n, k, _ptr(a), _ptr(b))


def qw_gptq_hessian_work_bytes(k, t):
    return lib().qw_gptq_hessian_work_bytes(k, t)


def qw_gptq_hessian(k, t, x, h, work, work_bytes, stream=None):
    return lib().qw_gptq_hessian(k, t, _ptr(x), _ptr(h), _ptr(work), work_bytes,
                                 _stream(stream))


def qw_gptq_factor_work_bytes(k):
    return lib().qw_gptq_factor_work_bytes(k)


def qw_gptq_factor(k, h, damp, u, info, work, work_bytes, stream=None):
    return lib().qw_gptq_factor(k, _ptr(h), damp, _ptr(u), _ptr(info), _ptr(work), work_bytes,
                                _stream(stream))


def qw_gptq_quantize_work_bytes(n, k):
    return lib().qw_gptq_quantize_work_bytes(n, k)


def qw_gptq_quantize_pack(bits, group, n, k, w, u, payload, scales, work, work_bytes,
                          stream=None):
    return lib().qw_gptq_quantize_pack(bits, group, n, k, _ptr(w), _ptr(u), _ptr(payload),
                                       _ptr(scales), _ptr(work), work_bytes, _stream(stream))


# -------------------------------------------------------- convenience layer


def _nk(shape):
    if len(shape) != 2:
        raise ValueError("weights are 2-D [n][k]")
    return int(shape[0]), int(shape[1])


def _check_tensor(t, dtype, numel, what, shape=None):
    """A tensor the kernels read or write: of `dtype`, contiguous, holding
    exactly `numel` elements (of `shape` when given).  The C ABI takes bare
    pointers and cannot see sizes, so a buffer that is too small would be read
    or written past its end on the device.  (``_on_device`` checks where the
    tensors live once all sizes have been checked.)"""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what} must be a torch tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{what} holds {t.numel()} elements, expected {numel}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _on_device(*ts):
    """Every non-empty tensor the call passes must be a device tensor."""
    for t in ts:
        if isinstance(t, dict):
            _on_device(t["payload"], t["scales"])
        elif isinstance(t, torch.Tensor) and t.numel() and not t.is_cuda:
            raise ValueError("libqw takes device tensors; a host tensor was passed")


def _check_rec(rec, what="record"):
    """(n, k) of a record whose payload and scales match its bits, group and
    shape (qw_payload_bytes / qw_num_scales)."""
    n, k = _nk(rec["shape"])
    bits, group = int(rec["bits"]), int(rec["group"])
    nb = lib().qw_payload_bytes(bits, n, k)
    ns = lib().qw_num_scales(group, n, k)
    if nb < 0 or ns < 0:
        raise ValueError(f"{what}: invalid bits {bits}, group {group} or shape {[n, k]}")
    _check_tensor(rec["payload"], torch.uint8, nb, f"{what} payload")
    _check_tensor(rec["scales"], torch.float32, ns, f"{what} scales")
    return n, k


def quantize_pack(w, bits, group, stream=None):
    """Quantize a contiguous fp32 device tensor [n][k]; returns a record
    ``{bits, group, shape, payload (uint8), scales (float32)}``."""
    if w.dtype != torch.float32 or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 tensor")
    n, k = _nk(w.shape)
    nb = lib().qw_payload_bytes(bits, n, k)
    ns = lib().qw_num_scales(group, n, k)
    if nb < 0 or ns < 0:
        _check(QW_EBITS if bits not in (4, 8) else -2 if ns < 0 else -3, "quantize_pack")
    payload = torch.empty(nb, dtype=torch.uint8, device=w.device)
    scales = torch.empty(ns, dtype=torch.float32, device=w.device)
    _check(qw_quantize_pack(bits, group, n, k, w, payload, scales, stream), "qw_quantize_pack")
    return dict(bits=bits, group=group, shape=[n, k], payload=payload, scales=scales)


def quantize_pack_batched(ws, bits, group, stream=None):
    """Quantize a list of contiguous fp32 [n][k] device tensors (same bits
    and group) in a few launches; returns their records."""
    recs = []
    for w in ws:
        if w.dtype != torch.float32 or not w.is_contiguous():
            raise ValueError("each w must be a contiguous float32 tensor")
        n, k = _nk(w.shape)
        nb, ns = lib().qw_payload_bytes(bits, n, k), lib().qw_num_scales(group, n, k)
        if nb < 0 or ns < 0:
            _check(-1 if bits not in (4, 8) else -2 if ns < 0 else -3, "quantize_pack_batched")
        recs.append(dict(bits=bits, group=group, shape=[n, k],
                         payload=torch.empty(nb, dtype=torch.uint8, device=w.device),
                         scales=torch.empty(ns, dtype=torch.float32, device=w.device)))
    arr, cnt = make_quant_descs((bits, group, r["shape"][0], r["shape"][1], w, r["payload"],
                                 r["scales"]) for w, r in zip(ws, recs))
    _check(qw_quantize_pack_batched(cnt, arr, stream), "qw_quantize_pack_batched")
    return recs


def unpack_batched(recs, outs=None, stream=None):
    """Unpack a list of records in a few launches; returns fp32 tensors of
    their shapes (or fills ``outs``)."""
    if outs is None:
        outs = [torch.empty(tuple(int(d) for d in r["shape"]), dtype=torch.float32,
                            device=r["payload"].device) for r in recs]
    if len(outs) != len(recs):
        raise ValueError("one output per record")
    items = []
    for r, o in zip(recs, outs):
        n, k = _check_rec(r)
        _check_tensor(o, torch.float32, n * k, "output")
        items.append((r["bits"], r["group"], n, k, r["payload"], r["scales"], o))
    _on_device(*recs, *outs)
    arr, cnt = make_unpack_descs(items)
    _check(qw_unpack_batched(cnt, arr, stream), "qw_unpack_batched")
    return outs


def unpack(rec, out=None, stream=None):
    n, k = _check_rec(rec)
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=rec["payload"].device)
    _check_tensor(out, torch.float32, n * k, "out")
    _on_device(rec, out)
    _check(qw_unpack(rec["bits"], rec["group"], n, k, rec["payload"], rec["scales"], out,
                     stream), "qw_unpack")
    return out


def gemv(rec, x, out=None, stream=None):
    """fp32 x [m][k] (m <= 8) times the quantized weight; returns y [m][n]."""
    n, k = _check_rec(rec)
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be a contiguous float32 [m][k] tensor")
    m = x.shape[0]
    _check_tensor(x, torch.float32, m * k, "x")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check_tensor(out, torch.float32, m * n, "out", (m, n))
    _on_device(rec, x, out)
    _check(qw_gemv(rec["bits"], rec["group"], n, k, rec["payload"], rec["scales"], m, x, out,
                   stream), "qw_gemv")
    return out


def gemv_batched(recs, xs, outs=None, stream=None):
    """Independent GEMVs (common m) in a few launches; returns the list of y."""
    if len(xs) != len(recs) or (outs is not None and len(outs) != len(recs)):
        raise ValueError("one x (and one output) per record")
    m = xs[0].shape[0]
    if outs is None:
        outs = [torch.empty((m, r["shape"][0]), dtype=torch.float32, device=x.device)
                for r, x in zip(recs, xs)]
    for r, x, y in zip(recs, xs, outs):
        n, k = _check_rec(r)
        _check_tensor(x, torch.float32, m * k, "x", (m, k))
        _check_tensor(y, torch.float32, m * n, "output", (m, n))
    _on_device(*recs, *xs, *outs)
    arr, cnt = make_gemv_descs((r["bits"], r["group"], r["shape"][0], r["shape"][1], r["payload"],
                                r["scales"], x, y) for r, x, y in zip(recs, xs, outs))
    _check(qw_gemv_batched(cnt, arr, m, stream), "qw_gemv_batched")
    return outs


def gemv_chain(recs, xs, ys, stages, stream=None):
    """A chained decode pass: product i computes ys[i] = xs[i] . W_i^T in
    stage stages[i]; an x may be the y of an earlier stage.  All tensors are
    preallocated, contiguous fp32 [m][k] / [m][n] with a common m."""
    if not len(recs) == len(xs) == len(ys) == len(stages):
        raise ValueError("one x, y and stage per record")
    m = xs[0].shape[0]
    for r, x, y in zip(recs, xs, ys):
        n, k = _check_rec(r)
        _check_tensor(x, torch.float32, m * k, "x", (m, k))
        _check_tensor(y, torch.float32, m * n, "y", (m, n))
    _on_device(*recs, *xs, *ys)
    arr, cnt = make_gemv_descs((r["bits"], r["group"], r["shape"][0], r["shape"][1], r["payload"],
                                r["scales"], x, y) for r, x, y in zip(recs, xs, ys))
    _check(qw_gemv_chain(cnt, arr, list(stages), m, stream), "qw_gemv_chain")
    return ys


def gemm(rec, x_bf16, out=None, stream=None):
    """bf16 x [m][k] (torch.bfloat16, or int16/uint16 bit patterns) times the
    quantized weight on the matrix cores; returns fp32 y [m][n]."""
    n, k = _check_rec(rec)
    if not isinstance(x_bf16, torch.Tensor) or x_bf16.dim() != 2 or x_bf16.shape[1] != k:
        raise ValueError("x must be a contiguous [m][k] tensor")
    m = x_bf16.shape[0]
    _check_tensor(x_bf16, (torch.bfloat16, torch.int16, torch.uint16), m * k, "x (bf16)")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x_bf16.device)
    _check_tensor(out, torch.float32, m * n, "out", (m, n))
    _on_device(rec, x_bf16, out)
    _check(qw_gemm(rec["bits"], rec["group"], n, k, rec["payload"], rec["scales"], m, x_bf16,
                   out, stream), "qw_gemm")
    return out


def matmul(rec, x, out=None, work=None, stream=None):
    """QuantizedMatmul: fp32 x [m][k] (any m) times the quantized weight;
    returns fp32 y [m][n].  Up to QW_MATMUL_GEMV_MAX_M rows (and up to 8 for
    matrices of at most 8192 rows the matrix-core GEMV takes) this is the
    codes GEMV; beyond, x is rounded to bf16 into ``work`` (allocated here
    when not given) and the matrix-core GEMM runs."""
    n, k = _check_rec(rec)
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be a contiguous float32 [m][k] tensor")
    m = x.shape[0]
    _check_tensor(x, torch.float32, m * k, "x")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check_tensor(out, torch.float32, m * n, "out", (m, n))
    nb = lib().qw_matmul_work_bytes(m, k)
    if work is None:
        work = _work(nb, x.device) if nb > 0 else None
    if work is not None and (not isinstance(work, torch.Tensor) or not work.is_contiguous()):
        raise ValueError("work must be a contiguous tensor")
    _on_device(rec, x, out, work)
    wb = work.numel() * work.element_size() if work is not None else 0
    _check(qw_matmul(rec["bits"], rec["group"], n, k, rec["payload"], rec["scales"], m, x, out,
                     work, wb, stream), "qw_matmul")
    return out


# ------------------------------------------------------------------ GPTQ


def _work(nbytes, device):
    if nbytes < 0:
        raise ValueError("invalid shape for a work-size query")
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def gptq_hessian(x, h=None, stream=None):
    """h += x^T x for a contiguous fp32 device tensor x [t][k]; allocates a
    zero fp64 [k][k] accumulator when ``h`` is None.  Returns h."""
    if x.dtype != torch.float32 or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous float32 [t][k] tensor")
    t, k = int(x.shape[0]), int(x.shape[1])
    if h is None:
        h = torch.zeros((k, k), dtype=torch.float64, device=x.device)
    if h.dtype != torch.float64 or not h.is_contiguous() or tuple(h.shape) != (k, k):
        raise ValueError("h must be a contiguous float64 [k][k] tensor")
    nb = lib().qw_gptq_hessian_work_bytes(k, t)
    work = _work(nb, x.device)
    _check(qw_gptq_hessian(k, t, x, h, work, nb, stream), "qw_gptq_hessian")
    return h


def gptq_factor(h, damp=0.01, stream=None, check=True):
    """U (fp64 [k][k], upper) with (h + damp*mean(diag h)*I)^-1 = U^T U.
    With ``check`` the stream is synchronized and a non-positive-definite h
    raises; otherwise (u, info) is returned with info a device int32."""
    if h.dtype != torch.float64 or not h.is_contiguous() or h.dim() != 2 \
            or h.shape[0] != h.shape[1]:
        raise ValueError("h must be a contiguous float64 [k][k] tensor")
    k = int(h.shape[0])
    u = torch.empty((k, k), dtype=torch.float64, device=h.device)
    info = torch.zeros(1, dtype=torch.int32, device=h.device)
    nb = lib().qw_gptq_factor_work_bytes(k)
    work = _work(nb, h.device)
    _check(qw_gptq_factor(k, h, float(damp), u, info, work, nb, stream), "qw_gptq_factor")
    if not check:
        return u, info
    if k and int(info.item()) != 0:
        raise QwError(-9, "qw_gptq_factor: the damped H is not positive definite")
    return u


def gptq_quantize_pack(w, u, bits, group, stream=None):
    """GPTQ codes of a contiguous fp32 device weight [n][k] with the factor
    ``u`` from gptq_factor; returns a record like quantize_pack."""
    if w.dtype != torch.float32 or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 tensor")
    n, k = _nk(w.shape)
    if u.dtype != torch.float64 or not u.is_contiguous() or tuple(u.shape) != (k, k):
        raise ValueError("u must be a contiguous float64 [k][k] tensor")
    nb = lib().qw_payload_bytes(bits, n, k)
    ns = lib().qw_num_scales(group, n, k)
    if nb < 0 or ns < 0:
        _check(QW_EBITS if bits not in (4, 8) else -2 if ns < 0 else -3, "gptq_quantize_pack")
    payload = torch.empty(nb, dtype=torch.uint8, device=w.device)
    scales = torch.empty(ns, dtype=torch.float32, device=w.device)
    wb = lib().qw_gptq_quantize_work_bytes(n, k)
    work = _work(wb, w.device)
    _check(qw_gptq_quantize_pack(bits, group, n, k, w, u, payload, scales, work, wb, stream),
           "qw_gptq_quantize_pack")
    return dict(bits=bits, group=group, shape=[n, k], payload=payload, scales=scales)


def gptq(w, h, bits, group, damp=0.01, stream=None):
    """The whole chain from an accumulated h: damping, factor, codes."""
    return gptq_quantize_pack(w, gptq_factor(h, damp, stream), bits, group, stream)
