// C ABI of libqw (declared in include/qw.h): argument validation and
// dispatch to the HIP kernels.  No allocation, no synchronization.
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/qw.h"
#include "qw_internal.h"

namespace {

thread_local char g_last_error[256] = {0};

int record(hipError_t e) {
  if (e == hipSuccess) return QW_OK;
  strncpy(g_last_error, hipGetErrorString(e), sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = 0;
  return QW_EHIP;
}

// 0 <= a, b and a * b <= lim (each factor bounded first, so the product
// cannot overflow).
bool within(int64_t a, int64_t b, int64_t lim = QW_MAX_ELEMENTS) {
  return a >= 0 && b >= 0 && a <= lim && b <= lim && (a == 0 || b <= lim / a);
}

// Validates bits / group / shape; fills `mt` on success.
int check_mat(int bits, int64_t group, int64_t n, int64_t k, qw::Mat* mt) {
  if (bits != 4 && bits != 8) return QW_EBITS;
  if (!within(n, k)) return QW_ESHAPE;
  if (group < 1) return QW_EGROUP;
  const int64_t count = n * k;
  if (count % group != 0) return QW_EGROUP;
  if (bits == 4 && count % 2 != 0) return QW_ESHAPE;
  mt->bits = bits;
  mt->group = group;
  mt->n = n;
  mt->k = k;
  return QW_OK;
}

}  // namespace

extern "C" {

int64_t qw_payload_bytes(int bits, int64_t n, int64_t k) {
  if ((bits != 4 && bits != 8) || !within(n, k)) return -1;
  if (bits == 4 && (n * k) % 2 != 0) return -1;
  return n * k * bits / 8;
}

int64_t qw_num_scales(int64_t group, int64_t n, int64_t k) {
  if (group < 1 || !within(n, k) || (n * k) % group != 0) return -1;
  return n * k / group;
}

const char* qw_status_string(int status) {
  switch (status) {
    case QW_OK: return "ok";
    case QW_EBITS: return "bits must be 4 or 8";
    case QW_EGROUP: return "group must be >= 1 and divide n*k";
    case QW_ESHAPE: return "invalid shape (negative, overflowing, or odd element count for int4)";
    case QW_EM: return "m out of range";
    case QW_ENULL: return "required pointer is NULL";
    case QW_EHIP: return "HIP launch failed (see qw_last_error)";
    case QW_ECOUNT: return "invalid batch count or descriptor";
    case QW_EWORK: return "work buffer missing or too small";
    case QW_EARG: return "argument out of range";
    case QW_ESCRATCH:
      return "input too large for the static scratch of qw_matmul_noalloc "
             "(m * k * 2 bytes of bf16 x above QW_MATMUL_NOALLOC_MAX_BYTES)";
    default: return "unknown status";
  }
}

const char* qw_last_error(void) { return g_last_error; }

int qw_quantize_pack(int bits, int64_t group, int64_t n, int64_t k, const float* w,
                     uint8_t* payload, float* scales, void* stream) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  if (n * k == 0) return QW_OK;
  if (!w || !payload || !scales) return QW_ENULL;
  return record(qw::launch_quantize_pack(mt, w, payload, scales, (hipStream_t)stream));
}

int qw_quantize_pack_batched(int count, const qw_quant_desc* descs, void* stream) {
  if (count < 0) return QW_ECOUNT;
  if (count == 0) return QW_OK;
  if (!descs) return QW_ENULL;
  for (int i = 0; i < count; ++i) {
    const qw_quant_desc& d = descs[i];
    if (d.reserved != 0) return QW_ECOUNT;
    qw::Mat mt;
    int st = check_mat(d.bits, d.group, d.n, d.k, &mt);
    if (st != QW_OK) return st;
    if (d.n * d.k > 0 && (!d.w || !d.payload || !d.scales)) return QW_ENULL;
  }
  const int kChunk = 256;
  qw::Mat mts[kChunk];
  const float* ws[kChunk];
  uint8_t* ps[kChunk];
  float* ss[kChunk];
  for (int base = 0; base < count; base += kChunk) {
    int nb = 0;
    for (int i = base; i < count && i < base + kChunk; ++i) {
      const qw_quant_desc& d = descs[i];
      if (d.n * d.k == 0) continue;
      check_mat(d.bits, d.group, d.n, d.k, &mts[nb]);
      ws[nb] = d.w;
      ps[nb] = d.payload;
      ss[nb] = d.scales;
      ++nb;
    }
    int st = record(qw::launch_quantize_pack_batched(mts, ws, ps, ss, nb, (hipStream_t)stream));
    if (st != QW_OK) return st;
  }
  return QW_OK;
}

int qw_unpack(int bits, int64_t group, int64_t n, int64_t k, const uint8_t* payload,
              const float* scales, float* w_out, void* stream) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  if (n * k == 0) return QW_OK;
  if (!payload || !scales || !w_out) return QW_ENULL;
  return record(qw::launch_unpack(mt, payload, scales, w_out, (hipStream_t)stream));
}

int qw_unpack_batched(int count, const qw_unpack_desc* descs, void* stream) {
  if (count < 0) return QW_ECOUNT;
  if (count == 0) return QW_OK;
  if (!descs) return QW_ENULL;
  for (int i = 0; i < count; ++i) {
    const qw_unpack_desc& d = descs[i];
    if (d.reserved != 0) return QW_ECOUNT;
    qw::Mat mt;
    int st = check_mat(d.bits, d.group, d.n, d.k, &mt);
    if (st != QW_OK) return st;
    if (d.n * d.k > 0 && (!d.payload || !d.scales || !d.w_out)) return QW_ENULL;
  }
  const int kChunk = 256;
  qw::Mat mts[kChunk];
  const uint8_t* ps[kChunk];
  const float* ss[kChunk];
  float* os[kChunk];
  for (int base = 0; base < count; base += kChunk) {
    int nb = 0;
    for (int i = base; i < count && i < base + kChunk; ++i) {
      const qw_unpack_desc& d = descs[i];
      if (d.n * d.k == 0) continue;
      check_mat(d.bits, d.group, d.n, d.k, &mts[nb]);
      ps[nb] = d.payload;
      ss[nb] = d.scales;
      os[nb] = d.w_out;
      ++nb;
    }
    int st = record(qw::launch_unpack_batched(mts, ps, ss, os, nb, (hipStream_t)stream));
    if (st != QW_OK) return st;
  }
  return QW_OK;
}

int qw_gemv(int bits, int64_t group, int64_t n, int64_t k, const uint8_t* payload,
            const float* scales, int64_t m, const float* x, float* y, void* stream) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  if (m < 0 || m > 8 || !within(m, n) || !within(m, k)) return QW_EM;
  if (m == 0 || n == 0) return QW_OK;
  if (!y) return QW_ENULL;
  if (k == 0) return record(qw::launch_fill_zero(y, m * n, (hipStream_t)stream));
  if (!payload || !scales || !x) return QW_ENULL;
  return record(qw::launch_gemv(mt, payload, scales, (int)m, x, y, (hipStream_t)stream));
}

int qw_gemv_batched(int count, const qw_gemv_desc* descs, int64_t m, void* stream) {
  if (count < 0) return QW_ECOUNT;
  if (count == 0) return QW_OK;
  if (!descs) return QW_ENULL;
  if (m < 0 || m > 8) return QW_EM;
  if (m == 0) return QW_OK;
  // validate everything before enqueuing anything
  for (int i = 0; i < count; ++i) {
    const qw_gemv_desc& d = descs[i];
    if (d.reserved != 0) return QW_ECOUNT;
    qw::Mat mt;
    int st = check_mat(d.bits, d.group, d.n, d.k, &mt);
    if (st != QW_OK) return st;
    if (!within(m, d.n) || !within(m, d.k)) return QW_EM;
    if (d.n == 0) continue;
    if (!d.y) return QW_ENULL;
    if (d.k > 0 && (!d.payload || !d.scales || !d.x)) return QW_ENULL;
  }
  const int kChunk = 256;
  qw::Mat mts[kChunk];
  const uint8_t* ps[kChunk];
  const float* ss[kChunk];
  const float* xs[kChunk];
  float* ys[kChunk];
  for (int base = 0; base < count; base += kChunk) {
    int nb = 0;
    for (int i = base; i < count && i < base + kChunk; ++i) {
      const qw_gemv_desc& d = descs[i];
      if (d.n == 0) continue;
      if (d.k == 0) {
        int st = record(qw::launch_fill_zero(d.y, m * d.n, (hipStream_t)stream));
        if (st != QW_OK) return st;
        continue;
      }
      check_mat(d.bits, d.group, d.n, d.k, &mts[nb]);
      ps[nb] = d.payload;
      ss[nb] = d.scales;
      xs[nb] = d.x;
      ys[nb] = d.y;
      ++nb;
    }
    int st = record(qw::launch_gemv_batched(mts, ps, ss, (int)m, xs, ys, nb, (hipStream_t)stream));
    if (st != QW_OK) return st;
  }
  return QW_OK;
}

int qw_gemv_chain(int count, const qw_gemv_desc* descs, const int32_t* stage, int64_t m,
                  void* stream) {
  if (count < 0) return QW_ECOUNT;
  if (count == 0) return QW_OK;
  if (!descs) return QW_ENULL;
  if (!stage) return QW_ECOUNT;
  if (m < 0 || m > 8) return QW_EM;
  for (int i = 1; i < count; ++i)
    if (stage[i] < stage[i - 1]) return QW_ECOUNT;
  for (int i = 0; i < count; ++i) {
    const qw_gemv_desc& d = descs[i];
    if (d.reserved != 0) return QW_ECOUNT;
    qw::Mat mt;
    int st = check_mat(d.bits, d.group, d.n, d.k, &mt);
    if (st != QW_OK) return st;
    if (!within(m, d.n) || !within(m, d.k)) return QW_EM;
    if (d.n == 0) continue;
    if (!d.y) return QW_ENULL;
    if (d.k > 0 && (!d.payload || !d.scales || !d.x)) return QW_ENULL;
  }
  if (m == 0) return QW_OK;
  // Stage by stage, in order: the zero fills of the stage's products with
  // k == 0, then one batched launch over its other products.  A y filled
  // here is read only by later stages, which are enqueued after it.
  std::vector<qw::Mat> mts;
  std::vector<const uint8_t*> ps;
  std::vector<const float*> ss, xs;
  std::vector<float*> ys;
  for (int i0 = 0; i0 < count;) {
    int i1 = i0 + 1;
    while (i1 < count && stage[i1] == stage[i0]) ++i1;
    mts.clear();
    ps.clear();
    ss.clear();
    xs.clear();
    ys.clear();
    for (int i = i0; i < i1; ++i) {
      const qw_gemv_desc& d = descs[i];
      if (d.n == 0) continue;
      if (d.k == 0) {
        int st = record(qw::launch_fill_zero(d.y, m * d.n, (hipStream_t)stream));
        if (st != QW_OK) return st;
        continue;
      }
      qw::Mat mt;
      check_mat(d.bits, d.group, d.n, d.k, &mt);
      mts.push_back(mt);
      ps.push_back(d.payload);
      ss.push_back(d.scales);
      xs.push_back(d.x);
      ys.push_back(d.y);
    }
    if (!mts.empty()) {
      int st = record(qw::launch_gemv_batched(mts.data(), ps.data(), ss.data(), (int)m,
                                              xs.data(), ys.data(), (int)mts.size(),
                                              (hipStream_t)stream));
      if (st != QW_OK) return st;
    }
    i0 = i1;
  }
  return QW_OK;
}

int qw_gemm(int bits, int64_t group, int64_t n, int64_t k, const uint8_t* payload,
            const float* scales, int64_t m, const uint16_t* x_bf16, float* y, void* stream) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  if (!within(m, n) || !within(m, k)) return QW_EM;
  if (m == 0 || n == 0) return QW_OK;
  if (!y) return QW_ENULL;
  if (k == 0) return record(qw::launch_fill_zero(y, m * n, (hipStream_t)stream));
  if (!payload || !scales || !x_bf16) return QW_ENULL;
  return record(qw::launch_gemm(mt, payload, scales, m, x_bf16, y, (hipStream_t)stream));
}

int64_t qw_matmul_work_bytes(int64_t m, int64_t k) {
  if (!within(m, k)) return -1;
  if (m <= QW_MATMUL_GEMV_MAX_M) return 0;
  return (m * k * 2 + 255) / 256 * 256;  // bf16 copy of x
}

}  // extern "C"

// The static scratch of qw_matmul_noalloc: each device holds its own copy
// from the library's first use on it until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is only a
// stand-in for the symbol); it passes the device address looked up once per
// device with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[QW_MATMUL_NOALLOC_MAX_BYTES];

namespace {

// qw_matmul with a resolved work pointer (the caller's buffer, or this
// device's static scratch).  Arguments are validated by the callers.
int matmul_with_work(const qw::Mat& mt, const uint8_t* payload, const float* scales, int64_t m,
                     const float* x, float* y, void* work, hipStream_t stream) {
  uint16_t* xb = (uint16_t*)work;
  hipError_t e = qw::launch_round_bf16(x, xb, m * mt.k, stream);
  if (e != hipSuccess) return record(e);
  return record(qw::launch_gemm(mt, payload, scales, m, xb, y, stream));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up on the first call on the
// device (the current device, on which `stream` must run).
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return record(e);
  if (dev < 0 || dev >= kMaxDevices) return QW_EARG;
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return record(e);
    if ((int)sdev != dev) return QW_EARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return record(e);
    if (!p) return QW_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QW_OK;
}

}  // namespace

extern "C" {

int qw_matmul(int bits, int64_t group, int64_t n, int64_t k, const uint8_t* payload,
              const float* scales, int64_t m, const float* x, float* y, void* work,
              int64_t work_bytes, void* stream) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  if (!within(m, n) || !within(m, k)) return QW_EM;
  if (m <= QW_MATMUL_GEMV_MAX_M || (m <= 8 && qw::matmul_prefers_gemv(mt, payload, x)))
    return qw_gemv(bits, group, n, k, payload, scales, m, x, y, stream);
  if (n == 0) return QW_OK;
  if (!y) return QW_ENULL;
  if (k == 0) return record(qw::launch_fill_zero(y, m * n, (hipStream_t)stream));
  if (!payload || !scales || !x) return QW_ENULL;
  if (!work || work_bytes < qw_matmul_work_bytes(m, k)) return QW_EWORK;
  return matmul_with_work(mt, payload, scales, m, x, y, work, (hipStream_t)stream);
}

int qw_matmul_noalloc(int bits, int64_t group, int64_t n, int64_t k, const uint8_t* payload,
                      const float* scales, int64_t m, const float* x, float* y, void* stream) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  if (!within(m, n) || !within(m, k)) return QW_EM;
  if (m <= QW_MATMUL_GEMV_MAX_M || (m <= 8 && qw::matmul_prefers_gemv(mt, payload, x)))
    return qw_gemv(bits, group, n, k, payload, scales, m, x, y, stream);
  if (n == 0) return QW_OK;
  if (qw_matmul_work_bytes(m, k) > QW_MATMUL_NOALLOC_MAX_BYTES) return QW_ESCRATCH;
  if (!y) return QW_ENULL;
  if (k == 0) return record(qw::launch_fill_zero(y, m * n, (hipStream_t)stream));
  if (!payload || !scales || !x) return QW_ENULL;
  void* work = nullptr;
  st = scratch_address((hipStream_t)stream, &work);
  if (st != QW_OK) return st;
  return matmul_with_work(mt, payload, scales, m, x, y, work, (hipStream_t)stream);
}

int64_t qw_gptq_hessian_work_bytes(int64_t k, int64_t t) {
  if (k < 0 || k > QW_GPTQ_MAX_K || !within(t, k, QW_GPTQ_MAX_ELEMENTS)) return -1;
  return qw::gptq_hessian_work_bytes(k, t);
}

int qw_gptq_hessian(int64_t k, int64_t t, const float* x, double* h, void* work,
                    int64_t work_bytes, void* stream) {
  if (k < 0 || k > QW_GPTQ_MAX_K || !within(t, k, QW_GPTQ_MAX_ELEMENTS)) return QW_ESHAPE;
  if (k == 0 || t == 0) return QW_OK;
  if (!x || !h) return QW_ENULL;
  if (!work || work_bytes < qw::gptq_hessian_work_bytes(k, t)) return QW_EWORK;
  return record(qw::launch_gptq_hessian(k, t, x, h, work, (hipStream_t)stream));
}

int64_t qw_gptq_factor_work_bytes(int64_t k) {
  if (k < 0 || k > QW_GPTQ_MAX_K) return -1;
  return qw::gptq_factor_work_bytes(k);
}

int qw_gptq_factor(int64_t k, const double* h, double damp, double* u, int32_t* info,
                   void* work, int64_t work_bytes, void* stream) {
  if (k < 0 || k > QW_GPTQ_MAX_K) return QW_ESHAPE;
  if (!(damp >= 0.0) || !(damp < 1e300)) return QW_EARG;
  if (k == 0) return QW_OK;
  if (!h || !u) return QW_ENULL;
  if (!work || work_bytes < qw::gptq_factor_work_bytes(k)) return QW_EWORK;
  return record(qw::launch_gptq_factor(k, h, damp, u, info, work, (hipStream_t)stream));
}

int64_t qw_gptq_quantize_work_bytes(int64_t n, int64_t k) {
  if (!within(n, k, QW_GPTQ_MAX_ELEMENTS) || n > QW_GPTQ_MAX_N || k > QW_GPTQ_MAX_K) return -1;
  return qw::gptq_quantize_work_bytes(n, k);
}

int qw_gptq_quantize_pack(int bits, int64_t group, int64_t n, int64_t k, const float* w,
                          const double* u, uint8_t* payload, float* scales, void* work,
                          int64_t work_bytes, void* stream) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  if (!within(n, k, QW_GPTQ_MAX_ELEMENTS) || n > QW_GPTQ_MAX_N || k > QW_GPTQ_MAX_K)
    return QW_ESHAPE;
  if (k > 0 && (k % group != 0 || (bits == 4 && group % 2 != 0))) return QW_EGROUP;
  if (n * k == 0) return QW_OK;
  if (!w || !u || !payload || !scales) return QW_ENULL;
  if (!work || work_bytes < qw::gptq_quantize_work_bytes(n, k)) return QW_EWORK;
  return record(qw::launch_gptq_quantize_pack(mt, w, u, payload, scales, work,
                                              (hipStream_t)stream));
}

// Which kernel family a call with these arguments would take (1 = fast,
// 2 = block, 3 = generic, 4 = matrix-core GEMV; for op 5, 1 = GEMV and
// 2 = GEMM; negative = invalid arguments).  Used by the tests to make sure
// every family is exercised.
int qw_debug_path(int op, int bits, int64_t group, int64_t n, int64_t k, const void* a,
                  const void* b) {
  qw::Mat mt;
  int st = check_mat(bits, group, n, k, &mt);
  if (st != QW_OK) return st;
  switch (op) {
    case 0: return qw::quantize_path(mt, (const float*)a, (const uint8_t*)b);
    case 1: return qw::unpack_path(mt, (const uint8_t*)a, (const float*)b);
    case 2: return qw::gemv_path(mt, (const uint8_t*)a, (const float*)b);
    case 3: return qw::gemm_path(mt, (const uint8_t*)a, (const uint16_t*)b);
    case 4: return qw::gemv_mfma_path(mt, (const uint8_t*)a, (const float*)b);
    case 5: return qw::matmul_prefers_gemv(mt, (const uint8_t*)a, (const float*)b) ? 1 : 2;
    default: return QW_ECOUNT;
  }
}

}  // extern "C"
