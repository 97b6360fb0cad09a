// Internal interfaces between the C ABI (qw_api.hip) and the kernel files.
// Not installed; the public interface is include/qw.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qw.h"

namespace qw {

// Problem description after validation by the C ABI.
struct Mat {
  int bits;        // 4 or 8
  int64_t group;   // elements per scale, divides n*k
  int64_t n, k;    // rows (output channels), row length (reduction axis)
};

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Each launcher enqueues on `stream` and returns hipSuccess or the launch
// error.  Shapes are already validated and non-empty.
hipError_t launch_quantize_pack(const Mat& mt, const float* w, uint8_t* payload,
                                float* scales, hipStream_t stream);
hipError_t launch_quantize_pack_batched(const Mat* mts, const float* const* ws,
                                        uint8_t* const* payloads, float* const* scales,
                                        int count, hipStream_t stream);
hipError_t launch_unpack(const Mat& mt, const uint8_t* payload,
                         const float* scales, float* w_out, hipStream_t stream);
// Several matrices, each exactly as launch_unpack writes it; vector-path
// matrices of one bit width share launches (QW_BATCH_PER_LAUNCH at a time).
hipError_t launch_unpack_batched(const Mat* mts, const uint8_t* const* payloads,
                                 const float* const* scales, float* const* outs, int count,
                                 hipStream_t stream);
hipError_t launch_gemv(const Mat& mt, const uint8_t* payload, const float* scales,
                       int m, const float* x, float* y, hipStream_t stream);
hipError_t launch_gemv_batched(const Mat* mts, const uint8_t* const* payloads,
                               const float* const* scales, int m, const float* const* xs,
                               float* const* ys, int count, hipStream_t stream);
hipError_t launch_gemm(const Mat& mt, const uint8_t* payload, const float* scales,
                       int64_t m, const uint16_t* x, float* y, hipStream_t stream);
hipError_t launch_fill_zero(float* y, int64_t count, hipStream_t stream);
// x fp32 [count] -> bf16 bit patterns, round to nearest even (gemm.hip).
hipError_t launch_round_bf16(const float* x, uint16_t* xb, int64_t count, hipStream_t stream);

// GPTQ (gptq.hip).  Work buffers are caller-provided device memory of at
// least the returned sizes.
int64_t gptq_hessian_work_bytes(int64_t k, int64_t t);
hipError_t launch_gptq_hessian(int64_t k, int64_t t, const float* x, double* h, void* work,
                               hipStream_t stream);
int64_t gptq_factor_work_bytes(int64_t k);
hipError_t launch_gptq_factor(int64_t k, const double* h, double damp, double* u, int32_t* info,
                              void* work, hipStream_t stream);
int64_t gptq_quantize_work_bytes(int64_t n, int64_t k);
hipError_t launch_gptq_quantize_pack(const Mat& mt, const float* w, const double* u,
                                     uint8_t* payload, float* scales, void* work,
                                     hipStream_t stream);

// Which kernel family a call takes (exposed for tests through qw_debug_path).
enum Path { PATH_NONE = 0, PATH_FAST = 1, PATH_BLOCK = 2, PATH_GENERIC = 3, PATH_MATRIX = 4 };
int quantize_path(const Mat& mt, const float* w, const uint8_t* payload);
int unpack_path(const Mat& mt, const uint8_t* payload, const float* w_out);
int gemv_path(const Mat& mt, const uint8_t* payload, const float* x);
// The kernel family of a lone GEMV at 8 rows of x (PATH_MATRIX: matrix cores).
int gemv_mfma_path(const Mat& mt, const uint8_t* payload, const float* x);
// Whether qw_matmul runs the GEMV instead of the GEMM at 5..8 rows of x.
bool matmul_prefers_gemv(const Mat& mt, const uint8_t* payload, const float* x);
int gemm_path(const Mat& mt, const uint8_t* payload, const uint16_t* x);

}  // namespace qw
