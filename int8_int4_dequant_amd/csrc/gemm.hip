// Dequantizing GEMM for prefill on the gfx950 matrix cores.
//
//   Y[m][i] = sum_j X[m][j] * bf16(w_hat[i][j]),   fp32 accumulation,
//   w_hat = fl32(q * S), X given as bf16.
//
// (page "Huit bits, puis quatre", section "Ranger des entiers dans des f32":
// large evaluation-time products compute more than they read and use the
// dequantized weights; section "La vitesse": the quantized batch tiles find
// a code's position once per group of neighbouring columns rather than per
// element.)  The weight is dequantized tile by tile into registers and fed to
// v_mfma_f32_32x32x16_bf16; no dequantized copy of the matrix is kept.
//
// Tiling (MFMA-bound: 2*M*N*K flops against bf16 dense peak):
//   * block = 256 threads = 4 waves, output tile 256 (m) x 256 (n), k-step 64.
//   * wave w owns columns [64w, 64w+64) of the tile and all 256 rows: 8 x 2
//     accumulators of 32x32 fp32 (256 accumulation registers per lane).
//   * X tile (256 x 64 bf16 = 32 KiB) is staged through LDS, double
//     buffered, with a 16-byte-chunk XOR swizzle so that the fragment reads
//     (32 consecutive rows, same k) hit distinct banks.
//   * Weight fragments come straight from global memory: within one MFMA the
//     k-slots are a free permutation shared by A and B, so lane group g
//     (lanes 32g..32g+31) takes the contiguous k range [32g, 32g+32) of the
//     step -- 16 bytes of int4 payload (32 for int8) of one output row per
//     lane -- and the matching X values.  The lane decodes its codes once
//     per step (fp8 nibble conversion, exact integer codes), multiplies by
//     its group's scale in fp32 and rounds to bf16 (RNE).
//   * Block order is XCD-aware: blocks land on the 8 XCDs round-robin, so
//     consecutive blocks of one XCD walk all M tiles of one N tile (the
//     weight tile stays in that XCD's L2 while the M tiles reuse it).
#include "qw_internal.h"

namespace qw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64;

struct GemmArgs {
  const uint16_t* x;
  const uint8_t* payload;
  const float* scales;
  float* y;
  int64_t m;
  int n, k;
  int row_stride_b;     // payload bytes per weight row
  int64_t group;
  int per_row_groups;   // 1: k % group == 0 ; 0: group % k == 0
  int64_t groups_per_row;
  int group_shift;      // log2(group) when per_row_groups and group is a power of two, else -1
  int tiles_m, tiles_n;
  int xcd_map;          // 1: XCD-aware block order
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// 8 int4 codes (one dword, element order) -> bf16(fl32(q * s)), packed in 4 dwords.
__device__ __forceinline__ uint4 dequant8_int4(uint32_t w, float s) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);  // e0, e2  (u * 2^-9)
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);   // e4, e6
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);  // e1, e3
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);   // e5, e7
  // q = u * 2^-9 * 512 - 8, exact; then one rounding for q * s.
  const float q0 = __builtin_fmaf(a.x, 512.0f, -8.0f) * s;
  const float q2 = __builtin_fmaf(a.y, 512.0f, -8.0f) * s;
  const float q4 = __builtin_fmaf(b.x, 512.0f, -8.0f) * s;
  const float q6 = __builtin_fmaf(b.y, 512.0f, -8.0f) * s;
  const float q1 = __builtin_fmaf(c.x, 512.0f, -8.0f) * s;
  const float q3 = __builtin_fmaf(c.y, 512.0f, -8.0f) * s;
  const float q5 = __builtin_fmaf(d.x, 512.0f, -8.0f) * s;
  const float q7 = __builtin_fmaf(d.y, 512.0f, -8.0f) * s;
  return make_uint4(pack_bf16x2(q0, q1), pack_bf16x2(q2, q3), pack_bf16x2(q4, q5),
                    pack_bf16x2(q6, q7));
}

// 8 int8 codes (two dwords, element order) -> 4 dwords of bf16 pairs.
__device__ __forceinline__ uint4 dequant8_int8(uint32_t w0, uint32_t w1, float s) {
  const float q0 = (float)(int)(int8_t)(w0) * s;
  const float q1 = (float)(int)(int8_t)(w0 >> 8) * s;
  const float q2 = (float)(int)(int8_t)(w0 >> 16) * s;
  const float q3 = (float)((int)w0 >> 24) * s;
  const float q4 = (float)(int)(int8_t)(w1) * s;
  const float q5 = (float)(int)(int8_t)(w1 >> 8) * s;
  const float q6 = (float)(int)(int8_t)(w1 >> 16) * s;
  const float q7 = (float)((int)w1 >> 24) * s;
  return make_uint4(pack_bf16x2(q0, q1), pack_bf16x2(q2, q3), pack_bf16x2(q4, q5),
                    pack_bf16x2(q6, q7));
}

template <int BITS>
struct BRegs {
  // raw payload of the lane's 32 codes for one N block
  uint4 p[BITS == 4 ? 1 : 2];
  float s;
};

template <int BITS>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * BK * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;    // lane group: k range [32g, 32g+32) of a step
  const int l32 = lane & 31;

  // ---- block -> tile (XCD-aware when the tile grid allows it)
  int tm, tn;
  {
    const int b = blockIdx.x;
    if (a.xcd_map) {
      const int xcd = b & 7, j = b >> 3;
      tm = j % a.tiles_m;
      tn = xcd + 8 * (j / a.tiles_m);
    } else {
      tm = b % a.tiles_m;
      tn = b / a.tiles_m;
    }
  }
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  // ---- per-lane weight rows (two 32-column blocks per wave)
  int nrow[2];
  bool nvalid[2];
  int64_t prow[2], srow[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int nn = n0 + 64 * wave + 32 * nb + l32;
    nvalid[nb] = nn < a.n;
    nrow[nb] = nvalid[nb] ? nn : a.n - 1;
    prow[nb] = (int64_t)nrow[nb] * a.row_stride_b;
    srow[nb] = a.per_row_groups ? (int64_t)nrow[nb] * a.groups_per_row
                                : ((int64_t)nrow[nb] * a.k) / a.group;
  }

  // ---- X tile loader: 2048 16-byte chunks, 8 per thread
  uint4 xa[8];
  auto load_x = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3, kc = id & 7;
      const int64_t mm = m0 + row;
      if (mm < a.m)
        xa[i] = *reinterpret_cast<const uint4*>(a.x + mm * a.k + k0 + kc * 8);
      else
        xa[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3, kc = id & 7;
      *reinterpret_cast<uint4*>(&lds[buf][row * 128 + ((kc ^ (row & 7)) << 4)]) = xa[i];
    }
  };

  BRegs<BITS> br[2];
  auto load_w = [&](int k0) {
    const int kk = k0 + 32 * g;  // first code of this lane's range
    int64_t gi;
    if (a.per_row_groups)
      gi = a.group_shift >= 0 ? (int64_t)(kk >> a.group_shift) : (int64_t)kk / a.group;
    else
      gi = 0;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint8_t* src = a.payload + prow[nb] + (int64_t)kk * BITS / 8;
      br[nb].p[0] = *reinterpret_cast<const uint4*>(src);
      if (BITS == 8) br[nb].p[BITS == 8 ? 1 : 0] = *reinterpret_cast<const uint4*>(src + 16);
      br[nb].s = a.scales[srow[nb] + gi];
    }
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = a.k / BK;
  load_x(0);
  load_w(0);
  store_x(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    // dequantize this step's weight fragments: bq[nb][s] = 8 bf16 of k = 32g + 8s ..
    uint4 bq[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float s = br[nb].s;
      if (BITS == 4) {
        const uint4 p = br[nb].p[0];
        bq[nb][0] = dequant8_int4(p.x, s);
        bq[nb][1] = dequant8_int4(p.y, s);
        bq[nb][2] = dequant8_int4(p.z, s);
        bq[nb][3] = dequant8_int4(p.w, s);
      } else {
        const uint4 p0 = br[nb].p[0], p1 = br[nb].p[BITS == 8 ? 1 : 0];
        bq[nb][0] = dequant8_int8(p0.x, p0.y, s);
        bq[nb][1] = dequant8_int8(p0.z, p0.w, s);
        bq[nb][2] = dequant8_int8(p1.x, p1.y, s);
        bq[nb][3] = dequant8_int8(p1.z, p1.w, s);
      }
    }
    if (ks + 1 < nk) {
      load_x((ks + 1) * BK);
      load_w((ks + 1) * BK);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int row = mb * 32 + l32;
        const int kc = 4 * g + s;
        const uint4 av = *reinterpret_cast<const uint4*>(&lds[buf][row * 128 + ((kc ^ (row & 7)) << 4)]);
        const bf16x8 af = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              af, __builtin_bit_cast(bf16x8, bq[nb][s]), acc[mb][nb], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) {
      store_x(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: D[i][j] of a 32x32 block sits in lane j + 32*((i/4)%2), register 4*(i/8) + i%4
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (!nvalid[nb]) continue;
      const int nn = n0 + 64 * wave + 32 * nb + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t mm = m0 + mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (mm < a.m) a.y[mm * a.n + nn] = acc[mb][nb][r];
      }
    }
}

// ---------------------------------------------------------- generic kernel

// One thread per output; any shape, group and alignment (slow; for shapes
// the tiled kernel does not take).  Same operand rounding as the tiled path.
template <int BITS>
__global__ __launch_bounds__(256) void gemm_generic_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ payload,
    const float* __restrict__ scales, float* __restrict__ y, int64_t m, int64_t n, int64_t k,
    int64_t group) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= m * n) return;
  const int64_t mm = t / n, nn = t % n;
  float sum = 0.0f;
  for (int64_t j = 0; j < k; ++j) {
    const int64_t e = nn * k + j;
    int q;
    if (BITS == 4) {
      const uint32_t b = payload[e >> 1];
      q = (int)((e & 1) ? (b >> 4) : (b & 15u)) - 8;
    } else {
      q = (int)(int8_t)payload[e];
    }
    const float wf = (float)(__bf16)((float)q * scales[e / group]);
    const float xf = __uint_as_float((uint32_t)x[mm * k + j] << 16);
    sum = __builtin_fmaf(xf, wf, sum);
  }
  y[mm * n + nn] = sum;
}

}  // namespace

int gemm_path(const Mat& mt, const uint8_t* payload, const uint16_t* x) {
  const bool shape_ok = mt.k % BK == 0 && mt.n < (1ll << 30) && mt.k < (1ll << 30) &&
                        mt.n * mt.k * mt.bits / 8 < (1ll << 62);
  const bool group_ok = (mt.k % mt.group == 0 && mt.group % 32 == 0) || (mt.group % mt.k == 0);
  if (shape_ok && group_ok && aligned(payload, 16) && aligned(x, 16)) return PATH_FAST;
  return PATH_GENERIC;
}

hipError_t launch_gemm(const Mat& mt, const uint8_t* payload, const float* scales, int64_t m,
                       const uint16_t* x, float* y, hipStream_t st) {
  if (gemm_path(mt, payload, x) == PATH_FAST) {
    GemmArgs a{};
    a.x = x;
    a.payload = payload;
    a.scales = scales;
    a.y = y;
    a.m = m;
    a.n = (int)mt.n;
    a.k = (int)mt.k;
    a.row_stride_b = (int)(mt.k * mt.bits / 8);
    a.group = mt.group;
    a.per_row_groups = mt.k % mt.group == 0 ? 1 : 0;
    a.groups_per_row = a.per_row_groups ? mt.k / mt.group : 0;
    a.group_shift = -1;
    if (a.per_row_groups && (mt.group & (mt.group - 1)) == 0) {
      int sh = 0;
      while ((1ll << sh) < mt.group) ++sh;
      a.group_shift = sh;
    }
    const int64_t tm = (m + BM - 1) / BM;
    const int64_t tn = (mt.n + BN - 1) / BN;
    if (tm * tn >= (1ll << 31)) return hipErrorInvalidValue;
    a.tiles_m = (int)tm;
    a.tiles_n = (int)tn;
    a.xcd_map = (tn % 8 == 0) ? 1 : 0;
    const unsigned grid = (unsigned)(tm * tn);
    if (mt.bits == 4)
      gemm_kernel<4><<<grid, 256, 0, st>>>(a);
    else
      gemm_kernel<8><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  const int64_t outs = m * mt.n;
  const unsigned grid = (unsigned)((outs + 255) / 256);
  if (mt.bits == 4)
    gemm_generic_kernel<4><<<grid, 256, 0, st>>>(x, payload, scales, y, m, mt.n, mt.k, mt.group);
  else
    gemm_generic_kernel<8><<<grid, 256, 0, st>>>(x, payload, scales, y, m, mt.n, mt.k, mt.group);
  return hipGetLastError();
}

}  // namespace qw
