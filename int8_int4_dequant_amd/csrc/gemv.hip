// Dequantizing GEMV for decode (M = 1..8), fp32 arithmetic, for gfx950.
//
//   y[m][i] = sum_j x[m][j] * q[i][j] * S[i][group of j]
//
// (page "Huit bits, puis quatre", section "Ranger des entiers dans des f32":
// the generation-time products of QuantizedMatmul read the codes and the
// scales directly; section "La vitesse": a GEMV that waits on one word per
// load, or that does an integer division per word to find its group, is
// slow -- the group is tracked per chunk here and one 16-byte load carries
// 32 int4 or 16 int8 codes.)
//
// Design (HBM-bound for M <= ~4; fp32-FMA bound beyond):
//   * A block of W waves owns R consecutive output rows.  Its 64*W lanes
//     split every row into 16-byte chunks (lane t takes chunks t, t+64W, ...),
//     so each payload load instruction is a fully coalesced 1 KiB run.
//   * Per chunk a lane loads the R rows' 16 bytes (R loads in flight), the
//     matching x values (shared by all R rows) and one scale per row.
//   * int4 decode: two masks split a dword into low and high nibbles as
//     bytes 0x0u; v_cvt_pk_f32_fp8 turns two such bytes into u * 2^-9
//     exactly (an OCP e4m3 byte 0x0u has value u * 2^-9 for u < 16), and
//     subtracting 8 * 2^-9 gives q * 2^-9 exactly.  int8 decode: one
//     sign-extending byte conversion per code.
//   * fp32 FMAs accumulate x * q per chunk; the chunk sum is scaled by S
//     (and 2^9 for int4) into the row accumulator.  Every product and the
//     scaling are exact or singly rounded, so the error is within
//     (chain length) * 2^-24 * sum|x * w_hat| -- well inside 1e-5 of it.
//   * The R*M partial sums per lane are reduced across the wave with a
//     butterfly reduce-scatter (each step halves the values a lane holds),
//     then across the W waves through LDS.
#include "qw_internal.h"

namespace qw {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load of packed codes: read once.
__device__ __forceinline__ uint4 ldnt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Unsigned division by a runtime constant d >= 1 for numerators < 2^31:
// q = (umulhi(n, mul) + n * add) >> shift  -- computed on the host
// (round-up method of Granlund & Montgomery).
struct FastDiv {
  uint32_t mul, shift, is_pow2, d;
};

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{};
  f.d = d;
  if ((d & (d - 1)) == 0) {
    f.is_pow2 = 1;
    f.shift = 0;
    while ((1u << f.shift) < d) ++f.shift;
    f.mul = 0;
    return f;
  }
  f.is_pow2 = 0;
  uint32_t l = 0;
  while ((1u << l) < d) ++l;  // l = ceil(log2 d)
  // m = floor(2^(32+l) / d) + 1 fits in 33 bits; store low 32 bits and use
  // the standard add-back form: q = (t + ((n - t) >> 1)) >> (l - 1), t = umulhi(n, m')
  const uint64_t m = ((1ull << (32 + l)) / d) + 1;
  f.mul = (uint32_t)(m & 0xffffffffu);
  f.shift = l;
  return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  if (f.is_pow2) return n >> f.shift;
  const uint32_t t = __umulhi(n, f.mul);
  return (t + ((n - t) >> 1)) >> (f.shift - 1);
}

// ---------------------------------------------------------- reduce-scatter

// After the call lane `lane` holds, in v[0], the wave-wide sum of the
// values originally at index idx(lane) = sum_s bit(5-s, lane) * (V >> (s+1)).
template <int V>
__device__ __forceinline__ void wave_reduce_scatter(float (&v)[V], int lane) {
  constexpr int LOGV = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : V == 16 ? 4 : V == 32 ? 5 : 6;
  static_assert((1 << LOGV) == V, "V must be a power of two <= 64");
#pragma unroll
  for (int s = 0; s < LOGV; ++s) {
    const int o = 32 >> s;
    const int h = V >> (s + 1);
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? v[i] : v[i + h];
      const float keep = up ? v[i + h] : v[i];
      v[i] = keep + __shfl_xor(send, o);
    }
  }
#pragma unroll
  for (int o = 32 >> LOGV; o >= 1; o >>= 1) v[0] += __shfl_xor(v[0], o);
}

template <int V>
__device__ __forceinline__ int scatter_index(int lane) {
  int idx = 0;
#pragma unroll
  for (int s = 0; (1 << s) < V; ++s)
    if (lane & (32 >> s)) idx += V >> (s + 1);
  return idx;
}

constexpr int pow2_at_least(int v) {
  return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : v <= 8 ? 8 : v <= 16 ? 16 : v <= 32 ? 32 : 64;
}

// ------------------------------------------------------------ decode helpers

// 8 int4 codes of one dword, in element order, as q * 2^-9 (exact).
__device__ __forceinline__ void decode8_int4(uint32_t w, float (&q)[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6 as bytes 0x0u
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  constexpr float off = 8.0f / 512.0f;  // the +8 offset in units of 2^-9
  q[0] = a.x - off; q[2] = a.y - off; q[4] = b.x - off; q[6] = b.y - off;
  q[1] = c.x - off; q[3] = c.y - off; q[5] = d.x - off; q[7] = d.y - off;
}

// 4 int8 codes of one dword, in element order, exact.
__device__ __forceinline__ void decode4_int8(uint32_t w, float (&q)[4]) {
  q[0] = (float)(int)(int8_t)(w);
  q[1] = (float)(int)(int8_t)(w >> 8);
  q[2] = (float)(int)(int8_t)(w >> 16);
  q[3] = (float)((int)w >> 24);
}

// ------------------------------------------------------------------ kernel

struct GemvArgs {
  const uint8_t* payload;
  const float* scales;
  const float* x;
  float* y;
  int n;             // rows
  int k;             // row length (elements)
  int nchunks;       // 16-byte chunks per row
  int row_stride_b;  // bytes per payload row (= k * bits / 8)
  int64_t group;
  int per_row_groups;  // 1: k % group == 0 ; 0: group % k == 0
  int64_t groups_per_row;  // k / group when per_row_groups
  FastDiv cpg;         // chunks per group (per_row_groups only)
};

template <int BITS, int M, int R>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  constexpr int CPC = BITS == 4 ? 32 : 16;  // codes per 16-byte chunk
  constexpr int V = pow2_at_least(R * M);
  __shared__ float red[4][V];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int row0 = blockIdx.x * R;

  int64_t rowoff[R];   // byte offset of each row's payload
  int64_t sbase[R];    // scale index of the row's first group
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, a.n - 1);
    rowoff[r] = (int64_t)row * a.row_stride_b;
    sbase[r] = a.per_row_groups ? (int64_t)row * a.groups_per_row
                                : ((int64_t)row * a.k) / a.group;
  }

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  for (int c = tid; c < a.nchunks; c += nthreads) {
    uint4 p[R];
    float s[R];
    const int gc = a.per_row_groups ? (int)fastdiv((uint32_t)c, a.cpg) : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      p[r] = ldnt(reinterpret_cast<const uint4*>(a.payload + rowoff[r]) + c);
      s[r] = a.scales[sbase[r] + gc];
    }
    float part[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) part[r][m] = 0.0f;

    const float* xc = a.x + (int64_t)c * CPC;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      constexpr int E = BITS == 4 ? 8 : 4;  // codes per dword
      float xv[M][E];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float4* xp = reinterpret_cast<const float4*>(xc + (int64_t)m * a.k + d * E);
        const float4 x0 = xp[0];
        xv[m][0] = x0.x; xv[m][1] = x0.y; xv[m][2] = x0.z; xv[m][3] = x0.w;
        if constexpr (E == 8) {
          const float4 x1 = xp[1];
          xv[m][4] = x1.x; xv[m][5] = x1.y; xv[m][6] = x1.z; xv[m][7] = x1.w;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w = d == 0 ? p[r].x : d == 1 ? p[r].y : d == 2 ? p[r].z : p[r].w;
        float q[E];
        if (BITS == 4) {
          float q8[8];
          decode8_int4(w, q8);
#pragma unroll
          for (int e = 0; e < E; ++e) q[e] = q8[e];
        } else {
          float q4[4];
          decode4_int8(w, q4);
#pragma unroll
          for (int e = 0; e < E; ++e) q[e] = q4[e];
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int e = 0; e < E; ++e) part[r][m] = __builtin_fmaf(xv[m][e], q[e], part[r][m]);
      }
    }
    constexpr float unit = BITS == 4 ? 512.0f : 1.0f;  // undo the 2^-9 of the int4 decode
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        acc[r * M + m] = __builtin_fmaf(part[r][m] * unit, s[r], acc[r * M + m]);
  }

  wave_reduce_scatter<V>(acc, lane);
  const int idx = scatter_index<V>(lane);
  const int nw = nthreads >> 6;
  if (nw == 1) {
    if ((lane & (64 / V - 1)) == 0 && idx < R * M) {
      const int r = idx / M, m = idx % M;
      if (row0 + r < a.n) a.y[(int64_t)m * a.n + row0 + r] = acc[0];
    }
    return;
  }
  if ((lane & (64 / V - 1)) == 0) red[wave][idx] = acc[0];
  __syncthreads();
  if (tid < R * M) {
    float t = red[0][tid];
    for (int w = 1; w < nw; ++w) t += red[w][tid];
    const int r = tid / M, m = tid % M;
    if (row0 + r < a.n) a.y[(int64_t)m * a.n + row0 + r] = t;
  }
}

// --------------------------------------------------------- generic kernel

// One wave per (row, m); any group dividing n*k and any alignment.
template <int BITS>
__global__ __launch_bounds__(256) void gemv_generic_kernel(
    const uint8_t* __restrict__ payload, const float* __restrict__ scales,
    const float* __restrict__ x, float* __restrict__ y, int64_t n, int64_t k, int m,
    int64_t group) {
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= n * m) return;
  const int64_t row = wid % n;
  const int64_t mm = wid / n;
  float sum = 0.0f;
  for (int64_t j = lane; j < k; j += 64) {
    const int64_t e = row * k + j;
    int q;
    if (BITS == 4) {
      const uint32_t b = payload[e >> 1];
      q = (int)((e & 1) ? (b >> 4) : (b & 15u)) - 8;
    } else {
      q = (int)(int8_t)payload[e];
    }
    sum = __builtin_fmaf(x[mm * k + j], (float)q * scales[e / group], sum);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) y[mm * n + row] = sum;
}

template <int BITS, int M>
hipError_t launch_fast(const GemvArgs& a, hipStream_t st) {
  constexpr int R = M <= 4 ? 8 : 4;
  const int w4 = (a.nchunks + 63) / 64;
  const int waves = w4 < 4 ? w4 : 4;
  const unsigned grid = (unsigned)((a.n + R - 1) / R);
  gemv_kernel<BITS, M, R><<<grid, 64 * waves, 0, st>>>(a);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_fast_bits(const GemvArgs& a, int m, hipStream_t st) {
  switch (m) {
    case 1: return launch_fast<BITS, 1>(a, st);
    case 2: return launch_fast<BITS, 2>(a, st);
    case 3: return launch_fast<BITS, 3>(a, st);
    case 4: return launch_fast<BITS, 4>(a, st);
    case 5: return launch_fast<BITS, 5>(a, st);
    case 6: return launch_fast<BITS, 6>(a, st);
    case 7: return launch_fast<BITS, 7>(a, st);
    default: return launch_fast<BITS, 8>(a, st);
  }
}

}  // namespace

int gemv_path(const Mat& mt, const uint8_t* payload, const float* x) {
  const int cpc = mt.bits == 4 ? 32 : 16;
  const bool shape_ok = mt.k % cpc == 0 && mt.n < (1ll << 31) && mt.k < (1ll << 31) &&
                        (int64_t)mt.k * mt.bits / 8 < (1ll << 31);
  const bool group_ok = (mt.k % mt.group == 0 && mt.group % cpc == 0) || (mt.group % mt.k == 0);
  if (shape_ok && group_ok && aligned(payload, 16) && aligned(x, 16)) return PATH_FAST;
  return PATH_GENERIC;
}

hipError_t launch_gemv(const Mat& mt, const uint8_t* payload, const float* scales, int m,
                       const float* x, float* y, hipStream_t st) {
  if (gemv_path(mt, payload, x) == PATH_FAST) {
    GemvArgs a{};
    const int cpc = mt.bits == 4 ? 32 : 16;
    a.payload = payload;
    a.scales = scales;
    a.x = x;
    a.y = y;
    a.n = (int)mt.n;
    a.k = (int)mt.k;
    a.row_stride_b = (int)(mt.k * mt.bits / 8);
    a.nchunks = a.row_stride_b / 16;
    a.group = mt.group;
    a.per_row_groups = mt.k % mt.group == 0 ? 1 : 0;
    a.groups_per_row = a.per_row_groups ? mt.k / mt.group : 0;
    a.cpg = make_fastdiv(a.per_row_groups ? (uint32_t)(mt.group / cpc) : 1u);
    return mt.bits == 4 ? launch_fast_bits<4>(a, m, st) : launch_fast_bits<8>(a, m, st);
  }
  const int64_t waves = mt.n * m;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (mt.bits == 4)
    gemv_generic_kernel<4><<<grid, 256, 0, st>>>(payload, scales, x, y, mt.n, mt.k, m, mt.group);
  else
    gemv_generic_kernel<8><<<grid, 256, 0, st>>>(payload, scales, x, y, mt.n, mt.k, m, mt.group);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* y, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) y[i] = 0.0f;
}

hipError_t launch_fill_zero(float* y, int64_t count, hipStream_t st) {
  fill_zero_kernel<<<(unsigned)((count + 255) / 256), 256, 0, st>>>(y, count);
  return hipGetLastError();
}

}  // namespace qw
