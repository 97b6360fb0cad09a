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
//   * One wave per work item = R consecutive rows of one matrix over the
//     whole row; the waves of a block are independent (no LDS, no barrier),
//     so a launch over many matrices (qw_gemv_batched) streams the weights.
//   * Lane l takes the 8-code chunks l, l+64, ... of each of its R rows:
//     every payload load instruction (4 B int4 / 8 B int8 per lane) is a
//     contiguous run across the wave, the chunk's 8 x values (two 16-byte
//     loads, also contiguous across the wave) serve all R rows, and the
//     group of a chunk is tracked incrementally, without a division.
//     (Measured alternatives -- 16-byte payload chunks with 128-byte x
//     slices per lane, x staged in LDS, persistent prefetching waves -- were
//     slower on gfx950: per-lane 128-byte x slices touch 64 cache lines per
//     load instruction.)  Generic kernel for any other group or alignment.
//   * int4 decode: two masks split a dword into low and high nibbles as
//     bytes 0x0u; v_cvt_pk_f32_fp8 turns two such bytes into u * 2^-9
//     exactly (an OCP e4m3 byte 0x0u has value u * 2^-9 for u < 16) and one
//     fma gives q = u - 8 exactly.  int8 decode: one sign-extending byte
//     conversion per code.
//   * fp32 FMAs accumulate x * q over a chunk (8 terms, one group); the chunk
//     sum times the group's scale is added to the row accumulator.  Every
//     product is exact or singly rounded, so the error stays within
//     (chain length) * 2^-24 * sum|x * w_hat| -- far inside 1e-5 of it.
//   * The R*M partial sums per lane are reduced across the wave with a
//     butterfly reduce-scatter (each step halves the values a lane holds).

#include "qw_internal.h"

namespace qw {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

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
    // lane-dependent choice by bit masks: a select between two array
    // elements can otherwise become a dynamically indexed (scratch) load
    const uint32_t up = (lane & o) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const uint32_t lo = __float_as_uint(v[i]), hi = __float_as_uint(v[i + h]);
      const float send = __uint_as_float((lo & up) | (hi & ~up));
      const float keep = __uint_as_float((hi & up) | (lo & ~up));
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

// 8 int4 codes of one dword, in element order, as exact floats q.  An OCP
// e4m3 byte 0x0u has the value u * 2^-9 for u < 16, so one conversion turns
// two nibble bytes into u * 2^-9; u * 2^-9 * 512 - 8 = q is exact in an fma.
__device__ __forceinline__ void decode8_int4(uint32_t w, float (&q)[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6 as bytes 0x0u
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  q[0] = __builtin_fmaf(a.x, 512.0f, -8.0f); q[2] = __builtin_fmaf(a.y, 512.0f, -8.0f);
  q[4] = __builtin_fmaf(b.x, 512.0f, -8.0f); q[6] = __builtin_fmaf(b.y, 512.0f, -8.0f);
  q[1] = __builtin_fmaf(c.x, 512.0f, -8.0f); q[3] = __builtin_fmaf(c.y, 512.0f, -8.0f);
  q[5] = __builtin_fmaf(d.x, 512.0f, -8.0f); q[7] = __builtin_fmaf(d.y, 512.0f, -8.0f);
}

// 4 int8 codes of one dword, in element order, exact.
__device__ __forceinline__ void decode4_int8(uint32_t w, float (&q)[4]) {
  q[0] = (float)(int)(int8_t)(w);
  q[1] = (float)(int)(int8_t)(w >> 8);
  q[2] = (float)(int)(int8_t)(w >> 16);
  q[3] = (float)((int)w >> 24);
}

// ------------------------------------------------------------------ kernels

// A buffer resource over one payload row (raw addressing, `bytes` long:
// reads past it return zero instead of leaving the row).  Loads through it
// take a 32-bit byte offset and the resource in scalar registers, so they
// need no per-lane 64-bit address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(row), (short)0, bytes,
                                           0x00020000 /* 32-bit data format */);
}

// The PW payload dwords of one 8-code chunk at byte offset `off`
// (non-temporal: each weight is read once).
template <int PW>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                           uint32_t (&p)[PW]) {
  constexpr int kNT = 2;  // cache policy: non-temporal
  if constexpr (PW == 1) {
    p[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, kNT);
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, kNT);
    p[0] = v.x;
    p[1] = v.y;
  }
}

// One matrix of a (possibly batched) call, validated on the host.
struct GemvDesc {
  const uint8_t* payload;
  const float* scales;
  const float* x;
  float* y;
  int64_t group;
  FastDiv cpg;         // 8-code chunks per group (per-row groups)
  int n;               // rows
  int k;               // row length (elements)
  int row_stride_b;    // payload bytes per row (= k * bits / 8)
  int per_row;         // 1: k % group == 0 ; 0: group % k == 0
  int gpr;             // groups per row when per_row
};

// Matrices per launch: the descriptors travel as kernel arguments (up to
// ~21 KB for a whole model's decode pass in one launch; a single matrix
// launches with a one-entry table).
constexpr int GEMV_NB = QW_BATCH_PER_LAUNCH;

template <int NB>
struct GemvBatch {
  int item0[NB];       // first work item of each matrix, ascending
  GemvDesc d[NB];
  int count;           // descriptors in use
  int items;           // total work items
};

// The matrix work item `item` belongs to: a binary search over item0
// (ascending, item0[0] = 0), read in place from the kernel-argument segment
// with scalar loads (indexing the by-value parameter would copy it to
// memory).  Wave-uniform.
template <int NB>
__device__ __forceinline__ int find_desc(const GemvBatch<NB>& b, int item) {
  if constexpr (NB == 1) return 0;
  typedef const __attribute__((address_space(4))) GemvBatch<NB>* KArg;
  const KArg kb = (KArg)__builtin_amdgcn_kernarg_segment_ptr();
  int lo = 0, hi = b.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kb->item0[mid] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int NB>
__device__ __forceinline__ GemvDesc load_desc(int di) {
  typedef const __attribute__((address_space(4))) GemvBatch<NB>* KArg;
  const KArg kb = (KArg)__builtin_amdgcn_kernarg_segment_ptr();
  const auto& d = kb->d[di];
  return GemvDesc{d.payload, d.scales, d.x, d.y, d.group,
                  {d.cpg.mul, d.cpg.shift, d.cpg.is_pow2, d.cpg.d},
                  d.n, d.k, d.row_stride_b, d.per_row, d.gpr};
}

// Streaming kernel: one work item (R rows of one matrix, rows row0 ..
// row0 + R - 1, clamped) per wave; 8-code chunks (4-byte int4 / 8-byte int8
// payload loads per lane and row, two 16-byte x loads per lane), any group
// that is a multiple of 8 codes (or spans whole rows).  The body stays in
// the kernel itself: moved into an inlined helper, the compiler stopped
// issuing the next chunk's loads ahead of the current chunk's arithmetic for
// M >= 4 (one wait per load; 106 -> 158 us for a 28672 x 8192 int4 matrix
// at m = 8).
template <int BITS, int M, int R, int NB>
__global__ __launch_bounds__(256) void gemv8_kernel(const GemvBatch<NB> b) {
  static_assert(R * M <= 64, "a lane holds at most 64 partial sums (one per lane after the"
                            " reduce-scatter)");
  constexpr int V = pow2_at_least(R * M);
  constexpr int PW = BITS == 4 ? 1 : 2;     // payload dwords per 8-code chunk
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= b.items) return;
  const int di = find_desc(b, item);
  const GemvDesc a = load_desc<NB>(di);
  typedef const __attribute__((address_space(4))) GemvBatch<NB>* KArg;
  const int row0 = (item - ((KArg)__builtin_amdgcn_kernarg_segment_ptr())->item0[di]) * R;
  const int nch = a.k / 8;

  __amdgpu_buffer_rsrc_t prsrc[R];
  const float* srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, a.n - 1);
    prsrc[r] = row_rsrc(a.payload + (int64_t)row * a.row_stride_b, a.row_stride_b);
    srow[r] = a.scales + (a.per_row ? (int64_t)row * a.gpr : ((int64_t)row * a.k) / a.group);
  }
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  // the group of chunk c, tracked without a division: chunk l of a lane
  // starts at group gl = l / cpg, and each step of 64 chunks advances the
  // group by 64 / cpg (+1 when the remainder wraps)
  const uint32_t cpg = a.per_row ? a.cpg.d : 0u;
  uint32_t gc = 0, rem = 0, step_g = 0, step_r = 0;
  if (cpg) {
    gc = fastdiv((uint32_t)lane, a.cpg);
    rem = (uint32_t)lane - gc * cpg;
    step_g = fastdiv(64u, a.cpg);
    step_r = 64u - step_g * cpg;
  }
  for (int c = lane; c < nch; c += 64) {
    // 32-bit byte offsets from the wave-uniform row bases: the loads then
    // take a scalar base and a 32-bit offset, with no 64-bit address add
    const uint32_t poff = (uint32_t)c * (4u * PW), soff = gc * 4u, xoff = (uint32_t)c * 32u;
    uint32_t p[R][PW];
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      load_chunk<PW>(prsrc[r], poff, p[r]);
      s[r] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(srow[r]) + soff);
    }
    float xv[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4* xp = reinterpret_cast<const float4*>(
          reinterpret_cast<const uint8_t*>(a.x + (int64_t)m * a.k) + xoff);
      const float4 x0 = xp[0], x1 = xp[1];
      xv[m][0] = x0.x; xv[m][1] = x0.y; xv[m][2] = x0.z; xv[m][3] = x0.w;
      xv[m][4] = x1.x; xv[m][5] = x1.y; xv[m][6] = x1.z; xv[m][7] = x1.w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float q[8];
      if constexpr (BITS == 4) {
        decode8_int4(p[r][0], q);
      } else {
        float q0[4], q1[4];
        decode4_int8(p[r][0], q0);
        decode4_int8(p[r][PW - 1], q1);
#pragma unroll
        for (int e = 0; e < 4; ++e) { q[e] = q0[e]; q[4 + e] = q1[e]; }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf(xv[m][e], q[e], part);
        acc[r * M + m] = __builtin_fmaf(part, s[r], acc[r * M + m]);
      }
    }
    if (cpg) {
      gc += step_g;
      rem += step_r;
      if (rem >= cpg) { rem -= cpg; ++gc; }
    }
  }

  wave_reduce_scatter<V>(acc, lane);
  const int idx = scatter_index<V>(lane);
  if ((lane & (64 / V - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    if (row0 + r < a.n) a.y[(int64_t)m * a.n + row0 + r] = acc[0];
  }
}

// Split-K kernel for matrices with few rows for the GPU (one matrix, or a
// batch such as one stage of a chained decode pass): a block takes one work
// item of R rows of one matrix; its 4 waves each take a quarter of the row's
// 8-code chunks (lane l of wave w: chunks q*w + l, q*w + l + 64, ... below
// q*(w+1)); the four partial sums meet in LDS and are added in wave order
// (deterministic).  Four times the waves of gemv8_kernel for the same rows,
// so a single decode matrix still fills the GPU.
template <int BITS, int M, int R, int NB>
__global__ __launch_bounds__(256) void gemv8_split_kernel(const GemvBatch<NB> b) {
  static_assert(R * M <= 64, "a lane holds at most 64 partial sums (one per lane after the"
                            " reduce-scatter)");
  constexpr int V = pow2_at_least(R * M);
  constexpr int PW = BITS == 4 ? 1 : 2;     // payload dwords per 8-code chunk
  __shared__ float part_lds[4][R * M];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x;               // one work item (R rows) per block
  // a lone matrix (grid = its items) needs no lookup: two dependent
  // kernel-argument loads fewer before the first payload load
  int di = 0, row0 = item * R;
  if constexpr (NB > 1) {
    if (item >= b.items) return;
    di = find_desc(b, item);
    typedef const __attribute__((address_space(4))) GemvBatch<NB>* KArg;
    row0 = (item - ((KArg)__builtin_amdgcn_kernarg_segment_ptr())->item0[di]) * R;
  }
  const GemvDesc a = load_desc<NB>(di);
  const int nch = a.k / 8;
  const int q = (nch + 3) >> 2;              // chunks per wave
  const int cbeg = wave * q;
  const int cend = min(nch, cbeg + q);

  __amdgpu_buffer_rsrc_t prsrc[R];
  const float* srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, a.n - 1);
    prsrc[r] = row_rsrc(a.payload + (int64_t)row * a.row_stride_b, a.row_stride_b);
    srow[r] = a.scales + (a.per_row ? (int64_t)row * a.gpr : ((int64_t)row * a.k) / a.group);
  }
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  const uint32_t cpg = a.per_row ? a.cpg.d : 0u;
  uint32_t gc = 0, rem = 0, step_g = 0, step_r = 0;
  if (cpg) {
    const uint32_t c0 = (uint32_t)(cbeg + lane);
    gc = fastdiv(c0, a.cpg);
    rem = c0 - gc * cpg;
    step_g = fastdiv(64u, a.cpg);
    step_r = 64u - step_g * cpg;
  }
  for (int c = cbeg + lane; c < cend; c += 64) {
    const uint32_t poff = (uint32_t)c * (4u * PW), soff = gc * 4u, xoff = (uint32_t)c * 32u;
    uint32_t p[R][PW];
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      load_chunk<PW>(prsrc[r], poff, p[r]);
      s[r] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(srow[r]) + soff);
    }
    float xv[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4* xp = reinterpret_cast<const float4*>(
          reinterpret_cast<const uint8_t*>(a.x + (int64_t)m * a.k) + xoff);
      const float4 x0 = xp[0], x1 = xp[1];
      xv[m][0] = x0.x; xv[m][1] = x0.y; xv[m][2] = x0.z; xv[m][3] = x0.w;
      xv[m][4] = x1.x; xv[m][5] = x1.y; xv[m][6] = x1.z; xv[m][7] = x1.w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float q8[8];
      if constexpr (BITS == 4) {
        decode8_int4(p[r][0], q8);
      } else {
        float q0[4], q1[4];
        decode4_int8(p[r][0], q0);
        decode4_int8(p[r][PW - 1], q1);
#pragma unroll
        for (int e = 0; e < 4; ++e) { q8[e] = q0[e]; q8[4 + e] = q1[e]; }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf(xv[m][e], q8[e], part);
        acc[r * M + m] = __builtin_fmaf(part, s[r], acc[r * M + m]);
      }
    }
    if (cpg) {
      gc += step_g;
      rem += step_r;
      if (rem >= cpg) { rem -= cpg; ++gc; }
    }
  }

  wave_reduce_scatter<V>(acc, lane);
  const int idx = scatter_index<V>(lane);
  if ((lane & (64 / V - 1)) == 0 && idx < R * M) part_lds[wave][idx] = acc[0];
  __syncthreads();
  if (wave == 0 && lane < R * M) {
    const float v = ((part_lds[0][lane] + part_lds[1][lane]) + part_lds[2][lane]) + part_lds[3][lane];
    const int r = lane / M, m = lane % M;
    if (row0 + r < a.n) a.y[(int64_t)m * a.n + row0 + r] = v;
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

// Rows per wave of the streaming kernel: 8 (x reused across more rows, fewer
// reductions; 8 * m <= 64 partial sums per lane).  Matrices with too few rows
// to give every SIMD waves that way take the split-K kernel instead (with
// 4 rows per wave at m > 4, a 28672-row matrix still streamed and took 108 us
// at m = 8; the split-K kernel takes 88 us).
template <int M>
constexpr int rows_big() { return 8; }
// Rows per block of the split-K kernel.  Every row of a block reuses the
// block's x chunks, so more rows cut x traffic (M rows of x against one
// payload row); fewer rows give a small matrix more blocks.  Measured on int4
// matrices of 4096 to 28672 rows: 8 rows are faster from m = 2 on every
// shape, and at m = 1 from 12288 rows (4096-row matrices prefer 4, 11008-row
// ones are even to slightly slower with 8).
template <int M>
constexpr int rows_split_many() { return 8; }
template <int M>
constexpr int rows_split_few() { return M == 1 ? 4 : 8; }
constexpr int64_t kSplitManyRows = 12288;
// Work items of R rows from which several matrices take the streaming kernel.
constexpr int kBigItemsMany = 2048;

// Launches `count` descriptors (same bits, m), GEMV_NB per launch, R rows per
// work item.
template <int BITS, int M, int R, int NB>
hipError_t launch_group(const GemvDesc* ds, int count, hipStream_t st) {
  for (int base = 0; base < count; base += NB) {
    GemvBatch<NB> b{};
    b.count = count - base < NB ? count - base : NB;
    int items = 0;
    for (int i = 0; i < b.count; ++i) {
      b.d[i] = ds[base + i];
      b.item0[i] = items;
      items += (b.d[i].n + R - 1) / R;
    }
    b.items = items;
    gemv8_kernel<BITS, M, R, NB><<<(unsigned)((items + 3) / 4), 256, 0, st>>>(b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The same for the split-K kernel: one block per work item of R rows.
template <int BITS, int M, int R, int NB>
hipError_t launch_split_group(const GemvDesc* ds, int count, hipStream_t st) {
  for (int base = 0; base < count; base += NB) {
    GemvBatch<NB> b{};
    b.count = count - base < NB ? count - base : NB;
    int items = 0;
    for (int i = 0; i < b.count; ++i) {
      b.d[i] = ds[base + i];
      b.item0[i] = items;
      items += (b.d[i].n + R - 1) / R;
    }
    b.items = items;
    gemv8_split_kernel<BITS, M, R, NB><<<(unsigned)items, 256, 0, st>>>(b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int M>
hipError_t launch_m(const GemvDesc* ds, int count, hipStream_t st) {
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += ds[i].n;
  // big items when they still give about two waves per SIMD (2048 items);
  // a lone matrix keeps the split-K kernel up to four per SIMD (4096 items),
  // since its waves each run a short loop whose load latency few waves hide
  // (int4 group 128 at m = 8: 14336 x 4096 34 -> 27 us, 8192 x 28672
  // 107 -> 86 us).  Below that, the split-K kernel: the 4 waves of a block
  // share R rows and split K, four times the waves for the same rows.
  constexpr int RB = rows_big<M>();
  constexpr int RSM = rows_split_many<M>(), RSF = rows_split_few<M>();
  const bool big = rows / RB >= (count == 1 ? 4096 : kBigItemsMany);
  const bool many = rows >= kSplitManyRows;
  if (count == 1) {
    if (big) return launch_group<BITS, M, RB, 1>(ds, count, st);
    return many ? launch_split_group<BITS, M, RSM, 1>(ds, count, st)
                : launch_split_group<BITS, M, RSF, 1>(ds, count, st);
  }
  if (big) return launch_group<BITS, M, RB, GEMV_NB>(ds, count, st);
  return many ? launch_split_group<BITS, M, RSM, GEMV_NB>(ds, count, st)
              : launch_split_group<BITS, M, RSF, GEMV_NB>(ds, count, st);
}

template <int BITS>
hipError_t launch_bits(const GemvDesc* ds, int count, int m, hipStream_t st) {
  switch (m) {
    case 1: return launch_m<BITS, 1>(ds, count, st);
    case 2: return launch_m<BITS, 2>(ds, count, st);
    case 3: return launch_m<BITS, 3>(ds, count, st);
    case 4: return launch_m<BITS, 4>(ds, count, st);
    case 5: return launch_m<BITS, 5>(ds, count, st);
    case 6: return launch_m<BITS, 6>(ds, count, st);
    case 7: return launch_m<BITS, 7>(ds, count, st);
    default: return launch_m<BITS, 8>(ds, count, st);
  }
}

GemvDesc make_desc(const Mat& mt, const uint8_t* payload, const float* scales, const float* x,
                   float* y) {
  GemvDesc d{};
  const int cpc = 8;  // codes per chunk
  d.payload = payload;
  d.scales = scales;
  d.x = x;
  d.y = y;
  d.n = (int)mt.n;
  d.k = (int)mt.k;
  d.row_stride_b = (int)(mt.k * mt.bits / 8);
  d.group = mt.group;
  d.per_row = mt.k % mt.group == 0 ? 1 : 0;
  d.gpr = d.per_row ? (int)(mt.k / mt.group) : 0;
  d.cpg = make_fastdiv(d.per_row ? (uint32_t)(mt.group / cpc) : 1u);
  return d;
}

hipError_t launch_generic(const Mat& mt, const uint8_t* payload, const float* scales, int m,
                          const float* x, float* y, hipStream_t st) {
  const int64_t waves = mt.n * m;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (mt.bits == 4)
    gemv_generic_kernel<4><<<grid, 256, 0, st>>>(payload, scales, x, y, mt.n, mt.k, m, mt.group);
  else
    gemv_generic_kernel<8><<<grid, 256, 0, st>>>(payload, scales, x, y, mt.n, mt.k, m, mt.group);
  return hipGetLastError();
}

}  // namespace

int gemv_path(const Mat& mt, const uint8_t* payload, const float* x) {
  const int cpc = 8;  // codes per chunk
  const bool shape_ok = mt.k % cpc == 0 && mt.n < (1ll << 30) && mt.k < (1ll << 30) &&
                        (int64_t)mt.k * mt.bits / 8 < (1ll << 31);
  const bool group_ok = (mt.k % mt.group == 0 && mt.group % cpc == 0) || (mt.group % mt.k == 0);
  if (shape_ok && group_ok && aligned(payload, mt.bits == 4 ? 4 : 8) && aligned(x, 16))
    return PATH_FAST;
  return PATH_GENERIC;
}

hipError_t launch_gemv(const Mat& mt, const uint8_t* payload, const float* scales, int m,
                       const float* x, float* y, hipStream_t st) {
  if (gemv_path(mt, payload, x) == PATH_FAST) {
    const GemvDesc d = make_desc(mt, payload, scales, x, y);
    return mt.bits == 4 ? launch_bits<4>(&d, 1, m, st) : launch_bits<8>(&d, 1, m, st);
  }
  return launch_generic(mt, payload, scales, m, x, y, st);
}

hipError_t launch_gemv_batched(const Mat* mts, const uint8_t* const* payloads,
                               const float* const* scales, int m, const float* const* xs,
                               float* const* ys, int count, hipStream_t st) {
  // fast-path matrices, grouped by bit width, go out GEMV_NB per launch;
  // the others take the generic kernel one by one.
  for (int bits = 4; bits <= 8; bits += 4) {
    GemvDesc ds[GEMV_NB];
    int nd = 0;
    for (int i = 0; i <= count; ++i) {
      const bool flush = (i == count) || nd == GEMV_NB;
      if (flush && nd) {
        hipError_t e = bits == 4 ? launch_bits<4>(ds, nd, m, st) : launch_bits<8>(ds, nd, m, st);
        if (e != hipSuccess) return e;
        nd = 0;
      }
      if (i == count) break;
      if (mts[i].bits != bits || mts[i].n * mts[i].k == 0) continue;
      if (gemv_path(mts[i], payloads[i], xs[i]) == PATH_FAST) {
        ds[nd++] = make_desc(mts[i], payloads[i], scales[i], xs[i], ys[i]);
      } else {
        hipError_t e = launch_generic(mts[i], payloads[i], scales[i], m, xs[i], ys[i], st);
        if (e != hipSuccess) return e;
      }
    }
  }
  return hipSuccess;
}

hipError_t launch_gemv_chain(const Mat* mts, const uint8_t* const* payloads,
                             const float* const* scales, int m, const float* const* xs,
                             float* const* ys, const int* stage, int count, hipStream_t st) {
  // each stage is exactly the batched call over its matrices, enqueued in
  // stage order on one stream
  for (int i0 = 0; i0 < count;) {
    int i1 = i0 + 1;
    while (i1 < count && stage[i1] == stage[i0]) ++i1;
    hipError_t e = launch_gemv_batched(mts + i0, payloads + i0, scales + i0, m, xs + i0, ys + i0,
                                       i1 - i0, st);
    if (e != hipSuccess) return e;
    i0 = i1;
  }
  return hipSuccess;
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
