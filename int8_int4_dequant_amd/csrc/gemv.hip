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
//   * int4 decode: flipping a nibble's top bit turns the stored u = q + 8
//     into q's 4-bit two's complement; moved into the top half of a byte it
//     is the signed byte 16 * q, which one sign-extending byte conversion
//     (v_cvt_f32_i32 with a byte select) turns into the exact float 16 * q.
//     Two three-input bit operations and one shift prepare the 8 codes of a
//     dword, so 8 codes cost 11 instructions.  The factor 16 is a power of
//     two: it scales every product, sum and the result exactly and is
//     removed once per output.  int8 decode: one sign-extending byte
//     conversion per code.
//   * fp32 FMAs accumulate x * q over a chunk (8 terms, one group); the chunk
//     sum times the group's scale is added to the row accumulator.  Every
//     product is exact or singly rounded, so the error stays within
//     (chain length) * 2^-24 * sum|x * w_hat| -- far inside 1e-5 of it.
//   * The R*M partial sums per lane are reduced across the wave with a
//     butterfly reduce-scatter (each step halves the values a lane holds).

#include "qw_internal.h"

#include <algorithm>
#include <vector>

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

// 8 int4 codes of one dword, in element order, as the exact floats 16 * q.
// Byte i of the dword holds u = q + 8 of elements 2i (low nibble) and 2i + 1
// (high nibble); u XOR 8 is q's 4-bit two's complement, so with that nibble
// in the top half of a byte (the low half zero) the byte, read as a signed
// 8-bit integer, is exactly 16 * q.
__device__ __forceinline__ void decode8_int4_x16(uint32_t w, float (&q)[8]) {
  const uint32_t hi = (w & 0xF0F0F0F0u) ^ 0x80808080u;          // elements 1, 3, 5, 7
  const uint32_t lo = ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u;   // elements 0, 2, 4, 6
  q[0] = (float)(int8_t)(lo);       q[1] = (float)(int8_t)(hi);
  q[2] = (float)(int8_t)(lo >> 8);  q[3] = (float)(int8_t)(hi >> 8);
  q[4] = (float)(int8_t)(lo >> 16); q[5] = (float)(int8_t)(hi >> 16);
  q[6] = (float)(int8_t)(lo >> 24); q[7] = (float)(int8_t)(hi >> 24);
}

// The factor the decoded codes carry (16 for int4, 1 for int8), removed from
// each output once.
template <int BITS>
constexpr float code_unscale() { return BITS == 4 ? 0.0625f : 1.0f; }

// 4 int8 codes of one dword, in element order, exact.
__device__ __forceinline__ void decode4_int8(uint32_t w, float (&q)[4]) {
  q[0] = (float)(int)(int8_t)(w);
  q[1] = (float)(int)(int8_t)(w >> 8);
  q[2] = (float)(int)(int8_t)(w >> 16);
  q[3] = (float)((int)w >> 24);
}

// ------------------------------------------------------------------ kernels

// acc += (sum over the chunk's 8 codes of x * code) * s.  With one x row the
// chunk sum runs as two chains of four products (independent instructions
// for the issue slots); with several rows the rows' chains interleave.
template <int M>
__device__ __forceinline__ void chunk_dot(const float (&xm)[8], const float (&q)[8], float s,
                                          float& acc) {
  float part;
  if constexpr (M == 1) {
    float p0 = xm[0] * q[0], p1 = xm[1] * q[1];
#pragma unroll
    for (int e = 2; e < 8; e += 2) {
      p0 = __builtin_fmaf(xm[e], q[e], p0);
      p1 = __builtin_fmaf(xm[e + 1], q[e + 1], p1);
    }
    part = p0 + p1;
  } else {
    part = xm[0] * q[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) part = __builtin_fmaf(xm[e], q[e], part);
  }
  acc = __builtin_fmaf(part, s, acc);
}

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
    // take a scalar base and a 32-bit offset, with no 64-bit address add.
    // x first, then each row's payload and scale together: loads complete
    // in issue order, so row r's arithmetic can start once its own loads
    // have landed while later rows' loads are still in flight (0.98x the
    // time of all payloads, then all scales, then x, on the 7B decode pass).
    const uint32_t poff = (uint32_t)c * (4u * PW), soff = gc * 4u, xoff = (uint32_t)c * 32u;
    float xv[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4* xp = reinterpret_cast<const float4*>(
          reinterpret_cast<const uint8_t*>(a.x + (int64_t)m * a.k) + xoff);
      const float4 x0 = xp[0], x1 = xp[1];
      xv[m][0] = x0.x; xv[m][1] = x0.y; xv[m][2] = x0.z; xv[m][3] = x0.w;
      xv[m][4] = x1.x; xv[m][5] = x1.y; xv[m][6] = x1.z; xv[m][7] = x1.w;
    }
    uint32_t p[R][PW];
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      load_chunk<PW>(prsrc[r], poff, p[r]);
      s[r] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(srow[r]) + soff);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float q[8];
      if constexpr (BITS == 4) {
        decode8_int4_x16(p[r][0], q);
      } else {
        float q0[4], q1[4];
        decode4_int8(p[r][0], q0);
        decode4_int8(p[r][PW - 1], q1);
#pragma unroll
        for (int e = 0; e < 4; ++e) { q[e] = q0[e]; q[4 + e] = q1[e]; }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) chunk_dot<M>(xv[m], q, s[r], acc[r * M + m]);
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
    if (row0 + r < a.n) a.y[(int64_t)m * a.n + row0 + r] = acc[0] * code_unscale<BITS>();
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
  // The chunk loop below; at M = 1, when no lane of the wave has more than two
  // chunks, both chunks' loads are issued before either is used (one trip to
  // memory instead of two; the same sums in the same order).  The second load
  // of a lane with one chunk is clamped to the row's last chunk and dropped.
  if (M == 1 && cend - cbeg <= 128 && cend > cbeg) {
    const int c0 = cbeg + lane, c1 = c0 + 64;
    const int l0 = c0 < nch ? c0 : nch - 1, l1 = c1 < nch ? c1 : nch - 1;
    const uint32_t glast = a.per_row ? (uint32_t)(a.gpr - 1) : 0u;
    uint32_t p0[R][PW], p1[R][PW];
    float s0[R], s1[R];
    const uint32_t g0 = gc < glast ? gc : glast;
    uint32_t g1 = gc;
    if (cpg) {
      g1 += step_g;
      if (rem + step_r >= cpg) ++g1;
    }
    g1 = g1 < glast ? g1 : glast;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      load_chunk<PW>(prsrc[r], (uint32_t)l0 * (4u * PW), p0[r]);
      load_chunk<PW>(prsrc[r], (uint32_t)l1 * (4u * PW), p1[r]);
      s0[r] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(srow[r]) + g0 * 4u);
      s1[r] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(srow[r]) + g1 * 4u);
    }
    float xv0[M][8], xv1[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4* xp0 = reinterpret_cast<const float4*>(a.x + (int64_t)m * a.k + 8 * (int64_t)l0);
      const float4* xp1 = reinterpret_cast<const float4*>(a.x + (int64_t)m * a.k + 8 * (int64_t)l1);
      const float4 x00 = xp0[0], x01 = xp0[1], x10 = xp1[0], x11 = xp1[1];
      xv0[m][0] = x00.x; xv0[m][1] = x00.y; xv0[m][2] = x00.z; xv0[m][3] = x00.w;
      xv0[m][4] = x01.x; xv0[m][5] = x01.y; xv0[m][6] = x01.z; xv0[m][7] = x01.w;
      xv1[m][0] = x10.x; xv1[m][1] = x10.y; xv1[m][2] = x10.z; xv1[m][3] = x10.w;
      xv1[m][4] = x11.x; xv1[m][5] = x11.y; xv1[m][6] = x11.z; xv1[m][7] = x11.w;
    }
    auto use = [&](const uint32_t (&p)[R][PW], const float (&sc)[R], const float (&xv)[M][8])
        __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float q8[8];
        if constexpr (BITS == 4) {
          decode8_int4_x16(p[r][0], q8);
        } else {
          float q0[4], q1[4];
          decode4_int8(p[r][0], q0);
          decode4_int8(p[r][PW - 1], q1);
#pragma unroll
          for (int e = 0; e < 4; ++e) { q8[e] = q0[e]; q8[4 + e] = q1[e]; }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) chunk_dot<M>(xv[m], q8, sc[r], acc[r * M + m]);
      }
    };
    if (c0 < cend) use(p0, s0, xv0);
    if (c1 < cend) use(p1, s1, xv1);
  } else {
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
          decode8_int4_x16(p[r][0], q8);
        } else {
          float q0[4], q1[4];
          decode4_int8(p[r][0], q0);
          decode4_int8(p[r][PW - 1], q1);
  #pragma unroll
          for (int e = 0; e < 4; ++e) { q8[e] = q0[e]; q8[4 + e] = q1[e]; }
        }
  #pragma unroll
        for (int m = 0; m < M; ++m) chunk_dot<M>(xv[m], q8, s[r], acc[r * M + m]);
      }
      if (cpg) {
        gc += step_g;
        rem += step_r;
        if (rem >= cpg) { rem -= cpg; ++gc; }
      }
    }
  }

  wave_reduce_scatter<V>(acc, lane);
  const int idx = scatter_index<V>(lane);
  if ((lane & (64 / V - 1)) == 0 && idx < R * M) part_lds[wave][idx] = acc[0];
  __syncthreads();
  if (wave == 0 && lane < R * M) {
    const float v = (((part_lds[0][lane] + part_lds[1][lane]) + part_lds[2][lane]) +
                     part_lds[3][lane]) * code_unscale<BITS>();
    const int r = lane / M, m = lane % M;
    if (row0 + r < a.n) a.y[(int64_t)m * a.n + row0 + r] = v;
  }
}

// ------------------------------------------- matrix-core GEMV (M = 3 .. 8)
//
// With several x rows the fp32 kernels above spend 8*M products and M scale
// FMAs per 8 codes on top of the decode, and the wave reductions of R*M
// partial sums; at M = 4 and 8 they are bound by VALU issue and latency, not
// by HBM.  Here the dot products run on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16) without giving up fp32 accuracy:
//   * the codes are small integers, exact in bf16 (int4 as 16*q, int8 as q);
//   * every x value is cut into three bf16 pieces, x = p0 + p1 + p2 exactly:
//     p0 is x with the low 16 bits of its encoding cleared, p1 the same of
//     x - p0, and p2 = x - p0 - p1 keeps at most 8 significant bits; both
//     subtractions are exact (x - p0 only drops bits p0 already holds) as
//     long as nothing underflows (|x| >= 2^-110);
//   * a product of a piece and a code has at most 12 significant bits, so
//     it is exact in the fp32 accumulator, and the only roundings are the
//     accumulator's additions.  Measured on this part, one instruction adds
//     its 32 products and the accumulator with a few roundings near fp32's
//     own (products are aligned to the largest before they are added, in
//     blocks of 8, with the bits below 2^-24 of it dropped, and the block
//     sums rounded as they meet): a handful of 2^-24 relative errors per
//     instruction, as a chain of fp32 additions of the same terms would.
// Layout: the A operand is the x pieces, one row per (piece, x row), piece
// major: 3*M rows in one (M <= 5) or two 16-row sets; rows past 3*M repeat
// the last one and their outputs are dropped.  The B operand is the weights
// (16 columns = 16 weight rows), so each lane's outputs belong to one weight
// row and need one scale per group.  Each (piece, x row, weight row) output
// keeps its own sum; the three pieces are added only in the final sum, so
// the big piece's roundings are not mixed with the small ones' (theirs are
// 2^-8 and 2^-16 smaller).
// Work split: a block takes R tiles of 16 weight rows over the whole row
// length; its W waves split the row into super-steps of 128 codes (a lane
// reads a row-contiguous 32-code slab per super-step: 16 B int4, 32 B int8,
// four lanes cover a 128 B line of a row), and their partial sums meet in
// LDS in wave order, so the result is deterministic.  Each super-step a wave
// cuts the 128*M x values once, two per lane, into pieces stored in its own
// LDS region, reads them back in the A layout, and uses them for its R
// tiles.  With groups of whole super-steps (multiples of 128 codes) a
// super-step's sums are multiplied by its group's scale into fp32
// accumulators (one FMA per output); groups of 32 or 64 codes take a
// transposed layout (see gemv_mfma_body) with one scale per group.
// Error chain of one output, in units of 2^-24 * sum|x * w_hat|: 4
// instructions per super-step on the big piece, one scale FMA, one addition
// per super-step of the wave (row length / 128 / W), W - 1 additions across
// waves and 2 for the pieces -- about 50 for the shapes here, 3e-6, inside
// the 1e-5 bound.

typedef __bf16 mx_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mx_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mx_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMxRowBytes = 272;  // one x row of one piece in LDS: 128 bf16 + 16 B pad
constexpr int kMxCodes = 128;     // codes per super-step
// Super-steps of payload, scales and x in flight per wave (measured on the
// 7B MLP shapes: 2 was as fast as 4 or faster, with 76 instead of 104
// registers at 4 rows of x)
constexpr int kMxAhead = 2;

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 h = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// 8 int4 codes (one dword, element order) -> 8 bf16 values 16*q (exact).
__device__ __forceinline__ mx_u32x4 bf16x8_int4_x16(uint32_t w) {
  float q[8];
  decode8_int4_x16(w, q);
  return mx_u32x4{bf16_pair(q[0], q[1]), bf16_pair(q[2], q[3]), bf16_pair(q[4], q[5]),
                  bf16_pair(q[6], q[7])};
}

// 8 int8 codes (two dwords, element order) -> 8 bf16 values q (exact).
__device__ __forceinline__ mx_u32x4 bf16x8_int8(uint32_t w0, uint32_t w1) {
  float a[4], b[4];
  decode4_int8(w0, a);
  decode4_int8(w1, b);
  return mx_u32x4{bf16_pair(a[0], a[1]), bf16_pair(a[2], a[3]), bf16_pair(b[0], b[1]),
                  bf16_pair(b[2], b[3])};
}

// The three bf16 pieces of x values a (low half) and b (high half), packed.
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& p0, uint32_t& p1,
                                            uint32_t& p2) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  const float a1 = a - __uint_as_float(ua & 0xffff0000u);
  const float b1 = b - __uint_as_float(ub & 0xffff0000u);
  const uint32_t ua1 = __float_as_uint(a1), ub1 = __float_as_uint(b1);
  const float a2 = a1 - __uint_as_float(ua1 & 0xffff0000u);
  const float b2 = b1 - __uint_as_float(ub1 & 0xffff0000u);
  // high halves of (a, b) -> one dword: a's bf16 low, b's high
  p0 = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
  p1 = __builtin_amdgcn_perm(ub1, ua1, 0x07060302u);
  p2 = __builtin_amdgcn_perm(__float_as_uint(b2), __float_as_uint(a2), 0x07060302u);
}

// 4 x 4 transpose between the four 16-lane rows of a wave and four
// registers: afterwards register s of a lane in row kb holds what register
// kb held in row s (same lane within the row).  Two swap stages, 32 then 16
// lanes apart.
__device__ __forceinline__ void xpose4_rows(uint32_t& w0, uint32_t& w1, uint32_t& w2,
                                            uint32_t& w3) {
  const auto a = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  w0 = c[0]; w1 = c[1]; w2 = d[0]; w3 = d[1];
}

// One block: R tiles of 16 weight rows from row 16 * tile0 of matrix `a`.
// GS: groups per super-step -- 1 for groups of whole super-steps (or whole
// rows), 4 for groups of 32 codes, 2 for 64.  With GS > 1 a lane still reads
// its row-contiguous 32-code slab; a transpose across the four lane blocks
// then gives MFMA step s the 32 codes s*32 .. s*32+31 of the super-step (8
// per lane block), the A operand reads x in that order, and the sums of a
// group's steps take that group's scale.
template <int BITS, int M, int R, int W, int P, int GS>
__device__ __forceinline__ void gemv_mfma_body(const GemvDesc& a, int ss_per_group, int tile0) {
  static_assert(M >= 3 && M <= 8 && R >= 1 && P >= 1 && (GS == 1 || GS == 2 || GS == 4),
                "shape of the matrix-core GEMV");
  constexpr bool XP = GS > 1;                     // transposed layout
  constexpr int SPG = 4 / GS;                     // MFMA steps per group (GS > 1)
  constexpr int PB = BITS == 4 ? 4 : 8;           // payload dwords per lane per super-step
  constexpr int NR = 3 * M;                       // A rows: (piece, x row), piece-major
  constexpr int NS = (NR + 15) / 16;              // 16-row MFMA sets
  // a wave's LDS region: the pieces of one super-step (NR rows of 128 bf16),
  // and after the loop its partial sums (R tiles x NS sets x 16 x 16 fp32)
  constexpr int XBYTES = NR * kMxRowBytes, PBYTES = R * NS * 1024;
  constexpr int REGION = XBYTES > PBYTES ? XBYTES : PBYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[W][REGION];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kb = lane >> 4;      // B column (weight row of the tile), k block
  const int ks = a.k / kMxCodes;                  // super-steps per row
  const int qs = (ks + W - 1) / W;
  const int ss0 = min(ks, wave * qs), ss1 = min(ks, ss0 + qs);

  // One buffer resource per tile (wave-uniform, so it stays in scalar
  // registers), bounded at the matrix's last row: a lane's rows past it
  // read zeros, and their outputs are dropped.
  __amdgpu_buffer_rsrc_t rs[R];
  const float* srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int trow = (tile0 + r) * 16;
    const int rows = max(0, min(16, a.n - trow));
    // (readfirstlane: the clamp is computed in vector registers, and a
    // resource there would cost a loop over the lanes' values at every load)
    rs[r] = row_rsrc(a.payload + (int64_t)min(trow, a.n - 1) * a.row_stride_b,
                     __builtin_amdgcn_readfirstlane(rows * a.row_stride_b));
    const int row = min(trow + col, a.n - 1);
    srow[r] = a.scales + (a.per_row ? (int64_t)row * a.gpr : ((int64_t)row * a.k) / a.group);
  }
  const int lane_off = col * a.row_stride_b + kb * (PB * 4);
  uint8_t* const xw = lds[wave];
  // this lane's A-operand rows, one per set (rows past NR repeat the last)
  uint32_t aoff[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t)
    aoff[t] = (uint32_t)(min(16 * t + col, NR - 1) * kMxRowBytes + kb * (XP ? 16 : 64));
  constexpr int SSTEP = XP ? 64 : 16;  // LDS bytes between MFMA steps' x

  mx_f32x4 acc[R][NS];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NS; ++t) acc[r][t] = mx_f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // The payload, scales and x of the next P super-steps are always in
  // flight (a ring of P register slots, refilled as each is used).  Loads
  // complete in issue order, so x goes out with its super-step's payload:
  // fetched a step ahead instead, waiting for it would also wait for the
  // payload issued before it.  The group of the next super-step to load is
  // tracked without a division.
  int lg = 0, lr = 0;  // group of the next super-step to load, and its place in it
  if (!XP && a.per_row) {
    lg = ss0 / ss_per_group;
    lr = ss0 - lg * ss_per_group;
  }
  uint32_t pw[P][R][PB];
  float sc[P][R][GS];
  f32x2 xv[P][M];
  auto load_slot = [&](int ss, uint32_t (&p)[R][PB], float (&sv)[R][GS], f32x2 (&xx)[M])
      __attribute__((always_inline)) {
    constexpr int kNT = 2;  // non-temporal: every weight is read once
#pragma unroll
    for (int m = 0; m < M; ++m)
      xx[m] = *reinterpret_cast<const f32x2*>(a.x + (int64_t)m * a.k + (int64_t)ss * kMxCodes +
                                              2 * lane);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int off = lane_off + ss * (kMxCodes * BITS / 8);
#pragma unroll
      for (int h = 0; h < PB / 4; ++h) {
        const mx_u32x4 v = __builtin_bit_cast(
            mx_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[r], off + 16 * h, 0, kNT));
        p[r][4 * h] = v.x; p[r][4 * h + 1] = v.y; p[r][4 * h + 2] = v.z; p[r][4 * h + 3] = v.w;
      }
      if constexpr (XP) {
#pragma unroll
        for (int g = 0; g < GS; ++g) sv[r][g] = srow[r][GS * ss + g];
      } else {
        sv[r][0] = srow[r][lg];
      }
    }
    if (!XP && a.per_row && ++lr == ss_per_group) { lr = 0; ++lg; }
  };
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (ss0 + j < ss1) load_slot(ss0 + j, pw[j], sc[j], xv[j]);

  for (int base = ss0; base < ss1; base += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int ss = base + j;
      if (ss >= ss1) break;

      // x pieces of this super-step into the wave's LDS region (row
      // piece * M + m) ...
#pragma unroll
      for (int m = 0; m < M; ++m) {
        uint32_t p0, p1, p2;
        split3_pair(xv[j][m].x, xv[j][m].y, p0, p1, p2);
        uint8_t* d = xw + m * kMxRowBytes + 4 * lane;
        *reinterpret_cast<uint32_t*>(d) = p0;
        *reinterpret_cast<uint32_t*>(d + M * kMxRowBytes) = p1;
        *reinterpret_cast<uint32_t*>(d + 2 * M * kMxRowBytes) = p2;
      }
      __builtin_amdgcn_wave_barrier();
      // ... and back in the A-operand layout (a wave's LDS accesses complete
      // in order, so the region needs no barrier)
      mx_u32x4 av[NS][4];
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          av[t][s] = *reinterpret_cast<const mx_u32x4*>(xw + aoff[t] + SSTEP * s);
      __builtin_amdgcn_wave_barrier();

      // Every output (piece, x row, weight row) sums its own products: the
      // pieces are added only at the end, so the big piece's roundings are
      // not mixed with the small ones'.
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t w[PB];
#pragma unroll
        for (int e = 0; e < PB; ++e) w[e] = pw[j][r][e];
        if constexpr (XP) {
          if constexpr (BITS == 4) {
            xpose4_rows(w[0], w[1], w[2], w[3]);
          } else {  // the two dwords of a step transposed as two sets
            xpose4_rows(w[0], w[2], w[4], w[6]);
            xpose4_rows(w[1], w[3], w[5], w[7]);
          }
        }
        mx_f32x4 d[NS];
#pragma unroll
        for (int t = 0; t < NS; ++t) d[t] = mx_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const mx_u32x4 bv = BITS == 4 ? bf16x8_int4_x16(w[s]) : bf16x8_int8(w[2 * s], w[2 * s + 1]);
#pragma unroll
          for (int t = 0; t < NS; ++t)
            d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(mx_bf16x8, av[t][s]), __builtin_bit_cast(mx_bf16x8, bv),
                d[t], 0, 0, 0);
          if constexpr (XP) {  // a group's last step: its sums take its scale
            if ((s + 1) % SPG == 0) {
#pragma unroll
              for (int t = 0; t < NS; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  acc[r][t][i] = __builtin_fmaf(d[t][i], sc[j][r][s / SPG], acc[r][t][i]);
                d[t] = mx_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
              }
            }
          }
        }
        if constexpr (!XP) {
#pragma unroll
          for (int t = 0; t < NS; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[r][t][i] = __builtin_fmaf(d[t][i], sc[j][r][0], acc[r][t][i]);
        }
      }
      // refill this slot with the super-step P ahead
      if (ss + P < ss1) load_slot(ss + P, pw[j], sc[j], xv[j]);
    }
  }

  // Partial sums into the wave's region as [tile][A row][column] ...
  float* const part = reinterpret_cast<float*>(xw);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part[(r * NS * 16 + 16 * t + 4 * kb + i) * 16 + col] = acc[r][t][i];
  __syncthreads();
  // ... then the block's threads, one output each at a time, add the waves'
  // sums in wave order, per piece, and the pieces.
  for (int o = threadIdx.x; o < R * M * 16; o += 64 * W) {
    const int r = o / (M * 16), m = (o / 16) % M, c = o % 16;
    const int row = (tile0 + r) * 16 + c;
    float sp[3];
#pragma unroll
    for (int pc = 0; pc < 3; ++pc) {
      const int idx = (r * NS * 16 + pc * M + m) * 16 + c;
      float v = reinterpret_cast<const float*>(lds[0])[idx];
#pragma unroll
      for (int w = 1; w < W; ++w) v += reinterpret_cast<const float*>(lds[w])[idx];
      sp[pc] = v;
    }
    if (row < a.n) a.y[(int64_t)m * a.n + row] = (sp[0] + (sp[1] + sp[2])) * code_unscale<BITS>();
  }
}

template <int BITS, int M, int R, int W, int P, int GS>
__global__ __launch_bounds__(64 * W) void gemv_mfma_kernel(const GemvDesc a, int ss_per_group) {
  gemv_mfma_body<BITS, M, R, W, P, GS>(a, ss_per_group, blockIdx.x * R);
}

// Several matrices in one launch: one block per work item of R tiles, the
// matrix found by the binary search over the items' first indices.
template <int BITS, int M, int R, int W, int P, int GS, int NB>
__global__ __launch_bounds__(64 * W) void gemv_mfma_batched_kernel(const GemvBatch<NB> b) {
  const int item = blockIdx.x;
  if (item >= b.items) return;
  const int di = find_desc(b, item);
  const GemvDesc a = load_desc<NB>(di);
  typedef const __attribute__((address_space(4))) GemvBatch<NB>* KArg;
  const int tile0 = (item - ((KArg)__builtin_amdgcn_kernarg_segment_ptr())->item0[di]) * R;
  const int spg = (GS == 1 && a.per_row) ? (int)(a.group / kMxCodes) : 1;
  gemv_mfma_body<BITS, M, R, W, P, GS>(a, spg, tile0);
}

// --------------------------------------------------------- generic kernel

// One wave per (row, m) at a time, the grid's waves striding over them; any
// group dividing n*k and any alignment.
template <int BITS>
__global__ __launch_bounds__(256) void gemv_generic_kernel(
    const uint8_t* __restrict__ payload, const float* __restrict__ scales,
    const float* __restrict__ x, float* __restrict__ y, int64_t n, int64_t k, int m,
    int64_t group) {
  const int lane = threadIdx.x & 63;
  for (int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); wid < n * m;
       wid += (int64_t)gridDim.x * 4) {
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
}

// Rows per wave of the streaming kernel: 16 at m = 1, 8 above (x reused
// across more rows, fewer reductions per row; R * m <= 64 partial sums per
// lane).  On the 7B stack's decode pass (224 matrices, one launch) 16 rows
// took 0.94x the time of 8 and 32 rows 1.14x (occupancy 4).  Matrices with
// too few rows to give every SIMD waves that way take the split-K kernel
// instead (with 4 rows per wave at m > 4, a 28672-row matrix still streamed
// and took 108 us at m = 8; the split-K kernel takes 88 us).
template <int M>
constexpr int rows_big() { return M == 1 ? 16 : 8; }
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
// Rows from which several matrices (or a lone one) take the streaming kernel.
constexpr int64_t kBigRowsMany = 16384;
constexpr int64_t kBigRowsLone = 32768;

// Work items one launch takes at most (2^23 blocks of 256 threads for the
// split-K kernel, 2^21 for the streaming one: both inside the 2^32
// work-items of a dispatch).  A matrix on the fast path has at most 2^26
// rows, at least 8 per item, so one always fits.
constexpr int64_t kMaxItems = 1 << 23;

// Fills `b` with descriptors ds[i..] (at most NB, at most kMaxItems work items
// of R rows) and returns the index of the first descriptor left over.
template <int R, int NB>
int fill_batch(const GemvDesc* ds, int i, int count, GemvBatch<NB>& b) {
  b = GemvBatch<NB>{};
  int64_t items = 0;
  for (; i < count && b.count < NB; ++i) {
    const int64_t it = (ds[i].n + R - 1) / R;
    if (b.count > 0 && items + it > kMaxItems) break;
    b.d[b.count] = ds[i];
    b.item0[b.count++] = (int)items;
    items += it;
  }
  b.items = (int)items;
  return i;
}

// Launches `count` descriptors (same bits, m), GEMV_NB per launch, R rows per
// work item.
template <int BITS, int M, int R, int NB>
hipError_t launch_group(const GemvDesc* ds, int count, hipStream_t st) {
  for (int i = 0; i < count;) {
    GemvBatch<NB> b;
    i = fill_batch<R, NB>(ds, i, count, b);
    gemv8_kernel<BITS, M, R, NB><<<(unsigned)((b.items + 3) / 4), 256, 0, st>>>(b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The same for the split-K kernel: one block per work item of R rows.
template <int BITS, int M, int R, int NB>
hipError_t launch_split_group(const GemvDesc* ds, int count, hipStream_t st) {
  for (int i = 0; i < count;) {
    GemvBatch<NB> b;
    i = fill_batch<R, NB>(ds, i, count, b);
    gemv8_split_kernel<BITS, M, R, NB><<<(unsigned)b.items, 256, 0, st>>>(b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int M>
hipError_t launch_m(const GemvDesc* ds, int count, hipStream_t st) {
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += ds[i].n;
  // streaming items when the rows still give about two waves per SIMD in
  // 8-row items (16384 rows); a lone matrix keeps the split-K kernel up to
  // four per SIMD (32768 rows), since its waves each run a short loop whose
  // load latency few waves hide
  // (int4 group 128 at m = 8: 14336 x 4096 34 -> 27 us, 8192 x 28672
  // 107 -> 86 us).  Below that, the split-K kernel: the 4 waves of a block
  // share R rows and split K, four times the waves for the same rows.
  constexpr int RB = rows_big<M>();
  constexpr int RSM = rows_split_many<M>(), RSF = rows_split_few<M>();
  const bool big = rows >= (count == 1 ? kBigRowsLone : kBigRowsMany);
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
  // at most 2^20 blocks (2^28 work-items); their waves stride over the rest
  const int64_t waves = mt.n * m;
  const unsigned grid = (unsigned)std::min<int64_t>((waves + 3) / 4, 1 << 20);
  if (mt.bits == 4)
    gemv_generic_kernel<4><<<grid, 256, 0, st>>>(payload, scales, x, y, mt.n, mt.k, m, mt.group);
  else
    gemv_generic_kernel<8><<<grid, 256, 0, st>>>(payload, scales, x, y, mt.n, mt.k, m, mt.group);
  return hipGetLastError();
}

// Whether the matrix-core kernel can take a lone matrix (at 3..8 x rows):
// rows of whole super-steps, groups of whole super-steps, of 32 or 64 codes,
// or of whole rows,
// 16-byte aligned payload rows and 8-byte aligned x rows, and the payload of
// 16 rows addressable with 32-bit offsets.
bool mfma_ok(const Mat& mt, const uint8_t* payload, const float* x) {
  return mt.k > 0 && mt.k % kMxCodes == 0 && mt.n <= (1ll << 26) &&
         16 * ((int64_t)mt.k * mt.bits / 8) < (1ll << 31) &&
         ((mt.k % mt.group == 0 &&
           (mt.group % kMxCodes == 0 || mt.group == 32 || mt.group == 64)) ||
          mt.group % mt.k == 0) &&
         aligned(payload, 16) && aligned(x, 8);
}

// Rows of x from which the matrix-core kernel beats the fp32 kernels, for a
// matrix (or batch) of `rows` weight rows
// (measured, int4 group 128: 11008 x 4096 at m = 2 9.9 against 10.3 us, at
// m = 3 12.2 against 11.1; 28672 x 8192 at m = 4 50.8 against 52.9 us, at
// m = 8 83 against 63).
int mfma_min_rows(int64_t rows) { return rows >= 16384 ? 5 : 3; }

template <int BITS, int M, int R, int W>
hipError_t launch_mfma_rw(const GemvDesc& d, hipStream_t st) {
  const int64_t blocks = ((d.n + 15) / 16 + R - 1) / R;  // at most 2^22
  if (d.per_row && d.group == 32) {
    gemv_mfma_kernel<BITS, M, R, W, kMxAhead, 4><<<(unsigned)blocks, 64 * W, 0, st>>>(d, 1);
  } else if (d.per_row && d.group == 64) {
    gemv_mfma_kernel<BITS, M, R, W, kMxAhead, 2><<<(unsigned)blocks, 64 * W, 0, st>>>(d, 1);
  } else {
    const int spg = d.per_row ? (int)(d.group / kMxCodes) : 1;
    gemv_mfma_kernel<BITS, M, R, W, kMxAhead, 1><<<(unsigned)blocks, 64 * W, 0, st>>>(d, spg);
  }
  return hipGetLastError();
}

// Work split by shape (measured on int4 group 128 and int8 per-channel
// weights, M = 3..8): tall matrices take two tiles per block over four waves,
// the others one tile per block, over 16 waves when few tiles would leave the
// GPU short of waves, else over 8 (4 for rows of fewer than 8 super-steps).
// 11008 x 4096 (688 tiles) runs best on 8 waves, 4096 x 11008 and 4096 x 4096
// (256 tiles) on 16, 28672 x 8192 (1792 tiles) on two tiles by four waves.
template <int BITS, int M>
hipError_t launch_mfma_m(const GemvDesc& d, hipStream_t st) {
  const int64_t tiles = (d.n + 15) / 16, ks = d.k / kMxCodes;
  if (tiles >= 1024) return launch_mfma_rw<BITS, M, 2, 4>(d, st);
  if (tiles <= 384 && ks >= 32) return launch_mfma_rw<BITS, M, 1, 16>(d, st);
  if (ks >= 8) return launch_mfma_rw<BITS, M, 1, 8>(d, st);
  return launch_mfma_rw<BITS, M, 1, 4>(d, st);
}

template <int BITS>
hipError_t launch_mfma_bits(const GemvDesc& d, int m, hipStream_t st) {
  switch (m) {
    case 3: return launch_mfma_m<BITS, 3>(d, st);
    case 4: return launch_mfma_m<BITS, 4>(d, st);
    case 5: return launch_mfma_m<BITS, 5>(d, st);
    case 6: return launch_mfma_m<BITS, 6>(d, st);
    case 7: return launch_mfma_m<BITS, 7>(d, st);
    default: return launch_mfma_m<BITS, 8>(d, st);
  }
}

// The same over a batch: one launch per QW_BATCH_PER_LAUNCH matrices, work
// items of R tiles.
template <int BITS, int M, int R, int W, int GS>
hipError_t launch_mfma_batched_rw(const GemvDesc* ds, int count, hipStream_t st) {
  for (int i = 0; i < count;) {
    GemvBatch<GEMV_NB> b;
    i = fill_batch<16 * R, GEMV_NB>(ds, i, count, b);
    gemv_mfma_batched_kernel<BITS, M, R, W, kMxAhead, GS, GEMV_NB>
        <<<(unsigned)b.items, 64 * W, 0, st>>>(b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int M, int GS>
hipError_t launch_mfma_batched_m(const GemvDesc* ds, int count, hipStream_t st) {
  int64_t tiles = 0, ks = INT64_MAX;
  for (int i = 0; i < count; ++i) {
    tiles += (ds[i].n + 15) / 16;
    ks = std::min<int64_t>(ks, ds[i].k / kMxCodes);
  }
  if (tiles >= 1024) return launch_mfma_batched_rw<BITS, M, 2, 4, GS>(ds, count, st);
  if (ks >= 8) return launch_mfma_batched_rw<BITS, M, 1, 8, GS>(ds, count, st);
  return launch_mfma_batched_rw<BITS, M, 1, 4, GS>(ds, count, st);
}

template <int BITS, int GS>
hipError_t launch_mfma_batched_g(const GemvDesc* ds, int count, int m, hipStream_t st) {
  switch (m) {
    case 3: return launch_mfma_batched_m<BITS, 3, GS>(ds, count, st);
    case 4: return launch_mfma_batched_m<BITS, 4, GS>(ds, count, st);
    case 5: return launch_mfma_batched_m<BITS, 5, GS>(ds, count, st);
    case 6: return launch_mfma_batched_m<BITS, 6, GS>(ds, count, st);
    case 7: return launch_mfma_batched_m<BITS, 7, GS>(ds, count, st);
    default: return launch_mfma_batched_m<BITS, 8, GS>(ds, count, st);
  }
}

// One launch family per layout: gs groups per super-step (1, 2 or 4).
template <int BITS>
hipError_t launch_mfma_batched_bits(const GemvDesc* ds, int count, int m, int gs,
                                    hipStream_t st) {
  return gs == 4 ? launch_mfma_batched_g<BITS, 4>(ds, count, m, st)
       : gs == 2 ? launch_mfma_batched_g<BITS, 2>(ds, count, m, st)
                 : launch_mfma_batched_g<BITS, 1>(ds, count, m, st);
}

}  // namespace

bool matmul_prefers_gemv(const Mat& mt, const uint8_t* payload, const float* x) {
  // measured at 5..8 rows, int4 g128 and int8 per channel: the matrix-core
  // GEMV beats the bf16 GEMM on 4096-row matrices by 20-50% and is within
  // a few percent of it at 11008 rows; from 14336 rows the GEMM leads
  return mt.n <= 8192 && mfma_ok(mt, payload, x);
}

int gemv_mfma_path(const Mat& mt, const uint8_t* payload, const float* x) {
  return mfma_ok(mt, payload, x) ? PATH_MATRIX : gemv_path(mt, payload, x);
}

int gemv_path(const Mat& mt, const uint8_t* payload, const float* x) {
  const int cpc = 8;  // codes per chunk
  const bool shape_ok = mt.k % cpc == 0 && mt.n <= (1ll << 26) && mt.k < (1ll << 30) &&
                        (int64_t)mt.k * mt.bits / 8 < (1ll << 31);
  const bool group_ok = mt.k > 0 && ((mt.k % mt.group == 0 && mt.group % cpc == 0) ||
                                      (mt.group % mt.k == 0));
  if (shape_ok && group_ok && aligned(payload, mt.bits == 4 ? 4 : 8) && aligned(x, 16))
    return PATH_FAST;
  return PATH_GENERIC;
}

hipError_t launch_gemv(const Mat& mt, const uint8_t* payload, const float* scales, int m,
                       const float* x, float* y, hipStream_t st) {
  if (m >= mfma_min_rows(mt.n) && mfma_ok(mt, payload, x)) {
    const GemvDesc d = make_desc(mt, payload, scales, x, y);
    return mt.bits == 4 ? launch_mfma_bits<4>(d, m, st) : launch_mfma_bits<8>(d, m, st);
  }
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
  // the others take the generic kernel one by one.  Within a launch the
  // matrices are taken longest rows first: work items of one row length
  // then stream back to back (the 7B decode pass in layer order, where
  // 4096- and 11008-code rows alternate, took 1.04x the time of either
  // sorted order).  Every product is computed by its own work items, so the
  // order does not change any result.
  std::vector<int> order(count);
  for (int i = 0; i < count; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return mts[a].k > mts[b].k; });
  // The matrix-core kernel takes the batch's eligible matrices from the row
  // counts a lone matrix of the batch's total rows would take it (measured
  // on 16 layers of the 7B stack at int4 group 128, graph-replayed: m = 3
  // 507 us on the fp32 kernels against 560, m = 4 607 against 591, m = 5 722
  // against 645, m = 8 1027 against 720).
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += mts[i].n;
  const bool mx_rows = m >= mfma_min_rows(rows);
  for (int bits = 4; bits <= 8; bits += 4) {
    GemvDesc ds[GEMV_NB], dx[3][GEMV_NB];  // by layout: 1, 2 or 4 groups per super-step
    int nd = 0, nx[3] = {0, 0, 0};
    for (int oi = 0; oi <= count; ++oi) {
      if (((oi == count) || nd == GEMV_NB) && nd) {
        hipError_t e = bits == 4 ? launch_bits<4>(ds, nd, m, st) : launch_bits<8>(ds, nd, m, st);
        if (e != hipSuccess) return e;
        nd = 0;
      }
      for (int g = 0; g < 3; ++g) {
        if (((oi == count) || nx[g] == GEMV_NB) && nx[g]) {
          hipError_t e = bits == 4 ? launch_mfma_batched_bits<4>(dx[g], nx[g], m, 1 << g, st)
                                   : launch_mfma_batched_bits<8>(dx[g], nx[g], m, 1 << g, st);
          if (e != hipSuccess) return e;
          nx[g] = 0;
        }
      }
      if (oi == count) break;
      const int i = order[oi];
      if (mts[i].bits != bits || mts[i].n * mts[i].k == 0) continue;
      if (mx_rows && mfma_ok(mts[i], payloads[i], xs[i])) {
        const bool pr = mts[i].k % mts[i].group == 0;
        const int g = pr && mts[i].group == 32 ? 2 : pr && mts[i].group == 64 ? 1 : 0;
        dx[g][nx[g]++] = make_desc(mts[i], payloads[i], scales[i], xs[i], ys[i]);
      } else if (gemv_path(mts[i], payloads[i], xs[i]) == PATH_FAST) {
        ds[nd++] = make_desc(mts[i], payloads[i], scales[i], xs[i], ys[i]);
      } else {
        hipError_t e = launch_generic(mts[i], payloads[i], scales[i], m, xs[i], ys[i], st);
        if (e != hipSuccess) return e;
      }
    }
  }
  return hipSuccess;
}

__global__ void fill_zero_kernel(float* y, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256)
    y[i] = 0.0f;
}

hipError_t launch_fill_zero(float* y, int64_t count, hipStream_t st) {
  // at most 2^20 blocks, striding over the rest
  fill_zero_kernel<<<(unsigned)std::min<int64_t>((count + 255) / 256, 1 << 20), 256, 0, st>>>(
      y, count);
  return hipGetLastError();
}

}  // namespace qw
