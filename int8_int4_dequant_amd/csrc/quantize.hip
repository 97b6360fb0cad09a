// One-pass quantize/pack and unpack kernels for gfx950.
//
// Method (page "量化推理：INT8/INT4 的体积、困惑度与速度为什么不同步", script
// functions `pack` / `unpack`; page "Huit bits, puis quatre", section
// "Arrondir"): per group of `group` consecutive weights, S = max|w| / qmax
// (IEEE fp32 division, S = 1 for an all-zero group); codes
// q = clip(rint(w / S), -qmax, qmax) with an IEEE fp32 division and
// round-half-even; int8 payload = two's-complement bytes; int4 payload =
// (q + 8) nibbles, element 2i in the low nibble of byte i.  Unpack gives
// fl32(float(q) * S).
//
// These kernels are HBM-bound (4 B read + bits/8 + 4/group B written per
// weight for quantize; the reverse for unpack).  Bit-exactness relies on the
// correctly rounded fp32 division HIP emits for `/` (no fast-math), on
// rintf (v_rndne_f32, ties to even) and on preserved fp32 denormals; the
// build never enables fast-math or denormal flushing.
//
// Kernel families:
//   subgroup  group a power of two in [8, 1024]: a wave owns 256
//             consecutive float4 vectors, each load instruction reading a
//             contiguous 1 KiB run; a group is consecutive lanes of one
//             instruction (or whole instructions for group >= 512) and its
//             max|w| is reduced with cross-lane shuffles.  One pass.
//   block     group % 4 == 0 and group <= 16384: one 256-thread block per
//             group; weights stay in registers between the max and the code
//             pass.
//   generic   any group dividing n*k, any alignment: a scale kernel (one
//             thread or one block per group) then a code kernel (one thread
//             per payload byte).
#include "qw_internal.h"

#include <algorithm>
#include <vector>

namespace qw {
namespace {

constexpr int QB_J = 16;  // float4 vectors per thread in the block kernel (group <= 16384)

typedef float f32x4 __attribute__((ext_vector_type(4)));
// Word types for the LDS staging buffers, which a wave writes with one word
// size and reads back with another: `may_alias` keeps the compiler from
// assuming that accesses of different types never overlap (and so from
// moving a read-back ahead of the writes it depends on).
typedef uint16_t __attribute__((may_alias)) u16_la;
typedef uint32_t __attribute__((may_alias)) u32_la;
typedef uint32_t u32x2_la __attribute__((ext_vector_type(2), may_alias));
typedef uint32_t u32x4_la __attribute__((ext_vector_type(4), may_alias));

// Streaming (non-temporal) 16-byte load / store: each weight is touched once.
__device__ __forceinline__ float4 ldnt(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stnt(float4* p, float4 v) {
  const f32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
}

template <int BITS>
__device__ __forceinline__ float qmax_f() { return BITS == 8 ? 127.0f : 7.0f; }

// The value held by a partner lane in the other half of this lane's aligned
// run of 2*H lanes.  Within 16-lane rows a DPP lane permutation does it with
// no separate instruction (quad_perm [1,0,3,2] and [2,3,0,1] for H = 1, 2;
// row_half_mirror and row_mirror, i <-> 7-i and i <-> 15-i, for H = 4, 8);
// wider runs take a cross-lane shuffle.  Every lane must be active.
template <int H>
__device__ __forceinline__ float partner(float v) {
  constexpr int ctrl = H == 1 ? 0xB1 : H == 2 ? 0x4E : H == 4 ? 0x141 : 0x140;
  if constexpr (H <= 8)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
  else
    return __shfl_xor(v, H);
}

// max of v with its partner's value (partner<H>) for v >= 0: non-negative
// floats order like their bit patterns, so an unsigned integer max gives the
// float max, and with 0 its identity the DPP move folds into the max
// (v_max_u32 with a DPP operand: one instruction per step).
template <int H>
__device__ __forceinline__ float pair_max_nonneg(float v) {
  const uint32_t u = __float_as_uint(v);
  uint32_t p;
  if constexpr (H <= 8) {
    constexpr int ctrl = H == 1 ? 0xB1 : H == 2 ? 0x4E : H == 4 ? 0x141 : 0x140;
    p = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, ctrl, 0xF, 0xF, false);
  } else {
    p = __float_as_uint(__shfl_xor(v, H));
  }
  return __uint_as_float(u > p ? u : p);
}

// max over an aligned run of R lanes (R a power of two <= 64) of values
// >= 0 (the |w| maxima of finite weights): each step combines the two halves
// of runs twice as long as the last.
template <int R>
__device__ __forceinline__ float run_max(float v) {
  if constexpr (R >= 2) v = pair_max_nonneg<1>(v);
  if constexpr (R >= 4) v = pair_max_nonneg<2>(v);
  if constexpr (R >= 8) v = pair_max_nonneg<4>(v);
  if constexpr (R >= 16) v = pair_max_nonneg<8>(v);
  if constexpr (R >= 32) v = pair_max_nonneg<16>(v);
  if constexpr (R >= 64) v = pair_max_nonneg<32>(v);
  return v;
}

// One code: IEEE division, ties-to-even rounding, clip.  -0 becomes 0.
template <int BITS>
__device__ __forceinline__ int code_of(float w, float s) {
  const float qm = qmax_f<BITS>();
  float r = rintf(w / s);
  r = fminf(fmaxf(r, -qm), qm);
  return (int)r;
}

template <int BITS>
__device__ __forceinline__ float scale_of(float m) {
  float s = m / qmax_f<BITS>();
  return s == 0.0f ? 1.0f : s;
}

// Rounded quotients rint(fl32(w[e] / s)) for the NE values of one lane,
// all in one group (scale s), returned as exact small integers in fp32.
//
// Shortcut: with R = v_rcp_f32(s) (the hardware reciprocal, within 1 ulp of
// 1/s; 2 ulps are assumed below) and t = fl32(w * R),
//   |t - fl32(w / s)| <= (2^-22 + 2^-24 + 2^-24 + O(2^-46)) |w / s|
//                     <= 1.5 * 2^-22 * qmax * (1 + 2^-23)
// (|w / s| <= qmax up to one ulp), i.e. below 2^-20 for int4 and 2^-16 for
// int8, provided 1/s is a normal number.  rint is constant between
// half-integers, so wherever t is farther than MARGIN (2^-17, resp. 2^-14)
// from a half-integer, rint(t) equals rint(fl32(w / s)) exactly.  Otherwise
// (a near-tie, about 2 * MARGIN of random codes) or when s is extreme, every
// value of the lane is recomputed with the IEEE division.  Both paths are
// exact.
template <int BITS, int NE>
__device__ __forceinline__ void rounded_quotients(const float (&w)[NE], float s, float (&r)[NE]) {
  // t must be the rounded product, and t - rint(t) a separate (exact)
  // subtraction: no contraction into an fma here.
#pragma clang fp contract(off)
  constexpr float kMargin = BITS == 4 ? 0x1p-17f : 0x1p-14f;
  bool fast = s >= 0x1p-125f && s <= 0x1p+125f;
  if (fast) {
    const float rs = __builtin_amdgcn_rcpf(s);
    float dmax = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const float t = w[e] * rs;
      const float rt = rintf(t);
      dmax = fmaxf(dmax, fabsf(t - rt));  // exact: t and rint(t) are close
      r[e] = rt;
    }
    fast = dmax < 0.5f - kMargin;
  }
  if (!fast) {
#pragma unroll
    for (int e = 0; e < NE; ++e) r[e] = rintf(w[e] / s);
  }
}

// ---------------------------------------------------------------- subgroup

// Packs 4 rounded quotients (element order): int4 -> 16 bits, int8 -> 32 bits.
// The quotients already lie in [-qmax, qmax] for finite inputs (|w / s|
// exceeds qmax by at most one ulp), so no clip is needed.  Each payload byte
// is formed as an exact small integer in fp32 and converted with the
// byte-inserting conversion (v_cvt_pk_u8_f32, which also clamps garbage from
// non-finite inputs into its own byte): int4 byte = (q0 + 8) + 16 (q1 + 8)
// = 16 q1 + q0 + 136 (one fma); int8 byte = q + 128, then the sign bit of
// each byte is flipped to give q's two's complement.
__device__ __forceinline__ uint32_t pack4_int4(const float* r) {
  const float b0 = __builtin_fmaf(r[1], 16.0f, r[0] + 136.0f);
  const float b1 = __builtin_fmaf(r[3], 16.0f, r[2] + 136.0f);
  return __builtin_amdgcn_cvt_pk_u8_f32(b1, 1, __builtin_amdgcn_cvt_pk_u8_f32(b0, 0, 0));
}
__device__ __forceinline__ uint32_t pack4_int8(const float* r) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) v = __builtin_amdgcn_cvt_pk_u8_f32(r[i] + 128.0f, i, v);
  return v ^ 0x80808080u;
}

constexpr int QV = 4;  // float4 vectors per lane in the unpack kernel

// Subgroup quantize kernel: float4 vectors per lane (a wave takes 64 * QVq)
// and waves per block.  Measured on the 7B stack (int4 group 32, one launch,
// interleaved with the 4-vector, 4-wave form): 2 vectors per lane in 2-wave
// blocks took 0.967 of the time, 2 in 4-wave blocks 0.97-0.98, 4 in 1-wave
// blocks 0.975, 4 in 8- or 16-wave blocks 1.02-1.03.  Groups of more than 64
// vectors span 2 or 4 load instructions, so they keep 4 vectors per lane.
template <int G>
constexpr int quant_qv() { return G <= 64 ? 2 : 4; }
constexpr int QUANT_WAVES = 2;
// Blocks per launch of the single-matrix fast kernels (of at most 256
// threads: 2^32 work-items, the limit of one dispatch); a larger matrix takes
// several launches, each with its first block index.
constexpr uint64_t kMaxLaunchBlocks = 1ull << 24;
// float4 vectors one block quantizes, for a group of `group` weights
inline uint64_t quant_block_vecs(int64_t group) {
  return (uint64_t)64 * (group / 4 <= 64 ? 2 : 4) * QUANT_WAVES;
}

// A wave owns 64*QVq consecutive float4 vectors; its j-th load instruction
// reads vectors [base + 64j, base + 64j + 64) -- one fully coalesced 1 KiB
// run per instruction.  A group of G vectors (G = group / 4, a power of two
// from 2 to 256) is G consecutive lanes of one instruction (G <= 64) or the
// same lane across 2 or 4 instructions (G = 128, 256); max|w| is reduced
// with cross-lane shuffles.  The wave's payload (2 or 4 bytes per vector)
// and scales are assembled in LDS and written with one wide non-temporal
// store per lane (4, 8 or 16 payload bytes): stores of 2 bytes per lane were
// the slowest part of the kernel.
template <int BITS, int G>
__device__ __forceinline__ void quant_subgroup_body(
    const float* __restrict__ w, uint8_t* __restrict__ payload,
    float* __restrict__ scales, uint64_t nvec, uint64_t block) {
  constexpr int QV = quant_qv<G>();         // float4 vectors per lane
  constexpr int PB = BITS / 2;               // payload bytes per vector (2 or 4)
  constexpr int NS = 64 * QV / G;            // scales per wave (1 .. 128)
  __shared__ __attribute__((aligned(16))) uint8_t stage_p[QUANT_WAVES][64 * QV * PB];
  __shared__ __attribute__((aligned(16))) float stage_s[QUANT_WAVES][NS];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const uint64_t base = (block * QUANT_WAVES + wv) * (64 * QV);
  float v[QV][4];
  float m[QV];
#pragma unroll
  for (int j = 0; j < QV; ++j) {
    const uint64_t idx = base + lane + 64 * j;
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (idx < nvec) f = ldnt(reinterpret_cast<const float4*>(w) + idx);
    v[j][0] = f.x; v[j][1] = f.y; v[j][2] = f.z; v[j][3] = f.w;
    m[j] = fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w)));
  }
  // Groups are aligned to G vectors and never straddle the end of the data
  // (nvec is a multiple of G), so inactive lanes only meet inactive lanes.
  if constexpr (G <= 64) {
#pragma unroll
    for (int j = 0; j < QV; ++j) m[j] = run_max<G>(m[j]);
  } else {
    constexpr int J = G / 64;  // instructions per group: 2 or 4
#pragma unroll
    for (int j0 = 0; j0 < QV; j0 += J) {
      float t = m[j0];
#pragma unroll
      for (int j = 1; j < J; ++j) t = fmaxf(t, m[j0 + j]);
      t = run_max<64>(t);
#pragma unroll
      for (int j = 0; j < J; ++j) m[j0 + j] = t;
    }
  }
  // The scales (one IEEE division each).  With two vectors per lane and
  // groups of G <= 64 lanes, every lane meets two groups; the lanes of a
  // group's upper half divide for its second group, those of the lower half
  // for its first, and partners in opposite halves swap results: one
  // division per lane instead of two, on the same operands.
  float sj[QV];
  if constexpr (QV == 2 && G <= 64) {
    const bool upper = (lane & (G / 2)) != 0;
    const float mine = scale_of<BITS>(upper ? m[1] : m[0]);
    const float other = partner<G / 2>(mine);
    sj[0] = upper ? other : mine;
    sj[1] = upper ? mine : other;
  } else {
#pragma unroll
    for (int j = 0; j < QV; ++j) sj[j] = scale_of<BITS>(m[j]);
  }
  // codes and scales into this wave's LDS stage (wave-private: LDS accesses
  // of one wave complete in order, no barrier needed)
#pragma unroll
  for (int j = 0; j < QV; ++j) {
    const int vi = lane + 64 * j;  // vector index within the wave
    const float s = sj[j];
    if (vi % G == 0) stage_s[wv][vi / G] = s;
    float r[4];
    rounded_quotients<BITS, 4>(v[j], s, r);
    if constexpr (BITS == 4)
      reinterpret_cast<u16_la*>(stage_p[wv])[vi] = (uint16_t)pack4_int4(r);
    else
      reinterpret_cast<u32_la*>(stage_p[wv])[vi] = pack4_int8(r);
  }
  // lane L writes vectors [QV*L, QV*L + QV) of the wave: QV * PB contiguous bytes
  const uint64_t v0 = base + (uint64_t)QV * lane;
  if (v0 + QV <= nvec) {
    if constexpr (QV * PB == 4) {
      __builtin_nontemporal_store((uint32_t)reinterpret_cast<const u32_la*>(stage_p[wv])[lane],
                                  reinterpret_cast<uint32_t*>(payload + v0 * PB));
    } else if constexpr (QV * PB == 8) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      __builtin_nontemporal_store((u32x2)reinterpret_cast<const u32x2_la*>(stage_p[wv])[lane],
                                  reinterpret_cast<u32x2*>(payload + v0 * PB));
    } else {
      static_assert(QV * PB == 16, "QV * PB must be 4, 8 or 16");
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store((u32x4)reinterpret_cast<const u32x4_la*>(stage_p[wv])[lane],
                                  reinterpret_cast<u32x4*>(payload + v0 * PB));
    }
  } else {
    for (int i = 0; i < QV && v0 + i < nvec; ++i)
      for (int bb = 0; bb < PB; ++bb)
        payload[(v0 + i) * PB + bb] = stage_p[wv][(QV * lane + i) * PB + bb];
  }
  // scales of the wave's groups: NS contiguous floats, one or two per lane
  const uint64_t g0 = base / G;
  const uint64_t ngr = (nvec - (base < nvec ? base : nvec)) / G;  // groups of this wave with data
  if constexpr (NS <= 64) {
    if (lane < NS && (uint64_t)lane < ngr)
      __builtin_nontemporal_store(stage_s[wv][lane], scales + g0 + lane);
  } else {
#pragma unroll
    for (int i = 0; i < NS / 64; ++i) {
      const int gi = (NS / 64) * lane + i;
      if ((uint64_t)gi < ngr) __builtin_nontemporal_store(stage_s[wv][gi], scales + g0 + gi);
    }
  }
}

// One matrix; a launch covers blocks [block_base, block_base + gridDim.x)
// (a matrix of more than 2^24 blocks takes several launches).
template <int BITS, int G>
__global__ __launch_bounds__(64 * QUANT_WAVES) void quant_subgroup_kernel(
    const float* __restrict__ w, uint8_t* __restrict__ payload,
    float* __restrict__ scales, uint64_t nvec, uint64_t block_base) {
  quant_subgroup_body<BITS, G>(w, payload, scales, nvec, block_base + blockIdx.x);
}

// Several matrices of the same bits and group in one launch: the matrices'
// descriptors travel in the kernel arguments (a whole model's linear layers
// fit one launch); block b finds its matrix by a wave-uniform binary search
// over the first-block table and quantizes that matrix's block (b - first
// block).
struct QuantDesc {
  const float* w;
  uint8_t* payload;
  float* scales;
  uint64_t nvec;    // float4 vectors of the matrix
};
constexpr int QUANT_NB = QW_BATCH_PER_LAUNCH;
struct QuantBatch {
  uint32_t block0[QUANT_NB];  // first block of each matrix, ascending, block0[0] = 0
  QuantDesc d[QUANT_NB];
  int count;
  int blocks;
};

template <int BITS, int G>
__global__ __launch_bounds__(64 * QUANT_WAVES) void quant_subgroup_batched_kernel(const QuantBatch b) {
  typedef const __attribute__((address_space(4))) QuantBatch* KArg;
  const KArg kb = (KArg)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t blk = blockIdx.x;
  int lo = 0, hi = b.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kb->block0[mid] <= blk) lo = mid; else hi = mid - 1;
  }
  quant_subgroup_body<BITS, G>(kb->d[lo].w, kb->d[lo].payload, kb->d[lo].scales, kb->d[lo].nvec,
                               blk - kb->block0[lo]);
}

// ------------------------------------------------------------------- block

// One 256-thread block per group (group % 4 == 0, group <= 4 * 256 * QB_J):
// thread t owns vectors t, t + 256, ... of the group (coalesced loads), all
// held in registers between the block-wide max and the code pass.
template <int BITS>
__global__ __launch_bounds__(256) void quant_block_kernel(
    const float* __restrict__ w, uint8_t* __restrict__ payload,
    float* __restrict__ scales, int vpg /* float4 vectors per group */) {
  __shared__ float red[4];
  const uint64_t g = blockIdx.x;
  const uint64_t base = g * (uint64_t)vpg;  // first vector of this group
  const int tid = threadIdx.x;
  float v[QB_J][4];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < QB_J; ++j) {
    const int c = tid + 256 * j;
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < vpg) f = ldnt(reinterpret_cast<const float4*>(w) + base + c);
    v[j][0] = f.x; v[j][1] = f.y; v[j][2] = f.z; v[j][3] = f.w;
    m = fmaxf(m, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
  }
  m = run_max<64>(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = scale_of<BITS>(m);
  if (tid == 0) scales[g] = s;
#pragma unroll
  for (int j = 0; j < QB_J; ++j) {
    const int c = tid + 256 * j;
    if (c < vpg) {
      float r[4];
      rounded_quotients<BITS, 4>(v[j], s, r);
      if constexpr (BITS == 4)
        reinterpret_cast<uint16_t*>(payload)[base + c] = (uint16_t)pack4_int4(r);
      else
        reinterpret_cast<uint32_t*>(payload)[base + c] = pack4_int8(r);
    }
  }
}

// ----------------------------------------------------------------- generic

// Scales, one thread per group (small groups).
template <int BITS>
__global__ __launch_bounds__(256) void scales_thread_kernel(
    const float* __restrict__ w, float* __restrict__ scales, uint64_t ngroups,
    uint64_t group) {
  for (uint64_t g = (uint64_t)blockIdx.x * 256u + threadIdx.x; g < ngroups;
       g += (uint64_t)gridDim.x * 256u) {
    const float* p = w + g * group;
    float m = 0.0f;
    for (uint64_t i = 0; i < group; ++i) m = fmaxf(m, fabsf(p[i]));
    scales[g] = scale_of<BITS>(m);
  }
}

// Scales, one block per group (large groups).
template <int BITS>
__global__ __launch_bounds__(256) void scales_block_kernel(
    const float* __restrict__ w, float* __restrict__ scales, uint64_t ngroups,
    uint64_t group) {
  __shared__ float red[4];
  // block-uniform loop over the groups (grid-stride): every thread reaches
  // both barriers of every pass
  for (uint64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const float* p = w + g * group;
    float m = 0.0f;
    for (uint64_t i = threadIdx.x; i < group; i += 256) m = fmaxf(m, fabsf(p[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
      scales[g] = scale_of<BITS>(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    __syncthreads();  // red is rewritten by the next pass
  }
}

// Codes, one thread per payload byte.
template <int BITS>
__global__ __launch_bounds__(256) void codes_generic_kernel(
    const float* __restrict__ w, const float* __restrict__ scales,
    uint8_t* __restrict__ payload, uint64_t nbytes, uint64_t group) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < nbytes;
       i += (uint64_t)gridDim.x * 256u) {
    if (BITS == 8) {
      payload[i] = (uint8_t)(code_of<8>(w[i], scales[i / group]) & 255);
    } else {
      const uint64_t e0 = 2 * i, e1 = 2 * i + 1;
      const int q0 = code_of<4>(w[e0], scales[e0 / group]);
      const int q1 = code_of<4>(w[e1], scales[e1 / group]);
      payload[i] = (uint8_t)(((q0 + 8) & 15) | (((q1 + 8) & 15) << 4));
    }
  }
}

// ------------------------------------------------------------------ unpack

template <int BITS>
__device__ __forceinline__ int nibble_or_byte(uint32_t v, int i) {
  return BITS == 4 ? (int)((v >> (4 * i)) & 15u) - 8 : (int)(int8_t)(v >> (8 * i));
}

// Unpack, vector kernel: a wave owns 64*QV consecutive float4 outputs.  Its
// payload (2 or 4 bytes per vector) is read with one contiguous 8- or
// 16-byte load per lane and redistributed through LDS, so that lane l then
// produces vectors l, l + 64, ... and every output store instruction is a
// contiguous 1 KiB run (non-temporal).  The scale of vector v is
// scales[v >> vshift] (groups of a power-of-two number of vectors), else
// scales[v / vpg].
template <int BITS>
__device__ __forceinline__ void unpack_vec_body(
    const uint8_t* __restrict__ payload, const float* __restrict__ scales,
    float* __restrict__ out, uint64_t nvec, uint64_t vpg /* vectors per group */, int vshift,
    uint64_t block) {
  constexpr int PB = BITS / 2;  // payload bytes per vector
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * QV * PB];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const uint64_t base = (block * 4 + wv) * (64 * QV);
  const uint64_t v0 = base + (uint64_t)QV * lane;  // first vector of this lane's load
  if (v0 + QV <= nvec) {
    if constexpr (QV * PB == 8) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      reinterpret_cast<u32x2_la*>(stage[wv])[lane] =
          __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(payload + v0 * PB));
    } else {
      static_assert(QV * PB == 16, "QV * PB must be 8 or 16");
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      reinterpret_cast<u32x4_la*>(stage[wv])[lane] =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(payload + v0 * PB));
    }
  } else {
    for (int i = 0; i < QV * PB && v0 * PB + i < nvec * PB; ++i)
      stage[wv][QV * PB * lane + i] = payload[v0 * PB + i];
  }
  // (the wave's own LDS writes above complete before its reads below)
#pragma unroll
  for (int j = 0; j < QV; ++j) {
    const int vi = lane + 64 * j;
    const uint64_t idx = base + vi;
    if (idx >= nvec) continue;
    const float s = scales[vshift >= 0 ? (idx >> vshift) : idx / vpg];
    float v[4];
    if constexpr (BITS == 4) {
      const uint32_t p = reinterpret_cast<const u16_la*>(stage[wv])[vi];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (float)((int)((p >> (4 * i)) & 15u) - 8) * s;
    } else {
      const uint32_t p = reinterpret_cast<const u32_la*>(stage[wv])[vi];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (float)(int)(int8_t)(p >> (8 * i)) * s;
    }
    stnt(reinterpret_cast<float4*>(out) + idx, make_float4(v[0], v[1], v[2], v[3]));
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void unpack_vec_kernel(
    const uint8_t* __restrict__ payload, const float* __restrict__ scales,
    float* __restrict__ out, uint64_t nvec, uint64_t vpg, int vshift, uint64_t block_base) {
  unpack_vec_body<BITS>(payload, scales, out, nvec, vpg, vshift, block_base + blockIdx.x);
}

// Several matrices of one bit width in one launch (any groups the vector
// kernel takes), found like the batched quantize: descriptors in the kernel
// arguments, a wave-uniform binary search over the first-block table.
struct UnpackDesc {
  const uint8_t* payload;
  const float* scales;
  float* out;
  uint64_t nvec;    // float4 vectors of the matrix
  uint64_t vpg;     // vectors per group
  int vshift;       // log2(vpg) when vpg is a power of two, else -1
  int pad;
};
constexpr int UNPACK_NB = QW_BATCH_PER_LAUNCH;
struct UnpackBatch {
  uint32_t block0[UNPACK_NB];  // first block of each matrix, ascending, block0[0] = 0
  UnpackDesc d[UNPACK_NB];
  int count;
  int blocks;
};

template <int BITS>
__global__ __launch_bounds__(256) void unpack_vec_batched_kernel(const UnpackBatch b) {
  typedef const __attribute__((address_space(4))) UnpackBatch* KArg;
  const KArg kb = (KArg)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t blk = blockIdx.x;
  int lo = 0, hi = b.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kb->block0[mid] <= blk) lo = mid; else hi = mid - 1;
  }
  const auto& d = kb->d[lo];
  unpack_vec_body<BITS>(d.payload, d.scales, d.out, d.nvec, d.vpg, d.vshift, blk - kb->block0[lo]);
}

// One thread per weight; any group and alignment.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_generic_kernel(
    const uint8_t* __restrict__ payload, const float* __restrict__ scales,
    float* __restrict__ out, uint64_t count, uint64_t group) {
  for (uint64_t e = (uint64_t)blockIdx.x * 256u + threadIdx.x; e < count;
       e += (uint64_t)gridDim.x * 256u) {
    int q;
    if (BITS == 4) {
      const uint32_t b = payload[e >> 1];
      q = (int)((e & 1) ? (b >> 4) : (b & 15u)) - 8;
    } else {
      q = (int)(int8_t)payload[e];
    }
    out[e] = (float)q * scales[e / group];
  }
}

// Blocks of 256 threads for a grid-stride kernel over `threads` items: at
// most 2^20 (2^28 work-items, far inside one dispatch's 2^32).
inline unsigned blocks_for(uint64_t threads) {
  return (unsigned)std::min<uint64_t>((threads + 255) / 256, 1u << 20);
}

template <int BITS>
hipError_t quantize_bits(const Mat& mt, const float* w, uint8_t* payload, float* scales,
                         hipStream_t st) {
  const uint64_t count = (uint64_t)mt.n * (uint64_t)mt.k;
  const uint64_t group = (uint64_t)mt.group;
  const int path = quantize_path(mt, w, payload);
  if (path == PATH_FAST) {
    const uint64_t nvec = count / 4;
    const uint64_t bv = quant_block_vecs(mt.group);
    const uint64_t blocks = (nvec + bv - 1) / bv;
    // launches of at most kMaxLaunchBlocks blocks
    for (uint64_t b0 = 0; b0 < blocks; b0 += kMaxLaunchBlocks) {
      const unsigned grid = (unsigned)std::min<uint64_t>(blocks - b0, kMaxLaunchBlocks);
#define QW_QSUB(Gv) \
  quant_subgroup_kernel<BITS, Gv><<<grid, 64 * QUANT_WAVES, 0, st>>>(w, payload, scales, nvec, b0)
      switch (group / 4) {
        case 2: QW_QSUB(2); break;
        case 4: QW_QSUB(4); break;
        case 8: QW_QSUB(8); break;
        case 16: QW_QSUB(16); break;
        case 32: QW_QSUB(32); break;
        case 64: QW_QSUB(64); break;
        case 128: QW_QSUB(128); break;
        default: QW_QSUB(256); break;
      }
#undef QW_QSUB
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else if (path == PATH_BLOCK) {
    const uint64_t ngroups = count / group;
    quant_block_kernel<BITS><<<(unsigned)ngroups, 256, 0, st>>>(w, payload, scales, (int)(group / 4));
  } else {
    const uint64_t ngroups = count / group;
    if (group <= 64)
      scales_thread_kernel<BITS><<<blocks_for(ngroups), 256, 0, st>>>(w, scales, ngroups, group);
    else
      scales_block_kernel<BITS><<<(unsigned)std::min<uint64_t>(ngroups, 1u << 20), 256, 0, st>>>(
          w, scales, ngroups, group);
    const uint64_t nbytes = count * BITS / 8;
    codes_generic_kernel<BITS><<<blocks_for(nbytes), 256, 0, st>>>(w, scales, payload, nbytes, group);
  }
  return hipGetLastError();
}

// log2(vpg) for a power of two, else -1 (the kernel then divides).
inline int vec_shift(uint64_t vpg) {
  if ((vpg & (vpg - 1)) != 0) return -1;
  int v = 0;
  while ((1ull << v) < vpg) ++v;
  return v;
}

template <int BITS>
hipError_t unpack_bits(const Mat& mt, const uint8_t* payload, const float* scales, float* out,
                       hipStream_t st) {
  const uint64_t count = (uint64_t)mt.n * (uint64_t)mt.k;
  const uint64_t group = (uint64_t)mt.group;
  if (unpack_path(mt, payload, out) == PATH_FAST) {
    const uint64_t nvec = count / 4;
    const uint64_t blocks = (nvec + 4 * 64 * QV - 1) / (4 * 64 * QV);
    const uint64_t vpg = group / 4;
    const int vshift = vec_shift(vpg);
    for (uint64_t b0 = 0; b0 < blocks; b0 += kMaxLaunchBlocks) {
      const unsigned grid = (unsigned)std::min<uint64_t>(blocks - b0, kMaxLaunchBlocks);
      unpack_vec_kernel<BITS><<<grid, 256, 0, st>>>(payload, scales, out, nvec, vpg, vshift, b0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    unpack_generic_kernel<BITS><<<blocks_for(count), 256, 0, st>>>(payload, scales, out, count, group);
  }
  return hipGetLastError();
}

}  // namespace

int quantize_path(const Mat& mt, const float* w, const uint8_t* payload) {
  const uint64_t count = (uint64_t)mt.n * (uint64_t)mt.k;
  const uint64_t group = (uint64_t)mt.group;
  const bool al = aligned(w, 16) && aligned(payload, mt.bits == 4 ? 4 : 8);
  const bool pow2 = (group & (group - 1)) == 0;
  // (the block kernel takes one block per group: below 2^24 groups, every
  // launch stays within the 2^32 work-items of one dispatch)
  if (al && pow2 && group >= 8 && group <= 1024) return PATH_FAST;
  if (al && group % 4 == 0 && group <= 256u * 4u * QB_J && count / group < (1ull << 24))
    return PATH_BLOCK;
  return PATH_GENERIC;
}

int unpack_path(const Mat& mt, const uint8_t* payload, const float* w_out) {
  const bool al = aligned(w_out, 16) && aligned(payload, mt.bits == 4 ? 8 : 16);
  if (al && mt.group % 4 == 0) return PATH_FAST;
  return PATH_GENERIC;
}

hipError_t launch_quantize_pack(const Mat& mt, const float* w, uint8_t* payload, float* scales,
                                hipStream_t st) {
  return mt.bits == 4 ? quantize_bits<4>(mt, w, payload, scales, st)
                      : quantize_bits<8>(mt, w, payload, scales, st);
}

namespace {

template <int BITS, int G>
hipError_t launch_quant_batch(const QuantBatch& b, hipStream_t st) {
  quant_subgroup_batched_kernel<BITS, G><<<b.blocks, 64 * QUANT_WAVES, 0, st>>>(b);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_quant_batch_g(const QuantBatch& b, int64_t group, hipStream_t st) {
  switch (group / 4) {
    case 2: return launch_quant_batch<BITS, 2>(b, st);
    case 4: return launch_quant_batch<BITS, 4>(b, st);
    case 8: return launch_quant_batch<BITS, 8>(b, st);
    case 16: return launch_quant_batch<BITS, 16>(b, st);
    case 32: return launch_quant_batch<BITS, 32>(b, st);
    case 64: return launch_quant_batch<BITS, 64>(b, st);
    case 128: return launch_quant_batch<BITS, 128>(b, st);
    default: return launch_quant_batch<BITS, 256>(b, st);
  }
}

}  // namespace

hipError_t launch_quantize_pack_batched(const Mat* mts, const float* const* ws,
                                        uint8_t* const* payloads, float* const* scales,
                                        int count, hipStream_t st) {
  // Matrices that take the subgroup kernel are bucketed by (bits, group) and
  // launched QUANT_NB at a time; any other matrix is launched on its own.
  struct Bucket {
    int bits;
    int64_t group;
    std::vector<int> idx;
  };
  std::vector<Bucket> buckets;
  for (int i = 0; i < count; ++i) {
    if (mts[i].n * mts[i].k == 0) continue;
    if (quantize_path(mts[i], ws[i], payloads[i]) != PATH_FAST) {
      hipError_t e = launch_quantize_pack(mts[i], ws[i], payloads[i], scales[i], st);
      if (e != hipSuccess) return e;
      continue;
    }
    Bucket* bk = nullptr;
    for (auto& b : buckets)
      if (b.bits == mts[i].bits && b.group == mts[i].group) bk = &b;
    if (!bk) {
      buckets.push_back(Bucket{mts[i].bits, mts[i].group, {}});
      bk = &buckets.back();
    }
    bk->idx.push_back(i);
  }
  // a launch takes up to QUANT_NB matrices and at most 2^24 blocks (of 128
  // threads: far inside the 2^32 work-items of a dispatch)
  const uint64_t kMaxBlocks = 1ull << 24;
  for (const auto& bk : buckets) {
    size_t j = 0;
    while (j < bk.idx.size()) {
      QuantBatch b{};
      uint64_t blocks = 0;
      for (; j < bk.idx.size() && b.count < QUANT_NB; ++j) {
        const int i = bk.idx[j];
        const uint64_t nvec = (uint64_t)(mts[i].n * mts[i].k) / 4;
        const uint64_t bv = quant_block_vecs(bk.group);
        const uint64_t nblk = (nvec + bv - 1) / bv;
        if (nblk > kMaxBlocks) {  // too large for a shared launch: on its own
          const hipError_t e = launch_quantize_pack(mts[i], ws[i], payloads[i], scales[i], st);
          if (e != hipSuccess) return e;
          continue;
        }
        if (blocks + nblk > kMaxBlocks) break;  // next launch
        b.block0[b.count] = (uint32_t)blocks;
        QuantDesc& d = b.d[b.count++];
        d.w = ws[i];
        d.payload = payloads[i];
        d.scales = scales[i];
        d.nvec = nvec;
        blocks += nblk;
      }
      if (b.count == 0) continue;  // only matrices launched on their own
      b.blocks = (int)blocks;
      hipError_t e = bk.bits == 4 ? launch_quant_batch_g<4>(b, bk.group, st)
                                  : launch_quant_batch_g<8>(b, bk.group, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_unpack_batched(const Mat* mts, const uint8_t* const* payloads,
                                 const float* const* scales, float* const* outs, int count,
                                 hipStream_t st) {
  // vector-path matrices of one bit width go out UNPACK_NB per launch (and
  // at most 2^23 blocks of 256 threads); any other matrix takes the single call
  const uint64_t kMaxBlocks = 1ull << 23;
  for (int bits = 4; bits <= 8; bits += 4) {
    UnpackBatch b{};
    uint64_t blocks = 0;
    auto flush = [&]() -> hipError_t {
      if (b.count == 0) return hipSuccess;
      b.blocks = (int)blocks;
      if (bits == 4)
        unpack_vec_batched_kernel<4><<<(unsigned)blocks, 256, 0, st>>>(b);
      else
        unpack_vec_batched_kernel<8><<<(unsigned)blocks, 256, 0, st>>>(b);
      b.count = 0;
      blocks = 0;
      return hipGetLastError();
    };
    for (int i = 0; i < count; ++i) {
      if (mts[i].bits != bits || mts[i].n * mts[i].k == 0) continue;
      if (unpack_path(mts[i], payloads[i], outs[i]) != PATH_FAST) {
        hipError_t e = launch_unpack(mts[i], payloads[i], scales[i], outs[i], st);
        if (e != hipSuccess) return e;
        continue;
      }
      const uint64_t nvec = (uint64_t)(mts[i].n * mts[i].k) / 4;
      const uint64_t nblk = (nvec + 4 * 64 * QV - 1) / (4 * 64 * QV);
      if (nblk > kMaxBlocks) {  // too large for a shared launch: on its own
        hipError_t e = launch_unpack(mts[i], payloads[i], scales[i], outs[i], st);
        if (e != hipSuccess) return e;
        continue;
      }
      if (b.count == UNPACK_NB || blocks + nblk > kMaxBlocks) {
        hipError_t e = flush();
        if (e != hipSuccess) return e;
      }
      b.block0[b.count] = (uint32_t)blocks;
      UnpackDesc& d = b.d[b.count++];
      d.payload = payloads[i];
      d.scales = scales[i];
      d.out = outs[i];
      d.nvec = nvec;
      d.vpg = (uint64_t)mts[i].group / 4;
      d.vshift = vec_shift(d.vpg);
      d.pad = 0;
      blocks += nblk;
    }
    hipError_t e = flush();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_unpack(const Mat& mt, const uint8_t* payload, const float* scales, float* w_out,
                         hipStream_t st) {
  return mt.bits == 4 ? unpack_bits<4>(mt, payload, scales, w_out, st)
                      : unpack_bits<8>(mt, payload, scales, w_out, st);
}

}  // namespace qw
