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
//   subgroup  group = 8*L, L in {1,2,...,64}: each lane owns 8 consecutive
//             weights (two 16-byte loads); the L lanes of a group reduce
//             max|w| with cross-lane shuffles.  One pass, fully coalesced.
//   block     group % 8 == 0 and group <= 256*8*QB_J: one 256-thread block
//             per group; weights stay in registers between the max and the
//             code pass.
//   generic   any group dividing n*k, any alignment: a scale kernel (one
//             thread or one block per group) then a code kernel (one thread
//             per payload byte).
#include "qw_internal.h"

namespace qw {
namespace {

constexpr int QB_J = 8;  // chunks of 8 weights per thread in the block kernel

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Pack 8 consecutive codes and store them at chunk index `c`.
template <int BITS>
__device__ __forceinline__ void store_chunk(uint8_t* payload, uint64_t c, const int (&q)[8]) {
  if (BITS == 4) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v |= (uint32_t)((q[i] + 8) & 15) << (4 * i);
    reinterpret_cast<uint32_t*>(payload)[c] = v;
  } else {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= (uint32_t)(q[i] & 255) << (8 * i);
      hi |= (uint32_t)(q[4 + i] & 255) << (8 * i);
    }
    reinterpret_cast<uint2*>(payload)[c] = make_uint2(lo, hi);
  }
}

__device__ __forceinline__ float absmax8(const float4& a, const float4& b) {
  float m = fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
  return fmaxf(m, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

template <int BITS>
__device__ __forceinline__ void quantize8(const float4& a, const float4& b, float s, int (&q)[8]) {
  q[0] = code_of<BITS>(a.x, s); q[1] = code_of<BITS>(a.y, s);
  q[2] = code_of<BITS>(a.z, s); q[3] = code_of<BITS>(a.w, s);
  q[4] = code_of<BITS>(b.x, s); q[5] = code_of<BITS>(b.y, s);
  q[6] = code_of<BITS>(b.z, s); q[7] = code_of<BITS>(b.w, s);
}

// ---------------------------------------------------------------- subgroup

template <int BITS, int L>
__global__ __launch_bounds__(256) void quant_subgroup_kernel(
    const float* __restrict__ w, uint8_t* __restrict__ payload,
    float* __restrict__ scales, uint64_t nchunks) {
  const uint64_t t = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  const bool active = t < nchunks;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  if (active) {
    const float4* p = reinterpret_cast<const float4*>(w) + 2 * t;
    a = ldnt(p);
    b = ldnt(p + 1);
  }
  float m = absmax8(a, b);
  // Groups never straddle the active / inactive boundary (nchunks is a
  // multiple of L), so inactive lanes only meet inactive lanes here.
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float s = scale_of<BITS>(m);
  if (!active) return;
  if ((t & (L - 1)) == 0) scales[t / L] = s;
  int q[8];
  quantize8<BITS>(a, b, s, q);
  store_chunk<BITS>(payload, t, q);
}

// ------------------------------------------------------------------- block

template <int BITS>
__global__ __launch_bounds__(256) void quant_block_kernel(
    const float* __restrict__ w, uint8_t* __restrict__ payload,
    float* __restrict__ scales, int cpg /* chunks of 8 per group */) {
  __shared__ float red[4];
  const uint64_t g = blockIdx.x;
  const uint64_t base = g * (uint64_t)cpg;  // first chunk of this group
  const int tid = threadIdx.x;
  float4 a[QB_J], b[QB_J];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < QB_J; ++j) {
    const int c = tid + 256 * j;
    a[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    b[j] = a[j];
    if (c < cpg) {
      const float4* p = reinterpret_cast<const float4*>(w) + 2 * (base + c);
      a[j] = ldnt(p);
      b[j] = ldnt(p + 1);
    }
    m = fmaxf(m, absmax8(a[j], b[j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = scale_of<BITS>(m);
  if (tid == 0) scales[g] = s;
#pragma unroll
  for (int j = 0; j < QB_J; ++j) {
    const int c = tid + 256 * j;
    if (c < cpg) {
      int q[8];
      quantize8<BITS>(a[j], b[j], s, q);
      store_chunk<BITS>(payload, base + c, q);
    }
  }
}

// ----------------------------------------------------------------- generic

// Scales, one thread per group (small groups).
template <int BITS>
__global__ __launch_bounds__(256) void scales_thread_kernel(
    const float* __restrict__ w, float* __restrict__ scales, uint64_t ngroups,
    uint64_t group) {
  const uint64_t g = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (g >= ngroups) return;
  const float* p = w + g * group;
  float m = 0.0f;
  for (uint64_t i = 0; i < group; ++i) m = fmaxf(m, fabsf(p[i]));
  scales[g] = scale_of<BITS>(m);
}

// Scales, one block per group (large groups).
template <int BITS>
__global__ __launch_bounds__(256) void scales_block_kernel(
    const float* __restrict__ w, float* __restrict__ scales, uint64_t group) {
  __shared__ float red[4];
  const uint64_t g = blockIdx.x;
  const float* p = w + g * group;
  float m = 0.0f;
  for (uint64_t i = threadIdx.x; i < group; i += 256) m = fmaxf(m, fabsf(p[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    scales[g] = scale_of<BITS>(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
}

// Codes, one thread per payload byte.
template <int BITS>
__global__ __launch_bounds__(256) void codes_generic_kernel(
    const float* __restrict__ w, const float* __restrict__ scales,
    uint8_t* __restrict__ payload, uint64_t nbytes, uint64_t group) {
  const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (i >= nbytes) return;
  if (BITS == 8) {
    payload[i] = (uint8_t)(code_of<8>(w[i], scales[i / group]) & 255);
  } else {
    const uint64_t e0 = 2 * i, e1 = 2 * i + 1;
    const int q0 = code_of<4>(w[e0], scales[e0 / group]);
    const int q1 = code_of<4>(w[e1], scales[e1 / group]);
    payload[i] = (uint8_t)(((q0 + 8) & 15) | (((q1 + 8) & 15) << 4));
  }
}

// ------------------------------------------------------------------ unpack

template <int BITS>
__device__ __forceinline__ int nibble_or_byte(uint32_t v, int i) {
  return BITS == 4 ? (int)((v >> (4 * i)) & 15u) - 8 : (int)(int8_t)(v >> (8 * i));
}

// One thread per chunk of 8 weights; group % 8 == 0.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_chunk_kernel(
    const uint8_t* __restrict__ payload, const float* __restrict__ scales,
    float* __restrict__ out, uint64_t nchunks, uint64_t cpg) {
  const uint64_t t = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (t >= nchunks) return;
  const float s = scales[t / cpg];
  float v[8];
  if (BITS == 4) {
    const uint32_t p = reinterpret_cast<const uint32_t*>(payload)[t];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)nibble_or_byte<4>(p, i) * s;
  } else {
    const uint2 p = reinterpret_cast<const uint2*>(payload)[t];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (float)nibble_or_byte<8>(p.x, i) * s;
      v[4 + i] = (float)nibble_or_byte<8>(p.y, i) * s;
    }
  }
  float4* o = reinterpret_cast<float4*>(out) + 2 * t;
  stnt(o, make_float4(v[0], v[1], v[2], v[3]));
  stnt(o + 1, make_float4(v[4], v[5], v[6], v[7]));
}

// One thread per weight; any group and alignment.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_generic_kernel(
    const uint8_t* __restrict__ payload, const float* __restrict__ scales,
    float* __restrict__ out, uint64_t count, uint64_t group) {
  const uint64_t e = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (e >= count) return;
  int q;
  if (BITS == 4) {
    const uint32_t b = payload[e >> 1];
    q = (int)((e & 1) ? (b >> 4) : (b & 15u)) - 8;
  } else {
    q = (int)(int8_t)payload[e];
  }
  out[e] = (float)q * scales[e / group];
}

inline unsigned blocks_for(uint64_t threads) { return (unsigned)((threads + 255) / 256); }

template <int BITS>
hipError_t quantize_bits(const Mat& mt, const float* w, uint8_t* payload, float* scales,
                         hipStream_t st) {
  const uint64_t count = (uint64_t)mt.n * (uint64_t)mt.k;
  const uint64_t group = (uint64_t)mt.group;
  const int path = quantize_path(mt, w, payload);
  if (path == PATH_FAST) {
    const uint64_t nchunks = count / 8;
    const unsigned grid = blocks_for(nchunks);
    switch (group / 8) {
      case 1: quant_subgroup_kernel<BITS, 1><<<grid, 256, 0, st>>>(w, payload, scales, nchunks); break;
      case 2: quant_subgroup_kernel<BITS, 2><<<grid, 256, 0, st>>>(w, payload, scales, nchunks); break;
      case 4: quant_subgroup_kernel<BITS, 4><<<grid, 256, 0, st>>>(w, payload, scales, nchunks); break;
      case 8: quant_subgroup_kernel<BITS, 8><<<grid, 256, 0, st>>>(w, payload, scales, nchunks); break;
      case 16: quant_subgroup_kernel<BITS, 16><<<grid, 256, 0, st>>>(w, payload, scales, nchunks); break;
      case 32: quant_subgroup_kernel<BITS, 32><<<grid, 256, 0, st>>>(w, payload, scales, nchunks); break;
      default: quant_subgroup_kernel<BITS, 64><<<grid, 256, 0, st>>>(w, payload, scales, nchunks); break;
    }
  } else if (path == PATH_BLOCK) {
    const uint64_t ngroups = count / group;
    quant_block_kernel<BITS><<<(unsigned)ngroups, 256, 0, st>>>(w, payload, scales, (int)(group / 8));
  } else {
    const uint64_t ngroups = count / group;
    if (group <= 64)
      scales_thread_kernel<BITS><<<blocks_for(ngroups), 256, 0, st>>>(w, scales, ngroups, group);
    else
      scales_block_kernel<BITS><<<(unsigned)ngroups, 256, 0, st>>>(w, scales, group);
    const uint64_t nbytes = count * BITS / 8;
    codes_generic_kernel<BITS><<<blocks_for(nbytes), 256, 0, st>>>(w, scales, payload, nbytes, group);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t unpack_bits(const Mat& mt, const uint8_t* payload, const float* scales, float* out,
                       hipStream_t st) {
  const uint64_t count = (uint64_t)mt.n * (uint64_t)mt.k;
  const uint64_t group = (uint64_t)mt.group;
  if (unpack_path(mt, payload, out) == PATH_FAST) {
    const uint64_t nchunks = count / 8;
    unpack_chunk_kernel<BITS><<<blocks_for(nchunks), 256, 0, st>>>(payload, scales, out, nchunks, group / 8);
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
  const uint64_t blocks_needed = (count / 8 + 255) / 256;
  if (al && group % 8 == 0 && group <= 512 && ((group / 8) & (group / 8 - 1)) == 0 &&
      blocks_needed < (1ull << 31))
    return PATH_FAST;
  if (al && group % 8 == 0 && group <= 256u * 8u * QB_J && count / group < (1ull << 31))
    return PATH_BLOCK;
  return PATH_GENERIC;
}

int unpack_path(const Mat& mt, const uint8_t* payload, const float* w_out) {
  const uint64_t count = (uint64_t)mt.n * (uint64_t)mt.k;
  const bool al = aligned(w_out, 16) && aligned(payload, mt.bits == 4 ? 4 : 8);
  if (al && mt.group % 8 == 0 && (count / 8 + 255) / 256 < (1ull << 31)) return PATH_FAST;
  return PATH_GENERIC;
}

hipError_t launch_quantize_pack(const Mat& mt, const float* w, uint8_t* payload, float* scales,
                                hipStream_t st) {
  return mt.bits == 4 ? quantize_bits<4>(mt, w, payload, scales, st)
                      : quantize_bits<8>(mt, w, payload, scales, st);
}

hipError_t launch_unpack(const Mat& mt, const uint8_t* payload, const float* scales, float* w_out,
                         hipStream_t st) {
  return mt.bits == 4 ? unpack_bits<4>(mt, payload, scales, w_out, st)
                      : unpack_bits<8>(mt, payload, scales, w_out, st);
}

}  // namespace qw
