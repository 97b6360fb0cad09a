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
//     buffered, rows padded to 144 bytes so that the fragment reads (16
//     consecutive rows per phase, same k) hit distinct banks.
//   * Weight fragments come straight from global memory: within one MFMA the
//     k-slots are a free permutation shared by A and B, so lane group g
//     (lanes 32g..32g+31) takes the contiguous k range [32g, 32g+32) of the
//     step -- 16 bytes of int4 payload (32 for int8) of one output row per
//     lane -- and the matching X values.  The lane decodes its codes once
//     per step into fl32(q * S) and rounds them to bf16 (RNE): an int4 code
//     takes one FMA on its exact fp8 nibble conversion (an int8 code, a
//     sign-extending conversion and a multiply).
//   * Block order is XCD-aware: blocks land on the 8 XCDs round-robin, so
//     consecutive blocks of one XCD walk all M tiles of one N tile (the
//     weight tile stays in that XCD's L2 while the M tiles reuse it).
#include "qw_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace qw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
// Rows of X up to which the small-M kernel runs: up to kSmallMaxM always, up
// to kSmallMaxMNarrow when the weight has at most kNarrowN rows (output
// columns), where the 256 x 256 tiles leave most compute units idle.
// Measured (us, 256-row tiles / small-M kernel, int4 g128): 28672 x 8192 at
// M = 64 121 / 93, 80 124 / 125, 96 126 / 135; 16384 x 8192 at M = 96
// 102 / 73, 128 104 / 94; 11008 x 4096 at M = 128 61 / 41; 4096 x 11008 at
// M = 128 120 / 38.
constexpr int kSmallMaxM = 64;
constexpr int kSmallMaxMNarrow = 128;
constexpr int64_t kNarrowN = 16384;
// LDS row stride of the X tile: 128 bytes of data + 16 bytes of padding, so
// that 16 consecutive rows (one 16-lane phase of a ds_read_b128) start 36
// dwords apart and cover 16 distinct 4-bank groups of the 64 banks.
constexpr int XS = BK * 2 + 16;

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
  // Scale index within a row, kk / group for kk < 2^31 and group >= 2, without a
  // division: t = umulhi(kk, gdiv_mul), q = (t + ((kk - t) >> 1)) >> (gdiv_shift - 1)
  // (Granlund and Montgomery, "Division by invariant integers using
  // multiplication", 1994).  gmask is 0 when a whole row shares one scale.
  uint32_t gdiv_mul, gdiv_shift, gmask;
  int tiles_m, tiles_n;
  int xcd_map;          // 1: XCD-aware tile order
  // Tiles [0, full_tiles) take one block each.  Every later tile takes two
  // blocks, one per half of the k-steps (the first nk_lo steps, then the
  // rest), which add their partial sums into Y (zeroed beforehand).
  int full_tiles;
  int nk_lo;
  // Small-M kernel: codes per scale along a row when that is a multiple of
  // the k-step (a k-step then inside one group, so a step that does not start
  // a group reuses the previous step's scales); 0 = load them every step.
  int64_t scale_period;
};

// Tile index -> (tile row, tile column).  With the XCD-aware order, tiles
// t, t+8, t+16, ... (dispatched to one XCD) walk all M tiles of one N tile,
// so that XCD's L2 keeps the weight tile while the M tiles reuse it.
__device__ __forceinline__ void tile_coords(const GemmArgs& a, int t, int& tm, int& tn) {
  if (a.xcd_map) {
    const int xcd = t & 7, j = t >> 3;
    tm = j % a.tiles_m;
    tn = xcd + 8 * (j / a.tiles_m);
  } else {
    tm = t % a.tiles_m;
    tn = t / a.tiles_m;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// 8 int4 codes (one dword, element order) -> bf16(fl32(q * s)), packed in 4 dwords.
__device__ __forceinline__ u32x4 dequant8_int4(uint32_t w, float s) {
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
  return u32x4{pack_bf16x2(q0, q1), pack_bf16x2(q2, q3), pack_bf16x2(q4, q5),
               pack_bf16x2(q6, q7)};
}

// 8 int8 codes (two dwords, element order) -> 4 dwords of bf16 pairs.
__device__ __forceinline__ u32x4 dequant8_int8(uint32_t w0, uint32_t w1, float s) {
  const float q0 = (float)(int)(int8_t)(w0) * s;
  const float q1 = (float)(int)(int8_t)(w0 >> 8) * s;
  const float q2 = (float)(int)(int8_t)(w0 >> 16) * s;
  const float q3 = (float)((int)w0 >> 24) * s;
  const float q4 = (float)(int)(int8_t)(w1) * s;
  const float q5 = (float)(int)(int8_t)(w1 >> 8) * s;
  const float q6 = (float)(int)(int8_t)(w1 >> 16) * s;
  const float q7 = (float)((int)w1 >> 24) * s;
  return u32x4{pack_bf16x2(q0, q1), pack_bf16x2(q2, q3), pack_bf16x2(q4, q5),
               pack_bf16x2(q6, q7)};
}

// One-FMA int4 decode.  Scales of magnitude below this limit keep 512 * s
// finite, and the decoder below then returns exactly the values of the
// two-step one above; a block that meets a larger scale recomputes its tile
// with the two-step decoder.  (int8 keeps the two-step decoder: there the
// sign-extending byte conversion is already one instruction, so an FMA form
// saves nothing.)
constexpr float kFmaScaleLimit = 0x1p118f;

// 8 int4 codes -> bf16(fl32(q * s)), one FMA per code: the fp8 conversion
// gives u * 2^-9 exactly (u = q + 8), and fma(u * 2^-9, 512 * s, -8 * s)
// forms the exact value (u - 8) * s = q * s before its single rounding.
__device__ __forceinline__ u32x4 dequant8_int4_fma(uint32_t w, float s512, float ns8) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);  // e0, e2
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);   // e4, e6
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);  // e1, e3
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);   // e5, e7
  return u32x4{pack_bf16x2(__builtin_fmaf(a.x, s512, ns8), __builtin_fmaf(c.x, s512, ns8)),
               pack_bf16x2(__builtin_fmaf(a.y, s512, ns8), __builtin_fmaf(c.y, s512, ns8)),
               pack_bf16x2(__builtin_fmaf(b.x, s512, ns8), __builtin_fmaf(d.x, s512, ns8)),
               pack_bf16x2(__builtin_fmaf(b.y, s512, ns8), __builtin_fmaf(d.y, s512, ns8))};
}

// Workgroup barrier for LDS hand-off only: wait for this wave's LDS
// accesses, then s_barrier.  (__syncthreads also waits for every
// outstanding global load, which would drain the prefetch pipeline below.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Scheduling patterns (group masks: 0x002 VALU, 0x008 MFMA, 0x020 global
// load, 0x100 LDS read, 0x200 LDS write).
// Sub-step with the X hand-off: 8 A reads, then MFMAs interleaved with the
// 8 LDS stores of X and the 8 global loads that refill its registers.
__device__ __forceinline__ void sched_substep_x() {
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
}
// Sub-step with NV VALU instructions after each MFMA and NG global loads at the end.
template <int NV, int NG>
__device__ __forceinline__ void sched_substep() {
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
  if constexpr (NG > 0) __builtin_amdgcn_sched_group_barrier(0x020, NG, 0);
}

template <int BITS>
struct BRegs {
  // raw payload of the lane's 32 codes for one N block
  u32x4 p[BITS == 4 ? 1 : 2];
  float s;
};

// The lane's 32 codes of one column block -> its 4 B fragments (bf16 pairs,
// one per k = 16 sub-step).  FMA (int4 only): the one-FMA decoder, for |s|
// below kFmaScaleLimit; else the two-step decoders (any scale).
template <int BITS, bool FMA>
__device__ __forceinline__ void dequant32(const BRegs<BITS>& br, float s, u32x4 (&bq)[4]) {
  static_assert(BITS == 4 || !FMA, "the one-FMA decoder is int4 only");
  if constexpr (BITS == 4) {
    const u32x4 p = br.p[0];
    if constexpr (FMA) {
      const float s512 = s * 512.0f, ns8 = s * -8.0f;
      bq[0] = dequant8_int4_fma(p.x, s512, ns8);
      bq[1] = dequant8_int4_fma(p.y, s512, ns8);
      bq[2] = dequant8_int4_fma(p.z, s512, ns8);
      bq[3] = dequant8_int4_fma(p.w, s512, ns8);
    } else {
      bq[0] = dequant8_int4(p.x, s);
      bq[1] = dequant8_int4(p.y, s);
      bq[2] = dequant8_int4(p.z, s);
      bq[3] = dequant8_int4(p.w, s);
    }
  } else {
    const u32x4 p0 = br.p[0], p1 = br.p[1];
    bq[0] = dequant8_int8(p0.x, p0.y, s);
    bq[1] = dequant8_int8(p0.z, p0.w, s);
    bq[2] = dequant8_int8(p1.x, p1.y, s);
    bq[3] = dequant8_int8(p1.z, p1.w, s);
  }
}

// Software pipeline.  A k-step (BK = 64) is four sub-steps of k = 16; one
// sub-step is 16 MFMAs per wave (8 row blocks x 2 column blocks).  Per
// k-step ks, with the X tile double-buffered in LDS (buffer ks&1), the A
// fragments double-buffered in registers and the dequantized B fragments of
// two k-steps in registers:
//   sub-step 0: store X(ks+1) (loaded one k-step ago) into LDS buffer
//               (ks+1)&1, issue the loads of X(ks+2);
//   sub-step 1: dequantize the first column block of W(ks+1);
//   sub-step 2: dequantize the second one, issue the loads of W(ks+3) into
//               the registers just freed, then the k-step's only barrier;
//   sub-step 3: (after the barrier) read A(ks+1, sub-step 0).
// Every sub-step also reads the next sub-step's A fragments from LDS while
// its MFMAs run.  A buffer is rewritten (sub-step 0 of step ks+2) only after
// the barrier of step ks+1, which every wave reaches after its last read of
// it (sub-step 2 of step ks), so one barrier per k-step suffices.  Loads past
// the last k-step re-read the last one (their results are never used), so
// the loop body has no branches and the compiler's wait counts stay exact.
template <int BITS>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BM * XS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;    // lane group: k range [32g, 32g+32) of a step
  const int l32 = lane & 31;

  // ---- block -> tile and k-step range
  int t, kbeg, kend;
  bool split;
  {
    const int b = blockIdx.x;
    const int nk = a.k / BK;
    if (b < a.full_tiles) {
      t = b;
      kbeg = 0;
      kend = nk;
      split = false;
    } else {
      const int i = b - a.full_tiles;
      t = a.full_tiles + (i >> 1);
      kbeg = (i & 1) ? a.nk_lo : 0;
      kend = (i & 1) ? nk : a.nk_lo;
      split = true;
    }
  }
  int tm, tn;
  tile_coords(a, t, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int nsteps = kend - kbeg;
  const int kfirst = kbeg * BK;
  const int klast = (kend - 1) * BK;

  // ---- per-lane weight rows (two 32-column blocks per wave)
  bool nvalid[2];
  const uint8_t* prow[2];
  const float* srow[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int nn = n0 + 64 * wave + 32 * nb + l32;
    nvalid[nb] = nn < a.n;
    const int row = nvalid[nb] ? nn : a.n - 1;
    prow[nb] = a.payload + (int64_t)row * a.row_stride_b + 16 * g * (BITS / 4);
    srow[nb] = a.scales + (a.per_row_groups ? (int64_t)row * a.groups_per_row
                                            : ((int64_t)row * a.k) / a.group);
  }
  // ---- per-thread X chunks: chunk i = tile row (tid>>3) + 32*i, 16-byte column tid&7.
  // Rows past the end of X (last M tile only) re-read row m-1; their outputs are never
  // stored.
  const uint16_t* xrow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t mm = m0 + (tid >> 3) + 32 * i;
    xrow[i] = a.x + (mm < a.m ? mm : a.m - 1) * a.k + (tid & 7) * 8;
  }
  const int wr_off = (tid >> 3) * XS + (tid & 7) * 16;   // + i * 32 * XS
  const int rd_off = l32 * XS + g * 64;                  // + mb * 32 * XS + s * 16

  auto load_x = [&](u32x4 (&xa)[8], int k0) __attribute__((always_inline)) {
    k0 = k0 < klast ? k0 : klast;
#pragma unroll
    for (int i = 0; i < 8; ++i) xa[i] = *reinterpret_cast<const u32x4*>(xrow[i] + k0);
  };
  auto store_x = [&](const u32x4 (&xv)[8], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(&lds[buf * (BM * XS) + wr_off + i * 32 * XS]) = xv[i];
  };
  auto load_w = [&](BRegs<BITS> (&br)[2], int k0) __attribute__((always_inline)) {
    k0 = k0 < klast ? k0 : klast;
    const uint32_t kk = (uint32_t)(k0 + 32 * g);  // first code of this lane's range
    const uint32_t t = __umulhi(kk, a.gdiv_mul);
    const uint32_t gi = ((t + ((kk - t) >> 1)) >> (a.gdiv_shift - 1)) & a.gmask;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint8_t* src = prow[nb] + (int64_t)k0 * BITS / 8;
      br[nb].p[0] = *reinterpret_cast<const u32x4*>(src);
      if constexpr (BITS == 8) br[nb].p[1] = *reinterpret_cast<const u32x4*>(src + 16);
      br[nb].s = srow[nb][gi];
    }
  };
  // Largest |scale| this wave decoded with the one-FMA decoder.
  float smax = 0.0f;
  auto dequant_nb = [&](auto fma, const BRegs<BITS>& br, u32x4 (&bq)[4])
      __attribute__((always_inline)) {
    constexpr bool F = decltype(fma)::value;
    if constexpr (F) smax = fmaxf(smax, fabsf(br.s));
    dequant32<BITS, F>(br, br.s, bq);
  };
  auto read_a = [&](u32x4 (&af)[8], int buf, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      af[mb] = *reinterpret_cast<const u32x4*>(
          &lds[buf * (BM * XS) + rd_off + mb * 32 * XS + s * 16]);
  };

  f32x16 acc[8][2];
  auto mfma16 = [&](const u32x4 (&af)[8], const u32x4 (&bq)[2][4], int s)
      __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, af[mb]), __builtin_bit_cast(bf16x8, bq[nb][s]),
            acc[mb][nb], 0, 0, 0);
  };

  // The tile's whole k loop, with the one-FMA int4 decoder (fma = true) or
  // the two-step decoders.  VALU instructions placed after each MFMA of the
  // two decoding sub-steps (the one-FMA decoder issues about 5 per MFMA
  // there, the two-step ones about 7; measured on the 70B MLP shape, 6 runs
  // fastest for the former, within 0.4% of 5, 2% ahead of 4 and 7).
  auto run = [&](auto fma) __attribute__((always_inline)) {
    constexpr bool F = decltype(fma)::value;
    constexpr int NV1 = F ? 6 : 8, NV2 = F ? 6 : 8;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // ---- prologue: X(0) in LDS buffer 0, X(1) in flight, B(0) dequantized, W(1) and
    // W(2) in flight, A(0, sub-step 0) in registers.
    u32x4 xa[8];
    BRegs<BITS> brE[2], brO[2];   // raw W of even / odd k-steps
    u32x4 bqE[2][4], bqO[2][4];   // dequantized B of even / odd k-steps
    u32x4 af0[8], af1[8];
    load_x(xa, kfirst);
    load_w(brE, kfirst);
    load_w(brO, kfirst + BK);
    store_x(xa, 0);
    load_x(xa, kfirst + BK);
    dequant_nb(fma, brE[0], bqE[0]);
    dequant_nb(fma, brE[1], bqE[1]);
    load_w(brE, kfirst + 2 * BK);
    lds_barrier();
    read_a(af0, 0, 0);

    // One k-step (i = local step number).  bq_cur = B(i); br_nxt = W(i+1), refilled with
    // W(i+3); bq_nxt <- B(i+1).
    auto kstep = [&](int i, const u32x4 (&bq_cur)[2][4], BRegs<BITS> (&br_nxt)[2],
                     u32x4 (&bq_nxt)[2][4]) __attribute__((always_inline)) {
      const int cur = i & 1, nxt = cur ^ 1;
      // sub-step 0
      read_a(af1, cur, 1);
      store_x(xa, nxt);
      load_x(xa, kfirst + (i + 2) * BK);
      mfma16(af0, bq_cur, 0);
      sched_substep_x();
      __builtin_amdgcn_sched_barrier(0);
      // sub-step 1
      read_a(af0, cur, 2);
      dequant_nb(fma, br_nxt[0], bq_nxt[0]);
      mfma16(af1, bq_cur, 1);
      sched_substep<NV1, 0>();
      __builtin_amdgcn_sched_barrier(0);
      // sub-step 2
      read_a(af1, cur, 3);
      dequant_nb(fma, br_nxt[1], bq_nxt[1]);
      load_w(br_nxt, kfirst + (i + 3) * BK);
      mfma16(af0, bq_cur, 2);
      sched_substep<NV2, 6>();
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      // sub-step 3
      read_a(af0, nxt, 0);
      mfma16(af1, bq_cur, 3);
      sched_substep<2, 0>();
      __builtin_amdgcn_sched_barrier(0);
    };
    int i = 0;
    for (; i + 1 < nsteps; i += 2) {
      kstep(i, bqE, brO, bqO);
      kstep(i + 1, bqO, brE, bqE);
    }
    if (i < nsteps) kstep(i, bqE, brO, bqO);
  };
  if constexpr (BITS == 4) {
    run(std::true_type{});
    // A scale too large for the one-FMA decoder anywhere in the block: the
    // whole block recomputes its tile with the two-step decoder (the LDS
    // buffers are free again once every wave has passed the barrier here).
    if (__syncthreads_or(smax >= kFmaScaleLimit)) run(std::false_type{});
  } else {
    run(std::false_type{});
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
        if (mm < a.m) {
          if (split)
            unsafeAtomicAdd(&a.y[mm * a.n + nn], acc[mb][nb][r]);
          else
            __builtin_nontemporal_store(acc[mb][nb][r], &a.y[mm * a.n + nn]);
        }
      }
    }
}

// Zeroes the output tiles that two blocks accumulate into: block (tile
// t = full_tiles + blockIdx.x / 16, 16-row slab blockIdx.x % 16).
__global__ __launch_bounds__(256) void gemm_zero_split_tiles(GemmArgs a) {
  const int t = a.full_tiles + (int)(blockIdx.x >> 4);
  int tm, tn;
  tile_coords(a, t, tm, tn);
  const int nn = tn * BN + (int)threadIdx.x;
  if (nn >= a.n) return;
  const int64_t r0 = (int64_t)tm * BM + 16 * (blockIdx.x & 15);
#pragma unroll 4
  for (int r = 0; r < 16; ++r)
    if (r0 + r < a.m) a.y[(r0 + r) * a.n + nn] = 0.0f;
}

// ------------------------------------------------------------ small-M kernel

// GEMM for few rows of X (decode batches, short prompts): an output tile of
// 32*MB rows x 32*NBW columns per block, its K split over the block's 4
// waves (contiguous quarters of the k-steps).  A wave reads its A fragments
// straight from global memory (X is small and cache-resident), dequantizes
// its own weights once (the same register recipe as the large kernel) and
// keeps 32*MB x 32*NBW fp32 accumulators; the four partial tiles meet in LDS
// and are added in wave order (deterministic).  The work is bound by
// streaming and dequantizing the weights, not by the matrix cores, so the
// tile is small enough to give every compute unit blocks.
template <int BITS, int MB, int NBW>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmArgs a) {
  constexpr int TILE = 32 * MB * 32 * NBW;  // outputs per block
  __shared__ float red[3][TILE];            // partial tiles of waves 1..3
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int tm = blockIdx.x % a.tiles_m;
  const int tn = blockIdx.x / a.tiles_m;
  const int64_t m0 = (int64_t)tm * 32 * MB;
  const int n0 = tn * 32 * NBW;
  const int nk = a.k / BK;
  const int q = (nk + 3) >> 2;
  const int ks0 = min(nk, wave * q);
  const int ks1 = min(nk, ks0 + q);

  // Weights.  A super-step is the k-steps whose codes fill 128 bytes of a row
  // (4 int4 k-steps, 2 int8 ones).  The wave loads a super-step's weights
  // row-contiguously -- lane L takes the 16 bytes at 16*(L%8) of rows L/8,
  // L/8 + 8, L/8 + 16, L/8 + 24 of each 32-row column block, 8 whole rows
  // per load instruction -- one super-step ahead, stages them in its own LDS
  // region and reads back its MFMA fragments there (lane l: row l%32, k range
  // [32g, 32g+32) of each k-step).  Loading the fragments straight from
  // memory touched 32 rows per instruction.  A piece past the end of its row
  // (a short row, or a super-step past the last k-step) is clamped onto the
  // row's last 16 bytes; such pieces are never read back.
  constexpr int SS = 128 / (BK * BITS / 8);       // k-steps per super-step
  constexpr int SP = 128 + 16;                    // LDS row pitch (bank spread)
  constexpr int FB = 16 * (BITS / 4);             // fragment bytes per lane and k-step
  __shared__ __attribute__((aligned(16))) uint8_t wst[4][NBW][32 * SP];
  const int prow_bytes = a.row_stride_b;
  const uint8_t* lrow[NBW][4];                    // rows this lane loads
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nn = min(n0 + 32 * nb + (lane >> 3) + 8 * j, a.n - 1);
      lrow[nb][j] = a.payload + (int64_t)nn * prow_bytes;
    }
  const float* srow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int nn = min(n0 + 32 * nb + l32, a.n - 1);
    srow[nb] = a.scales + (a.per_row_groups ? (int64_t)nn * a.groups_per_row
                                            : ((int64_t)nn * a.k) / a.group);
  }
  // X rows of the lane's A fragments (rows past M re-read row M-1)
  const uint16_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t mm = m0 + 32 * mb + l32;
    xrow[mb] = a.x + (mm < a.m ? mm : a.m - 1) * a.k + 32 * g;
  }
  // last k-step a load may touch (idle waves, ks0 == nk, still issue the prologue loads)
  const int klast = min(nk - 1, max(ks0, ks1 - 1)) * BK;

  // Scales: a k-step that starts no group (inside one scale period) keeps the
  // scales of the step before, so only steps that start a group load them.
  // kin_load / kin_use: position inside the period of the next step loaded /
  // dequantized (wave-uniform; both advance one k-step per call, in order).
  const int64_t kin0 = a.scale_period > 0 ? ((int64_t)ks0 * BK) % a.scale_period : 0;
  int64_t kin_load = kin0, kin_use = kin0;
  bool first_load = true, first_use = true;
  float s_cur[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) s_cur[nb] = 0.0f;
  auto advance = [&](int64_t& kin) __attribute__((always_inline)) {
    if (a.scale_period > 0) {
      kin += BK;
      if (kin >= a.scale_period) kin -= a.scale_period;
    }
  };
  // the scales of k-step ks (loaded only when it starts a group)
  auto load_s = [&](float (&sv)[NBW], int ks) __attribute__((always_inline)) {
    int k0 = ks * BK;
    k0 = k0 < klast ? k0 : klast;
    const uint32_t kk = (uint32_t)(k0 + 32 * g);
    const uint32_t t = __umulhi(kk, a.gdiv_mul);
    const uint32_t gi = ((t + ((kk - t) >> 1)) >> (a.gdiv_shift - 1)) & a.gmask;
    const bool need_s = a.scale_period == 0 || kin_load == 0 || first_load;
    first_load = false;
    advance(kin_load);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
      if (need_s) sv[nb] = srow[nb][gi];
  };
  // a super-step's weights, row-contiguous (16 bytes per lane and row piece)
  auto load_super = [&](u32x4 (&raw)[NBW][4], int kb) __attribute__((always_inline)) {
    const int off0 = kb * (BK * BITS / 8) + 16 * (lane & 7);
    const int off = off0 < prow_bytes - 16 ? off0 : prow_bytes - 16;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        raw[nb][j] = *reinterpret_cast<const u32x4*>(lrow[nb][j] + off);
  };
  auto store_super = [&](const u32x4 (&raw)[NBW][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(&wst[wave][nb][((lane >> 3) + 8 * j) * SP + 16 * (lane & 7)]) =
            raw[nb][j];
  };
  // the lane's fragment of k-step s of the staged super-step
  auto read_frag = [&](BRegs<BITS>& br, int nb, int s) __attribute__((always_inline)) {
    const uint8_t* src = &wst[wave][nb][l32 * SP + s * (BK * BITS / 8) + FB * g];
    br.p[0] = *reinterpret_cast<const u32x4*>(src);
    if constexpr (BITS == 8) br.p[1] = *reinterpret_cast<const u32x4*>(src + 16);
  };
  auto load_a = [&](u32x4 (&af)[MB][4], int k0) __attribute__((always_inline)) {
    k0 = k0 < klast ? k0 : klast;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int s = 0; s < 4; ++s) af[mb][s] = *reinterpret_cast<const u32x4*>(xrow[mb] + k0 + 8 * s);
  };
  f32x16 acc[MB][NBW];
  // Largest |scale| this wave decoded with the one-FMA int4 decoder.
  float smax = 0.0f;

  // The wave's k-steps, with the one-FMA int4 decoder (fma = true) or the
  // two-step decoders.
  auto run = [&](auto fma) __attribute__((always_inline)) {
  constexpr bool F = decltype(fma)::value;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  kin_load = kin_use = kin0;
  first_load = first_use = true;

  // super-step weights one super-step ahead, A fragments one k-step ahead
  u32x4 raw[NBW][4];
  float scur[SS][NBW], snxt[SS][NBW];
#pragma unroll
  for (int t = 0; t < SS; ++t)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) scur[t][nb] = snxt[t][nb] = 0.0f;
  u32x4 afE[MB][4], afO[MB][4];
  load_super(raw, ks0);
#pragma unroll
  for (int t = 0; t < SS; ++t) load_s(scur[t], ks0 + t);
  load_a(afE, ks0 * BK);
  // k-step ks (s-th of its super-step): its fragment br, A fragments af
  auto kstep = [&](int ks, int s, const BRegs<BITS> (&br)[NBW], const u32x4 (&af)[MB][4],
                   u32x4 (&af_nxt)[MB][4]) __attribute__((always_inline)) {
    const bool new_s = a.scale_period == 0 || kin_use == 0 || first_use;
    first_use = false;
    advance(kin_use);
    u32x4 bq[NBW][4];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (new_s) s_cur[nb] = scur[s][nb];
      if constexpr (F) smax = fmaxf(smax, fabsf(s_cur[nb]));
      dequant32<BITS, F>(br[nb], s_cur[nb], bq[nb]);
    }
    load_a(af_nxt, (ks + 1) * BK);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, af[mb][q4]), __builtin_bit_cast(bf16x8, bq[nb][q4]),
              acc[mb][nb], 0, 0, 0);
  };
  for (int kb = ks0; kb < ks1; kb += SS) {
    // stage this super-step (the wave's own LDS region: its LDS accesses
    // complete in order, so the reads below see these writes and the next
    // super-step's writes come after these reads), then load the next one
    store_super(raw);
    BRegs<BITS> br[SS][NBW];
#pragma unroll
    for (int t = 0; t < SS; ++t)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) read_frag(br[t][nb], nb, t);
    load_super(raw, kb + SS);
#pragma unroll
    for (int t = 0; t < SS; ++t) load_s(snxt[t], kb + SS + t);
#pragma unroll
    for (int t = 0; t < SS; t += 2) {
      if (kb + t < ks1) kstep(kb + t, t, br[t], afE, afO);
      if (kb + t + 1 < ks1) kstep(kb + t + 1, t + 1, br[t + 1], afO, afE);
    }
#pragma unroll
    for (int t = 0; t < SS; ++t)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) scur[t][nb] = snxt[t][nb];
  }
  };
  if constexpr (BITS == 4) {
    run(std::true_type{});
    // a scale too large for the one-FMA decoder: the wave redoes its k-steps
    // with the two-step decoder (its LDS stage is its own; no other wave waits)
    if (__builtin_amdgcn_ballot_w64(smax >= kFmaScaleLimit)) run(std::false_type{});
  } else {
    run(std::false_type{});
  }

  // ---- partial tiles of waves 1..3 into LDS (register layout), then every
  // thread adds the four partials of its outputs in wave order and stores
  if (wave > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[wave - 1][((mb * NBW + nb) * 16 + r) * 64 + lane] = acc[mb][nb][r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int nn = n0 + 32 * nb + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = ((mb * NBW + nb) * 16 + r) * 64 + lane;
          const float v = ((acc[mb][nb][r] + red[0][e]) + red[1][e]) + red[2][e];
          // D[i][j] of a 32x32 block: lane j + 32*((i/4)%2), register 4*(i/8) + i%4
          const int64_t mm = m0 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
          if (mm < a.m && nn < a.n) __builtin_nontemporal_store(v, &a.y[mm * a.n + nn]);
        }
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
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < m * n;
       t += (int64_t)gridDim.x * 256) {
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
}

// ------------------------------------------------------ activation rounding

// fp32 activations rounded to bf16 (round to nearest even: the conversion
// the tiled kernels apply to the weights) for the dequantizing GEMM; 8 values
// per thread, two 16-byte loads and one 16-byte store when both buffers are
// 16-byte aligned.
__global__ __launch_bounds__(256) void round_bf16_kernel(const float* __restrict__ x,
                                                         uint16_t* __restrict__ xb, int64_t count,
                                                         int vec) {
  for (int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i0 < count;
       i0 += (int64_t)gridDim.x * 256 * 8) {
    if (vec && i0 + 8 <= count) {
      const float4 a = *reinterpret_cast<const float4*>(x + i0);
      const float4 b = *reinterpret_cast<const float4*>(x + i0 + 4);
      *reinterpret_cast<u32x4*>(xb + i0) = u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w),
                                                 pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)};
    } else {
      for (int64_t i = i0; i < count && i < i0 + 8; ++i)
        xb[i] = (uint16_t)(pack_bf16x2(x[i], 0.0f) & 0xffffu);
    }
  }
}

}  // namespace

int gemm_path(const Mat& mt, const uint8_t* payload, const uint16_t* x) {
  const bool shape_ok = mt.k % BK == 0 && mt.n < (1ll << 30) && mt.k < (1ll << 30) &&
                        mt.n * mt.k * mt.bits / 8 < (1ll << 62);
  const bool group_ok = mt.k > 0 && ((mt.k % mt.group == 0 && mt.group % 32 == 0) ||
                                      (mt.group % mt.k == 0));
  if (shape_ok && group_ok && aligned(payload, 16) && aligned(x, 16)) return PATH_FAST;
  return PATH_GENERIC;
}

// Compute units of the current device (cached per device; threads that
// query a device for the first time at once store the same value).
static int compute_units() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
    if (a.per_row_groups) {
      // group >= 32 here, so l = ceil(log2 group) >= 5
      const uint32_t d = (uint32_t)mt.group;
      uint32_t l = 0;
      while ((1ull << l) < d) ++l;
      a.gdiv_mul = (uint32_t)((((1ull << (32 + l)) / d) + 1) & 0xffffffffu);
      a.gdiv_shift = l;
      a.gmask = 0xffffffffu;
    } else {
      a.gdiv_mul = 0;
      a.gdiv_shift = 1;
      a.gmask = 0;
    }
    // one scale per `group` codes along a row (per-row groups), or per row
    a.scale_period = a.per_row_groups ? (mt.group % BK == 0 ? mt.group : 0) : mt.k;
    // few rows: the small-M kernel, tile 32 x 32*NBW, K split over the block's
    // waves -- unless its grid (one block per tile) would pass 2^24 blocks; the
    // 256-row tiles then take it
    const bool few_rows = m <= kSmallMaxM || (m <= kSmallMaxMNarrow && mt.n <= kNarrowN);
    if (few_rows && ((m + 31) / 32) * ((mt.n + 31) / 32) < (1ll << 24)) {
      const int cus = compute_units();
      // Two column blocks per wave (half the A-fragment reads per weight) when that
      // still gives every compute unit a block.  Above 32 rows of X, 64-row tiles
      // (the weights read once per 64 rows) when their grid still gives every
      // compute unit 1.5 blocks: measured (us, 32- / 64-row tiles) 28672 x 8192
      // at M = 48 92 / 73, 64 93 / 84; 16384 x 8192 at M = 128 94 / 86; with
      // fewer blocks they lose (11008 x 4096 at M = 64 28 / 39, 4096 x 11008
      // 30 / 47).
      auto shape = [&](int mbv, int64_t& tmv, int& nbv, int64_t& tnv) {
        tmv = (m + 32 * mbv - 1) / (32 * mbv);
        nbv = tmv * ((mt.n + 63) / 64) >= cus ? 2 : 1;
        tnv = (mt.n + 32 * nbv - 1) / (32 * nbv);
      };
      int64_t tms, tns;
      int nbw;
      shape(2, tms, nbw, tns);
      const int mbk = m > 32 && 2 * tms * tns >= 3 * (int64_t)cus ? 2 : 1;
      if (mbk == 1) shape(1, tms, nbw, tns);
      a.tiles_m = (int)tms;
      a.tiles_n = (int)tns;
      const unsigned grid = (unsigned)(tms * tns);
#define QW_SMALL(B, MBv, NBv) gemm_small_kernel<B, MBv, NBv><<<grid, 256, 0, st>>>(a)
      if (mt.bits == 4) {
        if (mbk == 1) {
          if (nbw == 1) QW_SMALL(4, 1, 1); else QW_SMALL(4, 1, 2);
        } else {
          if (nbw == 1) QW_SMALL(4, 2, 1); else QW_SMALL(4, 2, 2);
        }
      } else {
        if (mbk == 1) {
          if (nbw == 1) QW_SMALL(8, 1, 1); else QW_SMALL(8, 1, 2);
        } else {
          if (nbw == 1) QW_SMALL(8, 2, 1); else QW_SMALL(8, 2, 2);
        }
      }
#undef QW_SMALL
      return hipGetLastError();
    }
    const int64_t tm = (m + BM - 1) / BM;
    const int64_t tn = (mt.n + BN - 1) / BN;
    if (tm * tn >= (1ll << 23)) return hipErrorInvalidValue;  // grid <= 2 * tiles blocks
    a.tiles_m = (int)tm;
    a.tiles_n = (int)tn;
    a.xcd_map = (tn % 8 == 0) ? 1 : 0;
    // One block per compute unit at a time (the block holds all of a CU's
    // registers).  If the last round of tiles would leave at least half the
    // compute units idle, split each of its tiles in two along K.
    const int tiles = (int)(tm * tn);
    const int nk = (int)(mt.k / BK);
    const int cus = compute_units();
    const int rem = tiles - ((tiles - 1) / cus) * cus;  // tiles in the last round
    a.full_tiles = tiles;
    a.nk_lo = 0;
    if (nk >= 2 && 2 * rem <= cus) {
      a.full_tiles = tiles - rem;
      a.nk_lo = nk / 2;
      gemm_zero_split_tiles<<<(unsigned)rem * 16, 256, 0, st>>>(a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const unsigned grid = (unsigned)(a.full_tiles + 2 * (tiles - a.full_tiles));
    if (mt.bits == 4)
      gemm_kernel<4><<<grid, 256, 0, st>>>(a);
    else
      gemm_kernel<8><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  // at most 2^20 blocks, striding over the outputs
  const int64_t outs = m * mt.n;
  const unsigned grid = (unsigned)std::min<int64_t>((outs + 255) / 256, 1 << 20);
  if (mt.bits == 4)
    gemm_generic_kernel<4><<<grid, 256, 0, st>>>(x, payload, scales, y, m, mt.n, mt.k, mt.group);
  else
    gemm_generic_kernel<8><<<grid, 256, 0, st>>>(x, payload, scales, y, m, mt.n, mt.k, mt.group);
  return hipGetLastError();
}

hipError_t launch_round_bf16(const float* x, uint16_t* xb, int64_t count, hipStream_t st) {
  const int64_t threads = (count + 7) / 8;
  const int vec = aligned(x, 16) && aligned(xb, 16) ? 1 : 0;
  // at most 2^20 blocks, striding over the rest
  round_bf16_kernel<<<(unsigned)std::min<int64_t>((threads + 255) / 256, 1 << 20), 256, 0, st>>>(
      x, xb, count, vec);
  return hipGetLastError();
}

}  // namespace qw
