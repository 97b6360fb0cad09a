// GPTQ codes on the GPU (page "Huit bits, puis quatre", section "Arrondir
// mieux : GPTQ"): the calibration matrix H = sum x^T x, its damping by a
// fraction of the mean diagonal, the upper factor U of H^-1 = U^T U, and the
// component-by-component rounding that carries each rounding error onto the
// later components of the same output channel, in the payload / scale
// format of the plain quantizer.
//
// Everything is fp64, as the section's host implementation is.  The dense
// contractions (H itself, the factorization's trailing updates, the
// triangular inverse, the carried-error updates) run on one fp64 MFMA GEMM
// (v_mfma_f64_16x16x4f64); the sequential parts are small kernels:
//
//   H       X^T X over token chunks into per-chunk partial sums, then a
//           fixed-order reduction into h (lower tiles only, mirrored), so a
//           call is deterministic.
//   U       With J the index reversal, JHJ = L L^T (lower Cholesky) gives
//           H = R R^T with R = J L J upper, hence H^-1 = (R^-1)^T R^-1 and
//           U = R^-1 = J L^-1 J.  One blocked Cholesky (64-wide diagonal
//           blocks factored by one wave in registers, panels solved one row
//           per thread, trailing updates as GEMMs on the lower tiles) and
//           one blocked triangular inverse (all diagonal block inverses in
//           one launch, then doubling: X21 = -X22 (L21 X11) for pairs of
//           ever larger blocks).
//   codes   The page's column loop, blocked: a block of up to 64 components
//           is rounded by one wave per output channel (lane j holds
//           component j of the block; the rounding error is broadcast with
//           readlane and carried to the later lanes at once); the errors of
//           the block are then applied to every later component with one
//           GEMM, W[:, after] -= D . V[block, after].  The error carried by
//           the page's loop, (w - w_hat) / U[c][c] times U[c][j], is used
//           as (w - w_hat) times V[c][j] with V[c][j] = U[c][j] / U[c][c]
//           computed once: the same arithmetic in another rounding order.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qw_internal.h"

namespace qw {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ GEMM
//
// C(i, j) = beta * C(i, j) + alpha * sum_kk A(i, kk) * B(kk, j)
// with A(i, kk) = a[i*a_sm + kk*a_sk], B(kk, j) = b[kk*b_sk + j*b_sn],
// C(i, j) = c[i*c_sm + j*c_sn]; blockIdx.z selects a batch entry whose
// operands are offset by a_sz, b_sz, c_sz elements.  Every entry reduces
// over kred terms, except that with kred_total > 0 (consecutive chunks of
// one long reduction) entry z reduces over min(kred, kred_total - z*kred).  64x64 tiles, 4 waves of 32x32,
// reduction staged through LDS in steps of 16.  With `lower` set the grid
// enumerates only the tiles (ti, tj) with ti >= tj (diagonal tiles whole).

struct G64 {
  const void* a;
  const void* b;
  double* c;
  int64_t a_sm, a_sk, a_sz;
  int64_t b_sk, b_sn, b_sz;
  int64_t c_sm, c_sn, c_sz;
  int64_t m, n, kred, kred_total;
  double alpha, beta;
  int32_t lower, tiles_n;
};

// Two shapes: WB = 2 (64 x 64 tiles, waves of 2 x 2 MFMA blocks, reduction
// stages of 32) and WB = 4 (128 x 128 tiles, waves of 4 x 4 blocks, stages
// of 16, registers capped so two waves share each SIMD: one wave issues at
// most one fp64 MFMA per 64 cycles and stalls at every stage boundary).
// The larger tile reads half as many LDS bytes per MFMA.  The global loads
// of the next stage are issued before the current stage's MFMAs.
template <int WB>
struct GShape {
  static constexpr int kTile = 32 * WB;       // 2 x 2 waves of 16*WB
  static constexpr int kStage = WB == 2 ? 32 : 16;
  static constexpr int kLd = kTile + 4;
  static constexpr int kPer = kTile * kStage / 256;  // staged elements per thread
};

// AI: A is contiguous along i (a_sm == 1), else along the reduction
// (a_sk == 1); BJ: B is contiguous along j (b_sn == 1), else along the
// reduction (b_sk == 1).  Each thread stages kPer elements of each operand
// per stage: one fixed index along the contiguous dimension and kPer
// indices a fixed step apart along the other, so a stage's addresses are
// one per-thread base plus uniform multiples of a stride.
template <typename TA, typename TB, int WB, bool AI, bool BJ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WB == 4 ? 2 : 1)))
void gemm64_kernel(G64 g) {
  using S = GShape<WB>;
  constexpr int kT = S::kTile, kS = S::kStage, kLd = S::kLd, kPer = S::kPer;
  __shared__ double as[2][kS][kLd];
  __shared__ double bs[2][kS][kLd];

  int64_t ti, tj;
  if (g.lower) {
    // linear index over the lower triangle of tiles: x = ti*(ti+1)/2 + tj
    const int64_t x = blockIdx.x;
    int64_t r = (int64_t)((sqrt(8.0 * (double)x + 1.0) - 1.0) * 0.5);
    while (r * (r + 1) / 2 > x) --r;
    while ((r + 1) * (r + 2) / 2 <= x) ++r;
    ti = r;
    tj = x - r * (r + 1) / 2;
  } else {
    ti = blockIdx.x / g.tiles_n;
    tj = blockIdx.x % g.tiles_n;
  }
  const int64_t z = blockIdx.z;
  // no __restrict__: the panel step of the factorization reads and writes
  // the same rows
  const TA* pa = (const TA*)g.a + z * g.a_sz;
  const TB* pb = (const TB*)g.b + z * g.b_sz;
  double* pc = g.c + z * g.c_sz;
  int64_t kred = g.kred;
  if (g.kred_total > 0 && g.kred_total - z * g.kred < kred) kred = g.kred_total - z * g.kred;
  const int64_t i0 = ti * kT, j0 = tj * kT;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  // A: element r of this thread is (ii, kk) of the tile
  constexpr int kAStep = AI ? 256 / kT : 256 / kS;
  const int a_fix = AI ? t % kT : t % kS;   // ii (AI) or kk
  const int a_var = AI ? t / kT : t / kS;   // kk (AI) or ii, plus kAStep * r
  const int64_t a_rstride = (int64_t)kAStep * (AI ? g.a_sk : g.a_sm);
  constexpr int kBStep = BJ ? 256 / kT : 256 / kS;
  const int b_fix = BJ ? t % kT : t % kS;
  const int b_var = BJ ? t / kT : t / kS;
  const int64_t b_rstride = (int64_t)kBStep * (BJ ? g.b_sk : g.b_sn);
  // raw operand values of the next stage and which of them lie inside the
  // operands; converted (or zeroed) only when stored to LDS, after the
  // current stage's MFMAs, so the loads' latency overlaps them
  TA ra[kPer];
  TB rb[kPer];
  uint32_t aok_mask = 0, bok_mask = 0;

  auto load_stage = [&](int64_t k0) {
    const TA* abase = AI ? pa + (i0 + a_fix) + (k0 + a_var) * g.a_sk
                         : pa + (i0 + a_var) * g.a_sm + (k0 + a_fix);
    const TB* bbase = BJ ? pb + (k0 + b_var) * g.b_sk + (j0 + b_fix)
                         : pb + (k0 + b_fix) + (j0 + b_var) * g.b_sn;
    aok_mask = 0;
    bok_mask = 0;
    // every load is issued unconditionally (an element outside the operand
    // reads element 0 instead and is replaced by zero when stored)
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int v = a_var + kAStep * r;
      const bool aok = AI ? (i0 + a_fix < g.m && k0 + v < kred) : (i0 + v < g.m && k0 + a_fix < kred);
      ra[r] = *(aok ? abase + r * a_rstride : pa);
      aok_mask |= (uint32_t)aok << r;
      const int w = b_var + kBStep * r;
      const bool bok = BJ ? (j0 + b_fix < g.n && k0 + w < kred) : (j0 + w < g.n && k0 + b_fix < kred);
      rb[r] = *(bok ? bbase + r * b_rstride : pb);
      bok_mask |= (uint32_t)bok << r;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const double av = ((aok_mask >> r) & 1) ? (double)ra[r] : 0.0;
      const int v = a_var + kAStep * r;
      if (AI) as[buf][v][a_fix] = av;
      else as[buf][a_fix][v] = av;
      const double bv = ((bok_mask >> r) & 1) ? (double)rb[r] : 0.0;
      const int w = b_var + kBStep * r;
      if (BJ) bs[buf][w][b_fix] = bv;
      else bs[buf][b_fix][w] = bv;
    }
  };

  d4 acc[WB][WB];
#pragma unroll
  for (int bi = 0; bi < WB; ++bi)
#pragma unroll
    for (int bj = 0; bj < WB; ++bj) acc[bi][bj] = (d4){0.0, 0.0, 0.0, 0.0};

  // D of v_mfma_f64_16x16x4f64: register r of lane l is row 4r + l/16,
  // column l%16 of the 16x16 block.  With beta != 0 the old values of C
  // are needed at the end; on the 64-wide tiles (registers to spare) they
  // are read here, in flight with the first stage's operands, since the
  // short reductions this shape serves (the Cholesky and code updates)
  // would otherwise wait for them after their few MFMAs.  Clamped
  // addresses as for the operands.
  const bool use_beta = g.beta != 0.0;
  double old[WB][WB][4];
  auto load_old = [&](int bi) {
#pragma unroll
    for (int bj = 0; bj < WB; ++bj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gi = i0 + wi * 16 * WB + bi * 16 + 4 * r + (lane >> 4);
        const int64_t gj = j0 + wj * 16 * WB + bj * 16 + (lane & 15);
        const bool ok = use_beta && gi < g.m && gj < g.n;
        const double v = *(ok ? pc + gi * g.c_sm + gj * g.c_sn : pc);
        old[bi][bj][r] = ok ? v : 0.0;
      }
  };
  if constexpr (WB == 2) {
    if (use_beta) {
#pragma unroll
      for (int bi = 0; bi < WB; ++bi) load_old(bi);
    } else {
      // beta == 0: C is never read (and may hold anything, even NaN)
#pragma unroll
      for (int bi = 0; bi < WB; ++bi)
#pragma unroll
        for (int bj = 0; bj < WB; ++bj)
#pragma unroll
          for (int r = 0; r < 4; ++r) old[bi][bj][r] = 0.0;
    }
  }

  const int64_t nstage = (kred + kS - 1) / kS;
  if (nstage > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  for (int64_t s = 0; s < nstage; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < nstage) load_stage((s + 1) * kS);
#pragma unroll
    for (int ks = 0; ks < kS / 4; ++ks) {
      const int kk = ks * 4 + (lane >> 4);
      double fa[WB], fb[WB];
#pragma unroll
      for (int bi = 0; bi < WB; ++bi) fa[bi] = as[buf][kk][wi * 16 * WB + bi * 16 + (lane & 15)];
#pragma unroll
      for (int bj = 0; bj < WB; ++bj) fb[bj] = bs[buf][kk][wj * 16 * WB + bj * 16 + (lane & 15)];
#pragma unroll
      for (int bi = 0; bi < WB; ++bi)
#pragma unroll
        for (int bj = 0; bj < WB; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[bi], fb[bj], acc[bi][bj], 0, 0, 0);
    }
    if (s + 1 < nstage) store_stage(buf ^ 1);
    __syncthreads();
  }

  // On the 128-wide tiles the old values of C are read here, one row of
  // blocks at a time (the reads of a row in flight together).
#pragma unroll
  for (int bi = 0; bi < WB; ++bi) {
    if constexpr (WB != 2) load_old(bi);
#pragma unroll
    for (int bj = 0; bj < WB; ++bj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gi = i0 + wi * 16 * WB + bi * 16 + 4 * r + (lane >> 4);
        const int64_t gj = j0 + wj * 16 * WB + bj * 16 + (lane & 15);
        if (gi < g.m && gj < g.n)
          pc[gi * g.c_sm + gj * g.c_sn] = g.alpha * acc[bi][bj][r] + g.beta * old[bi][bj][r];
      }
  }
}

template <typename TA, typename TB, int WB>
void gemm64_launch(const G64& g, unsigned grid, int batch, hipStream_t stream) {
  const bool ai = g.a_sm == 1, bj = g.b_sn == 1;
  if (ai && bj)
    hipLaunchKernelGGL((gemm64_kernel<TA, TB, WB, true, true>), dim3(grid, 1, (unsigned)batch),
                       dim3(256), 0, stream, g);
  else if (ai)
    hipLaunchKernelGGL((gemm64_kernel<TA, TB, WB, true, false>), dim3(grid, 1, (unsigned)batch),
                       dim3(256), 0, stream, g);
  else if (bj)
    hipLaunchKernelGGL((gemm64_kernel<TA, TB, WB, false, true>), dim3(grid, 1, (unsigned)batch),
                       dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm64_kernel<TA, TB, WB, false, false>), dim3(grid, 1, (unsigned)batch),
                       dim3(256), 0, stream, g);
}

// Launch with 128-wide tiles when the output has enough of them to fill the
// chip (or force_wb asks for a shape), else with 64-wide tiles.  Every
// operand must be contiguous along one of its dimensions (a_sm or a_sk is
// 1, b_sn or b_sk is 1).
template <typename TA, typename TB>
hipError_t gemm64(G64 g, int batch, hipStream_t stream, int force_wb = 0) {
  if (g.m <= 0 || g.n <= 0 || batch <= 0) return hipSuccess;
  if ((g.a_sm != 1 && g.a_sk != 1) || (g.b_sn != 1 && g.b_sk != 1)) return hipErrorInvalidValue;
  auto tiles_for = [&](int64_t tile) {
    const int64_t tm = (g.m + tile - 1) / tile, tn = (g.n + tile - 1) / tile;
    return g.lower ? tm * (tm + 1) / 2 : tm * tn;
  };
  int wb = force_wb;
  if (wb == 0) wb = (tiles_for(128) * batch >= 256 && g.kred >= 64) ? 4 : 2;
  const int64_t tile = wb == 4 ? 128 : 64;
  g.tiles_n = (int32_t)((g.n + tile - 1) / tile);
  const unsigned grid = (unsigned)tiles_for(tile);
  if (wb == 4) gemm64_launch<TA, TB, 4>(g, grid, batch, stream);
  else gemm64_launch<TA, TB, 2>(g, grid, batch, stream);
  return hipGetLastError();
}

G64 g64(const void* a, int64_t a_sm, int64_t a_sk, const void* b, int64_t b_sk, int64_t b_sn,
        double* c, int64_t c_sm, int64_t c_sn, int64_t m, int64_t n, int64_t kred,
        double alpha, double beta) {
  G64 g{};
  g.a = a; g.a_sm = a_sm; g.a_sk = a_sk;
  g.b = b; g.b_sk = b_sk; g.b_sn = b_sn;
  g.c = c; g.c_sm = c_sm; g.c_sn = c_sn;
  g.m = m; g.n = n; g.kred = kred; g.kred_total = 0;
  g.alpha = alpha; g.beta = beta;
  return g;
}

// ------------------------------------------------------------------ H

// One round of the chip: 512 work-groups of either tile shape (two per
// compute unit, set by LDS for 64-wide tiles and by registers for 128-wide
// ones).  The tokens are split into as many chunks as fit in one round
// without starting a second, partly filled one; the 128-wide tiles are used
// when they still fill most of the round.
constexpr int64_t kHessRound = 512;
constexpr int64_t kHessMinChunk = 256;  // tokens per partial sum, at least

int64_t hessian_splits_for(int64_t k, int64_t t, int64_t tile) {
  const int64_t tm = (k + tile - 1) / tile;
  const int64_t tiles = tm * (tm + 1) / 2;
  int64_t s = kHessRound / tiles;
  int64_t smax = t / kHessMinChunk;
  if (smax < 1) smax = 1;
  if (s > smax) s = smax;
  if (s > 65535) s = 65535;
  return s < 1 ? 1 : s;
}

int64_t hessian_tile(int64_t k, int64_t t) {
  const int64_t tm = (k + 127) / 128;
  const int64_t tiles = tm * (tm + 1) / 2;
  return tiles * hessian_splits_for(k, t, 128) * 5 >= kHessRound * 4 ? 128 : 64;
}

// Tokens per partial sum.  s equal chunks fill s * tiles slots of the round.
// When the slots left over can take at least half the tiles once more, the
// tokens are cut into s full chunks and a short last one instead: the short
// chunks' work-groups that find a free slot at the start finish early, the
// others take the slots they free, and all are done when the full chunks
// are, so the round lasts as long as a chunk of 2t / (2s + 1) tokens rather
// than t / s (the 1368-input map over 8192 tokens: 66 tiles, 8 chunks of at
// most 1093 tokens instead of 7 of 1171).
int64_t hessian_chunk(int64_t k, int64_t t) {
  const int64_t tile = hessian_tile(k, t);
  const int64_t tm = (k + tile - 1) / tile;
  const int64_t tiles = tm * (tm + 1) / 2;
  const int64_t s = hessian_splits_for(k, t, tile);
  int64_t chunk = (t + s - 1) / s;
  const int64_t spare = kHessRound - s * tiles;
  // only when the round, not the chunk floor, set s
  if (s == kHessRound / tiles && spare > 0 && tiles <= 2 * spare) {
    const int64_t c = (2 * t + 2 * s) / (2 * s + 1);  // ceil(2t / (2s + 1))
    if (c >= kHessMinChunk && (t + c - 1) / c == s + 1) chunk = c;
  }
  return chunk < 1 ? 1 : chunk;
}

// Partial sums (chunks) of one call.
int64_t hessian_splits(int64_t k, int64_t t) {
  const int64_t chunk = hessian_chunk(k, t);
  return t > 0 ? (t + chunk - 1) / chunk : 1;
}

// h[i][j] += sum_s part[s][max][min]: 32x32 tiles of the lower triangle,
// mirrored through LDS so both halves of h are written coalesced.
__global__ __launch_bounds__(256) void hess_reduce_kernel(const double* __restrict__ part,
                                                          int64_t splits, int64_t k,
                                                          double* __restrict__ h) {
  __shared__ double tile[32][33];
  const int64_t x = blockIdx.x;
  int64_t bi = (int64_t)((sqrt(8.0 * (double)x + 1.0) - 1.0) * 0.5);
  while (bi * (bi + 1) / 2 > x) --bi;
  while ((bi + 1) * (bi + 2) / 2 <= x) ++bi;
  const int64_t bj = x - bi * (bi + 1) / 2;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int64_t kk2 = k * k;
  // Each thread sums 4 entries (rows ty, ty + 8, ty + 16, ty + 24 of the
  // tile), adding the partial sums in chunk order; the loads of 8 chunks
  // of all 4 entries are issued before their additions (a chunk past the
  // last reads chunk 0 and is not added).
  const double* pp[4];
  bool ok[4];
  double s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t i = bi * 32 + ty + 8 * r, j = bj * 32 + tx;
    ok[r] = i < k && j < k && i >= j;
    pp[r] = part + (ok[r] ? i * k + j : 0);
    s[r] = 0.0;
  }
  for (int64_t p = 0; p < splits; p += 8) {
    double v[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 8; ++q) v[r][q] = pp[r][(p + q < splits ? p + q : 0) * kk2];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (p + q < splits) s[r] += v[r][q];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int yy = ty + 8 * r;
    const int64_t i = bi * 32 + yy, j = bj * 32 + tx;
    tile[yy][tx] = s[r];
    if (ok[r]) h[i * k + j] += s[r];
  }
  __syncthreads();
  // mirrored half: h[j][i] += s(i, j) for i > j, read transposed from LDS
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int yy = ty + 8 * r;
    const int64_t j = bj * 32 + yy, i = bi * 32 + tx;
    if (i < k && j < k && i > j) h[j * k + i] += tile[tx][yy];
  }
}

// ------------------------------------------------------------------ U

constexpr int kNb = 64;  // diagonal block of the factorization

// lam = frac * mean(diag h), summed in a fixed order; info = 0, or 1 when
// the mean diagonal is not positive or lam is not finite.
__global__ __launch_bounds__(256) void diag_mean_kernel(const double* __restrict__ h, int64_t k,
                                                        double frac, double* __restrict__ lam,
                                                        int32_t* __restrict__ info) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < k; i += 256) s += h[i * k + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = red[0] / (double)k;
    const double l = frac * mean;
    const bool ok = mean > 0.0 && l < INFINITY;
    *lam = ok ? l : 0.0;
    if (info) *info = ok ? 0 : 1;
  }
}

// a[r][c] (kp x kp) = h[k-1-r][k-1-c] + lam*(r == c) on the lower triangle
// of the reversed, damped matrix, 0 above it, identity on the padding.
__global__ __launch_bounds__(256) void reverse_damp_kernel(const double* __restrict__ h, int64_t k,
                                                           const double* __restrict__ lam,
                                                           double* __restrict__ a, int64_t kp) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= kp * kp) return;
  const int64_t r = idx / kp, c = idx % kp;
  double v = 0.0;
  if (r < k && c < k) {
    if (r >= c) v = h[(k - 1 - r) * k + (k - 1 - c)] + (r == c ? *lam : 0.0);
  } else if (r == c) {
    v = 1.0;
  }
  a[idx] = v;
}

__device__ inline double readlane_f64(double v, int lane) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Orders a wave's own LDS accesses: a read after this sees the wave's
// earlier writes (one wave's LDS operations run in issue order; this keeps
// the compiler from moving them).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// x[s] = fma(-xc, row[s], x[s]) for s0 <= s < kNb, in order of s, where
// row is a row of an LDS array that every lane reads at the same address.
// The values are read in chunks of 8 and each chunk's reads are issued
// before the previous chunk's FMAs, so the LDS latency is paid about once
// per row (left to itself the compiler waited for every pair of values
// before using it, one LDS round trip per two FMAs).  s0 must be a
// constant after unrolling.
__device__ inline void lds_axpy(double (&x)[kNb], double xc, const double* row, int s0) {
  constexpr int kC = 8;
  double buf[2][kC];
#pragma unroll
  for (int i = 0; i < kC; ++i)
    if (s0 + i < kNb) buf[0][i] = row[s0 + i];
#pragma unroll
  for (int ch = 0; ch < kNb / kC; ++ch) {
    if (s0 + ch * kC < kNb) {
      if (s0 + (ch + 1) * kC < kNb) {
#pragma unroll
        for (int i = 0; i < kC; ++i) {
          const int s = s0 + (ch + 1) * kC + i;
          if (s < kNb) buf[(ch + 1) & 1][i] = row[s];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kC; ++i) {
        const int s = s0 + ch * kC + i;
        if (s < kNb) x[s] = fma(-xc, buf[ch & 1][i], x[s]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The small kernels below run 64 dependent steps.  An fp64 operation takes
// about 36 cycles to produce its result and a division or square root is a
// chain of about ten of them, so the steps use reciprocals computed off the
// dependent chain (rsqrt for the pivot, 1/L[c][c] staged in LDS), and the
// triangular loops are unrolled so each step issues only the updates it
// needs.  The panel kernel factors the diagonal block and solves the rows
// below it in the same pass, so a block column costs one launch and one
// dependent chain of 64 pivots.

// The whole panel of block column p in one launch: the diagonal block and
// every row below it.  A work-group holds the 64 rows of the diagonal block
// (wave 0, recomputed by every work-group) and up to kPanelOther rows below
// it, one row per thread in registers.
//
// Wave 0 factors the diagonal block alone, column by column: the pivot of
// column c from lane c (readlane), the column scaled by rsqrt(pivot) and
// written to LDS as row c of lt (lt[c][s] = L[s][c]), then the later
// columns of every row updated.  The next pivot's column is updated first,
// with L[c+1][c] read from lane c + 1 (readlane), so the chain from one
// pivot to the next holds no LDS round trip; the other updates read lt.
// No barrier sits on that chain: the rows below follow one stage of
// kPanelStage columns behind, each thread scaling its entry of column c by
// the staged rsqrt and updating its later columns with lt[c], and one
// barrier per stage hands the columns over.  Every row sees the same
// operations in the same order as in the plain column loop.  Every
// work-group writes its own rows of the panel; work-group 0 writes the
// factored diagonal block to l11 (64 x 64, row-major, zero above the
// diagonal), not back into a: the other work-groups read the unfactored
// block from a when they start, and nothing orders that read after
// work-group 0 finishes.  info = 1 when a pivot is not positive.
constexpr int kPanelThreads = 256;
constexpr int kPanelOther = kPanelThreads - kNb;
constexpr int kPanelStage = 16;
static_assert(kNb % kPanelStage == 0, "whole stages");

// Stage ST of the diagonal block (wave 0): columns [ST*S, (ST+1)*S).
template <int ST>
__device__ inline void panel_diag_stage(double (&x)[kNb], double (*lt)[kNb], double* rps, int t,
                                        bool& bad) {
#pragma unroll
  for (int c = ST * kPanelStage; c < (ST + 1) * kPanelStage; ++c) {
    const double d = readlane_f64(x[c], c);
    bad = bad || !(d > 0.0);
    const double rp = rsqrt(d);
    x[c] = (t == c) ? d * rp : x[c] * rp;
    lt[c][t] = x[c];
    if (t == 0) rps[c] = rp;
    if (c + 1 < kNb) {
      x[c + 1] = fma(-x[c], readlane_f64(x[c], c + 1), x[c + 1]);
      wave_lds_sync();
      lds_axpy(x, x[c], lt[c], c + 2);
    }
  }
}

// Stage ST of a row below the diagonal block, once its columns are in lt.
template <int ST>
__device__ inline void panel_row_stage(double (&x)[kNb], const double (*lt)[kNb],
                                       const double* rps) {
  double r[kPanelStage];
#pragma unroll
  for (int i = 0; i < kPanelStage; ++i) r[i] = rps[ST * kPanelStage + i];
#pragma unroll
  for (int i = 0; i < kPanelStage; ++i) {
    const int c = ST * kPanelStage + i;
    x[c] *= r[i];
    lds_axpy(x, x[c], lt[c], c + 1);
  }
}

__global__ __launch_bounds__(kPanelThreads) void panel_factor_kernel(double* a, int64_t kp,
                                                                     int64_t p0,
                                                                     double* __restrict__ l11,
                                                                     int32_t* __restrict__ info) {
  static_assert(kNb / kPanelStage == 4, "the stages below are spelled out");
  __shared__ __align__(16) double lt[kNb][kNb];
  __shared__ double rps[kNb];
  const int t = threadIdx.x;
  const bool diag = t < kNb;
  const int64_t row = diag ? p0 + t : p0 + kNb + (int64_t)blockIdx.x * kPanelOther + (t - kNb);
  const bool active = diag || (row < kp);
  double x[kNb];
  const double* ar = a + (active ? row : p0) * kp + p0;
#pragma unroll
  for (int c = 0; c < kNb; ++c) {
    const double v = ar[c];
    x[c] = (active && (!diag || c <= t)) ? v : 0.0;
  }
  bool bad = false;
  if (diag) panel_diag_stage<0>(x, lt, rps, t, bad);
  __syncthreads();
  if (diag) panel_diag_stage<1>(x, lt, rps, t, bad);
  else panel_row_stage<0>(x, lt, rps);
  __syncthreads();
  if (diag) panel_diag_stage<2>(x, lt, rps, t, bad);
  else panel_row_stage<1>(x, lt, rps);
  __syncthreads();
  if (diag) panel_diag_stage<3>(x, lt, rps, t, bad);
  else panel_row_stage<2>(x, lt, rps);
  __syncthreads();
  if (!diag) panel_row_stage<3>(x, lt, rps);
  if (active && (!diag || blockIdx.x == 0)) {
    double* aw = diag ? l11 + t * kNb : a + row * kp + p0;
#pragma unroll
    for (int c = 0; c < kNb; ++c) aw[c] = (!diag || c <= t) ? x[c] : 0.0;
  }
  if (diag && bad && t == 0 && blockIdx.x == 0 && info) *info = 1;
}

// A lower triangular 64 x 64 block L (row-major, leading dimension 64)
// staged for the row solves by a work-group of 64 threads: lt[c][s] =
// L[s][c] (zero for s < c), rd[c] = 1 / L[c][c].  Thread s reads row s
// whole, so its 64 loads are in flight together.
__device__ inline void load_lt(double (*lt)[kNb], double* rd, const double* l) {
  const int s = threadIdx.x;
  double v[kNb];
#pragma unroll
  for (int c = 0; c < kNb; ++c) v[c] = l[s * kNb + c];
#pragma unroll
  for (int c = 0; c < kNb; ++c) lt[c][s] = (s >= c) ? v[c] : 0.0;
  rd[s] = 1.0 / l[s * kNb + s];
}

// x L^T = x0 for one row x: x_c *= 1/L[c][c], then x_s -= x_c L[s][c] for
// s > c.
__device__ inline void solve_lt(double (&x)[kNb], const double (*lt)[kNb], const double* rd) {
  constexpr int kG = 16;  // reciprocals read together
#pragma unroll
  for (int g = 0; g < kNb; g += kG) {
    double r[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) r[i] = rd[g + i];
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      const int c = g + i;
      x[c] = x[c] * r[i];
      lds_axpy(x, x[c], lt[c], c + 1);
    }
  }
}

// The inverse of every diagonal block of L (read from lblk, block p at
// lblk + p * 64 * 64) written into the diagonal blocks of a (one
// work-group per block; thread j solves x L^T = e_j, i.e. column j of
// L^-1).
__global__ __launch_bounds__(64) void trtri_diag_kernel(const double* __restrict__ lblk, double* a,
                                                        int64_t kp) {
  __shared__ __align__(16) double lt[kNb][kNb];
  __shared__ double rd[kNb];
  __shared__ double outb[kNb][kNb + 1];
  const int64_t p0 = (int64_t)blockIdx.x * kNb;
  load_lt(lt, rd, lblk + (int64_t)blockIdx.x * kNb * kNb);
  __syncthreads();
  const int j = threadIdx.x;
  double x[kNb];
#pragma unroll
  for (int c = 0; c < kNb; ++c) x[c] = (c == j) ? 1.0 : 0.0;
  solve_lt(x, lt, rd);
#pragma unroll
  for (int i = 0; i < kNb; ++i) outb[i][j] = (i >= j) ? x[i] : 0.0;
  __syncthreads();
  for (int i = 0; i < kNb; ++i) a[(p0 + i) * kp + p0 + j] = outb[i][j];
}

// u[i][j] = a[k-1-i][k-1-j] for i <= j, 0 below the diagonal.
__global__ __launch_bounds__(256) void reverse_out_kernel(const double* __restrict__ a, int64_t kp,
                                                          int64_t k, double* __restrict__ u) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= k * k) return;
  const int64_t i = idx / k, j = idx % k;
  u[idx] = (i <= j) ? a[(k - 1 - i) * kp + (k - 1 - j)] : 0.0;
}

// ------------------------------------------------------------------ codes

__global__ __launch_bounds__(256) void to_f64_kernel(const float* __restrict__ w,
                                                     double* __restrict__ wd, int64_t count) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < count) wd[idx] = (double)w[idx];
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// v[i][j] = u[i][j] / u[i][i] above and on the diagonal, 0 below: the
// carrying factors per unit of rounding error, e * U[i][j] with
// e = d / U[i][i] being d * v[i][j].  Computing them once, in parallel,
// keeps an fp64 division off every step of the sequential loop.
__global__ __launch_bounds__(256) void normalize_rows_kernel(const double* __restrict__ u,
                                                             int64_t k, double* __restrict__ v) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= k * k) return;
  const int64_t i = idx / k, j = idx % k;
  v[idx] = (j >= i) ? u[idx] / u[i * k + i] : 0.0;
}

// One block of components [k0, k0 + bsz) (bsz <= 64) for 4 output channels
// per work-group, one per wave.  Lane j holds component k0 + j of its
// channel.  For each component s in order: the group scale when s starts a
// group, the code of the component (same fp32 quantizer as the plain path),
// its rounding error d = w_s - w_hat_s, and w_j -= d * v[s][j] on the lanes
// j > s (v = the normalized rows of U).  The codes go to the payload, the
// errors to e_out [n][64] for the update of the later components.
template <int BITS>
__global__ __launch_bounds__(256) void gptq_block_kernel(
    const double* __restrict__ wd, const double* __restrict__ v, int64_t n, int64_t k,
    int64_t k0, int bsz, int64_t group, double* __restrict__ e_out,
    uint8_t* __restrict__ payload, float* __restrict__ scales) {
  __shared__ double ub[64][64];
  const int t = threadIdx.x;
  {
    // 16 values per thread, every load issued before the first store (an
    // element outside the block reads v[0] and stores 0)
    constexpr int kPer = 64 * 64 / 256;
    double tv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = t + 256 * i;
      const int s = e >> 6, j = e & 63;
      const bool ok = s < bsz && j < bsz;
      tv[i] = v[ok ? (k0 + s) * k + (k0 + j) : 0];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = t + 256 * i;
      const int s = e >> 6, j = e & 63;
      ub[s][j] = (s < bsz && j < bsz) ? tv[i] : 0.0;
    }
  }
  __syncthreads();
  const int lane = t & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (t >> 6);
  if (row >= n) return;
  constexpr float qmax = BITS == 8 ? 127.0f : 7.0f;
  const double* wr = wd + row * k;
  const int64_t ngroups = k / group;
  double w = lane < bsz ? wr[k0 + lane] : 0.0;
  float sc = 1.0f;
  if (group > bsz) {
    // the whole group starts at this block: its scale from the current
    // weights of all its components (later blocks' entries are in wd)
    if (k0 % group == 0) {
      float m = 0.0f;
      for (int64_t j = k0 + lane; j < k0 + group; j += 64) m = fmaxf(m, fabsf((float)wr[j]));
      m = wave_max(m);
      sc = m / qmax;
      if (sc == 0.0f) sc = 1.0f;
      if (lane == 0) scales[row * ngroups + k0 / group] = sc;
    } else {
      // a block inside a group: the scale was fixed at the group's start
      sc = scales[row * ngroups + k0 / group];
    }
  }
  int code = 0;
  double ev = 0.0;
  // Component s: its code from the current weight of lane s, its rounding
  // error, and that error carried to the later lanes.
  auto step = [&](int s) {
    const double us = ub[s][lane];
    const double ws = readlane_f64(w, s);
    const float r = (float)ws / sc;
    const float c = fminf(fmaxf(rintf(r), -qmax), qmax);
    const float what = c * sc;
    const double err = ws - (double)what;
    if (lane == s) {
      code = (int)c;
      ev = err;
    }
    if (lane > s) w = fma(-err, us, w);
  };
  if (group <= bsz) {
    // Whole groups, starting at the multiples of group (k0 and bsz are
    // multiples of group here): each group's scale from the current weights
    // of its components, then its components, with no test in the loop.
    for (int g0 = 0; g0 < bsz; g0 += (int)group) {
      const float aw = (lane >= g0 && lane < g0 + group) ? fabsf((float)w) : 0.0f;
      const float m = wave_max(aw);
      sc = m / qmax;
      if (sc == 0.0f) sc = 1.0f;
      if (lane == 0) scales[row * ngroups + (k0 + g0) / group] = sc;
      for (int s = g0; s < g0 + (int)group; ++s) step(s);
    }
  } else {
    for (int s = 0; s < bsz; ++s) step(s);
  }
  if (lane < bsz) e_out[row * 64 + lane] = ev;
  if (BITS == 8) {
    if (lane < bsz) payload[row * k + k0 + lane] = (uint8_t)(int8_t)code;
  } else {
    const int nib = code + 8;
    const int hi = __shfl_xor(nib, 1);
    if (lane < bsz && (lane & 1) == 0)
      payload[(row * k + k0 + lane) >> 1] = (uint8_t)(nib | (hi << 4));
  }
}

int block_size(int bits, int64_t group) {
  if (group <= 64) return (int)(group * (64 / group));
  for (int b = 64; b >= 1; --b)
    if (group % b == 0 && (bits == 8 || (b % 2) == 0)) return b;
  return bits == 8 ? 1 : 2;
}

inline unsigned grid1(int64_t count) { return (unsigned)((count + 255) / 256); }

}  // namespace

// ------------------------------------------------------------------ API

int64_t gptq_hessian_work_bytes(int64_t k, int64_t t) {
  return hessian_splits(k, t) * k * k * (int64_t)sizeof(double);
}

hipError_t launch_gptq_hessian(int64_t k, int64_t t, const float* x, double* h, void* work,
                               hipStream_t stream) {
  const int64_t chunk = hessian_chunk(k, t);
  double* part = (double*)work;
  // part[s] = X_s^T X_s with X_s the tokens [s*chunk, (s+1)*chunk)
  G64 g = g64(x, 1, k, x, k, 1, part, k, 1, k, k, chunk, 1.0, 0.0);
  g.lower = 1;
  g.a_sz = chunk * k;
  g.b_sz = chunk * k;
  g.c_sz = k * k;
  g.kred_total = t;
  const int64_t used = (t + chunk - 1) / chunk;
  hipError_t e = gemm64<float, float>(g, (int)used, stream, hessian_tile(k, t) == 128 ? 4 : 2);
  if (e != hipSuccess) return e;
  const int64_t tb = (k + 31) / 32;
  hipLaunchKernelGGL(hess_reduce_kernel, dim3((unsigned)(tb * (tb + 1) / 2)), dim3(256), 0,
                     stream, part, used, k, h);
  return hipGetLastError();
}

int64_t gptq_factor_work_bytes(int64_t k) {
  const int64_t kp = (k + kNb - 1) / kNb * kNb;
  // a (kp x kp), the doubling temporary (kp x kp) and lam
  return (2 * kp * kp + 2) * (int64_t)sizeof(double);
}

hipError_t launch_gptq_factor(int64_t k, const double* h, double damp, double* u, int32_t* info,
                              void* work, hipStream_t stream) {
  const int64_t kp = (k + kNb - 1) / kNb * kNb;
  const int64_t nblk = kp / kNb;
  double* a = (double*)work;
  double* tmp = a + kp * kp;
  double* lam = tmp + kp * kp;
  hipError_t e;

  hipLaunchKernelGGL(diag_mean_kernel, dim3(1), dim3(256), 0, stream, h, k, damp, lam, info);
  hipLaunchKernelGGL(reverse_damp_kernel, dim3(grid1(kp * kp)), dim3(256), 0, stream, h, k,
                     (const double*)lam, a, kp);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // blocked Cholesky of the reversed matrix: a = L below the diagonal
  // blocks, the diagonal blocks of L in tmp (block p at tmp + p * 64 * 64;
  // tmp is free until the doubling, which starts after they are inverted)
  for (int64_t p = 0; p < nblk; ++p) {
    const int64_t p0 = p * kNb;
    const int64_t rest = kp - p0 - kNb;
    // the diagonal block and the panel below it
    const int64_t pwg = rest > 0 ? (rest + kPanelOther - 1) / kPanelOther : 1;
    hipLaunchKernelGGL(panel_factor_kernel, dim3((unsigned)pwg), dim3(kPanelThreads), 0, stream,
                       a, kp, p0, tmp + p * kNb * kNb, info);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (rest <= 0) continue;
    // trailing: A22 -= L21 L21^T on the lower tiles
    double* a21 = a + (p0 + kNb) * kp + p0;
    double* a22 = a + (p0 + kNb) * kp + (p0 + kNb);
    G64 g = g64(a21, kp, 1, a21, 1, kp, a22, kp, 1, rest, rest, kNb, -1.0, 1.0);
    g.lower = 1;
    if ((e = gemm64<double, double>(g, 1, stream)) != hipSuccess) return e;
  }

  // triangular inverse in place: diagonal blocks first, then doubling
  hipLaunchKernelGGL(trtri_diag_kernel, dim3((unsigned)nblk), dim3(64), 0, stream,
                     (const double*)tmp, a, kp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int64_t b = kNb; b < kp; b *= 2) {
    const int64_t nfull = kp / (2 * b);
    const int64_t step = 2 * b * kp + 2 * b;  // next pair along the diagonal
    if (nfull > 0) {
      // T_j = L21_j X11_j
      G64 g1 = g64(a + b * kp, kp, 1, a, kp, 1, tmp, b, 1, b, b, b, 1.0, 0.0);
      g1.a_sz = step; g1.b_sz = step; g1.c_sz = b * b;
      if ((e = gemm64<double, double>(g1, (int)nfull, stream)) != hipSuccess) return e;
      // X21_j = -X22_j T_j
      G64 g2 = g64(a + b * kp + b, kp, 1, tmp, b, 1, a + b * kp, kp, 1, b, b, b, -1.0, 0.0);
      g2.a_sz = step; g2.b_sz = b * b; g2.c_sz = step;
      if ((e = gemm64<double, double>(g2, (int)nfull, stream)) != hipSuccess) return e;
    }
    const int64_t top0 = nfull * 2 * b, bot0 = top0 + b;
    if (bot0 < kp) {
      const int64_t bb = kp - bot0;
      double* tp = tmp + nfull * b * b;
      e = gemm64<double, double>(
          g64(a + bot0 * kp + top0, kp, 1, a + top0 * kp + top0, kp, 1, tp, b, 1, bb, b, b,
              1.0, 0.0),
          1, stream);
      if (e != hipSuccess) return e;
      e = gemm64<double, double>(
          g64(a + bot0 * kp + bot0, kp, 1, tp, b, 1, a + bot0 * kp + top0, kp, 1, bb, b, bb,
              -1.0, 0.0),
          1, stream);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(reverse_out_kernel, dim3(grid1(k * k)), dim3(256), 0, stream,
                     (const double*)a, kp, k, u);
  return hipGetLastError();
}

int64_t gptq_quantize_work_bytes(int64_t n, int64_t k) {
  // the fp64 weights being corrected, one block of errors, the normalized
  // rows of U
  return (n * k + n * 64 + k * k) * (int64_t)sizeof(double);
}

hipError_t launch_gptq_quantize_pack(const Mat& mt, const float* w, const double* u,
                                     uint8_t* payload, float* scales, void* work,
                                     hipStream_t stream) {
  const int64_t n = mt.n, k = mt.k;
  double* wd = (double*)work;
  double* eb = wd + n * k;
  double* v = eb + n * 64;
  hipLaunchKernelGGL(to_f64_kernel, dim3(grid1(n * k)), dim3(256), 0, stream, w, wd, n * k);
  hipLaunchKernelGGL(normalize_rows_kernel, dim3(grid1(k * k)), dim3(256), 0, stream, u, k, v);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int bsz = block_size(mt.bits, mt.group);
  const unsigned wgs = (unsigned)((n + 3) / 4);
  for (int64_t k0 = 0; k0 < k; k0 += bsz) {
    const int cur = (int)((k - k0) < bsz ? (k - k0) : bsz);
    if (mt.bits == 8)
      hipLaunchKernelGGL(gptq_block_kernel<8>, dim3(wgs), dim3(256), 0, stream,
                         (const double*)wd, (const double*)v, n, k, k0, cur, mt.group, eb,
                         payload, scales);
    else
      hipLaunchKernelGGL(gptq_block_kernel<4>, dim3(wgs), dim3(256), 0, stream,
                         (const double*)wd, (const double*)v, n, k, k0, cur, mt.group, eb,
                         payload, scales);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t k1 = k0 + cur;
    if (k1 < k) {
      // W[:, k1:] -= D V[k0:k1, k1:]
      e = gemm64<double, double>(g64(eb, 64, 1, v + k0 * k + k1, k, 1, wd + k1, k, 1, n, k - k1,
                                     cur, -1.0, 1.0),
                                 1, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace qw
