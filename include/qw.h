/*
 * qw.h -- C ABI of libqw: symmetric round-to-nearest group quantization of
 * linear-layer weights and the weight-only dequantizing matmul, for AMD
 * Instinct MI355X (gfx950).
 *
 * Formats (page "量化推理：INT8/INT4 的体积、困惑度与速度为什么不同步",
 * script functions `pack` and `unpack`; page "Huit bits, puis quatre",
 * section "Arrondir"):
 *
 *   weight    fp32 [n][k], row-major.  Row i is output channel i; k is the
 *             reduction axis and is contiguous.
 *   groups    consecutive runs of `group` elements in that storage order
 *             (so with k % group == 0 a group lies inside one row).
 *   scale     one fp32 per group: S = max|w| / qmax computed as an IEEE
 *             fp32 division, qmax = 2^(bits-1) - 1 (127 or 7); S = 1 for an
 *             all-zero group.
 *   code      q = clip(round_half_even(fl32(w / S)), -qmax, +qmax), where
 *             w / S is an IEEE fp32 division.
 *   payload   int8: one two's-complement byte per weight, storage order.
 *             int4: n*k/2 bytes; byte i = (q[2i] + 8) | (q[2i+1] + 8) << 4
 *             (element 2i in the low nibble).
 *   w_hat     fl32(float(q) * S) -- the dequantized weight.
 *
 * Matmul (page "Huit bits, puis quatre", section "Ranger des entiers dans
 * des f32", the QuantizedMatmul paragraph: generation products read the
 * codes, large evaluation products use the dequantized weights; both are
 * the same product up to summation order):
 *
 *   y[m][i] = sum_j x[m][j] * w_hat[i][j]
 *
 *   qw_gemv : decode-time product, fp32 activations, 1 <= m <= 8; every
 *             product exact or singly rounded, sums in fp32.  From 3 rows of
 *             x on (for the shapes qw_gemv lists), the products run on the
 *             bf16 matrix cores: each x value
 *             is cut into three bf16 pieces that add up to it exactly, and
 *             each piece times a code (an integer, exact in bf16) is exact in
 *             the fp32 accumulator.
 *             Error <= 1e-5 * sum_j |x[m][j] * w_hat[i][j]|.
 *   qw_gemm : prefill product, bf16 activations; the weights are dequantized
 *             to bf16 (round to nearest even of w_hat) and multiplied on the
 *             matrix cores with fp32 accumulation; m >= 1.
 *             Error <= 8e-3 * sum_j |x[m][j] * w_hat[i][j]| for weights that
 *             are zero or at least 2^-126 in magnitude; below that bf16
 *             keeps fewer bits than the 8 this bound assumes, though the
 *             matrix cores still multiply subnormal bf16 values exactly.
 *   Both bounds are relative ones and, as for any fp32 arithmetic, assume
 *   that the products and partial sums do not underflow below 2^-126 (for
 *   the three-piece GEMV: x values of magnitude 2^-110 or more, whose
 *   smallest piece is still a normal number).
 *
 * Conventions shared by every entry point:
 *   - All buffers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronizes; it keeps no state besides cached
 *     device properties and is safe to call from several threads.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls return
 *     once the work is enqueued; results are valid after the stream has
 *     synchronized.
 *   - Buffers must not overlap.  Inputs must be finite (NaN / Inf give
 *     unspecified codes and outputs).
 *   - Any pointer alignment is accepted; 16-byte aligned buffers (as every
 *     hipMalloc / torch allocation is) take the fast kernels.
 *   - Empty work (n*k == 0, or m == 0) is valid and enqueues nothing, except
 *     that a product with k == 0 writes zeros to y.  Pointers may then be
 *     NULL.
 *   - Errors are returned as negative status codes and never abort.  Every
 *     argument is validated before anything is enqueued, so a call that
 *     returns a validation error (any status but QW_EHIP) has enqueued
 *     nothing.  QW_EHIP means a kernel launch failed (its HIP error text is
 *     available from qw_last_error()); a call that makes several launches
 *     (the batched and chained calls, qw_gemm with a split tail, qw_matmul,
 *     the GPTQ calls) may already have enqueued the launches before the
 *     failing one, and its outputs are then undefined.
 */
#ifndef QW_H
#define QW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum qw_status {
    QW_OK = 0,
    QW_EBITS = -1,   /* bits is not 4 or 8                                   */
    QW_EGROUP = -2,  /* group < 1, or group does not divide n*k              */
    QW_ESHAPE = -3,  /* n < 0, k < 0, a size above its limit (below), or     */
                     /* int4 with odd n*k                                    */
    QW_EM = -4,      /* m out of range (gemv: 0..8, gemm: >= 0) or m*n, m*k  */
                     /* above QW_MAX_ELEMENTS                                */
    QW_ENULL = -5,   /* a required pointer is NULL                           */
    QW_EHIP = -6,    /* a HIP launch failed                                  */
    QW_ECOUNT = -7,  /* batched call: count < 0 or a descriptor is invalid   */
    QW_EWORK = -8,   /* work buffer NULL or smaller than the size query says */
    QW_EARG = -9,    /* another argument out of range (see the entry point)  */
    QW_ESCRATCH = -10 /* qw_matmul_noalloc: input larger than its scratch     */
};

/* Largest number of matrices the batched calls put into one kernel launch
 * (their descriptors travel as kernel arguments). */
#define QW_BATCH_PER_LAUNCH 256

/* Size limits.  One matrix holds at most QW_MAX_ELEMENTS weights: n, k and
 * n*k are each at most that (2^36 fp32 weights are 256 GiB, more than one
 * GPU's memory), and so are a product's m*k activations and m*n outputs.
 * Beyond them a call returns QW_ESHAPE (QW_EM for m) and enqueues nothing.
 * The GPTQ calls take smaller matrices: k <= QW_GPTQ_MAX_K (H and U are
 * k x k fp64, 8 GiB each at the limit), n <= QW_GPTQ_MAX_N, and n*k and
 * t*k at most QW_GPTQ_MAX_ELEMENTS. */
#define QW_MAX_ELEMENTS (1ll << 36)
#define QW_GPTQ_MAX_ELEMENTS (1ll << 31)
#define QW_GPTQ_MAX_K 32768
#define QW_GPTQ_MAX_N (1ll << 24)

/* Bytes of packed codes for an n x k matrix: n*k*bits/8 (-1 if invalid). */
int64_t qw_payload_bytes(int bits, int64_t n, int64_t k);

/* Number of fp32 scales for an n x k matrix: n*k/group (-1 if invalid). */
int64_t qw_num_scales(int64_t group, int64_t n, int64_t k);

/* Static text for a status code. */
const char* qw_status_string(int status);

/* Text of the last HIP error seen by this thread (empty if none). */
const char* qw_last_error(void);

/*
 * Quantize and pack (one pass over the weight).
 *   w        fp32 [n][k]                       (read)
 *   payload  uint8 [qw_payload_bytes(bits,n,k)] (written)
 *   scales   fp32 [qw_num_scales(group,n,k)]   (written)
 * group must divide n*k; int4 needs n*k even.  Codes, scales and payload are
 * bit-identical to the definitions above.
 */
int qw_quantize_pack(int bits, int64_t group, int64_t n, int64_t k,
                     const float* w, uint8_t* payload, float* scales,
                     void* stream);

/*
 * One matrix of a batched quantize/pack (see qw_quantize_pack_batched); the
 * fields mean what the qw_quantize_pack arguments of the same names mean.
 */
typedef struct qw_quant_desc {
    const float* w;      /* fp32 [n][k] */
    uint8_t* payload;    /* qw_payload_bytes(bits, n, k) bytes */
    float* scales;       /* qw_num_scales(group, n, k) floats */
    int64_t n;
    int64_t k;
    int64_t group;
    int32_t bits;
    int32_t reserved;    /* must be 0 */
} qw_quant_desc;

/*
 * Batched quantize/pack: `count` independent matrices (for instance every
 * linear layer of a model at load time), each exactly as qw_quantize_pack
 * would produce it, enqueued as a few large launches instead of one per
 * matrix (matrices of the same bits and group share a launch, up to
 * QW_BATCH_PER_LAUNCH of them).  `descs` is a HOST array read before the
 * call returns; outputs
 * must not overlap each other or any input.  Every entry is validated
 * first; on any invalid entry nothing is enqueued and its status (or
 * QW_ECOUNT for count < 0 / reserved != 0) is returned.
 */
int qw_quantize_pack_batched(int count, const qw_quant_desc* descs, void* stream);

/*
 * Unpack: w_out[i][j] = fl32(float(q) * S), bit-identical.
 *   payload, scales as written by qw_quantize_pack   (read)
 *   w_out    fp32 [n][k]                             (written)
 */
int qw_unpack(int bits, int64_t group, int64_t n, int64_t k,
              const uint8_t* payload, const float* scales, float* w_out,
              void* stream);

/*
 * One matrix of a batched unpack (see qw_unpack_batched); the fields mean
 * what the qw_unpack arguments of the same names mean.
 */
typedef struct qw_unpack_desc {
    const uint8_t* payload;  /* qw_payload_bytes(bits, n, k) bytes */
    const float* scales;     /* qw_num_scales(group, n, k) floats */
    float* w_out;            /* fp32 [n][k] */
    int64_t n;
    int64_t k;
    int64_t group;
    int32_t bits;
    int32_t reserved;        /* must be 0 */
} qw_unpack_desc;

/*
 * Batched unpack: `count` independent matrices (for instance a whole
 * model's layers turned back into fp32, the dequantized copy page "Huit bits,
 * puis quatre", section "Ranger des entiers dans des f32", keeps beside the
 * codes), each bit-identical to what qw_unpack writes, enqueued as a few
 * large launches instead of one per matrix (matrices of the same bit width
 * share a launch, up to QW_BATCH_PER_LAUNCH of them; matrices the vector
 * kernel does not take are launched on their own).  `descs` is a HOST array
 * read before the call returns; outputs must not overlap each other or any
 * input.  Every entry is validated first; on any invalid entry nothing is
 * enqueued and its status (or QW_ECOUNT for count < 0 / reserved != 0) is
 * returned.
 */
int qw_unpack_batched(int count, const qw_unpack_desc* descs, void* stream);

/*
 * Dequantizing GEMV (decode), fp32:
 *   x  fp32 [m][k]  (read),   y  fp32 [m][n]  (written),   0 <= m <= 8.
 * Any group dividing n*k is accepted; with k % 8 == 0 and either
 * k % group == 0 with group % 8 == 0, or group % k == 0, the streaming
 * kernels run.  At 3..8 rows of x (5..8 for matrices of 16384 rows or
 * more), rows of whole 128-code steps
 * (k % 128 == 0), groups of whole steps (group % 128 == 0), of 32 or 64
 * codes, or of whole rows (group % k == 0), a 16-byte aligned payload and an
 * 8-byte aligned x take
 * the matrix-core kernel.  Outputs are deterministic: the same call gives
 * the same bits.
 */
int qw_gemv(int bits, int64_t group, int64_t n, int64_t k,
            const uint8_t* payload, const float* scales,
            int64_t m, const float* x, float* y, void* stream);

/*
 * One matrix of a batched GEMV (see qw_gemv_batched).  Same meaning as the
 * qw_gemv arguments of the same names; pointers are device pointers.
 */
typedef struct qw_gemv_desc {
    const uint8_t* payload;
    const float* scales;
    const float* x;      /* fp32 [m][k] */
    float* y;            /* fp32 [m][n] */
    int64_t n;
    int64_t k;
    int64_t group;
    int32_t bits;
    int32_t reserved;    /* must be 0 */
} qw_gemv_desc;

/*
 * Batched dequantizing GEMV: `count` independent products y_i = x_i * W_i^T
 * with a common m (0 <= m <= 8), each within qw_gemv's error bound (the
 * kernel, and so the summation order, follows the rows of the whole launch:
 * a product may differ from a lone qw_gemv call in its last bits; the
 * matrix-core kernel takes the matrices qw_gemv would give it, from the row
 * counts of x that qw_gemv states for the batch's total weight rows), and
 * enqueued as a few launches (up to QW_BATCH_PER_LAUNCH matrices of one bit
 * width each) that stream the weights back to back instead of one launch
 * per matrix (the fixed cost of many short kernels is what
 * dominates a decode step otherwise -- page "Huit bits, puis quatre",
 * section "La vitesse").  `descs` is a HOST array of `count` entries, read
 * before the call returns.  No y_i may overlap another y_i or any input.
 * Every entry is validated first; on any invalid entry nothing is enqueued
 * and the entry's status (or QW_ECOUNT for count < 0 / reserved != 0) is
 * returned.
 */
int qw_gemv_batched(int count, const qw_gemv_desc* descs, int64_t m, void* stream);

/*
 * Chained decode pass: `count` GEMVs like qw_gemv_batched (common m,
 * 0 <= m <= 8), grouped into stages by `stage` (a HOST array of `count`
 * nondecreasing integers; equal values form one stage).  The products of a
 * stage are independent; a product's x may be the y of a product in an
 * earlier stage (a layer's output feeding the next layer), and sees that y
 * complete.  Within a stage no y may overlap another y or any x of the stage.
 * Each stage is the batched call over its matrices (one launch per bit
 * width), enqueued back to back in one call (a HIP graph can capture it), so
 * a stage's products come out exactly as qw_gemv_batched computes the same
 * group.  A decode step of many short kernels is dominated by their fixed
 * cost (page "Huit bits, puis quatre", section "La vitesse"), which the
 * stage grouping keeps to one launch per dependency level.  Validation as in
 * qw_gemv_batched, plus QW_ECOUNT when `stage` is NULL or decreases.
 */
int qw_gemv_chain(int count, const qw_gemv_desc* descs, const int32_t* stage, int64_t m,
                  void* stream);

/*
 * Dequantizing GEMM (prefill), bf16 matrix cores, fp32 accumulate:
 *   x_bf16  bf16 bit patterns [m][k]  (read),   y  fp32 [m][n]  (written).
 * Any group dividing n*k is accepted; k % 64 == 0 with k % group == 0 and
 * group % 32 == 0 (or group % k == 0) takes the MFMA kernel.
 */
int qw_gemm(int bits, int64_t group, int64_t n, int64_t k,
            const uint8_t* payload, const float* scales,
            int64_t m, const uint16_t* x_bf16, float* y, void* stream);

/*
 * QuantizedMatmul for any number of rows (page "Huit bits, puis quatre",
 * section "Ranger des entiers dans des f32": the generation products read
 * the codes, where the time goes to memory; the large products of an
 * evaluation use the dequantized weights, where it goes to arithmetic):
 *   x  fp32 [m][k]  (read),   y  fp32 [m][n]  (written),   m >= 0.
 * m <= QW_MATMUL_GEMV_MAX_M is qw_gemv itself: fp32 arithmetic on the codes,
 *   error <= 1e-5 * sum_j |x[m][j] * w_hat[i][j]|; no work buffer is needed.
 * 5 <= m <= 8 is also qw_gemv when the matrix has at most 8192 rows and
 *   qw_gemv's matrix-core kernel takes it (measured faster there than the
 *   GEMM, and more precise); `work` is then left untouched.
 * Otherwise x is rounded to bf16 (round to nearest even) into `work` and
 *   qw_gemm runs on it: the weights are dequantized in registers, not kept
 *   as a second copy.  Error <= 8e-3 * sum_j |x[m][j] * w_hat[i][j]|
 *   (rounding x adds at most 2^-9 of it to the GEMM's own bound).
 * The bound sits at the measured crossover on MI355X (int4 g128, 4096- to
 * 28672-row matrices: the GEMV is faster up to 3 rows on each, up to 6 on
 * the 4096-row one, the GEMM from 8 on each; at 4 rows the two are within
 * 10% on the wider matrices and the GEMV 22% faster on the 4096-row one, so
 * 4 rows stay on the more precise product).
 * `work`: a device buffer of at least qw_matmul_work_bytes(m, k)
 * bytes (may be NULL when that is 0); after a GEMM call it holds the bf16
 * bit patterns of x, row-major.  QW_EWORK when it is missing or too small;
 * other validation as in qw_gemv / qw_gemm.
 */
#define QW_MATMUL_GEMV_MAX_M 4
int64_t qw_matmul_work_bytes(int64_t m, int64_t k);
int qw_matmul(int bits, int64_t group, int64_t n, int64_t k,
              const uint8_t* payload, const float* scales,
              int64_t m, const float* x, float* y,
              void* work, int64_t work_bytes, void* stream);

/*
 * qw_matmul for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as qw_matmul (bit-identical outputs: the same
 * kernels run), without the work buffer: the bf16 copy of x goes to a
 * static device array of QW_MATMUL_NOALLOC_MAX_BYTES that the library holds
 * on every GPU it runs on until the process ends.  The call allocates and
 * frees nothing.
 *   - m * k * 2 (the bytes of x in bf16) above QW_MATMUL_NOALLOC_MAX_BYTES,
 *     for m > QW_MATMUL_GEMV_MAX_M, returns QW_ESCRATCH and enqueues
 *     nothing; up to QW_MATMUL_GEMV_MAX_M rows no scratch is used.
 *   - The scratch of the CURRENT device is used; `stream` (if not NULL)
 *     must belong to that device (QW_EARG otherwise).  Its address is looked
 *     up on the first call on each device.
 *   - Every call on one GPU shares that GPU's array: two calls whose work
 *     overlaps in time on one GPU (different streams, or host threads) race
 *     and give undefined results.  Calls ordered on one stream are safe.
 */
#define QW_MATMUL_NOALLOC_MAX_BYTES (32ll << 20)
int qw_matmul_noalloc(int bits, int64_t group, int64_t n, int64_t k,
                      const uint8_t* payload, const float* scales,
                      int64_t m, const float* x, float* y, void* stream);

/*
 * GPTQ codes (page "Huit bits, puis quatre", section "Arrondir mieux :
 * GPTQ").  Rounding every weight to its nearest code minimises each weight's
 * error, not the error of the layer's output X W^T on typical inputs X.
 * GPTQ rounds the input components (columns of the [n][k] weight) one after
 * the other and carries each rounding error onto the later components of
 * the same output channel, weighted by how correlated their inputs are.
 * What it needs from the inputs is H = sum x^T x over some calibration
 * tokens; the carrying factors are the rows of U, the upper triangular
 * factor of H^-1 = U^T U after H is damped by a fraction (the page: 1 %) of
 * its mean diagonal.  For component c of every channel, in order:
 *
 *   when c starts a group: S = fl32(max |fl32(w)| over the group's
 *                          current weights / qmax), 1 if zero
 *   q      = clip(round_half_even(fl32(fl32(w_c) / S)), -qmax, qmax)
 *   e      = (w_c - fl32(q * S)) / U[c][c]
 *   w_j   -= e * U[c][j]                      for every j > c
 *
 * The result uses the same payload and scale format as qw_quantize_pack
 * (so qw_unpack, qw_gemv and qw_gemm take it unchanged); with a diagonal H
 * it is bit-identical to qw_quantize_pack.  All of H, U and the carried
 * weights are fp64.  Three steps, each enqueued on `stream` like the other
 * entry points; each takes a caller-owned device work buffer of at least
 * the size its *_work_bytes query returns (contents undefined on return,
 * not shared between calls in flight).
 */

/* Work bytes for qw_gptq_hessian (-1 if k or t is negative). */
int64_t qw_gptq_hessian_work_bytes(int64_t k, int64_t t);

/*
 * Calibration accumulation: h += x^T x.
 *   x  fp32 [t][k] row-major, one row per token          (read)
 *   h  fp64 [k][k], symmetric                            (read-write)
 * The per-layer accumulator the page's calibration adds to before each
 * product; call once per batch.  Deterministic for given shapes.  t == 0 or
 * k == 0 enqueues nothing.
 */
int qw_gptq_hessian(int64_t k, int64_t t, const float* x, double* h,
                    void* work, int64_t work_bytes, void* stream);

/* Work bytes for qw_gptq_factor (-1 if k is negative). */
int64_t qw_gptq_factor_work_bytes(int64_t k);

/*
 * Damping and factor: u (fp64 [k][k], written) is upper triangular with
 * zeros below the diagonal and (h + damp * mean(diag h) * I)^-1 = u^T u.
 *   h     fp64 [k][k] symmetric (read)
 *   damp  fraction of the mean diagonal added to it (the page uses 0.01);
 *         finite and >= 0, else QW_EARG
 *   info  DEVICE int32 (written, may be NULL): 0 on success; 1 if the mean
 *         diagonal is not positive or the damped matrix is not positive
 *         definite, in which case u is undefined.  Read it after the stream
 *         synchronizes; the call itself does not wait.
 */
int qw_gptq_factor(int64_t k, const double* h, double damp, double* u, int32_t* info,
                   void* work, int64_t work_bytes, void* stream);

/* Work bytes for qw_gptq_quantize_pack (-1 if invalid). */
int64_t qw_gptq_quantize_work_bytes(int64_t n, int64_t k);

/*
 * GPTQ codes of one weight.
 *   w        fp32 [n][k]                        (read)
 *   u        fp64 [k][k] from qw_gptq_factor    (read; only its upper
 *            triangle is used)
 *   payload  uint8 [qw_payload_bytes(bits,n,k)] (written)
 *   scales   fp32 [qw_num_scales(group,n,k)]    (written)
 * group must divide k (a group lies inside one output channel) and be even
 * for int4; QW_EGROUP otherwise.  Matrices that share an input (and so an
 * H) can be stacked along n into one call.
 */
int qw_gptq_quantize_pack(int bits, int64_t group, int64_t n, int64_t k,
                          const float* w, const double* u,
                          uint8_t* payload, float* scales,
                          void* work, int64_t work_bytes, void* stream);

/*
 * Diagnostic: which kernel family a call with these arguments would take
 * (1 = streaming/tiled fast kernel, 2 = block-per-group kernel, 3 = generic
 * kernel, 4 = matrix-core GEMV) or a negative status for invalid arguments.
 * `op`: 0 quantize_pack (a = w, b = payload), 1 unpack (a = payload, b =
 * w_out), 2 gemv at one row of x (a = payload, b = x), 3 gemm (a = payload,
 * b = x_bf16), 4 gemv at 8 rows of x (a = payload, b = x; at fewer rows the
 * matrix-core kernel runs from the row counts qw_gemv states), 5 qw_matmul
 * at 5..8 rows of x (a = payload, b = x): 1 = it runs qw_gemv, 2 = the
 * GEMM.  Enqueues nothing.
 */
int qw_debug_path(int op, int bits, int64_t group, int64_t n, int64_t k,
                  const void* a, const void* b);

#ifdef __cplusplus
}
#endif

#endif /* QW_H */
