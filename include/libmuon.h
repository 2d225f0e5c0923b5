/*
 * libmuon — the Muon / Aurora-Muon matrix-optimizer step on AMD Instinct
 * MI355X (gfx950), as a C-ABI shared library.
 *
 * The operations follow two web pages:
 *   [Aurora page]  "modded-nanogpt Track 3 优化实录：Aurora 行均衡 polar +
 *                  Contra-Muon + u/w-floor 将 3.28 验证损失推进到 3175 步"
 *                  (www.xxmr.cn/news/295280);
 *   [Track-1 page] "Modded-NanoGPT 纪录解读：U-Net 式跳跃连接与学习率翻倍如何将
 *                  124M GPT 训练压到 7.23 分钟" (www.trdm.cn/news/788905).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Matrices are row-major, in device memory the caller owns. A descriptor
 *    names one matrix: element (i, j) lives at ptr + i * ld + j (elements).
 *    ld >= cols. ptr must be aligned to the element size. A matrix with
 *    rows == 0 or cols == 0 is skipped (its ptr may be NULL).
 *  - Batches: every call takes n descriptors of mixed shapes and types; each
 *    matrix is processed on its own (its own norms, preconditioner and power
 *    iteration) and the batch is fused into shared kernel launches.
 *  - Limits: rows, cols <= 65536, min(rows, cols) <= 16384,
 *    rows * cols < 2^31 and ld <= 2^40 per matrix.
 *  - Precision: a matrix whose input is MUON_BF16 runs Newton-Schulz on bf16
 *    matrix cores with fp32 accumulation; a MUON_F32 input runs it with fp32
 *    matrix-core arithmetic throughout. Norms, the preconditioner, the power
 *    iteration and every scalar are fp32.
 *  - Errors: no exception crosses the ABI. Calls return a muon_status; a
 *    negative value is an error. All arguments are validated on the host
 *    before anything is enqueued: on any error nothing is enqueued and no
 *    caller buffer is touched. muon_last_error() gives a message. (With
 *    MUON_FLAG_CHECK_FINITE a read-only device pass also checks the input
 *    values; a non-finite one is reported the same way, no buffer written.)
 *  - Asynchrony: compute calls enqueue on the handle's stream and return.
 *    Inputs must stay valid and unmodified until that stream reaches the
 *    work. Device faults surface as MUON_ERR_HIP on a later call or on the
 *    caller's synchronisation.
 *  - Determinism: reductions run in a fixed order with no floating-point
 *    atomics; two calls on the same inputs give bitwise-equal results.
 *  - Threads: a handle is not thread-safe; use one handle per thread.
 */
#ifndef LIBMUON_H
#define LIBMUON_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
  MUON_F32 = 0,
  MUON_BF16 = 1
} muon_dtype;

/* Status codes. */
typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = -1,      /* NULL pointer, bad count, bad config value */
  MUON_ERR_UNSUPPORTED_DTYPE = -2,/* dtype not in muon_dtype, or momentum not F32 */
  MUON_ERR_SHAPE_MISMATCH = -3,   /* grad/momentum/weight/out shapes differ, ld < cols, limits */
  MUON_ERR_ALLOC = -4,            /* device workspace allocation failed */
  MUON_ERR_HIP = -5,              /* a HIP runtime call failed */
  MUON_ERR_NO_DEVICE = -6,        /* no usable gfx950 device */
  MUON_ERR_TOO_LARGE = -7,        /* muon_update_static: the batch does not fit the static scratch */
  MUON_ERR_NONFINITE = -8         /* MUON_FLAG_CHECK_FINITE: an input element is NaN or Inf */
} muon_status_code;
typedef int muon_status;

/* One row-major device matrix (see conventions above). */
typedef struct {
  void*   ptr;
  int64_t rows;
  int64_t cols;
  int64_t ld;
  int32_t dtype; /* muon_dtype */
} muon_matrix;

/*
 * Step hyper-parameters. muon_config_default() fills the values the Aurora
 * page locks (§"完整的超参配置表" and the signature defaults in §"源码实现" and
 * §"组合优化栈"): ns_steps 12, (ns_a, ns_b, ns_c) = (2, -1.5, 0.5),
 * ns_eps 1e-7, pp_iterations 2, pp_beta 0.5, pp_eps 1e-7, mu 0.95,
 * nesterov 1, power_steps 5, contra 0.4, target_uw 0.35, lr 0.0375, flags 0.
 *
 *   ns_steps, ns_a/b/c  Newton-Schulz iteration count and polynomial
 *                       X <- a X + (b A + c A^2) X, A = X X^T (1..64 steps).
 *   ns_eps              added to the Frobenius norm before normalising.
 *   pp_iterations       Aurora passes (0 = plain NS, no preconditioner; 1 =
 *                       row-normalise then polar; 0..8).
 *   pp_beta, pp_eps     damping exponent of the D update; clamp of row norms
 *                       (pp_eps) and squared row norms (pp_eps^2).
 *   mu, nesterov        momentum coefficient in [0, 1]; Nesterov blend flag.
 *   power_steps         power iterations for the operator-norm estimate (1..64).
 *   contra              Contra-Muon coefficient; the step subtracts contra/2
 *                       times the unit-operator-norm direction (0 = off).
 *   target_uw           u/w-floor target ratio (0 = off).
 *   lr                  learning rate of the parameter add.
 *   flags               bitwise OR of MUON_FLAG_* below (0 = the Aurora
 *                       page's step); unknown bits are rejected
 *                       (MUON_ERR_INVALID_ARG).
 */
typedef struct {
  int32_t  ns_steps;
  float    ns_a, ns_b, ns_c, ns_eps;
  int32_t  pp_iterations;
  float    pp_beta, pp_eps;
  float    mu;
  int32_t  nesterov;
  int32_t  power_steps;
  float    contra;
  float    target_uw;
  float    lr;
  uint32_t flags;
} muon_config;

/*
 * MUON_FLAG_SGD_MOMENTUM — the momentum form of the classic Muon recipe,
 * [Track-1 page] §"训练管线与系统实现" ("SGD momentum" with Nesterov), read as
 * the heavy-ball buffer with no dampening: M <- mu M + G, X = G + mu M
 * (X = M without Nesterov). Without the flag the step keeps the Aurora page's
 * moving average, M <- M + (1 - mu)(G - M), X = G + mu (M - G). The two give
 * the same direction at constant mu from a zero buffer (the buffers differ
 * by 1/(1 - mu)) and different ones under a momentum warm-up.
 * muon_config_classic sets it.
 *
 * MUON_FLAG_WIDE_ROWS — [Aurora page] §"复现与扩展建议" names a later result
 * that applies the row-balanced polar to a wide matrix (the MLP output
 * projection) and gives no formula. With this flag a wide matrix (rows <
 * cols) is equilibrated on its own rows, the short side: D = 1/max(row
 * norm, pp_eps), then the same damped update with target 1 (the squared
 * row norm of a polar factor with orthonormal rows). Tall and square
 * matrices are unaffected. Since such a polar factor's rows are already
 * orthonormal, later passes move D only where Newton-Schulz has not
 * converged; pp_iterations 1 is row-normalise-then-polar on the rows.
 *
 * MUON_FLAG_FP8_GRAM — lower-precision Newton-Schulz, a research option (not
 * from the pages, which run the optimizer's products in their training
 * precision; the 3.8B page uses FP8 only for the model's GEMMs, in its
 * post-mortem). For bf16 matrices that run Newton-Schulz in blocks
 * (rectangular, short side >= 512), the first Gram of each pass, A = X0 X0^T
 * with K = the long side, reads an fp8 (OCP e4m3) copy of X0 written by the
 * pass prologue with a per-matrix power-of-two scale q (q |X0| <= 448,
 * bounded by the largest equilibrated line or row norm), runs on the fp8
 * matrix cores and divides by q^2 in its epilogue. The sums over the long
 * side average the operands' rounding: measured error stays at the bf16
 * path's level (about 5e-3 relative Frobenius). Later Grams, the short-side
 * products and X' = Q X stay bf16 (fp8 there costs 1e-2 to 5e-2).
 *
 * MUON_FLAG_CHECK_FINITE — an input check for callers that want a NaN or
 * Inf to stop the step instead of spreading through it (the pages define
 * no such check; without the flag a non-finite input gives non-finite
 * results for its matrix only). Before anything is written, one read-only
 * pass over every matrix's grad (the polar input), momentum and weight
 * looks for NaN or Inf; the call then waits for that pass on its stream
 * (the one case where a compute call synchronises). If any element is not
 * finite the call returns MUON_ERR_NONFINITE, names the first such matrix
 * in muon_last_error(), and leaves every caller buffer as it was;
 * otherwise the step runs as without the flag, with bitwise-equal results.
 * Costs one read of the inputs and the synchronisation.
 */
#define MUON_FLAG_SGD_MOMENTUM 0x1u
#define MUON_FLAG_WIDE_ROWS    0x2u
#define MUON_FLAG_FP8_GRAM     0x4u
#define MUON_FLAG_CHECK_FINITE 0x8u
#define MUON_FLAG_ALL          0xFu

/* Per-kernel-class timing gathered when profiling is on (see muon_profile_*).
   Each *_ms is the wall time the class's event pairs cover: their summed
   durations less the time they overlap (launches on the handle's second
   stream run beside those on the call's stream). */
typedef struct {
  int64_t gemm_launches;      /* Newton-Schulz matrix-core launches */
  double  gemm_ms;            /* event time of those launches */
  double  gemm_counted_flop;  /* 4 s^2 L + 2 s^3 per iteration per matrix (s <= L) */
  double  gemm_executed_flop; /* flops the tiles actually issue (symmetric results' lower tiles
                                 skipped, and on their diagonal tiles the 32x32 blocks wholly
                                 below the diagonal) */
  double  gemm_algorithmic_flop; /* flops the products need: the upper half of each symmetric
                                    result, no padding (3 s^2 L + (4 r - 3) s^3 per block of r
                                    iterations) */
  int64_t stream_launches;    /* bandwidth-bound launches of the step itself: momentum and
                                 norms, the weight norm, power iteration, tail (and the latency
                                 kernels between) */
  double  stream_ms;
  double  stream_bytes;       /* algorithmic HBM bytes of those launches */
  int64_t aux_launches;       /* Aurora vector kernels feeding the products: the pass prologue
                                 (X0 = scale D o T in one or both orientations) and the D update */
  double  aux_ms;
  double  aux_bytes;          /* HBM bytes of those launches (source read, iterate pair written;
                                 D update: one read of U) */
} muon_profile;

typedef struct muon_handle muon_handle;

/* Fill *cfg with the page's locked values (listed above). cfg must not be NULL. */
void muon_config_default(muon_config* cfg);

/*
 * Fill *cfg with the classic Muon recipe of the Track-1 record page
 * (§"训练管线与系统实现"): SGD momentum 0.95 with Nesterov
 * (flags = MUON_FLAG_SGD_MOMENTUM), Newton-Schulz with
 * (ns_a, ns_b, ns_c) = (3.4445, -4.7750, 2.0315) for ns_steps 5, no Aurora
 * preconditioner (pp_iterations 0), no Contra term (contra 0), no u/w-floor
 * (target_uw 0), the sqrt(max(1, rows/cols)) scale, lr 0.04. The remaining
 * fields keep muon_config_default's values. cfg must not be NULL.
 * That recipe's fixed point is deliberately not 1, so its update is not an
 * exact orthogonalisation.
 */
void muon_config_classic(muon_config* cfg);

/*
 * Momentum warm-up of the same page: frac = min(step / warmup_steps, 1),
 * mu = (1 - frac) * mu_start + frac * mu_end (the page uses 0.85 -> 0.95
 * over 500 steps). A host-side scalar for muon_config.mu; step < 0 counts as
 * 0, warmup_steps <= 0 returns mu_end. Computed in double, returned as float.
 */
float muon_momentum_warmup(int64_t step, float mu_start, float mu_end, int64_t warmup_steps);

/* Static text for a status code. Never NULL. */
const char* muon_status_string(muon_status s);

/* Library version string ("major.minor.patch"). */
const char* muon_version(void);

/*
 * Create a handle bound to the current HIP device and to `stream`
 * (a hipStream_t; NULL = the default stream). The stream is borrowed, not
 * owned. The handle owns its device workspace and plan cache; both grow on
 * demand and are freed by muon_destroy. It also owns a second stream of
 * default priority, made by the first call that uses it: on sets whose
 * product launches are small, a call runs part of each Newton-Schulz pass
 * there (the one-iteration matrices beside the blocked ones, or half of a
 * set with only one kind), and `stream` waits for it before the pass ends,
 * so every call still completes in order on `stream`. Returns
 * MUON_ERR_NO_DEVICE when no gfx950 device is current.
 *
 * Tuning (environment). The layout and tile edge give bitwise the default's
 * results; a forced block length changes the rounding only:
 *   MUON_NS_VARIANT=1      read here: Newton-Schulz products on 256x256 tiles
 *                          with 4 waves of 128x128 instead of 8 of 64x128.
 *   MUON_NS_TILE=128|256   read when a plan is built (first call with a new
 *                          set of shapes): force the product tile edge;
 *                          otherwise launches with fewer than 768 256-tiles
 *                          use 128-tiles.
 *   MUON_NS_BLOCK=1..8     read when a plan is built: Newton-Schulz
 *                          iterations per block for every rectangular matrix
 *                          (default 4 where the coefficients allow, below 512
 *                          on the short side 1).
 *   MUON_NS_SIDE=0|1       read here: 0 keeps every launch on `stream`, 1
 *                          uses the second stream in every pass that has
 *                          both one-iteration and blocked matrices, however
 *                          large (bitwise the same results either way).
 *   MUON_FUSED_TAIL=0      read when a plan is built: bf16 matrices of
 *                          muon_update take the tail's norms in a reduction
 *                          pass over U, X and W (and the operator-norm
 *                          estimate in its own X v launch) instead of in the
 *                          final Newton-Schulz product's epilogue and a
 *                          read-only pass over W (the same sums in another
 *                          order).
 *   MUON_TALL_X0=0         read when a plan is built: bf16 matrices of
 *                          muon_update with both sides multiples of 256 get
 *                          both orientations of the pass's first iterate
 *                          from the prologue, instead of the first X' = Q X
 *                          (tall matrices) or the first Gram (wide or square
 *                          ones without the preconditioner) reading the
 *                          blended update and scaling its output (the
 *                          same products, rounded once less).
 * Tracing: MUON_ROCTX=1, read here, wraps each phase of a call (momentum,
 * power iteration, each Newton-Schulz pass, the Aurora D update, the tail)
 * in a ROCTx range for rocprofv3 --marker-trace; the ROCTx library is loaded
 * at run time and the ranges are skipped when it is absent.
 */
muon_status muon_create(muon_handle** handle, void* stream);

/* Free the handle and its workspace (waits for the stream first). NULL is a no-op. */
muon_status muon_destroy(muon_handle* handle);

/* Rebind the handle to another stream of the same device. */
muon_status muon_set_stream(muon_handle* handle, void* stream);

/* Message of the handle's last error ("" if none). Valid until the next call. */
const char* muon_last_error(const muon_handle* handle);

/*
 * Host-only validation of a muon_update batch with the same rules as
 * muon_update; enqueues nothing and needs no device. weight and update_out
 * may be NULL. msg (may be NULL) receives a message of up to msg_len bytes.
 */
muon_status muon_check_update_args(int n, const muon_matrix* grad,
                                   const muon_matrix* momentum,
                                   const muon_matrix* weight,
                                   const muon_matrix* update_out,
                                   const muon_config* cfg,
                                   char* msg, int msg_len);

/* Host-only validation of an ns_polar / aurora_orthogonalize batch. */
muon_status muon_check_polar_args(int n, const muon_matrix* in,
                                  const muon_matrix* out,
                                  const muon_config* cfg,
                                  char* msg, int msg_len);

/*
 * Host-only consistency check of the launch plan a compute call would build
 * for a batch (for tests and for debugging the planner; needs no device).
 * kind: 0 muon_update, 1 ns_polar, 2 aurora_orthogonalize; only rows, cols
 * and dtype of `shapes` are read; cfg may be NULL (defaults). It checks that
 * every workspace region lies inside the workspace and overlaps no other;
 * that every tile of every Newton-Schulz product list lies inside its
 * matrix's padded tile grid and sits in the list of that matrix's pass,
 * block length class and element type; that every tile a product needs is
 * listed exactly once (the upper triangle of the symmetric products, the
 * whole grid of X' = Q X); and that the streaming launch lists have
 * consistent block offsets (the momentum pass's n_rt x n_seg tiles per
 * matrix). Returns MUON_OK, or MUON_ERR_INVALID_ARG with the first violation
 * in msg (NUL-terminated, at most msg_len bytes); shapes past the library's
 * limits give MUON_ERR_SHAPE_MISMATCH.
 */
muon_status muon_debug_check_plan(int kind, int n, const muon_matrix* shapes,
                                  const muon_config* cfg, char* msg, int msg_len);

/*
 * Grow the workspace so that batches with these shapes and types run without
 * any further device allocation (so a timed or captured region allocates
 * nothing). Only rows, cols and dtype of `shapes` are read.
 */
muon_status muon_reserve(muon_handle* handle, int n, const muon_matrix* shapes);

/*
 * ns_polar — out_i = NS(in_i): the Newton-Schulz approximation of the polar
 * factor, [Aurora page] §"源码实现" (the shared NS primitive): divide by the
 * Frobenius norm + ns_eps, then ns_steps times X <- a X + (b A + c A^2) X with
 * A = X X^T formed on the short side.
 *   in[i]   input, any shape, F32 or BF16; read only.
 *   out[i]  output, same shape as in[i], F32 or BF16 (rounded to nearest
 *           even). An output may share memory with any input, in place or
 *           not: every input is read before the first output is written.
 *           Outputs must not share an element with one another
 *           (MUON_ERR_INVALID_ARG); column slices of one buffer do not.
 *   cfg     ns_* fields are used; NULL = defaults.
 */
muon_status ns_polar(muon_handle* handle, int n, const muon_matrix* in,
                     const muon_matrix* out, const muon_config* cfg);

/*
 * aurora_orthogonalize — leverage-equilibrated polar, [Aurora page]
 * §"Aurora 是什么", §"Aurora 的迭代伪代码" and §"源码实现": square inputs get
 * plain NS; otherwise, in the tall orientation (m > n), D = 1/max(row norm,
 * pp_eps) and pp_iterations passes of U = NS(D * G), multiplying D by
 * (n/m / max(row_sq, pp_eps^2))^pp_beta between passes. Wide inputs are
 * handled as their transpose without materialising it.
 *   in, out, cfg as for ns_polar (pp_* and ns_* fields used).
 */
muon_status aurora_orthogonalize(muon_handle* handle, int n,
                                 const muon_matrix* in, const muon_matrix* out,
                                 const muon_config* cfg);

/*
 * muon_update — one Aurora + Contra-Muon + u/w-floor optimizer step,
 * [Aurora page] §"组合优化栈" (muon_update, the Contra-Muon and u/w-floor
 * parts) and §"完整的超参配置表":
 *   M <- M + (1 - mu)(G - M); X = G + mu (M - G) (X = M without Nesterov);
 *   N = X / max(sigma, 1e-7), sigma from power_steps power iterations on
 *   X^T X started from ones/sqrt(cols) (restart from the first largest-norm
 *   column if that start is annihilated);
 *   U = aurora_orthogonalize(X); V = U - (contra/2) N, rescaled to ||U||_F
 *   (clamp 1e-10); V *= sqrt(max(1, rows/cols));
 *   if ||V||/||W|| < target_uw (both clamped at 1e-8): V *= target_uw ||W||/||V||;
 *   W <- W - lr V.
 *   grad[i]       G, F32 or BF16; read only (unlike the page's in-place
 *                 lerp, the blended update goes to workspace).
 *   momentum[i]   M, F32, same shape; updated in place.
 *   weight        NULL, or weight[i] = W (F32 or BF16, same shape) updated in
 *                 place (bf16 rounded to nearest even); weight[i].ptr NULL
 *                 means no weight (and no floor) for matrix i.
 *   update_out    NULL, or update_out[i] receives V after the floor and
 *                 before lr (F32 or BF16; ptr NULL = not wanted).
 *   cfg           NULL = defaults.
 * Every buffer the call writes (momentum, weight, update_out) must not share
 * an element with any other buffer of the call, of the same matrix or
 * another: MUON_ERR_INVALID_ARG names the first such pair. Grads may share
 * memory with one another (they are only read), and column slices of one
 * buffer (same ld, disjoint columns) share no element.
 */
muon_status muon_update(muon_handle* handle, int n, const muon_matrix* grad,
                        const muon_matrix* momentum, const muon_matrix* weight,
                        const muon_matrix* update_out, const muon_config* cfg);

/*
 * muon_update_static — muon_update for callers that cannot allocate device
 * memory during the call: code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid allocation. Same arguments, rules,
 * validation, kernels and results as muon_update (bitwise), but the call
 * allocates nothing: its workspace and launch tables live in a file-scope
 * device array of 64 MiB per device (held until the process ends; its
 * address is taken once per device by muon_create, and a pinned 1 MiB table
 * stage is allocated there too), and no profiling events are recorded.
 *   Limit: the batch's workspace plus its launch tables must fit the 64 MiB
 *   (for example one 1024 x 3072 bf16 matrix, or a few 768 x 768 ones, with
 *   tables within 1 MiB); larger batches return MUON_ERR_TOO_LARGE with a
 *   message giving the bytes needed, before anything is enqueued.
 *   Sharing: every static call on a device uses that device's one array and
 *   leaves its contents there (nothing in it needs clearing: every call
 *   writes each part before reading it). Static calls that can overlap on
 *   one device (other handles, other streams) race: order them, e.g. on one
 *   stream.
 */
muon_status muon_update_static(muon_handle* handle, int n, const muon_matrix* grad,
                               const muon_matrix* momentum, const muon_matrix* weight,
                               const muon_matrix* update_out, const muon_config* cfg);

/*
 * Profiling of the library's own launches (for roofline reporting): when
 * enabled, each kernel launch is bracketed by HIP events on the handle's
 * stream and its time, its algorithmic flops or bytes are added to totals.
 * muon_profile_read synchronises those events and returns the totals since
 * the last reset.
 */
muon_status muon_profile_enable(muon_handle* handle, int enable);
muon_status muon_profile_reset(muon_handle* handle);
muon_status muon_profile_read(muon_handle* handle, muon_profile* out);

#ifdef __cplusplus
}
#endif

#endif /* LIBMUON_H */
