/*
 * lla.h -- C ABI of the causal Local Linear Attention (LLA) forward library
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b, head h and query row i; j runs over the
 * causal prefix 0..i, diagonal included). Source: "Local Linear Attention:
 * reading notes" on arXiv:2510.01450 (Zuo et al.), section 2.1, Eqs. (6)-(8):
 *
 *   s_ij    = c q_i . k_j,   c = 1/sqrt(d)
 *   w_ij    = exp(s_ij - max_{l<=i} s_il)           (largest weight is 1)
 *   z_ij    = k_j - q_i
 *   omega_i = sum_j w_ij,   mu_i = sum_j w_ij z_ij
 *   Sigma_i = sum_j w_ij z_ij z_ij^T + lambda I,   rho_i = Sigma_i^{-1} mu_i
 *   out_i   = sum_j w_ij (1 - z_ij^T rho_i) v_j / (omega_i - mu_i^T rho_i)
 *
 * i.e. the intercept of a kernel-weighted ridge regression of v on k around
 * q_i. How it is computed follows the blocked three-phase scheme of section
 * 2.2 (Algorithm 1) of the same page: per block of queries, (1) one scan over
 * the key blocks with an online row max accumulates omega_i and
 * mu~_i = sum_j w_ij k_j (Eqs. (10)-(11)); (2) matrix-free conjugate gradient,
 * each iteration re-scanning the key blocks to form a Gram-matrix product
 * (Eq. (12)); (3) a scan over the key/value blocks accumulates the output.
 * The n x n weights are never stored; working memory is linear in n.
 *
 * The CG of phase (2) runs on the system centred at the weighted key mean
 * kbar_i = mu~_i / omega_i instead of at q_i:
 *     Sigma_c = sum_j w_ij (k_j - kbar_i)(k_j - kbar_i)^T + lambda I
 *             = Sigma~_i - mu~_i mu~_i^T / omega_i,      Sigma_c rho_c = mu_i,
 *     out_i   = sum_j w_ij (1 - (k_j - kbar_i)^T rho_c) v_j / omega_i.
 * Since Sigma_i = Sigma_c + omega_i (kbar_i - q_i)(kbar_i - q_i)^T and
 * mu_i = omega_i (kbar_i - q_i), this is the same output exactly (Sherman-
 * Morrison), with rho_i = rho_c / (1 + (kbar_i - q_i)^T rho_c); it avoids the
 * division by the Schur complement omega_i - mu_i^T rho_i, which amplifies
 * any error in an unconverged CG iterate by omega_i / (omega_i - mu_i^T rho_i).
 *
 * CG policy (the pages leave it to an appendix that is not reproduced): x0 = 0,
 * r0 = p0 = mu_i; a query stops at the first k with ||r_k|| <= tol ||r_0||
 * (recurrence residual), on breakdown (p^T Sigma_c p <= 0 or r = 0), or at
 * k = cg_max_iters. cg_rel_tol = 0 runs exactly cg_max_iters steps;
 * cg_max_iters = 0 gives rho = 0, i.e. causal softmax attention. A stopped
 * query freezes while the rest of its block continues. Non-convergence is not
 * an error: it is reported through cg_iters / cg_resid.
 *
 * Conventions common to every entry point:
 *  - Tensors are DEVICE pointers, contiguous row-major [B][H][n][d] (d
 *    fastest), 16-byte aligned; value dimension = key dimension = d.
 *  - Inputs are never written. `out` (fp32) and every non-NULL optional
 *    output are fully written. The library keeps no pointer after the call
 *    and no state between calls; calls are reentrant and thread safe.
 *  - Asynchronous: the call returns after enqueueing work on `stream`
 *    (NULL = the default stream); the caller synchronises. Device faults
 *    surface at that synchronisation.
 *  - Validation runs on the host before any device work; on failure nothing
 *    is enqueued or written and a negative status is returned, with detail in
 *    lla_last_error().
 *  - NaN/Inf inputs are not checked; they propagate, but never to another
 *    head. Within a head, a NaN in q_i reaches output row i; a NaN in k_j or
 *    v_j reaches the rows from 32*floor(j/32) on (the diagonal tile is
 *    computed for 32 queries at once, and 0 * NaN is NaN). On the
 *    matrix-core path an infinite input changes its head's power-of-two
 *    scale, and with it the whole head.
 *  - Range on the matrix-core path: a head's keys take one power-of-two
 *    scale s (largest key row norm to (64, 128]) and its values another;
 *    both are then fp16. Queries enter the scores as q log2(e) / (sqrt(d) s)
 *    in fp16. The scales absorb key row norms from about 2^-93 to 2^106 and
 *    value rows of any bf16 magnitude. Within a head, key and value rows
 *    down to about 2^-17 of the head's largest keep full fp16 precision;
 *    smaller ones lose it gradually (fp16 subnormals; at 2^-20 the outputs
 *    stay within 2e-2). Limits: the query operand
 *    overflows when a query row norm times a key row norm exceeds about 2^25
 *    (score differences beyond a million nats); and where the fit
 *    extrapolates far outside its keys (|(k_j - kbar) . rho| >> 1, outputs
 *    many times the size of the values) the output scan's single fp16 term
 *    per weight loses the cancellation. The fp32 vector path has neither
 *    limit.
 */
#ifndef LLA_H
#define LLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLA_VERSION 100 /* 1.0.0 */

/* Status codes. */
enum {
  LLA_OK = 0,
  LLA_ERR_INVALID_ARG = -1, /* NULL required pointer, B/H/n < 1, lambda not
                               finite or <= 0, cg_max_iters < 0 or > 100000,
                               cg_rel_tol < 0 or NaN, out overlapping an
                               input, misaligned pointer, unknown dtype,
                               kernel or flag */
  LLA_ERR_UNSUPPORTED = -2, /* d not in {16, 32, 64, 128}; a kernel choice
                               not available for the dtype/d; sizes too
                               large: B*H >= 2^31, B*H*n > 2^40, n > 2^23
                               (forward, output given rho), n > 2^21 with
                               LLA_KERNEL_MFMA (forward) or on any path
                               (backward); decode: B*H > 65535, B*H*n > 2^36
                               or one head's cache (n*d elements) of 2 GiB
                               or more. Checked on the host before anything
                               is allocated or enqueued */
  LLA_ERR_HIP = -3,         /* a HIP launch or allocation failed */
  LLA_ERR_WORKSPACE = -4    /* caller workspace smaller than required */
};

/* Element type of q, k, v. */
enum { LLA_DTYPE_F32 = 0, LLA_DTYPE_BF16 = 1 };

/* Kernel selection for lla_forward_ex. */
enum {
  LLA_KERNEL_AUTO = 0, /* bf16 inputs with d in {64,128} and n <= 2^21: MFMA;
                          otherwise (fp32 inputs, other d, longer n) VALU */
  LLA_KERNEL_VALU = 1, /* fp32 vector-ALU kernel, any supported d/dtype,
                          n <= 2^23 */
  LLA_KERNEL_MFMA = 2  /* fp16 matrix-core kernel; bf16 inputs, d in {64,128},
                          n <= 2^21 (LLA_ERR_UNSUPPORTED otherwise) */
};

/* Flags for lla_forward_ex (bitwise OR). */
enum {
  LLA_FLAG_SPLIT_U = 1,    /* MFMA kernel: carry the CG tile W*(K p) as two fp16
                              terms (hi + lo) instead of one; slower, more exact */
  LLA_FLAG_PRECOND = 2,    /* MFMA kernel: preconditioned CG (below) whatever
                              the tolerance */
  LLA_FLAG_NO_PRECOND = 4  /* MFMA kernel: plain CG whatever the tolerance */
};
/* Preconditioned CG (matrix-core path). Without either flag, the forward's
   CG is preconditioned when cg_rel_tol > 0 (the caller asks for a solution
   to that tolerance) and plain with cg_rel_tol = 0 (a fixed number of plain
   CG steps). The preconditioner is not on the pages; it is added because
   small ridges on clustered keys leave plain CG far from the answer after any
   affordable number of steps. Queries are grouped in 32s (g = floor(i/32));
   row i uses a unit-weight scatter matrix plus the ridge:
     rows i < 256 (g < 8): P_i = sum_{j <= i} (k_j - m_g)(k_j - m_g)^T + lambda I,
       the row's whole prefix about its group's point m_0 = k_0, m_g = the mean
       of the first 32 g keys; applied as the group's matrix (the scatter of
       those 32 g keys, lambda I for g = 0) and a rank-r correction by the
       group's own keys (r = i - 32 g + 1 <= 32, Woodbury identity);
     rows i >= 256: P_g = sum_{j < N_g} (k_j - m)(k_j - m)^T + lambda I, the
       first N_g keys about their mean m, N_g = 32 g rounded down to a
       multiple of 32 * 2^(floor(log2 g) - 2) (four prefix lengths per
       doubling of g, each built once per head).
   Every key used is visible to the row. The recurrence is CG with
   z = P^{-1} r in the direction update (p = z + beta p, beta = r'z'/rz),
   x0 = 0 and the same stop rule on ||r||. The group matrices' inverses are
   formed in fp32 and applied in two fp16 terms. The vector path ignores both
   flags (plain CG). */

/* Full argument block of lla_forward_ex. Zero-initialise, then fill. */
typedef struct lla_fwd_args {
  int dtype;          /* LLA_DTYPE_F32 or LLA_DTYPE_BF16 */
  const void* q;      /* [B][H][n][d] dtype, device */
  const void* k;      /* [B][H][n][d] dtype, device */
  const void* v;      /* [B][H][n][d] dtype, device */
  float* out;         /* [B][H][n][d] fp32, device, written */
  int B, H, n, d;
  float lambda;       /* ridge on the local slope; > 0 */
  int cg_max_iters;   /* >= 0 */
  float cg_rel_tol;   /* >= 0; 0 = run exactly cg_max_iters steps */
  /* optional outputs, NULL = not wanted (device pointers) */
  float* omega;       /* [B][H][n]    omega_i */
  float* rho;         /* [B][H][n][d] rho_i = Sigma_i^{-1} mu_i (pages' rho) */
  float* rowmax;      /* [B][H][n]    max_{l<=i} c q_i . k_l */
  int32_t* cg_iters;  /* [B][H][n]    CG steps taken by the query */
  float* cg_resid;    /* [B][H][n]    ||r_k|| / ||r_0|| at exit (0 if r_0 = 0) */
  /* optional caller workspace (device); NULL = the library allocates and
     frees it stream-ordered on `stream`. With a workspace (or where none is
     needed) a call only launches kernels on `stream`: no allocation, memset
     or synchronisation, so it can be captured into a HIP graph */
  void* workspace;
  size_t workspace_bytes;
  int kernel;         /* LLA_KERNEL_* */
  int flags;          /* LLA_FLAG_* */
  /* optional timing events (created by the caller, NULL = none): recorded on
     `stream` immediately before and after the call's dominant kernel -- the
     conjugate-gradient kernel of the matrix-core path, the single fused
     kernel of the vector-ALU path; set-up kernels and the moment and output
     kernels of the matrix-core path fall outside them */
  hipEvent_t ev_main_begin;
  hipEvent_t ev_main_end;
  /* optional output, NULL = not wanted: [B][H][n][d] fp32, device -- the
     solution the forward solved for, rho_c = Sigma_c^{-1} omega_i (kbar_i -
     q_i) with Sigma_c centred at the weighted key mean kbar_i (the pages'
     rho_i = rho_c / (1 + (kbar_i - q_i) . rho_c)); the input of
     lla_backward_ex. Not available with lla_output_given_rho. */
  float* rho_c;
} lla_fwd_args;

/* out = LLA(q, k, v) for fp32 inputs. Arguments as in lla_fwd_args;
   returns LLA_OK or a negative status. Kernel: AUTO. */
int lla_forward_f32(const float* q, const float* k, const float* v, float* out,
                    int B, int H, int n, int d, float lambda, int cg_max_iters,
                    float cg_rel_tol, hipStream_t stream);

/* Same for bfloat16 inputs, passed as their 16-bit patterns. */
int lla_forward_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     float* out, int B, int H, int n, int d, float lambda,
                     int cg_max_iters, float cg_rel_tol, hipStream_t stream);

/* Full form: dtype, kernel choice, optional outputs, optional workspace. */
int lla_forward_ex(const lla_fwd_args* args, hipStream_t stream);

/* out = Eq. (8) of the reading notes' section 2.1 for a SUPPLIED rho_i
   instead of the solved one:
     out_i = sum_j w_ij (1 - (k_j - q_i)^T rho_i) v_j / (omega_i - mu_i^T rho_i)
   (the denominator formed as sum_j w_ij (1 - (k_j - q_i)^T rho_i), equal to it
   for every rho). This is the forward's moment and output scans with the CG
   solve left out, so the solve and the output can be run and timed apart; it
   is also the covariance form of the Parallax summary,
   out_i = vbar_i - eta_i C_i rho_i, written out.
   rho_in: [B][H][n][d] fp32, device, 16-byte aligned, read only; rho_i = 0
   gives causal softmax attention. args: as for lla_forward_ex;
   cg_max_iters, cg_rel_tol and LLA_FLAG_SPLIT_U have no effect; cg_iters and
   cg_resid (if requested) are written 0; rho (if requested) receives rho_in;
   the events bracket the output kernel of the matrix-core path. No output
   may overlap rho_in. Returns LLA_OK or a negative status, as lla_forward_ex.
   Unlike the forward, which works on the system centred at the weighted key
   mean, this follows the printed form, whose denominator can be small for a
   rho far from the solution. */
int lla_output_given_rho(const lla_fwd_args* args, const float* rho_in, hipStream_t stream);

/* The naive forward: the same out_i (Eqs. (6)-(8) of the reading notes'
   section 2.1), evaluated the way that page's section 2.2 describes a direct
   implementation, as the comparison point of its peak-memory figure (Fig. 2,
   FlashLLA against the naive form at d = 128): every pairwise difference
   z_ij = k_j - q_i (Theta(n^2 d) per head) and every moment matrix Sigma_i
   (Theta(n d^2)) are materialised in the workspace, and each
   Sigma_i rho_i = mu_i is solved exactly by Cholesky. fp32 arithmetic
   throughout (fp32 or bf16 inputs, d in {16, 32, 64, 128}); no CG, so
   cg_max_iters and cg_rel_tol are ignored and cg_iters / cg_resid (if
   requested) are written 0; omega, rho (the pages' rho_i) and rowmax are
   available. kernel must be LLA_KERNEL_AUTO, flags 0 and rho_c NULL
   (LLA_ERR_INVALID_ARG otherwise); n <= 2^16 and B*H <= 65535
   (LLA_ERR_UNSUPPORTED). Workspace: lla_naive_workspace_bytes, about
   4 B*H*n^2*(d + 1) bytes; NULL = allocated and freed stream-ordered. The
   events bracket the moment kernel. Returns LLA_OK or a negative status. */
int lla_forward_naive(const lla_fwd_args* args, hipStream_t stream);

/* Workspace bytes of lla_forward_naive; 0 for sizes it rejects. */
size_t lla_naive_workspace_bytes(int B, int H, int n, int d, int dtype);

/* Device workspace bytes lla_forward_ex (or lla_output_given_rho) needs for
   these sizes and this kernel choice (LLA_KERNEL_*; the matrix-core path needs
   a workspace linear in B*H*n, the vector path none, and AUTO resolves as in
   the call). Returns 0 where no workspace is needed, and for sizes or a kernel
   choice the call would reject (e.g. n > 2^21 with LLA_KERNEL_MFMA). */
size_t lla_workspace_bytes(int B, int H, int n, int d, int dtype, int kernel);

/* ------------------------------------------------------------------------
 * Decode: one new query per (batch, head) against a cache of n keys and
 * values, every one of them visible -- the last row of the causal forward
 * whose query sits at position n - 1 (q_{n-1} = q). Same estimator, same
 * mean-centred CG system and the same CG policy as lla_forward_ex.
 * The centred Gram matrix sum_j w_j (k_j - kbar)(k_j - kbar)^T of the query
 * (d x d) is formed once on the matrix cores and CG runs on it plus lambda I
 * in fp32; in exact arithmetic the iterates are those of the matrix-free CG.
 * bf16 caches: one pass over K and V yields, per chunk of keys and against
 * the chunk's max, the moments, the uncentred Gram matrix and the cross
 * moment sum_j w_j v_j k_j^T (bf16 products, w k and w v in two bf16 terms,
 * fp32 sums); the head's centred system follows by the parallel-axis
 * identity and the output in the covariance form
 * out = (sum w v - C rho_c + (sum w v)(kbar . rho_c)) / omega. The fp32 sums
 * need |k|^2 and |v||k| times the cache length within fp32's range. fp32
 * caches: the centred Gram matrix with fp16 operands in two terms each; the
 * cache is read three times. Working memory is O(d^2) floats per chunk of
 * keys (bf16) or n + O(d^2) floats per head (fp32).
 * ------------------------------------------------------------------------ */
typedef struct lla_decode_args {
  int dtype;          /* LLA_DTYPE_F32 or LLA_DTYPE_BF16 */
  const void* q;      /* [B][H][d] dtype, device: the new query of each head */
  const void* k;      /* [B][H][n][d] dtype, device: key cache (the new key included) */
  const void* v;      /* [B][H][n][d] dtype, device: value cache */
  float* out;         /* [B][H][d] fp32, device, written */
  int B, H, n, d;     /* d in {64, 128} */
  float lambda;       /* > 0 */
  int cg_max_iters;   /* >= 0 */
  float cg_rel_tol;   /* >= 0 */
  /* optional outputs, NULL = not wanted (device pointers) */
  float* omega;       /* [B][H]    */
  float* rho;         /* [B][H][d] the pages' rho */
  float* rowmax;      /* [B][H]    max_l c q . k_l */
  int32_t* cg_iters;  /* [B][H]    */
  float* cg_resid;    /* [B][H]    ||r_k|| / ||r_0|| at exit */
  void* workspace;    /* optional caller workspace (device), as for lla_forward_ex */
  size_t workspace_bytes;
  hipEvent_t ev_main_begin; /* optional: recorded around the main kernel (bf16: the
                               pass over the cache; fp32: the Gram kernel) */
  hipEvent_t ev_main_end;
} lla_decode_args;

/* out = LLA(q; k, v) for one query per head. Conventions, validation and
   status codes as for lla_forward_ex (LLA_ERR_UNSUPPORTED for d outside
   {64, 128}). */
int lla_decode_ex(const lla_decode_args* args, hipStream_t stream);

/* Device workspace bytes lla_decode_ex needs for these sizes (0 for invalid
   sizes). Linear in n. */
size_t lla_decode_workspace_bytes(int B, int H, int n, int d, int dtype);

/* For callers that cannot allocate device memory: code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc. Same
   computation, kernels and results as lla_decode_ex, but the scratch comes
   from a static device array of LLA_DECODE_NOALLOC_SCRATCH_BYTES (64 MiB)
   that each GPU the library runs on holds until the process ends; the call
   allocates nothing, frees nothing and only launches kernels on `stream`.
   args: as for lla_decode_ex, except that workspace must be NULL and
   workspace_bytes 0 (LLA_ERR_INVALID_ARG otherwise). The inputs and outputs
   are the caller's, as for lla_decode_ex. A call whose scratch need
   (lla_decode_workspace_bytes) exceeds the static size returns
   LLA_ERR_WORKSPACE before any device work. `stream` (NULL = the default
   stream) must belong to the current device, whose copy of the scratch is
   used (LLA_ERR_INVALID_ARG otherwise). All calls on one GPU share that GPU's
   scratch: calls that overlap in time on one GPU (other streams, other host
   threads) race and give wrong results; calls in one stream are ordered and
   safe. The scratch keeps the last call's contents; nothing in it needs to
   start at zero. */
#define LLA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lla_decode_noalloc(const lla_decode_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward: the gradient of L = sum_i dout_i . out_i with respect to q, k and
 * v for the causal forward, on either path: the matrix cores (bf16 inputs,
 * d in {64, 128}) or the fp32 vector ALU (fp32 or bf16 inputs, d in
 * {16, 32, 64, 128}; dk and dv accumulated with fp32 atomics, so their last
 * bits depend on the order of the additions). "Local Linear Attention: reading notes" (section 2.2, on
 * training; appendix D) states that the backward needs further linear
 * systems per query but prints none; the gradient is implicit
 * differentiation of Eqs. (6)-(8) in the form the forward solves (centred at
 * the weighted key mean), with one adjoint CG solve per query on the same
 * matrix Sigma_c and the same CG policy as the forward:
 *   Sigma_c y_i = C_i^T dout_i,  C_i = sum_j (w_ij / omega_i) v_j (k_j - kbar_i)^T,
 * and the max-normalisation's share of the gradient routed to the key that
 * attains the row max (weights are max-normalised, and lambda makes the fit
 * depend on their scale). Working memory is linear in n.
 * ------------------------------------------------------------------------ */
typedef struct lla_bwd_args {
  int dtype;          /* LLA_DTYPE_BF16 (LLA_ERR_UNSUPPORTED otherwise) */
  const void* q;      /* [B][H][n][d] bf16, device: the forward's inputs */
  const void* k;
  const void* v;
  const float* out;   /* [B][H][n][d] fp32, device: the forward's output */
  const float* dout;  /* [B][H][n][d] fp32, device: dL/dout */
  const float* rho_c; /* [B][H][n][d] fp32, device: the forward's rho_c output
                         (kept rather than rho: where (kbar - q) . rho_c is large
                         the pages' rho no longer fixes its scale in fp32) */
  float* dq;          /* [B][H][n][d] fp32, device, written */
  float* dk;
  float* dv;
  int B, H, n, d;     /* d in {64, 128} */
  float lambda;       /* > 0, as in the forward */
  int cg_max_iters;   /* >= 0: adjoint solve, same policy as the forward */
  float cg_rel_tol;   /* >= 0 */
  /* optional outputs, NULL = not wanted (device pointers) */
  int32_t* adj_iters; /* [B][H][n] CG steps of the adjoint solve */
  float* adj_resid;   /* [B][H][n] ||r_k|| / ||r_0|| of the adjoint solve at exit */
  void* workspace;    /* optional caller workspace (device), as for lla_forward_ex */
  size_t workspace_bytes;
  hipEvent_t ev_main_begin; /* optional: recorded around the adjoint CG kernel */
  hipEvent_t ev_main_end;
  int flags;          /* LLA_FLAG_SPLIT_U: the adjoint CG's products carry
                         w * (...) as two fp16 terms (slower, more exact; the
                         right-hand side and the moments always carry two).
                         LLA_FLAG_PRECOND,
                         LLA_FLAG_NO_PRECOND: as for the forward, whose rule
                         the adjoint solve follows (preconditioned when
                         cg_rel_tol > 0 unless a flag says otherwise); pass
                         the forward's flags */
  int kernel;         /* LLA_KERNEL_*: AUTO takes the matrix-core path for bf16
                         inputs with d in {64, 128}, the vector path otherwise;
                         use the forward's choice */
} lla_bwd_args;

/* dq, dk, dv for the forward lla_forward_ex computed with the same q, k, v,
   lambda, CG policy and kernel choice, given its out and rho_c outputs. Every element of dq, dk and dv is written; the inputs are not.
   Conventions as for lla_forward_ex: device pointers, 16-byte aligned, no
   output may overlap an input or another output; validation on the host
   before any device work (nothing is written on failure); asynchronous on
   `stream`. Returns LLA_OK, LLA_ERR_INVALID_ARG, LLA_ERR_UNSUPPORTED (dtype
   other than bf16 or d outside {64, 128} with LLA_KERNEL_MFMA, d outside
   {16, 32, 64, 128}, sizes too large), LLA_ERR_WORKSPACE or LLA_ERR_HIP. */
int lla_backward_ex(const lla_bwd_args* args, hipStream_t stream);

/* Device workspace bytes lla_backward_ex needs for these sizes with
   LLA_KERNEL_AUTO (the matrix-core path; linear in n). 0 where the vector path
   runs (it needs none) or for invalid sizes. */
size_t lla_backward_workspace_bytes(int B, int H, int n, int d, int dtype);

/* Static, human-readable name of a status code. */
const char* lla_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* lla_last_error(void);

/* LLA_VERSION of the loaded library. */
int lla_version(void);

/* Lower-case hex SHA-256 of the source files and compiler flags the library
   was built from, as the package's build script computes it ("unknown" for a
   build without it), so a caller can tell a library that no longer matches
   its sources. Static string. */
const char* lla_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H */
