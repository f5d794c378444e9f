/*
 * mo.h - C ABI of the MI355X (gfx950) owner-side Muon step, AdamW tail and
 * Shampoo step.
 *
 * Sources, cited by page title and section:
 *   [P] "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
 *       sharding" (academ.us article 2607.05895).
 *   [A] the same paper's abstract excerpt (pith.science record).
 *
 * Under owner-shaped ZeRO-3 placement every 2D weight is whole on one owner
 * rank, and backward reduction leaves the full gradient there, so the optimizer
 * step on that rank is purely local ([P §3], [P §4.4]).  This library is that
 * local step: one Muon step over a bucket of whole matrices the caller owns,
 * and one AdamW step over the packed non-2D tail.  It issues no collectives.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers (W, G, M, update_out, p, g, m, v, workspace) are device
 *     pointers on the device that is current for the calling thread; the
 *     descriptor array and hyperparameter struct are host memory read during
 *     the call only.  The caller owns every buffer.
 *   - Matrices are row-major with a row stride `ld_*` in elements (0 means
 *     "cols").  W, M, p, m, v are updated in place; G and g are only read.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous with respect to the host and ordered on `stream`.
 *   - Every argument check runs on the host before anything is enqueued.  On
 *     any error return nothing has been launched and no output is touched.
 *     Device-side faults are not detected by the call; they surface on the
 *     caller's next synchronisation.
 *   - Results are deterministic: the same inputs give bit-identical outputs,
 *     and a matrix's result does not depend on the other matrices of the bucket.
 */
#ifndef MATRIX_OPTIMIZERS_AMD_MO_H
#define MATRIX_OPTIMIZERS_AMD_MO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mo_status;
#define MO_OK                       0
#define MO_ERR_INVALID_ARG         -1  /* null pointer, negative size, bad stride, bad value */
#define MO_ERR_UNSUPPORTED         -2  /* dtype / option not implemented, size beyond limits */
#define MO_ERR_WORKSPACE_TOO_SMALL -3
#define MO_ERR_ALIAS               -4  /* overlapping tensors that must be disjoint */
#define MO_ERR_HIP                 -5  /* a HIP runtime call or kernel launch failed */

/* element types */
#define MO_F32  0
#define MO_BF16 1

/* learning-rate adjustment, the shape factor on lr (torch.optim.Muon's
 * adjust_lr_fn; [P §5.1] runs with match_rms_adamw) */
#define MO_LR_ORIGINAL        0  /* lr * sqrt(max(1, rows/cols)) */
#define MO_LR_MATCH_RMS_ADAMW 1  /* lr * 0.2 * sqrt(max(rows, cols)) */
#define MO_LR_NONE            2  /* lr */

/* One whole 2D matrix held by its owner ([P §3]).
 *   W          rows x cols weight, w_dtype, row stride ld_w; updated in place.
 *   G          rows x cols gradient, g_dtype, row stride ld_g; read only.  It is
 *              the already-reduced full gradient: the library neither averages
 *              nor scales it.
 *   M          rows x cols fp32 momentum, row stride ld_m; updated in place.
 *   update_out optional (NULL): rows x cols fp32, row stride ld_u, receives
 *              lr_eff * O, the orthogonalised update before it meets W.
 * rows == 0 or cols == 0 marks an empty shard (a non-owner's view of the
 * matrix, [P §4.4]); it is validated and skipped, its pointers may be NULL. */
typedef struct mo_matrix {
    void*       W;
    const void* G;
    float*      M;
    float*      update_out;
    int64_t     rows, cols;
    int64_t     ld_w, ld_g, ld_m, ld_u;
    int32_t     w_dtype, g_dtype;
} mo_matrix;

/* Muon hyperparameters ([P §5.1] lists lr, weight decay, momentum, the number
 * of Newton-Schulz steps and the lr adjustment; the quintic coefficients and
 * eps are torch.optim.Muon's: (3.4445, -4.7750, 2.0315), 1e-7).
 *   momentum  beta of the EMA  M' = beta*M + (1-beta)*G
 *   nesterov  nonzero: U = (1-beta)*G + beta*M'; zero: U = M'
 *   ns_steps  K >= 0 quintic iterations X <- a X + (b A + c A^2) X, A = X X^T,
 *             on X = U / max(||U||_F, eps) in the short-side frame (U^T when
 *             rows > cols)
 *   ns_dtype  MO_BF16: X, A, B are bf16 MFMA operands with fp32 accumulation
 *             and fp32 epilogues; MO_F32: fp32 throughout
 * The step is W' = (1 - lr*wd) * W - lr_eff * O with lr_eff per lr_adjust. */
typedef struct mo_muon_hparams {
    float   lr, weight_decay, momentum;
    int32_t nesterov, ns_steps;
    float   ns_a, ns_b, ns_c, eps;
    int32_t lr_adjust, ns_dtype;
} mo_muon_hparams;

/* Bytes of device workspace muon_owner_step needs for this bucket (including
 * the device copy of the work list and 256 bytes of alignment slack). */
mo_status muon_workspace_bytes(const mo_matrix* mats, int32_t n_mats,
                               const mo_muon_hparams* hp, size_t* bytes);

/* The host work list that muon_owner_step uploads, for inspection and tests.
 * If host_buf is NULL, *bytes_inout receives the size; otherwise *bytes_inout
 * must hold at least that size and the list is written to host_buf.  The byte
 * layout (little-endian, natural alignment, version 5):
 *   header   mo_wl_header (128 bytes); its 14th word is the number of
 *            wavefronts per workgroup of the GEMM kernels the list is built
 *            for (8 with a bf16 ns_dtype, 4 with fp32)
 *   matrices mo_wl_mat[n_live] (192 bytes each), one per non-empty descriptor,
 *            in descriptor order
 *   items    three dispatch lists of mo_wl_item (16 bytes: record index, tile
 *            row ti, tile column tj, width nb in {4, 2, 1}; the tile covers
 *            rows 256 ti .. +256 and columns 64 nb tj .. +64 nb): Gram, Poly,
 *            Update, each starting on a 256-byte boundary; entry b is the tile
 *            run by workgroup b
 * Gram and Poly cover the upper-triangle tiles (ti <= tj) of the m_pad x m_pad
 * product, Update all tiles of the m_pad x n_pad product.  Matrices are taken
 * in descending order of their per-phase work (ties by descriptor index) and
 * cut into super-blocks of 4 tile-rows x 8 tile-columns (row-major, tiles
 * row-major inside); each super-block goes to the one of 8 queues (one per
 * XCD) with the least K-length x tiles so far, ties to the lowest; if that
 * queue is below an even share ceil(total / 8) it takes only the tiles that
 * reach the share (at least one) and the rest goes on to the next queue.
 * Then, where full tiles would leave CUs idle, tiles are split by columns: a
 * queue of n <= 32 tiles (32 CUs per XCD) has every tile split, a longer one
 * the n % 32 tiles of its last round, into S = 4 quarter-width (nb = 1, fp32
 * lists only) or S = 2 half-width (nb = 2) tiles, the largest S with
 * S x (tiles split) <= 32;
 * the parts take the tile's place in the queue, in column order.  Entry 8 j + x
 * of a list is the j-th tile of queue x, or a pad entry (record index
 * 0xFFFFFFFF) where queue x is shorter. */
mo_status muon_build_worklist(const mo_matrix* mats, int32_t n_mats,
                              const mo_muon_hparams* hp, void* host_buf,
                              size_t* bytes_inout);

/* One Muon step on every non-empty matrix of the bucket ([P §3], [P §4.4]).
 * workspace: device memory of at least muon_workspace_bytes() bytes, disjoint
 * from every tensor; its contents are undefined afterwards and it must not be
 * shared by calls that may run concurrently.  n_mats == 0 is a no-op.
 * Errors: MO_ERR_INVALID_ARG (null pointer with numel > 0, negative size,
 * ld < cols, ns_steps < 0, non-finite hyperparameter, eps <= 0, unknown
 * lr_adjust), MO_ERR_UNSUPPORTED (dtype not MO_F32/MO_BF16, a side longer than
 * 2^23, more than 2^36 elements in one matrix, more than 2^26 tiles of 256 x 256
 * in the bucket), MO_ERR_WORKSPACE_TOO_SMALL,
 * MO_ERR_ALIAS (W, M, update_out of any
 * matrix overlap any tensor of the bucket or the workspace), MO_ERR_HIP. */
mo_status muon_owner_step(const mo_matrix* mats, int32_t n_mats,
                          const mo_muon_hparams* hp, void* workspace,
                          size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as muon_owner_step, with the same kernels and bit-identical results,
 * on a workspace that is a static array of the library instead of a caller
 * buffer.  It calls no hipMalloc, hipFree or other allocating routine: the
 * array (MO_NOALLOC_SCRATCH_BYTES = 512 MiB per device) is part of the
 * library's code object, loaded on a device with the first call there and
 * held until the process ends, and the work list is uploaded through kernel
 * arguments (one small launch per 3.5 KB of list), not a staging buffer.
 * Every call on a device shares that device's array: calls that may overlap
 * in time on one device (other streams, other threads) race and must be
 * serialised by the caller; stream-ordered calls on one stream are safe.
 * Nothing in the array needs to start at zero (every region is written before
 * it is read).  With mo_profile_enable on, the timing path creates its events
 * on first use.  Errors as muon_owner_step, with MO_ERR_WORKSPACE_TOO_SMALL
 * when the bucket's muon_workspace_bytes() exceeds MO_NOALLOC_SCRATCH_BYTES
 * (nothing is launched then). */
#define MO_NOALLOC_SCRATCH_BYTES ((size_t)512 << 20)
mo_status muon_owner_step_noalloc(const mo_matrix* mats, int32_t n_mats,
                                  const mo_muon_hparams* hp, void* stream);

/* One AdamW step on a packed fp32 tail of n elements, in place ([P §3]: the
 * non-2D tensors stay on the AdamW path; [P §5.1] gives the hyperparameters):
 *   m' = b1 m + (1-b1) g;  v' = b2 v + (1-b2) g^2;
 *   p' = p (1 - lr wd) - (lr / (1-b1^t)) m' / (sqrt(v') / sqrt(1-b2^t) + eps)
 * with the bias corrections formed on the host in fp64.  step t >= 1.
 * Errors: MO_ERR_INVALID_ARG (null pointer with n > 0, n < 0, step < 1,
 * non-finite hyperparameter), MO_ERR_ALIAS (p, g, m, v overlap), MO_ERR_HIP. */
mo_status adamw_tail_step(float* p, const float* g, float* m, float* v, int64_t n,
                          int64_t step, float lr, float beta1, float beta2, float eps,
                          float weight_decay, void* stream);

/* Human-readable name of a status code (static storage). */
const char* mo_status_string(mo_status status);

/* ---- measurement support (not part of the optimizer step) ---------------- */

/* Phase identifiers for per-kernel timing. */
#define MO_PHASE_MOMENTUM 0   /* momentum + Nesterov + norm partials + NS-frame layout */
#define MO_PHASE_NORM     1   /* per-matrix norm finalisation */
#define MO_PHASE_GRAM     2   /* A = X X^T (upper tiles, mirrored) */
#define MO_PHASE_POLY     3   /* B = b A + c A A */
#define MO_PHASE_UPDATE   4   /* X <- a X + B X (every step but the last) */
#define MO_PHASE_APPLY    5   /* K == 0 only: W <- (1-lr wd) W - lr_eff X */
#define MO_PHASE_ADAMW    6
#define MO_PHASE_COPY     7   /* mo_device_copy */
#define MO_PHASE_UPDATE_LAST 8 /* last Newton-Schulz step: O = a X + B X, W written */
#define MO_PHASE_SH_LAYOUT   9  /* Shampoo: padded G and G^T */
#define MO_PHASE_SH_STATS   10  /* Shampoo: L' = L + G G^T, R' = R + G^T G */
#define MO_PHASE_SH_ROOTPREP 11 /* Shampoo: norms, X_0, H_1 (three small launches) */
#define MO_PHASE_SH_ROOT    12  /* Shampoo: coupled Newton products */
#define MO_PHASE_SH_LEFT    13  /* Shampoo: T = H_L G */
#define MO_PHASE_SH_RIGHT   14  /* Shampoo: W <- decay W - lr T H_R */
#define MO_PHASE_SO_PREP    15  /* SOAP: padded G, first moment M' */
#define MO_PHASE_SO_STATS   16  /* SOAP: L' = L + G G^T, R' = R + G^T G */
#define MO_PHASE_SO_SOLVE   17  /* SOAP: Jacobi pair problems of one round */
#define MO_PHASE_SO_APPLY   18  /* SOAP: one round's rotations applied to A (both sides) and E */
#define MO_PHASE_SO_SORT    19  /* SOAP: E = I, eigenvalue sort, sorted fp32 eigenvectors */
#define MO_PHASE_SO_PRODUCTS 20 /* SOAP: the six eigenbasis products, V', N and W written */
#define MO_PHASE_SO_WARM    21  /* SOAP: a warm start's four products per eigendecomposition */
#define MO_PHASE_COUNT    22

/* Enable (1) or disable (0) per-launch timing on the calling thread.  While
 * enabled, every kernel launch is bracketed by HIP events on its own stream;
 * mo_profile_read() synchronises on them.  Timing costs a few microseconds of
 * host time per launch and does not change any result. */
mo_status mo_profile_enable(int32_t enable);

/* Wait for the recorded launches, then add their durations (ms) and counts to
 * ms[MO_PHASE_COUNT] and launches[MO_PHASE_COUNT] and forget them. */
mo_status mo_profile_read(double* ms, int64_t* launches);

/* A plain device-to-device copy kernel (16-byte vector loads and stores), used
 * to calibrate HBM byte counters against a transfer of known size.  dst and
 * src must not overlap; bytes must be a multiple of 16 and both pointers
 * 16-byte aligned.  Errors: MO_ERR_INVALID_ARG, MO_ERR_ALIAS, MO_ERR_HIP. */
mo_status mo_device_copy(void* dst, const void* src, size_t bytes, void* stream);

/* ---- Shampoo owner step --------------------------------------------------
 * [P §5.7]: with every 2D matrix whole on its owner, the owner can run any
 * single-device matrix optimizer; the paper swaps owner-Muon for Shampoo with
 * full left / right preconditioners and an inverse fourth root, in float32.
 * The pages name the method without its formulas; this library's readings:
 *   statistics  L' = L + G G^T and R' = R + G^T G, the published Shampoo
 *               update of a matrix (Gupta, Koren and Singer, 2018); the caller
 *               starts them at eps I and keeps them between steps
 *   roots       H ~ S'^{-1/4} for S' = L', R': root_iters steps of the coupled
 *               Newton iteration for the inverse p-th root (Guo and Higham,
 *               2006), p = 4, with the Frobenius scaling of Anil et al. (2020):
 *               z = (p + 1) / (2 ||S'||_F), M = z S', H = z^{1/p} I; each step
 *               X = ((p + 1) I - M) / p, H <- H X, M <- X^p M
 *   update      W' = (1 - lr wd) W - lr H_L G H_R (decoupled decay, as the
 *               Muon path of the same owner)
 * Statistics, roots and products are fp32 (fp32 MFMA, fp32 accumulation); W
 * and G may be bf16.  There is no momentum, grafting or root-reuse schedule.
 * The statistics and the X^2, X^4 and M products are symmetric: the library
 * computes one triangle and mirrors it, and it reads L[j][i] for L'[i][j] (the
 * same value for the symmetric L it always writes).  The H products are
 * computed whole and the final H is applied by its rows on both sides
 * (H_L^T G H_R), which keeps fp32 rounding in the near-null directions of a
 * rank-deficient S' away from the update.  S' must be positive definite; a
 * zero S' (eps = 0 and G = 0) gives non-finite results. */

/* One whole matrix with its statistics.
 *   W          rows x cols, w_dtype, row stride ld_w; updated in place
 *   G          rows x cols, g_dtype, row stride ld_g; read only
 *   L          rows x rows fp32, row stride ld_l; updated in place (L')
 *   R          cols x cols fp32, row stride ld_r; updated in place (R')
 *   update_out optional (NULL): rows x cols fp32, row stride ld_u, receives
 *              lr H_L G H_R
 * rows == 0 or cols == 0 marks an empty shard (skipped; pointers may be NULL).
 * Strides of 0 mean the natural ones (cols, rows for L, cols for R). */
typedef struct mo_shampoo_matrix {
    void*       W;
    const void* G;
    float*      L;
    float*      R;
    float*      update_out;
    int64_t     rows, cols;
    int64_t     ld_w, ld_g, ld_l, ld_r, ld_u;
    int32_t     w_dtype, g_dtype;
} mo_shampoo_matrix;

/* lr, weight decay, and the number of coupled Newton steps (1 .. 100). */
typedef struct mo_shampoo_hparams {
    float   lr, weight_decay;
    int32_t root_iters;
} mo_shampoo_hparams;

/* Bytes of device workspace shampoo_owner_step needs for this bucket: per
 * matrix three fp32 buffers of r_pad x c_pad, per root seven of m_pad x m_pad
 * (x_pad = x rounded up to 256), plus the work list and 256 bytes of slack. */
mo_status shampoo_workspace_bytes(const mo_shampoo_matrix* mats, int32_t n_mats,
                                  const mo_shampoo_hparams* hp, size_t* bytes);

/* One Shampoo step on every non-empty matrix of the bucket: at most
 * 3 root_iters + 1 grouped GEMM launches plus four small ones, each covering
 * every matrix of the bucket.
 * Workspace, stream and error conventions as muon_owner_step: MO_ERR_INVALID_ARG
 * (null pointer with numel > 0, negative size, a stride below its row length,
 * root_iters outside 1 .. 100, non-finite lr or weight decay),
 * MO_ERR_UNSUPPORTED (dtype not MO_F32/MO_BF16, a side longer than 2^16: each
 * side is also a root's; more than 2^26 tiles of 256 x 256 over the bucket's
 * roots and matrices), MO_ERR_WORKSPACE_TOO_SMALL, MO_ERR_ALIAS (W, L, R,
 * update_out of any matrix
 * overlap any tensor of the bucket or the workspace), MO_ERR_HIP. */
mo_status shampoo_owner_step(const mo_shampoo_matrix* mats, int32_t n_mats,
                             const mo_shampoo_hparams* hp, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---- SOAP owner step -----------------------------------------------------
 * [P §5.7]: next to Shampoo, the owner runs SOAP, which the paper describes as
 * Adam in the Shampoo eigenbasis, with the same placement.  The pages print no
 * formulas; this library follows the published SOAP algorithm (Vyas et al.,
 * 2024), each choice it leaves open in its plainest form:
 *   statistics  L' = L + G G^T, R' = R + G^T G (the caller starts them at
 *               eps I and keeps them between steps)
 *   eigenbasis  Q_L, Q_R: eigenvectors of L', R', recomputed every step, in
 *               ascending order of their eigenvalues (the second moment is
 *               indexed by that order; signs do not matter)
 *   moments     M' = b1 M + (1 - b1) G in the weight's frame;
 *               G~ = Q_L^T G Q_R, M~ = Q_L^T M' Q_R;
 *               V' = b2 V + (1 - b2) G~^2 in the eigenbasis
 *   update      N = (M~ / (1 - b1^t)) / (sqrt(V' / (1 - b2^t)) + eps);
 *               W' = (1 - lr wd) W - lr Q_L N Q_R^T
 * The eigenvectors come from a two-sided blocked Jacobi method whose
 * rotations and rotated matrix are fp64 (`sweeps` sweeps of all block pairs,
 * rotations in Rutishauser's form; an off-diagonal entry at or below
 * 2^-48 ||L'||_F (or ||R'||_F) is left unrotated, which moves an eigenvector
 * by at most that over its eigenvalue gap); the accumulated eigenvectors are
 * kept and updated in fp32, whose rounding moves them by a few fp32 units and
 * does not feed back into the rotations.  The statistics, moments and
 * products are stored in fp32; the products (and the statistics' G G^T)
 * take their sums in fp64.  Sides are at most 16384. */

/* One whole matrix with its SOAP state.
 *   W          rows x cols, w_dtype, row stride ld_w; updated in place
 *   G          rows x cols, g_dtype, row stride ld_g; read only
 *   L, R       rows x rows and cols x cols fp32 (strides ld_l, ld_r), symmetric;
 *              updated in place (L', R')
 *   M          rows x cols fp32 first moment (weight frame), stride ld_m; in place
 *   V          rows x cols fp32 second moment (eigenbasis), stride ld_v; in place
 *   update_out optional (NULL): rows x cols fp32, stride ld_u, receives
 *              lr Q_L N Q_R^T
 * rows == 0 or cols == 0 marks an empty shard (skipped; pointers may be NULL).
 * Strides of 0 mean the natural ones. */
typedef struct mo_soap_matrix {
    void*       W;
    const void* G;
    float*      L;
    float*      R;
    float*      M;
    float*      V;
    float*      update_out;
    int64_t     rows, cols;
    int64_t     ld_w, ld_g, ld_l, ld_r, ld_m, ld_v, ld_u;
    int32_t     w_dtype, g_dtype;
} mo_soap_matrix;

/* Adam hyperparameters, the step number t (>= 1) of the bias corrections, and
 * the number of outer Jacobi sweeps (1 .. 100). */
/* warm_start: 0, the eigensolver starts from the identity (each step on its
 * own); 1, it starts from the eigenbases the previous step of this bucket
 * left in this workspace (the reusable step objects of the binding pass 1
 * from their second call on).  A side whose workspace region does not hold
 * bases that a step wrote for a side of the same size m (the word the sort
 * writes beside them names m and its padding) runs cold; bases of another
 * matrix's side of that size are orthonormal and still a valid start, only a
 * slower one.  The previous bases are made orthonormal again by one
 * Newton-Schulz polar step, the new statistics are rotated into them, and
 * the sweeps start from that nearly diagonal matrix: the result is the same
 * eigendecomposition, to the sweeps' convergence, and fewer of the sweeps
 * still rotate. */
typedef struct mo_soap_hparams {
    float   lr, beta1, beta2, eps, weight_decay;
    int32_t step, sweeps, warm_start;
} mo_soap_hparams;

/* Bytes of device workspace soap_owner_step needs: per matrix four fp32
 * buffers of r_pad x c_pad; per side of size m three m_pad x m_pad buffers
 * (one fp64, two fp32) and m_pad / 64 fp64 pair rotations of 64 x 64
 * (x_pad = x rounded up to 64); plus the work list and 256 bytes of slack. */
mo_status soap_workspace_bytes(const mo_soap_matrix* mats, int32_t n_mats,
                               const mo_soap_hparams* hp, size_t* bytes);

/* One SOAP step on every non-empty matrix of the bucket.  The eigensolver's
 * launches are grouped over every statistics matrix of the bucket (two per
 * round, sweeps x (m_pad / 32 - 1) rounds for the longest side; a pair
 * left unrotated in a round costs its tiles nothing); the rest is
 * a few launches per matrix.  Workspace, stream and error conventions as
 * muon_owner_step: MO_ERR_INVALID_ARG (null pointer with numel > 0, negative
 * size, a stride below its row length, step < 1, sweeps outside 1 .. 100,
 * warm_start not 0 or 1, non-finite lr, betas, eps or weight decay, betas
 * outside [0, 1), eps < 0),
 * MO_ERR_UNSUPPORTED (dtype not MO_F32/MO_BF16, a side longer than 16384, more
 * than 2^30 rotation tiles of 64 x 64 over the bucket's sides),
 * MO_ERR_WORKSPACE_TOO_SMALL, MO_ERR_ALIAS (a written tensor overlaps any
 * tensor of the bucket or the workspace), MO_ERR_HIP. */
mo_status soap_owner_step(const mo_soap_matrix* mats, int32_t n_mats, const mo_soap_hparams* hp,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Convergence of the last soap_owner_step's eigensolver.  Call it with the
 * same bucket, hyperparameters and workspace as that step, on its stream,
 * before the workspace is reused; it waits for the step.  Cyclic Jacobi has
 * converged when a whole sweep rotates nothing: every off-diagonal entry is
 * then at or below 2^-48 ||A||_F.  rotating[2 i] (L' of matrix i) and
 * rotating[2 i + 1] (R') receive the number of pair slots (at most
 * m_pad / 64) whose pair problem still rotated during the final sweep: 0
 * means converged; otherwise the sweep count was too small for this input
 * and the eigenvectors, hence the update, may be off by more than the fp32
 * statistics fix.  Empty descriptors get 0.  rotating is host memory of 2 n
 * int32.  Errors: as soap_workspace_bytes, MO_ERR_INVALID_ARG (rotating NULL
 * with n > 0), MO_ERR_WORKSPACE_TOO_SMALL, MO_ERR_HIP. */
mo_status soap_converged(const mo_soap_matrix* mats, int32_t n_mats, const mo_soap_hparams* hp,
                         const void* workspace, size_t workspace_bytes, int32_t* rotating,
                         void* stream);

/* ---- owner planner (host only) --------------------------------------------
 * The step upstream of a bucket: which data-parallel rank owns each role
 * ([P §4.1]).  Every FSDP block contributes one role per 2D matrix and one
 * packed tail role for its non-2D tensors ([P §3]).  The greedy load is the
 * role's owner-resident numel, a proxy for its resident bytes and optimizer
 * work ([P §4.1]).  The pages describe the policies but do not print the
 * algorithm, so the readings below are this library's:
 *   MO_PLAN_ROLE_GREEDY   blocks in increasing block index; within a block,
 *                         roles by decreasing numel (ties: array order), each
 *                         to the rank with the least numel assigned so far over
 *                         all blocks (ties: lowest rank).  The default.
 *   MO_PLAN_SCOPE_GREEDY  all roles of all blocks pooled, by decreasing numel
 *                         (ties: array order), each to the least-loaded rank.
 *   MO_PLAN_COST_AWARE    the scope plan if its largest per-block owner share
 *                         max_{B,r} O_{B,r} (the numel one rank must send to
 *                         materialize block B, which sets C_owner of [P §4.2])
 *                         is at most block_cap, else the role plan; block_cap
 *                         0 means the role plan's own largest share.
 * All functions only read host arrays and run no device work. */
#define MO_ROLE_MATRIX 0
#define MO_ROLE_TAIL   1
#define MO_PLAN_ROLE_GREEDY  0
#define MO_PLAN_SCOPE_GREEDY 1
#define MO_PLAN_COST_AWARE   2

typedef struct {
    int32_t block;   /* FSDP block index, >= 0 */
    int32_t kind;    /* MO_ROLE_MATRIX or MO_ROLE_TAIL */
    int64_t rows;    /* matrix rows; for a tail, its numel */
    int64_t cols;    /* matrix cols; for a tail, 1 */
} mo_role;

/* owner_out[i] in [0, world) for each of the n_roles roles.  Errors:
 * MO_ERR_INVALID_ARG (null pointer with n_roles > 0, world < 1, n_roles < 0,
 * negative block, size or cap, a tail with cols != 1, unknown kind or
 * policy). */
mo_status mo_plan_owners(const mo_role* roles, int32_t n_roles, int32_t world, int32_t policy,
                         int64_t block_cap, int32_t* owner_out);

/* Resource scorer of a plan.  Per rank (arrays of `world`): rank_numel = its
 * owner-resident numel; rank_flops = nominal Newton-Schulz flops of one
 * iteration over its matrices, sum of 4 m^2 n + 2 m^3 with m = min(rows, cols),
 * n = max (tails count 0).  Per block (arrays of n_blocks = 1 + largest block
 * index; may be NULL): block_gamma = max_r O_{B,r} / (P_B / world), the owner
 * imbalance gamma_B of [P §4.2] (0 for an empty block), and block_owner_comm =
 * (world - 1) max_r O_{B,r}, its materialization volume C_owner in elements.
 * Errors as mo_plan_owners, plus an owner outside [0, world). */
mo_status mo_plan_score(const mo_role* roles, int32_t n_roles, int32_t world, const int32_t* owner,
                        double* rank_numel, double* rank_flops, int32_t n_blocks,
                        double* block_gamma, double* block_owner_comm);

/* Block-local layout of a plan: every rank keeps, per block, one flat buffer
 * holding the roles it owns, in role-array order and back to back; a role the
 * rank does not own has an empty segment there ([P §4.1]'s one contiguous
 * local segment per parameter).  offset_out[i] is role i's element offset in
 * its owner's buffer for its block.  Errors as mo_plan_score. */
mo_status mo_plan_layout(const mo_role* roles, int32_t n_roles, int32_t world, const int32_t* owner,
                         int64_t* offset_out);

#ifdef __cplusplus
}
#endif

#endif /* MATRIX_OPTIMIZERS_AMD_MO_H */
