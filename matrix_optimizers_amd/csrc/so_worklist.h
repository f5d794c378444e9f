// Work-list layout of the SOAP owner step, shared by the host builder and the
// device kernels: one packed little-endian byte string (header, one record
// per non-empty matrix, one per eigendecomposition) uploaded to the front of
// the workspace.  The GEMM launches take their operands from these records;
// the eigensolver launches are grouped over every eigendecomposition of the
// bucket and find their record from the item index.
#pragma once

#include <stddef.h>
#include <stdint.h>

#define MO_SO_MAGIC   0x4F534F4Du  // "MOSO"
#define MO_SO_VERSION 6u
#define MO_SO_ECOLS 8u     // 64-column tiles of E per rotation work item (one D_I load each)

#define MO_SO_PAD    64   // padding of every side (the eigensolver's pair of 32-wide blocks)
#define MO_SO_BLK    32   // Jacobi block width
#define MO_SO_MAXSIDE 16384  // the paper's MLP side; each side holds 16 bytes of workspace per m_pad^2 (A fp64, E and E32 fp32)

// fp32 products of the step (C = op(A) op(B), 64 x 64 tiles)
#define MO_SOK_STATS_L 0   // L' = L + G G^T: caller L and the fp64 copy the eigensolver works on
#define MO_SOK_STATS_R 1   // R' = R + G^T G
#define MO_SOK_LEFT_G  2   // T = Q_L^T G      (Q_L^T = E_L, rows are eigenvectors)
#define MO_SOK_RIGHT_G 3   // G~ = T Q_R; V' = b2 V + (1 - b2) G~^2 into the caller's V
#define MO_SOK_LEFT_M  4   // T = Q_L^T M'
#define MO_SOK_RIGHT_M 5   // M~ = T Q_R; N = (M~ / bc1) / (sqrt(V' / bc2) + eps)
#define MO_SOK_BACK_L  6   // T = Q_L N
#define MO_SOK_BACK_R  7   // D = T Q_R^T; W <- (1 - lr wd) W - lr D
#define MO_SOK_COUNT   8

// fp32 products of a warm start, per eigendecomposition (m_pad x m_pad; E32
// holds the previous step's sorted eigenvectors as rows)
#define MO_SOW_P 0   // Pm = E32 E32^T - I                  (fp32, into the A region)
#define MO_SOW_E 1   // E0 = E32 - Pm E32 / 2: one polar Newton-Schulz step (into E)
#define MO_SOW_T 2   // T = L' E0^T, L' the caller's statistics (into E32)
#define MO_SOW_A 3   // A0 = E0 T, the starting matrix of the sweeps (fp64, into A)

#define MO_SOF_W_BF16     0x1u
#define MO_SOF_G_BF16     0x2u
#define MO_SOF_HAS_UPDATE 0x4u

struct mo_so_header {
    uint32_t magic, version;
    uint32_t n_mats, n_eigs;
    uint32_t sweeps, max_rounds;          // outer Jacobi sweeps; rounds of the longest eigendecomposition
    uint32_t n_solve_items, n_apply_items; // pair problems; upper 64 x 64 tiles of A
    uint64_t mats_offset, eigs_offset;    // bytes from list start
    uint64_t wl_bytes, ws_bytes;
    uint32_t n_etile_items;               // 64 x 64 tiles of E
    uint32_t reserved[3];
};

struct mo_so_mat {
    uint64_t W, G, M, V, U;               // caller pointers (U = update_out or 0)
    int64_t  ld_w, ld_g, ld_m, ld_v, ld_u;
    uint64_t off_G, off_M, off_T, off_N;  // padded fp32 G, M', product scratch, N (r_pad x c_pad)
    uint32_t rows, cols, r_pad, c_pad;
    uint32_t flags, eig_l, eig_r, reserved0;
    float    decay, lr, beta1, beta2;     // 1 - lr wd; lr; Adam betas
    float    ibc1, ibc2, eps, reserved1;  // 1 / (1 - b1^t), 1 / (1 - b2^t), Adam eps
};

// One eigendecomposition (of L' or R' of matrix `mat`), side m padded to
// m_pad = 64 P: A (fp64, m_pad x m_pad) is rotated toward diagonal form (the
// statistics launch writes it whole; the rounds keep only its upper 32 x 32
// blocks, a lower block being the transpose of its mirror), E (fp32 between
// rounds) accumulates the rotations (rows are eigenvectors), D holds the P
// pair rotations of the current round (fp64, 64 x 64 each, as V - I), E32 the
// eigenvectors sorted by ascending eigenvalue (fp32), perm the sort, flag
// one word per pair: whether its rotation of the current round is not the
// identity; norm the per-row sums of squares of A and, after them, the
// rotation threshold 2^-48 ||A||_F (fp64); last one word per pair slot: set
// when that slot's pair problem rotated in some round of the final sweep
// (all zero: the final sweep rotated nothing, so A was diagonal to the
// threshold, the convergence test of cyclic Jacobi).  valid is one word the gather writes
// after E32 (MO_SO_MAGIC ^ (m_pad | m << 16)): a warm start uses E32 only when
// it holds it, so a workspace that never held bases of a side of this size
// runs cold.
struct mo_so_eig {
    uint64_t off_A, off_E, off_D, off_E32, off_perm, off_flag, off_norm, off_last;
    uint64_t ext;                         // caller statistics (L or R), m x m fp32, row stride ld_ext
    int64_t  ld_ext;
    uint32_t m, m_pad, P, mat;
    uint32_t rounds;                      // sweeps x (2P - 1)
    uint32_t solve_begin, apply_begin;    // first item of this decomposition in each grouped launch
    uint32_t etile_begin;
    uint64_t off_valid;                   // one word: MO_SO_MAGIC ^ (m_pad | m << 16) once the sort has written E32
};

static_assert(sizeof(mo_so_header) == 80, "header layout");
static_assert(sizeof(mo_so_mat) == 176, "matrix record layout");
static_assert(sizeof(mo_so_eig) == 120, "eig record layout");
