// Work-list layout of the Shampoo owner step, shared by the host builder and
// the device kernels.
//
// Like the Muon list, one packed little-endian byte string (header, one record
// per non-empty matrix, one per inverse root, one per GEMM product, then the
// dispatch lists of the grouped GEMM launches) is uploaded to the front of the
// workspace, and every kernel of the step reads its tables from there.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mo_worklist.h"

#define MO_SH_MAGIC   0x48534F4Du  // "MOSH"
#define MO_SH_VERSION 1u

// the root order p of the inverse p-th roots
#define MO_SH_P 4

// GEMM product kinds (epilogues), each C = P Q^T.  STATS, SQ, S4 and M are
// symmetric (upper tiles, mirrored); H, HT, LEFT and RIGHT are full.  The H
// products are full because H_{k-1} X is symmetric only in exact arithmetic:
// its rows carry the rounding of the small eigenvalues' directions scaled by
// H's range values, its columns scaled by the much larger null-space values,
// so the step keeps H unsymmetrised and uses the last one by its rows on both
// sides (HT stores it transposed for the left product).
#define MO_SHK_STATS 0   // S' = S + P P^T: caller statistics and its padded copy M_0
#define MO_SHK_SQ    1   // S2 = X X^T
#define MO_SHK_H     2   // H_k = H_{k-1} X^T
#define MO_SHK_S4    3   // S4 = S2 S2^T
#define MO_SHK_M     4   // M_k = alpha S4 M_{k-1}^T, X_k = ((p + 1) I - M_k) / p
#define MO_SHK_LEFT  5   // T = H_L^T G  (P = the stored H_L^T)
#define MO_SHK_RIGHT 6   // W <- decay W - lr T H_R  (Q = the stored H_R^T)
#define MO_SHK_HT    7   // H_K = H_{K-1} X^T, stored transposed

// dispatch lists, one per kind of grouped launch
#define MO_SHL_STATS 0   // every statistics product
#define MO_SHL_SQ    1   // S2 of every root (first iteration)
#define MO_SHL_SQH   2   // S2 and H of every root
#define MO_SHL_H     3   // HT of every root (last iteration)
#define MO_SHL_S4    4
#define MO_SHL_M     5
#define MO_SHL_LEFT  6
#define MO_SHL_RIGHT 7
#define MO_SHL_COUNT 8

// flags of mo_sh_mat
#define MO_SHF_W_BF16     0x1u
#define MO_SHF_G_BF16     0x2u
#define MO_SHF_HAS_UPDATE 0x4u

struct mo_sh_header {
    uint32_t magic, version;
    uint32_t n_mats, n_roots, n_prods, root_iters;
    uint32_t n_lay_items;                 // 64 x 64 tiles of the padded gradients
    uint32_t n_root_items;                // 64 x 64 tiles of the padded roots
    uint32_t n_items[MO_SHL_COUNT];
    uint64_t mats_offset, roots_offset, prods_offset;   // bytes from list start
    uint64_t list_offset[MO_SHL_COUNT];
    uint64_t wl_bytes, ws_bytes;
    uint32_t reserved[6];
};

struct mo_sh_mat {
    uint64_t W, G, U;                     // caller pointers (U = update_out or 0)
    int64_t  ld_w, ld_g, ld_u;
    uint64_t off_G, off_Gt, off_T;        // padded G (r_pad x c_pad), G^T (c_pad x r_pad), H_L G (r_pad x c_pad)
    uint32_t rows, cols, r_pad, c_pad;
    uint32_t flags, root_l, root_r;
    uint32_t lay_begin, lay_tiles_c;      // first layout item; 64-wide tiles per padded row
    float    decay, lr;                   // 1 - lr wd; lr
    uint32_t reserved[3];
};

// One inverse fourth root: of L (m = rows) or R (m = cols) of matrix `mat`.
// Seven m_pad x m_pad fp32 buffers: M (ping-pong; M[0] first holds the padded
// statistics), X, S2, S4, H (ping-pong).
struct mo_sh_root {
    uint64_t off_M[2], off_X, off_S2, off_S4, off_H[2];
    uint64_t off_partials, off_scale;     // per-tile sums of squares; z, z^(1/p)
    uint64_t ext;                         // caller statistics (L or R), m x m, row stride ld_ext
    int64_t  ld_ext;
    uint64_t off_op;                      // operand of the statistics product (padded G or G^T)
    uint32_t op_ld;                       // its row length (the K extent)
    uint32_t m, m_pad, mat;
    uint32_t item_begin, tiles_c, n_partials;
    uint32_t reserved;
};

struct mo_sh_prod {
    uint32_t kind;    // MO_SHK_*
    uint32_t ref;     // root index (root products), matrix index (LEFT, RIGHT)
};

static_assert(sizeof(mo_sh_header) == 192, "header layout");
static_assert(sizeof(mo_sh_mat) == 128, "matrix record layout");
static_assert(sizeof(mo_sh_root) == 128, "root record layout");
static_assert(sizeof(mo_sh_prod) == 8, "product layout");
static_assert(offsetof(mo_sh_header, mats_offset) == 64, "header layout");
static_assert(offsetof(mo_sh_mat, rows) == 72, "matrix record layout");
static_assert(offsetof(mo_sh_root, op_ld) == 96, "root record layout");
