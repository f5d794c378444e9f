// Work-list layout shared by the host builder and the device kernels.
//
// The host turns the caller's bucket of matrix descriptors into one packed,
// little-endian byte string: a header, one record per non-empty matrix, and
// the tile items of the three Newton-Schulz GEMM phases.  The same bytes are
// uploaded to the front of the device workspace, so every kernel of the step
// reads its matrix table and item list from there.
#pragma once

#include <stddef.h>
#include <stdint.h>

#define MO_WL_MAGIC   0x4C574F4Du  // "MOWL"
#define MO_WL_VERSION 5u

// matrix index of a padding entry in a dispatch list
#define MO_WL_PAD 0xFFFFFFFFu

// Tile edge of the Newton-Schulz GEMMs.  Every NS-frame dimension is padded
// to a multiple of it inside the workspace, with zeros, so the GEMM kernels
// never test bounds: zero rows/columns of X stay zero through every step.
#define MO_GEMM_TILE 256
// Tile of the momentum kernel in the weight's own frame.
#define MO_MOM_TILE 64
// Alignment of every workspace region.
#define MO_WS_ALIGN 256

// flags of mo_wl_mat
#define MO_WLF_TRANSPOSED 0x1u   // rows > cols: X = U^T (Gram side = cols)
#define MO_WLF_HAS_UPDATE 0x2u   // update_out given
#define MO_WLF_W_BF16     0x4u   // W is bf16 (else fp32)
#define MO_WLF_G_BF16     0x8u   // G is bf16 (else fp32)

// Every field sits at its natural alignment, so the structs need no packing
// pragma and the device reads them with full-width loads.
struct mo_wl_header {
    uint32_t magic, version;
    uint32_t n_mats, ns_steps, ns_dtype, gemm_tile, mom_tile, elem_bytes;
    uint32_t n_mom_items, n_gram_items, n_poly_items, n_upd_items;
    uint32_t max_partials;
    uint32_t gemm_waves;    // wavefronts per workgroup of the GEMM kernels (4 or 8)
    uint64_t mats_offset, gram_offset, poly_offset, upd_offset;  // bytes from list start
    uint64_t wl_bytes;      // size of the list, a multiple of MO_WS_ALIGN
    uint64_t ws_bytes;      // workspace bytes from the aligned base (list included)
    float    ns_a, ns_b, ns_c, eps;
    uint32_t reserved1[2];
};

struct mo_wl_mat {
    uint64_t W, G, M, U;                 // caller pointers (U = update_out or 0)
    int64_t  ld_w, ld_g, ld_m, ld_u;     // element strides
    uint64_t off_X, off_Xt0, off_Xt1;    // NS-frame buffers (m_pad x n_pad, n_pad x m_pad x2)
    uint64_t off_A, off_B;               // m_pad x m_pad
    uint64_t off_partials, off_scale;    // n_partials floats; 4 floats
    uint32_t rows, cols, m, n, m_pad, n_pad;
    uint32_t flags, desc_index;
    uint32_t mom_begin;                  // first momentum item of this matrix
    uint32_t mom_tiles_c;                // momentum tiles along the weight's columns
    uint32_t n_partials;                 // = momentum tiles of this matrix
    float    lr_eff, decay;              // lr * shape factor; 1 - lr * wd
    uint32_t reserved[5];
};

// One GEMM tile: rows [256 ti, 256 ti + 256) and columns [64 nb tj, 64 nb tj +
// 64 nb) of the phase's product; nb = 4 is the full 256 x 256 tile, 2 and 1 the
// half and quarter widths.
struct mo_wl_item {
    uint32_t mat;
    uint32_t ti, tj;
    uint32_t nb;
};

static_assert(sizeof(mo_wl_header) == 128, "header layout");
static_assert(sizeof(mo_wl_mat) == 192, "matrix record layout");
static_assert(sizeof(mo_wl_item) == 16, "item layout");
static_assert(offsetof(mo_wl_header, mats_offset) == 56, "header layout");
static_assert(offsetof(mo_wl_header, ns_a) == 104, "header layout");
static_assert(offsetof(mo_wl_mat, off_X) == 64, "matrix record layout");
static_assert(offsetof(mo_wl_mat, rows) == 120, "matrix record layout");
static_assert(offsetof(mo_wl_mat, lr_eff) == 164, "matrix record layout");
