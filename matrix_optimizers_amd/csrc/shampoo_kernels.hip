// gfx950 kernels of the owner-side Shampoo step (fp32 throughout).
//
// [P] = "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
// sharding", §5.7: the owner, holding each 2D matrix whole, runs Shampoo with
// full left / right preconditioners and an inverse fourth root, in float32.
// The step on one matrix (the readings are stated with the C entry point):
//   L' = L + G G^T,  R' = R + G^T G                  statistics products
//   H_L ~ L'^{-1/4},  H_R ~ R'^{-1/4}                 coupled Newton iterations
//   W' = (1 - lr wd) W - lr H_L G H_R                 two products, W written
//
// Every buffer is padded with zeros to multiples of MO_GEMM_TILE, and the
// identity of the root iteration lives on the true diagonal only, so padding
// stays zero through every product and the GEMMs never test bounds.  Root
// products are polynomials in one symmetric matrix, hence symmetric: only
// most of them compute their upper tiles and mirror them; the H products are
// kept unsymmetrised (see sh_worklist.h).  All products use the NT form
// C = P Q^T of the shared core (for a symmetric Q, P Q^T = P Q).
#include "device_common.h"
#include "gemm_core.h"
#include "mo_kernels.h"
#include "sh_worklist.h"

namespace {

using namespace mo_gemm;

constexpr int SH_THREADS = 256;
constexpr int ST = 64;   // tile of the elementwise kernels

MO_DEV const mo_sh_header* sh_header(const uint8_t* ws) {
    return reinterpret_cast<const mo_sh_header*>(ws);
}
MO_DEV const mo_sh_mat* sh_mats(const uint8_t* ws) {
    return reinterpret_cast<const mo_sh_mat*>(ws + sh_header(ws)->mats_offset);
}
MO_DEV const mo_sh_root* sh_roots(const uint8_t* ws) {
    return reinterpret_cast<const mo_sh_root*>(ws + sh_header(ws)->roots_offset);
}

// ============================================================================
// layout: G -> padded G (r_pad x c_pad) and G^T (c_pad x r_pad), fp32
// ============================================================================
//
// One workgroup per 64 x 64 tile of the padded frame; the transpose goes
// through LDS so both writes are row-contiguous.
__global__ __launch_bounds__(SH_THREADS) void sh_layout_kernel(uint8_t* ws) {
    __shared__ float tile[ST][ST + 1];
    const mo_sh_header* h = sh_header(ws);
    const mo_sh_mat* mats = sh_mats(ws);
    const uint32_t item = blockIdx.x;
    uint32_t lo = 0, hi = h->n_mats - 1;
    while (lo < hi) {   // last matrix whose first tile is <= item
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (mats[mid].lay_begin <= item) lo = mid; else hi = mid - 1;
    }
    const mo_sh_mat& mt = mats[lo];
    const uint32_t t = item - mt.lay_begin;
    const int64_t R0 = int64_t(t / mt.lay_tiles_c) * ST, C0 = int64_t(t % mt.lay_tiles_c) * ST;
    const bool gbf = mt.flags & MO_SHF_G_BF16;
    const void* G = reinterpret_cast<const void*>(mt.G);
    float* Gp = reinterpret_cast<float*>(ws + mt.off_G);
    float* Gt = reinterpret_cast<float*>(ws + mt.off_Gt);
    const int64_t rows = mt.rows, cols = mt.cols;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + SH_THREADS * i;
        const int r = q >> 3, cc = q & 7;
        const int64_t row = R0 + r, col0 = C0 + cc * 8;
        f32x8 g;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            g.v[e] = (row < rows && col0 + e < cols) ? load_elem(G, row * mt.ld_g + col0 + e, gbf) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[r][cc * 8 + e] = g.v[e];
        store8(Gp + row * mt.c_pad + col0, g);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + SH_THREADS * i;
        // 8 consecutive threads write 256 contiguous bytes of one row of G^T
        // (LDS bank of element e: rr * 8 + c + e, distinct over a wave)
        const int c = q >> 3, rr = q & 7;
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = tile[rr * 8 + e][c];
        store8(Gt + (C0 + c) * mt.r_pad + R0 + rr * 8, o);
    }
}

// ============================================================================
// root preparation: ||S'||_F, z = (p + 1) / (2 ||S'||_F), X_0 and H_1
// ============================================================================

MO_DEV const mo_sh_root& root_of_item(const uint8_t* ws, uint32_t item) {
    const mo_sh_header* h = sh_header(ws);
    const mo_sh_root* roots = sh_roots(ws);
    uint32_t lo = 0, hi = h->n_roots - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (roots[mid].item_begin <= item) lo = mid; else hi = mid - 1;
    }
    return roots[lo];
}

// One workgroup per 64 x 64 tile of a padded root: its sum of squares of M_0.
__global__ __launch_bounds__(SH_THREADS) void sh_sumsq_kernel(uint8_t* ws) {
    __shared__ float red[SH_THREADS / 64];
    const mo_sh_root& rt = root_of_item(ws, blockIdx.x);
    const uint32_t t = blockIdx.x - rt.item_begin;
    const int64_t R0 = int64_t(t / rt.tiles_c) * ST, C0 = int64_t(t % rt.tiles_c) * ST;
    const float* M0 = reinterpret_cast<const float*>(ws + rt.off_M[0]);
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + SH_THREADS * i;
        f32x8 v;
        load8(M0 + (R0 + (q >> 3)) * rt.m_pad + C0 + (q & 7) * 8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sq += v.v[e] * v.v[e];
    }
    const float tot = block_sum<SH_THREADS>(sq, red);
    if (threadIdx.x == 0) reinterpret_cast<float*>(ws + rt.off_partials)[t] = tot;
}

// One workgroup per root: fixed-order sum of the tile partials, then
// z = (p + 1) / (2 ||S'||_F) and z^(1/p).
__global__ __launch_bounds__(256) void sh_norm_kernel(uint8_t* ws) {
    __shared__ float red[4];
    const mo_sh_root& rt = sh_roots(ws)[blockIdx.x];
    const float* part = reinterpret_cast<const float*>(ws + rt.off_partials);
    float s = 0.f;
    for (uint32_t i = threadIdx.x; i < rt.n_partials; i += 256) s += part[i];
    const float tot = block_sum<256>(s, red);
    if (threadIdx.x == 0) {
        const float z = float(MO_SH_P + 1) / (2.0f * sqrtf(tot));
        float* scale = reinterpret_cast<float*>(ws + rt.off_scale);
        scale[0] = z;
        scale[1] = sqrtf(sqrtf(z));   // z^(1/4)
    }
}

// X_0 = ((p + 1) I - z M_0) / p and H_1 = z^(1/p) X_0, per 64 x 64 tile.
__global__ __launch_bounds__(SH_THREADS) void sh_init_kernel(uint8_t* ws) {
    const mo_sh_root& rt = root_of_item(ws, blockIdx.x);
    const uint32_t t = blockIdx.x - rt.item_begin;
    const int64_t R0 = int64_t(t / rt.tiles_c) * ST, C0 = int64_t(t % rt.tiles_c) * ST;
    const float* scale = reinterpret_cast<const float*>(ws + rt.off_scale);
    const float z = scale[0], zr = scale[1];
    const float* M0 = reinterpret_cast<const float*>(ws + rt.off_M[0]);
    float* X = reinterpret_cast<float*>(ws + rt.off_X);
    float* H1 = reinterpret_cast<float*>(ws + rt.off_H[1]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + SH_THREADS * i;
        const int64_t row = R0 + (q >> 3), col0 = C0 + (q & 7) * 8;
        const int64_t idx = row * rt.m_pad + col0;
        f32x8 v, x, hh;
        load8(M0 + idx, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float d = (row == col0 + e && row < rt.m) ? float(MO_SH_P + 1) : 0.f;
            x.v[e] = (d - z * v.v[e]) * (1.0f / MO_SH_P);
            hh.v[e] = zr * x.v[e];
        }
        store8(X + idx, x);
        store8(H1 + idx, hh);
    }
}

// ============================================================================
// grouped GEMM products
// ============================================================================

// Epilogue of one Shampoo product tile (fp32; see the kinds in sh_worklist.h).
struct ShEpi {
    static constexpr bool CAP = false;
    static constexpr bool KROT = true;   // see sh_tile
    int kind;
    float* out0;          // padded output (row stride ld_out)
    float* out1;          // M kind: X_k
    int64_t ld_out;
    uint32_t m;           // true side of a root (identity, caller bounds)
    float alpha;
    float* ext;           // STATS: caller statistics, m x m, row stride ld_ext
    int64_t ld_ext;
    bool vec_ext;
    const mo_sh_mat* mt;  // RIGHT: the weight
    bool vec_w, vec_u;
    bool off_diag;        // the tile lies off the diagonal of a square product

    MO_DEV EpiPasses passes(bool off_diag) const {
        EpiPasses p;
        if (kind == MO_SHK_LEFT || kind == MO_SHK_RIGHT || kind == MO_SHK_H) {
            p.run_b = false; p.write_b = false; p.run_a = true; p.hand_over = false;
        } else if (kind == MO_SHK_HT) {
            // the mirrored pass alone: every value at its transposed position
            p.run_b = true; p.write_b = true; p.run_a = false; p.hand_over = false;
        } else if (kind == MO_SHK_STATS) {
            // the old statistics are read in the mirrored pass, so it forms
            // every value and hands them over; it also writes the caller's
            // copy on diagonal tiles (see put)
            p.run_b = true; p.write_b = true; p.run_a = true; p.hand_over = true;
        } else {
            p.run_b = off_diag; p.write_b = off_diag; p.run_a = true; p.hand_over = false;
        }
        return p;
    }

    // STATS: the old statistics at row oj, columns oi .. oi + 7 (zero outside m x m)
    MO_DEV void operand(int64_t oj, int64_t oi, f32x8& o) const {
        if (kind != MO_SHK_STATS) return;
        const int64_t base = oj * ld_ext + oi;
        if (oj < m && oi + 8 <= m && vec_ext) {
            load8(ext + base, o);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o.v[e] = (oj < m && oi + e < m) ? ext[base + e] : 0.f;
        }
    }

    MO_DEV void combine(int64_t, int64_t, f32x8& v, const f32x8& o) const {
        if (kind == MO_SHK_STATS) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] += o.v[e];
        } else {
            tile_value(v);
        }
    }

    MO_DEV void tile_value(f32x8& v) const {
        if (kind == MO_SHK_M) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] *= alpha;
        }
    }

    // 8 values at row r, columns c .. c + 7 of the product, from the mirrored
    // pass (mirrored) or the tile pass.  STATS reads the caller's statistics
    // in the mirrored pass at exactly the elements that pass writes: on a
    // diagonal tile the tile pass covers the transposes of those elements, so
    // it must not write the caller's copy there (another wave, or a later
    // round of the same wave, may still read them); it writes the padded copy
    // only, and the mirrored pass writes the caller's copy only.
    MO_DEV void put(int64_t r, int64_t c, const f32x8& v, bool mirrored) const {
        if (kind == MO_SHK_RIGHT) {
            write_w(r, c, v);
            return;
        }
        const bool padded = kind != MO_SHK_STATS || off_diag || !mirrored;
        const bool caller = kind == MO_SHK_STATS && (off_diag || mirrored);
        if (padded) store8(out0 + r * ld_out + c, v);
        if (kind == MO_SHK_M) {
            f32x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = (r == c + e && r < m) ? float(MO_SH_P + 1) : 0.f;
                x.v[e] = (d - v.v[e]) * (1.0f / MO_SH_P);
            }
            store8(out1 + r * ld_out + c, x);
        } else if (caller && r < m) {
            const int64_t base = r * ld_ext + c;
            if (c + 8 <= m && vec_ext) {
                store8(ext + base, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (c + e < m) ext[base + e] = v.v[e];
            }
        }
    }
    MO_DEV void mirror(int64_t oj, int64_t oi, const f32x8& v) const { put(oj, oi, v, true); }
    MO_DEV void tile(int64_t gi, int64_t gj, const f32x8& v) const { put(gi, gj, v, false); }

    // W[r][c..c+7] <- decay * W - lr * O, clipped to the matrix
    MO_DEV void write_w(int64_t r, int64_t c, const f32x8& o) const {
        if (r >= mt->rows) return;
        const bool wbf = mt->flags & MO_SHF_W_BF16;
        void* W = reinterpret_cast<void*>(mt->W);
        float* U = reinterpret_cast<float*>(mt->U);
        const float decay = mt->decay, lr = mt->lr;
        const int64_t wi = r * mt->ld_w + c;
        if (c + 8 <= mt->cols && vec_w) {
            f32x8 w;
            if (wbf) load8(reinterpret_cast<const bf16_t*>(W) + wi, w);
            else load8(reinterpret_cast<const float*>(W) + wi, w);
#pragma unroll
            for (int e = 0; e < 8; ++e) w.v[e] = decay * w.v[e] - lr * o.v[e];
            if (wbf) store8(reinterpret_cast<bf16_t*>(W) + wi, w);
            else store8(reinterpret_cast<float*>(W) + wi, w);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (c + e < mt->cols) store_elem(W, wi + e, decay * load_elem(W, wi + e, wbf) - lr * o.v[e], wbf);
        }
        if (U) {
            const int64_t ui = r * mt->ld_u + c;
            if (c + 8 <= mt->cols && vec_u) {
                f32x8 u;
#pragma unroll
                for (int e = 0; e < 8; ++e) u.v[e] = lr * o.v[e];
                store8(U + ui, u);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (c + e < mt->cols) U[ui + e] = lr * o.v[e];
            }
        }
    }
};

// The epilogue of product `pr` at root iteration k (root products read
// H_{k-1} and M_{k-1} and write H_k, M_k, X_k; H_K sits in H[K & 1]).
MO_DEV ShEpi make_sh_epi(uint8_t* ws, const mo_sh_prod& pr, const mo_wl_item& it, int k) {
    const mo_sh_header* h = sh_header(ws);
    auto F = [&](uint64_t off) { return reinterpret_cast<float*>(ws + off); };
    ShEpi ep;
    ep.kind = int(pr.kind);
    ep.out0 = ep.out1 = nullptr;
    ep.alpha = 1.0f;
    ep.ext = nullptr;
    ep.ld_ext = 0;
    ep.vec_ext = false;
    ep.mt = nullptr;
    ep.vec_w = ep.vec_u = false;
    ep.m = 0;
    ep.off_diag = it.ti != it.tj * it.nb / 4;   // tile columns 64 nb tj ..
    if (pr.kind == MO_SHK_LEFT || pr.kind == MO_SHK_RIGHT) {
        const mo_sh_mat& mt = sh_mats(ws)[pr.ref];
        ep.ld_out = mt.c_pad;
        if (pr.kind == MO_SHK_LEFT) {
            ep.out0 = F(mt.off_T);
        } else {
            ep.mt = &mt;
            const int64_t wes = (mt.flags & MO_SHF_W_BF16) ? 2 : 4;
            ep.vec_w = ((mt.W | uint64_t(mt.ld_w * wes)) & 15) == 0;
            ep.vec_u = ((mt.U | uint64_t(mt.ld_u * 4)) & 15) == 0;
        }
        return ep;
    }
    const mo_sh_root& rt = sh_roots(ws)[pr.ref];
    ep.m = rt.m;
    ep.ld_out = rt.m_pad;
    const int ck = k & 1;
    if (pr.kind == MO_SHK_STATS) {
        ep.out0 = F(rt.off_M[0]);
        ep.ext = reinterpret_cast<float*>(rt.ext);
        ep.ld_ext = rt.ld_ext;
        ep.vec_ext = ((rt.ext | uint64_t(rt.ld_ext * 4)) & 15) == 0;
    } else if (pr.kind == MO_SHK_SQ) {
        ep.out0 = F(rt.off_S2);
    } else if (pr.kind == MO_SHK_H || pr.kind == MO_SHK_HT) {
        ep.out0 = F(rt.off_H[ck]);
    } else if (pr.kind == MO_SHK_S4) {
        ep.out0 = F(rt.off_S4);
    } else {   // MO_SHK_M
        ep.out0 = F(rt.off_M[ck]);
        ep.out1 = F(rt.off_X);
        ep.alpha = k == 1 ? reinterpret_cast<const float*>(ws + rt.off_scale)[0] : 1.0f;
    }
    (void)h;
    return ep;
}

// Operands of one product tile (see the kinds in sh_worklist.h).
template <int NB>
MO_DEV void sh_tile(uint8_t* smem, uint8_t* ws, const mo_wl_item& it, int k) {
    const mo_sh_header* h = sh_header(ws);
    const mo_sh_prod pr = reinterpret_cast<const mo_sh_prod*>(ws + h->prods_offset)[it.mat];
    auto F = [&](uint64_t off) { return reinterpret_cast<const float*>(ws + off); };
    const int kf = int(h->root_iters) & 1;
    const float* P;
    const float* Q;
    int64_t ld;
    if (pr.kind == MO_SHK_LEFT || pr.kind == MO_SHK_RIGHT) {
        const mo_sh_mat& mt = sh_mats(ws)[pr.ref];
        const mo_sh_root* roots = sh_roots(ws);
        if (pr.kind == MO_SHK_LEFT) {
            P = F(roots[mt.root_l].off_H[kf]); Q = F(mt.off_Gt); ld = mt.r_pad;
        } else {
            P = F(mt.off_T); Q = F(roots[mt.root_r].off_H[kf]); ld = mt.c_pad;
        }
    } else {
        const mo_sh_root& rt = sh_roots(ws)[pr.ref];
        const int pk = (k - 1) & 1;
        ld = rt.m_pad;
        if (pr.kind == MO_SHK_STATS) {
            P = Q = F(rt.off_op); ld = rt.op_ld;
        } else if (pr.kind == MO_SHK_SQ) {
            P = Q = F(rt.off_X);
        } else if (pr.kind == MO_SHK_H || pr.kind == MO_SHK_HT) {
            P = F(rt.off_H[pk]); Q = F(rt.off_X);
        } else if (pr.kind == MO_SHK_S4) {
            P = Q = F(rt.off_S2);
        } else {   // MO_SHK_M
            P = F(rt.off_S4); Q = F(rt.off_M[pk]);
        }
    }
    // K order.  The root products and both preconditioner products are
    // dominated by one term per output: k = i for X X^T, S4, M and H_L^T G
    // (diagonal-heavy left factor), k = j for H X^T and T H_R (diagonal-heavy
    // right factor).  A sequential fp32 sum drops the small terms that follow
    // a large one (each is below half a unit of the running sum), always
    // toward the same side, so the K loop starts after the 256-wide block
    // that holds the dominant term and ends with it.
    // The statistics product (K = the other side of G) has no such term and
    // keeps the plain order.  krot is reduced modulo the stage count, so every
    // stage index stays in [0, nk).
    const int last = (pr.kind == MO_SHK_H || pr.kind == MO_SHK_HT || pr.kind == MO_SHK_RIGHT)
                         ? int(it.tj * it.nb / 4) : int(it.ti);
    const int per_block = GT * int(sizeof(float)) / KB;          // K stages per 256 columns
    const int nk = int(ld * int64_t(sizeof(float)) / KB);
    const int krot = pr.kind == MO_SHK_STATS ? 0 : ((last + 1) * per_block) % nk;
    auto make_ep = [&]() __attribute__((always_inline)) { return make_sh_epi(ws, pr, it, k); };
    gemm_core<float, NB>(smem, P, Q, ld, int(it.ti), int(it.tj), make_ep, krot);
}

__global__ __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sh_gemm_f32(uint8_t* ws, int list, int k) {
    __shared__ __align__(16) uint8_t smem[GEMM_LDS];
    const mo_sh_header* h = sh_header(ws);
    const mo_wl_item it = reinterpret_cast<const mo_wl_item*>(ws + h->list_offset[list])[blockIdx.x];
    if (it.mat == MO_WL_PAD) return;
    if (it.nb == 4) sh_tile<4>(smem, ws, it, k);
    else if (it.nb == 2) sh_tile<2>(smem, ws, it, k);
    else sh_tile<1>(smem, ws, it, k);
}

}  // namespace

// ============================================================================
// launchers
// ============================================================================

hipError_t mo_launch_sh_layout(const mo_sh_header& h, uint8_t* ws, hipStream_t s) {
    if (h.n_lay_items == 0) return hipSuccess;
    hipLaunchKernelGGL(sh_layout_kernel, dim3(h.n_lay_items), dim3(SH_THREADS), 0, s, ws);
    return hipGetLastError();
}

hipError_t mo_launch_sh_rootprep(const mo_sh_header& h, uint8_t* ws, hipStream_t s) {
    if (h.n_root_items == 0) return hipSuccess;
    hipLaunchKernelGGL(sh_sumsq_kernel, dim3(h.n_root_items), dim3(SH_THREADS), 0, s, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sh_norm_kernel, dim3(h.n_roots), dim3(256), 0, s, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(sh_init_kernel, dim3(h.n_root_items), dim3(SH_THREADS), 0, s, ws);
    return hipGetLastError();
}

hipError_t mo_launch_sh_gemm(const mo_sh_header& h, uint8_t* ws, int list, int k, hipStream_t s) {
    if (list < 0 || list >= MO_SHL_COUNT) return hipErrorInvalidValue;
    if (h.n_items[list] == 0) return hipSuccess;
    hipLaunchKernelGGL(sh_gemm_f32, dim3(h.n_items[list]), dim3(G_THREADS), 0, s, ws, list, k);
    return hipGetLastError();
}
