// gfx950 kernels of the owner-side Muon step.
//
// [P] = "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
// sharding".  The owner applies Muon to the whole 2D gradient (§3), whose
// Newton-Schulz steps are built from products X X^T (§2); the optimizer the
// paper runs is torch.optim.Muon (§5.1), whose momentum, normalisation,
// quintic coefficients and lr adjustment these kernels reproduce.
//
// Frames.  For a rows x cols matrix, m = min(rows, cols) and n = max(rows, cols).
// X (m x n, row-major, "NS frame") is U when rows <= cols and U^T otherwise.
// Every buffer is padded with zeros to multiples of MO_GEMM_TILE; zero rows and
// columns stay zero through every step, so the GEMM kernels never test bounds.
// The workspace keeps X twice: X itself (m_pad x n_pad) and X^T (n_pad x
// m_pad, ping-pong).  Then all three products read both operands along their
// contiguous dimension ("NT" form, C = P Q^T):
//   Gram    A = X X^T         P = X,  Q = X      (upper tiles; mirrored)
//   Poly    A A = A A^T       P = A,  Q = A      (A symmetric; upper tiles)
//   Update  B X = B (X^T)^T   P = B,  Q = X^T
#include "device_common.h"
#include "gemm_core.h"
#include "gemm_core8.h"
#include "mo_kernels.h"

namespace {

// ============================================================================
// momentum + Nesterov + norm partials + NS-frame layout  (HBM-bound)
// ============================================================================
//
// One workgroup per 64 x 64 tile of the weight's own (padded) frame.  Reads G
// and M once, writes M' (fp32), writes U rounded to the NS dtype twice: into
// the buffer that shares the weight's frame (coalesced) and, through LDS, into
// the transposed one.  Each tile leaves one fp32 partial sum of u^2.

constexpr int MOM_THREADS = 256;

// Streaming (non-temporal) 16-byte loads: G and M are read once per step.
// Stores stay ordinary 16-byte stores: non-temporal ones measured slower for
// this kernel (10-14 % while the transposed tile went out in pieces of 64
// rows, still 2-18 % with every store a whole 128-byte line).
MO_DEV u32x4 ld_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
MO_DEV void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
MO_DEV void unpack_bf16x8(const u32x4& raw, f32x8& o) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = (float)b[e];
}
MO_DEV void unpack_f32x8(const u32x4& a, const u32x4& b, f32x8& o) {
    const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) { o.v[e] = fa[e]; o.v[4 + e] = fb[e]; }
}
// The Update's X' tile pass: non-temporal 16-byte stores.  Eight lanes write
// each whole 128-byte row segment, so nothing is left for L2 to merge, and X'
// is next read by another launch; kept out of L2, the stores leave it to the
// operand panels (Update 226 -> 220 us per launch on the decoder bucket, 814
// -> 778 on the batched one, unchanged on the large one).  The mirrored pass,
// whose four lanes per row cover half a line, keeps ordinary stores.
MO_DEV void store8_stream(bf16_t* p, const f32x8& o) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16_t)o.v[e];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, b), reinterpret_cast<u32x4*>(p));
}
MO_DEV void store8_stream(float* p, const f32x8& o) { store8(p, o); }
template <typename T> MO_DEV void st8v(T* p, const f32x8& v);
template <> MO_DEV void st8v<bf16_t>(bf16_t* p, const f32x8& v) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16_t)v.v[e];
    st16(p, __builtin_bit_cast(u32x4, b));
}
template <> MO_DEV void st8v<float>(float* p, const f32x8& v) {
    st16(p, __builtin_bit_cast(u32x4, f32x4{v.v[0], v.v[1], v.v[2], v.v[3]}));
    st16(p + 4, __builtin_bit_cast(u32x4, f32x4{v.v[4], v.v[5], v.v[6], v.v[7]}));
}

template <typename XT>
__global__ __launch_bounds__(MOM_THREADS) void momentum_kernel(uint8_t* ws, float beta,
                                                               int nesterov) {
    __shared__ float tile[MO_MOM_TILE][MO_MOM_TILE + 1];
    __shared__ float red[MOM_THREADS / 64];
    const mo_wl_header* h = wl_header(ws);
    const mo_wl_mat* mats = wl_mats(ws);
    const uint32_t item = blockIdx.x;
    uint32_t lo = 0, hi = h->n_mats - 1;
    while (lo < hi) {   // last matrix whose first tile is <= item
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (mats[mid].mom_begin <= item) lo = mid; else hi = mid - 1;
    }
    const mo_wl_mat& mt = mats[lo];
    const uint32_t t = item - mt.mom_begin;
    const int64_t R0 = int64_t(t / mt.mom_tiles_c) * MO_MOM_TILE;
    const int64_t C0 = int64_t(t % mt.mom_tiles_c) * MO_MOM_TILE;
    const bool trans = mt.flags & MO_WLF_TRANSPOSED;
    const bool gbf = mt.flags & MO_WLF_G_BF16;
    const int64_t rows = mt.rows, cols = mt.cols;
    XT* direct = reinterpret_cast<XT*>(ws + (trans ? mt.off_Xt0 : mt.off_X));
    XT* transp = reinterpret_cast<XT*>(ws + (trans ? mt.off_X : mt.off_Xt0));
    const int64_t ld_direct = trans ? mt.m_pad : mt.n_pad;   // padded cols of the weight frame
    const int64_t ld_transp = trans ? mt.n_pad : mt.m_pad;   // padded rows of the weight frame
    const void* G = reinterpret_cast<const void*>(mt.G);
    float* M = reinterpret_cast<float*>(mt.M);
    const int64_t gsz = gbf ? 2 : 4;
    const bool gvec = ((mt.G | uint64_t(mt.ld_g * gsz)) & 15) == 0;
    const bool mvec = ((mt.M | uint64_t(mt.ld_m * 4)) & 15) == 0;
    const float omb = 1.0f - beta;

    // Thread q of the tile owns row q / 8, columns 8 (q % 8) .. + 7, for q =
    // thread and thread + 256.  Whole 8-column chunks of 16-byte-aligned
    // rows go through streaming vector loads, all issued before any store;
    // the matrix's edge goes element by element (zeros outside it).
    f32x8 g[2], mm[2];
    bool fast[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + MOM_THREADS * i;
        const int64_t row = R0 + (q >> 3), col0 = C0 + (q & 7) * 8;
        fast[i] = row < rows && col0 + 8 <= cols && gvec && mvec;
        if (fast[i]) {
            const float* mp = M + row * mt.ld_m + col0;
            const u32x4 m0 = ld_nt(mp), m1 = ld_nt(mp + 4);
            if (gbf) {
                unpack_bf16x8(ld_nt(reinterpret_cast<const bf16_t*>(G) + row * mt.ld_g + col0), g[i]);
            } else {
                const float* gp = reinterpret_cast<const float*>(G) + row * mt.ld_g + col0;
                unpack_f32x8(ld_nt(gp), ld_nt(gp + 4), g[i]);
            }
            unpack_f32x8(m0, m1, mm[i]);
        } else {
            const bool inrow = row < rows;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool in = inrow && col0 + e < cols;
                g[i].v[e] = in ? load_elem(G, row * mt.ld_g + col0 + e, gbf) : 0.f;
                mm[i].v[e] = in ? M[row * mt.ld_m + col0 + e] : 0.f;
            }
        }
    }
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + MOM_THREADS * i;
        const int r = q >> 3, cc = q & 7;
        const int64_t row = R0 + r, col0 = C0 + cc * 8;
        f32x8 mn, u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float mnew = beta * mm[i].v[e] + omb * g[i].v[e];
            const float uu = nesterov ? omb * g[i].v[e] + beta * mnew : mnew;
            mn.v[e] = mnew;
            u.v[e] = quantize<XT>(uu);          // zero outside the matrix
            sq += u.v[e] * u.v[e];
            tile[r][cc * 8 + e] = u.v[e];
        }
        if (fast[i]) {
            st8v<float>(M + row * mt.ld_m + col0, mn);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (row < rows && col0 + e < cols) M[row * mt.ld_m + col0 + e] = mn.v[e];
        }
        st8v<XT>(direct + row * ld_direct + col0, u);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + MOM_THREADS * i;
        // 8 consecutive threads write one whole 128-byte row of the transposed
        // tile (LDS bank of element e: rr * 8 + c + e, distinct over a wave)
        const int c = q >> 3, rr = q & 7;
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = tile[rr * 8 + e][c];
        st8v<XT>(transp + (C0 + c) * ld_transp + R0 + rr * 8, o);
    }
    const float tot = block_sum<MOM_THREADS>(sq, red);
    if (threadIdx.x == 0) reinterpret_cast<float*>(ws + mt.off_partials)[t] = tot;
}

// One workgroup per matrix: fixed-order sum of the tile partials, then
// scale = 1 / max(||U||_F, eps) (a clamp, as torch.optim.Muon normalises).
__global__ __launch_bounds__(256) void norm_kernel(uint8_t* ws) {
    __shared__ float red[4];
    const mo_wl_header* h = wl_header(ws);
    const mo_wl_mat& mt = wl_mats(ws)[blockIdx.x];
    const float* part = reinterpret_cast<const float*>(ws + mt.off_partials);
    float s = 0.f;
    for (uint32_t i = threadIdx.x; i < mt.n_partials; i += 256) s += part[i];
    const float tot = block_sum<256>(s, red);
    if (threadIdx.x == 0) {
        const float sc = 1.0f / fmaxf(sqrtf(tot), h->eps);
        float* scale = reinterpret_cast<float*>(ws + mt.off_scale);
        scale[0] = sc;
        scale[1] = sc * sc;
    }
}

// K == 0: W <- (1 - lr wd) W - lr_eff * scale * U, tiled like the momentum pass.
template <typename XT>
__global__ __launch_bounds__(MOM_THREADS) void apply_kernel(uint8_t* ws) {
    const mo_wl_header* h = wl_header(ws);
    const mo_wl_mat* mats = wl_mats(ws);
    const uint32_t item = blockIdx.x;
    uint32_t lo = 0, hi = h->n_mats - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (mats[mid].mom_begin <= item) lo = mid; else hi = mid - 1;
    }
    const mo_wl_mat& mt = mats[lo];
    const uint32_t t = item - mt.mom_begin;
    const int64_t R0 = int64_t(t / mt.mom_tiles_c) * MO_MOM_TILE;
    const int64_t C0 = int64_t(t % mt.mom_tiles_c) * MO_MOM_TILE;
    const bool trans = mt.flags & MO_WLF_TRANSPOSED;
    const bool wbf = mt.flags & MO_WLF_W_BF16;
    const XT* direct = reinterpret_cast<const XT*>(ws + (trans ? mt.off_Xt0 : mt.off_X));
    const int64_t ld_direct = trans ? mt.m_pad : mt.n_pad;
    const float sc = reinterpret_cast<const float*>(ws + mt.off_scale)[0];
    void* W = reinterpret_cast<void*>(mt.W);
    float* U = reinterpret_cast<float*>(mt.U);
    for (int q = threadIdx.x; q < MO_MOM_TILE * MO_MOM_TILE; q += MOM_THREADS) {
        const int64_t row = R0 + (q >> 6), col = C0 + (q & 63);
        if (row >= mt.rows || col >= mt.cols) continue;
        const float o = sc * to_f32(direct[row * ld_direct + col]);
        const float w = load_elem(W, row * mt.ld_w + col, wbf);
        store_elem(W, row * mt.ld_w + col, mt.decay * w - mt.lr_eff * o, wbf);
        if (U) U[row * mt.ld_u + col] = mt.lr_eff * o;
    }
}

// ============================================================================
// Newton-Schulz products on the shared NT GEMM core (gemm_core.h)
// ============================================================================

using namespace mo_gemm;

enum { KIND_GRAM = 0, KIND_POLY = 1, KIND_UPDATE = 2 };

// Epilogue of the Newton-Schulz products, one workgroup tile.  The mirrored
// pass ("pass B": for a sub-tile column j, 8 consecutive rows) runs first and
// forms the final values; the tile pass ("pass A": for a sub-tile row, 8
// consecutive columns) writes them in the tile's own orientation.
template <typename T, int KIND, bool LAST>
struct Epi {
    // Poly reads its epilogue operand A[i][j] = A[j][i] (small, in L2).  The
    // Update has no operand: the a X term is folded into the Poly output,
    // B' = a I + b A + c A^2, so the Update is the plain product X' = B' X
    // (exactly a X + B X; with bf16 B' the emulated error against the fp64
    // reference is no larger than with a X added in the fp32 epilogue).
    static constexpr bool CAP = false;
    static constexpr bool KROT = false;
    const mo_wl_mat* mt;
    T *X, *Xt_cur, *Xt_nxt, *A, *B;
    float alpha, sx, na, nb, nc;
    int64_t m_pad, n_pad, m;
    bool trans;

    // Gram and Poly write the mirror of an off-diagonal tile; Update writes
    // X^T (or, last, W when the weight is the transposed frame).  The tile
    // pass writes everything except the last Update of a transposed weight.
    // Poly forms its values in the mirrored pass (it needs the operand) and
    // hands them to the tile pass through the staging slice; Gram and Update
    // scale in each pass (the same fp32 arithmetic, so the same values).  The
    // last Update of a weight in the NS frame needs no mirrored pass at all.
    MO_DEV EpiPasses passes(bool off_diag) const {
        EpiPasses p;
        p.run_b = KIND == KIND_GRAM ? off_diag : KIND == KIND_POLY ? true : (!LAST || trans);
        p.write_b = KIND == KIND_UPDATE ? (!LAST || trans) : off_diag;
        p.run_a = !(KIND == KIND_UPDATE && LAST && trans);
        p.hand_over = KIND == KIND_POLY && p.run_a;
        return p;
    }

    // the Poly operand when it is not captured
    MO_DEV void operand(int64_t oj, int64_t oi, f32x8& o) const {
        if (KIND == KIND_POLY) load8(A + oj * m_pad + oi, o);            // A[i][j] = A[j][i]
    }

    MO_DEV void tile_value(f32x8& v) const {
        if (KIND == KIND_GRAM) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] *= alpha;
        } else if (KIND == KIND_UPDATE) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] *= sx;
            if (!LAST) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v.v[e] = quantize<T>(v.v[e]);
            }
        }
    }

    // Final values of the mirrored pass at row oj, columns oi .. oi + 7 of the
    // mirrored product, from the product v and (Poly) the operand o = A[i][j]:
    // B' = c A A + b A, plus a on the matrix's diagonal (i = j < m; the
    // padding stays zero).
    MO_DEV void combine(int64_t oj, int64_t oi, f32x8& v, const f32x8& o) const {
        if (KIND == KIND_POLY) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = (oi + e == oj && oj < m) ? na : 0.0f;
                v.v[e] = quantize<T>(nc * v.v[e] + nb * o.v[e] + d);
            }
        } else {
            tile_value(v);
        }
    }

    // pass B output: 8 values at mirrored position (row oj, columns oi..oi+7)
    MO_DEV void mirror(int64_t oj, int64_t oi, const f32x8& v) const {
        if (KIND == KIND_GRAM) store8(A + oj * m_pad + oi, v);
        else if (KIND == KIND_POLY) store8(B + oj * m_pad + oi, v);   // B is symmetric
        else if (!LAST) store8(Xt_nxt + oj * m_pad + oi, v);
        else write_w(oj, oi, v);                                       // weight frame is the transpose
    }

    // pass A output: 8 values at tile position (row gi, columns gj..gj+7)
    MO_DEV void tile(int64_t gi, int64_t gj, const f32x8& v) const {
        if (KIND == KIND_GRAM) store8(A + gi * m_pad + gj, v);
        else if (KIND == KIND_POLY) store8(B + gi * m_pad + gj, v);
        else if (!LAST) store8_stream(X + gi * n_pad + gj, v);
        else write_w(gi, gj, v);                                       // weight frame == NS frame
    }

    // W[r][c..c+7] <- decay * W - lr_eff * O, clipped to the matrix; 16-byte
    // vector accesses when the chunk is whole and the rows are aligned.
    bool vec_w, vec_u;
    MO_DEV void write_w(int64_t r, int64_t c, const f32x8& o) const {
        if (r >= mt->rows) return;
        const bool wbf = mt->flags & MO_WLF_W_BF16;
        void* W = reinterpret_cast<void*>(mt->W);
        float* U = reinterpret_cast<float*>(mt->U);
        const float decay = mt->decay, lr = mt->lr_eff;
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

// One Newton-Schulz tile (width 256 or 128): the phase's operands and
// epilogue around the 8-wavefront GEMM core (gemm_core8.h).
//   Gram    A = X X^T         P = X,  Q = X      (upper tiles; mirrored)
//   Poly    A A = A A^T       P = A,  Q = A      (A symmetric; upper tiles)
//   Update  B' X = B' (X^T)^T P = B', Q = X^T
template <typename T, int KIND, bool LAST, int NB, bool EIGHT>
__device__ __forceinline__ void gemm_tile(uint8_t* smem, uint8_t* ws, const mo_wl_item& it, int first,
                                          int xt_cur) {
    const mo_wl_header* h = wl_header(ws);
    const mo_wl_mat& mt = wl_mats(ws)[it.mat];
    const int64_t m_pad = mt.m_pad, n_pad = mt.n_pad;
    T* X = reinterpret_cast<T*>(ws + mt.off_X);
    T* Xt_cur = reinterpret_cast<T*>(ws + (xt_cur ? mt.off_Xt1 : mt.off_Xt0));
    T* Xt_nxt = reinterpret_cast<T*>(ws + (xt_cur ? mt.off_Xt0 : mt.off_Xt1));
    T* A = reinterpret_cast<T*>(ws + mt.off_A);
    T* B = reinterpret_cast<T*>(ws + mt.off_B);
    const float* scale = reinterpret_cast<const float*>(ws + mt.off_scale);

    auto make_ep = [&]() __attribute__((always_inline)) {
        Epi<T, KIND, LAST> ep;
        ep.mt = &mt;
        ep.X = X; ep.Xt_cur = Xt_cur; ep.Xt_nxt = Xt_nxt; ep.A = A; ep.B = B;
        ep.alpha = (KIND == KIND_GRAM && first) ? scale[1] : 1.0f;
        ep.sx = (KIND == KIND_UPDATE && first) ? scale[0] : 1.0f;
        ep.na = h->ns_a; ep.nb = h->ns_b; ep.nc = h->ns_c;
        ep.m_pad = m_pad; ep.n_pad = n_pad; ep.m = mt.m;
        ep.trans = mt.flags & MO_WLF_TRANSPOSED;
        const int64_t wes = (mt.flags & MO_WLF_W_BF16) ? 2 : 4;
        ep.vec_w = ((mt.W | uint64_t(mt.ld_w * wes)) & 15) == 0;
        ep.vec_u = ((mt.U | uint64_t(mt.ld_u * 4)) & 15) == 0;
        return ep;
    };
    const int ti = int(it.ti), tj = int(it.tj);
    const T* P = KIND == KIND_GRAM ? X : KIND == KIND_POLY ? A : B;
    const T* Q = KIND == KIND_GRAM ? X : KIND == KIND_POLY ? A : Xt_cur;
    const int64_t ld = KIND == KIND_GRAM ? n_pad : m_pad;
    if constexpr (EIGHT) gemm_core8<T, NB>(smem, P, Q, ld, ti, tj, make_ep);
    else gemm_core<T, NB>(smem, P, Q, ld, ti, tj, make_ep);
}

// Entry b of the phase's dispatch list is workgroup b's tile; the tile width
// (NB) is uniform per workgroup.  bf16 products run on the 8-wavefront core
// (widths 256 and 128); fp32 ones, whose buckets are small and whose fp32
// MFMAs run at a sixteenth of the bf16 rate, on the 4-wavefront core, which
// also has the quarter width (64) and so spreads a small product over more
// CUs.
template <typename T, int KIND, bool LAST, int NB>
__device__ __forceinline__ void gemm_tile_any(uint8_t* smem, uint8_t* ws, const mo_wl_item& it, int first,
                                              int xt_cur) {
    if constexpr (sizeof(T) == 2) gemm_tile<T, KIND, LAST, NB, true>(smem, ws, it, first, xt_cur);
    else gemm_tile<T, KIND, LAST, NB, false>(smem, ws, it, first, xt_cur);
}

template <typename T, int KIND, bool LAST>
__device__ __forceinline__ void gemm_entry(uint8_t* ws, int first, int xt_cur) {
    __shared__ __align__(16) uint8_t smem[GEMM_LDS];
    const mo_wl_header* h = wl_header(ws);
    const uint64_t items_off = KIND == KIND_GRAM ? h->gram_offset
                             : KIND == KIND_POLY ? h->poly_offset : h->upd_offset;
    const mo_wl_item it = reinterpret_cast<const mo_wl_item*>(ws + items_off)[blockIdx.x];
    if (it.mat == MO_WL_PAD) return;
    if (it.nb == 4) gemm_tile_any<T, KIND, LAST, 4>(smem, ws, it, first, xt_cur);
    else if (it.nb == 2) gemm_tile_any<T, KIND, LAST, 2>(smem, ws, it, first, xt_cur);
    else if constexpr (sizeof(T) == 4) gemm_tile_any<T, KIND, LAST, 1>(smem, ws, it, first, xt_cur);
}

inline unsigned grid_for(uint32_t items) { return items; }   // dispatch lists are padded to 8

// One plainly named kernel per (phase, NS dtype), so profiles name them
// unambiguously: bf16 on 512 threads (two wavefronts per SIMD), fp32 on 256
// (one per SIMD, all 512 registers per lane).
#define MO_GEMM_KERNEL8(name, T, KIND, LAST)                                              \
    __global__ __launch_bounds__(G8_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))   \
    void name(uint8_t* ws, int first, int xt_cur) { gemm_entry<T, KIND, LAST>(ws, first, xt_cur); }
#define MO_GEMM_KERNEL4(name, T, KIND, LAST)                                              \
    __global__ __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))    \
    void name(uint8_t* ws, int first, int xt_cur) { gemm_entry<T, KIND, LAST>(ws, first, xt_cur); }
MO_GEMM_KERNEL8(gram_bf16, bf16_t, KIND_GRAM, false)
MO_GEMM_KERNEL4(gram_f32, float, KIND_GRAM, false)
MO_GEMM_KERNEL8(poly_bf16, bf16_t, KIND_POLY, false)
MO_GEMM_KERNEL4(poly_f32, float, KIND_POLY, false)
MO_GEMM_KERNEL8(update_bf16, bf16_t, KIND_UPDATE, false)
MO_GEMM_KERNEL4(update_f32, float, KIND_UPDATE, false)
MO_GEMM_KERNEL8(update_last_bf16, bf16_t, KIND_UPDATE, true)
MO_GEMM_KERNEL4(update_last_f32, float, KIND_UPDATE, true)
#undef MO_GEMM_KERNEL8
#undef MO_GEMM_KERNEL4

}  // namespace

// ============================================================================
// launchers
// ============================================================================

hipError_t mo_launch_momentum(const mo_wl_header& h, uint8_t* ws, float beta, int nesterov,
                              hipStream_t s) {
    if (h.n_mom_items == 0) return hipSuccess;
    if (h.ns_dtype == MO_BF16)
        hipLaunchKernelGGL(momentum_kernel<bf16_t>, dim3(h.n_mom_items), dim3(MOM_THREADS), 0, s, ws, beta, nesterov);
    else
        hipLaunchKernelGGL(momentum_kernel<float>, dim3(h.n_mom_items), dim3(MOM_THREADS), 0, s, ws, beta, nesterov);
    return hipGetLastError();
}

hipError_t mo_launch_norm(const mo_wl_header& h, uint8_t* ws, hipStream_t s) {
    if (h.n_mats == 0) return hipSuccess;
    hipLaunchKernelGGL(norm_kernel, dim3(h.n_mats), dim3(256), 0, s, ws);
    return hipGetLastError();
}

hipError_t mo_launch_apply(const mo_wl_header& h, uint8_t* ws, hipStream_t s) {
    if (h.n_mom_items == 0) return hipSuccess;
    if (h.ns_dtype == MO_BF16)
        hipLaunchKernelGGL(apply_kernel<bf16_t>, dim3(h.n_mom_items), dim3(MOM_THREADS), 0, s, ws);
    else
        hipLaunchKernelGGL(apply_kernel<float>, dim3(h.n_mom_items), dim3(MOM_THREADS), 0, s, ws);
    return hipGetLastError();
}

typedef void (*gemm_fn)(uint8_t*, int, int);

static hipError_t launch_gemm(const mo_wl_header& h, uint32_t items, gemm_fn bf, gemm_fn f32,
                              uint8_t* ws, int first, int xt_cur, hipStream_t s) {
    if (items == 0) return hipSuccess;
    const bool bf16 = h.ns_dtype == MO_BF16;
    const uint32_t threads = bf16 ? G8_THREADS : G_THREADS;
    if (h.gemm_waves != threads / 64) return hipErrorInvalidValue;   // list built for other kernels
    hipLaunchKernelGGL((bf16 ? bf : f32), dim3(grid_for(items)), dim3(threads), 0, s, ws, first, xt_cur);
    return hipGetLastError();
}

hipError_t mo_launch_gram(const mo_wl_header& h, uint8_t* ws, int first, int xt_cur, hipStream_t s) {
    return launch_gemm(h, h.n_gram_items, gram_bf16, gram_f32, ws, first, xt_cur, s);
}
hipError_t mo_launch_poly(const mo_wl_header& h, uint8_t* ws, hipStream_t s) {
    return launch_gemm(h, h.n_poly_items, poly_bf16, poly_f32, ws, 0, 0, s);
}
hipError_t mo_launch_update(const mo_wl_header& h, uint8_t* ws, int first, int last, int xt_cur,
                            hipStream_t s) {
    return last ? launch_gemm(h, h.n_upd_items, update_last_bf16, update_last_f32, ws, first, xt_cur, s)
                : launch_gemm(h, h.n_upd_items, update_bf16, update_f32, ws, first, xt_cur, s);
}
