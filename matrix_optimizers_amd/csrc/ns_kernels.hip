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

    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + MOM_THREADS * i;
        const int r = q >> 3, cc = q & 7;
        const int64_t row = R0 + r, col0 = C0 + cc * 8;
        f32x8 g, mm, u;
        const bool inrow = row < rows;
        const bool full = inrow && col0 + 8 <= cols;
        if (full && gvec) {
            if (gbf) load8(reinterpret_cast<const bf16_t*>(G) + row * mt.ld_g + col0, g);
            else load8(reinterpret_cast<const float*>(G) + row * mt.ld_g + col0, g);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                g.v[e] = (inrow && col0 + e < cols) ? load_elem(G, row * mt.ld_g + col0 + e, gbf) : 0.f;
        }
        if (full && mvec) {
            load8(M + row * mt.ld_m + col0, mm);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                mm.v[e] = (inrow && col0 + e < cols) ? M[row * mt.ld_m + col0 + e] : 0.f;
        }
        f32x8 mn;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float mnew = beta * mm.v[e] + omb * g.v[e];
            const float uu = nesterov ? omb * g.v[e] + beta * mnew : mnew;
            mn.v[e] = mnew;
            u.v[e] = quantize<XT>(uu);          // zero outside the matrix
            sq += u.v[e] * u.v[e];
            tile[r][cc * 8 + e] = u.v[e];
        }
        if (full && mvec) {
            store8(M + row * mt.ld_m + col0, mn);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (inrow && col0 + e < cols) M[row * mt.ld_m + col0 + e] = mn.v[e];
        }
        store8(direct + row * ld_direct + col0, u);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = threadIdx.x + MOM_THREADS * i;
        const int c = q & 63, rr = q >> 6;
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = tile[rr * 8 + e][c];
        store8(transp + (C0 + c) * ld_transp + R0 + rr * 8, o);
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
// NT GEMM family on MFMA:  C[i][j] = sum_k P[i][k] * Q[j][k]
// ============================================================================
//
// Workgroup tile 128 x 128, 256 threads = 4 wavefronts in a 2 x 2 grid, each
// wavefront owning 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.  K advances by 128
// bytes per stage (64 bf16 / 32 fp32) through double-buffered LDS; global loads
// of stage s+1 are in flight while stage s is multiplied.  LDS rows are 128
// bytes of eight 16-byte chunks, chunk index XOR (row & 7), so both the 16-byte
// stores of the global->LDS copy and the 16-byte fragment reads of 8 (32)
// consecutive rows hit distinct banks.
//
// MFMA operands.  bf16: v_mfma_f32_32x32x16_bf16 takes 8 consecutive k per
// lane; lane l supplies row (l % 32) and k-group (l / 32).  fp32:
// v_mfma_f32_32x32x2_f32 takes one k per lane; a 16-byte chunk of 4 floats feeds
// four of them.  A and B fragments use the same lane -> k assignment, so the
// sum over all k is exact regardless of how k is split among lanes.  The 32 x 32
// result sits in lane l, register v at row (v/4)*8 + (l/32)*4 + v%4, col l%32.
//
// Epilogue.  The fp32 tile is staged in LDS (128 x 132 floats), then written
// out in the tile's orientation (pass A) and, where the product is needed
// transposed, in the mirrored orientation (pass B), both as 16-byte chunks.

constexpr int GT = MO_GEMM_TILE;           // 128
constexpr int G_THREADS = 256;
constexpr int KB = 128;                    // bytes of K per LDS stage and row
constexpr int OPND_BYTES = GT * KB;        // 16 KB per operand per stage
constexpr int MAIN_LDS = 4 * OPND_BYTES;   // 2 stages x 2 operands
constexpr int ST = GT + 4;                 // staging row stride (floats)
constexpr int EPI_LDS = GT * ST * 4;
constexpr int GEMM_LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;

enum { KIND_GRAM = 0, KIND_POLY = 1, KIND_UPDATE = 2 };

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static MO_DEV void run(const u32x4& a, const u32x4& b, f32x16& acc) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static MO_DEV void run(const u32x4& a, const u32x4& b, f32x16& acc) {
        const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
    }
};

MO_DEV int swz(int row, int chunk) { return row * KB + ((chunk ^ (row & 7)) << 4); }

// Block index -> logical item.  Consecutive workgroups are dealt round-robin
// over the 8 XCDs; giving each XCD a contiguous run of items keeps the tiles
// that share operand panels on the same L2.
MO_DEV uint32_t xcd_item(uint32_t b, uint32_t nb) {
    const uint32_t chunk = nb >> 3;
    return (b & 7) * chunk + (b >> 3);
}

template <typename T, int KIND>
__global__ __launch_bounds__(G_THREADS, 2) void gemm_kernel(uint8_t* ws, int first, int last,
                                                            int xt_cur) {
    __shared__ __align__(16) uint8_t smem[GEMM_LDS];
    const mo_wl_header* h = wl_header(ws);
    const uint32_t n_items = KIND == KIND_GRAM ? h->n_gram_items
                           : KIND == KIND_POLY ? h->n_poly_items : h->n_upd_items;
    const uint64_t items_off = KIND == KIND_GRAM ? h->gram_offset
                             : KIND == KIND_POLY ? h->poly_offset : h->upd_offset;
    const uint32_t logical = xcd_item(blockIdx.x, gridDim.x);
    if (logical >= n_items) return;
    const mo_wl_item it = reinterpret_cast<const mo_wl_item*>(ws + items_off)[logical];
    const mo_wl_mat& mt = wl_mats(ws)[it.mat];
    const int ti = it.ti, tj = it.tj;
    const int64_t m_pad = mt.m_pad, n_pad = mt.n_pad;

    T* X = reinterpret_cast<T*>(ws + mt.off_X);
    T* Xt_cur = reinterpret_cast<T*>(ws + (xt_cur ? mt.off_Xt1 : mt.off_Xt0));
    T* Xt_nxt = reinterpret_cast<T*>(ws + (xt_cur ? mt.off_Xt0 : mt.off_Xt1));
    T* A = reinterpret_cast<T*>(ws + mt.off_A);
    T* B = reinterpret_cast<T*>(ws + mt.off_B);
    const float* scale = reinterpret_cast<const float*>(ws + mt.off_scale);

    const T* P;
    const T* Q;
    int64_t ld;
    if (KIND == KIND_GRAM) {
        ld = n_pad; P = X + int64_t(ti) * GT * ld; Q = X + int64_t(tj) * GT * ld;
    } else if (KIND == KIND_POLY) {
        ld = m_pad; P = A + int64_t(ti) * GT * ld; Q = A + int64_t(tj) * GT * ld;
    } else {
        ld = m_pad; P = B + int64_t(ti) * GT * ld; Q = Xt_cur + int64_t(tj) * GT * ld;
    }
    const int64_t ldb = ld * int64_t(sizeof(T));             // row stride in bytes
    const int nk = int(ld * int64_t(sizeof(T)) / KB);         // K stages

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, kg = lane >> 5;

    const uint8_t* Pb = reinterpret_cast<const uint8_t*>(P);
    const uint8_t* Qb = reinterpret_cast<const uint8_t*>(Q);
    u32x4 rp[4], rq[4];
    auto gload = [&](int ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + G_THREADS * i;
            const int row = q >> 3, cc = q & 7;
            const int64_t off = int64_t(row) * ldb + int64_t(ks) * KB + cc * 16;
            rp[i] = *reinterpret_cast<const u32x4*>(Pb + off);
            rq[i] = *reinterpret_cast<const u32x4*>(Qb + off);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* sp = smem + buf * 2 * OPND_BYTES;
        uint8_t* sq = sp + OPND_BYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + G_THREADS * i;
            const int row = q >> 3, cc = q & 7;
            *reinterpret_cast<u32x4*>(sp + swz(row, cc)) = rp[i];
            *reinterpret_cast<u32x4*>(sq + swz(row, cc)) = rq[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    auto compute = [&](int cur) {
        const uint8_t* sp = smem + cur * 2 * OPND_BYTES;
        const uint8_t* sq = sp + OPND_BYTES;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int chunk = 2 * s + kg;
            u32x4 fa[2], fb[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                fa[a] = *reinterpret_cast<const u32x4*>(sp + swz(wm * 64 + a * 32 + r32, chunk));
#pragma unroll
            for (int b = 0; b < 2; ++b)
                fb[b] = *reinterpret_cast<const u32x4*>(sq + swz(wn * 64 + b * 32 + r32, chunk));
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) Mfma<T>::run(fa[a], fb[b], acc[a][b]);
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks + 1 < nk; ++ks) {
        gload(ks + 1);
        compute(ks & 1);
        lstore((ks & 1) ^ 1);
        __syncthreads();
    }
    compute((nk - 1) & 1);
    __syncthreads();

    // ---- stage the fp32 tile in LDS ----
    float* st = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * 64 + a * 32 + (v >> 2) * 8 + kg * 4 + (v & 3);
                const int col = wn * 64 + b * 32 + r32;
                st[row * ST + col] = acc[a][b][v];
            }
    __syncthreads();

    const float na = h->ns_a, nb = h->ns_b, nc = h->ns_c;
    const bool trans = mt.flags & MO_WLF_TRANSPOSED;
    const int64_t gi0 = int64_t(ti) * GT, gj0 = int64_t(tj) * GT;

    // ---- pass A: the tile in its own orientation ----
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {
        const int q = tid + G_THREADS * i;
        const int cc = q & 15, row = q >> 4;
        const int64_t gi = gi0 + row, gj = gj0 + cc * 8;
        f32x8 v;
        load8(st + row * ST + cc * 8, v);
        if (KIND == KIND_GRAM) {
            const float alpha = first ? scale[1] : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] *= alpha;
            store8(A + gi * m_pad + gj, v);
        } else if (KIND == KIND_POLY) {
            f32x8 av;
            load8(A + gi * m_pad + gj, av);
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] = nc * v.v[e] + nb * av.v[e];
            store8(B + gi * m_pad + gj, v);
        } else {
            const float sx = first ? scale[0] : 1.0f;
            f32x8 xv;
            load8(X + gi * n_pad + gj, xv);
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] = sx * (na * xv.v[e] + v.v[e]);
            if (!last) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v.v[e] = quantize<T>(v.v[e]);
                store8(X + gi * n_pad + gj, v);
                store8(st + row * ST + cc * 8, v);
            } else if (!trans) {
                // weight frame == NS frame: row gi, cols gj..gj+7
                if (gi < mt.rows) {
                    const bool wbf = mt.flags & MO_WLF_W_BF16;
                    void* W = reinterpret_cast<void*>(mt.W);
                    float* U = reinterpret_cast<float*>(mt.U);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (gj + e < mt.cols) {
                            const int64_t wi = gi * mt.ld_w + gj + e;
                            const float w = load_elem(W, wi, wbf);
                            store_elem(W, wi, mt.decay * w - mt.lr_eff * v.v[e], wbf);
                            if (U) U[gi * mt.ld_u + gj + e] = mt.lr_eff * v.v[e];
                        }
                    }
                }
            } else {
                store8(st + row * ST + cc * 8, v);
            }
        }
    }

    // ---- pass B: the mirrored orientation ----
    bool need_b;
    if (KIND == KIND_UPDATE) {
        need_b = !last || trans;
        __syncthreads();   // pass A rewrote the staging tile
    } else {
        need_b = ti != tj;
    }
    if (!need_b) return;
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {
        const int q = tid + G_THREADS * i;
        const int j = q & 127, rr = q >> 7;           // output row j, cols rr*8..rr*8+7
        f32x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v.v[e] = st[(rr * 8 + e) * ST + j];
        const int64_t oj = gj0 + j, oi = gi0 + rr * 8;
        if (KIND == KIND_GRAM) {
            const float alpha = first ? scale[1] : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] *= alpha;
            store8(A + oj * m_pad + oi, v);
        } else if (KIND == KIND_POLY) {
            f32x8 av;
            load8(A + oj * m_pad + oi, av);     // A is exactly symmetric
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] = nc * v.v[e] + nb * av.v[e];
            store8(B + oj * m_pad + oi, v);
        } else if (!last) {
            store8(Xt_nxt + oj * m_pad + oi, v);
        } else {
            // weight frame is the transpose: W row oj (< rows = n), cols oi.. (< cols = m)
            if (oj < mt.rows) {
                const bool wbf = mt.flags & MO_WLF_W_BF16;
                void* W = reinterpret_cast<void*>(mt.W);
                float* U = reinterpret_cast<float*>(mt.U);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (oi + e < mt.cols) {
                        const int64_t wi = oj * mt.ld_w + oi + e;
                        const float w = load_elem(W, wi, wbf);
                        store_elem(W, wi, mt.decay * w - mt.lr_eff * v.v[e], wbf);
                        if (U) U[oj * mt.ld_u + oi + e] = mt.lr_eff * v.v[e];
                    }
                }
            }
        }
    }
}

inline unsigned grid_for(uint32_t items) { return (items + 7u) / 8u * 8u; }

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

template <int KIND>
static hipError_t launch_gemm(const mo_wl_header& h, uint32_t items, uint8_t* ws, int first,
                              int last, int xt_cur, hipStream_t s) {
    if (items == 0) return hipSuccess;
    if (h.ns_dtype == MO_BF16)
        hipLaunchKernelGGL((gemm_kernel<bf16_t, KIND>), dim3(grid_for(items)), dim3(G_THREADS), 0, s,
                           ws, first, last, xt_cur);
    else
        hipLaunchKernelGGL((gemm_kernel<float, KIND>), dim3(grid_for(items)), dim3(G_THREADS), 0, s,
                           ws, first, last, xt_cur);
    return hipGetLastError();
}

hipError_t mo_launch_gram(const mo_wl_header& h, uint8_t* ws, int first, int xt_cur, hipStream_t s) {
    return launch_gemm<KIND_GRAM>(h, h.n_gram_items, ws, first, 0, xt_cur, s);
}
hipError_t mo_launch_poly(const mo_wl_header& h, uint8_t* ws, hipStream_t s) {
    return launch_gemm<KIND_POLY>(h, h.n_poly_items, ws, 0, 0, 0, s);
}
hipError_t mo_launch_update(const mo_wl_header& h, uint8_t* ws, int first, int last, int xt_cur,
                            hipStream_t s) {
    return launch_gemm<KIND_UPDATE>(h, h.n_upd_items, ws, first, last, xt_cur, s);
}
