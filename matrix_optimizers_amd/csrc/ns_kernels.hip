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
// Workgroup tile 256 x 256, 256 threads = 4 wavefronts in a 2 x 2 grid; each
// wavefront owns a 128 x 128 sub-tile = 4 x 4 MFMA blocks of 32 x 32 (256 fp32
// accumulators per lane, held in AGPRs).  Per K stage every operand row
// contributes 64 bytes (32 bf16 / 16 fp32): 2 x 256 rows x 64 B = 32 KB, in a
// ring of five stages in LDS (all 160 KB of the CU's LDS, one workgroup per
// CU).  Global data goes straight to LDS (global_load_lds_dwordx4, no VGPR
// round trip), two stages at a time, spread between the MFMAs (see the main
// loop below).
//
// A direct-to-LDS load writes lane l's 16 bytes at (wave base + 16 l), so each
// lane fetches the global chunk that belongs at its physical (swizzled) slot.
//
// MFMA operands.  bf16: v_mfma_f32_32x32x16_bf16 takes 8 consecutive k per
// lane; lane l supplies row (l % 32) and k-group (l / 32).  fp32:
// v_mfma_f32_32x32x2_f32 takes one k per lane; a 16-byte chunk of 4 floats feeds
// four of them.  A and B fragments use the same lane -> k assignment, so the
// sum over all k is exact regardless of how k is split among lanes.  The 32 x 32
// result sits in lane l, register v at row (v/4)*8 + (l/32)*4 + v%4, col l%32.
//
// Epilogue, per wavefront and per 32-row block of its sub-tile: the fp32
// values are staged by column in a private 16 KB LDS slice, then written out
// as 16-byte chunks in the mirrored orientation (pass B, where the transposed
// product is needed; it also forms the final values) and in the tile's own
// orientation (pass A: 16 lanes cover one 128-column row).

constexpr int GT = MO_GEMM_TILE;           // 256
constexpr int G_THREADS = 256;
constexpr int KB = 64;                     // bytes of K per LDS stage and row
constexpr int NSTAGE = 5;                  // LDS ring depth
constexpr int OPND_BYTES = GT * KB;        // 16 KB per operand per stage
constexpr int GEMM_LDS = NSTAGE * 2 * OPND_BYTES;  // 160 KB at full width, all of the CU's LDS

enum { KIND_GRAM = 0, KIND_POLY = 1, KIND_UPDATE = 2 };

typedef __attribute__((address_space(3))) void lds_void_t;

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

// 64-byte rows of four 16-byte chunks; logical chunk c of row r sits at
// c ^ ((r >> 2) & 3).  The LDS serves 16 lanes x 16 bytes per clock from 64
// banks; 16 consecutive rows read at one logical chunk then fall on 16
// distinct 16-byte bank groups (four rows per 256-byte bank line, each at a
// different chunk).
MO_DEV int swz(int row, int chunk) { return row * KB + ((chunk ^ ((row >> 2) & 3)) << 4); }

// Staging slice of one wave (16 KB): the fp32 results of one 32-row block of
// its 128 x 128 sub-tile, stored by column.  Value (column j, row i) sits in
// the 256-byte line j / 2, in 16-byte group G (rows i & ~3 .. + 3 of the
// column); G XORs the group's position in the line with bits of j so that
// the three access patterns (16-byte accumulator writes of 16 consecutive
// columns, 16-byte reads of 4 columns x 4 row groups, and 4-byte reads of 16
// columns 8 apart x 4 rows) each hit distinct banks.
MO_DEV int st_off(int j, int i) {
    const int p = j >> 1;
    const int g = ((j & 1) | ((i >> 2) << 1)) ^ (((p & 7) << 1) ^ ((p >> 3) & 7));
    return p * 256 + g * 16 + (i & 3) * 4;
}

// Epilogue context of one workgroup tile.  The mirrored pass ("pass B": for
// a sub-tile column j, 8 consecutive rows) runs first and forms the final
// values; the tile pass ("pass A": for a sub-tile row, 8 consecutive columns)
// writes them in the tile's own orientation.
template <typename T, int KIND, bool LAST>
struct Epi {
    const mo_wl_mat* mt;
    T *X, *Xt_nxt, *A, *B;
    float alpha, sx, na, nb, nc;
    int64_t m_pad, n_pad;
    bool trans;

    // Final values from the product v and the epilogue operand o (A[i][j] for
    // Poly, X[i][j] for Update; unused for Gram).
    MO_DEV void combine(f32x8& v, const f32x8& o) const {
        if (KIND == KIND_GRAM) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] *= alpha;
        } else if (KIND == KIND_POLY) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] = quantize<T>(nc * v.v[e] + nb * o.v[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v.v[e] = sx * (na * o.v[e] + v.v[e]);
            if (!LAST) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v.v[e] = quantize<T>(v.v[e]);
            }
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
        else if (!LAST) store8(X + gi * n_pad + gj, v);
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

// One 256 x TN tile, TN = 64 NB (NB = 4: the full 256 x 256 tile; 2 and 1:
// the half and quarter widths the host uses where full tiles would leave CUs
// idle).  Each wavefront owns 128 x (TN / 2) = 4 x NB blocks of 32 x 32.  A
// narrower tile accumulates every output element over the same K in the same
// order, so its results are bit-identical to the full tile's.
template <typename T, int KIND, bool LAST, int NB>
__device__ __forceinline__ void gemm_tile(uint8_t* smem, uint8_t* ws, const mo_wl_item& it, int first,
                                          int xt_cur) {
    constexpr int TN = 64 * NB;                  // tile columns = rows of Q
    constexpr int SBYTES = OPND_BYTES + TN * KB; // one stage: P (256 rows) then Q (TN rows)
    constexpr int LS = 4 + NB;                   // load instructions per stage and wave
    constexpr int LP = 2 * LS;                   // ... per pair of stages
    constexpr int MF = 4 * NB;                   // MFMA blocks per wave and substep
    constexpr int NR = 4 + NB;                   // fragment reads per substep
    const mo_wl_header* h = wl_header(ws);
    const mo_wl_mat& mt = wl_mats(ws)[it.mat];
    const int ti = int(it.ti), tj = int(it.tj);
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
        ld = n_pad; P = X + int64_t(ti) * GT * ld; Q = X + int64_t(tj) * TN * ld;
    } else if (KIND == KIND_POLY) {
        ld = m_pad; P = A + int64_t(ti) * GT * ld; Q = A + int64_t(tj) * TN * ld;
    } else {
        ld = m_pad; P = B + int64_t(ti) * GT * ld; Q = Xt_cur + int64_t(tj) * TN * ld;
    }
    const int64_t ldb = ld * int64_t(sizeof(T));             // row stride in bytes
    const int nk = int(ldb / KB);                              // K stages

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, kg = lane >> 5;

    // direct-to-LDS loads: wave w fills rows [64 w, 64 w + 64) of P and rows
    // [TN/4 w, TN/4 (w + 1)) of Q, 16 rows (1 KB) per instruction; lane l ->
    // row + l/4, physical chunk l%4.  The rows of one instruction start at a
    // wave-uniform address (SGPRs); the lane's part, the same for every
    // instruction since the swizzle depends on the row modulo 16 only, is one
    // 32-bit offset (16 rows of at most 32 MB).
    const uint8_t* Pb = reinterpret_cast<const uint8_t*>(P);
    const uint8_t* Qb = reinterpret_cast<const uint8_t*>(Q);
    const int lrow = lane >> 2, pch = lane & 3;
    const uint32_t voff = uint32_t(lrow) * uint32_t(ldb) + uint32_t((pch ^ ((lrow >> 2) & 3)) << 4);
    // Load instruction i (0 .. LS-1) of stage ks: P rows 64 wave + 16 i (i < 4),
    // else Q rows TN/4 wave + 16 (i - 4).
    auto issue1 = [&](int ks, int i) __attribute__((always_inline)) {
        uint8_t* sp = smem + (ks % NSTAGE) * SBYTES;
        const uint8_t* g;
        if (i < 4) {
            sp += (wave * 64 + i * 16) * KB;
            g = Pb + int64_t(wave * 64 + i * 16) * ldb;
        } else {
            sp += OPND_BYTES + (wave * (TN / 4) + (i - 4) * 16) * KB;
            g = Qb + int64_t(wave * (TN / 4) + (i - 4) * 16) * ldb;
        }
        __builtin_amdgcn_global_load_lds(g + int64_t(ks) * KB + voff, (lds_void_t*)sp, 16, 0, 0);
    };

    f32x16 acc[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    // Fragment i of one 16-deep K substep: A chunk i (i < 4) or B chunk i - 4.
    auto rd1 = [&](int ks, int sub, int i, u32x4 (&fa)[4], u32x4 (&fb)[NB]) __attribute__((always_inline)) {
        const uint8_t* sp = smem + (ks % NSTAGE) * SBYTES;
        const int chunk = 2 * sub + kg;
        if (i < 4) fa[i] = *reinterpret_cast<const u32x4*>(sp + swz(wm * 128 + i * 32 + r32, chunk));
        else fb[i - 4] = *reinterpret_cast<const u32x4*>(sp + OPND_BYTES + swz(wn * (TN / 2) + (i - 4) * 32 + r32, chunk));
    };
    // Workgroup barrier without the release fence of __syncthreads(), which
    // would also drain the direct-to-LDS loads still in flight for later
    // stages.  Each thread first waits for its own loads of the stage being
    // published (explicit vmcnt: the number of its load instructions issued
    // after that stage's last one) and for its LDS reads (lgkmcnt).
    auto wait_loads = [&](int after) {
        if (after == 17) asm volatile("s_waitcnt vmcnt(17)" ::: "memory");
        else if (after == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (after == 13) asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
        else if (after == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        else if (after == 11) asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
        else if (after == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        else if (after == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        else if (after == 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
        else if (after == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else if (after == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // lgkmcnt(0) through the builtin (gfx9 encoding: vmcnt and expcnt at their
    // maxima), so the compiler knows every fragment read has landed and adds
    // no wait of its own after the barrier.
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // The MF MFMAs of one substep on (fa, fb).  The NR fragment reads of the
    // next substep (stage rks, substep rsub, into na / nb) follow the first
    // MFMAs, one each (the surplus after the last when NR > MF).  When ia >= 0,
    // quarter q of the LP loads of the pair (ia, ia + 1) is spread evenly over
    // the MFMAs, load l being instruction l / 2 of stage ia + (l & 1).  The
    // order is fixed (sched_barrier), so reads and loads stream out between
    // the MFMAs instead of in bursts that would stall instruction issue behind
    // a full load queue.
    auto substep = [&](const u32x4 (&fa)[4], const u32x4 (&fb)[NB], bool do_read, int rks, int rsub,
                       u32x4 (&na)[4], u32x4 (&nb)[NB], int ia, int q) __attribute__((always_inline)) {
        const int l0 = q * LP / 4, nl = (q + 1) * LP / 4 - l0;
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            Mfma<T>::run(fa[i / NB], fb[i % NB], acc[i / NB][i % NB]);
            __builtin_amdgcn_sched_barrier(0);
            if (do_read) {
                if (i < NR) rd1(rks, rsub, i, na, nb);
                if (i == MF - 1)
#pragma unroll
                    for (int r = MF; r < NR; ++r) rd1(rks, rsub, r, na, nb);
            }
            if (ia >= 0)
#pragma unroll
                for (int j = 0; j < nl; ++j)
                    if ((j + 1) * MF / nl - 1 == i) {
                        const int l = l0 + j;
                        issue1(ia + (l & 1), l >> 1);
                    }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Software pipeline over K (nk >= 8 and even: every padded dimension is a
    // multiple of 256).  Stage s occupies ring slot s % NSTAGE.  Entering step
    // ks, F0 holds the fragments of (ks, substep 0).  The barrier sits between
    // the two substeps, so the MFMAs after it use fragments already in
    // registers while the reads for the next stage land.
    //
    // Stages are loaded in pairs (2p, 2p + 1), whose 64-byte row pieces are
    // the two halves of the same 128-byte lines, with the two stages'
    // instructions alternating so both halves of a line are requested back to
    // back.  The pair (ks + 4, ks + 5) goes into the slots of stages ks - 1 and
    // ks, which every wave has finished reading once the barrier of even step
    // ks has passed; its LP loads are spread in quarters over the four
    // substeps that follow (second of step ks, both of ks + 1, first of
    // ks + 2).  At the barrier of step ks, stage ks + 1 must have landed: for
    // even ks it is the second of its pair and all LP loads of the next pair
    // came after it; for odd ks it is the first of its pair, followed by one
    // load of its partner and the first half of the next pair.
    constexpr int W_EVEN = LP, W_ODD = 1 + LP / 2, W_FIRST = 1 + LP;
    u32x4 f0a[4], f0b[NB], f1a[4], f1b[NB];
#pragma unroll
    for (int p = 0; p < 4; p += 2)
#pragma unroll
        for (int l = 0; l < LP; ++l) issue1(p + (l & 1), l >> 1);
    wait_loads(W_FIRST);
    barrier();
#pragma unroll
    for (int i = 0; i < NR; ++i) rd1(0, 0, i, f0a, f0b);
    __builtin_amdgcn_sched_barrier(0);
    // Epilogue operand capture (bf16 Poly / Update).  The Q operand holds the
    // values the epilogue combines with the product: X[i][j] = X^T[j][i] for
    // Update, A[i][j] = A[j][i] for Poly.  K stage 8 ti + 4 wm + r covers rows
    // 32 r .. 32 r + 31 of this wave's sub-tile, so while that stage is in LDS
    // each lane copies the 2 NB chunks its mirrored-pass tasks of round r need
    // (task t: column j = lane / 4 + 16 t, rows 8 (lane % 4) .. + 7) into
    // registers, and the epilogue reads nothing from global memory.
    constexpr bool CAP = sizeof(T) == 2 && KIND != KIND_GRAM;
    constexpr int NT = 2 * NB;                           // epilogue tasks per lane and pass
    const int64_t gi_w = int64_t(ti) * GT + wm * 128;   // this wave's sub-tile origin
    const int64_t gj_w = int64_t(tj) * TN + wn * (TN / 2);
    u32x4 pre[CAP ? 4 : 1][NT];
    const int cap0 = ti * (GT * int(sizeof(T)) / KB) + wm * 4;
    auto capture = [&](int ks) __attribute__((always_inline)) {
        if constexpr (CAP) {
            const int r = ks - cap0;   // wave-uniform
            if (r >= 0 && r < 4) {
                // Register selects rather than pre[r][t] = ..., which would
                // index the array dynamically and move it to scratch memory.
                const uint8_t* sq = smem + (ks % NSTAGE) * SBYTES + OPND_BYTES;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const u32x4 c = *reinterpret_cast<const u32x4*>(
                        sq + swz(wn * (TN / 2) + (lane >> 2) + 16 * t, lane & 3));
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) pre[rr][t] = r == rr ? c : pre[rr][t];
                }
            }
        }
    };

    // (pa, qa): pair and quarter of loads issued in this step's first
    // substep; (pb, qb) in its second (pair -1: none).
    auto step = [&](int ks, int after, int pa, int qa, int pb, int qb) __attribute__((always_inline)) {
        substep(f0a, f0b, true, ks, 1, f1a, f1b, pa, qa);
        capture(ks);   // stage ks is still resident until the barrier below
        wait_loads(after);
        barrier();     // stage ks+1 visible everywhere; every read of stage ks done
        __builtin_amdgcn_sched_barrier(0);
        substep(f1a, f1b, true, ks + 1, 0, f0a, f0b, pb, qb);
    };
    // the prologue issued pairs (0, 1) and (2, 3) whole
    step(0, W_EVEN, -1, 0, 4, 0);
    step(1, W_ODD, 4, 1, 4, 2);
    int ks = 2;
    for (; ks + 6 <= nk; ks += 2) {
        step(ks, W_EVEN, ks + 2, 3, ks + 4, 0);
        step(ks + 1, W_ODD, ks + 4, 1, ks + 4, 2);
    }
    // ks == nk - 4: the last pair (nk - 2, nk - 1) lacks its last quarter
    step(ks, W_EVEN, ks + 2, 3, -1, 0);
    step(ks + 1, 1, -1, 0, -1, 0);
    step(ks + 2, 0, -1, 0, -1, 0);
    substep(f0a, f0b, true, nk - 1, 1, f1a, f1b, -1, 0);
    capture(nk - 1);
    substep(f1a, f1b, false, 0, 0, f0a, f0b, -1, 0);
    __syncthreads();   // every wave is done with the operand stages

    Epi<T, KIND, LAST> ep;
    ep.mt = &mt;
    ep.X = X; ep.Xt_nxt = Xt_nxt; ep.A = A; ep.B = B;
    ep.alpha = (KIND == KIND_GRAM && first) ? scale[1] : 1.0f;
    ep.sx = (KIND == KIND_UPDATE && first) ? scale[0] : 1.0f;
    ep.na = h->ns_a; ep.nb = h->ns_b; ep.nc = h->ns_c;
    ep.m_pad = m_pad; ep.n_pad = n_pad;
    ep.trans = mt.flags & MO_WLF_TRANSPOSED;
    {
        const int64_t wes = (mt.flags & MO_WLF_W_BF16) ? 2 : 4;
        ep.vec_w = ((mt.W | uint64_t(mt.ld_w * wes)) & 15) == 0;
        ep.vec_u = ((mt.U | uint64_t(mt.ld_u * 4)) & 15) == 0;
    }
    // Which passes write where.  Gram and Poly write the mirror of an
    // off-diagonal tile; Update writes X^T (or, last, W when the weight is the
    // transposed frame).  The tile pass writes everything except the last
    // Update of a transposed weight.  Gram scales in each pass; the other
    // kinds form their values in the mirrored pass and hand them to the tile
    // pass through the staging slice.
    const bool off_diag = ti != tj * TN / GT;
    const bool run_b = KIND == KIND_GRAM ? off_diag : true;
    const bool write_b = KIND == KIND_UPDATE ? (!LAST || ep.trans) : off_diag;
    const bool run_a = !(KIND == KIND_UPDATE && LAST && ep.trans);
    const bool hand_over = KIND != KIND_GRAM && run_a;

    uint8_t* st = smem + wave * (32 * (TN / 2) * 4);   // 32 rows x TN/2 columns of fp32
    // One 32-row block of the wave's sub-tile; called with literal indices so
    // the accumulator and capture arrays are never indexed dynamically.
    auto round = [&](const int a, const f32x16 (&ac)[NB], const u32x4 (&pf)[NT]) __attribute__((always_inline)) {
        // accumulators: lane holds column 32 b + lane % 32, rows 8 g + 4 (lane / 32) .. + 3
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v4 = {ac[b][4 * g], ac[b][4 * g + 1], ac[b][4 * g + 2], ac[b][4 * g + 3]};
                *reinterpret_cast<f32x4*>(st + st_off(b * 32 + r32, g * 8 + kg * 4)) = v4;
            }
        __builtin_amdgcn_wave_barrier();
        if (run_b) {
            // mirrored pass: column j of the sub-tile, rows 8 ic .. 8 ic + 7
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int j = (lane >> 2) + 16 * t, ic = lane & 3;
                f32x4* s0 = reinterpret_cast<f32x4*>(st + st_off(j, ic * 8));
                f32x4* s1 = reinterpret_cast<f32x4*>(st + st_off(j, ic * 8 + 4));
                const f32x4 lo = *s0, hi = *s1;
                f32x8 v, o;
#pragma unroll
                for (int e = 0; e < 4; ++e) { v.v[e] = lo[e]; v.v[4 + e] = hi[e]; }
                const int64_t oj = gj_w + j, oi = gi_w + a * 32 + ic * 8;
                if constexpr (CAP) {
                    const bf16x8 raw = __builtin_bit_cast(bf16x8, pf[t]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o.v[e] = (float)raw[e];
                } else if (KIND == KIND_POLY) {
                    load8(A + oj * m_pad + oi, o);          // A[i][j] = A[j][i]
                } else if (KIND == KIND_UPDATE) {
                    load8(Xt_cur + oj * m_pad + oi, o);     // X[i][j] = X^T[j][i]
                }
                ep.combine(v, o);
                if (write_b) ep.mirror(oj, oi, v);
                if (hand_over) {
                    *s0 = f32x4{v.v[0], v.v[1], v.v[2], v.v[3]};
                    *s1 = f32x4{v.v[4], v.v[5], v.v[6], v.v[7]};
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (run_a) {
            // tile pass: row of the sub-tile, columns 8 cc .. 8 cc + 7 (4 NB lanes per row)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int cc = lane % (4 * NB), row = lane / (4 * NB) + (16 / NB) * t;
                f32x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v.v[e] = *reinterpret_cast<const float*>(st + st_off(cc * 8 + e, row));
                if (KIND == KIND_GRAM) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v.v[e] *= ep.alpha;
                }
                ep.tile(gi_w + a * 32 + row, gj_w + cc * 8, v);
            }
            __builtin_amdgcn_wave_barrier();
        }
    };
    round(0, acc[0], pre[0]);
    round(1, acc[1], pre[CAP ? 1 : 0]);
    round(2, acc[2], pre[CAP ? 2 : 0]);
    round(3, acc[3], pre[CAP ? 3 : 0]);
}

inline unsigned grid_for(uint32_t items) { return items; }   // dispatch lists are padded to 8

// Entry b of the phase's dispatch list is workgroup b's tile; the tile width
// (NB) is uniform per workgroup.
template <typename T, int KIND, bool LAST>
__device__ __forceinline__ void gemm_entry(uint8_t* ws, int first, int xt_cur) {
    __shared__ __align__(16) uint8_t smem[GEMM_LDS];
    const mo_wl_header* h = wl_header(ws);
    const uint64_t items_off = KIND == KIND_GRAM ? h->gram_offset
                             : KIND == KIND_POLY ? h->poly_offset : h->upd_offset;
    const mo_wl_item it = reinterpret_cast<const mo_wl_item*>(ws + items_off)[blockIdx.x];
    if (it.mat == MO_WL_PAD) return;
    if (it.nb == 4) gemm_tile<T, KIND, LAST, 4>(smem, ws, it, first, xt_cur);
    else if (it.nb == 2) gemm_tile<T, KIND, LAST, 2>(smem, ws, it, first, xt_cur);
    else gemm_tile<T, KIND, LAST, 1>(smem, ws, it, first, xt_cur);
}

// One plainly named kernel per (phase, NS dtype), so profiles name them unambiguously.
#define MO_GEMM_KERNEL(name, T, KIND, LAST)                                               \
    __global__ __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))    \
    void name(uint8_t* ws, int first, int xt_cur) { gemm_entry<T, KIND, LAST>(ws, first, xt_cur); }
MO_GEMM_KERNEL(gram_bf16, bf16_t, KIND_GRAM, false)
MO_GEMM_KERNEL(gram_f32, float, KIND_GRAM, false)
MO_GEMM_KERNEL(poly_bf16, bf16_t, KIND_POLY, false)
MO_GEMM_KERNEL(poly_f32, float, KIND_POLY, false)
MO_GEMM_KERNEL(update_bf16, bf16_t, KIND_UPDATE, false)
MO_GEMM_KERNEL(update_f32, float, KIND_UPDATE, false)
MO_GEMM_KERNEL(update_last_bf16, bf16_t, KIND_UPDATE, true)
MO_GEMM_KERNEL(update_last_f32, float, KIND_UPDATE, true)
#undef MO_GEMM_KERNEL

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
    hipLaunchKernelGGL((h.ns_dtype == MO_BF16 ? bf : f32), dim3(grid_for(items)), dim3(G_THREADS), 0, s,
                       ws, first, xt_cur);
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
