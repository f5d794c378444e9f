// gfx950 kernels of the owner-side SOAP step.
//
// [P] = "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
// sharding", §5.7: the owner runs SOAP, Adam in the Shampoo eigenbasis, on the
// whole matrices it owns, with no collective.  Per matrix (the readings are
// stated with the C entry point):
//   L' = L + G G^T,  R' = R + G^T G                      fp32 statistics
//   Q_L, Q_R = eigenvectors of L', R', ascending          blocked Jacobi (fp64 A)
//   M' = b1 M + (1 - b1) G
//   G~ = Q_L^T G Q_R,  M~ = Q_L^T M' Q_R                  fp32 products
//   V' = b2 V + (1 - b2) G~^2
//   N = (M~ / (1 - b1^t)) / (sqrt(V' / (1 - b2^t)) + eps)
//   W' = (1 - lr wd) W - lr Q_L N Q_R^T
//
// Eigensolver.  Two-sided blocked Jacobi (the cyclic Jacobi method of Jacobi
// 1846 applied to blocks, with the round-robin ("circle") ordering of the
// parallel Jacobi literature): the padded side is cut into 2P blocks of 32;
// each round pairs all blocks, one workgroup diagonalises each 64 x 64 pair
// problem in LDS by scalar cyclic Jacobi sweeps, and a second launch applies
// the P pair rotations to A (both sides) and to the accumulated eigenvectors E.
// Every rotation is applied in Rutishauser's form (the new value is the old
// one plus a correction proportional to sin), and the pair rotations are kept
// as V - I, so rounding scales with the correction, not with the matrix.  The
// rotations and the rotated matrix A are fp64: an fp32 A builds up a backward
// error of a few hundred units over the rounds, which the eigenvectors of
// closely spaced eigenvalues turn into large angle errors.  The accumulated
// eigenvectors E are fp32 (their rounding does not feed back into A; see the
// E path).
#include "device_common.h"
#include "so_worklist.h"
#include "mo_kernels.h"

namespace {

typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int SO_THREADS = 256;
constexpr int SV_THREADS = 512;        // the pair solve: one slot of 2 x 2 blocks per thread
constexpr int GB = 64;                 // GEMM tile
constexpr int GK = 16;                 // GEMM K chunk
constexpr int PW = 2 * MO_SO_BLK;      // pair width (64)

MO_DEV const mo_so_header* so_header(const uint8_t* ws) {
    return reinterpret_cast<const mo_so_header*>(ws);
}
MO_DEV const mo_so_mat* so_mats(const uint8_t* ws) {
    return reinterpret_cast<const mo_so_mat*>(ws + so_header(ws)->mats_offset);
}
MO_DEV const mo_so_eig* so_eigs(const uint8_t* ws) {
    return reinterpret_cast<const mo_so_eig*>(ws + so_header(ws)->eigs_offset);
}

// What the sort's gather writes beside the sorted eigenvectors E32, and what a
// warm start requires before it uses them: a workspace that never held bases
// of a side of this size (fresh memory, or another bucket's side whose size
// pads to the same m_pad) does not hold this word, and such a step runs cold.
// Any orthonormal basis of the m-dimensional side would still give the right
// result, only by more sweeps; bases of a smaller side lack directions the
// polar step cannot restore, and uninitialised memory is no basis at all.
// Sides are at most 16384 (15 bits), so m_pad and m do not overlap.
static_assert(MO_SO_MAXSIDE < (1 << 15), "m_pad and m share the validity word");
MO_DEV uint32_t valid_word(const mo_so_eig& eg) { return MO_SO_MAGIC ^ (eg.m_pad | (eg.m << 16)); }
MO_DEV bool bases_valid(const uint8_t* ws, const mo_so_eig& eg) {
    return *reinterpret_cast<const uint32_t*>(ws + eg.off_valid) == valid_word(eg);
}

// Round k (0 .. n - 2) of the circle ordering over n (even) indices: pair j
// (0 .. n/2 - 1).  Index 0 stays put and the others turn one place per round,
// so that every pair meets exactly once in n - 1 rounds.
MO_DEV void circle_pair(int n, int k, int j, int& a, int& b) {
    auto f = [&](int i) { return (i + k) % (n - 1) + 1; };
    if (j == 0) {
        a = 0;
        b = f(0);
    } else {
        a = f(j);
        b = f(n - 1 - j);
    }
}

// The same index one step later in the pair solve's 64-index circle ordering:
// 1 .. 62 move up by one, 63 wraps to 1, and index 0, the first of pair 0,
// stays.  keep is PW - 1 for an index that moves and 0 for that fixed one,
// so the update is three integer operations with no compare.
static_assert(PW == 64, "the wrap below is PW = 64");
MO_DEV int advance_circle(int i, int keep = PW - 1) {
    const int x = i + 1;
    return (x & keep) | (x >> 6);
}

// ============================================================================
// prep: padded G and M' = b1 M + (1 - b1) G (the caller's M updated)
// ============================================================================
__global__ __launch_bounds__(SO_THREADS) void so_prep_kernel(uint8_t* ws, uint32_t mi) {
    const mo_so_mat& mt = so_mats(ws)[mi];
    const int64_t idx = int64_t(blockIdx.x) * SO_THREADS + threadIdx.x;
    const int64_t total = int64_t(mt.r_pad) * mt.c_pad;
    if (idx >= total) return;
    const int64_t i = idx / mt.c_pad, j = idx % mt.c_pad;
    float g = 0.f, m = 0.f;
    if (i < mt.rows && j < mt.cols) {
        g = load_elem(reinterpret_cast<const void*>(mt.G), i * mt.ld_g + j, mt.flags & MO_SOF_G_BF16);
        float* M = reinterpret_cast<float*>(mt.M);
        m = mt.beta1 * M[i * mt.ld_m + j] + (1.0f - mt.beta1) * g;
        M[i * mt.ld_m + j] = m;
    }
    reinterpret_cast<float*>(ws + mt.off_G)[idx] = g;
    reinterpret_cast<float*>(ws + mt.off_M)[idx] = m;
}

// ============================================================================
// fp32 products C = op(A) op(B) on 64 x 64 tiles, with the step's epilogues
// ============================================================================
//
// Operand element (i, k) of A sits at A[i * a_i + k * a_k], (k, j) of B at
// B[k * b_k + j * b_j]; one of each pair of strides is 1, and the loads run
// along it.  Every dimension is a multiple of 64 (zero padding), so no bounds
// are tested until the epilogue writes the caller's tensors.
struct SoProd {
    const float* A;
    int64_t a_i, a_k;
    const float* B;
    int64_t b_k, b_j;
    int K;
    int64_t a_lim = 0;   // > 0: A is the caller's unpadded a_lim x a_lim matrix (zero outside, any stride)
};

MO_DEV SoProd so_prod(uint8_t* ws, const mo_so_mat& mt, int kind) {
    const mo_so_eig* eigs = so_eigs(ws);
    auto F = [&](uint64_t off) { return reinterpret_cast<const float*>(ws + off); };
    const int64_t rp = mt.r_pad, cp = mt.c_pad;
    const float* EL = F(eigs[mt.eig_l].off_E32);
    const float* ER = F(eigs[mt.eig_r].off_E32);
    SoProd p;
    switch (kind) {
    case MO_SOK_STATS_L: p = {F(mt.off_G), cp, 1, F(mt.off_G), 1, cp, int(cp)}; break;
    case MO_SOK_STATS_R: p = {F(mt.off_G), 1, cp, F(mt.off_G), cp, 1, int(rp)}; break;
    case MO_SOK_LEFT_G:  p = {EL, rp, 1, F(mt.off_G), cp, 1, int(rp)}; break;
    case MO_SOK_LEFT_M:  p = {EL, rp, 1, F(mt.off_M), cp, 1, int(rp)}; break;
    case MO_SOK_RIGHT_G:
    case MO_SOK_RIGHT_M: p = {F(mt.off_T), cp, 1, ER, 1, cp, int(cp)}; break;
    case MO_SOK_BACK_L:  p = {EL, 1, rp, F(mt.off_N), cp, 1, int(rp)}; break;
    default:             p = {F(mt.off_T), cp, 1, ER, cp, 1, int(cp)}; break;   // BACK_R
    }
    return p;
}

// The epilogue of one row of four results: row i, columns j .. j + 3.
MO_DEV void so_epilogue(uint8_t* ws, const mo_so_mat& mt, int kind, int64_t i, int64_t j, float v) {
    const int64_t cp = mt.c_pad;
    if (kind == MO_SOK_STATS_L || kind == MO_SOK_STATS_R) {
        const mo_so_eig& eg = so_eigs(ws)[kind == MO_SOK_STATS_L ? mt.eig_l : mt.eig_r];
        float* ext = reinterpret_cast<float*>(eg.ext);
        double* A = reinterpret_cast<double*>(ws + eg.off_A);
        float s = 0.f;
        if (i < eg.m && j < eg.m) {
            s = ext[i * eg.ld_ext + j] + v;
            ext[i * eg.ld_ext + j] = s;
        }
        A[i * eg.m_pad + j] = double(s);
        return;
    }
    if (kind == MO_SOK_RIGHT_G) {
        if (i < mt.rows && j < mt.cols) {
            float& x = reinterpret_cast<float*>(mt.V)[i * mt.ld_v + j];
            x = mt.beta2 * x + (1.0f - mt.beta2) * v * v;
        }
        return;
    }
    if (kind == MO_SOK_RIGHT_M) {
        const float* V = reinterpret_cast<const float*>(mt.V);
        float n = 0.f;
        if (i < mt.rows && j < mt.cols) n = (v * mt.ibc1) / (sqrtf(V[i * mt.ld_v + j] * mt.ibc2) + mt.eps);
        reinterpret_cast<float*>(ws + mt.off_N)[i * cp + j] = n;
        return;
    }
    if (kind == MO_SOK_BACK_R) {
        if (i < mt.rows && j < mt.cols) {
            const bool wbf = mt.flags & MO_SOF_W_BF16;
            void* W = reinterpret_cast<void*>(mt.W);
            const int64_t wi = i * mt.ld_w + j;
            store_elem(W, wi, mt.decay * load_elem(W, wi, wbf) - mt.lr * v, wbf);
            if (mt.U) reinterpret_cast<float*>(mt.U)[i * mt.ld_u + j] = mt.lr * v;
        }
        return;
    }
    // LEFT_G, LEFT_M, BACK_L: the padded scratch product
    reinterpret_cast<float*>(ws + mt.off_T)[i * cp + j] = v;
}

// One 64 x 64 tile of C = op(A) op(B) with fp64 accumulation: K runs up to the
// long side (16384), where a sequential fp32 sum drops the small terms that
// follow a large partial sum, always the same way.  The fp32 operands are
// staged in LDS and widened (exactly) for v_mfma_f64_16x16x4_f64; each wave
// owns a 32 x 32 quarter as 2 x 2 blocks of 16 x 16 (the lane layout of the
// A path below).  ep(i, j, v) receives the fp64 sum of element (i, j).
template <class Ep>
MO_DEV void so_tile(const SoProd& p, int64_t i0, int64_t j0, float (*As)[GB + 4], float (*Bs)[GB + 4],
                    const Ep& ep) {
    const int t = threadIdx.x;
    const int l = t & 63, w = t >> 6;
    const int rw = 32 * (w >> 1), cw = 32 * (w & 1);   // this wave's 32 x 32 quarter of the tile
    f64x4 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
    for (int k0 = 0; k0 < p.K; k0 += GK) {
        if (p.a_lim > 0) {  // the caller's matrix: element loads, zero outside it
            const int i = t / 4, kk = (t % 4) * 4;
            const int64_t gi = i0 + i;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t gk = k0 + kk + e;
                As[kk + e][i] = (gi < p.a_lim && gk < p.a_lim) ? p.A[gi * p.a_i + gk] : 0.f;
            }
        } else if (p.a_k == 1) {   // 4 consecutive k of one row i
            const int i = t / 4, kk = (t % 4) * 4;
            const f32x4 a = *reinterpret_cast<const f32x4*>(p.A + (i0 + i) * p.a_i + k0 + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e) As[kk + e][i] = a[e];
        } else {            // 4 consecutive i of one k
            const int kk = t / 16, i = (t % 16) * 4;
            *reinterpret_cast<f32x4*>(&As[kk][i]) =
                *reinterpret_cast<const f32x4*>(p.A + (k0 + kk) * p.a_k + i0 + i);
        }
        if (p.b_j == 1) {   // 4 consecutive j of one k
            const int kk = t / 16, j = (t % 16) * 4;
            *reinterpret_cast<f32x4*>(&Bs[kk][j]) =
                *reinterpret_cast<const f32x4*>(p.B + (k0 + kk) * p.b_k + j0 + j);
        } else {            // 4 consecutive k of one column j
            const int j = t / 4, kk = (t % 4) * 4;
            const f32x4 b = *reinterpret_cast<const f32x4*>(p.B + (j0 + j) * p.b_j + k0 + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e) Bs[kk + e][j] = b[e];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GK; kk += 4) {   // lane l: A(l % 16, l / 16), B(l / 16, l % 16)
            double a[2], b[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) a[x] = double(As[kk + (l >> 4)][rw + 16 * x + (l & 15)]);
#pragma unroll
            for (int y = 0; y < 2; ++y) b[y] = double(Bs[kk + (l >> 4)][cw + 16 * y + (l & 15)]);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
        }
        __syncthreads();
    }
    // register v of block (x, y): row 16 x + l / 16 + 4 v, column 16 y + l % 16 of the quarter
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                ep(i0 + rw + 16 * x + (l >> 4) + 4 * v, j0 + cw + 16 * y + (l & 15), acc[x][y][v]);
}

__global__ __launch_bounds__(SO_THREADS) void so_gemm_kernel(uint8_t* ws, uint32_t mi, int kind) {
    __shared__ __align__(16) float As[GK][GB + 4];
    __shared__ __align__(16) float Bs[GK][GB + 4];
    const mo_so_mat& mt = so_mats(ws)[mi];
    so_tile(so_prod(ws, mt, kind), int64_t(blockIdx.y) * GB, int64_t(blockIdx.x) * GB, As, Bs,
            [&](int64_t i, int64_t j, double a) {
                so_epilogue(ws, mt, kind, i, j, float(a));   // each result is rounded to fp32 once
            });
}

// The products of a warm start (MO_SOW_*), one launch each per
// eigendecomposition ei, m_pad / 64 x m_pad / 64 tiles.  E32 holds the
// previous step's sorted eigenvectors as rows (zero below row m); the polar
// step E0 = E32 - (E32 E32^T - I) E32 / 2 makes them orthonormal again to
// fp32 rounding (its error is quadratic in their deviation, a few fp32 units
// after a step), so the deviations of successive steps do not add up; the
// difference Pm is formed in fp64 and kept, not the product, so that its few
// units survive the rounding.  A0 = E0 L' E0^T is then the new statistics in
// the previous basis, nearly diagonal, and E0 the sweeps' starting E.  T is
// rounded to fp32, so the two orientations of A0 differ by fp32 rounding;
// the sweeps need a symmetric matrix (the lower half of a diagonal block
// would otherwise carry that difference, far above the rotation threshold,
// from round to round), so each upper entry is written with its mirror.  The
// difference Pm is symmetric too (each entry and its mirror sum the same
// products in the same order), so for both only the upper tiles run.
__global__ __launch_bounds__(SO_THREADS) void so_warm_kernel(uint8_t* ws, uint32_t ei, int kind) {
    __shared__ __align__(16) float As[GK][GB + 4];
    __shared__ __align__(16) float Bs[GK][GB + 4];
    const mo_so_eig& eg = so_eigs(ws)[ei];
    if (!bases_valid(ws, eg)) return;   // no previous bases here: the step runs cold
    if ((kind == MO_SOW_P || kind == MO_SOW_A) && blockIdx.y > blockIdx.x) return;   // symmetric results
    const int64_t mp = eg.m_pad;
    float* E32 = reinterpret_cast<float*>(ws + eg.off_E32);
    float* E = reinterpret_cast<float*>(ws + eg.off_E);
    float* Pm = reinterpret_cast<float*>(ws + eg.off_A);   // the A region, before A0 replaces it
    double* A = reinterpret_cast<double*>(ws + eg.off_A);
    SoProd p;
    switch (kind) {
    case MO_SOW_P: p = {E32, mp, 1, E32, 1, mp, int(mp)}; break;
    case MO_SOW_E: p = {Pm, mp, 1, E32, mp, 1, int(mp)}; break;
    case MO_SOW_T: p = {reinterpret_cast<const float*>(eg.ext), eg.ld_ext, 1, E, 1, mp, int(mp), eg.m}; break;
    default:       p = {E, mp, 1, E32, mp, 1, int(mp)}; break;   // MO_SOW_A: E0 T (T in E32)
    }
    so_tile(p, int64_t(blockIdx.y) * GB, int64_t(blockIdx.x) * GB, As, Bs,
            [&](int64_t i, int64_t j, double v) {
                const int64_t o = i * mp + j;
                if (kind == MO_SOW_E) E[o] = float(double(E32[o]) - 0.5 * v);
                else if (kind == MO_SOW_T) E32[o] = float(v);
                else if (i > j) return;   // a symmetric result: the upper value and its mirror
                else if (kind == MO_SOW_P) {
                    const float d = float(v - ((i == j && i < eg.m) ? 1.0 : 0.0));
                    Pm[o] = d;
                    Pm[j * mp + i] = d;
                } else {
                    A[o] = v;
                    A[j * mp + i] = v;
                }
            });
}
// ============================================================================
// eigensolver
// ============================================================================

template <typename Rec>
MO_DEV uint32_t find_rec(const Rec* recs, uint32_t n, uint32_t item, uint32_t Rec::*begin) {
    uint32_t lo = 0, hi = n - 1;
    while (lo < hi) {   // last record whose first item is <= item
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (recs[mid].*begin <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Global index of local index l (0 .. 63) of pair (p, q) of 32-wide blocks.
MO_DEV int64_t pair_index(int p, int q, int l) {
    return l < MO_SO_BLK ? int64_t(p) * MO_SO_BLK + l : int64_t(q) * MO_SO_BLK + (l - MO_SO_BLK);
}

// E = identity on the true diagonal (padding stays zero), one thread per
// element, unless a warm start has put its E0 there.
__global__ __launch_bounds__(SO_THREADS) void so_eig_init_kernel(uint8_t* ws, uint32_t ei, int warm) {
    const mo_so_eig& eg = so_eigs(ws)[ei];
    const int64_t idx = int64_t(blockIdx.x) * SO_THREADS + threadIdx.x;
    if (idx < int64_t(eg.P)) reinterpret_cast<uint32_t*>(ws + eg.off_last)[idx] = 0u;   // final-sweep flags
    if ((warm && bases_valid(ws, eg)) || idx >= int64_t(eg.m_pad) * eg.m_pad)
        return;   // a warm start's E0 is in place
    const int64_t i = idx / eg.m_pad, j = idx % eg.m_pad;
    reinterpret_cast<float*>(ws + eg.off_E)[idx] = (i == j && i < eg.m) ? 1.f : 0.f;
}

// Per row of A (one workgroup each), its sum of squares; then, in the row
// order, ||A||_F and the rotation threshold thr = 2^-48 ||A||_F.  The rotations
// leave ||A||_F unchanged, and after convergence the off-diagonal entries sit
// at fp64 rounding of the whole matrix, a few units of 2^-53 ||A||; below thr
// an entry is left as it is.  Leaving it moves an eigenvector by at most
// thr / gap, far below what the fp32 statistics fix.
__global__ __launch_bounds__(SO_THREADS) void so_norm_rows_kernel(uint8_t* ws, uint32_t ei) {
    __shared__ double red[SO_THREADS];
    const mo_so_eig& eg = so_eigs(ws)[ei];
    const double* A = reinterpret_cast<const double*>(ws + eg.off_A) + int64_t(blockIdx.x) * eg.m_pad;
    double s = 0.0;
    for (uint32_t c = threadIdx.x; c < eg.m_pad; c += SO_THREADS) s += A[c] * A[c];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = SO_THREADS / 2; w > 0; w >>= 1) {
        if (int(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) reinterpret_cast<double*>(ws + eg.off_norm)[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(SO_THREADS) void so_norm_final_kernel(uint8_t* ws, uint32_t ei) {
    __shared__ double red[SO_THREADS];
    const mo_so_eig& eg = so_eigs(ws)[ei];
    double* nrm = reinterpret_cast<double*>(ws + eg.off_norm);
    double s = 0.0;
    for (uint32_t r = threadIdx.x; r < eg.m_pad; r += SO_THREADS) s += nrm[r];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = SO_THREADS / 2; w > 0; w >>= 1) {
        if (int(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) nrm[eg.m_pad] = 0x1p-48 * sqrt(red[0]);
}

// 1/x and 1/sqrt(x) for normal x > 0: the hardware estimate (relative error
// about 2^-24) refined by one third-order step, to within two or three units
// of fp64 rounding (not correctly rounded; the rotation below needs accuracy
// and consistency, not IEEE division, whose scaling and fix-up steps dominated
// the pair solve).  With e the estimate's residual, 1/x = y / (1 - e) and
// 1/sqrt(x) = y / sqrt(1 - e), each taken to its e^2 term: three dependent
// operations after the estimate for 1/x and four for 1/sqrt(x), against four
// and six for two Newton steps.
MO_DEV double rcp_nr(double x) {
    const double y = __builtin_amdgcn_rcp(x);
    const double e = fma(-x, y, 1.0);              // 1 - x y
    return fma(y, fma(e, e, e), y);                // y (1 + e + e^2)
}
MO_DEV double rsq_nr(double x) {
    const double y = __builtin_amdgcn_rsq(x);
    const double e = fma(-(x * y), y, 1.0);        // 1 - x y^2
    return fma(y * e, fma(0.375, e, 0.5), y);      // y (1 + e/2 + 3 e^2/8)
}

// Rotation that zeroes S[a][b] of the symmetric 2 x 2 problem (app, apq; apq, aqq):
// t = tan, s = sin, tau = sin / (1 + cos) (Rutishauser's formulas), the smaller
// of the two angles.  With d = aqq - app, e = 2 apq, r = hypot(d, e) and
// w = |d| + r: t = sign(d e) |e| / w (+1 at d = 0), and since
// 1 + t^2 = 2 r / w, one reciprocal square root q = 1 / sqrt(2 r w) gives
// cos = w q and sin = sign(d e) |e| q; tau = sign(d e) |e| / (w + sqrt(2 r w)),
// with sqrt(2 r w) = 2 r w q.  The chain from the pivot to tau is then about
// twenty dependent operations, which sets the pair solve's step time.
// The entries are statistics of fp32 data, at most about 1e81 in magnitude,
// and a rotated |apq| is above the threshold 2^-48 ||A||_F, so d^2 + e^2 and
// 2 r w (between 2 r^2 and 4 r^2) stay far from fp64 overflow and underflow.
// An off-diagonal entry at or below the threshold is left as it is (no
// rotation).  Returns whether it rotates.
MO_DEV bool jacobi_rotation(double app, double aqq, double apq, double thr, double& t, double& s,
                            double& tau) {
    if (fabs(apq) <= thr) {
        t = s = tau = 0.0;
        return false;
    }
    const double d = aqq - app, e = 2.0 * apq;
    const double se = d * e >= 0.0 ? fabs(e) : -fabs(e);
    const double x = fma(d, d, e * e);
    const double y = rsq_nr(x);
    const double r = x * y;                        // hypot(d, e)
    const double w = fma(x, y, fabs(d));
    const double p = (r + r) * w;                  // 2 r w = w^2 + e^2
    const double q = rsq_nr(p);
    t = se * rcp_nr(w);
    s = se * q;
    tau = se * rcp_nr(fma(p, q, w));
    return true;
}

// Entry (i, j) of a symmetric 64 x 64 matrix kept as its packed upper triangle
// (row i holds columns i .. 63; 2080 entries).
// Row a starts at a PW - a (a - 1) / 2 - a = a (2 PW - 1 - a) / 2 (an even
// product), so the byte offset of (i, j) is 4 a (2 PW - 1 - a) + 8 b.
MO_DEV int tri_off(int i, int j) {
    const int a = min(i, j), b = max(i, j);
    return int(__umul24(unsigned(a), unsigned(4 * (2 * PW - 1) - 4 * a))) + 8 * b;
}
MO_DEV int tri(int i, int j) { return tri_off(i, j) >> 3; }

// Slot of 2 x 2 blocks that thread t updates in a step (a bijection of
// 0 .. 511).  Slot s is the unordered pair {u, v} of the step's 32 rotations
// with u = s / 16, v = u + 1 + s % 16 (mod 32); the pairs 16 apart come up
// twice and the copy from the higher u is idle.  The circle ordering turns
// one place per step, so pair j of step k + 1 joins one element of each of
// two pairs of step k, the same two at every step: pairs j - 1 and j + 1 for
// 1 <= j <= 30, 0 and 1 for j = 0, 30 and 31 for j = 31.  The block of those
// two pairs holds the next pivot S[a'][b'], and slot solve_slot(j) of thread
// j (0 .. 31, all in wave 0) is that block; the 29 slots this displaces from
// threads 2 .. 31 go, in order, to the threads whose own slot was taken.
MO_DEV int solve_slot(int t) {
    if (t < PW / 2) return t == 0 ? 0 : t == PW / 2 - 1 ? 480 : 16 * (t - 1) + 1;
    if (t == 480) return 31;
    if ((t & 15) == 1 && t <= 465) {
        const int i = (t >> 4) - 2;
        return i <= 14 ? i + 2 : i + 3;
    }
    return t;
}

// One workgroup per (decomposition, block pair) of round k: diagonalise the
// 64 x 64 pair problem S = A[pair][pair] by one scalar cyclic sweep (63 steps
// of 32 disjoint rotations; none if it is already diagonal to the threshold)
// and store its rotation as D = V - I (V^T S V ~ diagonal), and whether it
// rotated at all.  S is kept as its packed upper triangle (17 KB; with D, three
// workgroups fit a CU) and is updated in place: in a step every entry is read
// and written by one thread only.  A step is one barrier: threads 0 .. 31
// update the blocks that hold the next step's pivots, apply the two diagonal
// updates each next pivot needs and compute the next step's rotations into the
// other parameter buffer, while the other threads update the other blocks and
// waves 1 .. 7 accumulate D with the current rotations.  Every rounding of the
// updates is written out as an fma, so the results do not depend on which
// contractions the compiler chooses.
__global__ __launch_bounds__(SV_THREADS) void so_jac_solve_kernel(uint8_t* ws, uint32_t k) {
    constexpr int NP = PW / 2;   // rotations per step
    __shared__ double S[PW * (PW + 1) / 2];
    __shared__ double D[PW][PW + 1];
    __shared__ double rs[2][NP], rtau[2][NP], rt[2][NP], rapq[2][NP];   // by step parity
    __shared__ int flags[2];   // [0] an off-diagonal entry above the threshold, [1] a rotation happened
    const mo_so_header* h = so_header(ws);
    const mo_so_eig* eigs = so_eigs(ws);
    const mo_so_eig& eg = eigs[find_rec(eigs, h->n_eigs, blockIdx.x, &mo_so_eig::solve_begin)];
    if (k >= eg.rounds) return;
    const int j = int(blockIdx.x - eg.solve_begin);
    const int nb = 2 * int(eg.P);
    int bp, bq;
    circle_pair(nb, int(k % uint32_t(nb - 1)), j, bp, bq);
    const double* A = reinterpret_cast<const double*>(ws + eg.off_A);
    const int64_t ld = eg.m_pad;
    const int t = threadIdx.x;
    // the four 32 x 32 blocks of the pair problem, each from where A keeps it
    // (upper blocks only: a lower block is the transpose of its mirror)
    static_assert(MO_SO_BLK * MO_SO_BLK / 2 == SV_THREADS, "one 16-byte piece per block and thread");
    f64x2 piece[4];
    const int pi = t / (MO_SO_BLK / 2), pj = 2 * (t % (MO_SO_BLK / 2));
#pragma unroll
    for (int b = 0; b < 4; ++b) {   // all four loads first
        const int x = (b >> 1) ? bq : bp, y = (b & 1) ? bq : bp;
        const double* src = x <= y ? A + int64_t(x) * MO_SO_BLK * ld + int64_t(y) * MO_SO_BLK
                                   : A + int64_t(y) * MO_SO_BLK * ld + int64_t(x) * MO_SO_BLK;
        piece[b] = *reinterpret_cast<const f64x2*>(src + pi * ld + pj);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (b == 2) continue;   // the lower off-diagonal block: the transpose of block 1
        const int ho = MO_SO_BLK * (b >> 1), vo = MO_SO_BLK * (b & 1);
        const int x = (b >> 1) ? bq : bp, y = (b & 1) ? bq : bp;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int r = x <= y ? ho + pi : ho + pj + e, c = x <= y ? vo + pj + e : vo + pi;
            if (r <= c) S[tri(r, c)] = piece[b][e];
        }
    }
    for (int q = t; q < PW * PW; q += SV_THREADS) D[q / PW][q % PW] = 0.0;
    if (t == 0) flags[0] = flags[1] = 0;
    __syncthreads();
    // Already diagonal to the rotation threshold (every off-diagonal entry at or
    // below it): no step would rotate, D stays zero.
    const double thr = reinterpret_cast<const double*>(ws + eg.off_norm)[eg.m_pad];
    for (int q = t; q < PW * PW; q += SV_THREADS) {
        const int r = q / PW, c = q % PW;
        if (r < c && fabs(S[tri(r, c)]) > thr) flags[0] = 1;
    }
    __syncthreads();
    if (flags[0]) {   // uniform
        // Pair j of step k is circle_pair(PW, k, j).  From one step to the next
        // every index but 0 moves one place along 1 .. 63, so the indices a
        // thread needs are kept in registers and advanced (no LDS round trip
        // before a step's loads).
        const int sl = solve_slot(t);
        const int u = sl >> 4, dv = sl & 15, v = (u + 1 + dv) & 31;
        const bool on = dv != 15 || u < 16;
        int au, bu, av, bv;
        circle_pair(PW, 0, u, au, bu);
        circle_pair(PW, 0, v, av, bv);
        // S by byte offset (tri_off), and the keep masks of advance_circle: the
        // first index of pair 0 is the one that never moves
        auto Sb = [&](int off) -> double& { return *reinterpret_cast<double*>(reinterpret_cast<uint8_t*>(S) + off); };
        const int keep_u = u == 0 ? 0 : PW - 1, keep_v = v == 0 ? 0 : PW - 1;
        // D items of threads 64 .. 511: pair w in rows r0 + 14 i (the stride
        // 448 of the items is a multiple of 32, so every item has the same pair)
        constexpr int NT = SV_THREADS - 64, NR = (PW * NP + NT - 1) / NT;
        static_assert(NT % NP == 0, "one pair per D thread");
        const int w = (t - 64) & (NP - 1), r0 = (t - 64) >> 5;
        int aw, bw;
        circle_pair(PW, 0, w, aw, bw);
        const int keep_w = w == 0 ? 0 : PW - 1, keep_t = t == 0 ? 0 : PW - 1;
        // rotation t of the current step (threads 0 .. 31 compute it a step ahead)
        int at = 0, bt = 0;
        bool rot_t = false;
        if (t < NP) {   // the rotations of step 0
            circle_pair(PW, 0, t, at, bt);
            double tt, s, tau;
            const double apq = S[tri(at, bt)];
            rot_t = jacobi_rotation(S[tri(at, at)], S[tri(bt, bt)], apq, thr, tt, s, tau);
            if (rot_t) flags[1] = 1;
            rs[0][t] = s; rtau[0][t] = tau; rt[0][t] = tt; rapq[0][t] = apq;
        }
        __syncthreads();
        for (int step = 0; step < PW - 1; ++step) {
            const int cur = step & 1, nxt = cur ^ 1;
            // Two-sided update of this thread's off-diagonal 2 x 2 block (rows
            // a_u, b_u by J_u^T, then columns a_v, b_v by J_v, each in
            // Rutishauser's form), loads issued before the arithmetic.
            const int i00 = tri_off(au, av), i01 = tri_off(au, bv), i10 = tri_off(bu, av), i11 = tri_off(bu, bv);
            const double x00 = Sb(i00), x01 = Sb(i01), x10 = Sb(i10), x11 = Sb(i11);
            const double su = rs[cur][u], tu = rtau[cur][u], sv = rs[cur][v], tv = rtau[cur][v];
            // Threads 0 .. 31 also load, with the block, what the next pivot needs:
            // its two diagonal entries (written by no other thread in this step)
            // and the tan and pivot of this block's two rotations.  Pair t of the
            // next step is (a2, b2).
            const int a2 = advance_circle(at, keep_t), b2 = advance_circle(bt);
            double da = 0.0, db = 0.0, tU = 0.0, pU = 0.0, tV = 0.0, pV = 0.0;
            if (t < NP) {
                da = Sb(tri_off(a2, a2));
                db = Sb(tri_off(b2, b2));
                tU = rt[cur][u]; pU = rapq[cur][u]; tV = rt[cur][v]; pV = rapq[cur][v];
            }
            const double y00 = fma(-su, fma(tu, x00, x10), x00), y10 = fma(su, fma(-tu, x10, x00), x10);
            const double y01 = fma(-su, fma(tu, x01, x11), x01), y11 = fma(su, fma(-tu, x11, x01), x11);
            const double z00 = fma(-sv, fma(tv, y00, y01), y00), z01 = fma(sv, fma(-tv, y01, y00), y01);
            const double z10 = fma(-sv, fma(tv, y10, y11), y10), z11 = fma(sv, fma(-tv, y11, y10), y11);
            if (on) {
                Sb(i00) = z00; Sb(i01) = z01; Sb(i10) = z10; Sb(i11) = z11;
            }
            if (t < NP) {
                // Rotation t of this step is done: its pivot becomes zero (the
                // diagonal updates are applied below, by the thread whose next
                // pivot needs them).
                if (rot_t) Sb(tri_off(at, bt)) = 0.0;
                // Pair t of the next step: a' from one of this block's pairs,
                // b' from the other; every diagonal entry is in exactly one of
                // them, so every diagonal update is applied once.
                const bool a_in_u = a2 == au || a2 == bu;
                const int xa = a_in_u ? a2 : b2, ya = a_in_u ? b2 : a2;   // row of the block, column
                const double apq2 = xa == au ? (ya == av ? z00 : z01) : (ya == av ? z10 : z11);
                const double s_a = a_in_u ? su : sv, t_a = a_in_u ? tU : tV, p_a = a_in_u ? pU : pV;
                const double s_b = a_in_u ? sv : su, t_b = a_in_u ? tV : tU, p_b = a_in_u ? pV : pU;
                const int first_a = a_in_u ? au : av, first_b = a_in_u ? av : au;
                // the first index of a rotation loses t apq, the second gains it
                const double app2 = s_a != 0.0 ? fma(a2 == first_a ? -t_a : t_a, p_a, da) : da;
                const double aqq2 = s_b != 0.0 ? fma(b2 == first_b ? -t_b : t_b, p_b, db) : db;
                Sb(tri_off(a2, a2)) = app2;
                Sb(tri_off(b2, b2)) = aqq2;
                double tt, s, tau;
                rot_t = jacobi_rotation(app2, aqq2, apq2, thr, tt, s, tau) && step + 1 < PW - 1;
                if (rot_t) flags[1] = 1;
                rs[nxt][t] = s; rtau[nxt][t] = tau; rt[nxt][t] = tt; rapq[nxt][t] = apq2;
            } else if (t >= 64) {
                // D <- D J + (J - I) on waves 1 .. 7: item i is row r0 + 14 i of pair w.
                const double s2 = rs[cur][w], tau = rtau[cur][w];
                double dA[NR], dB[NR];
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    const int r = r0 + (NT / NP) * i;
                    if (r < PW) { dA[i] = D[r][aw]; dB[i] = D[r][bw]; }
                }
                // With V = I + D, entry (r, a) of V J - I is
                // D[r][a] - s (V[r][b] + tau V[r][a]) and entry (r, b) is
                // D[r][b] + s (V[r][a] - tau V[r][b]): the rotation's products
                // take V's entries (D plus 1 in rows a and b), the sums keep D.
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    const int r = r0 + (NT / NP) * i;
                    if (r >= PW) break;
                    const double va = dA[i] + (r == aw ? 1.0 : 0.0), vb = dB[i] + (r == bw ? 1.0 : 0.0);
                    D[r][aw] = fma(-s2, fma(tau, va, vb), dA[i]);
                    D[r][bw] = fma(s2, fma(-tau, vb, va), dB[i]);
                }
            }
            at = a2; bt = b2;
            au = advance_circle(au, keep_u); bu = advance_circle(bu);
            av = advance_circle(av, keep_v); bv = advance_circle(bv);
            aw = advance_circle(aw, keep_w); bw = advance_circle(bw);
            __syncthreads();
        }
    }
    const bool any = flags[1];   // read after the last barrier
    // D of a pair that did not rotate is zero and is never read (its A and E
    // products are skipped on the flag word), so it is not stored.
    double* Dout = reinterpret_cast<double*>(ws + eg.off_D) + int64_t(j) * PW * PW;
    if (any)
        for (int q = t; q < PW * PW / 2; q += SV_THREADS) {
            const int r = q / (PW / 2), c = 2 * (q % (PW / 2));
            *reinterpret_cast<f64x2*>(Dout + r * PW + c) = f64x2{D[r][c], D[r][c + 1]};
        }
    if (t == 0) reinterpret_cast<uint32_t*>(ws + eg.off_flag)[j] = any ? 1u : 0u;
    // rounds of the final sweep: mark this pair slot if its problem rotated
    if (t == 0 && any && k + uint32_t(nb - 1) >= eg.rounds)
        reinterpret_cast<uint32_t*>(ws + eg.off_last)[j] = 1u;
}

// The A path's products on fp64 MFMA (v_mfma_f64_16x16x4_f64): wave w owns
// rows 32 (w / 2) .. + 31 and columns 32 (w % 2) .. + 31 of the 64 x 64 tile
// as 2 x 2 blocks of 16 x 16, over 16 k-steps of 4.  Per instruction, lane l
// supplies A(l % 16, l / 16) and B(l / 16, l % 16) and holds results
// (l / 16 + 4 v, l % 16) in its registers v = 0..3 (the layout read off the
// instruction with one-hot operands).  Tile row and column of result register
// v of block (x, y) in this lane:
MO_DEV int mfma_row(int x, int v) { return 32 * (threadIdx.x >> 7) + 16 * x + ((threadIdx.x & 63) >> 4) + 4 * v; }
MO_DEV int mfma_col(int y) { return 32 * ((threadIdx.x >> 6) & 1) + 16 * y + (threadIdx.x & 15); }

// One workgroup per upper 64 x 64 tile (I, J) of pairs of A in round k:
// A' = V_I^T A V_J.  With V = I + D: C = X + X D_J, A' = C + D_I^T C.  A tile
// whose two pairs were not rotated is left untouched (the products would add
// exact zeros).  A is symmetric, and the rounds keep only its upper 32 x 32
// blocks (x <= y; a lower block is the transpose of its mirror), so each
// block of the tile is read once and written once, in whichever orientation
// A keeps it.  One 64 x 65 fp64 buffer in LDS (33 KB, so several workgroups
// share a CU) holds X^T, then C, then the result; D_J and D_I come straight
// from the round's rotations (L2).
MO_DEV void apply_a_tile(uint8_t* ws, uint32_t k, uint32_t blk, double (*C)[PW + 1]) {
    const mo_so_header* h = so_header(ws);
    const mo_so_eig* eigs = so_eigs(ws);
    const mo_so_eig& eg = eigs[find_rec(eigs, h->n_eigs, blk, &mo_so_eig::apply_begin)];
    if (k >= eg.rounds) return;
    const int P = int(eg.P);
    const int nb = 2 * P;
    const int kr = int(k % uint32_t(nb - 1));
    int item = int(blk - eg.apply_begin);
    int I = 0;
    while (item >= P - I) { item -= P - I; ++I; }
    const int J = I + item;
    const uint32_t* flag = reinterpret_cast<const uint32_t*>(ws + eg.off_flag);
    // A pair that did not rotate has D = 0 (not stored): its product would add
    // exact zeros and is skipped (both: the tile stays as it is).
    const bool rot_I = flag[I] != 0, rot_J = flag[J] != 0;
    if (!rot_I && !rot_J) return;
    int pI, qI, pJ, qJ;
    circle_pair(nb, kr, I, pI, qI);
    circle_pair(nb, kr, J, pJ, qJ);
    const double* Dall = reinterpret_cast<const double*>(ws + eg.off_D);
    const double* DI = Dall + int64_t(I) * PW * PW;
    const double* DJ = Dall + int64_t(J) * PW * PW;
    double* M = reinterpret_cast<double*>(ws + eg.off_A);
    const int64_t ld = eg.m_pad;
    const int t = threadIdx.x;
    const int l = t & 63, w = t >> 6;
    const int r0 = 32 * (w >> 1) + (l & 15), c0 = 32 * (w & 1) + (l & 15);
    // X^T (rows of pair J, columns of pair I) staged in the buffer, block by
    // block of 32 x 32: block (x, y) of X is kept by A as itself when x < y,
    // which is transposed into the buffer, and as the rows of its transpose
    // (y, x) otherwise (on a diagonal tile, the diagonal blocks as stored).
    // The buffer then takes C.
    // All eight loads of the thread are issued before the first LDS write;
    // they are non-temporal, as each block is read once per round here
    // (rotation launches 0.9 % faster on the decoder bucket).
    constexpr int SQ = MO_SO_BLK * MO_SO_BLK / 2 / SO_THREADS;   // 16-byte pieces per block and thread
    f64x2 stage[4][SQ];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int x = (b >> 1) ? qI : pI, y = (b & 1) ? qJ : pJ;
        const double* src = x < y ? M + int64_t(x) * MO_SO_BLK * ld + int64_t(y) * MO_SO_BLK
                                  : M + int64_t(y) * MO_SO_BLK * ld + int64_t(x) * MO_SO_BLK;
#pragma unroll
        for (int u = 0; u < SQ; ++u) {
            const int q = t + u * SO_THREADS;
            const int i = q / (MO_SO_BLK / 2), j = 2 * (q % (MO_SO_BLK / 2));
            stage[b][u] = __builtin_nontemporal_load(reinterpret_cast<const f64x2*>(src + i * ld + j));
        }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int ro = MO_SO_BLK * (b >> 1), co = MO_SO_BLK * (b & 1);
        const int x = (b >> 1) ? qI : pI, y = (b & 1) ? qJ : pJ;
#pragma unroll
        for (int u = 0; u < SQ; ++u) {
            const int q = t + u * SO_THREADS;
            const int i = q / (MO_SO_BLK / 2), j = 2 * (q % (MO_SO_BLK / 2));
            if (x < y) {
                C[co + j][ro + i] = stage[b][u][0];
                C[co + j + 1][ro + i] = stage[b][u][1];
            } else {
                C[co + i][ro + j] = stage[b][u][0];
                C[co + i][ro + j + 1] = stage[b][u][1];
            }
        }
    }
    __syncthreads();
    f64x4 acc[2][2];
    double own[2][2][4];
    if (rot_J) {   // uniform
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int k0 = 0; k0 < PW; k0 += 4) {   // X D_J
            const int kq = k0 + (l >> 4);
            double a[2], b[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) a[x] = C[kq][r0 + 16 * x];   // X[r][kq] = X^T[kq][r]
#pragma unroll
            for (int y = 0; y < 2; ++y) b[y] = DJ[kq * PW + c0 + 16 * y];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int v = 0; v < 4; ++v) own[x][y][v] = C[mfma_col(y)][mfma_row(x, v)] + acc[x][y][v];
        __syncthreads();                          // X^T fully read: C replaces it
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int v = 0; v < 4; ++v) C[mfma_row(x, v)][mfma_col(y)] = own[x][y][v];
        __syncthreads();
    }
    // C is in the buffer by rows, or (D_J = 0) C = X is still there as X^T,
    // read transposed below.
    if (rot_I) {   // uniform
        const bool ct = !rot_J;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int k0 = 0; k0 < PW; k0 += 4) {   // D_I^T C
            const int kq = k0 + (l >> 4);
            double a[2], b[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) a[x] = DI[kq * PW + r0 + 16 * x];
#pragma unroll
            for (int y = 0; y < 2; ++y) b[y] = ct ? C[c0 + 16 * y][kq] : C[kq][c0 + 16 * y];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    own[x][y][v] = (ct ? C[mfma_col(y)][mfma_row(x, v)] : C[mfma_row(x, v)][mfma_col(y)]) + acc[x][y][v];
        __syncthreads();                          // C fully read: the result replaces it
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int v = 0; v < 4; ++v) C[mfma_row(x, v)][mfma_col(y)] = own[x][y][v];
        __syncthreads();
    }
    // each block of the result goes to where A keeps it: an upper block by
    // rows, a lower one as its transpose; on a diagonal tile the lower one of
    // the two off-diagonal blocks is the mirror of the other and is not written.
    // The stores are non-temporal: the next round reads these blocks from other
    // XCDs, and out of L2 they leave it to D and the E lines (the rotation
    // launches 1.2 % faster on the decoder bucket, results bit-identical).
    for (int b = 0; b < 4; ++b) {
        const int ro = MO_SO_BLK * (b >> 1), co = MO_SO_BLK * (b & 1);
        const int x = (b >> 1) ? qI : pI, y = (b & 1) ? qJ : pJ;
        if (x <= y) {
            double* dst = M + int64_t(x) * MO_SO_BLK * ld + int64_t(y) * MO_SO_BLK;
            for (int q = t; q < MO_SO_BLK * MO_SO_BLK / 2; q += SO_THREADS) {
                const int i = q / (MO_SO_BLK / 2), j = 2 * (q % (MO_SO_BLK / 2));
                __builtin_nontemporal_store(f64x2{C[ro + i][co + j], C[ro + i][co + j + 1]},
                                            reinterpret_cast<f64x2*>(dst + i * ld + j));
            }
        } else if (I != J) {
            double* dst = M + int64_t(y) * MO_SO_BLK * ld + int64_t(x) * MO_SO_BLK;
            for (int q = t; q < MO_SO_BLK * MO_SO_BLK / 2; q += SO_THREADS) {
                const int i = q / (MO_SO_BLK / 2), j = 2 * (q % (MO_SO_BLK / 2));
                __builtin_nontemporal_store(f64x2{C[ro + j][co + i], C[ro + j + 1][co + i]},
                                            reinterpret_cast<f64x2*>(dst + i * ld + j));
            }
        }
    }
}

// One workgroup per pair I and MO_SO_ECOLS consecutive 64-column tiles of the
// accumulated eigenvectors E in round k: E' = V_I^T E = X + D_I^T X, in fp32
// (E is kept in fp32 between rounds; D_I is rounded to fp32 for the product
// on v_mfma_f32_16x16x4f32, at twice the fp64 rate).  Each round's rounding
// moves an eigenvector by about an fp32 unit, a random walk of a few 1e-6
// over the longest solves, and none of it feeds back into A, whose rounding
// is what the eigenvectors of close eigenvalues amplify; the rotations
// themselves stay fp64.  D_I sits in LDS (fp32, rows
// padded to ED floats so that the four row groups of a read fall in separate
// banks; loaded once for the workgroup's tiles).  Each wave takes whole
// strips of 64 rows x 32 columns, so no wave reads what another writes and
// the strips need no barrier.  A lane holds two adjacent columns of a row (one
// 8-byte access; 16 lanes cover a 128-byte line) and runs two column sets of
// products with each D_I value it reads.  In this instruction lane l holds
// result row 4 (l / 16) + v of a 16 x 16 block in register v (read off the
// instruction with one-hot operands), so the sum over the pair's 64 rows is
// taken in the order k-step kk, lane group g -> pair row 16 (kk / 4) + 4 g +
// kk % 4: the B operand a lane loads at k-step 4 x + v is then the old value
// of its result register v of block x, kept instead of read again.  Unrotated
// pairs are skipped.
constexpr int ED = PW + 4;   // LDS row of D_I in the E path (floats)

MO_DEV void apply_e_tile(uint8_t* ws, uint32_t k, uint32_t blk, float (*DI)[ED]) {
    const mo_so_header* h = so_header(ws);
    const mo_so_eig* eigs = so_eigs(ws);
    const mo_so_eig& eg = eigs[find_rec(eigs, h->n_eigs, blk, &mo_so_eig::etile_begin)];
    if (k >= eg.rounds) return;
    const int P = int(eg.P);
    const int nb = 2 * P;
    const int kr = int(k % uint32_t(nb - 1));
    const int item = int(blk - eg.etile_begin);
    const int ngrp = (P + int(MO_SO_ECOLS) - 1) / int(MO_SO_ECOLS);
    const int I = item / ngrp, cc0 = (item % ngrp) * int(MO_SO_ECOLS);
    if (!reinterpret_cast<const uint32_t*>(ws + eg.off_flag)[I]) return;
    int pI, qI;
    circle_pair(nb, kr, I, pI, qI);
    const int64_t ld = eg.m_pad;
    {
        const f64x2* src = reinterpret_cast<const f64x2*>(reinterpret_cast<const double*>(ws + eg.off_D) +
                                                          int64_t(I) * PW * PW);
        for (int q = threadIdx.x; q < PW * PW / 2; q += SO_THREADS) {
            const f64x2 v = src[q];
            const int r = q / (PW / 2), c = 2 * (q % (PW / 2));
            DI[r][c] = float(v[0]);
            DI[r][c + 1] = float(v[1]);
        }
    }
    __syncthreads();
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = l >> 4;
    const int nstrip = 2 * min(int(MO_SO_ECOLS), P - cc0);
    // Row 4 g of block p and of block q, the lane's two columns of the strip;
    // k-step kk then reads block row 16 ((kk / 4) % 2) + kk % 4 further on, of
    // block p for kk < 8 and of block q after.  Byte offsets from the E region
    // (at most 16384^2 x 4 bytes = 2^30), so each access takes the region's
    // uniform base plus one 32-bit lane offset.
    uint8_t* Eb = ws + eg.off_E;
    const uint32_t ldb = uint32_t(ld) * 4u;
    const uint32_t op = (uint32_t(pI) * MO_SO_BLK + 4u * g) * ldb + uint32_t(cc0) * PW * 4u + 8u * (l & 15);
    const uint32_t oq = (uint32_t(qI) * MO_SO_BLK + 4u * g) * ldb + uint32_t(cc0) * PW * 4u + 8u * (l & 15);
    auto at = [&](int kk, int st) -> f32x2* {   // k-step kk's row (or register v = kk % 4 of block kk / 4)
        return reinterpret_cast<f32x2*>(Eb + ((kk < 8 ? op : oq) + uint32_t(16 * ((kk >> 2) & 1) + (kk & 3)) * ldb +
                                              uint32_t(st) * 128u));
    };
    f32x2 cur[16];
#pragma unroll 1
    for (int st = w; st < nstrip; st += 4) {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) cur[kk] = *at(kk, st);
        f32x4 acc[4][2];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int h = 0; h < 2; ++h) acc[x][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int kq = 16 * (kk >> 2) + 4 * g + (kk & 3);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float d = DI[kq][16 * x + (l & 15)];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[x][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(d, cur[kk][h], acc[x][h], 0, 0, 0);
            }
            // this k-step's D_I reads stay with its products: hoisted over the
            // whole strip they would take 64 more registers and spill
            __builtin_amdgcn_sched_barrier(0);
        }
        // block x, register v: pair row 16 x + 4 g + v, loaded at k-step 4 x + v
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                *at(4 * x + v, st) = f32x2{cur[4 * x + v][0] + acc[x][0][v], cur[4 * x + v][1] + acc[x][1][v]};
    }
}

// All rotations of round k in one launch: the upper tiles of A and the E
// items, interleaved in block order in proportion to their counts, so that
// the fp64-MFMA-heavy A tiles and the memory-heavy E items share the CUs.
// The A path keeps one 64 x 64 fp64 tile in LDS (33 KB: four workgroups per
// CU), the E path an fp32 pair rotation (17 KB), and the registers are held
// to four waves per SIMD to match.
__global__ __launch_bounds__(SO_THREADS) __attribute__((amdgpu_waves_per_eu(4)))
void so_jac_rotate_kernel(uint8_t* ws, uint32_t k) {
    __shared__ __align__(16) double buf[PW * (PW + 1)];
    const mo_so_header* h = so_header(ws);
    const uint64_t ne = h->n_etile_items, tot = uint64_t(h->n_apply_items) + ne;
    const uint64_t b = blockIdx.x;
    const uint64_t e0 = b * ne / tot, e1 = (b + 1) * ne / tot;
    if (e1 > e0) apply_e_tile(ws, k, uint32_t(e0), reinterpret_cast<float (*)[ED]>(buf));
    else apply_a_tile(ws, k, uint32_t(b - e0), reinterpret_cast<double (*)[PW + 1]>(buf));
}

// The eigenvalues in ascending order, as a permutation: lam[i] = A[i][i] for
// i < m, +inf for padding (and for a NaN, which has no order), then the rank
// of each, counting the smaller keys and, among equal keys, the lower
// indices.  The keys and indices give a total order, so the ranks are a
// permutation of 0 .. m_pad - 1 for any input.  lam reuses the row sums of
// squares of the norm launch, whose threshold (entry m_pad) stays.
__global__ __launch_bounds__(SO_THREADS) void so_eig_diag_kernel(uint8_t* ws, uint32_t ei) {
    const mo_so_eig& eg = so_eigs(ws)[ei];
    const int64_t i = int64_t(blockIdx.x) * SO_THREADS + threadIdx.x;
    if (i >= eg.m_pad) return;
    double v = __builtin_huge_val();
    if (i < eg.m) {
        const double d = reinterpret_cast<const double*>(ws + eg.off_A)[i * eg.m_pad + i];
        if (d == d) v = d;
    }
    reinterpret_cast<double*>(ws + eg.off_norm)[i] = v;
}

constexpr int RANK_CHUNK = 1024;
__global__ __launch_bounds__(SO_THREADS) void so_eig_rank_kernel(uint8_t* ws, uint32_t ei) {
    __shared__ double chunk[RANK_CHUNK];
    const mo_so_eig& eg = so_eigs(ws)[ei];
    const double* lam = reinterpret_cast<const double*>(ws + eg.off_norm);
    const int n = int(eg.m_pad);
    const int i = int(blockIdx.x) * SO_THREADS + int(threadIdx.x);
    const double key = i < n ? lam[i] : 0.0;
    int rank = 0;
    for (int c0 = 0; c0 < n; c0 += RANK_CHUNK) {
        const int len = min(RANK_CHUNK, n - c0);
        __syncthreads();
        for (int q = threadIdx.x; q < len; q += SO_THREADS) chunk[q] = lam[c0 + q];
        __syncthreads();
        for (int q = 0; q < len; ++q) {
            const double v = chunk[q];
            rank += (v < key) || (v == key && c0 + q < i);
        }
    }
    if (i < n) reinterpret_cast<int*>(ws + eg.off_perm)[rank] = i;
}

// E32 row r = E row perm[r] (fp32) for r < m, zero below.
__global__ __launch_bounds__(SO_THREADS) void so_eig_gather_kernel(uint8_t* ws, uint32_t ei) {
    const mo_so_eig& eg = so_eigs(ws)[ei];
    const int64_t idx = int64_t(blockIdx.x) * SO_THREADS + threadIdx.x;
    if (idx >= int64_t(eg.m_pad) * eg.m_pad) return;
    const int64_t r = idx / eg.m_pad, c = idx % eg.m_pad;
    const int* perm = reinterpret_cast<const int*>(ws + eg.off_perm);
    const float* E = reinterpret_cast<const float*>(ws + eg.off_E);
    // the permutation is total (see the rank kernel); the row read is bounded
    // all the same
    float v = 0.f;
    if (r < eg.m) {
        const int64_t pr = perm[r];
        v = (pr >= 0 && pr < eg.m_pad) ? E[pr * eg.m_pad + c] : __builtin_nanf("");
    }
    reinterpret_cast<float*>(ws + eg.off_E32)[idx] = v;
    if (idx == 0) *reinterpret_cast<uint32_t*>(ws + eg.off_valid) = valid_word(eg);
}

}  // namespace

// ============================================================================
// launchers
// ============================================================================

hipError_t mo_launch_so_prep(const mo_so_mat& mt, uint8_t* ws, uint32_t mi, hipStream_t s) {
    const int64_t total = int64_t(mt.r_pad) * mt.c_pad;
    hipLaunchKernelGGL(so_prep_kernel, dim3(unsigned((total + SO_THREADS - 1) / SO_THREADS)), dim3(SO_THREADS),
                       0, s, ws, mi);
    return hipGetLastError();
}

hipError_t mo_launch_so_gemm(const mo_so_mat& mt, uint8_t* ws, uint32_t mi, int kind, hipStream_t s) {
    uint32_t rows = mt.r_pad, cols = mt.c_pad;
    if (kind == MO_SOK_STATS_L) cols = mt.r_pad;
    if (kind == MO_SOK_STATS_R) rows = mt.c_pad;
    hipLaunchKernelGGL(so_gemm_kernel, dim3(cols / GB, rows / GB), dim3(SO_THREADS), 0, s, ws, mi, kind);
    return hipGetLastError();
}

hipError_t mo_launch_so_eig_init(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, int warm, hipStream_t s) {
    const int64_t total = int64_t(eg.m_pad) * eg.m_pad;
    hipLaunchKernelGGL(so_eig_init_kernel, dim3(unsigned((total + SO_THREADS - 1) / SO_THREADS)),
                       dim3(SO_THREADS), 0, s, ws, ei, warm);
    return hipGetLastError();
}

hipError_t mo_launch_so_warm(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, int kind, hipStream_t s) {
    const unsigned n = unsigned(eg.m_pad / GB);
    hipLaunchKernelGGL(so_warm_kernel, dim3(n, n), dim3(SO_THREADS), 0, s, ws, ei, kind);
    return hipGetLastError();
}

hipError_t mo_launch_so_norm(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, hipStream_t s) {
    hipLaunchKernelGGL(so_norm_rows_kernel, dim3(eg.m_pad), dim3(SO_THREADS), 0, s, ws, ei);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(so_norm_final_kernel, dim3(1), dim3(SO_THREADS), 0, s, ws, ei);
    return hipGetLastError();
}

hipError_t mo_launch_so_solve(const mo_so_header& h, uint8_t* ws, uint32_t k, hipStream_t s) {
    hipLaunchKernelGGL(so_jac_solve_kernel, dim3(h.n_solve_items), dim3(SV_THREADS), 0, s, ws, k);
    return hipGetLastError();
}

hipError_t mo_launch_so_rotate(const mo_so_header& h, uint8_t* ws, uint32_t k, hipStream_t s) {
    hipLaunchKernelGGL(so_jac_rotate_kernel, dim3(h.n_apply_items + h.n_etile_items), dim3(SO_THREADS), 0, s,
                       ws, k);
    return hipGetLastError();
}

hipError_t mo_launch_so_rank(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, hipStream_t s) {
    const unsigned blocks = (eg.m_pad + SO_THREADS - 1) / SO_THREADS;
    hipLaunchKernelGGL(so_eig_diag_kernel, dim3(blocks), dim3(SO_THREADS), 0, s, ws, ei);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(so_eig_rank_kernel, dim3(blocks), dim3(SO_THREADS), 0, s, ws, ei);
    return hipGetLastError();
}

hipError_t mo_launch_so_gather(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, hipStream_t s) {
    const int64_t total = int64_t(eg.m_pad) * eg.m_pad;
    hipLaunchKernelGGL(so_eig_gather_kernel, dim3(unsigned((total + SO_THREADS - 1) / SO_THREADS)),
                       dim3(SO_THREADS), 0, s, ws, ei);
    return hipGetLastError();
}
