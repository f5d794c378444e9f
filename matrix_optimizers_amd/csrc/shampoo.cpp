// Host side of the Shampoo owner step: argument checks, the work list, the
// workspace plan and the launch sequence.
//
// [P] = "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
// sharding", §5.7: the owner runs Shampoo (full left / right preconditioners,
// inverse fourth root, float32) on the whole matrices it owns, with no
// collective.  The readings of the step are stated with the entry points in
// mo.h.  Per bucket, stream-ordered, each launch covering every matrix:
//   layout            G -> padded G and G^T (fp32)
//   stats             L' = L + G G^T, R' = R + G^T G (also the padded M_0)
//   rootprep          ||S'||_F per root, X_0, H_1 (three small launches)
//   k = 1 .. K-1:     S2 = X X (and H_k = H_{k-1} X for k >= 2); S4 = S2 S2;
//                     M_k = alpha S4 M_{k-1}, X_k = ((p + 1) I - M_k) / p
//   K >= 2:           H_K = H_{K-1} X, stored transposed
//   left, right       T = H_L G;  W <- (1 - lr wd) W - lr T H_R, each H used by
//                     its rows (sh_worklist.h)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/mo.h"
#include "host_common.h"
#include "mo_kernels.h"
#include "sh_worklist.h"
#include "tile_dispatch.h"

using namespace mo_host;

namespace {

// Each side is also the side of a root, whose seven m_pad x m_pad fp32 buffers
// take 7 * 4 * m_pad^2 bytes (120 GB at 65536) and whose upper tiles the
// planner lists on the host.
constexpr int64_t kMaxSide = int64_t(1) << 16;
constexpr int32_t kMaxIters = 100;
// Tiles of 256 x 256 over all roots and matrices of a bucket: bounds the work
// lists and the host memory that builds them.
constexpr int64_t kMaxTiles = int64_t(1) << 26;

mo_status validate_hp(const mo_shampoo_hparams* hp) {
    if (!hp) return MO_ERR_INVALID_ARG;
    if (!finite(hp->lr) || !finite(hp->weight_decay)) return MO_ERR_INVALID_ARG;
    if (hp->root_iters < 1 || hp->root_iters > kMaxIters) return MO_ERR_INVALID_ARG;
    return MO_OK;
}

struct Strides { int64_t w, g, l, r, u; };

Strides strides(const mo_shampoo_matrix& d) {
    return Strides{d.ld_w ? d.ld_w : d.cols, d.ld_g ? d.ld_g : d.cols, d.ld_l ? d.ld_l : d.rows,
                   d.ld_r ? d.ld_r : d.cols, d.ld_u ? d.ld_u : d.cols};
}

mo_status validate(const mo_shampoo_matrix* mats, int32_t n, std::vector<Range>* ranges) {
    if (n < 0) return MO_ERR_INVALID_ARG;
    if (n > 0 && !mats) return MO_ERR_INVALID_ARG;
    int64_t tiles = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mo_shampoo_matrix& d = mats[i];
        if (d.rows < 0 || d.cols < 0) return MO_ERR_INVALID_ARG;
        if (d.ld_w < 0 || d.ld_g < 0 || d.ld_l < 0 || d.ld_r < 0 || d.ld_u < 0) return MO_ERR_INVALID_ARG;
        if (d.rows == 0 || d.cols == 0) continue;   // empty shard: skipped
        if (d.w_dtype != MO_F32 && d.w_dtype != MO_BF16) return MO_ERR_UNSUPPORTED;
        if (d.g_dtype != MO_F32 && d.g_dtype != MO_BF16) return MO_ERR_UNSUPPORTED;
        if (!d.W || !d.G || !d.L || !d.R) return MO_ERR_INVALID_ARG;
        const Strides s = strides(d);
        if (s.w < d.cols || s.g < d.cols || s.l < d.rows || s.r < d.cols || s.u < d.cols)
            return MO_ERR_INVALID_ARG;
        if (d.rows > kMaxSide || d.cols > kMaxSide) return MO_ERR_UNSUPPORTED;
        const int64_t tr = (d.rows + 255) / 256, tc = (d.cols + 255) / 256;
        tiles += tr * tr + tc * tc + tr * tc;
        if (tiles > kMaxTiles) return MO_ERR_UNSUPPORTED;
        if (ranges) {
            ranges->push_back(matrix_range(d.W, d.rows, d.cols, s.w, elem_size(d.w_dtype), 1));
            ranges->push_back(matrix_range(d.G, d.rows, d.cols, s.g, elem_size(d.g_dtype), 0));
            ranges->push_back(matrix_range(d.L, d.rows, d.rows, s.l, 4, 1));
            ranges->push_back(matrix_range(d.R, d.cols, d.cols, s.r, 4, 1));
            if (d.update_out) ranges->push_back(matrix_range(d.update_out, d.rows, d.cols, s.u, 4, 1));
        }
    }
    return MO_OK;
}

struct ShPlan {
    std::vector<uint8_t> bytes;   // the work list
    mo_sh_header header;
};

// Builds the work list and workspace plan (validated inputs only).
void build_plan(const mo_shampoo_matrix* mats, int32_t n, const mo_shampoo_hparams* hp, ShPlan* plan) {
    const uint64_t T = MO_GEMM_TILE, ST = 64;
    std::vector<mo_sh_mat> recs;
    std::vector<mo_sh_root> roots;
    uint32_t lay_total = 0, root_items = 0;
    auto add_root = [&](uint32_t m, uint32_t m_pad, uint32_t mat, const float* ext, int64_t ld_ext,
                        uint32_t op_ld) {
        mo_sh_root rt;
        std::memset(&rt, 0, sizeof(rt));
        rt.m = m;
        rt.m_pad = m_pad;
        rt.mat = mat;
        rt.ext = reinterpret_cast<uint64_t>(ext);
        rt.ld_ext = ld_ext;
        rt.op_ld = op_ld;
        rt.item_begin = root_items;
        rt.tiles_c = uint32_t(m_pad / ST);
        rt.n_partials = rt.tiles_c * rt.tiles_c;
        root_items += rt.n_partials;
        roots.push_back(rt);
        return uint32_t(roots.size() - 1);
    };
    for (int32_t i = 0; i < n; ++i) {
        const mo_shampoo_matrix& d = mats[i];
        if (d.rows == 0 || d.cols == 0) continue;
        const Strides s = strides(d);
        mo_sh_mat r;
        std::memset(&r, 0, sizeof(r));
        r.W = reinterpret_cast<uint64_t>(d.W);
        r.G = reinterpret_cast<uint64_t>(d.G);
        r.U = reinterpret_cast<uint64_t>(d.update_out);
        r.ld_w = s.w;
        r.ld_g = s.g;
        r.ld_u = s.u;
        r.rows = uint32_t(d.rows);
        r.cols = uint32_t(d.cols);
        r.r_pad = uint32_t(align_up(uint64_t(d.rows), T));
        r.c_pad = uint32_t(align_up(uint64_t(d.cols), T));
        r.flags = (d.w_dtype == MO_BF16 ? MO_SHF_W_BF16 : 0u) | (d.g_dtype == MO_BF16 ? MO_SHF_G_BF16 : 0u) |
                  (d.update_out ? MO_SHF_HAS_UPDATE : 0u);
        r.lay_begin = lay_total;
        r.lay_tiles_c = uint32_t(r.c_pad / ST);
        lay_total += uint32_t((r.r_pad / ST) * (r.c_pad / ST));
        r.decay = float(1.0 - double(hp->lr) * double(hp->weight_decay));
        r.lr = hp->lr;
        const uint32_t mi = uint32_t(recs.size());
        r.root_l = add_root(r.rows, r.r_pad, mi, d.L, s.l, r.c_pad);   // L' = L + G G^T: K = cols
        r.root_r = add_root(r.cols, r.c_pad, mi, d.R, s.r, r.r_pad);   // R' = R + G^T G: K = rows
        recs.push_back(r);
    }
    const uint32_t nm = uint32_t(recs.size()), nr = uint32_t(roots.size());

    // products: six per root (stats, S2, H, HT, S4, M), two per matrix
    std::vector<mo_sh_prod> prods;
    auto prod_of = [&](uint32_t kind, uint32_t ref) {
        prods.push_back({kind, ref});
        return uint32_t(prods.size() - 1);
    };
    std::vector<mo_gemm_job> jl[MO_SHL_COUNT];
    std::vector<uint64_t> wl[MO_SHL_COUNT];
    auto add_job = [&](int list, uint32_t idx, uint32_t tm, uint32_t tn, bool upper, uint64_t klen) {
        const uint64_t tiles = upper ? uint64_t(tm) * (tm + 1) / 2 : uint64_t(tm) * tn;
        jl[list].push_back({idx, tm, tn, upper, klen});
        wl[list].push_back(tiles * klen);
    };
    for (uint32_t j = 0; j < nr; ++j) {
        const mo_sh_root& rt = roots[j];
        const uint32_t t = uint32_t(rt.m_pad / T);
        add_job(MO_SHL_STATS, prod_of(MO_SHK_STATS, j), t, t, true, rt.op_ld);
        const uint32_t sq = prod_of(MO_SHK_SQ, j), hh = prod_of(MO_SHK_H, j);
        add_job(MO_SHL_SQ, sq, t, t, true, rt.m_pad);
        add_job(MO_SHL_SQH, sq, t, t, true, rt.m_pad);
        add_job(MO_SHL_SQH, hh, t, t, false, rt.m_pad);
        add_job(MO_SHL_H, prod_of(MO_SHK_HT, j), t, t, false, rt.m_pad);
        add_job(MO_SHL_S4, prod_of(MO_SHK_S4, j), t, t, true, rt.m_pad);
        add_job(MO_SHL_M, prod_of(MO_SHK_M, j), t, t, true, rt.m_pad);
    }
    for (uint32_t i = 0; i < nm; ++i) {
        const mo_sh_mat& r = recs[i];
        add_job(MO_SHL_LEFT, prod_of(MO_SHK_LEFT, i), uint32_t(r.r_pad / T), uint32_t(r.c_pad / T), false, r.r_pad);
        add_job(MO_SHL_RIGHT, prod_of(MO_SHK_RIGHT, i), uint32_t(r.r_pad / T), uint32_t(r.c_pad / T), false, r.c_pad);
    }
    // Each list: products by descending work (tiles x K; ties in product
    // order), then to the XCD queues (tile_dispatch.h).
    std::vector<mo_wl_item> items[MO_SHL_COUNT];
    for (int l = 0; l < MO_SHL_COUNT; ++l) {
        std::vector<size_t> ord(jl[l].size());
        for (size_t q = 0; q < ord.size(); ++q) ord[q] = q;
        std::stable_sort(ord.begin(), ord.end(), [&](size_t a, size_t b) { return wl[l][a] > wl[l][b]; });
        std::vector<mo_gemm_job> js;
        for (size_t q : ord) js.push_back(jl[l][q]);
        mo_dispatch_tiles(js, items[l]);
    }

    mo_sh_header h;
    std::memset(&h, 0, sizeof(h));
    h.magic = MO_SH_MAGIC;
    h.version = MO_SH_VERSION;
    h.n_mats = nm;
    h.n_roots = nr;
    h.n_prods = uint32_t(prods.size());
    h.root_iters = uint32_t(hp->root_iters);
    h.n_lay_items = lay_total;
    h.n_root_items = root_items;
    uint64_t off = align_up(sizeof(mo_sh_header), MO_WS_ALIGN);
    h.mats_offset = off;
    off = align_up(off + uint64_t(nm) * sizeof(mo_sh_mat), MO_WS_ALIGN);
    h.roots_offset = off;
    off = align_up(off + uint64_t(nr) * sizeof(mo_sh_root), MO_WS_ALIGN);
    h.prods_offset = off;
    off = align_up(off + prods.size() * sizeof(mo_sh_prod), MO_WS_ALIGN);
    for (int l = 0; l < MO_SHL_COUNT; ++l) {
        h.n_items[l] = uint32_t(items[l].size());
        h.list_offset[l] = off;
        off = align_up(off + items[l].size() * sizeof(mo_wl_item), MO_WS_ALIGN);
    }
    h.wl_bytes = off;

    // workspace regions
    auto take = [&](uint64_t bytes) { uint64_t o = off; off = align_up(off + bytes, MO_WS_ALIGN); return o; };
    for (mo_sh_mat& r : recs) {
        const uint64_t rc = uint64_t(r.r_pad) * r.c_pad * 4;
        r.off_G = take(rc);
        r.off_Gt = take(rc);
        r.off_T = take(rc);
    }
    for (mo_sh_root& rt : roots) {
        const uint64_t mm = uint64_t(rt.m_pad) * rt.m_pad * 4;
        rt.off_M[0] = take(mm);
        rt.off_M[1] = take(mm);
        rt.off_X = take(mm);
        rt.off_S2 = take(mm);
        rt.off_S4 = take(mm);
        rt.off_H[0] = take(mm);
        rt.off_H[1] = take(mm);
        rt.off_partials = take(uint64_t(rt.n_partials) * 4);
        rt.off_scale = take(16);
        const mo_sh_mat& r = recs[rt.mat];
        rt.off_op = (&rt - roots.data()) == int64_t(r.root_l) ? r.off_G : r.off_Gt;
    }
    h.ws_bytes = off;

    plan->header = h;
    plan->bytes.assign(h.wl_bytes, 0);
    std::memcpy(plan->bytes.data(), &h, sizeof(h));
    if (nm) std::memcpy(plan->bytes.data() + h.mats_offset, recs.data(), nm * sizeof(mo_sh_mat));
    if (nr) std::memcpy(plan->bytes.data() + h.roots_offset, roots.data(), nr * sizeof(mo_sh_root));
    if (!prods.empty())
        std::memcpy(plan->bytes.data() + h.prods_offset, prods.data(), prods.size() * sizeof(mo_sh_prod));
    for (int l = 0; l < MO_SHL_COUNT; ++l)
        if (!items[l].empty())
            std::memcpy(plan->bytes.data() + h.list_offset[l], items[l].data(), items[l].size() * sizeof(mo_wl_item));
}

}  // namespace

extern "C" {

mo_status shampoo_workspace_bytes(const mo_shampoo_matrix* mats, int32_t n, const mo_shampoo_hparams* hp,
                                  size_t* bytes) {
    if (!bytes) return MO_ERR_INVALID_ARG;
    mo_status st = validate_hp(hp);
    if (st != MO_OK) return st;
    if ((st = validate(mats, n, nullptr)) != MO_OK) return st;
    ShPlan plan;
    build_plan(mats, n, hp, &plan);
    *bytes = size_t(plan.header.ws_bytes) + MO_WS_ALIGN;
    return MO_OK;
}

mo_status shampoo_owner_step(const mo_shampoo_matrix* mats, int32_t n, const mo_shampoo_hparams* hp,
                             void* workspace, size_t workspace_bytes, void* stream) {
    mo_status st = validate_hp(hp);
    if (st != MO_OK) return st;
    std::vector<Range> ranges;
    if ((st = validate(mats, n, &ranges)) != MO_OK) return st;
    if (n == 0) return MO_OK;
    ShPlan plan;
    build_plan(mats, n, hp, &plan);
    const mo_sh_header& h = plan.header;
    if (h.n_mats == 0) return MO_OK;
    const size_t need = size_t(h.ws_bytes) + MO_WS_ALIGN;
    if (!workspace || workspace_bytes < need) return MO_ERR_WORKSPACE_TOO_SMALL;
    ranges.push_back(Range{reinterpret_cast<uintptr_t>(workspace),
                           reinterpret_cast<uintptr_t>(workspace) + workspace_bytes, 1});
    if (ranges_conflict(ranges)) return MO_ERR_ALIAS;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = reinterpret_cast<uint8_t*>(align_up(reinterpret_cast<uintptr_t>(workspace), MO_WS_ALIGN));
    if (upload(plan.bytes.data(), plan.bytes.size(), ws, s) != hipSuccess) return MO_ERR_HIP;
    auto gemm = [&](int phase, int list, int k) {
        return timed_launch(phase, s, [&] { return mo_launch_sh_gemm(h, ws, list, k, s); }) == hipSuccess;
    };
    if (timed_launch(MO_PHASE_SH_LAYOUT, s, [&] { return mo_launch_sh_layout(h, ws, s); }) != hipSuccess)
        return MO_ERR_HIP;
    if (!gemm(MO_PHASE_SH_STATS, MO_SHL_STATS, 0)) return MO_ERR_HIP;
    if (timed_launch(MO_PHASE_SH_ROOTPREP, s, [&] { return mo_launch_sh_rootprep(h, ws, s); }) != hipSuccess)
        return MO_ERR_HIP;
    const int K = hp->root_iters;
    for (int k = 1; k < K; ++k) {
        if (!gemm(MO_PHASE_SH_ROOT, k == 1 ? MO_SHL_SQ : MO_SHL_SQH, k)) return MO_ERR_HIP;
        if (!gemm(MO_PHASE_SH_ROOT, MO_SHL_S4, k)) return MO_ERR_HIP;
        if (!gemm(MO_PHASE_SH_ROOT, MO_SHL_M, k)) return MO_ERR_HIP;
    }
    if (K >= 2 && !gemm(MO_PHASE_SH_ROOT, MO_SHL_H, K)) return MO_ERR_HIP;
    if (!gemm(MO_PHASE_SH_LEFT, MO_SHL_LEFT, 0)) return MO_ERR_HIP;
    if (!gemm(MO_PHASE_SH_RIGHT, MO_SHL_RIGHT, 0)) return MO_ERR_HIP;
    return MO_OK;
}

}  // extern "C"
