// Host side of the SOAP owner step: argument checks, the work list, the
// workspace plan and the launch sequence.
//
// [P] = "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
// sharding", §5.7: the owner runs SOAP (Adam in the Shampoo eigenbasis) on the
// whole matrices it owns, with no collective.  The readings of the step are
// stated with the entry points in mo.h.  Per bucket, stream-ordered:
//   prep        per matrix: padded G, M' = b1 M + (1 - b1) G
//   stats       per matrix: L' = L + G G^T, R' = R + G^T G (+ fp64 copies)
//   E = I       per statistics matrix, and its rotation threshold 2^-48 ||A||_F
//   rounds      grouped over all statistics matrices: pair problems, then
//               their rotations applied to A and to E (two launches per round)
//   sort        eigenvalues ascending, sorted fp32 eigenvectors
//   products    per matrix: Q_L^T G, x Q_R (V'), Q_L^T M', x Q_R (N), Q_L N,
//               x Q_R^T (W)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/mo.h"
#include "host_common.h"
#include "mo_kernels.h"
#include "so_worklist.h"

using namespace mo_host;

namespace {

constexpr int32_t kMaxSweeps = 100;
// 64 x 64 work items of one grouped rotation launch (upper A tiles plus E tiles
// over every side of the bucket): bounds the 32-bit item counts and the grid.
constexpr int64_t kMaxItems = int64_t(1) << 30;

mo_status validate_hp(const mo_soap_hparams* hp) {
    if (!hp) return MO_ERR_INVALID_ARG;
    if (!finite(hp->lr) || !finite(hp->weight_decay) || !finite(hp->beta1) || !finite(hp->beta2) ||
        !finite(hp->eps))
        return MO_ERR_INVALID_ARG;
    if (hp->beta1 < 0.f || hp->beta1 >= 1.f || hp->beta2 < 0.f || hp->beta2 >= 1.f || hp->eps < 0.f)
        return MO_ERR_INVALID_ARG;
    if (hp->step < 1 || hp->sweeps < 1 || hp->sweeps > kMaxSweeps) return MO_ERR_INVALID_ARG;
    if (hp->warm_start != 0 && hp->warm_start != 1) return MO_ERR_INVALID_ARG;
    return MO_OK;
}

struct Strides { int64_t w, g, l, r, m, v, u; };

Strides strides(const mo_soap_matrix& d) {
    return Strides{d.ld_w ? d.ld_w : d.cols, d.ld_g ? d.ld_g : d.cols, d.ld_l ? d.ld_l : d.rows,
                   d.ld_r ? d.ld_r : d.cols, d.ld_m ? d.ld_m : d.cols, d.ld_v ? d.ld_v : d.cols,
                   d.ld_u ? d.ld_u : d.cols};
}

mo_status validate(const mo_soap_matrix* mats, int32_t n, std::vector<Range>* ranges) {
    if (n < 0) return MO_ERR_INVALID_ARG;
    if (n > 0 && !mats) return MO_ERR_INVALID_ARG;
    int64_t items = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mo_soap_matrix& d = mats[i];
        if (d.rows < 0 || d.cols < 0) return MO_ERR_INVALID_ARG;
        if (d.ld_w < 0 || d.ld_g < 0 || d.ld_l < 0 || d.ld_r < 0 || d.ld_m < 0 || d.ld_v < 0 || d.ld_u < 0)
            return MO_ERR_INVALID_ARG;
        if (d.rows == 0 || d.cols == 0) continue;   // empty shard: skipped
        if (d.w_dtype != MO_F32 && d.w_dtype != MO_BF16) return MO_ERR_UNSUPPORTED;
        if (d.g_dtype != MO_F32 && d.g_dtype != MO_BF16) return MO_ERR_UNSUPPORTED;
        if (!d.W || !d.G || !d.L || !d.R || !d.M || !d.V) return MO_ERR_INVALID_ARG;
        const Strides s = strides(d);
        if (s.w < d.cols || s.g < d.cols || s.l < d.rows || s.r < d.cols || s.m < d.cols || s.v < d.cols ||
            s.u < d.cols)
            return MO_ERR_INVALID_ARG;
        if (d.rows > MO_SO_MAXSIDE || d.cols > MO_SO_MAXSIDE) return MO_ERR_UNSUPPORTED;
        for (int64_t m : {d.rows, d.cols}) {
            const int64_t P = (m + MO_SO_PAD - 1) / MO_SO_PAD;
            items += P * (P + 1) / 2 + P * P;
        }
        if (items > kMaxItems) return MO_ERR_UNSUPPORTED;
        if (ranges) {
            ranges->push_back(matrix_range(d.W, d.rows, d.cols, s.w, elem_size(d.w_dtype), 1));
            ranges->push_back(matrix_range(d.G, d.rows, d.cols, s.g, elem_size(d.g_dtype), 0));
            ranges->push_back(matrix_range(d.L, d.rows, d.rows, s.l, 4, 1));
            ranges->push_back(matrix_range(d.R, d.cols, d.cols, s.r, 4, 1));
            ranges->push_back(matrix_range(d.M, d.rows, d.cols, s.m, 4, 1));
            ranges->push_back(matrix_range(d.V, d.rows, d.cols, s.v, 4, 1));
            if (d.update_out) ranges->push_back(matrix_range(d.update_out, d.rows, d.cols, s.u, 4, 1));
        }
    }
    return MO_OK;
}

struct SoPlan {
    std::vector<uint8_t> bytes;   // the work list
    mo_so_header header;
    std::vector<mo_so_mat> mats;
    std::vector<mo_so_eig> eigs;
};

// Builds the work list and workspace plan (validated inputs only).
void build_plan(const mo_soap_matrix* mats, int32_t n, const mo_soap_hparams* hp, SoPlan* plan) {
    const uint64_t PAD = MO_SO_PAD;
    std::vector<mo_so_mat>& recs = plan->mats;
    std::vector<mo_so_eig>& eigs = plan->eigs;
    recs.clear();
    eigs.clear();
    uint32_t solve_items = 0, apply_items = 0, etile_items = 0, max_rounds = 0;
    auto add_eig = [&](uint32_t m, uint32_t mat, const float* ext, int64_t ld_ext) {
        mo_so_eig e;
        std::memset(&e, 0, sizeof(e));
        e.m = m;
        e.m_pad = uint32_t(align_up(m, PAD));
        e.P = e.m_pad / PAD;
        e.mat = mat;
        e.ext = reinterpret_cast<uint64_t>(ext);
        e.ld_ext = ld_ext;
        e.rounds = uint32_t(hp->sweeps) * (2 * e.P - 1);
        e.solve_begin = solve_items;
        e.apply_begin = apply_items;
        e.etile_begin = etile_items;
        solve_items += e.P;
        apply_items += e.P * (e.P + 1) / 2;
        etile_items += e.P * ((e.P + MO_SO_ECOLS - 1) / MO_SO_ECOLS);
        max_rounds = std::max(max_rounds, e.rounds);
        eigs.push_back(e);
        return uint32_t(eigs.size() - 1);
    };
    const double b1 = hp->beta1, b2 = hp->beta2;
    const double bc1 = 1.0 - std::pow(b1, double(hp->step)), bc2 = 1.0 - std::pow(b2, double(hp->step));
    for (int32_t i = 0; i < n; ++i) {
        const mo_soap_matrix& d = mats[i];
        if (d.rows == 0 || d.cols == 0) continue;
        const Strides s = strides(d);
        mo_so_mat r;
        std::memset(&r, 0, sizeof(r));
        r.W = reinterpret_cast<uint64_t>(d.W);
        r.G = reinterpret_cast<uint64_t>(d.G);
        r.M = reinterpret_cast<uint64_t>(d.M);
        r.V = reinterpret_cast<uint64_t>(d.V);
        r.U = reinterpret_cast<uint64_t>(d.update_out);
        r.ld_w = s.w;
        r.ld_g = s.g;
        r.ld_m = s.m;
        r.ld_v = s.v;
        r.ld_u = s.u;
        r.rows = uint32_t(d.rows);
        r.cols = uint32_t(d.cols);
        r.r_pad = uint32_t(align_up(uint64_t(d.rows), PAD));
        r.c_pad = uint32_t(align_up(uint64_t(d.cols), PAD));
        r.flags = (d.w_dtype == MO_BF16 ? MO_SOF_W_BF16 : 0u) | (d.g_dtype == MO_BF16 ? MO_SOF_G_BF16 : 0u) |
                  (d.update_out ? MO_SOF_HAS_UPDATE : 0u);
        r.decay = float(1.0 - double(hp->lr) * double(hp->weight_decay));
        r.lr = hp->lr;
        r.beta1 = hp->beta1;
        r.beta2 = hp->beta2;
        r.ibc1 = float(1.0 / bc1);
        r.ibc2 = float(1.0 / bc2);
        r.eps = hp->eps;
        const uint32_t mi = uint32_t(recs.size());
        r.eig_l = add_eig(r.rows, mi, d.L, s.l);
        r.eig_r = add_eig(r.cols, mi, d.R, s.r);
        recs.push_back(r);
    }
    const uint32_t nm = uint32_t(recs.size()), ne = uint32_t(eigs.size());
    mo_so_header h;
    std::memset(&h, 0, sizeof(h));
    h.magic = MO_SO_MAGIC;
    h.version = MO_SO_VERSION;
    h.n_mats = nm;
    h.n_eigs = ne;
    h.sweeps = uint32_t(hp->sweeps);
    h.max_rounds = max_rounds;
    h.n_solve_items = solve_items;
    h.n_apply_items = apply_items;
    h.n_etile_items = etile_items;
    uint64_t off = align_up(sizeof(mo_so_header), MO_WS_ALIGN);
    h.mats_offset = off;
    off = align_up(off + uint64_t(nm) * sizeof(mo_so_mat), MO_WS_ALIGN);
    h.eigs_offset = off;
    off = align_up(off + uint64_t(ne) * sizeof(mo_so_eig), MO_WS_ALIGN);
    h.wl_bytes = off;
    auto take = [&](uint64_t bytes) { uint64_t o = off; off = align_up(off + bytes, MO_WS_ALIGN); return o; };
    for (mo_so_mat& r : recs) {
        const uint64_t rc = uint64_t(r.r_pad) * r.c_pad * 4;
        r.off_G = take(rc);
        r.off_M = take(rc);
        r.off_T = take(rc);
        r.off_N = take(rc);
    }
    for (mo_so_eig& e : eigs) {
        const uint64_t mm = uint64_t(e.m_pad) * e.m_pad;
        e.off_A = take(mm * 8);
        e.off_E = take(mm * 4);
        e.off_D = take(uint64_t(e.P) * 64 * 64 * 8);
        e.off_E32 = take(mm * 4);
        e.off_perm = take(uint64_t(e.m_pad) * 4);
        e.off_flag = take(uint64_t(e.P) * 4);
        e.off_last = take(uint64_t(e.P) * 4);
        e.off_norm = take(uint64_t(e.m_pad + 1) * 8);
        e.off_valid = take(8);
    }
    h.ws_bytes = off;
    plan->header = h;
    plan->bytes.assign(h.wl_bytes, 0);
    std::memcpy(plan->bytes.data(), &h, sizeof(h));
    if (nm) std::memcpy(plan->bytes.data() + h.mats_offset, recs.data(), nm * sizeof(mo_so_mat));
    if (ne) std::memcpy(plan->bytes.data() + h.eigs_offset, eigs.data(), ne * sizeof(mo_so_eig));
}

}  // namespace

extern "C" {

mo_status soap_workspace_bytes(const mo_soap_matrix* mats, int32_t n, const mo_soap_hparams* hp,
                               size_t* bytes) {
    if (!bytes) return MO_ERR_INVALID_ARG;
    mo_status st = validate_hp(hp);
    if (st != MO_OK) return st;
    if ((st = validate(mats, n, nullptr)) != MO_OK) return st;
    SoPlan plan;
    build_plan(mats, n, hp, &plan);
    *bytes = size_t(plan.header.ws_bytes) + MO_WS_ALIGN;
    return MO_OK;
}

mo_status soap_owner_step(const mo_soap_matrix* mats, int32_t n, const mo_soap_hparams* hp, void* workspace,
                          size_t workspace_bytes, void* stream) {
    mo_status st = validate_hp(hp);
    if (st != MO_OK) return st;
    std::vector<Range> ranges;
    if ((st = validate(mats, n, &ranges)) != MO_OK) return st;
    if (n == 0) return MO_OK;
    SoPlan plan;
    build_plan(mats, n, hp, &plan);
    const mo_so_header& h = plan.header;
    if (h.n_mats == 0) return MO_OK;
    const size_t need = size_t(h.ws_bytes) + MO_WS_ALIGN;
    if (!workspace || workspace_bytes < need) return MO_ERR_WORKSPACE_TOO_SMALL;
    ranges.push_back(Range{reinterpret_cast<uintptr_t>(workspace),
                           reinterpret_cast<uintptr_t>(workspace) + workspace_bytes, 1});
    if (ranges_conflict(ranges)) return MO_ERR_ALIAS;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = reinterpret_cast<uint8_t*>(align_up(reinterpret_cast<uintptr_t>(workspace), MO_WS_ALIGN));
    if (upload(plan.bytes.data(), plan.bytes.size(), ws, s) != hipSuccess) return MO_ERR_HIP;
    auto ok = [&](int phase, auto&& launch) { return timed_launch(phase, s, launch) == hipSuccess; };
    for (uint32_t i = 0; i < h.n_mats; ++i) {
        const mo_so_mat& mt = plan.mats[i];
        if (!ok(MO_PHASE_SO_PREP, [&] { return mo_launch_so_prep(mt, ws, i, s); })) return MO_ERR_HIP;
        if (!ok(MO_PHASE_SO_STATS, [&] { return mo_launch_so_gemm(mt, ws, i, MO_SOK_STATS_L, s); }))
            return MO_ERR_HIP;
        if (!ok(MO_PHASE_SO_STATS, [&] { return mo_launch_so_gemm(mt, ws, i, MO_SOK_STATS_R, s); }))
            return MO_ERR_HIP;
    }
    const int warm = hp->warm_start;
    for (uint32_t e = 0; e < h.n_eigs; ++e) {
        if (warm)
            for (int kind : {MO_SOW_P, MO_SOW_E, MO_SOW_T, MO_SOW_A})
                if (!ok(MO_PHASE_SO_WARM, [&] { return mo_launch_so_warm(plan.eigs[e], ws, e, kind, s); }))
                    return MO_ERR_HIP;
        if (!ok(MO_PHASE_SO_SORT, [&] { return mo_launch_so_eig_init(plan.eigs[e], ws, e, warm, s); }))
            return MO_ERR_HIP;
        if (!ok(MO_PHASE_SO_SORT, [&] { return mo_launch_so_norm(plan.eigs[e], ws, e, s); })) return MO_ERR_HIP;
    }
    for (uint32_t k = 0; k < h.max_rounds; ++k) {
        if (!ok(MO_PHASE_SO_SOLVE, [&] { return mo_launch_so_solve(h, ws, k, s); })) return MO_ERR_HIP;
        if (!ok(MO_PHASE_SO_APPLY, [&] { return mo_launch_so_rotate(h, ws, k, s); })) return MO_ERR_HIP;
    }
    for (uint32_t e = 0; e < h.n_eigs; ++e) {
        if (!ok(MO_PHASE_SO_SORT, [&] { return mo_launch_so_rank(plan.eigs[e], ws, e, s); })) return MO_ERR_HIP;
        if (!ok(MO_PHASE_SO_SORT, [&] { return mo_launch_so_gather(plan.eigs[e], ws, e, s); })) return MO_ERR_HIP;
    }
    static const int kProducts[] = {MO_SOK_LEFT_G, MO_SOK_RIGHT_G, MO_SOK_LEFT_M,
                                    MO_SOK_RIGHT_M, MO_SOK_BACK_L,  MO_SOK_BACK_R};
    for (uint32_t i = 0; i < h.n_mats; ++i)
        for (int kind : kProducts)
            if (!ok(MO_PHASE_SO_PRODUCTS, [&] { return mo_launch_so_gemm(plan.mats[i], ws, i, kind, s); }))
                return MO_ERR_HIP;
    return MO_OK;
}

mo_status soap_converged(const mo_soap_matrix* mats, int32_t n, const mo_soap_hparams* hp,
                         const void* workspace, size_t workspace_bytes, int32_t* rotating, void* stream) {
    mo_status st = validate_hp(hp);
    if (st != MO_OK) return st;
    if ((st = validate(mats, n, nullptr)) != MO_OK) return st;
    if (n > 0 && !rotating) return MO_ERR_INVALID_ARG;
    for (int32_t i = 0; i < 2 * n; ++i) rotating[i] = 0;
    SoPlan plan;
    build_plan(mats, n, hp, &plan);
    const mo_so_header& h = plan.header;
    if (h.n_mats == 0) return MO_OK;
    const size_t need = size_t(h.ws_bytes) + MO_WS_ALIGN;
    if (!workspace || workspace_bytes < need) return MO_ERR_WORKSPACE_TOO_SMALL;
    const uint8_t* ws = reinterpret_cast<const uint8_t*>(
        align_up(reinterpret_cast<uintptr_t>(workspace), MO_WS_ALIGN));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the flag words of every decomposition, copied after the step's work on s
    std::vector<std::vector<uint32_t>> words(h.n_eigs);
    for (uint32_t e = 0; e < h.n_eigs; ++e) {
        words[e].assign(plan.eigs[e].P, 0u);
        if (hipMemcpyAsync(words[e].data(), ws + plan.eigs[e].off_last, size_t(plan.eigs[e].P) * 4,
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            return MO_ERR_HIP;
    }
    if (hipStreamSynchronize(s) != hipSuccess) return MO_ERR_HIP;
    uint32_t live = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (mats[i].rows == 0 || mats[i].cols == 0) continue;
        const mo_so_mat& mt = plan.mats[live++];
        for (int side = 0; side < 2; ++side) {
            int32_t c = 0;
            for (uint32_t w : words[side ? mt.eig_r : mt.eig_l]) c += w ? 1 : 0;
            rotating[2 * i + side] = c;
        }
    }
    return MO_OK;
}

}  // extern "C"
