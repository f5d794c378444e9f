// Host side of the Muon step's C ABI: argument validation, the work-list
// builder, the workspace planner and the phase launcher (the upload and timing
// helpers are in host_common.cpp).
//
// One step over a bucket is 2 + 3K stream-ordered launches, each covering every
// matrix of the bucket ([P] = "MatrixFSDP: communication-free matrix optimizers
// under ZeRO-3 parameter sharding", §3: each owner updates its whole matrices
// locally, with no collective):
//   momentum  (EMA + Nesterov, fp32 M', U in the short-side frame, norm partials)
//   norm      (one fixed-order sum per matrix -> 1/max(||U||_F, eps))
//   K times:  gram (A = X X^T), poly (B = b A + c A A), update (X <- a X + B X;
//             the last one writes W)
// or, when K == 0, an apply pass that writes W from the normalised U.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/mo.h"
#include "mo_kernels.h"
#include "host_common.h"
#include "mo_worklist.h"
#include "tile_dispatch.h"


using namespace mo_host;

namespace {

constexpr int64_t kMaxSide = int64_t(1) << 23;   // 32768 tiles of 256: tile indexes fit 16 bits
// Elements per matrix: bounds the work list (at most 2^20 tiles per phase and
// matrix) and the host memory the planner needs to build it.
constexpr int64_t kMaxElems = int64_t(1) << 36;

mo_status validate_hparams(const mo_muon_hparams* hp) {
    if (!hp) return MO_ERR_INVALID_ARG;
    if (hp->ns_steps < 0) return MO_ERR_INVALID_ARG;
    if (!finite(hp->lr) || !finite(hp->weight_decay) || !finite(hp->momentum) ||
        !finite(hp->ns_a) || !finite(hp->ns_b) || !finite(hp->ns_c) || !finite(hp->eps))
        return MO_ERR_INVALID_ARG;
    if (!(hp->eps > 0.f)) return MO_ERR_INVALID_ARG;
    if (hp->lr_adjust != MO_LR_ORIGINAL && hp->lr_adjust != MO_LR_MATCH_RMS_ADAMW &&
        hp->lr_adjust != MO_LR_NONE)
        return MO_ERR_INVALID_ARG;
    if (hp->ns_dtype != MO_F32 && hp->ns_dtype != MO_BF16) return MO_ERR_UNSUPPORTED;
    return MO_OK;
}

// Tiles of 256 x 256 in all Update products of a bucket (the largest phase):
// bounds the work list and the host memory that builds it.
constexpr int64_t kMaxTiles = int64_t(1) << 26;

// Checks every descriptor; collects the byte ranges of live tensors.
mo_status validate_mats(const mo_matrix* mats, int32_t n, std::vector<Range>* ranges) {
    if (n < 0) return MO_ERR_INVALID_ARG;
    if (n > 0 && !mats) return MO_ERR_INVALID_ARG;
    int64_t tiles = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mo_matrix& d = mats[i];
        if (d.rows < 0 || d.cols < 0) return MO_ERR_INVALID_ARG;
        if (d.ld_w < 0 || d.ld_g < 0 || d.ld_m < 0 || d.ld_u < 0) return MO_ERR_INVALID_ARG;
        if (d.rows == 0 || d.cols == 0) continue;   // empty shard: skipped
        if (d.w_dtype != MO_F32 && d.w_dtype != MO_BF16) return MO_ERR_UNSUPPORTED;
        if (d.g_dtype != MO_F32 && d.g_dtype != MO_BF16) return MO_ERR_UNSUPPORTED;
        if (!d.W || !d.G || !d.M) return MO_ERR_INVALID_ARG;
        const int64_t ldw = d.ld_w ? d.ld_w : d.cols, ldg = d.ld_g ? d.ld_g : d.cols;
        const int64_t ldm = d.ld_m ? d.ld_m : d.cols, ldu = d.ld_u ? d.ld_u : d.cols;
        if (ldw < d.cols || ldg < d.cols || ldm < d.cols || ldu < d.cols)
            return MO_ERR_INVALID_ARG;
        if (d.rows > kMaxSide || d.cols > kMaxSide) return MO_ERR_UNSUPPORTED;
        if (d.rows * d.cols > kMaxElems) return MO_ERR_UNSUPPORTED;
        tiles += ((d.rows + 255) / 256) * ((d.cols + 255) / 256);
        if (tiles > kMaxTiles) return MO_ERR_UNSUPPORTED;
        if (ranges) {
            ranges->push_back(matrix_range(d.W, d.rows, d.cols, ldw, elem_size(d.w_dtype), 1));
            ranges->push_back(matrix_range(d.G, d.rows, d.cols, ldg, elem_size(d.g_dtype), 0));
            ranges->push_back(matrix_range(d.M, d.rows, d.cols, ldm, 4, 1));
            if (d.update_out)
                ranges->push_back(matrix_range(d.update_out, d.rows, d.cols, ldu, 4, 1));
        }
    }
    return MO_OK;
}

struct Plan {
    std::vector<uint8_t> bytes;   // the work list
    mo_wl_header header;
};

// Wavefronts per workgroup of the Newton-Schulz GEMM kernels: bf16 products
// run on 8 (two per SIMD; tiles of full and half width), fp32 ones on 4 (one
// per SIMD; full, half and quarter width).
uint32_t gemm_waves(int32_t ns_dtype) { return ns_dtype == MO_BF16 ? 8u : 4u; }

double lr_factor(int64_t rows, int64_t cols, int32_t adjust) {
    if (adjust == MO_LR_ORIGINAL) return std::sqrt(std::max(1.0, double(rows) / double(cols)));
    if (adjust == MO_LR_MATCH_RMS_ADAMW) return 0.2 * std::sqrt(double(std::max(rows, cols)));
    return 1.0;
}

// Builds the work list (validated inputs only).  Layout documented in mo.h.
void build_plan(const mo_matrix* mats, int32_t n, const mo_muon_hparams* hp, Plan* plan) {
    const uint64_t T = MO_GEMM_TILE, MT = MO_MOM_TILE;
    const uint64_t es = hp->ns_dtype == MO_BF16 ? 2 : 4;
    std::vector<mo_wl_mat> recs;
    uint32_t mom_total = 0, max_partials = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mo_matrix& d = mats[i];
        if (d.rows == 0 || d.cols == 0) continue;
        mo_wl_mat r;
        std::memset(&r, 0, sizeof(r));
        const bool tr = d.rows > d.cols;
        r.W = reinterpret_cast<uint64_t>(d.W);
        r.G = reinterpret_cast<uint64_t>(d.G);
        r.M = reinterpret_cast<uint64_t>(d.M);
        r.U = reinterpret_cast<uint64_t>(d.update_out);
        r.ld_w = d.ld_w ? d.ld_w : d.cols;
        r.ld_g = d.ld_g ? d.ld_g : d.cols;
        r.ld_m = d.ld_m ? d.ld_m : d.cols;
        r.ld_u = d.ld_u ? d.ld_u : d.cols;
        r.rows = uint32_t(d.rows);
        r.cols = uint32_t(d.cols);
        r.m = uint32_t(std::min(d.rows, d.cols));
        r.n = uint32_t(std::max(d.rows, d.cols));
        r.m_pad = uint32_t(align_up(r.m, T));
        r.n_pad = uint32_t(align_up(r.n, T));
        r.flags = (tr ? MO_WLF_TRANSPOSED : 0u) | (d.update_out ? MO_WLF_HAS_UPDATE : 0u) |
                  (d.w_dtype == MO_BF16 ? MO_WLF_W_BF16 : 0u) |
                  (d.g_dtype == MO_BF16 ? MO_WLF_G_BF16 : 0u);
        r.desc_index = uint32_t(i);
        const uint32_t r_pad = tr ? r.n_pad : r.m_pad, c_pad = tr ? r.m_pad : r.n_pad;
        r.mom_tiles_c = uint32_t(c_pad / MT);
        r.n_partials = uint32_t((r_pad / MT) * (c_pad / MT));
        r.mom_begin = mom_total;
        mom_total += r.n_partials;
        max_partials = std::max(max_partials, r.n_partials);
        r.lr_eff = float(double(hp->lr) * lr_factor(d.rows, d.cols, hp->lr_adjust));
        r.decay = float(1.0 - double(hp->lr) * double(hp->weight_decay));
        recs.push_back(r);
    }
    const uint32_t nm = uint32_t(recs.size());

    // item lists
    struct Key { uint64_t work; uint32_t idx; };
    auto order = [&](auto work_of) {
        std::vector<Key> ks;
        for (uint32_t j = 0; j < nm; ++j) ks.push_back({work_of(recs[j]), j});
        std::stable_sort(ks.begin(), ks.end(),
                         [](const Key& a, const Key& b) { return a.work > b.work; });
        return ks;
    };
    auto upper = [&](const mo_wl_mat& r) { uint64_t t = r.m_pad / T; return t * (t + 1) / 2; };
    auto jobs = [&](const std::vector<Key>& mats_order, bool upper_only, bool k_is_n) {
        std::vector<mo_gemm_job> js;
        for (const Key& k : mats_order) {
            const mo_wl_mat& r = recs[k.idx];
            js.push_back({k.idx, uint32_t(r.m_pad / T), uint32_t((upper_only ? r.m_pad : r.n_pad) / T),
                          upper_only, k_is_n ? r.n_pad : r.m_pad});
        }
        return js;
    };
    // Dispatch lists: tiles to XCD queues (tile_dispatch.h).
    const uint32_t waves = gemm_waves(hp->ns_dtype), max_split = waves == 8 ? 2 : 4;
    std::vector<mo_wl_item> gram, poly, upd;
    mo_dispatch_tiles(jobs(order([&](const mo_wl_mat& r) { return upper(r) * r.n_pad; }), true, true), gram,
                      max_split);
    mo_dispatch_tiles(jobs(order([&](const mo_wl_mat& r) { return upper(r) * r.m_pad; }), true, false), poly,
                      max_split);
    mo_dispatch_tiles(jobs(order([&](const mo_wl_mat& r) {
                               return uint64_t(r.m_pad / T) * (r.n_pad / T) * r.m_pad; }), false, false),
                      upd, max_split);

    mo_wl_header h;
    std::memset(&h, 0, sizeof(h));
    h.magic = MO_WL_MAGIC;
    h.version = MO_WL_VERSION;
    h.n_mats = nm;
    h.ns_steps = uint32_t(hp->ns_steps);
    h.ns_dtype = uint32_t(hp->ns_dtype);
    h.gemm_tile = uint32_t(T);
    h.mom_tile = uint32_t(MT);
    h.elem_bytes = uint32_t(es);
    h.n_mom_items = mom_total;
    h.n_gram_items = uint32_t(gram.size());
    h.n_poly_items = uint32_t(poly.size());
    h.n_upd_items = uint32_t(upd.size());
    h.max_partials = max_partials;
    h.gemm_waves = waves;
    h.mats_offset = sizeof(mo_wl_header);
    h.gram_offset = align_up(h.mats_offset + uint64_t(nm) * sizeof(mo_wl_mat), MO_WS_ALIGN);
    h.poly_offset = align_up(h.gram_offset + gram.size() * sizeof(mo_wl_item), MO_WS_ALIGN);
    h.upd_offset = align_up(h.poly_offset + poly.size() * sizeof(mo_wl_item), MO_WS_ALIGN);
    h.wl_bytes = align_up(h.upd_offset + upd.size() * sizeof(mo_wl_item), MO_WS_ALIGN);
    h.ns_a = hp->ns_a;
    h.ns_b = hp->ns_b;
    h.ns_c = hp->ns_c;
    h.eps = hp->eps;

    // workspace regions, per matrix in descriptor order
    uint64_t off = h.wl_bytes;
    auto take = [&](uint64_t bytes) { uint64_t o = off; off = align_up(off + bytes, MO_WS_ALIGN); return o; };
    for (mo_wl_mat& r : recs) {
        const uint64_t mn = uint64_t(r.m_pad) * r.n_pad, mm = uint64_t(r.m_pad) * r.m_pad;
        r.off_X = take(mn * es);
        r.off_Xt0 = take(mn * es);
        r.off_Xt1 = take(mn * es);
        r.off_A = take(mm * es);
        r.off_B = take(mm * es);
        r.off_partials = take(uint64_t(r.n_partials) * 4);
        r.off_scale = take(16);
    }
    h.ws_bytes = off;

    plan->header = h;
    plan->bytes.assign(h.wl_bytes, 0);
    std::memcpy(plan->bytes.data(), &h, sizeof(h));
    if (nm) std::memcpy(plan->bytes.data() + h.mats_offset, recs.data(), nm * sizeof(mo_wl_mat));
    if (!gram.empty())
        std::memcpy(plan->bytes.data() + h.gram_offset, gram.data(), gram.size() * sizeof(mo_wl_item));
    if (!poly.empty())
        std::memcpy(plan->bytes.data() + h.poly_offset, poly.data(), poly.size() * sizeof(mo_wl_item));
    if (!upd.empty())
        std::memcpy(plan->bytes.data() + h.upd_offset, upd.data(), upd.size() * sizeof(mo_wl_item));
}

}  // namespace

namespace {

// The launches of one step on the uploaded work list at ws.
mo_status run_phases(const mo_wl_header& h, const mo_muon_hparams* hp, uint8_t* ws, hipStream_t s) {
    const float beta = hp->momentum;
    const int nest = hp->nesterov ? 1 : 0;
    if (timed_launch(MO_PHASE_MOMENTUM, s, [&] { return mo_launch_momentum(h, ws, beta, nest, s); }) != hipSuccess)
        return MO_ERR_HIP;
    if (timed_launch(MO_PHASE_NORM, s, [&] { return mo_launch_norm(h, ws, s); }) != hipSuccess)
        return MO_ERR_HIP;
    const int K = hp->ns_steps;
    if (K == 0) {
        if (timed_launch(MO_PHASE_APPLY, s, [&] { return mo_launch_apply(h, ws, s); }) != hipSuccess)
            return MO_ERR_HIP;
        return MO_OK;
    }
    int xt = 0;   // which transposed buffer holds the current X^T
    for (int k = 0; k < K; ++k) {
        const int first = k == 0, last = k == K - 1;
        if (timed_launch(MO_PHASE_GRAM, s, [&] { return mo_launch_gram(h, ws, first, xt, s); }) != hipSuccess)
            return MO_ERR_HIP;
        if (timed_launch(MO_PHASE_POLY, s, [&] { return mo_launch_poly(h, ws, s); }) != hipSuccess)
            return MO_ERR_HIP;
        if (timed_launch(last ? MO_PHASE_UPDATE_LAST : MO_PHASE_UPDATE, s,
                         [&] { return mo_launch_update(h, ws, first, last, xt, s); }) != hipSuccess)
            return MO_ERR_HIP;
        xt ^= 1;
    }
    return MO_OK;
}

}  // namespace

extern "C" {

const char* mo_status_string(mo_status st) {
    switch (st) {
        case MO_OK: return "MO_OK";
        case MO_ERR_INVALID_ARG: return "MO_ERR_INVALID_ARG: invalid argument";
        case MO_ERR_UNSUPPORTED: return "MO_ERR_UNSUPPORTED: unsupported dtype, option or size";
        case MO_ERR_WORKSPACE_TOO_SMALL: return "MO_ERR_WORKSPACE_TOO_SMALL: workspace too small";
        case MO_ERR_ALIAS: return "MO_ERR_ALIAS: overlapping tensors";
        case MO_ERR_HIP: return "MO_ERR_HIP: HIP runtime or launch failure";
        default: return "unknown mo_status";
    }
}

mo_status muon_workspace_bytes(const mo_matrix* mats, int32_t n, const mo_muon_hparams* hp,
                               size_t* bytes) {
    if (!bytes) return MO_ERR_INVALID_ARG;
    mo_status st = validate_hparams(hp);
    if (st != MO_OK) return st;
    if ((st = validate_mats(mats, n, nullptr)) != MO_OK) return st;
    Plan plan;
    build_plan(mats, n, hp, &plan);
    *bytes = size_t(plan.header.ws_bytes) + MO_WS_ALIGN;
    return MO_OK;
}

mo_status muon_build_worklist(const mo_matrix* mats, int32_t n, const mo_muon_hparams* hp,
                              void* host_buf, size_t* bytes_inout) {
    if (!bytes_inout) return MO_ERR_INVALID_ARG;
    mo_status st = validate_hparams(hp);
    if (st != MO_OK) return st;
    if ((st = validate_mats(mats, n, nullptr)) != MO_OK) return st;
    Plan plan;
    build_plan(mats, n, hp, &plan);
    if (!host_buf) {
        *bytes_inout = plan.bytes.size();
        return MO_OK;
    }
    if (*bytes_inout < plan.bytes.size()) return MO_ERR_INVALID_ARG;
    std::memcpy(host_buf, plan.bytes.data(), plan.bytes.size());
    *bytes_inout = plan.bytes.size();
    return MO_OK;
}

mo_status muon_owner_step(const mo_matrix* mats, int32_t n, const mo_muon_hparams* hp,
                          void* workspace, size_t workspace_bytes, void* stream) {
    mo_status st = validate_hparams(hp);
    if (st != MO_OK) return st;
    std::vector<Range> ranges;
    if ((st = validate_mats(mats, n, &ranges)) != MO_OK) return st;
    if (n == 0) return MO_OK;
    Plan plan;
    build_plan(mats, n, hp, &plan);
    const mo_wl_header& h = plan.header;
    if (h.n_mats == 0) return MO_OK;
    const size_t need = size_t(h.ws_bytes) + MO_WS_ALIGN;
    if (!workspace || workspace_bytes < need) return MO_ERR_WORKSPACE_TOO_SMALL;
    ranges.push_back(Range{reinterpret_cast<uintptr_t>(workspace),
                           reinterpret_cast<uintptr_t>(workspace) + workspace_bytes, 1});
    if (ranges_conflict(ranges)) return MO_ERR_ALIAS;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = reinterpret_cast<uint8_t*>(
        align_up(reinterpret_cast<uintptr_t>(workspace), MO_WS_ALIGN));
    if (upload(plan.bytes.data(), plan.bytes.size(), ws, s) != hipSuccess) return MO_ERR_HIP;
    return run_phases(h, hp, ws, s);
}

mo_status muon_owner_step_noalloc(const mo_matrix* mats, int32_t n, const mo_muon_hparams* hp,
                                  void* stream) {
    mo_status st = validate_hparams(hp);
    if (st != MO_OK) return st;
    std::vector<Range> ranges;
    if ((st = validate_mats(mats, n, &ranges)) != MO_OK) return st;
    if (n == 0) return MO_OK;
    Plan plan;
    build_plan(mats, n, hp, &plan);
    const mo_wl_header& h = plan.header;
    if (h.n_mats == 0) return MO_OK;
    // the array is 256-byte aligned, so no alignment slack is needed
    if (size_t(h.ws_bytes) > MO_NOALLOC_SCRATCH_BYTES) return MO_ERR_WORKSPACE_TOO_SMALL;
    void* scratch = nullptr;
    if (mo_static_scratch(&scratch) != hipSuccess) return MO_ERR_HIP;
    ranges.push_back(Range{reinterpret_cast<uintptr_t>(scratch),
                           reinterpret_cast<uintptr_t>(scratch) + MO_NOALLOC_SCRATCH_BYTES, 1});
    if (ranges_conflict(ranges)) return MO_ERR_ALIAS;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = reinterpret_cast<uint8_t*>(scratch);
    if (mo_launch_wl_upload(ws, plan.bytes.data(), plan.bytes.size(), s) != hipSuccess) return MO_ERR_HIP;
    return run_phases(h, hp, ws, s);
}

mo_status adamw_tail_step(float* p, const float* g, float* m, float* v, int64_t n, int64_t step,
                          float lr, float beta1, float beta2, float eps, float weight_decay,
                          void* stream) {
    if (n < 0 || step < 1) return MO_ERR_INVALID_ARG;
    if (!finite(lr) || !finite(beta1) || !finite(beta2) || !finite(eps) || !finite(weight_decay))
        return MO_ERR_INVALID_ARG;
    if (n == 0) return MO_OK;
    if (!p || !g || !m || !v) return MO_ERR_INVALID_ARG;
    std::vector<Range> rs = {matrix_range(p, 1, n, n, 4, 1), matrix_range(g, 1, n, n, 4, 0),
                             matrix_range(m, 1, n, n, 4, 1), matrix_range(v, 1, n, n, 4, 1)};
    if (ranges_conflict(rs)) return MO_ERR_ALIAS;
    // bias corrections in fp64 on the host
    const double bc1 = 1.0 - std::pow(double(beta1), double(step));
    const double bc2 = 1.0 - std::pow(double(beta2), double(step));
    const float step_size = float(double(lr) / bc1);
    const float inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));
    const float decay = float(1.0 - double(lr) * double(weight_decay));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (timed_launch(MO_PHASE_ADAMW, s, [&] {
            return mo_launch_adamw(p, g, m, v, n, decay, beta1, beta2, step_size, inv_sqrt_bc2, eps, s);
        }) != hipSuccess)
        return MO_ERR_HIP;
    return MO_OK;
}

mo_status mo_device_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (bytes == 0) return MO_OK;
    if (!dst || !src || (bytes % 16) || (reinterpret_cast<uintptr_t>(dst) % 16) ||
        (reinterpret_cast<uintptr_t>(src) % 16))
        return MO_ERR_INVALID_ARG;
    std::vector<Range> rs = {{reinterpret_cast<uintptr_t>(dst), reinterpret_cast<uintptr_t>(dst) + bytes, 1},
                             {reinterpret_cast<uintptr_t>(src), reinterpret_cast<uintptr_t>(src) + bytes, 0}};
    if (ranges_conflict(rs)) return MO_ERR_ALIAS;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (timed_launch(MO_PHASE_COPY, s, [&] { return mo_launch_copy(dst, src, bytes, s); }) != hipSuccess)
        return MO_ERR_HIP;
    return MO_OK;
}

}  // extern "C"
