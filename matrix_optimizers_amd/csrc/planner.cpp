// Owner planner: which data-parallel rank owns each role.
//
// [P] = "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
// parameter sharding".  Each FSDP block is converted into roles, one per 2D
// matrix plus one packed tail of its non-2D tensors (§3, §4.1); a global greedy
// over owner-resident numel assigns the roles to ranks (§4.1).  RoleGreedy is
// the memory-conservative default, ScopeGreedy pools the roles of all blocks,
// CostAware takes the scope plan only within a cap on its per-block owner
// shares; the scorer reports per-rank load and the per-block owner imbalance
// gamma_B and materialization volume of §4.2.  The pages do not print the
// algorithm; the readings are stated with each entry point in mo.h.
#include <algorithm>
#include <cstring>
#include <map>
#include <utility>
#include <vector>

#include "../../include/mo.h"

namespace {

constexpr int64_t MAX_SIDE = int64_t(1) << 31;   // keeps rows * cols inside int64

bool valid_roles(const mo_role* roles, int32_t n, int32_t world) {
    if (n < 0 || world < 1) return false;
    if (n > 0 && roles == nullptr) return false;
    for (int32_t i = 0; i < n; ++i) {
        const mo_role& r = roles[i];
        if (r.block < 0 || r.rows < 0 || r.cols < 0 || r.rows >= MAX_SIDE || r.cols >= MAX_SIDE) return false;
        if (r.kind == MO_ROLE_TAIL) {
            if (r.cols != 1) return false;
        } else if (r.kind != MO_ROLE_MATRIX) {
            return false;
        }
    }
    return true;
}

bool valid_owners(const int32_t* owner, int32_t n, int32_t world) {
    if (n > 0 && owner == nullptr) return false;
    for (int32_t i = 0; i < n; ++i)
        if (owner[i] < 0 || owner[i] >= world) return false;
    return true;
}

int64_t numel(const mo_role& r) { return r.rows * r.cols; }

// Roles of `idx` by decreasing numel; equal numel keeps the given order.
std::vector<int32_t> by_numel(std::vector<int32_t> idx, const mo_role* roles) {
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int32_t a, int32_t b) { return numel(roles[a]) > numel(roles[b]); });
    return idx;
}

// Each role in `order` goes to the rank with the least numel so far (ties:
// the lowest rank); `load` carries over between calls.
void assign(const std::vector<int32_t>& order, const mo_role* roles, std::vector<int64_t>& load,
            int32_t* owner) {
    for (int32_t i : order) {
        size_t x = 0;
        for (size_t y = 1; y < load.size(); ++y)
            if (load[y] < load[x]) x = y;
        owner[i] = int32_t(x);
        load[x] += numel(roles[i]);
    }
}

void role_greedy(const mo_role* roles, int32_t n, int32_t world, int32_t* owner) {
    std::map<int32_t, std::vector<int32_t>> blocks;   // increasing block index
    for (int32_t i = 0; i < n; ++i) blocks[roles[i].block].push_back(i);
    std::vector<int64_t> load(size_t(world), 0);
    for (auto& kv : blocks) assign(by_numel(kv.second, roles), roles, load, owner);
}

void scope_greedy(const mo_role* roles, int32_t n, int32_t world, int32_t* owner) {
    std::vector<int32_t> all(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) all[size_t(i)] = i;
    std::vector<int64_t> load(size_t(world), 0);
    assign(by_numel(all, roles), roles, load, owner);
}

// max over blocks B and ranks r of the numel rank r owns in block B
int64_t block_peak(const mo_role* roles, int32_t n, const int32_t* owner) {
    std::map<std::pair<int32_t, int32_t>, int64_t> share;
    int64_t peak = 0;
    for (int32_t i = 0; i < n; ++i) {
        int64_t& v = share[{roles[i].block, owner[i]}];
        v += numel(roles[i]);
        peak = std::max(peak, v);
    }
    return peak;
}

}  // namespace

extern "C" {

mo_status mo_plan_owners(const mo_role* roles, int32_t n_roles, int32_t world, int32_t policy,
                         int64_t block_cap, int32_t* owner_out) {
    if (!valid_roles(roles, n_roles, world) || block_cap < 0) return MO_ERR_INVALID_ARG;
    if (policy != MO_PLAN_ROLE_GREEDY && policy != MO_PLAN_SCOPE_GREEDY && policy != MO_PLAN_COST_AWARE)
        return MO_ERR_INVALID_ARG;
    if (n_roles == 0) return MO_OK;
    if (owner_out == nullptr) return MO_ERR_INVALID_ARG;
    if (policy == MO_PLAN_ROLE_GREEDY) {
        role_greedy(roles, n_roles, world, owner_out);
    } else if (policy == MO_PLAN_SCOPE_GREEDY) {
        scope_greedy(roles, n_roles, world, owner_out);
    } else {
        std::vector<int32_t> scope(static_cast<size_t>(n_roles)), role(static_cast<size_t>(n_roles));
        scope_greedy(roles, n_roles, world, scope.data());
        role_greedy(roles, n_roles, world, role.data());
        const int64_t cap = block_cap > 0 ? block_cap : block_peak(roles, n_roles, role.data());
        const std::vector<int32_t>& pick = block_peak(roles, n_roles, scope.data()) <= cap ? scope : role;
        std::memcpy(owner_out, pick.data(), sizeof(int32_t) * size_t(n_roles));
    }
    return MO_OK;
}

mo_status mo_plan_score(const mo_role* roles, int32_t n_roles, int32_t world, const int32_t* owner,
                        double* rank_numel, double* rank_flops, int32_t n_blocks,
                        double* block_gamma, double* block_owner_comm) {
    if (!valid_roles(roles, n_roles, world) || !valid_owners(owner, n_roles, world)) return MO_ERR_INVALID_ARG;
    if (rank_numel == nullptr || rank_flops == nullptr || n_blocks < 0) return MO_ERR_INVALID_ARG;
    const bool per_block = block_gamma != nullptr || block_owner_comm != nullptr;
    for (int32_t i = 0; i < n_roles; ++i)
        if (per_block && roles[i].block >= n_blocks) return MO_ERR_INVALID_ARG;
    for (int32_t r = 0; r < world; ++r) rank_numel[r] = rank_flops[r] = 0.0;
    std::vector<double> total(per_block ? size_t(n_blocks) : 0, 0.0);
    std::map<std::pair<int32_t, int32_t>, double> share;
    for (int32_t i = 0; i < n_roles; ++i) {
        const mo_role& ro = roles[i];
        const double e = double(numel(ro));
        rank_numel[owner[i]] += e;
        if (ro.kind == MO_ROLE_MATRIX) {
            const double m = double(std::min(ro.rows, ro.cols)), nn = double(std::max(ro.rows, ro.cols));
            rank_flops[owner[i]] += 4.0 * m * m * nn + 2.0 * m * m * m;
        }
        if (per_block) {
            total[size_t(ro.block)] += e;
            share[{ro.block, owner[i]}] += e;
        }
    }
    if (!per_block) return MO_OK;
    std::vector<double> peak(size_t(n_blocks), 0.0);
    for (const auto& kv : share) peak[size_t(kv.first.first)] = std::max(peak[size_t(kv.first.first)], kv.second);
    for (int32_t b = 0; b < n_blocks; ++b) {
        if (block_gamma)
            block_gamma[b] = total[size_t(b)] > 0 ? peak[size_t(b)] / (total[size_t(b)] / double(world)) : 0.0;
        if (block_owner_comm) block_owner_comm[b] = double(world - 1) * peak[size_t(b)];
    }
    return MO_OK;
}

mo_status mo_plan_layout(const mo_role* roles, int32_t n_roles, int32_t world, const int32_t* owner,
                         int64_t* offset_out) {
    if (!valid_roles(roles, n_roles, world) || !valid_owners(owner, n_roles, world)) return MO_ERR_INVALID_ARG;
    if (n_roles > 0 && offset_out == nullptr) return MO_ERR_INVALID_ARG;
    std::map<std::pair<int32_t, int32_t>, int64_t> cursor;   // (block, rank) -> next free element
    for (int32_t i = 0; i < n_roles; ++i) {
        int64_t& c = cursor[{roles[i].block, owner[i]}];
        offset_out[i] = c;
        c += numel(roles[i]);
    }
    return MO_OK;
}

}  // extern "C"
