// gfx950 kernels for the packed non-2D tail (AdamW) and the copy used to
// calibrate HBM byte counters.
//
// [P] = "MatrixFSDP: communication-free matrix optimizers under ZeRO-3 parameter
// sharding", §3: the non-matrix tensors of a unit are packed into one tail role
// kept on the AdamW path; §5.1 gives lr, weight decay, betas and eps.  The
// update is decoupled-weight-decay Adam; AdamW is coordinate-wise, so one flat
// pass over the packed tail is the whole step.  HBM-bound: 16 bytes read and
// 12 bytes written per element.
#include "device_common.h"
#include "mo_kernels.h"

namespace {

constexpr int TAIL_THREADS = 256;

struct AdamWArgs {
    float decay, beta1, beta2, step_size, inv_sqrt_bc2, eps;
};

MO_DEV void adamw_one(float& p, float g, float& m, float& v, const AdamWArgs& a) {
    const float mn = a.beta1 * m + (1.0f - a.beta1) * g;
    const float vn = a.beta2 * v + (1.0f - a.beta2) * g * g;
    const float denom = sqrtf(vn) * a.inv_sqrt_bc2 + a.eps;
    p = p * a.decay - a.step_size * mn / denom;
    m = mn;
    v = vn;
}

// Two 16-byte groups of 4 elements per thread per iteration, one workgroup
// width apart (so each instruction of a wave covers 1 KB contiguous), all
// loads issued before any store; streaming (non-temporal) accesses, since
// nothing here is read again soon.  Grid-stride; a last partial group goes
// one 16-byte access per thread, and the ragged end (n % 4) element-wise.
MO_DEV f32x4 ld_nt(const f32x4* p) { return __builtin_nontemporal_load(p); }
MO_DEV void st_nt(f32x4* p, const f32x4& v) { __builtin_nontemporal_store(v, p); }
MO_DEV void adamw4(f32x4& p, const f32x4& g, f32x4& m, f32x4& v, const AdamWArgs& a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float pe = p[e], me = m[e], ve = v[e];
        adamw_one(pe, g[e], me, ve, a);
        p[e] = pe; m[e] = me; v[e] = ve;
    }
}

__global__ __launch_bounds__(TAIL_THREADS) void adamw_vec_kernel(float* __restrict__ p,
                                                                 const float* __restrict__ g,
                                                                 float* __restrict__ m,
                                                                 float* __restrict__ v,
                                                                 int64_t n, AdamWArgs a) {
    const int64_t n4 = n >> 2;
    const int64_t stride = int64_t(gridDim.x) * TAIL_THREADS * 2;
    f32x4* p4 = reinterpret_cast<f32x4*>(p);
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    f32x4* v4 = reinterpret_cast<f32x4*>(v);
    int64_t i = int64_t(blockIdx.x) * TAIL_THREADS * 2 + threadIdx.x;
    for (; i + TAIL_THREADS < n4; i += stride) {
        f32x4 pp[2], gg[2], mm[2], vv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t j = i + h * TAIL_THREADS;
            pp[h] = ld_nt(p4 + j);
            gg[h] = ld_nt(g4 + j);
            mm[h] = ld_nt(m4 + j);
            vv[h] = ld_nt(v4 + j);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t j = i + h * TAIL_THREADS;
            adamw4(pp[h], gg[h], mm[h], vv[h], a);
            st_nt(p4 + j, pp[h]);
            st_nt(m4 + j, mm[h]);
            st_nt(v4 + j, vv[h]);
        }
    }
    if (i < n4) {   // this thread's share of the last, partial group
        f32x4 pp = p4[i], mm = m4[i], vv = v4[i];
        adamw4(pp, g4[i], mm, vv, a);
        p4[i] = pp; m4[i] = mm; v4[i] = vv;
    }
    if (blockIdx.x == 0) {
        const int64_t k = (n4 << 2) + threadIdx.x;
        if (k < n) {
            float pp = p[k], mm = m[k], vv = v[k];
            adamw_one(pp, g[k], mm, vv, a);
            p[k] = pp; m[k] = mm; v[k] = vv;
        }
    }
}

__global__ __launch_bounds__(TAIL_THREADS) void adamw_scalar_kernel(float* p, const float* g,
                                                                    float* m, float* v, int64_t n,
                                                                    AdamWArgs a) {
    const int64_t stride = int64_t(gridDim.x) * TAIL_THREADS;
    for (int64_t i = int64_t(blockIdx.x) * TAIL_THREADS + threadIdx.x; i < n; i += stride) {
        float pp = p[i], mm = m[i], vv = v[i];
        adamw_one(pp, g[i], mm, vv, a);
        p[i] = pp; m[i] = mm; v[i] = vv;
    }
}

// 4 x 16 bytes per thread per iteration, loads before stores, streaming
// accesses: the pattern that measured fastest on MI355X among simple copies.
__global__ __launch_bounds__(TAIL_THREADS) void copy_kernel(u32x4* __restrict__ dst,
                                                            const u32x4* __restrict__ src,
                                                            int64_t n16) {
    const int64_t stride = int64_t(gridDim.x) * TAIL_THREADS * 4;
    int64_t i = int64_t(blockIdx.x) * TAIL_THREADS * 4 + threadIdx.x;
    for (; i + 3 * TAIL_THREADS < n16; i += stride) {
        u32x4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load(src + i + u * TAIL_THREADS);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(x[u], dst + i + u * TAIL_THREADS);
    }
    for (; i < n16; i += TAIL_THREADS) dst[i] = src[i];   // the last, partial group
}

// Workgroups for a grid-stride pass over `units` per-thread items: one
// workgroup per TAIL_THREADS items, up to 131072 (2^28 AdamW elements in one
// pass).  Looping a smaller grid over the data measured slower from 2^27
// elements on: at a cap of 16384 the AdamW pass fell to 0.69-0.67 of HBM at
// 2^27-2^28 elements, at this cap it holds 0.73.
inline unsigned stream_grid(int64_t units) {
    const int64_t want = (units + TAIL_THREADS - 1) / TAIL_THREADS;
    return unsigned(want < 1 ? 1 : (want > 131072 ? 131072 : want));
}

}  // namespace

hipError_t mo_launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float decay,
                           float beta1, float beta2, float step_size, float inv_sqrt_bc2,
                           float eps, hipStream_t s) {
    AdamWArgs a{decay, beta1, beta2, step_size, inv_sqrt_bc2, eps};
    const bool aligned = ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g) |
                           reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v)) & 15) == 0;
    if (aligned)
        hipLaunchKernelGGL(adamw_vec_kernel, dim3(stream_grid((n + 7) / 8)), dim3(TAIL_THREADS), 0, s,
                           p, g, m, v, n, a);
    else
        hipLaunchKernelGGL(adamw_scalar_kernel, dim3(stream_grid(n)), dim3(TAIL_THREADS), 0, s,
                           p, g, m, v, n, a);
    return hipGetLastError();
}

hipError_t mo_launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
    const int64_t n16 = int64_t(bytes / 16);
    hipLaunchKernelGGL(copy_kernel, dim3(stream_grid((n16 + 3) / 4)), dim3(TAIL_THREADS), 0, s,
                       reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), n16);
    return hipGetLastError();
}
