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

// 4 elements per thread per iteration with 16-byte accesses (all four tensors
// 16-byte aligned), grid-stride; the ragged end is handled element-wise.
__global__ __launch_bounds__(TAIL_THREADS) void adamw_vec_kernel(float* __restrict__ p,
                                                                 const float* __restrict__ g,
                                                                 float* __restrict__ m,
                                                                 float* __restrict__ v,
                                                                 int64_t n, AdamWArgs a) {
    const int64_t n4 = n >> 2;
    const int64_t stride = int64_t(gridDim.x) * TAIL_THREADS;
    for (int64_t i = int64_t(blockIdx.x) * TAIL_THREADS + threadIdx.x; i < n4; i += stride) {
        float4 pp = reinterpret_cast<float4*>(p)[i];
        const float4 gg = reinterpret_cast<const float4*>(g)[i];
        float4 mm = reinterpret_cast<float4*>(m)[i];
        float4 vv = reinterpret_cast<float4*>(v)[i];
        adamw_one(pp.x, gg.x, mm.x, vv.x, a);
        adamw_one(pp.y, gg.y, mm.y, vv.y, a);
        adamw_one(pp.z, gg.z, mm.z, vv.z, a);
        adamw_one(pp.w, gg.w, mm.w, vv.w, a);
        reinterpret_cast<float4*>(p)[i] = pp;
        reinterpret_cast<float4*>(m)[i] = mm;
        reinterpret_cast<float4*>(v)[i] = vv;
    }
    const int64_t tail = n4 << 2;
    const int64_t k = tail + int64_t(blockIdx.x) * TAIL_THREADS + threadIdx.x;
    if (blockIdx.x == 0 && k < n) {
        float pp = p[k], mm = m[k], vv = v[k];
        adamw_one(pp, g[k], mm, vv, a);
        p[k] = pp; m[k] = mm; v[k] = vv;
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

__global__ __launch_bounds__(TAIL_THREADS) void copy_kernel(uint4* __restrict__ dst,
                                                            const uint4* __restrict__ src,
                                                            int64_t n16) {
    const int64_t stride = int64_t(gridDim.x) * TAIL_THREADS;
    for (int64_t i = int64_t(blockIdx.x) * TAIL_THREADS + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

// enough workgroups to keep every CU streaming (256 CUs x 8), capped by the work
inline unsigned stream_grid(int64_t units) {
    const int64_t want = (units + TAIL_THREADS - 1) / TAIL_THREADS;
    return unsigned(want < 1 ? 1 : (want > 2048 ? 2048 : want));
}

}  // namespace

hipError_t mo_launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float decay,
                           float beta1, float beta2, float step_size, float inv_sqrt_bc2,
                           float eps, hipStream_t s) {
    AdamWArgs a{decay, beta1, beta2, step_size, inv_sqrt_bc2, eps};
    const bool aligned = ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g) |
                           reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v)) & 15) == 0;
    if (aligned)
        hipLaunchKernelGGL(adamw_vec_kernel, dim3(stream_grid((n + 3) / 4)), dim3(TAIL_THREADS), 0, s,
                           p, g, m, v, n, a);
    else
        hipLaunchKernelGGL(adamw_scalar_kernel, dim3(stream_grid(n)), dim3(TAIL_THREADS), 0, s,
                           p, g, m, v, n, a);
    return hipGetLastError();
}

hipError_t mo_launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
    const int64_t n16 = int64_t(bytes / 16);
    hipLaunchKernelGGL(copy_kernel, dim3(stream_grid(n16)), dim3(TAIL_THREADS), 0, s,
                       reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n16);
    return hipGetLastError();
}
