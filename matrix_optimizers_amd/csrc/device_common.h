// Device-side primitives shared by the gfx950 kernels: element types, vector
// loads/stores, fp32 <-> bf16 conversion (round to nearest even, the hardware
// v_cvt_pk_bf16_f32), and wavefront/workgroup reductions in a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mo.h"
#include "mo_worklist.h"

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// native clang vectors (HIP's uint4/float4 are union-based classes that can
// defeat register promotion of arrays)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define MO_DEV __device__ __forceinline__

// ---- element conversion ---------------------------------------------------

MO_DEV float to_f32(bf16_t x) { return (float)x; }
MO_DEV float to_f32(float x) { return x; }

template <typename T> MO_DEV T from_f32(float x);
template <> MO_DEV float from_f32<float>(float x) { return x; }
template <> MO_DEV bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

// Round-trip through the storage type (what a later reader of the buffer sees).
template <typename T> MO_DEV float quantize(float x) { return to_f32(from_f32<T>(x)); }

// ---- 8-element chunks: 16 bytes of bf16 or 32 bytes of fp32 ------------------

struct f32x8 { float v[8]; };

MO_DEV void load8(const bf16_t* p, f32x8& o) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(p);
    bf16x8 b = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = (float)b[e];
}
MO_DEV void load8(const float* p, f32x8& o) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    o.v[0] = a[0]; o.v[1] = a[1]; o.v[2] = a[2]; o.v[3] = a[3];
    o.v[4] = b[0]; o.v[5] = b[1]; o.v[6] = b[2]; o.v[7] = b[3];
}
MO_DEV void store8(bf16_t* p, const f32x8& o) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16_t)o.v[e];
    *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, b);
}
MO_DEV void store8(float* p, const f32x8& o) {
    *reinterpret_cast<f32x4*>(p) = f32x4{o.v[0], o.v[1], o.v[2], o.v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{o.v[4], o.v[5], o.v[6], o.v[7]};
}

// Guarded element access for caller tensors of either dtype.
MO_DEV float load_elem(const void* base, int64_t idx, bool bf16) {
    return bf16 ? (float)reinterpret_cast<const bf16_t*>(base)[idx]
                : reinterpret_cast<const float*>(base)[idx];
}
MO_DEV void store_elem(void* base, int64_t idx, float v, bool bf16) {
    if (bf16) reinterpret_cast<bf16_t*>(base)[idx] = (bf16_t)v;
    else reinterpret_cast<float*>(base)[idx] = v;
}

// ---- reductions ----------------------------------------------------------------

// Butterfly sum over the 64 lanes of a wavefront; every lane gets the total.
// The pairing pattern is fixed, so the result is bit-reproducible.
MO_DEV float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over a workgroup of NT threads (NT a multiple of 64); result valid in
// thread 0.  `red` must hold NT/64 floats of LDS.  Waves are combined in index
// order, so the value is bit-reproducible.
template <int NT>
MO_DEV float block_sum(float x, float* red) {
    x = wave_sum(x);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = x;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) t += red[w];
    }
    return t;
}

// ---- work list access ------------------------------------------------------------

MO_DEV const mo_wl_header* wl_header(const uint8_t* ws) {
    return reinterpret_cast<const mo_wl_header*>(ws);
}
MO_DEV const mo_wl_mat* wl_mats(const uint8_t* ws) {
    return reinterpret_cast<const mo_wl_mat*>(ws + wl_header(ws)->mats_offset);
}
