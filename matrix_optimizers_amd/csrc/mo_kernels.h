// Host-side launchers of the gfx950 kernels (defined in the .hip files).
// Each returns the status of its launch; arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mo.h"
#include "mo_worklist.h"

// `ws` is the 256-byte-aligned workspace base; the work list sits at ws[0].
hipError_t mo_launch_momentum(const mo_wl_header& h, uint8_t* ws, float beta, int nesterov,
                              hipStream_t s);
hipError_t mo_launch_norm(const mo_wl_header& h, uint8_t* ws, hipStream_t s);
hipError_t mo_launch_gram(const mo_wl_header& h, uint8_t* ws, int first, int xt_cur,
                          hipStream_t s);
hipError_t mo_launch_poly(const mo_wl_header& h, uint8_t* ws, hipStream_t s);
hipError_t mo_launch_update(const mo_wl_header& h, uint8_t* ws, int first, int last, int xt_cur,
                            hipStream_t s);
hipError_t mo_launch_apply(const mo_wl_header& h, uint8_t* ws, hipStream_t s);
hipError_t mo_launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float decay,
                           float beta1, float beta2, float step_size, float inv_sqrt_bc2,
                           float eps, hipStream_t s);
hipError_t mo_launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

// Allocation-free Muon step (static_scratch.hip): this device's static scratch
// array (MO_NOALLOC_SCRATCH_BYTES), and a work-list upload carried in kernel
// arguments.
hipError_t mo_static_scratch(void** ptr);
hipError_t mo_launch_wl_upload(uint8_t* dst, const uint8_t* src, size_t bytes, hipStream_t s);

// Shampoo step (shampoo_kernels.hip); `ws` holds the Shampoo work list.
struct mo_sh_header;
hipError_t mo_launch_sh_layout(const mo_sh_header& h, uint8_t* ws, hipStream_t s);
hipError_t mo_launch_sh_rootprep(const mo_sh_header& h, uint8_t* ws, hipStream_t s);
hipError_t mo_launch_sh_gemm(const mo_sh_header& h, uint8_t* ws, int list, int k, hipStream_t s);

// SOAP step (soap_kernels.hip); `ws` holds the SOAP work list.
struct mo_so_header;
struct mo_so_mat;
struct mo_so_eig;
hipError_t mo_launch_so_prep(const mo_so_mat& mt, uint8_t* ws, uint32_t mi, hipStream_t s);
hipError_t mo_launch_so_gemm(const mo_so_mat& mt, uint8_t* ws, uint32_t mi, int kind, hipStream_t s);
hipError_t mo_launch_so_eig_init(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, int warm, hipStream_t s);
hipError_t mo_launch_so_warm(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, int kind, hipStream_t s);
hipError_t mo_launch_so_norm(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, hipStream_t s);
hipError_t mo_launch_so_solve(const mo_so_header& h, uint8_t* ws, uint32_t k, hipStream_t s);
hipError_t mo_launch_so_rotate(const mo_so_header& h, uint8_t* ws, uint32_t k, hipStream_t s);
hipError_t mo_launch_so_rank(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, hipStream_t s);
hipError_t mo_launch_so_gather(const mo_so_eig& eg, uint8_t* ws, uint32_t ei, hipStream_t s);
