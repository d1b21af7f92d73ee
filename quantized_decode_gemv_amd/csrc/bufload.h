// bufload.h -- raw buffer loads (gfx950) used by the GEMV kernels.
//
// A buffer descriptor bounds every load by its extent: a load whose bytes fall
// past it returns zeros without a memory request. Streamed weight planes are read
// with the non-temporal policy (each byte is read once per call); small shared
// fields keep the default policy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q6k {

constexpr int POLICY_STREAM = 2;    // buffer-load cache policy: non-temporal
constexpr int POLICY_DEFAULT = 0;
constexpr int DESC_WORD3 = 0x00020000;  // raw buffer, 32-bit format fields unused

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3v __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// Descriptor of `extent` bytes at p (0: every load returns zeros, no request).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_desc(const void *p, uint32_t extent)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, (int)extent, DESC_WORD3);
}

// Loads with cache policy POLICY, vector loads returned as plain structs (elements are copied into integers: a bit
// cast applied straight to a vector element reads element 0).
template <int POLICY>
__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int POLICY>
__device__ __forceinline__ uint3 load_b96(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x3v v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, POLICY);
    return make_uint3(v.x, v.y, v.z);
}

template <int POLICY>
__device__ __forceinline__ uint2 load_b64(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POLICY);
    return make_uint2(v.x, v.y);
}

template <int POLICY>
__device__ __forceinline__ uint32_t load_b32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POLICY);
}

template <int POLICY>
__device__ __forceinline__ uint32_t load_b16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, POLICY);
}

}  // namespace q6k
