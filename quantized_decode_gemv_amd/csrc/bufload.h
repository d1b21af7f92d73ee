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

namespace q6k {

// One wave instruction that copies 16 bytes per lane, from buffer offset voff + soff,
// into LDS at lds + 16 * lane (a buffer load whose destination is LDS, non-temporal
// like the streamed planes). The LDS base travels in M0, which the compiler loads
// for the statement. The compiler does not count this load: a caller waits for it
// with vm_wait before reading the bytes from LDS, and issues no LDS reads of the
// destination that could be served before it.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         uint32_t lds)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(lds)
                 : "memory");
}

// Waits until at most N vector memory instructions of this wave are outstanding.
// Loads complete in issue order, so after the wait every load issued before the
// last N vector memory instructions has completed (stores only add to the count).
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace q6k
