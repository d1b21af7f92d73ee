// Read-bandwidth probe for the measurement harness (bench.py --read-ceiling); not part
// of the GEMV library. Two kinds of kernel, both with no arithmetic beyond an XOR
// that keeps the loads alive:
//  - the row walk: the GEMV's own load form -- 16-byte non-temporal buffer loads, 1 KB
//    per wave instruction, one buffer descriptor per row -- over 4 KB rows walked the
//    way the GEMV walks its rows (wave w takes rows w, w + waves, ...), DEPTH rows in
//    flight per wave;
//  - plain streams that share nothing with the GEMV's form: the buffer is cut into
//    tiles of 64 * W * U bytes, wave w reads tiles w, w + waves, ..., each lane U
//    loads of W bytes (4, 8 or 16) at lane-contiguous offsets, by buffer loads or by
//    global loads, with the non-temporal or the default cache policy.
// The best time over forms and launch shapes for a size is the read ceiling the GEMV
// of that many bytes is compared with.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t ROW = 4096;       // bytes per row: 4 loads of 16 B per lane
constexpr int WG = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t *p, uint32_t r,
                                                         uint32_t nrows)
{
    // rows past the end get an empty descriptor: their loads return zeros
    const bool real = r < nrows;
    return __builtin_amdgcn_make_buffer_rsrc((void *)(p + (size_t)(real ? r : 0u) * ROW),
                                             (short)0, real ? (int)ROW : 0, 0x00020000);
}

template <int DEPTH>
__global__ __launch_bounds__(WG) void read_rows(const uint8_t *__restrict__ p, uint32_t nrows,
                                                uint32_t *__restrict__ sink)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * (WG / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * (WG / 64);
    uint32_t acc = 0;
    for (uint32_t r0 = wave; r0 < nrows; r0 += nw * DEPTH) {
        u32x4 v[DEPTH][4];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const __amdgpu_buffer_rsrc_t rs = row_rsrc(p, r0 + (uint32_t)d * nw, nrows);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                v[d][c] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(1024u * c + 16u * lane), 0, 2);
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc ^= v[d][c].x ^ v[d][c].y ^ v[d][c].z ^ v[d][c].w;
    }
    // a store no input makes (the XOR of random bytes equals this word with
    // probability 2^-32; sink must hold WG words)
    if (acc == 0x9E3779B9u)
        sink[threadIdx.x] = acc;
}

// Plain stream forms.
enum StreamForm : int { BUF_NT = 0, BUF_DEFAULT = 1, GLOBAL_NT = 2, GLOBAL_DEFAULT = 3 };

template <int FORM, int W>
__device__ __forceinline__ uint32_t load_fold(__amdgpu_buffer_rsrc_t rs, const uint8_t *p,
                                              uint32_t off)
{
    constexpr int POL = FORM == BUF_NT ? 2 : 0;
    if constexpr (FORM == BUF_NT || FORM == BUF_DEFAULT) {
        if constexpr (W == 16) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, POL);
            return v.x ^ v.y ^ v.z ^ v.w;
        } else if constexpr (W == 8) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, POL);
            return v.x ^ v.y;
        } else {
            return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, POL);
        }
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        if constexpr (W == 16) {
            const u32x4 *q = reinterpret_cast<const u32x4 *>(p + off);
            u32x4 v;
            if constexpr (FORM == GLOBAL_NT)
                v = __builtin_nontemporal_load(q);
            else
                v = *q;
            return v.x ^ v.y ^ v.z ^ v.w;
        } else if constexpr (W == 8) {
            const u32x2 *q = reinterpret_cast<const u32x2 *>(p + off);
            u32x2 v;
            if constexpr (FORM == GLOBAL_NT)
                v = __builtin_nontemporal_load(q);
            else
                v = *q;
            return v.x ^ v.y;
        } else {
            const uint32_t *q = reinterpret_cast<const uint32_t *>(p + off);
            if constexpr (FORM == GLOBAL_NT)
                return __builtin_nontemporal_load(q);
            else
                return *q;
        }
    }
}

// Tiles of 64 * W * U bytes; ntiles = nbytes / tile (the host passes whole tiles), so
// the last byte read is ntiles * tile - 1 < nbytes.
template <int FORM, int W, int U>
__global__ __launch_bounds__(WG) void read_stream(const uint8_t *__restrict__ p, uint32_t ntiles,
                                                  uint32_t *__restrict__ sink)
{
    constexpr uint32_t TILE = 64u * W * U;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * (WG / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * (WG / 64);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, (int)(ntiles * TILE), 0x00020000);
    uint32_t acc = 0;
    for (uint32_t t = wave; t < ntiles; t += nw) {
        uint32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load_fold<FORM, W>(rs, p, t * TILE + ((uint32_t)u * 64u + lane) * W);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u];
    }
    if (acc == 0x9E3779B9u)
        sink[threadIdx.x] = acc;
}

template <int FORM, int W>
hipError_t launch_stream(int unroll, const uint8_t *p, uint32_t nbytes, int grid, uint32_t *sink,
                         hipStream_t s)
{
    switch (unroll) {
    case 4: hipLaunchKernelGGL((read_stream<FORM, W, 4>), dim3(grid), dim3(WG), 0, s, p,
                               nbytes / (64u * W * 4u), sink); break;
    case 8: hipLaunchKernelGGL((read_stream<FORM, W, 8>), dim3(grid), dim3(WG), 0, s, p,
                               nbytes / (64u * W * 8u), sink); break;
    default: hipLaunchKernelGGL((read_stream<FORM, W, 16>), dim3(grid), dim3(WG), 0, s, p,
                                nbytes / (64u * W * 16u), sink); break;
    }
    return hipGetLastError();
}

template <int FORM>
hipError_t launch_form(int width, int unroll, const uint8_t *p, uint32_t nbytes, int grid,
                       uint32_t *sink, hipStream_t s)
{
    switch (width) {
    case 4: return launch_stream<FORM, 4>(unroll, p, nbytes, grid, sink, s);
    case 8: return launch_stream<FORM, 8>(unroll, p, nbytes, grid, sink, s);
    default: return launch_stream<FORM, 16>(unroll, p, nbytes, grid, sink, s);
    }
}

}  // namespace

extern "C" {

// Streams nbytes / 4096 whole rows of buf (device, 16-B aligned) with `depth` (1..4)
// rows in flight per wave on `grid` workgroups of 256 threads, on `stream`. sink: 256
// device words, written only with probability 2^-32. Returns 0, -1 on bad arguments,
// -2 if the launch fails.
int q6k_read_probe(const void *buf, int64_t nbytes, int depth, int grid, uint32_t *sink,
                   void *stream)
{
    if (!buf || !sink || nbytes < (int64_t)ROW || nbytes / ROW > 0xFFFFFFFFll || grid < 1 ||
        depth < 1 || depth > 4 || (reinterpret_cast<uintptr_t>(buf) & 15u))
        return -1;
    const uint32_t nrows = (uint32_t)(nbytes / ROW);
    const uint8_t *p = static_cast<const uint8_t *>(buf);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (depth) {
    case 1: hipLaunchKernelGGL(read_rows<1>, dim3(grid), dim3(WG), 0, s, p, nrows, sink); break;
    case 2: hipLaunchKernelGGL(read_rows<2>, dim3(grid), dim3(WG), 0, s, p, nrows, sink); break;
    case 3: hipLaunchKernelGGL(read_rows<3>, dim3(grid), dim3(WG), 0, s, p, nrows, sink); break;
    default: hipLaunchKernelGGL(read_rows<4>, dim3(grid), dim3(WG), 0, s, p, nrows, sink); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Streams the first nbytes of buf (device, 16-B aligned) in the plain form `form`
// (0 buffer loads, non-temporal; 1 buffer loads, default policy; 2 global loads,
// non-temporal; 3 global loads, default policy), `width` bytes per lane and load (4,
// 8 or 16), `unroll` loads in flight per lane (4, 8 or 16), on `grid` workgroups of
// 256 threads, on `stream`. nbytes must be a multiple of 65536 (so every tile is whole)
// and below 2^32. sink: 256 device words, written only with probability 2^-32.
// Returns 0, -1 on bad arguments, -2 if the launch fails.
int q6k_read_probe_stream(const void *buf, int64_t nbytes, int form, int width, int unroll,
                          int grid, uint32_t *sink, void *stream)
{
    if (!buf || !sink || nbytes < 65536 || nbytes % 65536 || nbytes >= (1ll << 32) || grid < 1 ||
        form < 0 || form > 3 || (width != 4 && width != 8 && width != 16) ||
        (unroll != 4 && unroll != 8 && unroll != 16) ||
        (reinterpret_cast<uintptr_t>(buf) & 15u))
        return -1;
    const uint8_t *p = static_cast<const uint8_t *>(buf);
    const uint32_t n = (uint32_t)nbytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (form) {
    case BUF_NT: e = launch_form<BUF_NT>(width, unroll, p, n, grid, sink, s); break;
    case BUF_DEFAULT: e = launch_form<BUF_DEFAULT>(width, unroll, p, n, grid, sink, s); break;
    case GLOBAL_NT: e = launch_form<GLOBAL_NT>(width, unroll, p, n, grid, sink, s); break;
    default: e = launch_form<GLOBAL_DEFAULT>(width, unroll, p, n, grid, sink, s); break;
    }
    return e == hipSuccess ? 0 : -2;
}

}  // extern "C"
