// repack.hip -- raw GGUF k-quant rows -> split-plane rows, on the device and on the
// host, for every type of kq_format.h.
//
// A byte permutation: for row r and super-block b, each field of the block is
// copied to its plane (for q6_K the permutation of D4-4 §3.2 Excerpt A: bytes
// [0,128) to the ql plane at b*128, [128,192) to the qh plane at nbe*128 + b*64,
// [192,208) to the sc plane at nbe*192 + b*16, [208,210) to the d plane at
// nbe*208 + b*2); the row tail up to the 16-byte stride is zero.
// The device kernel takes one row per workgroup and writes each 32-bit word of the
// split-plane row once (pad included), reading its source bytes as one word or two
// 16-bit halves of the raw block.

#include <string.h>

#include "kq_format.h"
#include "q6k_internal.h"

namespace q6k {

namespace {

// Bytes [0, n) of src as a little-endian word: as one word (ALIGN 4), two 16-bit
// halves (ALIGN 2) or single bytes (ALIGN 1, any address).
template <int ALIGN>
__device__ __forceinline__ uint32_t read_le(const uint8_t *src, uint32_t n)
{
    if constexpr (ALIGN == 4) {
        return *reinterpret_cast<const uint32_t *>(src);
    } else if constexpr (ALIGN == 2) {
        const uint16_t *h = reinterpret_cast<const uint16_t *>(src);
        return (uint32_t)h[0] | (n > 2u ? (uint32_t)h[1] << 16 : 0u);
    } else {
        uint32_t v = 0;
        for (uint32_t k = 0; k < n; ++k)
            v |= (uint32_t)src[k] << (8u * k);
        return v;
    }
}

// One 32-bit word of a split-plane row: bytes [o, o + 4) of the row at raw_row.
// Plane starts (nbe times the sizes of the planes before) are multiples of 4, as are
// the field sizes but q6_K's 2-byte d, so a word holds 4 bytes of one block's field
// or (d) the fields of blocks b and b + 1; bytes past the row's raw length are the
// zero pad. ALIGN: the alignment the raw rows guarantee for each field read (q6_K
// blocks of 210 B give 2 on an even base, q4_K / q5_K blocks of 144 / 176 B give 4
// on a base that is a multiple of 4; 1 for any other base).
template <int TYPE, int ALIGN>
__device__ __forceinline__ uint32_t dpl_word(const uint8_t *__restrict__ raw_row, uint32_t o,
                                             uint32_t nbe)
{
    constexpr PlaneMap m = plane_map(TYPE);
    uint32_t start = 0;
#pragma unroll
    for (uint32_t p = 0; p < m.n; ++p) {
        const uint32_t len = m.size[p] * nbe;
        if (o < start + len) {
            const uint32_t r = o - start;
            const uint32_t b = r / m.size[p], within = r - b * m.size[p];
            const uint8_t *src = raw_row + (size_t)b * m.block + m.off[p] + within;
            if (m.size[p] == 2u) {   // d of blocks b and b + 1 (the pad past the last)
                const uint32_t hi = b + 1u < nbe ? read_le<ALIGN>(src + m.block, 2u) : 0u;
                return read_le<ALIGN>(src, 2u) | (hi << 16);
            }
            return read_le<ALIGN>(src, 4u);
        }
        start += len;
    }
    return 0u;
}

// One workgroup per row; the threads walk its words.
template <int TYPE, int ALIGN>
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t *__restrict__ raw,
                                                     uint32_t *__restrict__ dpl, uint32_t nbe,
                                                     uint32_t stride)
{
    const uint64_t row = blockIdx.x;
    const uint8_t *src = raw + row * ((uint64_t)plane_map(TYPE).block * nbe);
    uint32_t *dst = dpl + row * (stride / 4u);
    for (uint32_t i = threadIdx.x; i < stride / 4u; i += 256u)
        dst[i] = dpl_word<TYPE, ALIGN>(src, 4u * i, nbe);
}

template <int TYPE>
const void *repack_kernel_for(const void *raw)
{
    constexpr int A = TYPE == KQT_Q6_K ? 2 : 4;
    return (uintptr_t)raw % A == 0 ? (const void *)repack_kernel<TYPE, A>
                                   : (const void *)repack_kernel<TYPE, 1>;
}

}  // namespace

hipError_t launch_repack(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K,
                         hipStream_t s)
{
    uint32_t nbe = (uint32_t)(K / 256);
    uint32_t stride = (uint32_t)kq_row_stride(type, nbe);
    uint32_t *out = reinterpret_cast<uint32_t *>(dpl);
    if (N > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const void *kern = type == KQT_Q6_K   ? repack_kernel_for<KQT_Q6_K>(raw)
                       : type == KQT_Q5_K ? repack_kernel_for<KQT_Q5_K>(raw)
                                          : repack_kernel_for<KQT_Q4_K>(raw);
    void *args[] = {(void *)&raw, (void *)&out, (void *)&nbe, (void *)&stride};
    return hipLaunchKernel(kern, dim3((uint32_t)N), dim3(256), args, 0, s);
}

void repack_host(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K)
{
    const PlaneMap m = plane_map(type);
    const int64_t nbe = K / 256;
    const int64_t rs = nbe * m.block, ds = (int64_t)kq_row_stride(type, nbe);
    for (int64_t r = 0; r < N; ++r) {
        const uint8_t *src = raw + r * rs;
        uint8_t *dst = dpl + r * ds;
        int64_t base = 0;
        for (uint32_t p = 0; p < m.n; ++p) {
            for (int64_t b = 0; b < nbe; ++b)
                memcpy(dst + base + b * m.size[p], src + b * m.block + m.off[p], m.size[p]);
            base += nbe * m.size[p];
        }
        memset(dst + rs, 0, (size_t)(ds - rs));
    }
}

void unpack_host(int type, const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K)
{
    const PlaneMap m = plane_map(type);
    const int64_t nbe = K / 256;
    const int64_t rs = nbe * m.block, ds = (int64_t)kq_row_stride(type, nbe);
    for (int64_t r = 0; r < N; ++r) {
        const uint8_t *src = dpl + r * ds;
        uint8_t *dst = raw + r * rs;
        int64_t base = 0;
        for (uint32_t p = 0; p < m.n; ++p) {
            for (int64_t b = 0; b < nbe; ++b)
                memcpy(dst + b * m.block + m.off[p], src + base + b * m.size[p], m.size[p]);
            base += nbe * m.size[p];
        }
    }
}

}  // namespace q6k
