// repack.hip -- raw GGUF q6_K rows -> dpl rows, on the device and on the host.
//
// The byte permutation of D4-4 §3.2 Excerpt A: for row r and super-block b, the
// block's bytes [0,128) go to the ql plane at b*128, [128,192) to the qh plane at
// nbe*128 + b*64, [192,208) to the sc plane at nbe*192 + b*16 and [208,210) to the d
// plane at nbe*208 + b*2; the row tail up to the 16-byte stride is zero.
// The device kernel writes one 32-bit word of the dpl row per thread, gathering its
// four source bytes, so every dpl byte (pad included) is written exactly once.

#include <string.h>

#include "q6k_internal.h"

namespace q6k {

namespace {

__device__ __forceinline__ uint32_t src_byte(const uint8_t *__restrict__ raw_row, uint32_t o,
                                             uint32_t nbe)
{
    uint32_t blk, off, field;
    if (o < 128u * nbe) {
        blk = o / 128u; off = o % 128u; field = 0;
    } else if (o < 192u * nbe) {
        o -= 128u * nbe; blk = o / 64u; off = o % 64u; field = 128;
    } else if (o < 208u * nbe) {
        o -= 192u * nbe; blk = o / 16u; off = o % 16u; field = 192;
    } else if (o < 210u * nbe) {
        o -= 208u * nbe; blk = o / 2u; off = o % 2u; field = 208;
    } else {
        return 0u;
    }
    return raw_row[(size_t)blk * 210u + field + off];
}

__global__ __launch_bounds__(256) void repack_kernel(const uint8_t *__restrict__ raw,
                                                     uint32_t *__restrict__ dpl, uint64_t words,
                                                     uint32_t nbe, uint32_t stride)
{
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i >= words)
        return;
    const uint32_t wpr = stride / 4u;
    const uint64_t row = i / wpr;
    const uint32_t o = (uint32_t)(i % wpr) * 4u;
    const uint8_t *src = raw + row * (uint64_t)(210u * nbe);
    const uint32_t v = src_byte(src, o, nbe) | (src_byte(src, o + 1, nbe) << 8) |
                       (src_byte(src, o + 2, nbe) << 16) | (src_byte(src, o + 3, nbe) << 24);
    dpl[i] = v;
}

}  // namespace

hipError_t launch_repack(const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K, hipStream_t s)
{
    uint32_t nbe = (uint32_t)(K / 256);
    uint32_t stride = (uint32_t)(((int64_t)nbe * 210 + 15) & ~(int64_t)15);
    uint64_t words = (uint64_t)N * stride / 4u;
    uint32_t *out = reinterpret_cast<uint32_t *>(dpl);
    const uint64_t grid = (words + 255u) / 256u;
    if (grid > 0x7FFFFFFFull)
        return hipErrorInvalidValue;
    void *args[] = {(void *)&raw, (void *)&out, (void *)&words, (void *)&nbe, (void *)&stride};
    return hipLaunchKernel((const void *)repack_kernel, dim3((uint32_t)grid), dim3(256), args, 0,
                           s);
}

void repack_host(const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K)
{
    const int64_t nbe = K / 256;
    const int64_t rs = nbe * 210, ds = (nbe * 210 + 15) & ~(int64_t)15;
    for (int64_t r = 0; r < N; ++r) {
        const uint8_t *src = raw + r * rs;
        uint8_t *dst = dpl + r * ds;
        for (int64_t b = 0; b < nbe; ++b) {
            memcpy(dst + b * 128, src + b * 210, 128);
            memcpy(dst + nbe * 128 + b * 64, src + b * 210 + 128, 64);
            memcpy(dst + nbe * 192 + b * 16, src + b * 210 + 192, 16);
            memcpy(dst + nbe * 208 + b * 2, src + b * 210 + 208, 2);
        }
        memset(dst + rs, 0, (size_t)(ds - rs));
    }
}

void unpack_host(const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K)
{
    const int64_t nbe = K / 256;
    const int64_t rs = nbe * 210, ds = (nbe * 210 + 15) & ~(int64_t)15;
    for (int64_t r = 0; r < N; ++r) {
        const uint8_t *src = dpl + r * ds;
        uint8_t *dst = raw + r * rs;
        for (int64_t b = 0; b < nbe; ++b) {
            memcpy(dst + b * 210, src + b * 128, 128);
            memcpy(dst + b * 210 + 128, src + nbe * 128 + b * 64, 64);
            memcpy(dst + b * 210 + 192, src + nbe * 192 + b * 16, 16);
            memcpy(dst + b * 210 + 208, src + nbe * 208 + b * 2, 2);
        }
    }
}

}  // namespace q6k
