// repack.hip -- raw GGUF k-quant rows -> split-plane rows, on the device and on the
// host, for every type of kq_format.h.
//
// A byte permutation: for row r and super-block b, each field of the block is
// copied to its plane (for q6_K the permutation of D4-4 §3.2 Excerpt A: bytes
// [0,128) to the ql plane at b*128, [128,192) to the qh plane at nbe*128 + b*64,
// [192,208) to the sc plane at nbe*192 + b*16, [208,210) to the d plane at
// nbe*208 + b*2); the row tail up to the 16-byte stride is zero.
// The device kernel writes one 32-bit word of the split-plane row per thread,
// gathering its four source bytes, so every output byte (pad included) is written
// exactly once.

#include <string.h>

#include "kq_format.h"
#include "q6k_internal.h"

namespace q6k {

namespace {

// Raw source byte of split-plane row byte o (0 for the tail pad).
__device__ __forceinline__ uint32_t src_byte(const uint8_t *__restrict__ raw_row, uint32_t o,
                                             uint32_t nbe, const PlaneMap &m)
{
    uint32_t base = 0;
    for (uint32_t p = 0; p < m.n; ++p) {
        const uint32_t len = m.size[p] * nbe;
        if (o < base + len) {
            const uint32_t r = o - base;
            return raw_row[(size_t)(r / m.size[p]) * m.block + m.off[p] + r % m.size[p]];
        }
        base += len;
    }
    return 0u;
}

__global__ __launch_bounds__(256) void repack_kernel(const uint8_t *__restrict__ raw,
                                                     uint32_t *__restrict__ dpl, uint64_t words,
                                                     uint32_t nbe, uint32_t stride, PlaneMap m)
{
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i >= words)
        return;
    const uint32_t wpr = stride / 4u;
    const uint64_t row = i / wpr;
    const uint32_t o = (uint32_t)(i % wpr) * 4u;
    const uint8_t *src = raw + row * (uint64_t)(m.block * nbe);
    const uint32_t v = src_byte(src, o, nbe, m) | (src_byte(src, o + 1, nbe, m) << 8) |
                       (src_byte(src, o + 2, nbe, m) << 16) | (src_byte(src, o + 3, nbe, m) << 24);
    dpl[i] = v;
}

}  // namespace

hipError_t launch_repack(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K,
                         hipStream_t s)
{
    uint32_t nbe = (uint32_t)(K / 256);
    uint32_t stride = (uint32_t)kq_row_stride(type, nbe);
    uint64_t words = (uint64_t)N * stride / 4u;
    uint32_t *out = reinterpret_cast<uint32_t *>(dpl);
    PlaneMap m = plane_map(type);
    const uint64_t grid = (words + 255u) / 256u;
    if (grid > 0x7FFFFFFFull)
        return hipErrorInvalidValue;
    void *args[] = {(void *)&raw, (void *)&out, (void *)&words, (void *)&nbe, (void *)&stride,
                    (void *)&m};
    return hipLaunchKernel((const void *)repack_kernel, dim3((uint32_t)grid), dim3(256), args, 0,
                           s);
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
