// kq_format.h -- the k-quant weight types the library takes and their row layouts,
// for host and device code.
//
// Raw rows are GGUF super-blocks of 256 weights back to back. The split-plane row
// keeps each field of the block in its own plane (the q6_K dpl row of D4-4 §2 and
// §3.2 Excerpts A and B; the q4_K and q5_K rows follow the same rule), the planes in
// the order listed below, plane p starting at nbe * (sum of the sizes before it),
// block b's field at plane start + b * size. The row stride is nbe * block bytes
// rounded up to 16 (a no-op for q4_K and q5_K, whose blocks are 144 and 176 B).
//
// Block fields (byte offset in the raw block, size), in plane order:
//   q6_K (210 B): low bits (0, 128), high bits (128, 64), int8 scales (192, 16),
//                 d (208, 2)
//   q4_K (144 B): codes (16, 128), packed scales/mins (4, 12), d and dmin (0, 4)
//   q5_K (176 B): codes (48, 128), fifth bits (16, 32), packed scales/mins (4, 12),
//                 d and dmin (0, 4)
// The q4_K and q5_K block layouts are the public GGUF definitions (the pages name
// these classes but print no layout).
#pragma once

#include <stdint.h>

namespace q6k {

enum KqType : int { KQT_Q4_K = 12, KQT_Q5_K = 13, KQT_Q6_K = 14 };   // GGUF type ids

struct PlaneMap {
    uint32_t block;      // bytes per super-block
    uint32_t n;          // planes
    uint32_t off[4];     // field offset in the raw block
    uint32_t size[4];    // field bytes per block
};

__host__ __device__ constexpr bool kq_known(int type)
{
    return type == KQT_Q4_K || type == KQT_Q5_K || type == KQT_Q6_K;
}

__host__ __device__ constexpr PlaneMap plane_map(int type)
{
    return type == KQT_Q6_K ? PlaneMap{210, 4, {0, 128, 192, 208}, {128, 64, 16, 2}}
         : type == KQT_Q5_K ? PlaneMap{176, 4, {48, 16, 4, 0}, {128, 32, 12, 4}}
                           : PlaneMap{144, 3, {16, 4, 0, 0}, {128, 12, 4, 0}};
}

__host__ __device__ constexpr uint32_t kq_block_bytes(int type) { return plane_map(type).block; }

__host__ __device__ constexpr uint64_t kq_row_stride(int type, uint64_t nbe)
{
    return (nbe * kq_block_bytes(type) + 15u) & ~(uint64_t)15u;
}

}  // namespace q6k
