// q6k_norm.h -- the RMSNorm -> q8 body shared by the fused RMSNorm -> q8 producer
// and the fused RMSNorm -> q8 -> GEMV kernel, so that both compute bit-identical
// activations, and the q8 block quantizer of every producer.
//
// q8 (D3-5 §3.2, the per-32-block body): amax = max|y| over the block, d = amax/127,
// di = d != 0 ? 1/d : 0 (IEEE f32 divisions), q = clamp(rint(y*di), -128, 127) with
// ties to even (v_rndne_f32), stored scale f16(d). No add sits next to a product to
// contract, so each code follows from its input value and its block's amax alone
// (max is exact under any association).
//
// RMSNorm (D3-5 §3.2, the fused rms producer; its body is not printed): r =
// 1 / sqrt(mean(x^2) + eps) with the mean summed in fp64 (each x^2 is exact in fp64,
// so each step acc + x^2 is one rounding, written as one fp64 fma) and r rounded once
// to f32; y = (x * r) * gamma in f32. The sum has one fixed order for every caller,
// by a workgroup of NORM_WG threads:
//  - thread t takes the float4s t, t + NORM_WG, t + 2 * NORM_WG, ... of the row
//    (past the row: zeros, which add exactly +0) and chains their elements in
//    order: acc = (((acc + x0^2) + x1^2) + x2^2) + x3^2;
//  - each wave adds its 64 chains by wave_sum_f64 (pairs, quads, 8 and 16 lanes by
//    DPP, then 32-lane and 16-lane swaps);
//  - the workgroup's total is (W0 + W1) + (W2 + W3) of its four wave sums.
// Addition is commutative in IEEE arithmetic, so lanes that combine the same two
// partial sums in either order agree bit for bit.

// Thread geometry of quant_group8: a lane holds 4 consecutive values (one float4),
// 8 consecutive lanes hold one 32-value block, and the block's amax is a DPP max over
// those 8 lanes (pairs, quads, then mirrored half-rows). Every lane of a wave runs
// it; lanes past the end carry zeros and store nothing, so no lane leaves before a
// cross-lane step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bufload.h"

namespace q6k {

constexpr int NORM_WG = 256;

// float4 f of a row through its descriptor (zeros past the descriptor's extent).
__device__ __forceinline__ float4 load_f4_desc(__amdgpu_buffer_rsrc_t r, uint32_t f)
{
    const uint4 v = load_b128<POLICY_DEFAULT>(r, 16u * f);
    const uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    return make_float4(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b),
                       __builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}

__device__ __forceinline__ float amax4(float4 v)
{
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ int q8_code(float v, float di)
{
    int q = (int)rintf(v * di);
    return q < -128 ? -128 : (q > 127 ? 127 : q);
}

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v)
{
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false)));
}

// 1 / d, or 0 for an all-zero block.
__device__ __forceinline__ float q8_inv(float d)
{
    return (d != 0.0f) ? 1.0f / d : 0.0f;
}

// The q8 codes of four values, byte i from component i.
__device__ __forceinline__ uint32_t q8_pack4(float4 v, float di)
{
    return (uint32_t)(uint8_t)q8_code(v.x, di) | ((uint32_t)(uint8_t)q8_code(v.y, di) << 8) |
           ((uint32_t)(uint8_t)q8_code(v.z, di) << 16) |
           ((uint32_t)(uint8_t)q8_code(v.w, di) << 24);
}

struct Q8Out {
    uint32_t packed;   // 4 int8 codes
    uint16_t d16;      // f16 block scale (meaningful on every lane of the group)
};

// All 64 lanes must call this together; lanes 8m..8m+7 form one block.
__device__ __forceinline__ Q8Out quant_group8(float4 v)
{
    float m = amax4(v);
    m = dpp_max<0xB1>(m);    // quad_perm [1,0,3,2]: pairs
    m = dpp_max<0x4E>(m);    // quad_perm [2,3,0,1]: quads
    m = dpp_max<0x141>(m);   // row_half_mirror: the two quads of each 8 lanes
    const float d = m / 127.0f;
    Q8Out o;
    o.packed = q8_pack4(v, q8_inv(d));
    o.d16 = __builtin_bit_cast(uint16_t, (_Float16)d);
    return o;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

// v plus the value of the lane 32 lanes away (SWAP32) or of the neighbouring 16-lane
// row (otherwise). The swap results are copied into plain integers before use: a bit
// cast applied straight to an element of the returned pair reads element 0.
template <bool SWAP32>
__device__ __forceinline__ double swap_add_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const unsigned lo = (unsigned)b, hi = (unsigned)(b >> 32);
    unsigned l0, l1, h0, h1;
    if constexpr (SWAP32) {
        const auto L = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto H = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        l0 = L[0]; l1 = L[1]; h0 = H[0]; h1 = H[1];
    } else {
        const auto L = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto H = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        l0 = L[0]; l1 = L[1]; h0 = H[0]; h1 = H[1];
    }
    return __builtin_bit_cast(double, (uint64_t)l0 | ((uint64_t)h0 << 32)) +
           __builtin_bit_cast(double, (uint64_t)l1 | ((uint64_t)h1 << 32));
}

// Sum over the 64 lanes of a wave (every lane must call it; every lane gets the
// total). Each step adds two partial sums of the same lanes on every lane.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
    v += dpp_f64<0x4E>(v);    // quad_perm [2,3,0,1]: quads
    v += dpp_f64<0x141>(v);   // row_half_mirror: the two quads of each 8 lanes
    v += dpp_f64<0x140>(v);   // row_mirror: the two halves of each 16-lane row
    v = swap_add_f64<true>(v);
    return swap_add_f64<false>(v);
}

// acc + the squares of v's elements, in order.
__device__ __forceinline__ double sq_chain4(double acc, float4 v)
{
    acc = __builtin_fma((double)v.x, (double)v.x, acc);
    acc = __builtin_fma((double)v.y, (double)v.y, acc);
    acc = __builtin_fma((double)v.z, (double)v.z, acc);
    return __builtin_fma((double)v.w, (double)v.w, acc);
}

// The workgroup's total of one fp64 value per thread (NORM_WG threads, all of which
// must call it), by the fixed tree above. part: NORM_WG / 64 doubles of LDS, written
// once per call (a caller that calls it again must put a barrier between the calls).
__device__ __forceinline__ double norm_block_total(double v, double *part)
{
    static_assert(NORM_WG == 256, "four wave sums");
    v = wave_sum_f64(v);
    if ((threadIdx.x & 63u) == 0)
        part[threadIdx.x >> 6] = v;
    __syncthreads();
    return (part[0] + part[1]) + (part[2] + part[3]);
}

__device__ __forceinline__ float norm_factor(double sumsq, uint32_t K, float eps)
{
    return (float)(1.0 / sqrt(sumsq / (double)K + (double)eps));
}

__device__ __forceinline__ float4 rms_scale(float4 x, float4 g, float r)
{
    return make_float4((x.x * r) * g.x, (x.y * r) * g.y, (x.z * r) * g.z, (x.w * r) * g.w);
}

// RMSNorm -> q8 of NT token rows held in registers by a NORM_WG-thread workgroup:
// xv[t][v] and gv[v] are the float4s threadIdx.x + v * NORM_WG of token t's x and of
// gamma (zeros past K/4). Calls put(t, f, y, q8) for every live float4 index f
// (q8.d16 is the scale of block f / 8) of group `only` (v == only; every group when
// only < 0; only is the same for the whole workgroup). The sum always covers every
// group, so r does not depend on `only`. Every thread must call it; part holds
// NORM_WG / 64 doubles of LDS per token.
template <int NT, int VPT, bool SKIP_PAST = false, typename Put>
__device__ __forceinline__ void norm_quant_rows(const float4 (&xv)[NT][VPT],
                                                const float4 (&gv)[VPT], uint32_t K, float eps,
                                                double *part, Put &&put, int only = -1)
{
    const uint32_t K4 = K / 4u;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        double acc = 0.0;
        // SKIP_PAST: a group v with v * NORM_WG >= K4 holds only the zeros past the
        // row (each would add +0) and no output, so the whole workgroup skips it; the
        // results are the same either way
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            if (!SKIP_PAST || (uint32_t)v * NORM_WG < K4)
                acc = sq_chain4(acc, xv[t][v]);
        const float r = norm_factor(norm_block_total(acc, part + t * (NORM_WG / 64)), K, eps);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            if (SKIP_PAST && (uint32_t)v * NORM_WG >= K4)
                break;
            if (only >= 0 && v != only)
                continue;
            const uint32_t f = threadIdx.x + v * NORM_WG;
            const float4 yv = rms_scale(xv[t][v], gv[v], r);
            const Q8Out o = quant_group8(yv);
            if (f < K4)
                put(t, f, yv, o);
        }
    }
}

}  // namespace q6k
