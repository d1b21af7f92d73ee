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
// 1 / sqrt(mean(x^2) + eps) with the mean summed in fp64 (each x^2 is exact in fp64)
// and r rounded once to f32; y = (x * r) * gamma in f32. The sum has one fixed order
// for every caller: a 256-thread workgroup, thread t adding the float4s t, t + 256,
// ... of the row in turn (each as x^2 + y^2 + z^2 + w^2), then an xor tree inside
// each wave and the four wave sums in order.
//
// Thread geometry: a lane holds 4 consecutive values (one float4), 8 consecutive
// lanes hold one 32-value block, and the block's amax is a DPP max over those 8
// lanes (pairs, quads, then mirrored half-rows). Every lane of a wave runs it;
// lanes past the end carry zeros and store nothing, so no lane leaves before a
// cross-lane step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q6k {

constexpr int NORM_WG = 256;

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
    const float di = (d != 0.0f) ? 1.0f / d : 0.0f;
    Q8Out o;
    o.packed = (uint32_t)(uint8_t)q8_code(v.x, di) | ((uint32_t)(uint8_t)q8_code(v.y, di) << 8) |
               ((uint32_t)(uint8_t)q8_code(v.z, di) << 16) |
               ((uint32_t)(uint8_t)q8_code(v.w, di) << 24);
    o.d16 = __builtin_bit_cast(uint16_t, (_Float16)d);
    return o;
}

__device__ __forceinline__ double sq_sum4(float4 v)
{
    double s = (double)v.x * (double)v.x;
    s += (double)v.y * (double)v.y;
    s += (double)v.z * (double)v.z;
    s += (double)v.w * (double)v.w;
    return s;
}

// Workgroup-wide sums of NT fp64 values per thread (NORM_WG threads), each by the
// same tree: an xor tree inside each wave, then the NORM_WG / 64 wave sums in order.
// part holds NT * NORM_WG / 64 doubles of LDS. Every thread gets the same totals.
template <int NT>
__device__ __forceinline__ void norm_block_sum(double (&v)[NT], double *part)
{
    constexpr int NWAVE = NORM_WG / 64;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        double a = v[t];
        a += __shfl_xor(a, 32);
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 8);
        a += __shfl_xor(a, 4);
        a += __shfl_xor(a, 2);
        a += __shfl_xor(a, 1);
        if ((threadIdx.x & 63u) == 0)
            part[t * NWAVE + (threadIdx.x >> 6)] = a;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        double tot = 0.0;
#pragma unroll
        for (int i = 0; i < NWAVE; ++i)
            tot += part[t * NWAVE + i];
        v[t] = tot;
    }
    __syncthreads();   // part may be reused by the caller
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
// gamma (zeros past K/4). Calls put(t, f, y, q8) for every token and live float4
// index f (q8.d16 is the scale of block f / 8). Each token's arithmetic is the same
// for every NT. Every thread of the workgroup must call it together.
template <int NT, int VPT, typename Put>
__device__ __forceinline__ void norm_quant_rows(const float4 (&xv)[NT][VPT],
                                                const float4 (&gv)[VPT], uint32_t K, float eps,
                                                double *part, Put &&put)
{
    const uint32_t K4 = K / 4u;
    double ss[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        ss[t] = 0.0;
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            if (threadIdx.x + v * NORM_WG < K4)
                ss[t] += sq_sum4(xv[t][v]);
    }
    norm_block_sum<NT>(ss, part);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float r = norm_factor(ss[t], K, eps);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t f = threadIdx.x + v * NORM_WG;
            const float4 yv = rms_scale(xv[t][v], gv[v], r);
            const Q8Out o = quant_group8(yv);
            if (f < K4)
                put(t, f, yv, o);
        }
    }
}

}  // namespace q6k
