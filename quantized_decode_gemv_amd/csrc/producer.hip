// producer.hip -- q8 activation producers for gfx950: the standalone quantizer, the
// fused RMSNorm -> q8 producer and the fused SwiGLU -> q8 producer.
//
// The q8 body follows the per-32-block quantizer of D3-5 §3.2: amax = max|x|,
// d = amax/127 (f32 division), di = d != 0 ? 1/d : 0 (f32 division),
// q = clamp(rint(x*di), -128, 127) with ties to even, stored scale f16(d).
// HIP's default f32 division and rintf (v_rndne_f32) are IEEE, and there is no
// add next to a product to contract, so every byte follows from its own input value
// and its block's amax (max is exact under any association).
//
// Thread geometry: a lane holds 4 consecutive values (one float4), 8 consecutive
// lanes hold one 32-value block, and the block's amax is a DPP max over those 8
// lanes (pairs, quads, then mirrored half-rows). Every lane of a wave runs it;
// lanes past the end carry zeros and store nothing, so no lane leaves before a
// cross-lane step.

#include "q6k_internal.h"

namespace q6k {

namespace {

struct Q8Out {
    uint32_t packed;   // 4 int8 codes
    uint16_t d16;      // f16 block scale (meaningful on every lane of the group)
};

__device__ __forceinline__ int q_of(float v, float di)
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

// All 64 lanes must call this together; lanes 8m..8m+7 form one block.
__device__ __forceinline__ Q8Out quant_group8(float4 v)
{
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    m = dpp_max<0xB1>(m);    // quad_perm [1,0,3,2]: pairs
    m = dpp_max<0x4E>(m);    // quad_perm [2,3,0,1]: quads
    m = dpp_max<0x141>(m);   // row_half_mirror: the two quads of each 8 lanes
    const float d = m / 127.0f;
    const float di = (d != 0.0f) ? 1.0f / d : 0.0f;
    Q8Out o;
    o.packed = (uint32_t)(uint8_t)q_of(v.x, di) | ((uint32_t)(uint8_t)q_of(v.y, di) << 8) |
               ((uint32_t)(uint8_t)q_of(v.z, di) << 16) | ((uint32_t)(uint8_t)q_of(v.w, di) << 24);
    o.d16 = __builtin_bit_cast(uint16_t, (_Float16)d);
    return o;
}

constexpr int QWG = 256;

// x: nt*K floats (t-major), one float4 per lane over the flattened array; the q8
// plane's two sections are t-major too, so flat index f maps to qs[4f..4f+3] and
// block f/8.
__global__ __launch_bounds__(QWG) void quant_q8_kernel(const float4 *__restrict__ x,
                                                       uint32_t *__restrict__ qs,
                                                       uint16_t *__restrict__ d8, uint32_t nf4)
{
    const uint32_t f = blockIdx.x * QWG + threadIdx.x;
    const bool live = f < nf4;
    const float4 v = live ? x[f] : make_float4(0.f, 0.f, 0.f, 0.f);
    const Q8Out o = quant_group8(v);
    if (live) {
        qs[f] = o.packed;
        if ((f & 7u) == 0)
            d8[f >> 3] = o.d16;
    }
}

// SwiGLU then q8 (D3-5 §3.2, the fused swiglu producer): y = (g / (1 + e^-g)) * u
// in f32 -- IEEE division, the library expf -- stored and quantized from registers.
// Each lane reads its g and u before it writes y, so y may be g or u itself.
__global__ __launch_bounds__(QWG) void swiglu_quant_kernel(const float4 *g, const float4 *u,
                                                           float4 *y, uint32_t *__restrict__ qs,
                                                           uint16_t *__restrict__ d8, uint32_t nf4)
{
    const uint32_t f = blockIdx.x * QWG + threadIdx.x;
    const bool live = f < nf4;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 gv = live ? g[f] : zero;
    const float4 uv = live ? u[f] : zero;
    float4 yv;
    yv.x = (gv.x / (1.0f + expf(-gv.x))) * uv.x;
    yv.y = (gv.y / (1.0f + expf(-gv.y))) * uv.y;
    yv.z = (gv.z / (1.0f + expf(-gv.z))) * uv.z;
    yv.w = (gv.w / (1.0f + expf(-gv.w))) * uv.w;
    const Q8Out o = quant_group8(yv);
    if (live) {
        y[f] = yv;
        qs[f] = o.packed;
        if ((f & 7u) == 0)
            d8[f >> 3] = o.d16;
    }
}

__device__ __forceinline__ double block_sum_f64(double v, double *part, int nwaves)
{
    v += __shfl_xor(v, 32);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    if ((threadIdx.x & 63u) == 0)
        part[threadIdx.x >> 6] = v;
    __syncthreads();
    double tot = 0.0;
    for (int i = 0; i < nwaves; ++i)    // every thread adds in the same order
        tot += part[i];
    return tot;
}

__device__ __forceinline__ float4 rms_scale(float4 x, float4 g, float r)
{
    return make_float4((x.x * r) * g.x, (x.y * r) * g.y, (x.z * r) * g.z, (x.w * r) * g.w);
}

__device__ __forceinline__ double sq_sum(float4 v)
{
    double s = (double)v.x * (double)v.x;
    s += (double)v.y * (double)v.y;
    s += (double)v.z * (double)v.z;
    s += (double)v.w * (double)v.w;
    return s;
}

// One workgroup per token row, the whole row held in registers (VPT float4 per
// thread, K/4 <= BS*VPT). The sum of squares is fp64 (each x^2 is exact in fp64)
// in a fixed reduction order; r = f32(1 / sqrt(mean + eps)); y = (x*r)*g in f32 is
// stored and quantized from the same registers (the bytes equal quant_q8 applied
// to y).
template <int BS, int VPT>
__global__ __launch_bounds__(BS) void rmsnorm_quant_regs(const float4 *__restrict__ x,
                                                         const float4 *__restrict__ g,
                                                         float eps, float4 *__restrict__ y,
                                                         uint32_t *__restrict__ qs,
                                                         uint16_t *__restrict__ d8, uint32_t K)
{
    const uint32_t t = blockIdx.x;
    const uint32_t K4 = K / 4u;
    const float4 *xr = x + (size_t)t * K4;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 xv[VPT], gv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t f = threadIdx.x + v * BS;
        xv[v] = f < K4 ? xr[f] : zero;
        gv[v] = f < K4 ? g[f] : zero;
    }
    double ss = 0.0;
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        ss += sq_sum(xv[v]);
    __shared__ double part[BS / 64];
    const double tot = block_sum_f64(ss, part, BS / 64);
    const float r = (float)(1.0 / sqrt(tot / (double)K + (double)eps));

    float4 *yr = y + (size_t)t * K4;
    uint32_t *qr = qs + (size_t)t * K4;
    uint16_t *dr = d8 + (size_t)t * (K / 32u);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t f = threadIdx.x + v * BS;
        const bool live = f < K4;
        const float4 yv = rms_scale(xv[v], gv[v], r);
        const Q8Out o = quant_group8(yv);
        if (live) {
            yr[f] = yv;
            qr[f] = o.packed;
            if ((f & 7u) == 0)
                dr[f >> 3] = o.d16;
        }
    }
}

// Any row length: the same computation, walking the row twice from memory.
template <int BS>
__global__ __launch_bounds__(BS) void rmsnorm_quant_loop(const float4 *__restrict__ x,
                                                         const float4 *__restrict__ g,
                                                         float eps, float4 *__restrict__ y,
                                                         uint32_t *__restrict__ qs,
                                                         uint16_t *__restrict__ d8, uint32_t K)
{
    const uint32_t t = blockIdx.x;
    const uint32_t K4 = K / 4u;
    const float4 *xr = x + (size_t)t * K4;
    double ss = 0.0;
    for (uint32_t f = threadIdx.x; f < K4; f += BS)
        ss += sq_sum(xr[f]);
    __shared__ double part[BS / 64];
    const double tot = block_sum_f64(ss, part, BS / 64);
    const float r = (float)(1.0 / sqrt(tot / (double)K + (double)eps));

    float4 *yr = y + (size_t)t * K4;
    uint32_t *qr = qs + (size_t)t * K4;
    uint16_t *dr = d8 + (size_t)t * (K / 32u);
    const uint32_t iters = (K4 + BS - 1) / BS;
    for (uint32_t it = 0; it < iters; ++it) {
        const uint32_t f = it * BS + threadIdx.x;
        const bool live = f < K4;
        const float4 yv = live ? rms_scale(xr[f], g[f], r) : make_float4(0.f, 0.f, 0.f, 0.f);
        const Q8Out o = quant_group8(yv);
        if (live) {
            yr[f] = yv;
            qr[f] = o.packed;
            if ((f & 7u) == 0)
                dr[f >> 3] = o.d16;
        }
    }
}

}  // namespace

hipError_t launch_quant(const float *x, uint8_t *q8, int64_t K, int nt, hipStream_t s)
{
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    uint32_t *qs = reinterpret_cast<uint32_t *>(q8);
    uint16_t *d8 = reinterpret_cast<uint16_t *>(q8 + (size_t)nt * K);
    uint32_t nf4 = (uint32_t)((int64_t)nt * K / 4);
    const uint32_t grid = (nf4 + QWG - 1) / QWG;
    void *args[] = {(void *)&x4, (void *)&qs, (void *)&d8, (void *)&nf4};
    return hipLaunchKernel((const void *)quant_q8_kernel, dim3(grid), dim3(QWG), args, 0, s);
}

hipError_t launch_swiglu_quant(const float *g, const float *u, float *y, uint8_t *q8, int64_t K,
                               int nt, hipStream_t s)
{
    const float4 *g4 = reinterpret_cast<const float4 *>(g);
    const float4 *u4 = reinterpret_cast<const float4 *>(u);
    float4 *y4 = reinterpret_cast<float4 *>(y);
    uint32_t *qs = reinterpret_cast<uint32_t *>(q8);
    uint16_t *d8 = reinterpret_cast<uint16_t *>(q8 + (size_t)nt * K);
    uint32_t nf4 = (uint32_t)((int64_t)nt * K / 4);
    const uint32_t grid = (nf4 + QWG - 1) / QWG;
    void *args[] = {(void *)&g4, (void *)&u4, (void *)&y4, (void *)&qs, (void *)&d8, (void *)&nf4};
    return hipLaunchKernel((const void *)swiglu_quant_kernel, dim3(grid), dim3(QWG), args, 0, s);
}

hipError_t launch_rmsnorm_quant(const float *x, const float *gamma, float eps, float *y,
                                uint8_t *q8, int64_t K, int nt, hipStream_t s)
{
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const float4 *g4 = reinterpret_cast<const float4 *>(gamma);
    float4 *y4 = reinterpret_cast<float4 *>(y);
    uint32_t *qs = reinterpret_cast<uint32_t *>(q8);
    uint16_t *d8 = reinterpret_cast<uint16_t *>(q8 + (size_t)nt * K);
    uint32_t Ku = (uint32_t)K;
    void *args[] = {(void *)&x4, (void *)&g4, (void *)&eps, (void *)&y4,
                    (void *)&qs, (void *)&d8, (void *)&Ku};
    const int64_t K4 = K / 4;
    const void *kern;
    int bs;
    if (K4 <= 256 * 2) { kern = (const void *)rmsnorm_quant_regs<256, 2>; bs = 256; }
    else if (K4 <= 256 * 4) { kern = (const void *)rmsnorm_quant_regs<256, 4>; bs = 256; }
    else if (K4 <= 256 * 8) { kern = (const void *)rmsnorm_quant_regs<256, 8>; bs = 256; }
    else if (K4 <= 1024 * 4) { kern = (const void *)rmsnorm_quant_regs<1024, 4>; bs = 1024; }
    else if (K4 <= 1024 * 8) { kern = (const void *)rmsnorm_quant_regs<1024, 8>; bs = 1024; }
    else { kern = (const void *)rmsnorm_quant_loop<1024>; bs = 1024; }
    return hipLaunchKernel(kern, dim3(nt), dim3(bs), args, 0, s);
}

}  // namespace q6k
