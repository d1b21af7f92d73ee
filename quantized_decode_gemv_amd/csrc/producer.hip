// producer.hip -- q8 activation producers for gfx950: the standalone quantizer, the
// fused RMSNorm -> q8 producer and the fused SwiGLU -> q8 producer. The q8 block
// body, its thread geometry and the RMSNorm body are in q6k_norm.h.

#include "q6k_internal.h"
#include "q6k_norm.h"

namespace q6k {

namespace {

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
// Each lane reads its g and u before it writes y, so y may be g or u itself; y may
// be null (not stored).
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
        if (y)
            y[f] = yv;
        qs[f] = o.packed;
        if ((f & 7u) == 0)
            d8[f >> 3] = o.d16;
    }
}

// Workgroups of NORM_WG threads, each computing a token row's whole sum in the order
// of q6k_norm.h (so every workgroup of a row finds the same r) and then normalizing
// and quantizing one group of it: workgroup (s, t) takes the float4s s * NORM_WG ..
// s * NORM_WG + NORM_WG - 1 of token t, and the grid holds ceil(K / (4 * NORM_WG))
// workgroups per token. One workgroup per token doing every group spent most of its
// time on the q8 arithmetic of groups processed one after another on one CU. Rows of
// up to NORM_WG * VPT float4s keep their x in registers; longer rows are read again
// after the sum. y is stored (when y is not null) and quantized from registers, so
// the bytes equal quant_q8 applied to y.
template <int VPT>
__global__ __launch_bounds__(NORM_WG) void rmsnorm_quant_regs(const float4 *__restrict__ x,
                                                              const float4 *__restrict__ g,
                                                              float eps, float4 *__restrict__ y,
                                                              uint32_t *__restrict__ qs,
                                                              uint16_t *__restrict__ d8, uint32_t K)
{
    __shared__ double part[NORM_WG / 64];
    const uint32_t t = blockIdx.y;
    const int grp = (int)blockIdx.x;
    const uint32_t K4 = K / 4u;
    const __amdgpu_buffer_rsrc_t rx = buf_desc(x + (size_t)t * K4, 16u * K4),
                                 rg = buf_desc(g, 16u * K4);
    float4 xv[1][VPT], gv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t f = threadIdx.x + v * NORM_WG;
        xv[0][v] = load_f4_desc(rx, f);
        gv[v] = load_f4_desc(rg, f);
    }
    float4 *yr = y ? y + (size_t)t * K4 : nullptr;
    uint32_t *qr = qs + (size_t)t * K4;
    uint16_t *dr = d8 + (size_t)t * (K / 32u);
    norm_quant_rows<1, VPT>(
        xv, gv, K, eps, part,
        [&](int, uint32_t f, float4 yv, const Q8Out &o) {
            if (yr)
                yr[f] = yv;
            qr[f] = o.packed;
            if ((f & 7u) == 0)
                dr[f >> 3] = o.d16;
        },
        grp);
}

// Longer rows: every workgroup of a token sums the whole row (same order, same r),
// then workgroup s normalizes and quantizes the passes s, s + S, ... of NORM_WG
// float4s (S = gridDim.x workgroups per token).
__global__ __launch_bounds__(NORM_WG) void rmsnorm_quant_loop(const float4 *__restrict__ x,
                                                              const float4 *__restrict__ g,
                                                              float eps, float4 *__restrict__ y,
                                                              uint32_t *__restrict__ qs,
                                                              uint16_t *__restrict__ d8, uint32_t K)
{
    __shared__ double part[NORM_WG / 64];
    const uint32_t t = blockIdx.y;
    const uint32_t K4 = K / 4u;
    const float4 *xr = x + (size_t)t * K4;
    const uint32_t iters = (K4 + NORM_WG - 1) / NORM_WG;
    double acc = 0.0;
    for (uint32_t it = 0; it < iters; ++it) {
        const uint32_t f = it * NORM_WG + threadIdx.x;
        if (f < K4)
            acc = sq_chain4(acc, xr[f]);
    }
    const float r = norm_factor(norm_block_total(acc, part), K, eps);
    float4 *yr = y ? y + (size_t)t * K4 : nullptr;
    uint32_t *qr = qs + (size_t)t * K4;
    uint16_t *dr = d8 + (size_t)t * (K / 32u);
    for (uint32_t it = blockIdx.x; it < iters; it += gridDim.x) {
        const uint32_t f = it * NORM_WG + threadIdx.x;
        const bool live = f < K4;
        const float4 yv = live ? rms_scale(xr[f], g[f], r) : make_float4(0.f, 0.f, 0.f, 0.f);
        const Q8Out o = quant_group8(yv);
        if (live) {
            if (yr)
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
    // workgroups per token: one per group of NORM_WG float4s (the looping form: at
    // most 16, each taking every 16th pass)
    const uint32_t groups = (uint32_t)((K4 + NORM_WG - 1) / NORM_WG);
    const void *kern;
    uint32_t per = groups;
    if (K4 <= NORM_WG * 2)
        kern = (const void *)rmsnorm_quant_regs<2>;
    else if (K4 <= NORM_WG * 4)
        kern = (const void *)rmsnorm_quant_regs<4>;
    else if (K4 <= NORM_WG * 8)
        kern = (const void *)rmsnorm_quant_regs<8>;
    else {
        kern = (const void *)rmsnorm_quant_loop;
        per = groups < 16u ? groups : 16u;
    }
    return hipLaunchKernel(kern, dim3(per, nt), dim3(NORM_WG), args, 0, s);
}

}  // namespace q6k
