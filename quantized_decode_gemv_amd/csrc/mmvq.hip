// mmvq.hip -- q6_K (dpl rows) x q8 decode GEMV kernels for gfx950, and their shape
// dispatch.
//
// What is computed (D4-2 §3.2 Excerpt C, the per-unit accumulation; D4-4 §3.2
// Excerpt B, the dpl unit load): y[t][r] = sum over the row's 16-element sub-blocks
// of d * sc * d8 * D, D the exact int32 dot of (q - 32) with the int8 activations.
//
// Geometry (one design for every shape):
//  - one wave64 owns one row at a time and walks rows with a stride of the grid's
//    wave count, so at any moment the waves of the grid stream neighbouring rows;
//  - lane L takes the row's low-bit chunks Q = L, L + 64, ... (q6k_unit.h), so each
//    low-bit load instruction is 1 KB contiguous, each high-bit load 512 B
//    contiguous (two lanes share a chunk), each scale load 128 B, each d load 16 B;
//  - a lane's chunk positions are the same for every row it visits, so its
//    activation operands can be loaded once per wave and kept in registers
//    (HOIST) when they fit, otherwise they are re-read per row (they stay cached);
//  - every row is finished with a wave64 butterfly sum, written by lane 0.
// The chunks per lane (CPL = ceil(8*nbe/64)) is a template parameter up to
// MAX_CPL, so all of a row's loads are issued before any arithmetic; longer rows
// take the generic kernel, which walks a row in runtime steps of 4 chunks per lane.
// Every lane guards every chunk with Q < 8*nbe and every row with row < N, so each
// kernel covers all units of all rows for any shape it is launched on (the lesson
// of D4-2 §2: a dispatch that routes a shape to a kernel that covers fewer units
// silently drops work).

#include "q6k_internal.h"
#include "q6k_unit.h"

namespace q6k {

constexpr int WG = 256;             // 4 waves per workgroup
constexpr int WAVES_PER_WG = WG / 64;
constexpr int MAX_CPL = 12;         // nbe <= 96 take the unrolled kernels
constexpr int WAVES_PER_CU = 16;    // persistent grid: waves resident per CU
constexpr int MAX_NT_KERNEL = 4;    // token columns per launch (more -> several launches)

template <int NT, int CPL, bool HOIST>
__global__ __launch_bounds__(WG) void mmvq_unrolled(const uint8_t *__restrict__ w,
                                                    const int8_t *__restrict__ qs,
                                                    const uint16_t *__restrict__ d8,
                                                    float *__restrict__ y, uint32_t N,
                                                    uint32_t nbe, uint32_t stride, uint32_t K,
                                                    uint32_t ldy)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * WAVES_PER_WG + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * WAVES_PER_WG;
    const uint32_t C = 8u * nbe;

    ChunkAct act[HOIST ? CPL : 1][NT];
    if constexpr (HOIST) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t Q = lane + 64u * i;
            if (Q < C) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    act[i][t] = load_act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), Q);
            }
        }
    }

    for (uint32_t row = wave; row < N; row += nwaves) {
        const uint8_t *r = w + (size_t)row * stride;
        ChunkW wt[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t Q = lane + 64u * i;
            if (Q < C)
                wt[i] = load_w(r, nbe, Q);
        }
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t Q = lane + 64u * i;
            if (Q < C) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if constexpr (HOIST) {
                        acc[t] += chunk_partial(wt[i], act[i][t], Q);
                    } else {
                        const ChunkAct a =
                            load_act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), Q);
                        acc[t] += chunk_partial(wt[i], a, Q);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float s = wave_sum(acc[t]);
            if (lane == 0)
                y[(size_t)t * ldy + row] = s;
        }
    }
}

// Any row length: a row is walked in steps of 4 chunks per lane.
template <int NT>
__global__ __launch_bounds__(WG) void mmvq_generic(const uint8_t *__restrict__ w,
                                                   const int8_t *__restrict__ qs,
                                                   const uint16_t *__restrict__ d8,
                                                   float *__restrict__ y, uint32_t N, uint32_t nbe,
                                                   uint32_t stride, uint32_t K, uint32_t ldy)
{
    constexpr int STEP = 4;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * WAVES_PER_WG + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * WAVES_PER_WG;
    const uint32_t C = 8u * nbe;

    for (uint32_t row = wave; row < N; row += nwaves) {
        const uint8_t *r = w + (size_t)row * stride;
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = 0.0f;
        for (uint32_t base = 0; base < C; base += 64u * STEP) {
            ChunkW wt[STEP];
#pragma unroll
            for (int i = 0; i < STEP; ++i) {
                const uint32_t Q = base + lane + 64u * i;
                if (Q < C)
                    wt[i] = load_w(r, nbe, Q);
            }
#pragma unroll
            for (int i = 0; i < STEP; ++i) {
                const uint32_t Q = base + lane + 64u * i;
                if (Q < C) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const ChunkAct a =
                            load_act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), Q);
                        acc[t] += chunk_partial(wt[i], a, Q);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float s = wave_sum(acc[t]);
            if (lane == 0)
                y[(size_t)t * ldy + row] = s;
        }
    }
}

// Test kernel: the exact sub-block dots, one wave per row, any row length.
__global__ __launch_bounds__(WG) void mmvq_subdots_kernel(const uint8_t *__restrict__ w,
                                                          const int8_t *__restrict__ qs,
                                                          int32_t *__restrict__ dots, uint32_t N,
                                                          uint32_t nbe, uint32_t stride,
                                                          uint32_t K, uint32_t nt)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * WAVES_PER_WG + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * WAVES_PER_WG;
    const uint32_t C = 8u * nbe;
    const uint32_t nsub = K / 16u;
    for (uint32_t row = wave; row < N; row += nwaves) {
        const uint8_t *r = w + (size_t)row * stride;
        for (uint32_t Q = lane; Q < C; Q += 64u) {
            const ChunkW wt = load_w(r, nbe, Q);
            const uint32_t j = Q + 4u * (Q >> 2);   // sub-block of the chunk's low nibbles
            for (uint32_t t = 0; t < nt; ++t) {
                ChunkAct a;
                const int8_t *qt = qs + (size_t)t * K;
                a.xa = *reinterpret_cast<const uint4 *>(qt + 16u * j);
                a.xb = *reinterpret_cast<const uint4 *>(qt + 16u * j + 64u);
                a.na = -32 * sum16_i8(a.xa);
                a.nb = -32 * sum16_i8(a.xb);
                int Da, Db;
                chunk_dots(wt, a, Q, Da, Db);
                int32_t *o = dots + ((size_t)t * N + row) * nsub;
                o[j] = Da;
                o[j + 4u] = Db;
            }
        }
    }
}

namespace {

template <typename Kern>
hipError_t launch(Kern kern, uint32_t grid, hipStream_t s, const uint8_t *w, const int8_t *qs,
                  const uint16_t *d8, float *y, uint32_t N, uint32_t nbe, uint32_t stride,
                  uint32_t K, uint32_t ldy)
{
    void *args[] = {(void *)&w, (void *)&qs, (void *)&d8, (void *)&y, (void *)&N,
                    (void *)&nbe, (void *)&stride, (void *)&K, (void *)&ldy};
    return hipLaunchKernel((const void *)kern, dim3(grid), dim3(WG), args, 0, s);
}

template <int NT, int CPL>
hipError_t launch_cpl(bool hoist, uint32_t grid, hipStream_t s, const uint8_t *w,
                      const int8_t *qs, const uint16_t *d8, float *y, uint32_t N, uint32_t nbe,
                      uint32_t stride, uint32_t K, uint32_t ldy)
{
    if (hoist)
        return launch(mmvq_unrolled<NT, CPL, true>, grid, s, w, qs, d8, y, N, nbe, stride, K, ldy);
    return launch(mmvq_unrolled<NT, CPL, false>, grid, s, w, qs, d8, y, N, nbe, stride, K, ldy);
}

template <int NT, int... CPLS>
hipError_t dispatch_cpl(int cpl, bool hoist, std::integer_sequence<int, CPLS...>, uint32_t grid,
                        hipStream_t s, const uint8_t *w, const int8_t *qs, const uint16_t *d8,
                        float *y, uint32_t N, uint32_t nbe, uint32_t stride, uint32_t K,
                        uint32_t ldy)
{
    hipError_t e = hipErrorInvalidValue;
    (void)((cpl == CPLS + 1 ? (e = launch_cpl<NT, CPLS + 1>(hoist, grid, s, w, qs, d8, y, N, nbe,
                                                     stride, K, ldy),
                         true)
                      : false) ||
           ...);
    return e;
}

template <int NT>
hipError_t dispatch_nt(uint32_t grid, hipStream_t s, const uint8_t *w, const int8_t *qs,
                       const uint16_t *d8, float *y, uint32_t N, uint32_t nbe, uint32_t stride,
                       uint32_t K, uint32_t ldy)
{
    const int cpl = (int)((8u * nbe + 63u) / 64u);
    if (cpl <= MAX_CPL) {
        const bool hoist = NT * cpl <= 6;
        return dispatch_cpl<NT>(cpl, hoist, std::make_integer_sequence<int, MAX_CPL>{}, grid, s,
                                w, qs, d8, y, N, nbe, stride, K, ldy);
    }
    return launch(mmvq_generic<NT>, grid, s, w, qs, d8, y, N, nbe, stride, K, ldy);
}

uint32_t grid_for(int64_t N, int num_cu)
{
    const int64_t max_waves = (int64_t)num_cu * WAVES_PER_CU;
    const int64_t waves = N < max_waves ? N : max_waves;
    return (uint32_t)((waves + WAVES_PER_WG - 1) / WAVES_PER_WG);
}

}  // namespace

MmvqPlan plan_mmvq(int64_t N, int64_t K, int nt, int num_cu)
{
    MmvqPlan p;
    const int64_t nbe = K / 256;
    p.grid = grid_for(N, num_cu);
    p.cpl = (int)((8 * nbe + 63) / 64);
    p.unrolled = p.cpl <= MAX_CPL;
    p.launches = (nt + MAX_NT_KERNEL - 1) / MAX_NT_KERNEL;
    const int nt0 = nt < MAX_NT_KERNEL ? nt : MAX_NT_KERNEL;
    p.hoist = p.unrolled && nt0 * p.cpl <= 6;
    return p;
}

hipError_t launch_mmvq(const uint8_t *w, const uint8_t *q8, float *y, int64_t N, int64_t K,
                       int nt, int num_cu, hipStream_t s)
{
    const uint32_t nbe = (uint32_t)(K / 256);
    const uint32_t stride = (uint32_t)(((int64_t)nbe * 210 + 15) & ~(int64_t)15);
    const int8_t *qs = reinterpret_cast<const int8_t *>(q8);
    const uint16_t *d8 = reinterpret_cast<const uint16_t *>(q8 + (size_t)nt * K);
    const uint32_t grid = grid_for(N, num_cu);
    const uint32_t Ku = (uint32_t)K, Nu = (uint32_t)N;
    for (int t0 = 0; t0 < nt; t0 += MAX_NT_KERNEL) {
        const int n = nt - t0 < MAX_NT_KERNEL ? nt - t0 : MAX_NT_KERNEL;
        const int8_t *qs_t = qs + (size_t)t0 * K;
        const uint16_t *d8_t = d8 + (size_t)t0 * (K / 32);
        float *y_t = y + (size_t)t0 * N;
        hipError_t e;
        switch (n) {
        case 1: e = dispatch_nt<1>(grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
        case 2: e = dispatch_nt<2>(grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
        case 3: e = dispatch_nt<3>(grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
        default: e = dispatch_nt<4>(grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_subdots(const uint8_t *w, const uint8_t *q8, int32_t *dots, int64_t N,
                          int64_t K, int nt, int num_cu, hipStream_t s)
{
    uint32_t nbe = (uint32_t)(K / 256);
    uint32_t stride = (uint32_t)(((int64_t)nbe * 210 + 15) & ~(int64_t)15);
    const int8_t *qs = reinterpret_cast<const int8_t *>(q8);
    uint32_t grid = grid_for(N, num_cu);
    uint32_t Nu = (uint32_t)N, Ku = (uint32_t)K, ntu = (uint32_t)nt;
    void *args[] = {(void *)&w, (void *)&qs, (void *)&dots, (void *)&Nu,
                    (void *)&nbe, (void *)&stride, (void *)&Ku, (void *)&ntu};
    return hipLaunchKernel((const void *)mmvq_subdots_kernel, dim3(grid), dim3(WG), args, 0, s);
}

}  // namespace q6k
