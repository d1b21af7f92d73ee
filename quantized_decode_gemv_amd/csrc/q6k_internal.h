// q6k_internal.h -- launchers shared between the C ABI layer and the kernel files.
// Shapes and pointers reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace q6k {

// How mmvq_q6k_q8 will run a shape (for tests and reports).
struct MmvqPlan {
    uint32_t grid = 0;      // workgroups of 256 threads (before the occupancy clamp)
    int cpl = 0;            // low-bit chunks per lane per row
    bool unrolled = false;  // a fixed-CPL kernel (else the generic stepping kernel)
    bool shared = false;    // the rows shared by a workgroup's four waves (cpl is then
                            // per thread of the 256)
    bool paired = false;    // two rows per wave, the last chunk slot split between them
    bool tiles = false;     // 16-row tiles on the int8 matrix cores (tiles.hip)
    int act_mode = 0;       // activation operands across rows: 0 re-read per row,
                            // 1 registers, 2 staged in LDS once per workgroup
    int launches = 0;       // one launch per group of up to 4 token columns
    int depth = 1;          // rows (paired: pairs) in flight per wave; tiles: tile
                            // buffers per workgroup
};

MmvqPlan plan_mmvq(int type, int64_t N, int64_t K, int nt, int num_cu);

// Workgroups of `kern` (256 threads) that fit on one CU at once, with `lds` bytes of
// dynamic LDS; 0 if the runtime cannot say. Kept per device, kernel and size.
int wg_fit(const void *kern, uint32_t lds = 0);

// The q6_K GEMV at 3-4 tokens on 16-row tiles with the int8 matrix cores (tiles.hip):
// rows of 20 super-blocks, at least 12 (4 tokens) or 24 (3 tokens) tiles per CU. qs, d8:
// the token group's q8 plane fields; y: [nt][ldy].
bool tiles_ok(int type, int64_t N, int64_t K, int nt, int num_cu);
hipError_t launch_tiles(const uint8_t *w, const int8_t *qs, const uint16_t *d8, float *y,
                        int64_t N, int64_t ldy, int nt, int num_cu, hipStream_t s);
// type: a KqType of kq_format.h (the weight rows are that type's split-plane rows).
hipError_t launch_mmvq(int type, const uint8_t *w, const uint8_t *q8, float *y, int64_t N,
                       int64_t K, int nt, int num_cu, hipStream_t s);
hipError_t launch_subdots(int type, const uint8_t *w, const uint8_t *q8, int32_t *dots,
                          int64_t N, int64_t K, int nt, int num_cu, hipStream_t s);
// RMSNorm -> q8 -> GEMV: one kernel when rmsnorm_mmvq_fused(K, nt), else the
// producer then the GEMV (same results bit for bit). xn may be null.
bool rmsnorm_mmvq_fused(int64_t K, int nt);
hipError_t launch_rmsnorm_mmvq(int type, const uint8_t *w, const float *x, const float *gamma,
                               float eps, float *xn, uint8_t *q8, float *y, int64_t N, int64_t K,
                               int nt, int num_cu, hipStream_t s);
// Form B: gate+up GEMV, SwiGLU and q8 of one token in one kernel when
// gate_up_swiglu_fused(K), else the GEMV then the SwiGLU producer (same results bit
// for bit). w: 2*Nh rows (gate, then up); gu: float [2*Nh]; y may be null.
bool gate_up_swiglu_fused(int64_t K);
hipError_t launch_gate_up_swiglu(int type, const uint8_t *w, const uint8_t *q8_in, float *gu,
                                 float *y, uint8_t *q8_out, int64_t Nh, int64_t K, int num_cu,
                                 hipStream_t s);
hipError_t launch_quant(const float *x, uint8_t *q8, int64_t K, int nt, hipStream_t s);
hipError_t launch_rmsnorm_quant(const float *x, const float *gamma, float eps, float *y,
                                uint8_t *q8, int64_t K, int nt, hipStream_t s);
// y may be null (not stored).
hipError_t launch_swiglu_quant(const float *g, const float *u, float *y, uint8_t *q8, int64_t K,
                               int nt, hipStream_t s);
hipError_t launch_repack(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K,
                         hipStream_t s);
void repack_host(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K);
void unpack_host(int type, const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K);

}  // namespace q6k
