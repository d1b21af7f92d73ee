// abi.hip -- the extern "C" entry points of libq6kdpl.so (include/q6kdpl.h).
//
// Each entry point validates every argument (shape, NULL, 16-byte alignment,
// output/input overlap) before queuing anything, then queues its kernels on the
// caller's stream and returns. No entry point allocates, synchronises or keeps data
// of a call. Process-wide state: the per-device table of compute-unit counts below,
// and the per-device, per-kernel occupancy table of the launchers (wg_fit in
// mmvq.hip); both are filled on first use and kept until the process ends.

#include <atomic>

#include "../../include/q6kdpl.h"
#include "kq_format.h"
#include "q6k_internal.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

bool weight_shape_ok(int64_t N, int64_t K)
{
    return N >= 1 && N <= Q6K_MAX_N && K > 0 && K <= Q6K_MAX_K && K % 256 == 0;
}

bool act_shape_ok(int64_t K, int nt)
{
    return K > 0 && K <= Q6K_MAX_K && K % 32 == 0 && nt >= 1 && nt <= Q6K_MAX_NT;
}

int from_hip(hipError_t e) { return e == hipSuccess ? Q6K_OK : Q6K_E_HIP; }

// Sub-block dots per row written by the subdots test entry: q6_K 16-element
// sub-blocks, q4_K / q5_K 32-element ones.
int64_t subdots_per_row(int type, int64_t K) { return type == q6k::KQT_Q6_K ? K / 16 : K / 32; }

constexpr int MAX_DEV = 64;
std::atomic<int> g_cu_count[MAX_DEV];

// Compute units of the device that owns `s` (the current device for NULL).
int cu_count(hipStream_t s, int *cu)
{
    int dev = 0;
    if (s != nullptr) {
        if (hipStreamGetDevice(s, &dev) != hipSuccess)
            return Q6K_E_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return Q6K_E_HIP;
    }
    if (dev < 0 || dev >= MAX_DEV)
        return Q6K_E_HIP;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            return Q6K_E_HIP;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    *cu = n;
    return Q6K_OK;
}

}  // namespace

extern "C" {

const char *q6k_strerror(int code)
{
    switch (code) {
    case Q6K_OK: return "ok";
    case Q6K_E_SHAPE: return "shape out of range (N, K or nt; K must be a multiple of 256 for "
                             "weights, of 32 for activations)";
    case Q6K_E_NULL: return "a required pointer is NULL";
    case Q6K_E_ALIGN: return "a device pointer is not 16-byte aligned";
    case Q6K_E_ALIAS: return "an output range overlaps an input range";
    case Q6K_E_HIP: return "the HIP runtime refused a launch or device query";
    case Q6K_E_TYPE: return "unknown weight type (KQ_Q4_K, KQ_Q5_K and KQ_Q6_K are taken)";
    default: return "unknown q6kdpl error code";
    }
}

const char *q6k_version(void) { return "q6kdpl 0.1 gfx950"; }

size_t kq_block_bytes(int type) { return q6k::kq_known(type) ? q6k::kq_block_bytes(type) : 0; }

size_t kq_dpl_row_stride(int type, int64_t K)
{
    if (!q6k::kq_known(type) || K <= 0 || K > Q6K_MAX_K || K % 256)
        return 0;
    return (size_t)q6k::kq_row_stride(type, (uint64_t)(K / 256));
}

size_t kq_dpl_bytes(int type, int64_t N, int64_t K)
{
    if (!q6k::kq_known(type) || !weight_shape_ok(N, K))
        return 0;
    return (size_t)N * kq_dpl_row_stride(type, K);
}

size_t kq_raw_bytes(int type, int64_t N, int64_t K)
{
    if (!q6k::kq_known(type) || !weight_shape_ok(N, K))
        return 0;
    return (size_t)N * (size_t)(K / 256) * q6k::kq_block_bytes(type);
}

size_t q6k_dpl_row_stride(int64_t K) { return kq_dpl_row_stride(KQ_Q6_K, K); }
size_t q6k_dpl_bytes(int64_t N, int64_t K) { return kq_dpl_bytes(KQ_Q6_K, N, K); }
size_t q6k_raw_bytes(int64_t N, int64_t K) { return kq_raw_bytes(KQ_Q6_K, N, K); }

size_t q8_plane_bytes(int64_t K, int nt)
{
    if (!act_shape_ok(K, nt))
        return 0;
    return (size_t)nt * (size_t)K + (size_t)nt * (size_t)(K / 32) * 2u;
}

int repack_kq_dpl_host(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (!weight_shape_ok(N, K))
        return Q6K_E_SHAPE;
    if (!raw || !dpl)
        return Q6K_E_NULL;
    if (overlap(raw, kq_raw_bytes(type, N, K), dpl, kq_dpl_bytes(type, N, K)))
        return Q6K_E_ALIAS;
    q6k::repack_host(type, raw, dpl, N, K);
    return Q6K_OK;
}

int unpack_kq_dpl_host(int type, const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (!weight_shape_ok(N, K))
        return Q6K_E_SHAPE;
    if (!raw || !dpl)
        return Q6K_E_NULL;
    if (overlap(raw, kq_raw_bytes(type, N, K), dpl, kq_dpl_bytes(type, N, K)))
        return Q6K_E_ALIAS;
    q6k::unpack_host(type, dpl, raw, N, K);
    return Q6K_OK;
}

int repack_kq_dpl(int type, const void *raw_dev, void *dpl_dev, int64_t N, int64_t K,
                  void *stream)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (!weight_shape_ok(N, K))
        return Q6K_E_SHAPE;
    if (!raw_dev || !dpl_dev)
        return Q6K_E_NULL;
    if (!aligned16(dpl_dev))
        return Q6K_E_ALIGN;
    if (overlap(raw_dev, kq_raw_bytes(type, N, K), dpl_dev, kq_dpl_bytes(type, N, K)))
        return Q6K_E_ALIAS;
    return from_hip(q6k::launch_repack(type, (const uint8_t *)raw_dev, (uint8_t *)dpl_dev, N, K,
                                       (hipStream_t)stream));
}

int repack_q6k_dpl_host(const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K)
{
    return repack_kq_dpl_host(KQ_Q6_K, raw, dpl, N, K);
}

int unpack_q6k_dpl_host(const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K)
{
    return unpack_kq_dpl_host(KQ_Q6_K, dpl, raw, N, K);
}

int repack_q6k_dpl(const void *raw_dev, void *dpl_dev, int64_t N, int64_t K, void *stream)
{
    return repack_kq_dpl(KQ_Q6_K, raw_dev, dpl_dev, N, K, stream);
}

int quant_q8(const float *x, void *q8, int64_t K, int nt, void *stream)
{
    if (!act_shape_ok(K, nt))
        return Q6K_E_SHAPE;
    if (!x || !q8)
        return Q6K_E_NULL;
    if (!aligned16(x) || !aligned16(q8))
        return Q6K_E_ALIGN;
    if (overlap(x, (size_t)nt * K * 4u, q8, q8_plane_bytes(K, nt)))
        return Q6K_E_ALIAS;
    return from_hip(q6k::launch_quant(x, (uint8_t *)q8, K, nt, (hipStream_t)stream));
}

int rmsnorm_quant_q8(const float *x, const float *gamma, float eps, float *y, void *q8,
                     int64_t K, int nt, void *stream)
{
    if (!act_shape_ok(K, nt))
        return Q6K_E_SHAPE;
    if (!x || !gamma || !y || !q8)
        return Q6K_E_NULL;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(y) || !aligned16(q8))
        return Q6K_E_ALIGN;
    const size_t nx = (size_t)nt * K * 4u, ng = (size_t)K * 4u, nq = q8_plane_bytes(K, nt);
    if (overlap(y, nx, x, nx) || overlap(y, nx, gamma, ng) || overlap(q8, nq, x, nx) ||
        overlap(q8, nq, gamma, ng) || overlap(q8, nq, y, nx))
        return Q6K_E_ALIAS;
    return from_hip(
        q6k::launch_rmsnorm_quant(x, gamma, eps, y, (uint8_t *)q8, K, nt, (hipStream_t)stream));
}

int swiglu_quant_q8(const float *g, const float *u, float *y, void *q8, int64_t K, int nt,
                    void *stream)
{
    if (!act_shape_ok(K, nt))
        return Q6K_E_SHAPE;
    if (!g || !u || !y || !q8)
        return Q6K_E_NULL;
    if (!aligned16(g) || !aligned16(u) || !aligned16(y) || !aligned16(q8))
        return Q6K_E_ALIGN;
    const size_t nx = (size_t)nt * K * 4u, nq = q8_plane_bytes(K, nt);
    // y may be g or u exactly (in place); any other overlap is refused
    if ((y != g && overlap(y, nx, g, nx)) || (y != u && overlap(y, nx, u, nx)) ||
        overlap(q8, nq, g, nx) || overlap(q8, nq, u, nx) || overlap(q8, nq, y, nx))
        return Q6K_E_ALIAS;
    return from_hip(q6k::launch_swiglu_quant(g, u, y, (uint8_t *)q8, K, nt, (hipStream_t)stream));
}

int mmvq_kq_q8(int type, const void *w_dpl, const void *q8, float *y, int64_t N, int64_t K,
               int nt, void *stream)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (!weight_shape_ok(N, K) || !act_shape_ok(K, nt))
        return Q6K_E_SHAPE;
    if (!w_dpl || !q8 || !y)
        return Q6K_E_NULL;
    if (!aligned16(w_dpl) || !aligned16(q8) || !aligned16(y))
        return Q6K_E_ALIGN;
    const size_t ny = (size_t)nt * N * 4u;
    if (overlap(y, ny, w_dpl, kq_dpl_bytes(type, N, K)) || overlap(y, ny, q8, q8_plane_bytes(K, nt)))
        return Q6K_E_ALIAS;
    int cu = 0;
    int rc = cu_count((hipStream_t)stream, &cu);
    if (rc != Q6K_OK)
        return rc;
    return from_hip(q6k::launch_mmvq(type, (const uint8_t *)w_dpl, (const uint8_t *)q8, y, N, K,
                                     nt, cu, (hipStream_t)stream));
}

int mmvq_q6k_q8(const void *w_dpl, const void *q8, float *y, int64_t N, int64_t K, int nt,
                void *stream)
{
    return mmvq_kq_q8(KQ_Q6_K, w_dpl, q8, y, N, K, nt, stream);
}

int mmvq_kq_rmsnorm_q8(int type, const void *w_dpl, const float *x, const float *gamma,
                       float eps, float *xn, void *q8, float *y, int64_t N, int64_t K, int nt,
                       void *stream)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (!weight_shape_ok(N, K) || !act_shape_ok(K, nt))
        return Q6K_E_SHAPE;
    if (!w_dpl || !x || !gamma || !q8 || !y)
        return Q6K_E_NULL;
    if (!aligned16(w_dpl) || !aligned16(x) || !aligned16(gamma) || !aligned16(q8) ||
        !aligned16(y) || (xn && !aligned16(xn)))
        return Q6K_E_ALIGN;
    const size_t nw = kq_dpl_bytes(type, N, K), nx = (size_t)nt * K * 4u, ng = (size_t)K * 4u;
    const size_t nq = q8_plane_bytes(K, nt), ny = (size_t)nt * N * 4u;
    // every output against every input and every other output
    const void *in[3] = {w_dpl, x, gamma};
    const size_t in_n[3] = {nw, nx, ng};
    const void *out[3] = {q8, y, xn};
    const size_t out_n[3] = {nq, ny, xn ? nx : 0};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 3; ++i)
            if (overlap(out[o], out_n[o], in[i], in_n[i]))
                return Q6K_E_ALIAS;
        for (int p = o + 1; p < 3; ++p)
            if (overlap(out[o], out_n[o], out[p], out_n[p]))
                return Q6K_E_ALIAS;
    }
    int cu = 0;
    int rc = cu_count((hipStream_t)stream, &cu);
    if (rc != Q6K_OK)
        return rc;
    return from_hip(q6k::launch_rmsnorm_mmvq(type, (const uint8_t *)w_dpl, x, gamma, eps, xn,
                                             (uint8_t *)q8, y, N, K, nt, cu,
                                             (hipStream_t)stream));
}

int mmvq_q6k_rmsnorm_q8(const void *w_dpl, const float *x, const float *gamma, float eps,
                        float *xn, void *q8, float *y, int64_t N, int64_t K, int nt, void *stream)
{
    return mmvq_kq_rmsnorm_q8(KQ_Q6_K, w_dpl, x, gamma, eps, xn, q8, y, N, K, nt, stream);
}

int q6k_rmsnorm_mmvq_fused(int64_t N, int64_t K, int nt)
{
    if (!weight_shape_ok(N, K) || !act_shape_ok(K, nt))
        return Q6K_E_SHAPE;
    return q6k::rmsnorm_mmvq_fused(K, nt) ? 1 : 0;
}

int mmvq_kq_gate_up_swiglu_q8(int type, const void *w_gu, const void *q8_in, float *gu, float *y,
                              void *q8_out, int64_t Nh, int64_t K, int nt, void *stream)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (nt != 1 || Nh < 1 || Nh % 32 || Nh > Q6K_MAX_K || !weight_shape_ok(2 * Nh, K) ||
        !act_shape_ok(K, 1))
        return Q6K_E_SHAPE;
    if (!w_gu || !q8_in || !gu || !q8_out)
        return Q6K_E_NULL;
    if (!aligned16(w_gu) || !aligned16(q8_in) || !aligned16(gu) || !aligned16(q8_out) ||
        (y && !aligned16(y)))
        return Q6K_E_ALIGN;
    const size_t nw = kq_dpl_bytes(type, 2 * Nh, K), nq = q8_plane_bytes(K, 1);
    const size_t ngu = (size_t)2 * Nh * 4u, ny = (size_t)Nh * 4u, nqo = q8_plane_bytes(Nh, 1);
    const void *in[2] = {w_gu, q8_in};
    const size_t in_n[2] = {nw, nq};
    const void *out[3] = {gu, q8_out, y};
    const size_t out_n[3] = {ngu, nqo, y ? ny : 0};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 2; ++i)
            if (overlap(out[o], out_n[o], in[i], in_n[i]))
                return Q6K_E_ALIAS;
        for (int p = o + 1; p < 3; ++p)
            if (overlap(out[o], out_n[o], out[p], out_n[p]))
                return Q6K_E_ALIAS;
    }
    int cu = 0;
    int rc = cu_count((hipStream_t)stream, &cu);
    if (rc != Q6K_OK)
        return rc;
    return from_hip(q6k::launch_gate_up_swiglu(type, (const uint8_t *)w_gu, (const uint8_t *)q8_in,
                                               gu, y, (uint8_t *)q8_out, Nh, K, cu,
                                               (hipStream_t)stream));
}

int kq_gate_up_swiglu_fused(int64_t Nh, int64_t K)
{
    if (Nh < 1 || Nh % 32 || Nh > Q6K_MAX_K || !weight_shape_ok(2 * Nh, K))
        return Q6K_E_SHAPE;
    return q6k::gate_up_swiglu_fused(K) ? 1 : 0;
}

int mmvq_kq_q8_subdots(int type, const void *w_dpl, const void *q8, int32_t *dots, int64_t N,
                       int64_t K, int nt, void *stream)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (!weight_shape_ok(N, K) || !act_shape_ok(K, nt))
        return Q6K_E_SHAPE;
    if (!w_dpl || !q8 || !dots)
        return Q6K_E_NULL;
    if (!aligned16(w_dpl) || !aligned16(q8) || !aligned16(dots))
        return Q6K_E_ALIGN;
    const size_t nd = (size_t)nt * N * subdots_per_row(type, K) * 4u;
    if (overlap(dots, nd, w_dpl, kq_dpl_bytes(type, N, K)) ||
        overlap(dots, nd, q8, q8_plane_bytes(K, nt)))
        return Q6K_E_ALIAS;
    int cu = 0;
    int rc = cu_count((hipStream_t)stream, &cu);
    if (rc != Q6K_OK)
        return rc;
    return from_hip(q6k::launch_subdots(type, (const uint8_t *)w_dpl, (const uint8_t *)q8, dots, N,
                                        K, nt, cu, (hipStream_t)stream));
}

int mmvq_q6k_q8_subdots(const void *w_dpl, const void *q8, int32_t *dots, int64_t N, int64_t K,
                        int nt, void *stream)
{
    return mmvq_kq_q8_subdots(KQ_Q6_K, w_dpl, q8, dots, N, K, nt, stream);
}

int kq_mmvq_plan(int type, int64_t N, int64_t K, int nt, int num_cu, int32_t *out6)
{
    if (!q6k::kq_known(type))
        return Q6K_E_TYPE;
    if (!weight_shape_ok(N, K) || !act_shape_ok(K, nt) || num_cu < 1)
        return Q6K_E_SHAPE;
    if (!out6)
        return Q6K_E_NULL;
    const q6k::MmvqPlan p = q6k::plan_mmvq(type, N, K, nt, num_cu);
    out6[0] = (int32_t)p.grid;
    out6[1] = p.cpl;
    out6[2] = p.tiles ? 4 : p.paired ? 3 : p.shared ? 2 : p.unrolled ? 1 : 0;
    out6[3] = p.act_mode;
    out6[4] = p.launches;
    out6[5] = p.depth;
    return Q6K_OK;
}

int q6k_mmvq_plan(int64_t N, int64_t K, int nt, int num_cu, int32_t *out6)
{
    return kq_mmvq_plan(KQ_Q6_K, N, K, nt, num_cu, out6);
}

}  // extern "C"
