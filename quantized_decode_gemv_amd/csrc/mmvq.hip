// mmvq.hip -- q6_K (dpl rows) x q8 decode GEMV kernels for gfx950, and their shape
// dispatch.
//
// What is computed (D4-2 §3.2 Excerpt C, the per-unit accumulation; D4-4 §3.2
// Excerpt B, the dpl unit load): y[t][r] = sum over the row's 16-element sub-blocks
// of d * sc * d8 * D, D the exact int32 dot of (q - 32) with the int8 activations.
//
// Geometry (one design for every shape):
//  - one wave64 owns one row at a time and walks rows with a stride of the grid's
//    wave count, so the grid streams neighbouring rows together;
//  - lane L takes the row's 16-byte low-bit chunks Q = L, L + 64, ... (q6k_unit.h):
//    each low-bit load instruction is one contiguous 1 KB request, each high-bit
//    load 512 B (two lanes share a chunk), each scale load 128 B, each d load 16 B;
//  - a lane's byte offsets inside a row are the same for every row, so they are
//    computed once; each row gets a buffer descriptor whose extent is the row's
//    bytes, and loads are buffer loads at those offsets. The low/high-bit loads are
//    non-temporal (each weight byte is read once per call); the small scale loads
//    keep the default policy (each 64-byte line of them is touched by three load
//    instructions of the same row);
//  - lanes past the row's last chunk load a duplicate of the last chunk and
//    contribute exactly 0, and a wave's look-ahead past the last row uses an empty
//    descriptor (its loads return zeros without touching memory), so loads are
//    branch-free and their waits are counted exactly;
//  - DEPTH rows are in flight per wave: the next rows' loads are issued before the
//    current row's arithmetic (scheduling barriers keep the compiler from sinking
//    them), so a wave never idles with nothing requested;
//  - a lane's activation operands are the same for every row; they stay in
//    registers (HOIST) when they fit, else they are re-read per row (cached);
//  - a row ends with one reduction for all its token columns (DPP inside each
//    16-lane row, lane swaps across rows); lanes 0..NT-1 write the NT outputs.
// The chunks per lane (CPL = ceil(8*nbe/64)) is a template parameter up to
// MAX_CPL, so a row's loads are issued back to back; longer rows take the generic
// kernel, which walks a row in runtime steps of 4 chunks per lane. Every kernel
// masks every chunk with Q < 8*nbe and loops rows while row < N, so it covers all
// units of all rows of any shape it is launched on (D4-2 §2: a dispatch that routes
// a shape to a kernel covering fewer units silently drops work).

#include "q6k_internal.h"
#include "q6k_unit.h"

namespace q6k {

constexpr int WG = 256;             // 4 waves per workgroup
constexpr int WAVES_PER_WG = WG / 64;
constexpr int MAX_CPL = 12;         // nbe <= 96 take the fixed-length kernels
constexpr int MAX_NT_KERNEL = 4;    // token columns per launch (more -> several launches)
constexpr int POLICY_STREAM = 2;    // buffer-load cache policy: non-temporal
constexpr int POLICY_DEFAULT = 0;
constexpr int DESC_WORD3 = 0x00020000;  // raw buffer, 32-bit format fields unused

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// Byte offsets of one chunk's operands inside a row.
struct ChunkOffs {
    uint32_t ql, qh, sc, d;
};

__device__ __forceinline__ ChunkOffs chunk_offsets(uint32_t Q, uint32_t nbe)
{
    const uint32_t G = Q >> 2;
    ChunkOffs o;
    o.ql = 16u * Q;
    o.qh = 128u * nbe + 16u * (2u * G + (Q & 1u));
    o.sc = 192u * nbe + 8u * G;
    o.d = 208u * nbe + 2u * (Q >> 3);
    return o;
}

// Descriptor of one row; extent 0 for a look-ahead row past the end, whose loads
// then return zeros without a memory request.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_desc(const uint8_t *w, uint32_t row,
                                                           uint32_t stride, bool real = true)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)(w + (size_t)row * stride), (short)0,
                                             real ? (int)stride : 0, DESC_WORD3);
}

__device__ __forceinline__ ChunkW load_chunk(__amdgpu_buffer_rsrc_t r, const ChunkOffs &o)
{
    const u32x4v a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)o.ql, 0, POLICY_STREAM);
    const u32x4v b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)o.qh, 0, POLICY_STREAM);
    const u32x2v c = __builtin_amdgcn_raw_buffer_load_b64(r, (int)o.sc, 0, POLICY_DEFAULT);
    const uint16_t d = __builtin_amdgcn_raw_buffer_load_b16(r, (int)o.d, 0, POLICY_DEFAULT);
    ChunkW w;
    w.ql = make_uint4(a.x, a.y, a.z, a.w);
    w.qh = make_uint4(b.x, b.y, b.z, b.w);
    w.sc = make_uint2(c.x, c.y);
    w.d = d;
    return w;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + dpp_mov<CTRL>(v);
}

// Sums over a wave64 of NT <= 4 per-lane values (one per token column). The
// first steps transpose while they add: at the pair step a lane keeps the tokens
// of its parity and hands the others to its partner, at the quad step likewise by
// the second lane bit, so afterwards lane l carries only token (l & 3) (for NT = 2:
// l & 1). Rotations by 4 and 8 lanes finish each 16-lane row; two lane-swaps add
// the four rows. Lane l then holds the total of token (l & 3) (NT = 1: of the only
// token). The adds always pair the same lanes in the same order, so results are
// reproducible run to run.
template <int NT>
__device__ __forceinline__ float reduce_tokens(const float (&a)[NT], uint32_t lane)
{
    static_assert(NT >= 1 && NT <= 4, "one to four token columns per reduction");
    float v;
    if constexpr (NT == 1) {
        v = dpp_add<0xB1>(a[0]);                     // quad_perm [1,0,3,2]
        v = dpp_add<0x4E>(v);                        // quad_perm [2,3,0,1]
    } else {
        const bool b0 = (lane & 1u) != 0;
        if constexpr (NT == 2) {
            v = (b0 ? a[1] : a[0]) + dpp_mov<0xB1>(b0 ? a[0] : a[1]);
            v = dpp_add<0x4E>(v);
        } else {
            const bool b1 = (lane & 2u) != 0;
            const float a2 = a[2], a3 = NT > 3 ? a[NT - 1] : 0.0f;
            const float p = (b0 ? a[1] : a[0]) + dpp_mov<0xB1>(b0 ? a[0] : a[1]);
            const float q = (b0 ? a3 : a2) + dpp_mov<0xB1>(b0 ? a2 : a3);
            v = (b1 ? q : p) + dpp_mov<0x4E>(b1 ? p : q);
        }
    }
    v = dpp_add<0x124>(v);                           // row_ror:4
    v = dpp_add<0x128>(v);                           // row_ror:8
    // (each swap's two results are copied into plain integers before their bit
    // casts: a bit cast applied straight to an element of the returned pair reads
    // element 0 for both)
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned h0 = h[0], h1 = h[1];
    v = __builtin_bit_cast(float, h0) + __builtin_bit_cast(float, h1);
    const unsigned u2 = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u2, u2, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// The lane that holds token t's total after reduce_tokens.
template <int NT>
__device__ __forceinline__ bool stores_token(uint32_t lane, uint32_t &t)
{
    t = NT == 1 ? 0u : lane;
    return lane < (uint32_t)NT;
}

// Per-lane state that is the same for every row a wave visits.
template <int NT, int CPL, bool HOIST>
struct LaneState {
    ChunkOffs off[CPL];
    uint32_t Q[CPL];        // chunk index (clamped to the last chunk past the row end)
    bool live[CPL];         // false: duplicate load, contributes 0
    ChunkAct act[HOIST ? CPL : 1][NT];
};

template <int NT, int CPL, bool HOIST>
__device__ __forceinline__ void lane_init(LaneState<NT, CPL, HOIST> &st, uint32_t lane,
                                          uint32_t nbe, const int8_t *qs, const uint16_t *d8,
                                          uint32_t K)
{
    const uint32_t C = 8u * nbe;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const uint32_t Q = lane + 64u * i;
        st.live[i] = Q < C;
        st.Q[i] = st.live[i] ? Q : C - 1u;
        st.off[i] = chunk_offsets(st.Q[i], nbe);
        if constexpr (HOIST) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                st.act[i][t] = load_act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), st.Q[i]);
        }
    }
}

template <int NT, int CPL, bool HOIST>
__device__ __forceinline__ void load_row(ChunkW (&dst)[CPL], const uint8_t *w, uint32_t row,
                                         uint32_t N, uint32_t stride,
                                         const LaneState<NT, CPL, HOIST> &st)
{
    const bool real = row < N;
    const __amdgpu_buffer_rsrc_t r = row_desc(w, real ? row : 0u, stride, real);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        dst[i] = load_chunk(r, st.off[i]);
}

template <int NT, int CPL, bool HOIST>
__device__ __forceinline__ void finish_row(const ChunkW (&src)[CPL],
                                           const LaneState<NT, CPL, HOIST> &st,
                                           const int8_t *qs, const uint16_t *d8, uint32_t K,
                                           float *y, uint32_t ldy, uint32_t row, uint32_t lane)
{
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const float d = st.live[i] ? f16_bits_to_f32(src[i].d) : 0.0f;   // 0 drops the chunk
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if constexpr (HOIST) {
                acc[t] += chunk_partial_d(src[i], st.act[i][t], st.Q[i], d);
            } else {
                const ChunkAct a =
                    load_act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), st.Q[i]);
                acc[t] += chunk_partial_d(src[i], a, st.Q[i], d);
            }
        }
    }
    const float s = reduce_tokens<NT>(acc, lane);
    uint32_t t;
    if (stores_token<NT>(lane, t))
        y[(size_t)t * ldy + row] = s;
}

// Rows with at most MAX_CPL chunks per lane; DEPTH rows in flight per wave.
template <int NT, int CPL, int DEPTH, bool HOIST>
__global__ __launch_bounds__(WG) void mmvq_rows(const uint8_t *__restrict__ w,
                                                const int8_t *__restrict__ qs,
                                                const uint16_t *__restrict__ d8,
                                                float *__restrict__ y, uint32_t N, uint32_t nbe,
                                                uint32_t stride, uint32_t K, uint32_t ldy)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * WAVES_PER_WG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * WAVES_PER_WG;
    LaneState<NT, CPL, HOIST> st;
    lane_init(st, lane, nbe, qs, d8, K);
    if (wave >= N)
        return;
    // look-ahead rows past the end get an empty descriptor (load_row), so every load
    // stays unconditional and their results are never reduced
#define Q6K_FINISH(BUF, ROW) finish_row<NT, CPL, HOIST>(BUF, st, qs, d8, K, y, ldy, ROW, lane)
    if constexpr (DEPTH == 1) {
        ChunkW A[CPL];
        for (uint32_t row = wave; row < N; row += nw) {
            load_row(A, w, row, N, stride, st);
            Q6K_FINISH(A, row);
        }
    } else if constexpr (DEPTH == 2) {
        ChunkW A[CPL], B[CPL];
        uint32_t row = wave;
        load_row(A, w, row, N, stride, st);
        for (;;) {
            const uint32_t r1 = row + nw;
            load_row(B, w, r1, N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
            Q6K_FINISH(A, row);
            if (r1 >= N)
                break;
            const uint32_t r2 = r1 + nw;
            load_row(A, w, r2, N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
            Q6K_FINISH(B, r1);
            if (r2 >= N)
                break;
            row = r2;
        }
    } else {
        ChunkW A[CPL], B[CPL], Cb[CPL];
        uint32_t row = wave;
        load_row(A, w, row, N, stride, st);
        load_row(B, w, row + nw, N, stride, st);
        for (;;) {
            const uint32_t r1 = row + nw, r2 = r1 + nw, r3 = r2 + nw;
            load_row(Cb, w, r2, N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
            Q6K_FINISH(A, row);
            if (r1 >= N)
                break;
            load_row(A, w, r3, N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
            Q6K_FINISH(B, r1);
            if (r2 >= N)
                break;
            load_row(B, w, r3 + nw, N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
            Q6K_FINISH(Cb, r2);
            if (r3 >= N)
                break;
            row = r3;
        }
    }
#undef Q6K_FINISH
}

// Any row length: a row is walked in steps of STEP chunks per lane.
template <int NT>
__global__ __launch_bounds__(WG) void mmvq_long(const uint8_t *__restrict__ w,
                                                const int8_t *__restrict__ qs,
                                                const uint16_t *__restrict__ d8,
                                                float *__restrict__ y, uint32_t N, uint32_t nbe,
                                                uint32_t stride, uint32_t K, uint32_t ldy)
{
    constexpr int STEP = 4;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * WAVES_PER_WG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * WAVES_PER_WG;
    const uint32_t C = 8u * nbe;
    for (uint32_t row = wave; row < N; row += nw) {
        const __amdgpu_buffer_rsrc_t r = row_desc(w, row, stride);
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = 0.0f;
        for (uint32_t base = 0; base < C; base += 64u * STEP) {
            ChunkW wt[STEP];
            uint32_t Qs[STEP];
            bool live[STEP];
#pragma unroll
            for (int i = 0; i < STEP; ++i) {
                const uint32_t Q = base + lane + 64u * i;
                live[i] = Q < C;
                Qs[i] = live[i] ? Q : C - 1u;
                wt[i] = load_chunk(r, chunk_offsets(Qs[i], nbe));
            }
#pragma unroll
            for (int i = 0; i < STEP; ++i) {
                const float d = live[i] ? f16_bits_to_f32(wt[i].d) : 0.0f;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const ChunkAct a =
                        load_act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), Qs[i]);
                    acc[t] += chunk_partial_d(wt[i], a, Qs[i], d);
                }
            }
        }
        const float s = reduce_tokens<NT>(acc, lane);
        uint32_t t;
        if (stores_token<NT>(lane, t))
            y[(size_t)t * ldy + row] = s;
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

// The fixed-length kernel's shape for (NT, CPL): rows in flight per wave, whether the
// activation operands stay in registers, and workgroups per CU, chosen so that
// weights-in-flight plus activation registers stay near 150 VGPRs.
struct RowsCfg {
    int depth;
    bool hoist;
    int wg_per_cu;
};

RowsCfg rows_cfg(int nt, int cpl)
{
    const int work = nt * cpl;
    if (work <= 3)
        return {3, true, 1};
    if (work <= 6 || (cpl <= 3 && work <= 12))
        return {2, true, 2};
    return {1, false, 2};
}

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
hipError_t launch_cpl(const RowsCfg &c, uint32_t grid, hipStream_t s, const uint8_t *w,
                      const int8_t *qs, const uint16_t *d8, float *y, uint32_t N, uint32_t nbe,
                      uint32_t stride, uint32_t K, uint32_t ldy)
{
    // only the (depth, hoist) pairs rows_cfg can pick for this NT * CPL are built
    if constexpr (NT * CPL <= 3) {
        if (c.depth == 3)
            return launch(mmvq_rows<NT, CPL, 3, true>, grid, s, w, qs, d8, y, N, nbe, stride, K, ldy);
    } else if constexpr (NT * CPL <= 6 || (CPL <= 3 && NT * CPL <= 12)) {
        if (c.depth == 2)
            return launch(mmvq_rows<NT, CPL, 2, true>, grid, s, w, qs, d8, y, N, nbe, stride, K, ldy);
    } else {
        if (c.depth == 1)
            return launch(mmvq_rows<NT, CPL, 1, false>, grid, s, w, qs, d8, y, N, nbe, stride, K, ldy);
    }
    return hipErrorInvalidValue;
}

template <int NT, int... CPLS>
hipError_t dispatch_cpl(int cpl, const RowsCfg &c, std::integer_sequence<int, CPLS...>,
                        uint32_t grid, hipStream_t s, const uint8_t *w, const int8_t *qs,
                        const uint16_t *d8, float *y, uint32_t N, uint32_t nbe, uint32_t stride,
                        uint32_t K, uint32_t ldy)
{
    hipError_t e = hipErrorInvalidValue;
    (void)((cpl == CPLS + 1 ? (e = launch_cpl<NT, CPLS + 1>(c, grid, s, w, qs, d8, y, N, nbe,
                                                            stride, K, ldy),
                               true)
                            : false) ||
           ...);
    return e;
}

// Workgroups: whole multiples of the CU count (an uneven count leaves some CUs one
// workgroup short), never more waves than rows.
uint32_t grid_for(int64_t N, int num_cu, int wg_per_cu)
{
    const int64_t need = (N + WAVES_PER_WG - 1) / WAVES_PER_WG;
    const int64_t full = (int64_t)num_cu * wg_per_cu;
    return (uint32_t)(need < full ? need : full);
}

}  // namespace

MmvqPlan plan_mmvq(int64_t N, int64_t K, int nt, int num_cu)
{
    MmvqPlan p;
    const int64_t nbe = K / 256;
    p.cpl = (int)((8 * nbe + 63) / 64);
    p.unrolled = p.cpl <= MAX_CPL;
    p.launches = (nt + MAX_NT_KERNEL - 1) / MAX_NT_KERNEL;
    const int nt0 = nt < MAX_NT_KERNEL ? nt : MAX_NT_KERNEL;
    const RowsCfg c = p.unrolled ? rows_cfg(nt0, p.cpl) : RowsCfg{1, false, 2};
    p.hoist = p.unrolled && c.hoist;
    p.depth = c.depth;
    p.grid = grid_for(N, num_cu, c.wg_per_cu);
    return p;
}

hipError_t launch_mmvq(const uint8_t *w, const uint8_t *q8, float *y, int64_t N, int64_t K,
                       int nt, int num_cu, hipStream_t s)
{
    const uint32_t nbe = (uint32_t)(K / 256);
    const uint32_t stride = (uint32_t)(((int64_t)nbe * 210 + 15) & ~(int64_t)15);
    const int8_t *qs = reinterpret_cast<const int8_t *>(q8);
    const uint16_t *d8 = reinterpret_cast<const uint16_t *>(q8 + (size_t)nt * K);
    const uint32_t Ku = (uint32_t)K, Nu = (uint32_t)N;
    const int cpl = (int)((8u * nbe + 63u) / 64u);
    for (int t0 = 0; t0 < nt; t0 += MAX_NT_KERNEL) {
        const int n = nt - t0 < MAX_NT_KERNEL ? nt - t0 : MAX_NT_KERNEL;
        const int8_t *qs_t = qs + (size_t)t0 * K;
        const uint16_t *d8_t = d8 + (size_t)t0 * (K / 32);
        float *y_t = y + (size_t)t0 * N;
        hipError_t e;
        if (cpl <= MAX_CPL) {
            const RowsCfg c = rows_cfg(n, cpl);
            const uint32_t grid = grid_for(N, num_cu, c.wg_per_cu);
            const auto seq = std::make_integer_sequence<int, MAX_CPL>{};
            switch (n) {
            case 1: e = dispatch_cpl<1>(cpl, c, seq, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            case 2: e = dispatch_cpl<2>(cpl, c, seq, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            case 3: e = dispatch_cpl<3>(cpl, c, seq, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            default: e = dispatch_cpl<4>(cpl, c, seq, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            }
        } else {
            const uint32_t grid = grid_for(N, num_cu, 2);
            switch (n) {
            case 1: e = launch(mmvq_long<1>, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            case 2: e = launch(mmvq_long<2>, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            case 3: e = launch(mmvq_long<3>, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            default: e = launch(mmvq_long<4>, grid, s, w, qs_t, d8_t, y_t, Nu, nbe, stride, Ku, Nu); break;
            }
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
    uint32_t grid = grid_for(N, num_cu, 4);
    uint32_t Nu = (uint32_t)N, Ku = (uint32_t)K, ntu = (uint32_t)nt;
    void *args[] = {(void *)&w, (void *)&qs, (void *)&dots, (void *)&Nu,
                    (void *)&nbe, (void *)&stride, (void *)&Ku, (void *)&ntu};
    return hipLaunchKernel((const void *)mmvq_subdots_kernel, dim3(grid), dim3(WG), args, 0, s);
}

}  // namespace q6k
