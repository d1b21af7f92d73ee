// mmvq.hip -- k-quant (split-plane rows) x q8 decode GEMV kernels for gfx950, and
// their shape dispatch. One row machine serves q6_K, q4_K and q5_K through a format
// policy F (q6k_unit.h: FmtQ6K; kq_unit.h: FmtQ4K, FmtQ5K) that gives a chunk's byte
// offsets, its loads, its activation operands and its contribution.
//
// What is computed, q6_K (D4-2 §3.2 Excerpt C, the per-unit accumulation; D4-4 §3.2
// Excerpt B, the dpl unit load): y[t][r] = sum over the row's 16-element sub-blocks
// of d * sc * d8 * D, D the exact int32 dot of (q - 32) with the int8 activations.
// q4_K / q5_K: y[t][r] = sum over 32-element sub-blocks of d8 * (d * sc * Dq -
// dmin * m * Sx), Dq the exact code dot and Sx the activation sum.
//
// Geometry (one design for every shape and format):
//  - one wave64 owns one row at a time and walks rows with a stride of the grid's
//    wave count, so the grid streams neighbouring rows together;
//  - lane L takes the row's 16-byte low-bit (code) chunks Q = L, L + 64, ...: each
//    code load instruction is one contiguous 1 KB request; the other planes' loads
//    are smaller contiguous requests;
//  - a lane's byte offsets inside a row are the same for every row, so they are
//    computed once; each row gets a buffer descriptor whose extent is the row's
//    bytes, and loads are buffer loads at those offsets. The code planes are read
//    non-temporal (each weight byte is read once per call); the small scale loads
//    keep the default policy;
//  - lanes past the row's last chunk load a duplicate of the last chunk and
//    contribute exactly 0, and a wave's look-ahead past the last row uses an empty
//    descriptor (its loads return zeros without touching memory), so loads are
//    branch-free and their waits are counted exactly;
//  - DEPTH rows are in flight per wave: the next rows' loads are issued before the
//    current row's arithmetic (scheduling barriers keep the compiler from sinking
//    them), so a wave never idles with nothing requested;
//  - a lane's activation operands are the same for every row; they stay in
//    registers (ACT_REGS) when they fit next to the weight buffers, else the
//    workgroup stages them once in LDS and reads them per row (ACT_LDS; the
//    generic long-row kernel re-reads them from the q8 plane);
//  - a row ends with one reduction for all its token columns (DPP inside each
//    16-lane row, lane swaps across rows); lanes 0..NT-1 write the NT outputs.
// The chunks per lane (CPL = ceil(8*nbe/64)) is a template parameter up to
// MAX_CPL, so a row's loads are issued back to back; longer rows take the generic
// kernel, which walks a row in runtime steps of 4 chunks per lane. Every kernel
// masks every chunk with Q < 8*nbe and loops rows while row < N, so it covers all
// units of all rows of any shape it is launched on (D4-2 §2: a dispatch that routes
// a shape to a kernel covering fewer units silently drops work).

#include <map>
#include <mutex>
#include <tuple>
#include <unordered_map>

#include "kq_unit.h"
#include "q6k_internal.h"
#include "q6k_norm.h"

namespace q6k {

constexpr int WG = 256;             // 4 waves per workgroup
constexpr int WAVES_PER_WG = WG / 64;

// A workgroup's place in the row order. Workgroups are dealt to the eight XCDs in turn
// (workgroup b to XCD b % 8), each with its own L2, and a round of the row walk gives
// place p the rows 4p .. 4p + 3. In each run of 64 workgroups the eight of one XCD take
// eight neighbouring places, so that the 32 outputs of a 128-byte line of y (one token)
// are all written through one L2; in the plain order each line took eight 16-byte pieces
// from eight L2s. At lm_head (152064 x 5120) this measured 1.5-1.9 us faster at one
// token and 0.9 us at two; writing the outputs of the plain row order at the grouped
// places gained nearly as much, so the gain is in the output lines, not the order of the
// weight reads. Grids that are not a multiple of 64 keep the plain order.
__device__ __forceinline__ uint32_t wg_place()
{
    const uint32_t b = blockIdx.x;
    return gridDim.x % 64u == 0 ? (b & ~63u) + 8u * (b & 7u) + ((b >> 3) & 7u) : b;
}

constexpr int MAX_CPL = 12;         // nbe <= 96 take the fixed-length kernels
constexpr int MAX_NT_KERNEL = 4;    // token columns per launch (more -> several launches)

// Descriptor of one row; extent 0 for a look-ahead row past the end, whose loads
// then return zeros without a memory request.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_desc(const uint8_t *w, uint32_t row,
                                                           uint32_t stride, bool real = true)
{
    return buf_desc(w + (size_t)row * stride, real ? stride : 0u);
}

// float4 f of an n-float4 row through its descriptor (zeros past n).
__device__ __forceinline__ float4 load_f4(__amdgpu_buffer_rsrc_t r, uint32_t f)
{
    const uint4 v = load_b128<POLICY_DEFAULT>(r, 16u * f);
    const uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    return make_float4(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b),
                       __builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
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

// Sums over each 16-lane row of NT <= 4 per-lane values (one per token column). The
// first steps transpose while they add: at the pair step a lane keeps the tokens of
// its parity and hands the others to its partner, at the quad step likewise by the
// second lane bit, so afterwards lane l carries only token (l & 3) (for NT = 2:
// l & 1). Rotations by 4 and 8 lanes finish each row: every lane then holds its
// row's total of token (l & 3) (NT = 1: of the only token).
template <int NT>
__device__ __forceinline__ float row_sums(const float (&a)[NT], uint32_t lane)
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
    return dpp_add<0x128>(v);                        // row_ror:8
}

// The sum of v over the two 16-lane rows of each half wave (rows 0 + 1, rows 2 + 3).
// v_permlane16_swap exchanges the odd rows of its first operand with the even rows
// of its second, so with both operands v the two results hold (r0, r0, r2, r2) and
// (r1, r1, r3, r3); their sum does not depend on which is which. (Each swap's two
// results are copied into plain integers before their bit casts: a bit cast applied
// straight to an element of the returned pair reads element 0 for both.)
__device__ __forceinline__ float half_pair_sum(float v)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// Sums over a wave64 of NT <= 4 per-lane values: the row sums, then two lane swaps
// add the four rows. Lane l then holds the total of token (l & 3) (NT = 2: l & 1;
// NT = 1: of the only token). The adds always pair the same lanes in the same order,
// so results are reproducible run to run.
template <int NT>
__device__ __forceinline__ float reduce_tokens(const float (&a)[NT], uint32_t lane)
{
    float v = row_sums<NT>(a, lane);
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned h0 = h[0], h1 = h[1];
    v = __builtin_bit_cast(float, h0) + __builtin_bit_cast(float, h1);
    return half_pair_sum(v);
}

// Stores a row's totals after reduce_tokens: lanes 0 .. NT - 1 hold them (token t in
// lane t). (Every lane holds a total of its token, but not all in the same order of
// additions: the row rotations add a 16-lane row's quads as (q0 + q1) + (q2 + q3) in
// quads 0 and 2 and as (q1 + q2) + (q3 + q0) in quads 1 and 3.)
template <int NT>
__device__ __forceinline__ void store_row(float *y, uint32_t ldy, uint32_t row, float s,
                                          uint32_t lane)
{
    if (lane < (uint32_t)NT)
        y[(size_t)(NT == 1 ? 0u : lane) * ldy + row] = s;
}

// Where a lane's activation operands live across rows: re-read from the q8 plane
// per row (ACT_GLOBAL), held in registers (ACT_REGS), or staged once per workgroup
// in LDS and read per row (ACT_LDS; for rows whose operands do not fit registers).
enum ActMode : int { ACT_GLOBAL = 0, ACT_REGS = 1, ACT_LDS = 2 };

// Per-lane state that is the same for every row a wave visits.
template <class F, int NT, int CPL, int AM>
struct LaneState {
    typename F::Offs off[CPL];
    uint32_t Q[CPL];        // chunk index (clamped to the last chunk past the row end)
    bool live[CPL];         // false: duplicate load, contributes 0
    typename F::Act act[AM == ACT_REGS ? CPL : 1][NT];
    // ACT_LDS: three planes (first halves, second halves, scalars) of `plane` 16-byte
    // entries; token t's entry of chunk slot i at t * tstride + ent[i], where a slot
    // past the row points at the token's all-zero entry
    uint32_t ent[AM == ACT_LDS ? CPL : 1];
    const uint4 *lds;
    uint32_t plane, tstride;
};

// A lane's chunks Q = lane + SPAN * i: SPAN = 64 when one wave owns a row, 256 when
// the four waves of a workgroup share it (lane then counts the workgroup's threads).
template <class F, int NT, int CPL, int AM, uint32_t SPAN = 64u>
__device__ __forceinline__ void lane_chunks(LaneState<F, NT, CPL, AM> &st, uint32_t lane,
                                            uint32_t nbe)
{
    const uint32_t C = 8u * nbe;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const uint32_t Q = lane + SPAN * i;
        st.live[i] = Q < C;
        st.Q[i] = st.live[i] ? Q : C - 1u;
        st.off[i] = F::offsets(st.Q[i], nbe);
    }
}

// qs, d8: the activation rows (global memory or LDS), token t at qs + t * K and
// d8 + t * (K / 32). A chunk past the row gets dropped operands (F::drop), so the
// row loop needs no per-row select for it.
template <class F, int NT, int CPL>
__device__ __forceinline__ void lane_acts(LaneState<F, NT, CPL, ACT_REGS> &st, const int8_t *qs,
                                          const uint16_t *d8, uint32_t K)
{
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            st.act[i][t] = F::act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), st.Q[i]);
            if (!st.live[i])
                F::drop(st.act[i][t]);
        }
    }
}

// lane_acts with a step between the operand loads and their arithmetic: the loads are
// issued, then `between` (which may issue loads of its own), then the arithmetic,
// whose waits cover the operand loads only (nothing later is scheduled before it).
// The same operands as lane_acts.
template <class F, int NT, int CPL, typename Between>
__device__ __forceinline__ void lane_acts_around(LaneState<F, NT, CPL, ACT_REGS> &st,
                                                 const int8_t *qs, const uint16_t *d8,
                                                 uint32_t K, Between &&between)
{
    ActRaw raw[CPL][NT];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            raw[i][t] = F::act_raw(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), st.Q[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            st.act[i][t] = F::act_finish(raw[i][t]);
            if (!st.live[i])
                F::drop(st.act[i][t]);
        }
    }
    // the arithmetic stays here, where it waits for the operands only
    __builtin_amdgcn_sched_barrier(0);
}

template <class F, int NT, int CPL, int AM>
__device__ __forceinline__ void load_row(typename F::W (&dst)[CPL], const uint8_t *w,
                                         uint32_t row, uint32_t N, uint32_t stride,
                                         const LaneState<F, NT, CPL, AM> &st)
{
    const bool real = row < N;
    const __amdgpu_buffer_rsrc_t r = row_desc(w, real ? row : 0u, stride, real);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        dst[i] = F::load(r, st.off[i]);
}

// A zero the compiler cannot see through, different for every row (row & 0 by an
// instruction it does not evaluate): ACT_LDS reads indexed with it stay inside the
// row loop, where they would otherwise be hoisted into registers, which is what that
// mode is there to avoid.
__device__ __forceinline__ uint32_t row_zero(uint32_t row)
{
    uint32_t z;
    asm("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(row));
    return z;
}

// The row's totals for its token columns: lane l holds the total of token
// (l & 3) (NT = 2: l & 1; NT = 1: every lane the only token's).
template <class F, int NT, int CPL, int AM>
__device__ __forceinline__ float row_total(const typename F::W (&src)[CPL],
                                           const LaneState<F, NT, CPL, AM> &st,
                                           const int8_t *qs, const uint16_t *d8, uint32_t K,
                                           uint32_t lane, uint32_t row = 0)
{
    const uint32_t z = AM == ACT_LDS ? row_zero(row) : 0u;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if constexpr (AM == ACT_REGS) {
                // dead chunks' operands were dropped in lane_acts
                acc[t] = F::accumulate(acc[t], src[i], st.act[i][t], st.Q[i], true);
            } else if constexpr (AM == ACT_LDS) {
                // dead chunks read the all-zero entry
                const uint32_t e = t * st.tstride + st.ent[i] + z;
                const typename F::Act a =
                    F::from_words(st.lds[e], st.lds[st.plane + e], st.lds[2u * st.plane + e]);
                acc[t] = F::accumulate(acc[t], src[i], a, st.Q[i], true);
            } else {
                const typename F::Act a =
                    F::act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), st.Q[i]);
                acc[t] = F::accumulate(acc[t], src[i], a, st.Q[i], st.live[i]);
            }
        }
    }
    return reduce_tokens<NT>(acc, lane);
}

template <class F, int NT, int CPL, int AM>
__device__ __forceinline__ void finish_row(const typename F::W (&src)[CPL],
                                           const LaneState<F, NT, CPL, AM> &st,
                                           const int8_t *qs, const uint16_t *d8, uint32_t K,
                                           float *y, uint32_t ldy, uint32_t row, uint32_t lane)
{
    store_row<NT>(y, ldy, row, row_total<F, NT, CPL, AM>(src, st, qs, d8, K, lane, row), lane);
}

// The weight buffers of the rows a wave has in flight (up to three; a kernel's
// unused ones are never touched and cost nothing). A fourth row in flight measured
// slower on lm_head-shaped rows (GEMV 91.2 vs 90.8 us, fused 93.6 vs 93.0 us).
template <class F, int CPL>
struct RowBufs {
    typename F::W A[CPL], B[CPL], C[CPL];
};

// Requests rows FROM .. TO - 1 of a wave's walk (row, row + nw, ...), the first
// DEPTH of which go to A, B and C in that order. Each row's loads are their own
// scheduling region, so they are issued in walk order: the loads in flight when the
// walk's loop is entered are then in the order every later pass of the loop leaves
// them in, and the compiler's wait counts at the loop head stay exact.
template <class F, int NT, int CPL, int FROM, int TO, int AM>
__device__ __forceinline__ void prime_rows(RowBufs<F, CPL> &b, const uint8_t *w, uint32_t row,
                                           uint32_t nw, uint32_t N, uint32_t stride,
                                           const LaneState<F, NT, CPL, AM> &st)
{
    if constexpr (FROM <= 0 && TO > 0) {
        load_row(b.A, w, row, N, stride, st);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FROM <= 1 && TO > 1) {
        load_row(b.B, w, row + nw, N, stride, st);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FROM <= 2 && TO > 2) {
        load_row(b.C, w, row + 2u * nw, N, stride, st);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Rows row, row + nw, ... below N: how many a wave walks.
__device__ __forceinline__ uint32_t walk_rows(uint32_t row, uint32_t nw, uint32_t N)
{
    return row < N ? (N - row + nw - 1u) / nw : 0u;
}

// One step of a walk: request row `next` into buffer NB, then reduce row `row` held
// in buffer CB (the request comes first: with the reduction first, the compiler
// waits for every load at the loop head; the scheduling barrier keeps it from
// sinking the loads below the arithmetic).
#define Q6K_STEP(NB, NEXT, CB, ROW)                                                            \
    do {                                                                                        \
        load_row(b.NB, w, NEXT, N, stride, st);                                                 \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        finish_row<F, NT, CPL, AM>(b.CB, st, qs, d8, K, y, ldy, ROW, lane);                     \
    } while (0)

// A wave's walk over rows row, row + nw, ... < N with DEPTH rows in flight, the
// first DEPTH - 1 of them already requested by prime_rows. The walk's length is
// counted first and the loop runs whole rounds of DEPTH steps with no exit inside
// them; the last n % DEPTH rows follow the loop. A loop left from the middle of a
// round (one exit test per step) is restructured by the compiler into merged exit
// blocks that also lead back to the loop head, and its wait counts at the head then
// assume the look-ahead rows were issued before the row being reduced: the head step
// waited for every row in flight (measured: the lm_head GEMV at 1 token 91.4 -> 90.5
// us, the fused kernel 93.6 -> 92.4, tall-K 11.1 -> 10.7, attn_v 3.36 -> 3.20 with
// the counted rounds; the results are the same bit for bit). Look-ahead rows past the
// end get an empty descriptor (load_row), so every load stays unconditional and their
// results are never reduced.
template <class F, int NT, int CPL, int DEPTH, int AM>
__device__ __forceinline__ void stream_rows(RowBufs<F, CPL> &b, const uint8_t *w, uint32_t row,
                                            uint32_t nw, uint32_t N, uint32_t stride,
                                            const LaneState<F, NT, CPL, AM> &st,
                                            const int8_t *qs, const uint16_t *d8, uint32_t K,
                                            float *y, uint32_t ldy, uint32_t lane)
{
    static_assert(DEPTH >= 1 && DEPTH <= 3, "one to three rows in flight");
    const uint32_t n = walk_rows(row, nw, N);
    if constexpr (DEPTH == 1) {
        // all of the row's loads before any of its arithmetic (without the barrier
        // the compiler interleaves them, waiting for one group of loads before it
        // issues the next)
        for (uint32_t k = 0; k < n; ++k, row += nw) {
            load_row(b.A, w, row, N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
            finish_row<F, NT, CPL, AM>(b.A, st, qs, d8, K, y, ldy, row, lane);
        }
    } else if constexpr (DEPTH == 2) {
        for (uint32_t g = n / 2u; g; --g) {
            const uint32_t r1 = row + nw, r2 = r1 + nw;
            Q6K_STEP(B, r1, A, row);
            Q6K_STEP(A, r2, B, r1);
            row = r2;
        }
        if (n & 1u)
            finish_row<F, NT, CPL, AM>(b.A, st, qs, d8, K, y, ldy, row, lane);
    } else {
        for (uint32_t g = n / 3u; g; --g) {
            const uint32_t r1 = row + nw, r2 = r1 + nw, r3 = r2 + nw;
            Q6K_STEP(C, r2, A, row);
            Q6K_STEP(A, r3, B, r1);
            Q6K_STEP(B, r3 + nw, C, r2);
            row = r3;
        }
        const uint32_t rem = n % 3u;
        if (rem >= 1u)
            finish_row<F, NT, CPL, AM>(b.A, st, qs, d8, K, y, ldy, row, lane);
        if (rem == 2u)
            finish_row<F, NT, CPL, AM>(b.B, st, qs, d8, K, y, ldy, row + nw, lane);
    }
}

// The same walk with all DEPTH first rows already requested: the first row reduced,
// then DEPTH - 2 steps that refill as they go, which leaves the buffers as
// stream_rows expects them, DEPTH - 1 rows on.
template <class F, int NT, int CPL, int DEPTH, int AM>
__device__ __forceinline__ void stream_rows_primed(RowBufs<F, CPL> &b, const uint8_t *w,
                                                   uint32_t row, uint32_t nw, uint32_t N,
                                                   uint32_t stride,
                                                   const LaneState<F, NT, CPL, AM> &st,
                                                   const int8_t *qs, const uint16_t *d8,
                                                   uint32_t K, float *y, uint32_t ldy,
                                                   uint32_t lane)
{
    const uint32_t r1 = row + nw, r2 = r1 + nw, r3 = r2 + nw;
    finish_row<F, NT, CPL, AM>(b.A, st, qs, d8, K, y, ldy, row, lane);
    if (r1 >= N)
        return;
    if constexpr (DEPTH == 1) {
        stream_rows<F, NT, CPL, DEPTH, AM>(b, w, r1, nw, N, stride, st, qs, d8, K, y, ldy, lane);
    } else if constexpr (DEPTH == 2) {
        Q6K_STEP(A, r2, B, r1);
        if (r2 >= N)
            return;
        stream_rows<F, NT, CPL, DEPTH, AM>(b, w, r2, nw, N, stride, st, qs, d8, K, y, ldy, lane);
    } else {
        Q6K_STEP(A, r3, B, r1);
        if (r2 >= N)
            return;
        Q6K_STEP(B, r3 + nw, C, r2);
        if (r3 >= N)
            return;
        stream_rows<F, NT, CPL, DEPTH, AM>(b, w, r3, nw, N, stride, st, qs, d8, K, y, ldy, lane);
    }
}
#undef Q6K_STEP

// Bytes of LDS the ACT_LDS kernels stage for NT tokens of C chunks: three planes of
// NT * (C + 1) 16-byte entries (each token's chunks, then its all-zero entry).
constexpr uint32_t act_lds_bytes(int nt, uint32_t C)
{
    return 3u * 16u * (uint32_t)nt * (C + 1u);
}

// ACT_LDS staging, by every thread of the workgroup: the operands of token t, chunk Q
// (first halves, second halves, scalars) at entry t * (C + 1) + Q of each plane, and
// zeros at entry t * (C + 1) + C. Ends with a barrier.
template <class F, int NT>
__device__ __forceinline__ void stage_acts(uint4 *lds, const int8_t *qs, const uint16_t *d8,
                                           uint32_t K, uint32_t C)
{
    const uint32_t per = C + 1u, plane = (uint32_t)NT * per;
    for (uint32_t e = threadIdx.x; e < plane; e += WG) {
        const uint32_t t = e / per, Q = e - t * per;
        uint4 xa = make_uint4(0u, 0u, 0u, 0u), xb = xa, sc = xa;
        if (Q < C)
            F::to_words(F::act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), Q), xa, xb, sc);
        lds[e] = xa;
        lds[plane + e] = xb;
        lds[2u * plane + e] = sc;
    }
    __syncthreads();
}

// Rows with at most MAX_CPL chunks per lane; DEPTH rows in flight per wave.
template <class F, int NT, int CPL, int DEPTH, int AM>
__global__ __launch_bounds__(WG) void mmvq_rows(const uint8_t *__restrict__ w,
                                                const int8_t *__restrict__ qs,
                                                const uint16_t *__restrict__ d8,
                                                float *__restrict__ y, uint32_t N, uint32_t nbe,
                                                uint32_t stride, uint32_t K, uint32_t ldy)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = wg_place() * WAVES_PER_WG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * WAVES_PER_WG;
    LaneState<F, NT, CPL, AM> st;
    RowBufs<F, CPL> bufs;
    if constexpr (AM == ACT_LDS) {
        extern __shared__ uint4 s_act[];
        const uint32_t C = 8u * nbe;
        lane_chunks(st, lane, nbe);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            st.ent[i] = st.live[i] ? st.Q[i] : C;
        st.lds = s_act;
        st.tstride = C + 1u;
        st.plane = (uint32_t)NT * (C + 1u);
        // the first rows' weights are requested before the staging (a wave with no row
        // primes empty descriptors), so the weight stream is under way meanwhile
        prime_rows<F, NT, CPL, 0, DEPTH - 1, AM>(bufs, w, wave, nw, N, stride, st);
        __builtin_amdgcn_sched_barrier(0);
        stage_acts<F, NT>(s_act, qs, d8, K, C);
        if (wave >= N)
            return;
    } else {
        // Order of the start: the activation operands' loads, then the first rows'
        // requests (one row with DEPTH 1, which then walks primed; DEPTH - 1
        // otherwise), then the operand arithmetic, which waits for the operand loads
        // only. Rows requested before the operand loads made that wait cover the rows
        // too, and the compiler's wait counts at the row loop's head then covered the
        // look-ahead rows as well (measured slower on every shape it changed); rows
        // requested after the operand arithmetic started a wave's weight stream up to
        // about 1 us late (per-wave clock stamps, 5120 x 13824 at one token).
        lane_chunks(st, lane, nbe);
        if (wave >= N)
            return;
        auto first_rows = [&] {
            prime_rows<F, NT, CPL, 0, DEPTH == 1 ? 1 : DEPTH - 1, AM>(bufs, w, wave, nw, N,
                                                                     stride, st);
        };
        if constexpr (AM == ACT_REGS)
            lane_acts_around(st, qs, d8, K, first_rows);
        else
            first_rows();
        if constexpr (DEPTH == 1) {
            stream_rows_primed<F, NT, CPL, 1, AM>(bufs, w, wave, nw, N, stride, st, qs, d8, K,
                                                  y, ldy, lane);
            return;
        }
    }
    stream_rows<F, NT, CPL, DEPTH, AM>(bufs, w, wave, nw, N, stride, st, qs, d8, K, y, ldy,
                                       lane);
}

// Long rows that are few for the grid: the four waves of a workgroup share each row.
// Workgroup b owns the R consecutive rows from b * R; every wave walks all of them
// (DEPTH in flight, the row machine above, one row apart) over its quarter of the
// chunks (Q = thread + 256 i), reduces its share of a row over its 64 lanes and
// leaves it in LDS. After the walk one barrier, then each output is the four shares
// added in a fixed order, (w0 + w1) + (w2 + w3). With one wave per row, a grid of
// 2048 waves gives such shapes 1.75-2.5 rows per wave: the waves with one row more
// set the time, and each row's loads wait a whole memory latency. Here every wave has
// R rows of a quarter the bytes, R is the same for every workgroup but the last, and
// the chunks per lane fall to what the one-wave rows of lm_head have.
// LDS: the shares, 4 * NT * R floats.
template <class F, int NT, int CPL, int DEPTH, int AM>
__global__ __launch_bounds__(WG) void mmvq_split(const uint8_t *__restrict__ w,
                                                 const int8_t *__restrict__ qs,
                                                 const uint16_t *__restrict__ d8,
                                                 float *__restrict__ y, uint32_t N, uint32_t nbe,
                                                 uint32_t stride, uint32_t K, uint32_t ldy,
                                                 uint32_t R)
{
    static_assert(AM == ACT_REGS, "a thread's 2-3 chunks keep their operands in registers");
    extern __shared__ uint4 s_split[];
    const uint32_t row0 = blockIdx.x * R;
    if (row0 >= N)
        return;   // the whole workgroup: no barrier is reached
    const uint32_t nr = N - row0 < R ? N - row0 : R;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t *wb = w + (size_t)row0 * stride;
    float *part = reinterpret_cast<float *>(s_split);
    float *share = part + wv * (uint32_t)NT * R;
    LaneState<F, NT, CPL, AM> st;
    RowBufs<F, CPL> bufs;
    lane_chunks<F, NT, CPL, AM, 256u>(st, threadIdx.x, nbe);
    // the first rows right behind the operand loads, before the operand arithmetic
    lane_acts_around(st, qs, d8, K, [&] {
        prime_rows<F, NT, CPL, 0, DEPTH - 1, AM>(bufs, wb, 0u, 1u, nr, stride, st);
    });
    // the shares go where the one-wave kernel stores its outputs: token t of local
    // row j at share[t * R + j]
    stream_rows<F, NT, CPL, DEPTH, AM>(bufs, wb, 0u, 1u, nr, stride, st, qs, d8, K, share, R,
                                       lane);
    __syncthreads();
    for (uint32_t e = threadIdx.x; e < (uint32_t)NT * nr; e += WG) {
        const uint32_t t = e / nr, j = e - t * nr;
        const float *p = part + t * R + j;
        const uint32_t ws = (uint32_t)NT * R;
        y[(size_t)t * ldy + row0 + j] = (p[0] + p[ws]) + (p[2u * ws] + p[3u * ws]);
    }
}

// Rows whose chunk count is an odd multiple of 32 (8 * nbe = 64 * (CPL - 1) + 32; K =
// 5120: 160 chunks, 2.5 per lane) at several tokens. With one wave per row the upper
// half of the wave idles in the last chunk slot: at three slots a sixth of the ALU
// work, which at several tokens is what bounds the kernel. Here a wave takes the
// rows A = 2p and B = 2p + 1 together and every lane does useful work in every slot:
//  - buffer X, CPL slots: the full slots of row A in lanes 0-31 and of row B in lanes
//    32-63, and the last, half slot (chunk 64 * (CPL - 1) + lane % 32) of that row;
//  - buffer Y, CPL - 1 slots: the full slots of the other row.
// One descriptor covers both rows; a lane's byte offsets pick its row (+stride for
// B), so no per-lane selects. The activation operands are those of the one-row
// kernel (the last slot's chunk is lane % 32 past 64 * (CPL - 1) in either half).
// A = X over lanes 0-31 + Y over lanes 32-63 and B the other way round: each half
// sums X and Y on its own (row sums, then rows 0 + 1, 2 + 3), then one lane swap
// brings each half the other half's Y.
template <int NT>
__device__ __forceinline__ float reduce_pair(const float (&x)[NT], const float (&yv)[NT],
                                             uint32_t lane)
{
    const float sx = half_pair_sum(row_sums<NT>(x, lane));
    const float sy = half_pair_sum(row_sums<NT>(yv, lane));
    // v_permlane32_swap exchanges the upper half of its first operand with the lower
    // half of its second: with both sy, the first result holds the lower half's sum
    // in both halves and the second the upper half's
    const unsigned u = __builtin_bit_cast(unsigned, sy);
    const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned lo = h[0], hi = h[1];
    return sx + __builtin_bit_cast(float, lane < 32u ? hi : lo);
}

template <class F, int NT, int CPL>
struct PairState {
    typename F::Offs ox[CPL], oy[CPL > 1 ? CPL - 1 : 1];
    uint32_t Q[CPL];
    typename F::Act act[CPL][NT];
};

template <class F, int CPL>
struct PairBufs {
    typename F::W X[CPL], Y[CPL > 1 ? CPL - 1 : 1];
};

template <class F, int CPL>
struct PairRing {
    PairBufs<F, CPL> A, B, C;
};

template <class F, int NT, int CPL>
__device__ __forceinline__ void pair_init(PairState<F, NT, CPL> &st, uint32_t lane,
                                          uint32_t nbe, uint32_t stride)
{
    const uint32_t bx = lane < 32u ? 0u : stride, by = lane < 32u ? stride : 0u;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const uint32_t Q = i < CPL - 1 ? lane + 64u * i : 64u * (CPL - 1) + (lane & 31u);
        const typename F::Offs o = F::offsets(Q, nbe);
        st.Q[i] = Q;
        st.ox[i] = F::shifted(o, bx);
        if (i < CPL - 1)
            st.oy[i] = F::shifted(o, by);
    }
}

// The lane's activation operands, with `between` (the first pairs' requests) issued
// after their loads and before their arithmetic, as lane_acts_around.
template <class F, int NT, int CPL, typename Between>
__device__ __forceinline__ void pair_acts_around(PairState<F, NT, CPL> &st, const int8_t *qs,
                                                 const uint16_t *d8, uint32_t K,
                                                 Between &&between)
{
    ActRaw raw[CPL][NT];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            raw[i][t] = F::act_raw(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), st.Q[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            st.act[i][t] = F::act_finish(raw[i][t]);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Pair p's loads: rows 2p and 2p + 1 below N under one descriptor (pairs past the
// end: an empty one, whose loads return zeros without a memory request).
template <class F, int NT, int CPL>
__device__ __forceinline__ void load_pair(PairBufs<F, CPL> &b, const uint8_t *w, uint32_t p,
                                          uint32_t N, uint32_t stride,
                                          const PairState<F, NT, CPL> &st)
{
    const uint32_t r0 = 2u * p;
    const uint32_t rows = r0 < N ? (N - r0 < 2u ? N - r0 : 2u) : 0u;
    const __amdgpu_buffer_rsrc_t r = buf_desc(w + (size_t)(rows ? r0 : 0u) * stride, rows * stride);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        b.X[i] = F::load(r, st.ox[i]);
#pragma unroll
    for (int i = 0; i < CPL - 1; ++i)
        b.Y[i] = F::load(r, st.oy[i]);
}

template <class F, int NT, int CPL>
__device__ __forceinline__ void finish_pair(const PairBufs<F, CPL> &b,
                                            const PairState<F, NT, CPL> &st, float *y,
                                            uint32_t ldy, uint32_t p, uint32_t N, uint32_t lane)
{
    float ax[NT], ay[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        ax[t] = 0.0f;
        ay[t] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            ax[t] = F::accumulate(ax[t], b.X[i], st.act[i][t], st.Q[i], true);
            if (i < CPL - 1)
                ay[t] = F::accumulate(ay[t], b.Y[i], st.act[i][t], st.Q[i], true);
        }
    }
    const float s = reduce_pair<NT>(ax, ay, lane);
    // lanes 0-31 hold row 2p, lanes 32-63 row 2p + 1 (token lane % 32 in each half)
    const uint32_t row = 2u * p + (lane >> 5);
    uint32_t t = lane & 31u;
    if (t < (uint32_t)NT && row < N)
        y[(size_t)t * ldy + row] = s;
}

#define PAIR_STEP(NB, NEXT, CB, P)                                                              \
    do {                                                                                        \
        load_pair(b.NB, w, NEXT, N, stride, st);                                                \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        finish_pair<F, NT, CPL>(b.CB, st, y, ldy, P, N, lane);                                  \
    } while (0)

template <class F, int NT, int CPL, int DEPTH>
__global__ __launch_bounds__(WG) void mmvq_pairs(const uint8_t *__restrict__ w,
                                                 const int8_t *__restrict__ qs,
                                                 const uint16_t *__restrict__ d8,
                                                 float *__restrict__ y, uint32_t N, uint32_t nbe,
                                                 uint32_t stride, uint32_t K, uint32_t ldy)
{
    static_assert(DEPTH >= 1 && DEPTH <= 3, "one to three pairs in flight");
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = wg_place() * WAVES_PER_WG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * WAVES_PER_WG;
    const uint32_t P = (N + 1u) / 2u;
    if (wave >= P)
        return;
    PairState<F, NT, CPL> st;
    pair_init(st, lane, nbe, stride);
    PairRing<F, CPL> b;
    uint32_t p = wave;
    // the first pairs (DEPTH - 1, one at DEPTH 1) are requested right behind the
    // operand loads and before the operand arithmetic, so the weight stream starts at
    // once
    pair_acts_around(st, qs, d8, K, [&] {
        load_pair(b.A, w, p, N, stride, st);
        if constexpr (DEPTH == 3) {
            __builtin_amdgcn_sched_barrier(0);
            load_pair(b.B, w, p + nw, N, stride, st);
        }
    });
    if constexpr (DEPTH == 1) {
        for (;;) {
            finish_pair<F, NT, CPL>(b.A, st, y, ldy, p, N, lane);
            p += nw;
            if (p >= P)
                break;
            load_pair(b.A, w, p, N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (DEPTH == 2) {
        for (;;) {
            const uint32_t p1 = p + nw, p2 = p1 + nw;
            PAIR_STEP(B, p1, A, p);
            if (p1 >= P)
                break;
            PAIR_STEP(A, p2, B, p1);
            if (p2 >= P)
                break;
            p = p2;
        }
    } else {
        for (;;) {
            const uint32_t p1 = p + nw, p2 = p1 + nw, p3 = p2 + nw;
            PAIR_STEP(C, p2, A, p);
            if (p1 >= P)
                break;
            PAIR_STEP(A, p3, B, p1);
            if (p2 >= P)
                break;
            PAIR_STEP(B, p3 + nw, C, p2);
            if (p3 >= P)
                break;
            p = p3;
        }
    }
}
#undef PAIR_STEP

// RMSNorm -> q8 -> GEMV in one kernel, for the shapes whose activation operands
// stay in registers. Every workgroup normalizes and quantizes the NT activation
// rows itself, into LDS, with the RMSNorm -> q8 producer's own body and order
// (q6k_norm.h), so its operands equal that producer's q8 plane bit for bit and the
// outputs equal those of the producer followed by the GEMV. Workgroup 0 also
// stores the q8 plane and, when xn is not null, the normalized rows. The weight
// rows do not depend on the activations: a wave requests its first rows right
// after its activation loads, so the weight stream is under way while the norm
// runs (the activation loads are issued first, so waiting for them does not wait
// for the weights). The re-reads of x (K * 4 B per token and workgroup) hit L2
// after the first workgroup of each die.
template <class F, int NT, int CPL, int DEPTH>
__global__ __launch_bounds__(WG) void mmvq_rmsnorm_rows(
    const uint8_t *__restrict__ w, const float4 *__restrict__ x, const float4 *__restrict__ gamma,
    float eps, float4 *__restrict__ xn, uint32_t *__restrict__ qs_out,
    uint16_t *__restrict__ d8_out, float *__restrict__ y, uint32_t N, uint32_t nbe,
    uint32_t stride, uint32_t K, uint32_t ldy)
{
    static_assert(WG == NORM_WG, "the norm body assumes one 256-thread workgroup");
    constexpr int VPT = 2 * CPL;               // NORM_WG * VPT float4s >= K / 4 = 64 * nbe
    constexpr int K4_MAX = NORM_WG * VPT;
    // rows requested before the norm: all DEPTH, unless x, gamma and the weight
    // buffers would pass about 200 registers while the norm runs (two workgroups per
    // CU, DEPTH 2, leave 256 per lane); then the last one after it
    constexpr int PRE = (DEPTH == 2 && CPL * (8 * NT + 8 + 22) > 200) ? DEPTH - 1 : DEPTH;
    __shared__ __align__(16) uint32_t s_qs[NT][K4_MAX];
    __shared__ __align__(16) uint16_t s_d8[NT][K4_MAX / 8];
    __shared__ double part[NT * (NORM_WG / 64)];

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = wg_place() * WAVES_PER_WG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * WAVES_PER_WG;
    const uint32_t K4 = K / 4u;

    // buffer loads with a per-row extent of K4 float4s: past the end they return
    // zeros, which the norm body expects there
    float4 xv[NT][VPT], gv[VPT];
    {
        const __amdgpu_buffer_rsrc_t rg = buf_desc(gamma, 16u * K4);
        __amdgpu_buffer_rsrc_t rx[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            rx[t] = buf_desc(x + (size_t)t * K4, 16u * K4);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t f = threadIdx.x + v * NORM_WG;
            gv[v] = load_f4(rg, f);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                xv[t][v] = load_f4(rx[t], f);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    LaneState<F, NT, CPL, ACT_REGS> st;
    lane_chunks(st, lane, nbe);
    RowBufs<F, CPL> bufs;
    // a wave with no row primes empty descriptors (no memory traffic); it still
    // takes part in the workgroup's norm below
    prime_rows<F, NT, CPL, 0, PRE, ACT_REGS>(bufs, w, wave, nw, N, stride, st);
    __builtin_amdgcn_sched_barrier(0);

    const bool store = blockIdx.x == 0;
    // the groups past the row are skipped (graph-replayed, same bits out: lm_head
    // 152064 x 5120 92.5 -> 92.1-92.2 us; attn_v 1024 x 5120 5.13 -> 5.2 us; the
    // standalone producer ran 3.2 -> 3.3 us with it, so it keeps every group)
    norm_quant_rows<NT, VPT, true>(xv, gv, K, eps, part,
                                   [&](int t, uint32_t f, float4 yv, const Q8Out &o) {
                                       s_qs[t][f] = o.packed;
                                       if ((f & 7u) == 0)
                                           s_d8[t][f >> 3] = o.d16;
                                       if (store) {
                                           if (xn)
                                               xn[(size_t)t * K4 + f] = yv;
                                           qs_out[(size_t)t * K4 + f] = o.packed;
                                           if ((f & 7u) == 0)
                                               d8_out[(size_t)t * (K / 32u) + (f >> 3)] = o.d16;
                                       }
                                   });
    __syncthreads();
    // the activation rows in LDS have the layout of the q8 plane: token t at
    // s_qs[t] (K bytes) and s_d8[t]
    lane_acts(st, reinterpret_cast<const int8_t *>(&s_qs[0][0]), &s_d8[0][0], 4u * K4_MAX);
    if (wave >= N)
        return;
    prime_rows<F, NT, CPL, PRE, DEPTH, ACT_REGS>(bufs, w, wave, nw, N, stride, st);
    __builtin_amdgcn_sched_barrier(0);
    stream_rows_primed<F, NT, CPL, DEPTH, ACT_REGS>(bufs, w, wave, nw, N, stride, st, nullptr,
                                                    nullptr, K, y, ldy, lane);
}

// Form B (D4-4 §3.5, the archived fused gate+up+SwiGLU+q8 shape; §5 its closing
// numbers): the gate+up GEMV of one token, then y = silu(gate) * up and its q8 plane,
// in one kernel. The matrix holds the Nh gate rows, then the Nh up rows. Output block
// b (32 activations, one q8 block) needs gate rows 32b .. 32b+31 and up rows Nh + 32b
// .. Nh + 32b + 31: a workgroup takes whole blocks (wave v: gate and up rows 32b + 8v
// .. +7, 16 rows, DEPTH 2 in flight), stores the 64 row totals to gu and LDS, and wave
// 0 then forms the block's 32 outputs and quantizes them. Row totals, SwiGLU and the
// q8 body are the GEMV's and the SwiGLU producer's own code (row_total; the
// producer's expression; q6k_norm.h), so gu, y and the q8 plane equal mmvq_kq_q8
// followed by swiglu_quant_q8 bit for bit. The cost against those two kernels is
// granularity: a q8 block's 64 rows must sit in one workgroup, so Nh / 32 blocks
// spread over the CUs unevenly (13824 / 32 = 432 blocks on 256 CUs).
template <class F, int CPL>
__global__ __launch_bounds__(WG) void gate_up_swiglu_rows(
    const uint8_t *__restrict__ w, const int8_t *__restrict__ qs, const uint16_t *__restrict__ d8,
    float *__restrict__ gu, float *__restrict__ y, uint8_t *__restrict__ qs_out,
    uint16_t *__restrict__ d8_out, uint32_t Nh, uint32_t nbe, uint32_t stride, uint32_t K)
{
    constexpr uint32_t ROWS = 16;   // per wave and block: 8 gate rows, then 8 up rows
    __shared__ float s_g[32], s_u[32];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    LaneState<F, 1, CPL, ACT_REGS> st;
    lane_chunks(st, lane, nbe);
    const uint32_t N = 2u * Nh, nblk = Nh / 32u;
    // row i of this wave's 16 in block b (past the last block: N, an empty request)
    auto block_row = [&](uint32_t b, uint32_t i) {
        return b < nblk ? (i < 8u ? 0u : Nh) + 32u * b + 8u * wv + (i & 7u) : N;
    };
    typename F::W A[CPL], B[CPL];
    // the first row is requested right behind the operand loads and before their
    // arithmetic; each block's last step requests the next block's first row
    lane_acts_around(st, qs, d8, K,
                     [&] { load_row(A, w, block_row(blockIdx.x, 0u), N, stride, st); });
    for (uint32_t b = blockIdx.x; b < nblk; b += gridDim.x) {
        auto row_of = [&](uint32_t i) { return block_row(b, i); };
        auto take = [&](uint32_t i, float v) {
            if (lane == 0) {
                gu[row_of(i)] = v;
                (i < 8u ? s_g : s_u)[8u * wv + (i & 7u)] = v;
            }
        };
#pragma unroll
        for (uint32_t i = 0; i < ROWS; i += 2) {
            load_row(B, w, row_of(i + 1), N, stride, st);
            __builtin_amdgcn_sched_barrier(0);
            take(i, row_total<F, 1, CPL, ACT_REGS>(A, st, nullptr, nullptr, K, lane));
            load_row(A, w, i + 2 < ROWS ? row_of(i + 2) : block_row(b + gridDim.x, 0u), N,
                     stride, st);
            __builtin_amdgcn_sched_barrier(0);
            take(i + 1, row_total<F, 1, CPL, ACT_REGS>(B, st, nullptr, nullptr, K, lane));
        }
        __syncthreads();
        if (wv == 0) {
            // lanes 0..31: the block's outputs; lanes 32..63 carry 0 through the max
            float v = 0.0f;
            if (lane < 32u) {
                const float g = s_g[lane], u = s_u[lane];
                v = (g / (1.0f + expf(-g))) * u;
            }
            float m = fabsf(v);
            m = fmaxf(m, __shfl_xor(m, 32));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 8));
            m = fmaxf(m, __shfl_xor(m, 4));
            m = fmaxf(m, __shfl_xor(m, 2));
            m = fmaxf(m, __shfl_xor(m, 1));
            const float d = m / 127.0f;
            const float di = (d != 0.0f) ? 1.0f / d : 0.0f;
            if (lane < 32u) {
                qs_out[32u * b + lane] = (uint8_t)q8_code(v, di);
                if (y)
                    y[32u * b + lane] = v;
            }
            if (lane == 0)
                d8_out[b] = __builtin_bit_cast(uint16_t, (_Float16)d);
        }
        __syncthreads();   // s_g, s_u are rewritten by the next block
    }
}

// Any row length: a row is walked in steps of STEP chunks per lane. Each step's
// chunks are summed in f32 (at most STEP roundings) and the step sums are added in
// f64, so a lane's rounding error does not grow with the row length (a row of 2^20
// weights is 512 steps per lane); the lane total is rounded once to f32 before the
// wave reduction.
template <class F, int NT>
__global__ __launch_bounds__(WG) void mmvq_long(const uint8_t *__restrict__ w,
                                                const int8_t *__restrict__ qs,
                                                const uint16_t *__restrict__ d8,
                                                float *__restrict__ y, uint32_t N, uint32_t nbe,
                                                uint32_t stride, uint32_t K, uint32_t ldy)
{
    constexpr int STEP = 4;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = wg_place() * WAVES_PER_WG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * WAVES_PER_WG;
    const uint32_t C = 8u * nbe;
    for (uint32_t row = wave; row < N; row += nw) {
        const __amdgpu_buffer_rsrc_t r = row_desc(w, row, stride);
        double lane_sum[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            lane_sum[t] = 0.0;
        for (uint32_t base = 0; base < C; base += 64u * STEP) {
            typename F::W wt[STEP];
            uint32_t Qs[STEP];
            bool live[STEP];
#pragma unroll
            for (int i = 0; i < STEP; ++i) {
                const uint32_t Q = base + lane + 64u * i;
                live[i] = Q < C;
                Qs[i] = live[i] ? Q : C - 1u;
                wt[i] = F::load(r, F::offsets(Qs[i], nbe));
            }
            __builtin_amdgcn_sched_barrier(0);
            float acc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = 0.0f;
#pragma unroll
            for (int i = 0; i < STEP; ++i) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const typename F::Act a =
                        F::act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), Qs[i]);
                    acc[t] = F::accumulate(acc[t], wt[i], a, Qs[i], live[i]);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
                lane_sum[t] += (double)acc[t];
        }
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = (float)lane_sum[t];
        store_row<NT>(y, ldy, row, reduce_tokens<NT>(acc, lane), lane);
    }
}

// Test kernel (q4_K / q5_K): the exact code dots Dq of every 32-element sub-block,
// one wave per row, any row length. Chunks Q and Q ^ 1 (lanes L and L ^ 1) hold the
// two 16-element halves of the same two sub-blocks; C is a multiple of 8, so both
// lanes of a pair run the loop together.
template <bool Q5>
__global__ __launch_bounds__(WG) void kq_subdots_kernel(const uint8_t *__restrict__ w,
                                                        const int8_t *__restrict__ qs,
                                                        const uint16_t *__restrict__ d8,
                                                        int32_t *__restrict__ dots, uint32_t N,
                                                        uint32_t nbe, uint32_t stride,
                                                        uint32_t K, uint32_t nt)
{
    using F = FmtKq<Q5>;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * WAVES_PER_WG + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * WAVES_PER_WG;
    const uint32_t C = 8u * nbe;
    const uint32_t nsub = K / 32u;
    for (uint32_t row = wave; row < N; row += nwaves) {
        const __amdgpu_buffer_rsrc_t r = row_desc(w, row, stride);
        for (uint32_t Q = lane; Q < C; Q += 64u) {
            const KqW wt = F::load(r, F::offsets(Q, nbe));
            const uint32_t s = 2u * (Q >> 1);   // sub-block of the low-nibble half
            for (uint32_t t = 0; t < nt; ++t) {
                const KqAct a = kq_load_act(qs + (size_t)t * K, d8 + (size_t)t * (K / 32), Q);
                int Da, Db;
                kq_chunk_dots<Q5>(wt, a, Q, Da, Db);
                Da += __shfl_xor(Da, 1);
                Db += __shfl_xor(Db, 1);
                if ((Q & 1u) == 0) {
                    int32_t *o = dots + ((size_t)t * N + row) * nsub;
                    o[s] = Da;
                    o[s + 1u] = Db;
                }
            }
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

// Workgroups of `kern` that fit on one CU at once (its registers and LDS), from the
// runtime's occupancy calculator. Some long-row kernels need more than the 256
// registers per lane that two workgroups per CU leave; a grid sized for two would
// then run in two rounds.
// lds: the launch's dynamic LDS bytes (the kernel's own static LDS is known to the
// runtime); past 64 KB the kernel is first allowed that much.
// Process-wide state: the answer is kept per (current device, kernel, lds) for the
// life of the process, behind a mutex, so the query runs once per kernel and size.
int wg_fit(const void *kern, uint32_t lds)
{
    static std::mutex mu;
    static std::map<std::tuple<int, const void *, uint32_t>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_tuple(dev, kern, lds);
    auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    if (lds > 65536u &&
        hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
            hipSuccess)
        return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, WG, lds) != hipSuccess || n < 1)
        return 0;
    cache.emplace(key, n);
    return n;
}

namespace {

// The fixed-length kernel's shape: rows in flight per wave, whether the activation
// operands stay in registers, and workgroups per CU (a launch takes fewer if the
// kernel's registers fit fewer). Chosen per weight type, tokens per launch and chunks
// per lane from measurements on MI355X (sweeps at about 100 MB per matrix and on
// the workload shapes; choices within about 2 % of each other are merged):
//  - short rows (1-2 chunks per lane) need many rows in flight per CU: more
//    workgroups and depth 2-3;
//  - q4_K / q5_K rows carry more ALU work per byte than q6_K rows and gain from two
//    waves per SIMD where q6_K keeps one wave at depth 3 (1-3 chunks);
//  - middle rows (4-7 chunks) take depth 2 with the activation in registers;
//  - long rows (8-12 chunks, and 7 for q5_K) take depth 1, activations re-read.
// Several tokens multiply the activation registers; past 4 chunks they take the
// register-budget rule: depth 2 in registers while nt * chunks <= 6, else depth 1.
struct RowsCfg {
    int depth;
    int mode;       // ActMode
    int wg_per_cu;
};

constexpr RowsCfg rows_cfg(int type, int nt, int cpl)
{
    const bool q6 = type == KQT_Q6_K, q4 = type == KQT_Q4_K;
    if (nt == 1) {
        if (cpl == 1)
            return {2, ACT_REGS, 4};
        if (cpl == 2)
            return {2, ACT_REGS, 2};
        if (cpl == 3)
            return q6 ? RowsCfg{3, ACT_REGS, 1} : RowsCfg{2, ACT_REGS, 2};
        if (cpl <= 6)
            return {2, ACT_REGS, 1};
        // long rows: q4_K/q5_K operands (and q6_K's from 11 chunks) staged in LDS
        // leave registers for two workgroups per CU
        if (!q6 || cpl >= 11)
            return {1, ACT_LDS, 2};
        return {1, ACT_REGS, cpl <= 8 ? 1 : 2};
    }
    if (cpl == 1)
        return {3, ACT_REGS, 2};
    if (cpl == 2)
        return (nt == 2 && !q6) ? RowsCfg{3, ACT_REGS, 2} : RowsCfg{2, ACT_REGS, 2};
    if (cpl == 4 && nt == 2 && q6)
        return {2, ACT_REGS, 1};
    // long rows at several tokens: the columns' operands no longer fit in registers
    // next to the weight buffers, and staging them in LDS (read per row) measured
    // faster than registers, than re-reading them from the plane, and than one or
    // two columns per launch (q6_K 4096x24576 at 4 columns: 60 us in two launches of
    // two, 34 us with LDS); q4_K and q5_K carry more operand registers per chunk and
    // cross over earlier
    const bool lds = q6 ? (cpl >= 11 || (cpl >= 8 && nt >= 3))
                        : q4 ? (cpl >= 7 || (cpl == 6 && nt >= 3))
                             : (cpl >= 9 || (cpl >= 7 && nt >= 3) || (cpl == 6 && nt == 4));
    if (lds)
        return {2, ACT_LDS, 2};
    if (cpl <= 6)
        return {2, ACT_REGS, 2};
    if (nt == 2)
        return (q6 && cpl >= 8) ? RowsCfg{1, ACT_REGS, 2} : RowsCfg{2, ACT_REGS, 1};
    return {1, ACT_REGS, 2};
}

struct GemvArgs {
    const uint8_t *w;
    const int8_t *qs;
    const uint16_t *d8;
    float *y;
    uint32_t N, nbe, stride, K, ldy;
};

// Workgroups: whole multiples of the CU count (an uneven count leaves some CUs one
// workgroup short), never more waves than rows, at most as many per CU as fit.
uint32_t grid_for(int64_t N, int num_cu, int wg_per_cu)
{
    const int64_t need = (N + WAVES_PER_WG - 1) / WAVES_PER_WG;
    const int64_t full = (int64_t)num_cu * wg_per_cu;
    return (uint32_t)(need < full ? need : full);
}

template <typename Kern>
hipError_t launch(Kern kern, int num_cu, int wg_per_cu, hipStream_t s, GemvArgs a,
                  uint32_t lds = 0)
{
    const int fit = wg_fit((const void *)kern, lds);
    if (fit < 1)
        return hipErrorInvalidValue;
    const uint32_t grid = grid_for(a.N, num_cu, wg_per_cu < fit ? wg_per_cu : fit);
    void *args[] = {(void *)&a.w, (void *)&a.qs, (void *)&a.d8, (void *)&a.y, (void *)&a.N,
                    (void *)&a.nbe, (void *)&a.stride, (void *)&a.K, (void *)&a.ldy};
    return hipLaunchKernel((const void *)kern, dim3(grid), dim3(WG), args, lds, s);
}

template <class F, int NT, int CPL>
hipError_t launch_cpl(const RowsCfg &c, int num_cu, hipStream_t s, const GemvArgs &a)
{
    // the one (depth, operand mode) pair rows_cfg picks for this type, NT and CPL is built,
    // for the token counts a launch of this CPL can have
    constexpr RowsCfg k = rows_cfg(F::TYPE, NT, CPL);
    if (c.depth != k.depth || c.mode != k.mode)
        return hipErrorInvalidValue;
    const uint32_t lds = k.mode == ACT_LDS ? act_lds_bytes(NT, 8u * a.nbe) : 0u;
    return launch(mmvq_rows<F, NT, CPL, k.depth, k.mode>, num_cu, c.wg_per_cu, s, a, lds);
}

template <class F, int NT, int... CPLS>
hipError_t dispatch_cpl(int cpl, const RowsCfg &c, std::integer_sequence<int, CPLS...>,
                        int num_cu, hipStream_t s, const GemvArgs &a)
{
    hipError_t e = hipErrorInvalidValue;
    (void)((cpl == CPLS + 1 ? (e = launch_cpl<F, NT, CPLS + 1>(c, num_cu, s, a), true) : false) ||
           ...);
    return e;
}

// The fused RMSNorm -> q8 -> GEMV kernel is used for one token whose activation
// operands stay in registers (up to FUSED_MAX_CPL chunks per lane, K <= 12288).
// With more tokens the norm work in every workgroup's prologue (one token's worth
// per token) is no longer hidden behind the first weight rows, and the producer
// kernel followed by the GEMV measured faster on lm_head 152064 x 5120 (nt = 2:
// equal; nt = 3, 4: 2 and 4 us faster), so those shapes take the two kernels (with
// the same results bit for bit).
constexpr int FUSED_MAX_CPL = 6;

constexpr bool fused_ok(int nt, int cpl)
{
    return nt == 1 && cpl >= 1 && cpl <= FUSED_MAX_CPL;
}

// Form B keeps one token's activation operands in registers (hoisted), which the
// row table does for up to 6 chunks per lane (K <= 12288).
constexpr int GATE_UP_MAX_CPL = 6;

constexpr bool gate_up_ok(int cpl)
{
    return cpl >= 1 && cpl <= GATE_UP_MAX_CPL;
}

struct FusedArgs {
    const uint8_t *w;
    const float4 *x, *gamma;
    float eps;
    float4 *xn;
    uint32_t *qs;
    uint16_t *d8;
    float *y;
    uint32_t N, nbe, stride, K, ldy;
};

template <class F, int NT, int CPL>
hipError_t launch_fused_cpl(int depth, int num_cu, int wg_per_cu, hipStream_t s, FusedArgs a)
{
    if constexpr (fused_ok(NT, CPL)) {
        void *args[] = {(void *)&a.w, (void *)&a.x, (void *)&a.gamma, (void *)&a.eps,
                        (void *)&a.xn, (void *)&a.qs, (void *)&a.d8, (void *)&a.y,
                        (void *)&a.N, (void *)&a.nbe, (void *)&a.stride, (void *)&a.K,
                        (void *)&a.ldy};
        // the depth rows_cfg picks for this type, NT and CPL (always in registers here)
        constexpr RowsCfg k = rows_cfg(F::TYPE, NT, CPL);
        static_assert(k.mode == ACT_REGS, "the fused kernel keeps the activation in registers");
        const void *kern = depth == k.depth ? (const void *)mmvq_rmsnorm_rows<F, NT, CPL, k.depth>
                                            : nullptr;
        const int fit = kern ? wg_fit(kern) : 0;
        if (fit >= 1) {
            const uint32_t g = grid_for(a.N, num_cu, wg_per_cu < fit ? wg_per_cu : fit);
            return hipLaunchKernel(kern, dim3(g), dim3(WG), args, 0, s);
        }
    }
    return hipErrorInvalidValue;
}

template <class F, int NT, int... CPLS>
hipError_t dispatch_fused(int cpl, int depth, std::integer_sequence<int, CPLS...>, int num_cu,
                          int wg_per_cu, hipStream_t s, const FusedArgs &a)
{
    hipError_t e = hipErrorInvalidValue;
    (void)((cpl == CPLS + 1
                ? (e = launch_fused_cpl<F, NT, CPLS + 1>(depth, num_cu, wg_per_cu, s, a), true)
                : false) ||
           ...);
    return e;
}

// When the shared-row kernel (mmvq_split) runs a launch of nt <= 4 tokens, from its
// rows' chunks per lane under one wave per row (cpl), measured against the one-wave
// kernels (graph-replayed, one MI355X):
//  - several tokens, cpl >= 7, and cpl = 6 from 3 tokens: every shape measured gains,
//    most where the one-wave form stages the operands in LDS or runs at depth 1
//    (q6_K 3584 x 18944 at 4 tokens 28 -> 14 us, 5120 x 13824 19.6 -> 13.4,
//    16384 x 18944 87 -> 45-49; cpl 6 at 4 tokens 36-39 -> 33); at cpl 5 it loses;
//  - one token, q4_K / q5_K, cpl >= 7: their one-wave long rows read the operands
//    from LDS per row; 4-5 % faster (q4_K 5120 x 13824 9.4 -> 9.0 us, 16384 x 24576
//    38.2 -> 36.3);
//  - one token, q6_K, cpl >= 7: only when the one-wave grid has fewer than 4 rows per
//    wave (3584 x 18944 12.5 -> 11.1-11.5 us); with 5 or more it loses 2-4 %
//    (5120 x 13824, 8192 x 13824, 16384 x 18944).
// Its chunks per lane are then ceil(cpl / 4) = 2 or 3, its rows per workgroup at most
// SPLIT_MAX_R (N <= 131072 at two workgroups per CU, 65536 at one); longer rows
// (cpl > MAX_CPL) take the generic stepping kernel.
constexpr int64_t SPLIT_ROWS_PER_WAVE = 4;
constexpr uint32_t SPLIT_MAX_R = 256;   // rows per workgroup (LDS: 16 * nt * R bytes)

// Depth, operand mode and workgroups per CU of the shared-row kernel (fitted to the
// same sweeps: 2 chunks per lane at depth 2 and 2/CU, 3 at depth 3 and 1/CU).
constexpr RowsCfg split_cfg(int type, int nt, int cpl4)
{
    (void)type;
    (void)nt;
    return cpl4 <= 2 ? RowsCfg{2, ACT_REGS, 2} : RowsCfg{3, ACT_REGS, 1};
}

// Rows per workgroup for N rows over num_cu * wg_per_cu workgroups.
constexpr uint32_t split_rows(int64_t N, int num_cu, int wg_per_cu)
{
    const int64_t slots = (int64_t)num_cu * wg_per_cu;
    return (uint32_t)((N + slots - 1) / slots);
}

bool split_ok(int type, int nt, int cpl, int64_t N, int num_cu)
{
    const int n = nt < MAX_NT_KERNEL ? nt : MAX_NT_KERNEL;
    if (n < 1 || cpl > MAX_CPL || cpl < 6 || (cpl == 6 && n < 3))
        return false;
    if (split_rows(N, num_cu, split_cfg(type, n, (cpl + 3) / 4).wg_per_cu) > SPLIT_MAX_R)
        return false;
    if (n > 1 || type != KQT_Q6_K)
        return true;
    const int64_t waves = (int64_t)num_cu * rows_cfg(type, n, cpl).wg_per_cu * WAVES_PER_WG;
    return N < SPLIT_ROWS_PER_WAVE * waves;
}

template <class F, int NT, int CPL4>
hipError_t launch_split(int num_cu, hipStream_t s, GemvArgs a)
{
    constexpr RowsCfg k = split_cfg(F::TYPE, NT, CPL4);
    const void *kern = (const void *)mmvq_split<F, NT, CPL4, k.depth, k.mode>;
    // split_ok bounds R by SPLIT_MAX_R at the table's workgroups per CU; a lower
    // occupancy clamp only raises R (the shares' LDS, 16 * NT * R bytes, stays small)
    int wpc = k.wg_per_cu;
    uint32_t R = 0, lds = 0;
    for (;;) {
        R = split_rows(a.N, num_cu, wpc);
        lds = 16u * (uint32_t)NT * R;
        const int fit = wg_fit(kern, lds);
        if (fit < 1)
            return hipErrorInvalidValue;
        if (fit >= wpc)
            break;
        wpc = fit;
    }
    const uint32_t grid = (a.N + R - 1u) / R;
    void *args[] = {(void *)&a.w, (void *)&a.qs, (void *)&a.d8, (void *)&a.y, (void *)&a.N,
                    (void *)&a.nbe, (void *)&a.stride, (void *)&a.K, (void *)&a.ldy,
                    (void *)&R};
    return hipLaunchKernel(kern, dim3(grid), dim3(WG), args, lds, s);
}

template <class F, int NT>
hipError_t dispatch_split(int cpl, int num_cu, hipStream_t s, const GemvArgs &a)
{
    switch ((cpl + 3) / 4) {
    case 2: return launch_split<F, NT, 2>(num_cu, s, a);
    case 3: return launch_split<F, NT, 3>(num_cu, s, a);
    default: return hipErrorInvalidValue;
    }
}

// Pairs of rows (mmvq_pairs) at 2..4 tokens when a row's chunk count is an odd
// multiple of 32 with at most 3 chunks per lane (K = 1024, 3072, 5120) and the pairs
// fill the grid at least twice over. Measured against one wave per row
// (graph-replayed GEMV, one MI355X): lm_head 152064 x 5120 at 2 / 3 / 4 tokens
// 97.3 -> 92.6, 104.5 -> 96.2, 110.6 -> 108.3 us; q4_K 27648 x 5120 at 4 tokens
// 23.9 -> 21.8; q5_K 27648 x 5120 at 2 tokens 22.5 -> 20.5; q6_K 16384 x 3072 at 4
// tokens 13.2 -> 11.2. At 4 and 5 chunks per lane (K = 7168, 9216) the pair's
// registers cost more than the idle half slot and it measured 3-25 % slower; with
// fewer pairs than waves (attn_v 1024 rows at 4 tokens: 4.3 -> 4.9 us) the halved
// wave count loses. Depth 2 (two pairs in flight) at one workgroup per CU.
constexpr int PAIRS_MAX_CPL = 3;

constexpr RowsCfg pairs_cfg(int type, int nt, int cpl)
{
    (void)type;
    (void)nt;
    (void)cpl;
    return RowsCfg{2, ACT_REGS, 1};
}

bool pairs_ok(int type, int nt, int cpl, int64_t N, int64_t K, int num_cu)
{
    const int n = nt < MAX_NT_KERNEL ? nt : MAX_NT_KERNEL;
    if (n < 2 || cpl > PAIRS_MAX_CPL || (K / 256 * 8) % 64 != 32)
        return false;
    const int64_t waves = (int64_t)num_cu * pairs_cfg(type, n, cpl).wg_per_cu * WAVES_PER_WG;
    return (N + 1) / 2 >= 2 * waves;
}

template <class F, int NT, int CPL>
hipError_t launch_pairs(int num_cu, hipStream_t s, GemvArgs a)
{
    constexpr RowsCfg k = pairs_cfg(F::TYPE, NT, CPL);
    const void *kern = (const void *)mmvq_pairs<F, NT, CPL, k.depth>;
    const int fit = wg_fit(kern);
    if (fit < 1)
        return hipErrorInvalidValue;
    const uint32_t grid = grid_for((a.N + 1u) / 2u, num_cu, k.wg_per_cu < fit ? k.wg_per_cu : fit);
    void *args[] = {(void *)&a.w, (void *)&a.qs, (void *)&a.d8, (void *)&a.y, (void *)&a.N,
                    (void *)&a.nbe, (void *)&a.stride, (void *)&a.K, (void *)&a.ldy};
    return hipLaunchKernel(kern, dim3(grid), dim3(WG), args, 0, s);
}

template <class F, int NT>
hipError_t dispatch_pairs(int cpl, int num_cu, hipStream_t s, const GemvArgs &a)
{
    switch (cpl) {
    case 1: return launch_pairs<F, NT, 1>(num_cu, s, a);
    case 2: return launch_pairs<F, NT, 2>(num_cu, s, a);
    case 3: return launch_pairs<F, NT, 3>(num_cu, s, a);
    default: return hipErrorInvalidValue;
    }
}

template <class F>
hipError_t launch_mmvq_fmt(const uint8_t *w, const uint8_t *q8, float *y, int64_t N, int64_t K,
                           int nt, int num_cu, hipStream_t s)
{
    const uint32_t nbe = (uint32_t)(K / 256);
    const int8_t *qs = reinterpret_cast<const int8_t *>(q8);
    const uint16_t *d8 = reinterpret_cast<const uint16_t *>(q8 + (size_t)nt * K);
    const int cpl = (int)((8u * nbe + 63u) / 64u);
    for (int t0 = 0; t0 < nt; t0 += MAX_NT_KERNEL) {
        const int n = nt - t0 < MAX_NT_KERNEL ? nt - t0 : MAX_NT_KERNEL;
        GemvArgs a;
        a.w = w;
        a.qs = qs + (size_t)t0 * K;
        a.d8 = d8 + (size_t)t0 * (K / 32);
        a.y = y + (size_t)t0 * N;
        a.N = (uint32_t)N;
        a.nbe = nbe;
        a.stride = (uint32_t)kq_row_stride(F::TYPE, nbe);
        a.K = (uint32_t)K;
        a.ldy = (uint32_t)N;
        hipError_t e;
        if (tiles_ok(F::TYPE, N, K, n, num_cu)) {
            e = launch_tiles(w, a.qs, a.d8, a.y, N, a.ldy, n, num_cu, s);
        } else if (pairs_ok(F::TYPE, n, cpl, N, K, num_cu)) {
            switch (n) {
            case 2: e = dispatch_pairs<F, 2>(cpl, num_cu, s, a); break;
            case 3: e = dispatch_pairs<F, 3>(cpl, num_cu, s, a); break;
            default: e = dispatch_pairs<F, 4>(cpl, num_cu, s, a); break;
            }
        } else if (split_ok(F::TYPE, n, cpl, N, num_cu)) {
            switch (n) {
            case 1: e = dispatch_split<F, 1>(cpl, num_cu, s, a); break;
            case 2: e = dispatch_split<F, 2>(cpl, num_cu, s, a); break;
            case 3: e = dispatch_split<F, 3>(cpl, num_cu, s, a); break;
            default: e = dispatch_split<F, 4>(cpl, num_cu, s, a); break;
            }
        } else if (cpl <= MAX_CPL) {
            const RowsCfg c = rows_cfg(F::TYPE, n, cpl);
            const auto seq = std::make_integer_sequence<int, MAX_CPL>{};
            switch (n) {
            case 1: e = dispatch_cpl<F, 1>(cpl, c, seq, num_cu, s, a); break;
            case 2: e = dispatch_cpl<F, 2>(cpl, c, seq, num_cu, s, a); break;
            case 3: e = dispatch_cpl<F, 3>(cpl, c, seq, num_cu, s, a); break;
            default: e = dispatch_cpl<F, 4>(cpl, c, seq, num_cu, s, a); break;
            }
        } else {
            switch (n) {
            case 1: e = launch(mmvq_long<F, 1>, num_cu, 2, s, a); break;
            case 2: e = launch(mmvq_long<F, 2>, num_cu, 2, s, a); break;
            case 3: e = launch(mmvq_long<F, 3>, num_cu, 2, s, a); break;
            default: e = launch(mmvq_long<F, 4>, num_cu, 2, s, a); break;
            }
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <class F>
hipError_t launch_fused_fmt(const uint8_t *w, const float *x, const float *gamma, float eps,
                            float *xn, uint8_t *q8, float *y, int64_t N, int64_t K, int num_cu,
                            hipStream_t s)
{
    const uint32_t nbe = (uint32_t)(K / 256);
    const int cpl = (int)((8u * nbe + 63u) / 64u);
    const RowsCfg c = rows_cfg(F::TYPE, 1, cpl);
    FusedArgs a;
    a.w = w;
    a.x = reinterpret_cast<const float4 *>(x);
    a.gamma = reinterpret_cast<const float4 *>(gamma);
    a.eps = eps;
    a.xn = reinterpret_cast<float4 *>(xn);
    a.qs = reinterpret_cast<uint32_t *>(q8);
    a.d8 = reinterpret_cast<uint16_t *>(q8 + (size_t)K);
    a.y = y;
    a.N = (uint32_t)N;
    a.nbe = nbe;
    a.stride = (uint32_t)kq_row_stride(F::TYPE, nbe);
    a.K = (uint32_t)K;
    a.ldy = (uint32_t)N;
    // q6_K rows of three to six chunks per lane: two workgroups per CU, where the GEMV
    // alone keeps one. The norm phase runs at one wave per SIMD, bound by its dependent
    // arithmetic; with two workgroups per CU it runs at two, half the rows per wave (same
    // bits out; one token, K = 5120: 152064 rows 90.26 -> 90.03 us, 65536 rows 41.69 ->
    // 40.38, where the GEMV alone at two ran 88.30 -> 89.53 and 39.76 -> 39.81; 32768
    // rows at K = 8192 35.31 -> 33.42, 10240 43.60 -> 41.45, 12288 51.54 -> 50.01). Only
    // from four rows per wave at two workgroups per CU: every workgroup redoes the norm,
    // and 4096 rows at K = 10240 (two rows per wave) measured 10.86 -> 12.28.
    const bool two = F::TYPE == KQT_Q6_K && cpl >= 3 && cpl <= 6 &&
                     N >= (int64_t)4 * 2 * WAVES_PER_WG * num_cu;
    const int wpc = two ? 2 : c.wg_per_cu;
    return dispatch_fused<F, 1>(cpl, c.depth, std::make_integer_sequence<int, FUSED_MAX_CPL>{},
                                num_cu, wpc, s, a);
}

template <class F, int CPL>
hipError_t launch_gate_up_cpl(int num_cu, hipStream_t s, const uint8_t *w, const int8_t *qs,
                              const uint16_t *d8, float *gu, float *y, uint8_t *qs_out,
                              uint16_t *d8_out, uint32_t Nh, uint32_t nbe, uint32_t stride,
                              uint32_t K)
{
    const void *kern = (const void *)gate_up_swiglu_rows<F, CPL>;
    const int fit = wg_fit(kern);
    if (fit < 1)
        return hipErrorInvalidValue;
    const uint32_t nblk = Nh / 32u;
    const uint32_t slots = (uint32_t)num_cu * (uint32_t)(fit < 2 ? fit : 2);
    const uint32_t grid = nblk < slots ? nblk : slots;
    void *args[] = {(void *)&w, (void *)&qs, (void *)&d8, (void *)&gu, (void *)&y,
                    (void *)&qs_out, (void *)&d8_out, (void *)&Nh, (void *)&nbe,
                    (void *)&stride, (void *)&K};
    return hipLaunchKernel(kern, dim3(grid), dim3(WG), args, 0, s);
}

template <class F, int... CPLS>
hipError_t dispatch_gate_up(int cpl, std::integer_sequence<int, CPLS...>, int num_cu,
                            hipStream_t s, const uint8_t *w, const int8_t *qs, const uint16_t *d8,
                            float *gu, float *y, uint8_t *qs_out, uint16_t *d8_out, uint32_t Nh,
                            uint32_t nbe, uint32_t stride, uint32_t K)
{
    hipError_t e = hipErrorInvalidValue;
    (void)((cpl == CPLS + 1 ? (e = launch_gate_up_cpl<F, CPLS + 1>(num_cu, s, w, qs, d8, gu, y,
                                                                   qs_out, d8_out, Nh, nbe,
                                                                   stride, K),
                               true)
                            : false) ||
           ...);
    return e;
}

template <class F>
hipError_t launch_gate_up_fmt(const uint8_t *w, const uint8_t *q8_in, float *gu, float *y,
                              uint8_t *q8_out, int64_t Nh, int64_t K, int num_cu, hipStream_t s)
{
    const uint32_t nbe = (uint32_t)(K / 256);
    const int cpl = (int)((8u * nbe + 63u) / 64u);
    const int8_t *qs = reinterpret_cast<const int8_t *>(q8_in);
    const uint16_t *d8 = reinterpret_cast<const uint16_t *>(q8_in + (size_t)K);
    uint16_t *d8_out = reinterpret_cast<uint16_t *>(q8_out + (size_t)Nh);
    return dispatch_gate_up<F>(cpl, std::make_integer_sequence<int, GATE_UP_MAX_CPL>{}, num_cu, s,
                               w, qs, d8, gu, y, q8_out, d8_out, (uint32_t)Nh, nbe,
                               (uint32_t)kq_row_stride(F::TYPE, nbe), (uint32_t)K);
}

}  // namespace

MmvqPlan plan_mmvq(int type, int64_t N, int64_t K, int nt, int num_cu)
{
    MmvqPlan p;
    const int64_t nbe = K / 256;
    p.cpl = (int)((8 * nbe + 63) / 64);
    p.unrolled = p.cpl <= MAX_CPL;
    p.launches = (nt + MAX_NT_KERNEL - 1) / MAX_NT_KERNEL;
    const int nt0 = nt < MAX_NT_KERNEL ? nt : MAX_NT_KERNEL;
    if (tiles_ok(type, N, K, nt0, num_cu)) {
        p.tiles = true;
        p.act_mode = ACT_REGS;
        p.depth = 2;
        const int64_t T = (N + 15) / 16;
        p.grid = (uint32_t)(T < num_cu ? T : num_cu);
        return p;
    }
    if (pairs_ok(type, nt0, p.cpl, N, K, num_cu)) {
        p.paired = true;
        const RowsCfg c = pairs_cfg(type, nt0, p.cpl);
        p.act_mode = c.mode;
        p.depth = c.depth;
        p.grid = grid_for((N + 1) / 2, num_cu, c.wg_per_cu);
        return p;
    }
    if (split_ok(type, nt0, p.cpl, N, num_cu)) {
        p.shared = true;
        p.cpl = (p.cpl + 3) / 4;
        const RowsCfg c = split_cfg(type, nt0, p.cpl);
        const uint32_t R = split_rows(N, num_cu, c.wg_per_cu);
        p.act_mode = c.mode;
        p.depth = c.depth;
        p.grid = (uint32_t)((N + R - 1) / R);
        return p;
    }
    const RowsCfg c = p.unrolled ? rows_cfg(type, nt0, p.cpl) : RowsCfg{1, ACT_GLOBAL, 2};
    p.act_mode = c.mode;
    p.depth = c.depth;
    p.grid = grid_for(N, num_cu, c.wg_per_cu);
    return p;
}

hipError_t launch_mmvq(int type, const uint8_t *w, const uint8_t *q8, float *y, int64_t N,
                       int64_t K, int nt, int num_cu, hipStream_t s)
{
    switch (type) {
    case KQT_Q6_K: return launch_mmvq_fmt<FmtQ6K>(w, q8, y, N, K, nt, num_cu, s);
    case KQT_Q4_K: return launch_mmvq_fmt<FmtQ4K>(w, q8, y, N, K, nt, num_cu, s);
    case KQT_Q5_K: return launch_mmvq_fmt<FmtQ5K>(w, q8, y, N, K, nt, num_cu, s);
    default: return hipErrorInvalidValue;
    }
}

bool rmsnorm_mmvq_fused(int64_t K, int nt)
{
    return fused_ok(nt, (int)((K / 256 * 8 + 63) / 64));
}

hipError_t launch_rmsnorm_mmvq(int type, const uint8_t *w, const float *x, const float *gamma,
                               float eps, float *xn, uint8_t *q8, float *y, int64_t N, int64_t K,
                               int nt, int num_cu, hipStream_t s)
{
    if (!rmsnorm_mmvq_fused(K, nt)) {
        // the producer writes the q8 plane, then the GEMV reads it
        const hipError_t e = launch_rmsnorm_quant(x, gamma, eps, xn, q8, K, nt, s);
        if (e != hipSuccess)
            return e;
        return launch_mmvq(type, w, q8, y, N, K, nt, num_cu, s);
    }
    switch (type) {
    case KQT_Q6_K: return launch_fused_fmt<FmtQ6K>(w, x, gamma, eps, xn, q8, y, N, K, num_cu, s);
    case KQT_Q4_K: return launch_fused_fmt<FmtQ4K>(w, x, gamma, eps, xn, q8, y, N, K, num_cu, s);
    case KQT_Q5_K: return launch_fused_fmt<FmtQ5K>(w, x, gamma, eps, xn, q8, y, N, K, num_cu, s);
    default: return hipErrorInvalidValue;
    }
}

bool gate_up_swiglu_fused(int64_t K)
{
    return gate_up_ok((int)((K / 256 * 8 + 63) / 64));
}

hipError_t launch_gate_up_swiglu(int type, const uint8_t *w, const uint8_t *q8_in, float *gu,
                                 float *y, uint8_t *q8_out, int64_t Nh, int64_t K, int num_cu,
                                 hipStream_t s)
{
    if (!gate_up_swiglu_fused(K)) {
        // the GEMV writes gu, then the SwiGLU producer reads its two halves
        const hipError_t e = launch_mmvq(type, w, q8_in, gu, 2 * Nh, K, 1, num_cu, s);
        if (e != hipSuccess)
            return e;
        return launch_swiglu_quant(gu, gu + Nh, y, q8_out, Nh, 1, s);
    }
    switch (type) {
    case KQT_Q6_K: return launch_gate_up_fmt<FmtQ6K>(w, q8_in, gu, y, q8_out, Nh, K, num_cu, s);
    case KQT_Q4_K: return launch_gate_up_fmt<FmtQ4K>(w, q8_in, gu, y, q8_out, Nh, K, num_cu, s);
    case KQT_Q5_K: return launch_gate_up_fmt<FmtQ5K>(w, q8_in, gu, y, q8_out, Nh, K, num_cu, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_subdots(int type, const uint8_t *w, const uint8_t *q8, int32_t *dots,
                          int64_t N, int64_t K, int nt, int num_cu, hipStream_t s)
{
    uint32_t nbe = (uint32_t)(K / 256);
    uint32_t stride = (uint32_t)kq_row_stride(type, nbe);
    const int8_t *qs = reinterpret_cast<const int8_t *>(q8);
    const uint16_t *d8 = reinterpret_cast<const uint16_t *>(q8 + (size_t)nt * K);
    const void *kern = type == KQT_Q6_K  ? (const void *)mmvq_subdots_kernel
                       : type == KQT_Q5_K ? (const void *)kq_subdots_kernel<true>
                                          : (const void *)kq_subdots_kernel<false>;
    const int fit = wg_fit(kern);
    if (fit < 1)
        return hipErrorInvalidValue;
    uint32_t grid = grid_for(N, num_cu, fit < 4 ? fit : 4);
    uint32_t Nu = (uint32_t)N, Ku = (uint32_t)K, ntu = (uint32_t)nt;
    if (type == KQT_Q6_K) {
        void *args[] = {(void *)&w, (void *)&qs, (void *)&dots, (void *)&Nu,
                        (void *)&nbe, (void *)&stride, (void *)&Ku, (void *)&ntu};
        return hipLaunchKernel(kern, dim3(grid), dim3(WG), args, 0, s);
    }
    void *args[] = {(void *)&w, (void *)&qs, (void *)&d8, (void *)&dots, (void *)&Nu,
                    (void *)&nbe, (void *)&stride, (void *)&Ku, (void *)&ntu};
    return hipLaunchKernel(kern, dim3(grid), dim3(WG), args, 0, s);
}

}  // namespace q6k
