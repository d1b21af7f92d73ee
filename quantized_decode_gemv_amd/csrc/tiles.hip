// tiles.hip -- q6_K x q8 decode GEMV for 3-4 tokens on the int8 matrix cores
// (gfx950 v_mfma_i32_16x16x64_i8), rows of 20 super-blocks (K = 5120, lm_head width).
//
// What is computed is the row kernels' sum (D4-2 §3.2 Excerpt C; D4-4 §3.2 Excerpt B):
// y[t][r] = sum over the row's 16-element sub-blocks of d * sc * d8 * D, D the exact
// int32 dot of (q - 32) with the token's int8 activations. Only the order of the float
// additions differs from the row kernels.
//
// At several tokens the row kernels spend most of a wave's issue cycles on the dot
// products and their conversions. Here one matrix instruction takes the integer dots
// of 16 rows x 4 sub-blocks x 4 tokens:
//  - B (64 x 16, one column per weight row): lane (r, g), g = lane / 16, holds 16 codes
//    of row r, those of one sub-block; which sub-block the K-group g carries is fixed
//    per step (below), the same for all 16 rows;
//  - A (16 x 64, one row per (token t, sub-block slot s), row index 4s + t): the token's
//    16 activations of slot s's sub-block in K-group s, zeros in the other K-groups;
//  - C: -32 * (sum of those 16 activations), which folds the code offset in;
//  - D = A * B + C, lane (r, g) receives rows 4g .. 4g + 3 of column r: the four tokens'
//    exact sub-block dots of its own row and slot g, next to that row's scales.
// The K order inside a K-group is whatever the instruction uses; A and B share it, and
// a K-group holds one whole sub-block in both, so the result does not depend on it.
//
// Tiles of 16 consecutive rows are one contiguous run of 16 * stride bytes. A
// workgroup's four waves copy a tile into LDS with buffer-to-LDS loads in 1 KB pieces
// (contiguous requests, no registers held in flight; per-row runs of a few hundred
// bytes measured markedly slower, as the row stride is not a multiple of the 128-byte
// line) into one of two tile buffers, while they compute the other. Wave v computes
// super-blocks 5v .. 5v + 4 of all 16 rows; the four partial sums of a row meet in
// LDS, and wave t adds them for token t and stores y after a later tile's landing
// (every tile at 4 tokens, every fourth at 3). Its activation operands (A, C and the
// q8 block scales, as fp16 pairs) depend only on the wave's K quarter, so they are
// loaded once and stay in registers for every tile (about 256 registers at 4 tokens; C
// read from an LDS table per step instead measured about 4 us slower). Per tile: two
// barriers (buffer free; tile landed), each wave's own copies awaited with a counted
// wait (vm_wait), as the compiler does not count buffer-to-LDS loads. An output store
// made after tile s - 1's landing lies between the copies of tile s and those of tile
// s + 1 in issue order; loads complete in issue order, so while a copy of tile s is
// outstanding all RUNS copies of tile s + 1 are too, and a count of at most RUNS
// still means that tile s has landed, whenever the store completes.
//
// What bounds it: two 66 KB tile buffers are what LDS holds, so a CU has at most one
// tile in flight, and none between the landing of one tile's copies and the issue of
// the next, which waits for the compute of the tile before. The copies alone (no
// arithmetic) run the matrix in 92 us, the arithmetic alone in 58 us. Rows past the
// last whole round of 16-row tiles are shared out evenly, one short tile per workgroup
// (at lm_head 2 rows each, where 32 of 256 workgroups would otherwise take a 38th tile
// alone); with whole tiles known to be 16 rows the loop also compiles tighter (1.3 us
// less at 65536 rows, which have no remainder). Measured and not kept: eight waves (two
// per K quarter, each two of a super-block's four steps) and codes built with 64-bit
// shifts were slower at 3 tokens and equal at 4; loading the activation operands into
// the first tile's buffer, or into an LDS area of their own beside two smaller tiles,
// was slower at 4 tokens.
//
// Super-block sb of a row, lane K-group g = 2c + a (c the 128-element half, a the
// 32-element unit inside it): the lane's 32 low-bit bytes (ql 128 sb + 32 g) hold
// the codes of unit a (low nibbles) and unit a + 2 (high nibbles), positions 0..31;
// their 2-bit fields are the 32 qh bytes at 64 sb + 32 c, fields 2a and 2a + 4. The
// four steps of a super-block take, in K-group g: step 0 unit a positions 0..15,
// step 1 positions 16..31, steps 2 and 3 the same of unit a + 2, i.e. sub-blocks
// 8c + 2a + {0, 1, 4, 5}, whose scales are bytes 2a + {0, 1, 4, 5} of the 8-byte group
// at 16 sb + 8c of the scale plane. Steps 0 and 1 lie in one q8 block (8 sb + 4c + a),
// steps 2 and 3 in block + 2, so each pair's two scaled dots add exactly in int32
// (|sc * D| <= 128 * 16 * 32 * 128 = 2^23, their sum at most 2^24, exact in f32) before
// one conversion.

#include "q6k_internal.h"
#include "q6k_unit.h"

namespace q6k {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t TILE_ROWS = 16;
constexpr uint32_t TILE_NBE = 20;        // super-blocks per row (K = 5120)

template <uint32_t NBE>
struct TileGeom {
    static constexpr int WAVES = 4;                             // one per K quarter
    static constexpr uint32_t STRIDE = (uint32_t)kq_row_stride(KQT_Q6_K, NBE);
    static constexpr uint32_t BYTES = TILE_ROWS * STRIDE;
    static constexpr uint32_t RUNS = (BYTES + 1024u * WAVES - 1u) / (1024u * WAVES);   // 1 KB
                                                                 // copies per wave per tile
    static constexpr uint32_t BUF = WAVES * RUNS * 1024u;       // one tile buffer (copies past
                                                                 // the tile land zeros here)
    static constexpr uint32_t SPW = NBE / 4;                    // super-blocks per K quarter
    static_assert(NBE % 4 == 0, "whole K quarters");
    static_assert(RUNS <= 63, "vmcnt range");
};

__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t *)p;
}

// x + (x of lane l ^ 32), and x + (x of lane l ^ 16): the values and the order of
// x + __shfl_xor(x, 32 or 16), with the lanes exchanged in the vector ALU
// (v_permlane32_swap / v_permlane16_swap) instead of by a permute through LDS, whose
// round trip sat in every tile's reduction. With both operands x, the 32-lane swap
// returns (x of lane l - 32 in the upper half) and (x of lane l + 32 in the lower
// half); the 16-lane swap does the same for the odd and even 16-lane rows. (The two
// results are copied into plain integers before their bit casts: a bit cast applied
// straight to an element of the returned pair reads element 0 for both.)
__device__ __forceinline__ float add_xor32(float x, uint32_t lane)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned h0 = h[0], h1 = h[1];
    return x + __builtin_bit_cast(float, lane < 32u ? h1 : h0);
}

__device__ __forceinline__ float add_xor16(float x, uint32_t lane)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto h = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned h0 = h[0], h1 = h[1];
    return x + __builtin_bit_cast(float, (lane & 16u) ? h0 : h1);
}

__device__ __forceinline__ i32x4 as_i32x4(uint4 v)
{
    i32x4 r;
    r.x = (int)v.x;
    r.y = (int)v.y;
    r.z = (int)v.z;
    r.w = (int)v.w;
    return r;
}

template <int NT, uint32_t NBE>
__global__ __launch_bounds__(256) void mmvq_tiles(const uint8_t *__restrict__ w,
                                                  const int8_t *__restrict__ qs,
                                                  const uint16_t *__restrict__ d8,
                                                  float *__restrict__ y, uint32_t N, uint32_t ldy)
{
    using TG = TileGeom<NBE>;
    constexpr int WAVES = TG::WAVES;
    constexpr uint32_t SPW = TG::SPW;
    constexpr uint32_t K = 256u * NBE;
    __shared__ __align__(16) uint8_t tbuf[2 * TG::BUF];
    // tiles per output store (see store_tiles), and the partial sums of the last PSLOTS
    // tiles: [tile % PSLOTS][wave][token][row]. At 3 tokens one store per four tiles
    // measured 0.1-0.8 us faster than one per tile; at 4 tokens, where the loop holds
    // about 256 registers, the wider store path measured 2-3 us slower.
    constexpr uint32_t PER = NT == 4 ? 1u : 4u;
    constexpr uint32_t PSLOTS = 2u * PER;
    __shared__ float part[PSLOTS][WAVES][4][TILE_ROWS];

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // K quarter
    const uint32_t r = lane & 15u, g = lane >> 4, c = g >> 1, a = g & 1u;
    // Tiles: FR rounds of whole 16-row tiles, tile blockIdx.x + s * NG in round s (the grid
    // streams neighbouring tiles together), then, if rows remain (fewer than 16 * NG), one
    // round in which every workgroup takes an equal share of them (at most 16 rows), so
    // that no few workgroups run a round alone. Every workgroup has S tiles.
    const uint32_t NG = gridDim.x;
    const uint32_t FR = N / (TILE_ROWS * NG);
    const uint32_t rows_full = FR * TILE_ROWS * NG;
    const uint32_t rest = N - rows_full;
    const uint32_t share = (rest + NG - 1u) / NG;
    const uint32_t S = FR + (rest ? 1u : 0u);
    // the workgroup's place in a round of whole tiles: workgroup b runs on XCD b % 8, and
    // the two tiles whose outputs share a 128-byte line of y (16 rows x 4 bytes each, per
    // token) go to two workgroups of one XCD, so that the line is written through one L2
    // (pieces of a line written back from several L2s measured slower)
    const uint32_t bx = blockIdx.x;
    const uint32_t place = NG % 16u == 0 ? (bx & ~15u) + 2u * (bx & 7u) + ((bx >> 3) & 1u) : bx;
    // first row and rows of tile s (none past the last)
    auto tile_rows = [&](uint32_t s, uint32_t &r0) -> uint32_t {
        if (s < FR) {
            r0 = (place + s * NG) * TILE_ROWS;
            return TILE_ROWS;
        }
        r0 = rows_full + blockIdx.x * share;
        return s == FR && r0 < N ? (N - r0 < share ? N - r0 : share) : 0u;
    };
    const uint32_t lds0 = lds_offset(tbuf);

    // tile s into buffer b (the copies of rows past the tile's, and of a tile past the
    // last, write zeros without a memory request)
    auto copy_tile = [&](uint32_t b, uint32_t s) {
        uint32_t r0;
        const uint32_t rows = tile_rows(s, r0);
        const __amdgpu_buffer_rsrc_t rs =
            buf_desc(w + (size_t)(rows ? r0 : 0u) * TG::STRIDE, rows * TG::STRIDE);
#pragma unroll
        for (uint32_t m = 0; m < TG::RUNS; ++m) {
            const uint32_t run = wv + WAVES * m;
            dma_b128(rs, 16u * lane, 1024u * run, lds0 + b * TG::BUF + 1024u * run);
        }
    };
    // wave t (a token) stores token t's outputs of tiles j0 .. j0 + PER - 1 (those below
    // S) in one store: lane l takes row l % 16 of tile j0 + l / 16, the sum of the waves'
    // partial sums of that row, added in wave order
    auto store_tiles = [&](uint32_t j0) {
        uint32_t r0 = 0, rows, j, rr;
        if constexpr (PER == 1) {
            j = j0;
            rr = lane;
            rows = tile_rows(j0, r0);
        } else {
            j = j0 + (lane >> 4u);
            rr = lane & 15u;
            rows = (lane >> 4u) < PER && j < S ? tile_rows(j, r0) : 0u;
        }
        if (rr < rows) {
            const uint32_t sl = j % PSLOTS;
            float tot = part[sl][0][wv][rr];
#pragma unroll
            for (int u = 1; u < WAVES; ++u)
                tot += part[sl][u][wv][rr];
            y[(size_t)wv * ldy + r0 + rr] = tot;
        }
    };

    // the wave's activation operands, the same for every tile: A and C in registers, the
    // q8 block scales as fp16 pairs (tokens 0, 1 and 2, 3). They are requested before the
    // first tile's copies, as a wave's loads complete in issue order and would otherwise
    // wait behind them. The scales come as one 16-byte load per token and super-block.
    i32x4 A[4 * SPW], C[4 * SPW];
    const i32x4 NEG32 = {(int)0xE0E0E0E0u, (int)0xE0E0E0E0u, (int)0xE0E0E0E0u, (int)0xE0E0E0E0u};
    const i32x4 ZERO4 = {0, 0, 0, 0};
    uint32_t Fh[2 * SPW][2];
    {
        const uint32_t ia = lane & 15u, ta = ia & 3u, sa = ia >> 2;
        const bool live = sa == g && ta < (uint32_t)NT;
        const __amdgpu_buffer_rsrc_t xr = buf_desc(qs, NT * K);
        const uint32_t xbase = live ? ta * K : NT * K;   // past the extent: zeros
#pragma unroll
        for (uint32_t m = 0; m < SPW; ++m) {
            const uint32_t sb = SPW * wv + m;
#pragma unroll
            for (uint32_t j = 0; j < 4; ++j) {
                const uint32_t off = 256u * sb + 128u * c + 32u * a + 64u * (j >> 1) + 16u * (j & 1u);
                const uint4 x = load_b128<POLICY_DEFAULT>(xr, xbase + (live ? off : 0u));
                A[4 * m + j] = as_i32x4(x);
                // C = A times a B of all -32: every column holds -32 * (the sum of each A
                // row), and lane (r, g) receives rows 4g .. 4g + 3, the four tokens' sums
                // of slot g, in the layout the step's own product adds them to (exact:
                // at most 16 * 128 * 32 in magnitude)
                C[4 * m + j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[4 * m + j], NEG32, ZERO4, 0, 0, 0);
            }
            // the super-block's 8 q8 block scales of each token (16 bytes), of which
            // blocks 4c + a and 4c + a + 2 are this lane's
            const __amdgpu_buffer_rsrc_t dr = buf_desc(d8, NT * (K / 32u) * 2u);
            uint32_t hv[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint4 q = load_b128<POLICY_DEFAULT>(dr, (uint32_t)t * (K / 16u) + 16u * sb);
                // block 4c + a is half a of word 2c, block 4c + a + 2 half a of word 2c + 1
                const uint32_t lo = c ? q.z : q.x, hi2 = c ? q.w : q.y;
                hv[0][t] = (lo >> (16u * a)) & 0xFFFFu;
                hv[1][t] = (hi2 >> (16u * a)) & 0xFFFFu;
            }
#pragma unroll
            for (uint32_t p = 0; p < 2; ++p) {
                Fh[2 * m + p][0] = hv[p][0] | (hv[p][1] << 16);
                Fh[2 * m + p][1] = hv[p][2] | (hv[p][3] << 16);
            }
        }
    }
    copy_tile(0, 0);

    const uint32_t sh = 2u * a, up = 4u - sh;
    const uint32_t M = 0x33333333u << sh;
    for (uint32_t s = 0; s < S; ++s) {
        const uint32_t b = s & 1u;
        __syncthreads();            // every wave is done with buffer b ^ 1 (tile s - 1)
        copy_tile(b ^ 1u, s + 1u);
        vm_wait<(int)TG::RUNS>();   // this wave's copies of tile s have landed
        __syncthreads();            // and every wave's
        if (s % PER == 0 && s > 0 && wv < (uint32_t)NT)
            store_tiles(s - PER);
        const uint8_t *rb = tbuf + b * TG::BUF + r * TG::STRIDE;
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = 0.0f;
#pragma unroll
        for (uint32_t m = 0; m < SPW; ++m) {
            const uint32_t sb = SPW * wv + m;
            const uint4 q0 = *reinterpret_cast<const uint4 *>(rb + 128u * sb + 32u * g);
            const uint4 q1 = *reinterpret_cast<const uint4 *>(rb + 128u * sb + 32u * g + 16u);
            const uint4 h0 = *reinterpret_cast<const uint4 *>(rb + 128u * NBE + 64u * sb + 32u * c);
            const uint4 h1 = *reinterpret_cast<const uint4 *>(rb + 128u * NBE + 64u * sb + 32u * c + 16u);
            const uint32_t dbits = *reinterpret_cast<const uint16_t *>(rb + 208u * NBE + 2u * sb);
            const float d = f16_bits_to_f32(dbits);
            const uint2 sc = *reinterpret_cast<const uint2 *>(rb + 192u * NBE + 16u * sb + 8u * c);
            uint4 k0, k1, k2, k3;
            uint32_t hm;
            hm = h0.x & M; k0.x = codes_lo(q0.x, hm, up); k2.x = codes_hi(q0.x, hm, sh);
            hm = h0.y & M; k0.y = codes_lo(q0.y, hm, up); k2.y = codes_hi(q0.y, hm, sh);
            hm = h0.z & M; k0.z = codes_lo(q0.z, hm, up); k2.z = codes_hi(q0.z, hm, sh);
            hm = h0.w & M; k0.w = codes_lo(q0.w, hm, up); k2.w = codes_hi(q0.w, hm, sh);
            hm = h1.x & M; k1.x = codes_lo(q1.x, hm, up); k3.x = codes_hi(q1.x, hm, sh);
            hm = h1.y & M; k1.y = codes_lo(q1.y, hm, up); k3.y = codes_hi(q1.y, hm, sh);
            hm = h1.z & M; k1.z = codes_lo(q1.z, hm, up); k3.z = codes_hi(q1.z, hm, sh);
            hm = h1.w & M; k1.w = codes_lo(q1.w, hm, up); k3.w = codes_hi(q1.w, hm, sh);
            const i32x4 D0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[4 * m + 0], as_i32x4(k0), C[4 * m + 0], 0, 0, 0);
            const i32x4 D1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[4 * m + 1], as_i32x4(k1), C[4 * m + 1], 0, 0, 0);
            const i32x4 D2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[4 * m + 2], as_i32x4(k2), C[4 * m + 2], 0, 0, 0);
            const i32x4 D3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[4 * m + 3], as_i32x4(k3), C[4 * m + 3], 0, 0, 0);
            const int s0 = (int)(int8_t)(uint8_t)(sc.x >> (16u * a));
            const int s1 = (int)(int8_t)(uint8_t)(sc.x >> (16u * a + 8u));
            const int s2 = (int)(int8_t)(uint8_t)(sc.y >> (16u * a));
            const int s3 = (int)(int8_t)(uint8_t)(sc.y >> (16u * a + 8u));
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int i0 = __mul24(s0, D0[t]) + __mul24(s1, D1[t]);
                const int i1 = __mul24(s2, D2[t]) + __mul24(s3, D3[t]);
                const float f0 = f16_bits_to_f32(Fh[2 * m][t >> 1] >> (16 * (t & 1)));
                const float f1 = f16_bits_to_f32(Fh[2 * m + 1][t >> 1] >> (16 * (t & 1)));
                // d * (d8 * i0 + d8' * i1): the super-block's two q8 blocks, then its scale
                const float u = __builtin_fmaf(f1, (float)i1, (float)i0 * f0);
                acc[t] = __builtin_fmaf(d, u, acc[t]);
            }
        }
        // row r's sum over the four K-groups (the same value in all four lanes), then
        // lane (r, g) posts token g's
        float mine = 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float x = acc[t];
            x = add_xor32(x, lane);
            x = add_xor16(x, lane);
            mine = g == (uint32_t)t ? x : mine;
        }
        part[s % PSLOTS][wv][g][r] = mine;
    }
    __syncthreads();
    if (wv < (uint32_t)NT)
        store_tiles((S - 1u) / PER * PER);
    // no copy may still be landing in LDS when the workgroup ends
    vm_wait<0>();
}

template <int NT>
hipError_t launch_nt(const uint8_t *w, const int8_t *qs, const uint16_t *d8, float *y,
                     uint32_t N, uint32_t ldy, int num_cu, hipStream_t s)
{
    constexpr int threads = 64 * TileGeom<TILE_NBE>::WAVES;   // 256, the size wg_fit assumes
    const void *kern = (const void *)mmvq_tiles<NT, TILE_NBE>;
    const int fit = wg_fit(kern);
    if (fit < 1)
        return hipErrorInvalidValue;
    const uint32_t T = (N + TILE_ROWS - 1u) / TILE_ROWS;
    const uint32_t full = (uint32_t)num_cu * (uint32_t)fit;
    const uint32_t grid = T < full ? T : full;
    void *args[] = {(void *)&w, (void *)&qs, (void *)&d8, (void *)&y, (void *)&N, (void *)&ldy};
    return hipLaunchKernel(kern, dim3(grid), dim3(threads), args, 0, s);
}

}  // namespace

// Measured against the row pairs (graph-replayed GEMV at K = 5120, one MI355X, the
// libraries on one box): lm_head 152064 rows at 4 tokens 105.6 -> 95.8 us (the LDS ring
// this kernel replaced measured 100.5-102.2), at 3 tokens 95.6 -> 94.3. Each
// workgroup pays a fixed start (its operands, the first tile's copy) that only many
// tiles amortize. At 4 tokens the tiles beat the register row pairs from 45056 rows (11
// tiles per CU: 32.9 -> 32.7 us; 49152 rows, 12 per CU, 35.9 -> 35.0) and lose below
// (40960 rows 30.0 -> 30.3, 32768 rows 24.6 -> 25.7, 1024 rows 4.0 -> 7.4); at 3 tokens
// from 90112 rows (22 per CU: 58.0 -> 57.3 us; 98304 rows 62.3 -> 62.0; 131072 rows
// 83.2 -> 80.8) and lose at 81920 (52.5 -> 53.0). The thresholds keep one (4 tokens)
// and two (3 tokens) tiles per CU of margin above the crossings. At 2 tokens the first
// form of this kernel measured 92.6 -> 94.8 us at lm_head, so 2 tokens keep the pairs.
bool tiles_ok(int type, int64_t N, int64_t K, int nt, int num_cu)
{
    if (type != KQT_Q6_K || K != 256 * (int64_t)TILE_NBE || nt < 3 || nt > 4)
        return false;
    const int64_t tiles = (N + TILE_ROWS - 1) / TILE_ROWS;
    return tiles >= (int64_t)(nt == 4 ? 12 : 24) * num_cu;
}

hipError_t launch_tiles(const uint8_t *w, const int8_t *qs, const uint16_t *d8, float *y,
                        int64_t N, int64_t ldy, int nt, int num_cu, hipStream_t s)
{
    switch (nt) {
    case 3: return launch_nt<3>(w, qs, d8, y, (uint32_t)N, (uint32_t)ldy, num_cu, s);
    case 4: return launch_nt<4>(w, qs, d8, y, (uint32_t)N, (uint32_t)ldy, num_cu, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace q6k
