/*
 * q6k_oracle.c -- the oracle for the q6_K x q8 batch-1 decode GEMV (MMVQ) path.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load the library built from this file. The HIP library
 * (quantized_decode_gemv_amd/) never calls it, and the two share no code, header,
 * table or helper.
 *
 * Plain, slow, scalar C, written to be checked against the pages by eye. Floating
 * point is fp64 except where the pages fix f32 (the q8 quantizer) or the stated
 * reading fixes f32 (the rounding of the RMSNorm factor and output).
 * Build: gcc -O2 -fPIC -shared -std=gnu11 -ffp-contract=off -fno-fast-math -fopenmp -lm
 *
 * Sources (page titles; the section, excerpt or equation is given at each function):
 *   [D4-4] "76 · D4-4 -- the endgame kernel session: dpl dense split-plane q6_K
 *           decode MMVQ lands (bitwise)"
 *   [D4-2] "74 · D4-2 -- B0 latent correctness fix + all bitwise occupancy/prefetch
 *           axes closed"
 *   [D3-5] "70 · D3-5 -- decode-alignment plan Stage 1: fused-producer decode
 *           A-quantize"
 *
 * The SwiGLU producer (orc_swiglu) is the plain definition silu(g) * u evaluated in
 * fp64 (libm exp, then three fp64 operations, each relative error ~2^-53) and rounded
 * to f32 at the end: within an f32 ulp of the exactly rounded value, not always equal
 * to it. The pages' f32 body rounds at each step, so the HIP producer is compared to
 * it within a few ulp (its last bits are not pinned).
 *
 * Parity pins (tests/test_oracle_*.py): every function here is pinned by something
 * other than itself -- hand-worked addressing fixtures, closed forms, exact
 * integer sums, brute force on tiny inputs and the raw == padded == dpl invariant.
 * The RMSNorm reduction order is the one part whose bit pattern is not fixed by the
 * pages; its value is pinned by closed forms only (see orc_rmsnorm).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_SHAPE (-1)
#define ORC_E_VALUE (-2)

/* Row layouts of a q6_K weight matrix. */
#define ORC_RAW 0    /* GGUF super-blocks back to back, 210 B each                     */
#define ORC_PAD224 1 /* each 210 B block followed by 14 zero bytes (224 B stride)      */
#define ORC_DPL 2    /* per row [ql: nbe*128][qh: nbe*64][sc: nbe*16][d: nbe*2], pad   */

/* ------------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary64 / binary32                                           */
/* ------------------------------------------------------------------------------ */

/* Exact value of a binary16 bit pattern. Infinities and NaNs map to +-inf / NaN. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even (IEEE 754 default). */
uint16_t orc_f32_to_f16(float f)
{
    double a = fabs((double)f);
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return sign | 0x7E00;
    if (a >= 65520.0) /* at or above the midpoint between 65504 and 2^16 */
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);            /* a = fr * 2^ex, fr in [0.5, 1) -> unbiased exponent ex-1 */
    int E = ex - 1;
    if (E < -14)
        E = -14;              /* subnormal range: quantum 2^-24                          */
    double quantum = ldexp(1.0, E - 10);
    double n = rint(a / quantum); /* a/quantum is exact; rint is ties-to-even           */
    /* n * quantum may have carried into the next binade; encode from the integer. */
    if (E == -14 && n < 1024.0)
        return sign | (uint16_t)n;            /* subnormal                                */
    if (n >= 2048.0) {                        /* carried: 2^(E+1), mantissa 0            */
        n = 1024.0;
        E += 1;
    }
    int biased = E + 15;
    if (biased >= 31)
        return sign | 0x7C00;
    return sign | (uint16_t)(biased << 10) | (uint16_t)((int)n - 1024);
}

/* ------------------------------------------------------------------------------ */
/* Row layouts                                                                     */
/* ------------------------------------------------------------------------------ */

/* Bytes per row. The dpl stride pads nbe*210 content bytes up to a multiple of 16
 * ([D4-4] §2 "The dpl split-plane's layout ledger" and §3.2 Excerpt A: nbe*210
 * rounded up with (x + 15) & ~15; the worked case nbe 54 -> 11340 -> 11344). */
int64_t orc_row_stride(int layout, int64_t K)
{
    if (K <= 0 || K % 256)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    switch (layout) {
    case ORC_RAW: return nbe * 210;
    case ORC_PAD224: return nbe * 224;
    case ORC_DPL: return (nbe * 210 + 15) & ~(int64_t)15;
    default: return ORC_E_SHAPE;
    }
}

typedef struct {
    const uint8_t *ql, *qh, *sc, *d;
} orc_blk;

/* The four fields of super-block b of a row.
 * RAW / PAD224: ql at +0 (128 B), qh at +128 (64 B), sc at +192 (16 B), d at +208
 *   (2 B, fp16) -- the field split of [D4-4] §3.2 Excerpt A and the intra-block
 *   offsets of [D4-2] §3.2 Excerpt C (d at blk+208, sc at blk+192, qh at blk+128).
 * DPL: the same fields, each taken from its own plane at section bases 0, nbe*128,
 *   nbe*192 and nbe*208 ([D4-4] §3.2 Excerpt B). */
static orc_blk orc_block(int layout, const uint8_t *row, int64_t nbe, int64_t b)
{
    orc_blk r;
    if (layout == ORC_DPL) {
        r.ql = row + b * 128;
        r.qh = row + nbe * 128 + b * 64;
        r.sc = row + nbe * 192 + b * 16;
        r.d = row + nbe * 208 + b * 2;
    } else {
        const uint8_t *base = row + b * (layout == ORC_RAW ? 210 : 224);
        r.ql = base;
        r.qh = base + 128;
        r.sc = base + 192;
        r.d = base + 208;
    }
    return r;
}

/* 6-bit code q in [0, 63] of element e (0..255) of a super-block.
 * [D4-4] §3.2 Excerpt B (and [D4-2] §3.2 Excerpt C): the 32-element unit
 * ("is-pair") p = e / 32 has chunk = p >> 2 and g = p & 3; its low-bit bytes are the
 * 32 bytes at ql + chunk*64 + (g&1)*32, its high-bit bytes the 32 bytes at
 * qh + chunk*32, and its 2-bit field sits at shift 2g of the qh byte.
 * Readings where the excerpt is elided: element l of the unit is byte l of both
 * windows; units with g < 2 take the low nibble of the ql byte and units with
 * g >= 2 the high nibble (g and g+2 share the bytes, so they must use different
 * nibbles, low first); q = low4 | high2 << 4. */
static int orc_q(orc_blk b, int e)
{
    int p = e >> 5, l = e & 31;
    int chunk = p >> 2, g = p & 3;
    int qlb = b.ql[chunk * 64 + (g & 1) * 32 + l];
    int low4 = (g < 2) ? (qlb & 0x0F) : (qlb >> 4);
    int high2 = (b.qh[chunk * 32 + l] >> (2 * g)) & 3;
    return low4 | (high2 << 4);
}

/* int8 scale of element e: sub-block j = e / 16, i.e. sc[2*pair] for the first 16
 * elements of a unit and sc[2*pair+1] for the last 16 ([D4-4] §3.2 Excerpt B). */
static int orc_sc(orc_blk b, int e) { return (int8_t)b.sc[e >> 4]; }

/* fp16 super-block scale, little-endian. */
static uint16_t orc_d16(orc_blk b) { return (uint16_t)(b.d[0] | (b.d[1] << 8)); }

/* Decode every element: q codes [N][K], sub-block scales [N][K/16], super-block
 * scale bits [N][K/256]. Any output may be NULL. */
int orc_decode(int layout, const uint8_t *W, int64_t N, int64_t K,
               uint8_t *q, int8_t *sc, uint16_t *d16)
{
    int64_t stride = orc_row_stride(layout, K);
    if (stride < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++) {
        const uint8_t *row = W + r * stride;
        for (int64_t b = 0; b < nbe; b++) {
            orc_blk blk = orc_block(layout, row, nbe, b);
            for (int e = 0; e < 256; e++) {
                if (q)
                    q[r * K + b * 256 + e] = (uint8_t)orc_q(blk, e);
                if (sc && (e & 15) == 0)
                    sc[r * (K / 16) + b * 16 + (e >> 4)] = (int8_t)orc_sc(blk, e);
            }
            if (d16)
                d16[r * nbe + b] = orc_d16(blk);
        }
    }
    return ORC_OK;
}

/* Dequantized weights w = f16(d) * sc * (q - 32) in fp64 (exact), [N][K]. */
int orc_dequant(int layout, const uint8_t *W, int64_t N, int64_t K, double *w)
{
    int64_t stride = orc_row_stride(layout, K);
    if (stride < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++)
        for (int64_t b = 0; b < nbe; b++) {
            orc_blk blk = orc_block(layout, W + r * stride, nbe, b);
            double d = orc_f16_to_f64(orc_d16(blk));
            for (int e = 0; e < 256; e++)
                w[r * K + b * 256 + e] = d * (double)orc_sc(blk, e) * (double)(orc_q(blk, e) - 32);
        }
    return ORC_OK;
}

/* raw -> dpl: for row r and block b, ql <- blk[0..128), qh <- blk[128..192),
 * sc <- blk[192..208), d <- blk[208..210); the row tail after nbe*210 content bytes
 * is zero ([D4-4] §3.2 Excerpt A: the plane starts zero-filled). */
int orc_repack_dpl(const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K)
{
    int64_t rs = orc_row_stride(ORC_RAW, K), ds = orc_row_stride(ORC_DPL, K);
    if (rs < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    memset(dpl, 0, (size_t)(N * ds));
    for (int64_t r = 0; r < N; r++) {
        const uint8_t *src = raw + r * rs;
        uint8_t *dst = dpl + r * ds;
        for (int64_t b = 0; b < nbe; b++) {
            const uint8_t *blk = src + b * 210;
            memcpy(dst + b * 128, blk, 128);
            memcpy(dst + nbe * 128 + b * 64, blk + 128, 64);
            memcpy(dst + nbe * 192 + b * 16, blk + 192, 16);
            memcpy(dst + nbe * 208 + b * 2, blk + 208, 2);
        }
    }
    return ORC_OK;
}

/* dpl -> raw, the inverse byte permutation (tail pad bytes are dropped). */
int orc_unpack_dpl(const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K)
{
    int64_t rs = orc_row_stride(ORC_RAW, K), ds = orc_row_stride(ORC_DPL, K);
    if (rs < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++) {
        const uint8_t *src = dpl + r * ds;
        uint8_t *dst = raw + r * rs;
        for (int64_t b = 0; b < nbe; b++) {
            uint8_t *blk = dst + b * 210;
            memcpy(blk, src + b * 128, 128);
            memcpy(blk + 128, src + nbe * 128 + b * 64, 64);
            memcpy(blk + 192, src + nbe * 192 + b * 16, 16);
            memcpy(blk + 208, src + nbe * 208 + b * 2, 2);
        }
    }
    return ORC_OK;
}

/* raw -> padded 224 B stride (14 zero bytes after each block), the layout dpl
 * replaces ([D4-4] §2 "The padded layout's true cost on DRAM"). */
int orc_pad224(const uint8_t *raw, uint8_t *pad, int64_t N, int64_t K)
{
    if (orc_row_stride(ORC_RAW, K) < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nblk = N * (K / 256);
    for (int64_t i = 0; i < nblk; i++) {
        memcpy(pad + i * 224, raw + i * 210, 210);
        memset(pad + i * 224 + 210, 0, 14);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Activation producers                                                            */
/* ------------------------------------------------------------------------------ */

/* q8 quantization of nt rows of K floats in blocks of 32 ([D3-5] §3.2, the per-32-
 * block body shared by the standalone and the fused producers):
 *   amax = max |x| over the block (exact under any order);
 *   d    = amax / 127            (f32 division);
 *   di   = d != 0 ? 1 / d : 0    (f32 division);
 *   q    = clamp(rint(x * di), -128, 127) with the product rounded to f32 and rint
 *          rounding ties to even;
 *   the stored scale is f16(d), rounded to nearest even.
 * Note the quantizer uses the unrounded f32 di while a consumer uses the f16 d.
 * Outputs: qs [nt][K] int8, d16 [nt][K/32] fp16 bits. Inputs must be finite. */
int orc_quant_q8(const float *x, int64_t K, int nt, int8_t *qs, uint16_t *d16)
{
    if (K <= 0 || K % 32 || nt < 1)
        return ORC_E_SHAPE;
    int64_t nblk = (int64_t)nt * (K / 32);
    for (int64_t blk = 0; blk < nblk; blk++) {
        const float *xb = x + blk * 32;
        float amax = 0.0f;
        for (int i = 0; i < 32; i++) {
            if (!isfinite(xb[i]))
                return ORC_E_VALUE;
            amax = fmaxf(amax, fabsf(xb[i]));
        }
        float d = amax / 127.0f;
        float di = (d != 0.0f) ? 1.0f / d : 0.0f;
        for (int i = 0; i < 32; i++) {
            float p = xb[i] * di;
            float r = rintf(p);
            int q = (int)r;
            if (q < -128) q = -128;
            if (q > 127) q = 127;
            qs[blk * 32 + i] = (int8_t)q;
        }
        d16[blk] = orc_f32_to_f16(d);
    }
    return ORC_OK;
}

/* RMSNorm of nt rows of K floats. The pages fuse an RMSNorm in front of the
 * quantizer ([D3-5] §3.2, the fused rms epilogue) but do not print its body.
 * Reading: y = (x * r) * gamma with r = 1 / sqrt(mean(x^2) + eps); the mean is
 * summed in fp64 (each x^2 is exact in fp64), r is rounded once to f32, and both
 * products are f32 products, each rounded. The order of the fp64 sum is not fixed
 * by the pages, so only the value of y (not its last bit) is pinned. */
int orc_rmsnorm(const float *x, const float *gamma, float eps, int64_t K, int nt, float *y)
{
    if (K <= 0 || nt < 1)
        return ORC_E_SHAPE;
    for (int t = 0; t < nt; t++) {
        const float *xr = x + (int64_t)t * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; k++)
            ss += (double)xr[k] * (double)xr[k];
        double ms = ss / (double)K;
        float r = (float)(1.0 / sqrt(ms + (double)eps));
        for (int64_t k = 0; k < K; k++) {
            float xn = xr[k] * r;
            y[(int64_t)t * K + k] = xn * gamma[k];
        }
    }
    return ORC_OK;
}

/* SwiGLU of nt rows of K gate/up pairs: y = silu(g) * u = g / (1 + e^-g) * u
 * ([D3-5] §3.2, the fused swiglu producer's body), evaluated in fp64 (libm exp) and
 * rounded to f32 once at the end; the fp64 evaluation's own error (a few 2^-53
 * relative) can move the f32 result by one ulp where the value lies near a rounding
 * boundary. */
int orc_swiglu(const float *g, const float *u, int64_t K, int nt, float *y)
{
    if (K <= 0 || nt < 1)
        return ORC_E_SHAPE;
    for (int64_t i = 0; i < (int64_t)nt * K; i++) {
        const double gd = (double)g[i];
        y[i] = (float)(gd / (1.0 + exp(-gd)) * (double)u[i]);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* The GEMV                                                                        */
/* ------------------------------------------------------------------------------ */

/* Sub-block dots D[t][r][j] = sum over the 16 elements k of sub-block j of
 * (q_rk - 32) * x8_tk, exact in int32 (|D| <= 16*32*128).
 * The unit of work on the pages is the 32-element pair whose two 16-element halves
 * carry their own scales sc0/sc1 and give dot0/dot1 ([D4-2] §3.2 Excerpt C, the
 * per-unit accumulation); the half-unit dot is the sub-block dot here. The element
 * of row position 32u + l meets q8 block u, byte l ([D4-4] §3.2 Excerpt B: the
 * activation block of unit u). */
int orc_subdots(int layout, const uint8_t *W, int64_t N, int64_t K, int nt,
                const int8_t *qs, int32_t *dots)
{
    int64_t stride = orc_row_stride(layout, K);
    if (stride < 0 || N < 0 || nt < 1)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256, nsub = K / 16;
    for (int t = 0; t < nt; t++)
        for (int64_t r = 0; r < N; r++)
            for (int64_t b = 0; b < nbe; b++) {
                orc_blk blk = orc_block(layout, W + r * stride, nbe, b);
                for (int j = 0; j < 16; j++) {
                    int32_t D = 0;
                    for (int i = 0; i < 16; i++) {
                        int e = 16 * j + i;
                        D += (orc_q(blk, e) - 32) * (int32_t)qs[(int64_t)t * K + b * 256 + e];
                    }
                    dots[((int64_t)t * N + r) * nsub + b * 16 + j] = D;
                }
            }
    return ORC_OK;
}

/* The MMVQ in fp64: y[t][r] = sum over super-blocks b (ascending) and sub-blocks j
 * (ascending) of  T = f16(d_rb) * sc_rbj * f16(d8_t,8b+j/2) * D_trbj,
 * each T exact in fp64 (11 + 11 + 8 + 17 significant bits), the running sum
 * rounded per term. A[t][r] = sum |T| is the error-bound denominator. The per-unit
 * form on the pages is acc += d8*sc0*d*dot0 + d8*sc1*d*dot1 ([D4-2] §3.2 Excerpt C);
 * output row r of token t is y[t*N + r] (the reduce writes output[t*od + row]).
 * Rows are independent; nthreads > 1 splits rows over OpenMP threads without
 * changing any result. */
int orc_mmvq(int layout, const uint8_t *W, int64_t N, int64_t K, int nt,
             const int8_t *qs, const uint16_t *d8, double *y, double *A, int nthreads)
{
    int64_t stride = orc_row_stride(layout, K);
    if (stride < 0 || N < 0 || nt < 1)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t r = 0; r < N; r++) {
        for (int t = 0; t < nt; t++) {
            const int8_t *xq = qs + (int64_t)t * K;
            const uint16_t *xd = d8 + (int64_t)t * (K / 32);
            double acc = 0.0, aabs = 0.0;
            for (int64_t b = 0; b < nbe; b++) {
                orc_blk blk = orc_block(layout, W + r * stride, nbe, b);
                double d = orc_f16_to_f64(orc_d16(blk));
                for (int j = 0; j < 16; j++) {
                    int32_t D = 0;
                    for (int i = 0; i < 16; i++) {
                        int e = 16 * j + i;
                        D += (orc_q(blk, e) - 32) * (int32_t)xq[b * 256 + e];
                    }
                    double T = d * (double)orc_sc(blk, 16 * j) *
                               orc_f16_to_f64(xd[b * 8 + j / 2]) * (double)D;
                    acc += T;
                    aabs += fabs(T);
                }
            }
            y[(int64_t)t * N + r] = acc;
            if (A)
                A[(int64_t)t * N + r] = aabs;
        }
    }
    return ORC_OK;
}

/* Integer value of a finite fp16 times 2^24 (every finite fp16 is a multiple of
 * 2^-24); sets *ok = 0 for inf / NaN. */
static int64_t orc_f16_scaled(uint16_t h, int *ok)
{
    int e = (h >> 10) & 31, m = h & 1023;
    int64_t v;
    if (e == 31) {
        *ok = 0;
        return 0;
    }
    v = (e == 0) ? m : ((int64_t)(1024 + m) << (e - 1));
    return (h & 0x8000) ? -v : v;
}

/* The same sum computed exactly: every T is an integer multiple of 2^-48, so the
 * sum is accumulated as a 128-bit integer count of 2^-48 and rounded once to fp64.
 * |T * 2^48| <= 2^40 * 2^40 * 2^7 * 2^16 = 2^103, so 2^20 terms cannot overflow. */
int orc_mmvq_exact(int layout, const uint8_t *W, int64_t N, int64_t K, int nt,
                   const int8_t *qs, const uint16_t *d8, double *y)
{
    int64_t stride = orc_row_stride(layout, K);
    if (stride < 0 || N < 0 || nt < 1)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++)
        for (int t = 0; t < nt; t++) {
            __int128 acc = 0;
            int ok = 1;
            for (int64_t b = 0; b < nbe; b++) {
                orc_blk blk = orc_block(layout, W + r * stride, nbe, b);
                int64_t d = orc_f16_scaled(orc_d16(blk), &ok);
                for (int j = 0; j < 16; j++) {
                    int64_t D = 0;
                    for (int i = 0; i < 16; i++) {
                        int e = 16 * j + i;
                        D += (int64_t)(orc_q(blk, e) - 32) * qs[(int64_t)t * K + b * 256 + e];
                    }
                    int64_t dx = orc_f16_scaled(d8[(int64_t)t * (K / 32) + b * 8 + j / 2], &ok);
                    acc += (__int128)d * dx * (__int128)(orc_sc(blk, 16 * j) * D);
                }
            }
            if (!ok)
                return ORC_E_VALUE;
            y[(int64_t)t * N + r] = ldexp((double)acc, -48);
        }
    return ORC_OK;
}
