/*
 * kq_oracle.c -- the oracle for the q4_K and q5_K x q8 decode GEMV, the two sibling
 * k-quant classes of the q6_K path.
 *
 * TEST INFRASTRUCTURE, like q6k_oracle.c: only tests/, __graft_entry__.smoke() and
 * the cpu_baseline leg of bench.py may load the library built from this file. The
 * HIP library never calls it, and the two share no code, header, table or helper.
 *
 * The pages name these classes -- the q4_K decode class whose stream rate the q6_K
 * work is measured against ("74 · D4-2", §1 and §2; "76 · D4-4", §1), the
 * group-split control rearranged "q4_K-style" into 16-B groups ("76 · D4-4",
 * §3.1), and the three MMVQ entries q4_K/q5_K/q6_K that consult the producer's
 * q8 cache ("70 · D3-5", §3.2) -- but print neither block layout. The layouts below
 * are the public GGUF definitions of the two types, restated from the format's
 * description (no third-party code is used):
 *
 *   q4_K super-block, 144 B per 256 weights:
 *     bytes 0..1   d     (fp16, the scale of the sub-block scales)
 *     bytes 2..3   dmin  (fp16, the scale of the sub-block mins)
 *     bytes 4..15  12 bytes packing eight 6-bit scales sc[s] and eight 6-bit mins
 *                  m[s], one per 32-element sub-block s = e / 32
 *     bytes 16..143  128 bytes of 4-bit codes
 *   q5_K super-block, 176 B: bytes 0..15 as q4_K, bytes 16..47 32 bytes of fifth
 *     code bits, bytes 48..175 the 128 bytes of 4-bit codes.
 *
 *   Element e = 64*j + 32*h + l (j < 4, h < 2, l < 32) takes the low (h = 0) or high
 *   (h = 1) nibble of code byte 32*j + l; in q5_K bit 2*j + h of fifth-bit byte l is
 *   its bit 4. So sub-block s = 2*j + h takes nibble h of code bytes 32*j .. 32*j+31
 *   and bit s of the 32 fifth-bit bytes.
 *   Scale packing, bytes p[0..11]: for s < 4, sc = p[s] & 63 and m = p[s+4] & 63;
 *   for s >= 4, sc = (p[s+4] & 15) | (p[s-4] >> 6) << 4 and
 *   m = (p[s+4] >> 4) | (p[s] >> 6) << 4.
 *   Weight value: f16(d) * sc * q - f16(dmin) * m, q in 0..15 (q4_K) or 0..31 (q5_K).
 *
 * The split-plane ("dpl-style") row used by the GEMV keeps each field in its own
 * plane, like the q6_K dpl row ("76 · D4-4", §2 and §3.2 Excerpts A and B):
 *   q4_K: [codes nbe*128][scales nbe*12][d,dmin pairs nbe*4], stride nbe*144;
 *   q5_K: [codes nbe*128][fifth bits nbe*32][scales nbe*12][d,dmin pairs nbe*4],
 *         stride nbe*176.
 * Both block sizes are multiples of 16, so no row pad is needed; the stride formula
 * still rounds up to 16 like the q6_K one.
 *
 * The GEMV against a q8 activation row (the same q8 plane as the q6_K path): per
 * 32-element sub-block s of super-block b, with q8 block 8b + s,
 *   T = f16(d) * sc * f16(d8) * Dq  -  f16(dmin) * m * f16(d8) * Sx,
 * Dq = sum of q * x8 and Sx = sum of x8 over the sub-block (exact integers). Each
 * product is exact in fp64 (at most 11 + 6 + 11 + 17 significant bits).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_SHAPE (-1)
#define ORC_E_VALUE (-2)

#define ORC_RAW 0
#define ORC_DPL 2

/* GGUF type ids. */
#define ORC_Q4_K 12
#define ORC_Q5_K 13

double orc_f16_to_f64(uint16_t h); /* q6k_oracle.c */

/* Bytes of one super-block; 0 for an unknown type. */
int64_t orc_kq_block_bytes(int type)
{
    return type == ORC_Q4_K ? 144 : (type == ORC_Q5_K ? 176 : 0);
}

/* Bytes per row of K weights: nbe * block bytes, rounded up to 16 for the
 * split-plane row (a no-op for these block sizes). */
int64_t orc_kq_row_stride(int type, int layout, int64_t K)
{
    int64_t B = orc_kq_block_bytes(type);
    if (B == 0 || K <= 0 || K % 256 || (layout != ORC_RAW && layout != ORC_DPL))
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    return layout == ORC_RAW ? nbe * B : (nbe * B + 15) & ~(int64_t)15;
}

typedef struct {
    const uint8_t *qs;   /* 128 code bytes        */
    const uint8_t *qh;   /* 32 fifth-bit bytes (q5_K only) */
    const uint8_t *sc;   /* 12 packed scale bytes */
    const uint8_t *dm;   /* d then dmin, fp16     */
} orc_kblk;

/* The fields of super-block b of a row, raw (from the block's own offsets) or
 * split-plane (from each field's plane). */
static orc_kblk orc_kblock(int type, int layout, const uint8_t *row, int64_t nbe, int64_t b)
{
    orc_kblk r;
    int q5 = type == ORC_Q5_K;
    if (layout == ORC_DPL) {
        int64_t base_sc = nbe * 128 + (q5 ? nbe * 32 : 0);
        r.qs = row + b * 128;
        r.qh = q5 ? row + nbe * 128 + b * 32 : NULL;
        r.sc = row + base_sc + b * 12;
        r.dm = row + base_sc + nbe * 12 + b * 4;
    } else {
        const uint8_t *blk = row + b * orc_kq_block_bytes(type);
        r.dm = blk;
        r.sc = blk + 4;
        r.qh = q5 ? blk + 16 : NULL;
        r.qs = blk + (q5 ? 48 : 16);
    }
    return r;
}

/* Code of element e (0..255) of a super-block. */
static int orc_kq_code(orc_kblk b, int e)
{
    int j = e >> 6, h = (e >> 5) & 1, l = e & 31;
    int byte = b.qs[32 * j + l];
    int q = h ? (byte >> 4) : (byte & 15);
    if (b.qh)
        q |= ((b.qh[l] >> (2 * j + h)) & 1) << 4;
    return q;
}

/* 6-bit scale and min of sub-block s (0..7). */
static void orc_kq_scale_min(orc_kblk b, int s, int *sc, int *m)
{
    const uint8_t *p = b.sc;
    if (s < 4) {
        *sc = p[s] & 63;
        *m = p[s + 4] & 63;
    } else {
        *sc = (p[s + 4] & 15) | ((p[s - 4] >> 6) << 4);
        *m = (p[s + 4] >> 4) | ((p[s] >> 6) << 4);
    }
}

static uint16_t orc_kq_d16(orc_kblk b) { return (uint16_t)(b.dm[0] | (b.dm[1] << 8)); }
static uint16_t orc_kq_dmin16(orc_kblk b) { return (uint16_t)(b.dm[2] | (b.dm[3] << 8)); }

/* Decode every element: codes [N][K], sub-block scales and mins [N][K/32], d and
 * dmin bits [N][K/256]. Any output may be NULL. */
int orc_kq_decode(int type, int layout, const uint8_t *W, int64_t N, int64_t K, uint8_t *q,
                  uint8_t *sc, uint8_t *m, uint16_t *d16, uint16_t *dmin16)
{
    int64_t stride = orc_kq_row_stride(type, layout, K);
    if (stride < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++)
        for (int64_t b = 0; b < nbe; b++) {
            orc_kblk blk = orc_kblock(type, layout, W + r * stride, nbe, b);
            if (q)
                for (int e = 0; e < 256; e++)
                    q[r * K + b * 256 + e] = (uint8_t)orc_kq_code(blk, e);
            for (int s = 0; s < 8; s++) {
                int a, c;
                orc_kq_scale_min(blk, s, &a, &c);
                if (sc)
                    sc[r * (K / 32) + b * 8 + s] = (uint8_t)a;
                if (m)
                    m[r * (K / 32) + b * 8 + s] = (uint8_t)c;
            }
            if (d16)
                d16[r * nbe + b] = orc_kq_d16(blk);
            if (dmin16)
                dmin16[r * nbe + b] = orc_kq_dmin16(blk);
        }
    return ORC_OK;
}

/* Dequantized weights f16(d) * sc * q - f16(dmin) * m in fp64 (exact), [N][K]. */
int orc_kq_dequant(int type, int layout, const uint8_t *W, int64_t N, int64_t K, double *w)
{
    int64_t stride = orc_kq_row_stride(type, layout, K);
    if (stride < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++)
        for (int64_t b = 0; b < nbe; b++) {
            orc_kblk blk = orc_kblock(type, layout, W + r * stride, nbe, b);
            double d = orc_f16_to_f64(orc_kq_d16(blk));
            double dmin = orc_f16_to_f64(orc_kq_dmin16(blk));
            for (int e = 0; e < 256; e++) {
                int sc, m;
                orc_kq_scale_min(blk, e >> 5, &sc, &m);
                w[r * K + b * 256 + e] = d * sc * orc_kq_code(blk, e) - dmin * m;
            }
        }
    return ORC_OK;
}

/* raw -> split-plane, field by field (the planes of the header comment); the
 * inverse below. */
int orc_kq_repack_dpl(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K)
{
    int64_t rs = orc_kq_row_stride(type, ORC_RAW, K), ds = orc_kq_row_stride(type, ORC_DPL, K);
    if (rs < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    memset(dpl, 0, (size_t)(N * ds));
    for (int64_t r = 0; r < N; r++)
        for (int64_t b = 0; b < nbe; b++) {
            orc_kblk src = orc_kblock(type, ORC_RAW, raw + r * rs, nbe, b);
            orc_kblk dst = orc_kblock(type, ORC_DPL, dpl + r * ds, nbe, b);
            memcpy((uint8_t *)dst.qs, src.qs, 128);
            if (src.qh)
                memcpy((uint8_t *)dst.qh, src.qh, 32);
            memcpy((uint8_t *)dst.sc, src.sc, 12);
            memcpy((uint8_t *)dst.dm, src.dm, 4);
        }
    return ORC_OK;
}

int orc_kq_unpack_dpl(int type, const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K)
{
    int64_t rs = orc_kq_row_stride(type, ORC_RAW, K), ds = orc_kq_row_stride(type, ORC_DPL, K);
    if (rs < 0 || N < 0)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++)
        for (int64_t b = 0; b < nbe; b++) {
            orc_kblk src = orc_kblock(type, ORC_DPL, dpl + r * ds, nbe, b);
            orc_kblk dst = orc_kblock(type, ORC_RAW, raw + r * rs, nbe, b);
            memcpy((uint8_t *)dst.qs, src.qs, 128);
            if (src.qh)
                memcpy((uint8_t *)dst.qh, src.qh, 32);
            memcpy((uint8_t *)dst.sc, src.sc, 12);
            memcpy((uint8_t *)dst.dm, src.dm, 4);
        }
    return ORC_OK;
}

/* Exact code dots Dq[t][r][s] = sum over the 32 elements of sub-block s of
 * q * x8 (int32; |Dq| <= 32 * 31 * 128). */
int orc_kq_subdots(int type, int layout, const uint8_t *W, int64_t N, int64_t K, int nt,
                   const int8_t *qs, int32_t *dots)
{
    int64_t stride = orc_kq_row_stride(type, layout, K);
    if (stride < 0 || N < 0 || nt < 1)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256, nsub = K / 32;
    for (int t = 0; t < nt; t++)
        for (int64_t r = 0; r < N; r++)
            for (int64_t b = 0; b < nbe; b++) {
                orc_kblk blk = orc_kblock(type, layout, W + r * stride, nbe, b);
                for (int s = 0; s < 8; s++) {
                    int32_t D = 0;
                    for (int i = 0; i < 32; i++) {
                        int e = 32 * s + i;
                        D += orc_kq_code(blk, e) * (int32_t)qs[(int64_t)t * K + b * 256 + e];
                    }
                    dots[((int64_t)t * N + r) * nsub + b * 8 + s] = D;
                }
            }
    return ORC_OK;
}

/* The GEMV in fp64: y[t][r] = sum over super-blocks b (ascending) and sub-blocks s
 * (ascending) of T1 - T2 with
 *   T1 = f16(d) * sc * f16(d8) * Dq,  T2 = f16(dmin) * m * f16(d8) * Sx,
 * the q8 block being 8b + s; each term exact in fp64, the running sum rounded per
 * term (T1 added, then T2 subtracted). A[t][r] = sum of |T1| + |T2|. Rows are
 * independent; nthreads > 1 splits rows over OpenMP threads without changing any
 * result. */
int orc_kq_mmvq(int type, int layout, const uint8_t *W, int64_t N, int64_t K, int nt,
                const int8_t *qs, const uint16_t *d8, double *y, double *A, int nthreads)
{
    int64_t stride = orc_kq_row_stride(type, layout, K);
    if (stride < 0 || N < 0 || nt < 1)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t r = 0; r < N; r++)
        for (int t = 0; t < nt; t++) {
            const int8_t *xq = qs + (int64_t)t * K;
            const uint16_t *xd = d8 + (int64_t)t * (K / 32);
            double acc = 0.0, aabs = 0.0;
            for (int64_t b = 0; b < nbe; b++) {
                orc_kblk blk = orc_kblock(type, layout, W + r * stride, nbe, b);
                double d = orc_f16_to_f64(orc_kq_d16(blk));
                double dmin = orc_f16_to_f64(orc_kq_dmin16(blk));
                for (int s = 0; s < 8; s++) {
                    int32_t Dq = 0, Sx = 0;
                    for (int i = 0; i < 32; i++) {
                        int e = 32 * s + i;
                        Dq += orc_kq_code(blk, e) * (int32_t)xq[b * 256 + e];
                        Sx += xq[b * 256 + e];
                    }
                    int sc, m;
                    orc_kq_scale_min(blk, s, &sc, &m);
                    double dx = orc_f16_to_f64(xd[b * 8 + s]);
                    double T1 = d * (double)sc * dx * (double)Dq;
                    double T2 = dmin * (double)m * dx * (double)Sx;
                    acc += T1;
                    acc -= T2;
                    aabs += fabs(T1) + fabs(T2);
                }
            }
            y[(int64_t)t * N + r] = acc;
            if (A)
                A[(int64_t)t * N + r] = aabs;
        }
    return ORC_OK;
}

/* Integer value of a finite fp16 times 2^24; *ok = 0 for inf / NaN. */
static int64_t orc_kq_f16_scaled(uint16_t h, int *ok)
{
    int e = (h >> 10) & 31, mt = h & 1023;
    if (e == 31) {
        *ok = 0;
        return 0;
    }
    int64_t v = (e == 0) ? mt : ((int64_t)(1024 + mt) << (e - 1));
    return (h & 0x8000) ? -v : v;
}

/* The same sum computed exactly as a 128-bit count of 2^-48 (every term is an
 * integer multiple of it), rounded once to fp64. */
int orc_kq_mmvq_exact(int type, int layout, const uint8_t *W, int64_t N, int64_t K, int nt,
                      const int8_t *qs, const uint16_t *d8, double *y)
{
    int64_t stride = orc_kq_row_stride(type, layout, K);
    if (stride < 0 || N < 0 || nt < 1)
        return ORC_E_SHAPE;
    int64_t nbe = K / 256;
    for (int64_t r = 0; r < N; r++)
        for (int t = 0; t < nt; t++) {
            __int128 acc = 0;
            int ok = 1;
            for (int64_t b = 0; b < nbe; b++) {
                orc_kblk blk = orc_kblock(type, layout, W + r * stride, nbe, b);
                int64_t d = orc_kq_f16_scaled(orc_kq_d16(blk), &ok);
                int64_t dmin = orc_kq_f16_scaled(orc_kq_dmin16(blk), &ok);
                for (int s = 0; s < 8; s++) {
                    int64_t Dq = 0, Sx = 0;
                    for (int i = 0; i < 32; i++) {
                        int e = 32 * s + i;
                        Dq += (int64_t)orc_kq_code(blk, e) * qs[(int64_t)t * K + b * 256 + e];
                        Sx += qs[(int64_t)t * K + b * 256 + e];
                    }
                    int sc, m;
                    orc_kq_scale_min(blk, s, &sc, &m);
                    int64_t dx = orc_kq_f16_scaled(d8[(int64_t)t * (K / 32) + b * 8 + s], &ok);
                    acc += (__int128)d * dx * (__int128)(sc * Dq);
                    acc -= (__int128)dmin * dx * (__int128)(m * Sx);
                }
            }
            if (!ok)
                return ORC_E_VALUE;
            y[(int64_t)t * N + r] = ldexp((double)acc, -48);
        }
    return ORC_OK;
}
