/*
 * q6kdpl.h -- C ABI of libq6kdpl.so: the q6_K x q8 batch-1 decode GEMV (MMVQ) over
 * the dense split-plane ("dpl") row layout, its sibling q4_K and q5_K classes over
 * the same kind of row, and the q8 activation producers, for AMD MI355X (gfx950).
 *
 * Sources (page titles; sections cited at each entry point):
 *   [D4-4] "76 · D4-4 -- the endgame kernel session: dpl dense split-plane q6_K
 *           decode MMVQ lands (bitwise)"
 *   [D4-2] "74 · D4-2 -- B0 latent correctness fix + all bitwise occupancy/prefetch
 *           axes closed"
 *   [D3-5] "70 · D3-5 -- decode-alignment plan Stage 1: fused-producer decode
 *           A-quantize"
 *
 * Conventions for every entry point:
 *  - Return 0 (Q6K_OK) on success, a negative Q6K_E_* code on failure. Every
 *    argument is validated before any device work is queued; on an error nothing
 *    is launched and no output byte is written. Text: q6k_strerror(code).
 *  - Device entry points take device pointers (hipMalloc'd memory, e.g. a torch
 *    tensor's data_ptr()) and `stream`, a hipStream_t passed as void* (NULL means
 *    the null stream of the current device). They only queue work on `stream`
 *    and return without synchronising; results are visible after the stream is
 *    synchronised. Host entry points take host pointers and run synchronously.
 *  - The caller owns every buffer. The library allocates no memory, keeps no data
 *    of any call and reads no environment; calls are reentrant. Calls that share
 *    an output buffer must be ordered by the caller.
 *  - Process-wide state: two tables, filled on first use and kept until the
 *    process ends, both about the hardware and the kernels, never about a call's
 *    data: the compute-unit count of each device (lock-free), and, per device,
 *    kernel and dynamic LDS size, how many 256-thread workgroups of that kernel fit
 *    on one compute unit (from hipOccupancyMaxActiveBlocksPerMultiprocessor, behind
 *    a mutex; a kernel that needs more than 64 KB of LDS is first allowed it with
 *    hipFuncSetAttribute). The grid of a launch is sized from them.
 *  - Sizes: K is the row length (number of weights per row), N the number of
 *    rows, nt the number of activation rows ("tokens"). Shape limits:
 *    1 <= N <= Q6K_MAX_N, 1 <= nt <= Q6K_MAX_NT, 0 < K <= Q6K_MAX_K, and K a
 *    multiple of 256 for weights (K a multiple of 32 for the producers).
 *    Anything else is Q6K_E_SHAPE -- there is no silent fallback and no clipping.
 *
 * Data layouts (all little-endian):
 *  raw q6_K row: K/256 super-blocks of 210 B: ql[128] (low 4 bits), qh[64] (high
 *    2 bits), sc[16] (int8 scale per 16 weights), d (fp16 scale) at bytes 208..209
 *    ([D4-4] §3.2 Excerpt A). Code q = low4 | high2 << 4 in 0..63, weight value
 *    d * sc * (q - 32).
 *  dpl row: [ql: nbe*128][qh: nbe*64][sc: nbe*16][d: nbe*2][zero pad], nbe = K/256,
 *    row stride (nbe*210 + 15) & ~15 bytes; rows back to back ([D4-4] §2 "The dpl
 *    split-plane's layout ledger", §3.2 Excerpts A and B).
 *  q8 plane for nt rows of K activations: [qs: int8 nt*K][d8: fp16 nt*(K/32)],
 *    t-major in both sections: qs[t*K + k], d8[t*(K/32) + k/32]. Block b of 32
 *    activations of row t is represented by qs * f16(d8) ([D3-5] §3.2). Both
 *    sections start 16-B aligned when the plane does. Size q8_plane_bytes(K, nt).
 *  y: float32 [nt][N], y[t*N + r] (the reduction writes output[t*od + row],
 *    [D4-2] §3.2 Excerpt B).
 *  q4_K / q5_K (the kq_* entry points; the pages name these classes but print no
 *    layout, so the blocks are the public GGUF definitions): raw super-blocks of
 *    144 B (q4_K: fp16 d, fp16 dmin, 12 bytes packing eight 6-bit scales and eight
 *    6-bit mins, 128 bytes of 4-bit codes) or 176 B (q5_K: the same with 32 bytes of
 *    fifth code bits before the codes); weight value d*sc*q - dmin*m per 32-element
 *    sub-block. Split-plane row: [codes nbe*128]([fifth bits nbe*32])[scales
 *    nbe*12][(d, dmin) nbe*4], stride nbe*144 or nbe*176 (already multiples of 16).
 */
#ifndef Q6KDPL_H
#define Q6KDPL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q6K_OK 0
#define Q6K_E_SHAPE (-1) /* N, K or nt out of range, or K not a multiple of 256/32     */
#define Q6K_E_NULL (-2)  /* a required pointer is NULL                                  */
#define Q6K_E_ALIGN (-3) /* a pointer is not 16-byte aligned                            */
#define Q6K_E_ALIAS (-4) /* an output byte range overlaps an input byte range           */
#define Q6K_E_HIP (-5)   /* the HIP runtime refused a launch or a device query          */
#define Q6K_E_TYPE (-6)  /* unknown weight type                                         */

/* Weight types of the kq_* entry points (GGUF type ids). */
#define KQ_Q4_K 12
#define KQ_Q5_K 13
#define KQ_Q6_K 14

#define Q6K_MAX_N ((int64_t)1 << 30)
#define Q6K_MAX_K ((int64_t)1 << 20)
#define Q6K_MAX_NT 256

/* Text for a return code (static storage; never NULL). */
const char *q6k_strerror(int code);

/* Library version, e.g. "q6kdpl 0.1 gfx950". */
const char *q6k_version(void);

/* dpl row stride in bytes, ((K/256)*210 + 15) & ~15 ([D4-4] §2: nbe 54 -> 11344).
 * Returns 0 when K is not a positive multiple of 256 (or above Q6K_MAX_K). */
size_t q6k_dpl_row_stride(int64_t K);

/* Bytes of a dpl matrix: N * q6k_dpl_row_stride(K); 0 on a bad shape. */
size_t q6k_dpl_bytes(int64_t N, int64_t K);

/* Bytes of a raw q6_K matrix: N * (K/256) * 210; 0 on a bad shape. */
size_t q6k_raw_bytes(int64_t N, int64_t K);

/* Bytes of a q8 plane: nt*K + nt*(K/32)*2; 0 when K is not a positive multiple of
 * 32 or nt is out of range. */
size_t q8_plane_bytes(int64_t K, int nt);

/* Host repack raw -> dpl ([D4-4] §3.2 Excerpt A: per row and block, ql, qh, sc, d
 * are copied into their planes; the row tail after nbe*210 bytes is zeroed).
 * raw: q6k_raw_bytes(N, K) host bytes; dpl: q6k_dpl_bytes(N, K) host bytes, every
 * byte written. The ranges must not overlap (Q6K_E_ALIAS). No alignment needed. */
int repack_q6k_dpl_host(const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K);

/* Host inverse of repack_q6k_dpl_host (dpl -> raw; pad bytes are ignored). */
int unpack_q6k_dpl_host(const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K);

/* Device repack raw -> dpl, byte-identical to repack_q6k_dpl_host. raw_dev needs
 * no alignment; dpl_dev must be 16-byte aligned. Every byte of dpl_dev
 * (q6k_dpl_bytes(N, K)) is written, pad bytes with zero. */
int repack_q6k_dpl(const void *raw_dev, void *dpl_dev, int64_t N, int64_t K, void *stream);

/* Standalone q8 producer ([D3-5] §3.2, the per-32-block body): for each block of
 * 32 floats, amax = max|x|, d = amax/127 (f32), di = d != 0 ? 1/d : 0 (f32),
 * q = clamp(rint(x*di), -128, 127) with ties to even; stores qs and f16(d).
 * x: float32 [nt][K] device, 16-B aligned, finite values. q8: q8_plane_bytes(K, nt)
 * device bytes, 16-B aligned. K must be a multiple of 32. */
int quant_q8(const float *x, void *q8, int64_t K, int nt, void *stream);

/* Fused producer: RMSNorm then q8 ([D3-5] §3.2, the fused rms epilogue):
 * r = 1/sqrt(mean(x^2) + eps) with the mean summed in fp64 and r rounded once to
 * f32, y = (x*r)*gamma in f32, then the q8 body of quant_q8 applied to y.
 * x: float32 [nt][K]; gamma: float32 [K]; y: float32 [nt][K] (written); q8: as for
 * quant_q8. All device, 16-B aligned; y and q8 may not overlap x, gamma or each
 * other. The q8 bytes equal quant_q8 applied to the y this call writes. */
int rmsnorm_quant_q8(const float *x, const float *gamma, float eps, float *y, void *q8,
                     int64_t K, int nt, void *stream);

/* Fused SwiGLU producer ([D3-5] §3.2, the fused swiglu producer): y = (g / (1 + e^-g))
 * * u in f32 (IEEE division, the device library's expf), then the q8 body of quant_q8
 * applied to y. g, u: float32 [nt][K] (e.g. the gate and up halves of one buffer);
 * y: float32 [nt][K] (written; y may be exactly g or exactly u, i.e. in place, but
 * may not otherwise overlap them); q8: as for quant_q8, overlapping none of g, u, y.
 * All device, 16-B aligned, finite inputs; K a multiple of 32. */
int swiglu_quant_q8(const float *g, const float *u, float *y, void *q8, int64_t K, int nt,
                    void *stream);

/* The MMVQ: y[t][r] = sum over super-blocks b and sub-blocks j of
 * f16(d_rb) * sc_rbj * f16(d8_t,8b+j/2) * D_trbj, with D the exact int32 dot of the
 * 16 codes (q - 32) and the 16 int8 activations of sub-block j ([D4-2] §3.2
 * Excerpt C, the per-unit accumulation; [D4-4] §3.2 Excerpt B, the dpl unit load).
 * Sub-block dots are exact; scaling and summation are f32 (error well inside
 * 1e-5 * sum|terms|). The order of the f32 sums follows the kernel kind that
 * q6k_mmvq_plan reports for the shape and is fixed for it, so a shape's results
 * repeat bit for bit. Every unit of every row is covered for every N, K, nt in
 * range (no shape reaches a kernel that skips work; [D4-2] §2).
 * w_dpl: q6k_dpl_bytes(N, K) device bytes, 16-B aligned; q8: q8_plane_bytes(K, nt)
 * device bytes, 16-B aligned; y: float32 [nt][N] device, 16-B aligned, written. */
int mmvq_q6k_q8(const void *w_dpl, const void *q8, float *y, int64_t N, int64_t K, int nt,
                void *stream);

/* RMSNorm -> q8 -> MMVQ in one call: the outputs of
 *   rmsnorm_quant_q8(x, gamma, eps, xn, q8, K, nt) then mmvq_q6k_q8(w_dpl, q8, y, N, K, nt),
 * bit for bit ([D3-5] §3.2, the fused rms producer and the per-32-block body; [D4-2]
 * §3.2 Excerpt C and [D4-4] §3.2 Excerpt B for the MMVQ). Where
 * q6k_rmsnorm_mmvq_fused(N, K, nt) is 1 (one token, K <= 12288) this is a single
 * kernel: each workgroup normalizes and quantizes the activations itself and the
 * weight stream starts before the norm ends; otherwise the two kernels are queued.
 * w_dpl: q6k_dpl_bytes(N, K) device bytes; x: float32 [nt][K]; gamma: float32 [K];
 * xn: float32 [nt][K] written with the normalized rows, or NULL to skip them; q8:
 * q8_plane_bytes(K, nt) device bytes, written (the q8 plane of xn, reusable by
 * mmvq_q6k_q8 for other weights); y: float32 [nt][N], written. All device, 16-B
 * aligned; no output may overlap an input or another output. K a multiple of 256. */
int mmvq_q6k_rmsnorm_q8(const void *w_dpl, const float *x, const float *gamma, float eps,
                        float *xn, void *q8, float *y, int64_t N, int64_t K, int nt,
                        void *stream);

/* Diagnostics: 1 when mmvq_q6k_rmsnorm_q8 runs (N, K, nt) as one fused kernel, 0
 * when it queues the producer and the MMVQ, Q6K_E_SHAPE on a bad shape. Host only. */
int q6k_rmsnorm_mmvq_fused(int64_t N, int64_t K, int nt);

/* Test entry: the exact sub-block dots D of mmvq_q6k_q8, dots[(t*N + r)*(K/16) + j]
 * (int32, device, 16-B aligned, nt*N*(K/16) entries). Same inputs as mmvq_q6k_q8. */
int mmvq_q6k_q8_subdots(const void *w_dpl, const void *q8, int32_t *dots, int64_t N, int64_t K,
                        int nt, void *stream);

/* ---- q4_K / q5_K (and q6_K) by weight type ------------------------------------- */
/* Every kq_* entry takes `type` (KQ_Q4_K, KQ_Q5_K or KQ_Q6_K; anything else is
 * Q6K_E_TYPE) and otherwise behaves as its q6_K counterpart above, which it equals
 * for KQ_Q6_K. The q4_K and q5_K classes are the siblings of the q6_K one on the
 * same decode step ([D4-2] §1 and §2: the q4_K class's stream rate is the bar the
 * q6_K work is measured against; [D3-5] §3.2: the three MMVQ entries q4_K/q5_K/q6_K
 * take the same q8 activation plane). */

/* Bytes of one super-block of 256 weights (144, 176, 210); 0 for an unknown type. */
size_t kq_block_bytes(int type);

/* Split-plane row stride, (K/256 * block bytes + 15) & ~15; 0 on a bad type or K. */
size_t kq_dpl_row_stride(int type, int64_t K);

/* Bytes of a split-plane matrix (N * stride) / of a raw matrix (N * K/256 * block
 * bytes); 0 on a bad type or shape. */
size_t kq_dpl_bytes(int type, int64_t N, int64_t K);
size_t kq_raw_bytes(int type, int64_t N, int64_t K);

/* Host repack raw -> split-plane rows (each block field copied to its plane, the
 * row tail zeroed) and its inverse; as repack_q6k_dpl_host / unpack_q6k_dpl_host. */
int repack_kq_dpl_host(int type, const uint8_t *raw, uint8_t *dpl, int64_t N, int64_t K);
int unpack_kq_dpl_host(int type, const uint8_t *dpl, uint8_t *raw, int64_t N, int64_t K);

/* Device repack, byte-identical to repack_kq_dpl_host; as repack_q6k_dpl. */
int repack_kq_dpl(int type, const void *raw_dev, void *dpl_dev, int64_t N, int64_t K,
                  void *stream);

/* The MMVQ over split-plane rows of `type` with the q8 plane of quant_q8 (and the
 * other producers). q4_K / q5_K: y[t][r] = sum over super-blocks b and 32-element
 * sub-blocks s of f16(d8_t,8b+s) * (f16(d_rb) * sc_rbs * Dq - f16(dmin_rb) * m_rbs * Sx),
 * Dq the exact int32 dot of the sub-block's codes with its int8 activations and Sx
 * the activations' sum; scaling and summation in f32 (error well inside
 * 1e-5 * sum|terms|, terms counted as the scale and min products). Arguments,
 * alignment, coverage and errors as mmvq_q6k_q8, with w_dpl of kq_dpl_bytes(type,
 * N, K) bytes. */
int mmvq_kq_q8(int type, const void *w_dpl, const void *q8, float *y, int64_t N, int64_t K,
               int nt, void *stream);

/* RMSNorm -> q8 -> MMVQ for `type`, as mmvq_q6k_rmsnorm_q8 (one kernel where
 * q6k_rmsnorm_mmvq_fused(N, K, nt) is 1, for every type). */
int mmvq_kq_rmsnorm_q8(int type, const void *w_dpl, const float *x, const float *gamma,
                       float eps, float *xn, void *q8, float *y, int64_t N, int64_t K, int nt,
                       void *stream);

/* Form B: gate+up GEMV, SwiGLU and q8 of one token ([D4-4] §3.5, the archived fused
 * gate+up+SwiGLU+q8 shape, and §5, its closing numbers; [D3-5] §3.2, the SwiGLU
 * producer's body). w_gu holds 2*Nh split-plane rows of `type`: the Nh gate rows,
 * then the Nh up rows. With x the q8 activation row q8_in (K activations):
 *   gu = W x (float32 [2*Nh], as mmvq_kq_q8 writes it),
 *   y = (g / (1 + e^-g)) * u for g = gu[0:Nh], u = gu[Nh:2Nh] (float32 [Nh], written
 *       when y is not NULL), and q8_out = its q8 plane (q8_plane_bytes(Nh, 1) bytes),
 * bit for bit as mmvq_kq_q8 followed by swiglu_quant_q8. Where
 * kq_gate_up_swiglu_fused(Nh, K) is 1 (K <= 12288) this is one kernel, each
 * workgroup taking the 64 rows behind whole 32-output q8 blocks; otherwise the two
 * kernels are queued. nt must be 1 and Nh a multiple of 32 (Q6K_E_SHAPE otherwise).
 * All device, 16-B aligned; no output may overlap an input or another output. */
int mmvq_kq_gate_up_swiglu_q8(int type, const void *w_gu, const void *q8_in, float *gu, float *y,
                              void *q8_out, int64_t Nh, int64_t K, int nt, void *stream);

/* Diagnostics: 1 when mmvq_kq_gate_up_swiglu_q8 runs (Nh, K) as one kernel, 0 when it
 * queues the GEMV and the SwiGLU producer, Q6K_E_SHAPE on a bad shape. Host only. */
int kq_gate_up_swiglu_fused(int64_t Nh, int64_t K);

/* Test entry: the exact integer dots of mmvq_kq_q8. KQ_Q6_K: as mmvq_q6k_q8_subdots
 * (K/16 per row). KQ_Q4_K / KQ_Q5_K: Dq per 32-element sub-block,
 * dots[(t*N + r)*(K/32) + s] (int32, device, 16-B aligned). */
int mmvq_kq_q8_subdots(int type, const void *w_dpl, const void *q8, int32_t *dots, int64_t N,
                       int64_t K, int nt, void *stream);

/* Diagnostics: how mmvq_q6k_q8 runs a shape on a device with num_cu compute units.
 * out6[0] = workgroups per launch (256 threads each; a launch uses fewer where the
 *   kernel's registers fit fewer workgroups per CU);
 * out6[1] = low-bit chunks per lane per row (per thread of the workgroup when
 *   out6[2] is 2);
 * out6[2] = the kernel kind:
 *   0 the generic stepping kernel;
 *   1 a fixed-length kernel, one wave per row;
 *   2 a fixed-length kernel whose workgroup's four waves share each row (long rows
 *     that are few for the grid, or at several tokens); each output adds the four
 *     waves' shares in a fixed order;
 *   3 a fixed-length kernel with two rows per wave (2..4 tokens, K = 1024, 3072 or
 *     5120, whose rows hold an odd multiple of 32 chunks, and at least 4 rows per wave
 *     of its grid); each half of the wave takes one row's last chunk slot;
 *   4 16-row tiles on the int8 matrix cores (q6_K, K = 5120, 4 tokens with at least 12
 *     tiles of 16 rows per CU, 3 tokens with at least 24):
 *     a workgroup's four waves copy 16 consecutive rows into LDS and each takes a
 *     quarter of K; each output adds the four quarters in a fixed order;
 * out6[3] = where activation operands live across rows (0: re-read from the q8
 *   plane per row, 1: registers, 2: staged once per workgroup in LDS);
 * out6[4] = launches (one per group of up to 4 token columns);
 * out6[5] = rows (kind 3: row pairs) in flight per wave; kind 4: tile buffers per
 *   workgroup.
 * The kernel fields describe the first launch. Host only. */
int q6k_mmvq_plan(int64_t N, int64_t K, int nt, int num_cu, int32_t *out6);

/* The same for mmvq_kq_q8 with weight type `type` (Q6K_E_TYPE for an unknown one);
 * the shape choices depend on the type. */
int kq_mmvq_plan(int type, int64_t N, int64_t K, int nt, int num_cu, int32_t *out6);

#ifdef __cplusplus
}
#endif

#endif /* Q6KDPL_H */
