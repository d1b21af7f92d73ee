// kq_unit.h -- per-lane work on one 16-byte code chunk of a q4_K / q5_K split-plane
// row (gfx950), and the format policies the GEMV kernels are written against.
//
// Row planes (kq_format.h): [codes nbe*128]([fifth bits nbe*32])[scales nbe*12]
// [d,dmin nbe*4]. The code plane is cut into 16-byte chunks; a wave64 takes 64
// consecutive chunks per instruction, so every code load is one contiguous 1 KB
// request, as in the q6_K GEMV.
//
// Chunk Q = 8*kbx + 2*j + h (kbx the super-block, j its 64-element group, h the
// 16-byte half of the group's 32 code bytes) holds, by the block layout (public
// GGUF definition; element 64j + 32h' + l is nibble h' of code byte 32j + l):
//   - low nibbles: elements 64j + 16h .. +15 of the block, sub-block s = 2j;
//   - high nibbles: elements 64j + 32 + 16h .. +15, sub-block s = 2j + 1;
//   - q5_K fifth bits: the 16 bytes at fifth plane + 32*kbx + 16*h, bit 2j for the
//     low-nibble codes and bit 2j + 1 for the high-nibble ones;
//   - scales: the 12 packed bytes of super-block kbx, d and dmin its 4-byte record;
//   - activations: the 16 int8 at k = 64*(Q >> 1) + 16*h and at k + 32, in q8
//     blocks 2*(Q >> 1) and 2*(Q >> 1) + 1.
// Since 64 is a multiple of 8, Q & 7 (hence j and h) is the same for every chunk a
// lane takes.
//
// Per chunk the contribution is, with Dq the exact code dots and Sx the activation
// sums of the two 16-element halves (a: sub-block 2j, b: 2j + 1),
//   d * (d8a * sca*Dqa + d8b * scb*Dqb) - dmin * (d8a * ma*Sxa + d8b * mb*Sxb).
#pragma once

#include "bufload.h"
#include "kq_format.h"
#include "q6k_unit.h"

namespace q6k {

// Activation operands of one q4_K / q5_K chunk for one token.
struct KqAct {
    uint4 xa, xb;   // the 16 int8 activations of each half
    float da, db;   // their q8 block scales (fp16 values, exact in f32)
    float dsa, dsb; // da * sum(xa), db * sum(xb): exact (11-bit scale x 12-bit sum)
};

// Weight operands of one chunk.
struct KqW {
    uint4 qs;       // 16 code bytes (32 codes)
    uint4 qh;       // q5_K: 16 fifth-bit bytes
    uint3 sc;       // the super-block's 12 packed scale/min bytes
    uint32_t dm;    // fp16 d | fp16 dmin << 16
};

struct KqOffs {
    uint32_t qs, qh, sc, dm;
};

__device__ __forceinline__ ActRaw kq_load_act_raw(const int8_t *__restrict__ qs_t,
                                                  const uint16_t *__restrict__ d8_t, uint32_t Q)
{
    const uint32_t k = 64u * (Q >> 1) + 16u * (Q & 1u);
    const uint32_t blk = 2u * (Q >> 1);
    ActRaw r;
    r.xa = *reinterpret_cast<const uint4 *>(qs_t + k);
    r.xb = *reinterpret_cast<const uint4 *>(qs_t + k + 32);
    r.ha = d8_t[blk];
    r.hb = d8_t[blk + 1];
    return r;
}

__device__ __forceinline__ KqAct kq_act_from_raw(const ActRaw &r)
{
    KqAct a;
    a.xa = r.xa;
    a.xb = r.xb;
    a.da = f16_bits_to_f32(r.ha);
    a.db = f16_bits_to_f32(r.hb);
    a.dsa = a.da * (float)sum16_i8(a.xa);
    a.dsb = a.db * (float)sum16_i8(a.xb);
    return a;
}

__device__ __forceinline__ KqAct kq_load_act(const int8_t *__restrict__ qs_t,
                                             const uint16_t *__restrict__ d8_t, uint32_t Q)
{
    return kq_act_from_raw(kq_load_act_raw(qs_t, d8_t, Q));
}

// 6-bit scales and mins of the chunk's sub-blocks s = 2j and 2j + 1 (j = (Q >> 1) & 3)
// from the 12 packed bytes (words p0: bytes 0..3, p1: 4..7, p2: 8..11): for s < 4,
// sc = byte s & 63 and m = byte s+4 & 63; for s >= 4 (i = s - 4),
// sc = (byte i+8 & 15) | (byte i >> 6) << 4 and m = (byte i+8 >> 4) | (byte i+4 >> 6) << 4.
// Both forms are "a low field of width 6 or 4, or-ed with a high field of width 0 or 2
// shifted to bit 4", so each value is two bitfield extracts with per-lane offsets and
// widths (a width-0 extract is 0).
__device__ __forceinline__ void kq_scale_min2(uint3 p, uint32_t Q, int &sca, int &ma, int &scb,
                                              int &mb)
{
    const uint32_t j = (Q >> 1) & 3u;
    const bool hi = j >= 2u;
    const uint32_t o = 16u * (j & 1u);        // bit offset of byte (2j) & 3
    const uint32_t A = hi ? p.z : p.x, Am = hi ? p.z : p.y;
    const uint32_t wl = hi ? 4u : 6u, om = hi ? 4u : 0u, wh = hi ? 2u : 0u;
    const auto bfe = [](uint32_t v, uint32_t off, uint32_t w) {
        return __builtin_amdgcn_ubfe(v, off, w);
    };
    sca = (int)(bfe(A, o, wl) | (bfe(p.x, o + 6u, wh) << 4));
    scb = (int)(bfe(A, o + 8u, wl) | (bfe(p.x, o + 14u, wh) << 4));
    ma = (int)(bfe(Am, o + om, wl) | (bfe(p.y, o + 6u, wh) << 4));
    mb = (int)(bfe(Am, o + 8u + om, wl) | (bfe(p.y, o + 14u, wh) << 4));
}

// The chunk's four codes per 32-bit word: low nibbles (sub-block 2j) or high
// nibbles (2j + 1), with the q5_K fifth bit at bit 4 of each byte (h5: the fifth-bit
// word shifted right by 2j).
template <bool Q5>
__device__ __forceinline__ uint32_t kq_codes_lo(uint32_t q, uint32_t h5)
{
    uint32_t c = q & 0x0F0F0F0Fu;
    if constexpr (Q5)
        c |= (h5 & 0x01010101u) << 4;
    return c;
}
template <bool Q5>
__device__ __forceinline__ uint32_t kq_codes_hi(uint32_t q, uint32_t h5)
{
    uint32_t c = (q >> 4) & 0x0F0F0F0Fu;
    if constexpr (Q5)
        c |= ((h5 >> 1) & 0x01010101u) << 4;
    return c;
}

// Exact code dots of the chunk's two halves.
template <bool Q5>
__device__ __forceinline__ void kq_chunk_dots(const KqW &w, const KqAct &a, uint32_t Q, int &Da,
                                              int &Db)
{
    const uint32_t sh = 2u * ((Q >> 1) & 3u);
    uint32_t h;
    h = Q5 ? w.qh.x >> sh : 0u;
    int da = sdot4_from0((int)kq_codes_lo<Q5>(w.qs.x, h), (int)a.xa.x);
    int db = sdot4_from0((int)kq_codes_hi<Q5>(w.qs.x, h), (int)a.xb.x);
    h = Q5 ? w.qh.y >> sh : 0u;
    da = __builtin_amdgcn_sdot4((int)kq_codes_lo<Q5>(w.qs.y, h), (int)a.xa.y, da, false);
    db = __builtin_amdgcn_sdot4((int)kq_codes_hi<Q5>(w.qs.y, h), (int)a.xb.y, db, false);
    h = Q5 ? w.qh.z >> sh : 0u;
    da = __builtin_amdgcn_sdot4((int)kq_codes_lo<Q5>(w.qs.z, h), (int)a.xa.z, da, false);
    db = __builtin_amdgcn_sdot4((int)kq_codes_hi<Q5>(w.qs.z, h), (int)a.xb.z, db, false);
    h = Q5 ? w.qh.w >> sh : 0u;
    da = __builtin_amdgcn_sdot4((int)kq_codes_lo<Q5>(w.qs.w, h), (int)a.xa.w, da, false);
    db = __builtin_amdgcn_sdot4((int)kq_codes_hi<Q5>(w.qs.w, h), (int)a.xb.w, db, false);
    Da = da;
    Db = db;
}

// acc + d * (d8a * sca*Dqa + d8b * scb*Dqb) - dmin * (d8a * ma*Sxa + d8b * mb*Sxb),
// d and dmin passed in (zero drops the chunk). sc*Dq (|Dq| <= 16*31*128) is an exact
// integer below 2^23, so its f32 conversion is exact; d8*Sx is exact in f32 (an fp16
// value times a 12-bit sum), so m * (d8*Sx) rounds the same real number d8*(m*Sx) does,
// once. Every multiply-add is written out.
template <bool Q5>
__device__ __forceinline__ float kq_chunk_accumulate(float acc, const KqW &w, const KqAct &a,
                                                     uint32_t Q, float d, float dmin)
{
    int Da, Db, sca, ma, scb, mb;
    kq_chunk_dots<Q5>(w, a, Q, Da, Db);
    kq_scale_min2(w.sc, Q, sca, ma, scb, mb);
    const float pd = __builtin_fmaf(a.da, (float)__mul24(sca, Da), a.db * (float)__mul24(scb, Db));
    const float pm = __builtin_fmaf((float)ma, a.dsa, (float)mb * a.dsb);
    return __builtin_fmaf(-dmin, pm, __builtin_fmaf(d, pd, acc));
}

// Format policy for q4_K (Q5 = false) and q5_K (Q5 = true) split-plane rows.
template <bool Q5>
struct FmtKq {
    static constexpr int TYPE = Q5 ? KQT_Q5_K : KQT_Q4_K;
    using W = KqW;
    using Act = KqAct;
    using Offs = KqOffs;

    __device__ static Offs offsets(uint32_t Q, uint32_t nbe)
    {
        const uint32_t kbx = Q >> 3;
        const uint32_t sc_base = (Q5 ? 160u : 128u) * nbe;
        Offs o;
        o.qs = 16u * Q;
        o.qh = 128u * nbe + 32u * kbx + 16u * (Q & 1u);
        o.sc = sc_base + 12u * kbx;
        o.dm = sc_base + 12u * nbe + 4u * kbx;
        return o;
    }

    // The same chunk `b` bytes further (a later row under one descriptor).
    __device__ static Offs shifted(const Offs &o, uint32_t b)
    {
        Offs r;
        r.qs = o.qs + b;
        r.qh = o.qh + b;
        r.sc = o.sc + b;
        r.dm = o.dm + b;
        return r;
    }

    __device__ static W load(__amdgpu_buffer_rsrc_t r, const Offs &o)
    {
        W w;
        w.qs = load_b128<POLICY_STREAM>(r, o.qs);
        if constexpr (Q5)
            w.qh = load_b128<POLICY_STREAM>(r, o.qh);
        else
            w.qh = make_uint4(0u, 0u, 0u, 0u);
        w.sc = load_b96<POLICY_DEFAULT>(r, o.sc);
        w.dm = load_b32<POLICY_DEFAULT>(r, o.dm);
        return w;
    }

    __device__ static Act act(const int8_t *qs_t, const uint16_t *d8_t, uint32_t Q)
    {
        return kq_load_act(qs_t, d8_t, Q);
    }

    // act() in two steps: the loads, then the arithmetic on what they returned
    __device__ static ActRaw act_raw(const int8_t *qs_t, const uint16_t *d8_t, uint32_t Q)
    {
        return kq_load_act_raw(qs_t, d8_t, Q);
    }
    __device__ static Act act_finish(const ActRaw &r) { return kq_act_from_raw(r); }

    // live = false drops the chunk (d = dmin = 0); callers whose operands were
    // dropped already pass true
    __device__ static float accumulate(float acc, const W &w, const Act &a, uint32_t Q, bool live)
    {
        const float d = live ? f16_bits_to_f32(w.dm & 0xFFFFu) : 0.0f;
        const float dmin = live ? f16_bits_to_f32(w.dm >> 16) : 0.0f;
        return kq_chunk_accumulate<Q5>(acc, w, a, Q, d, dmin);
    }

    // Operands that make the chunk contribute exactly zero: the block scales, which
    // multiply everything else, set to 0 (the weights are finite).
    __device__ static void drop(Act &a)
    {
        a.da = 0.0f;
        a.db = 0.0f;
        a.dsa = 0.0f;
        a.dsb = 0.0f;
    }

    // The operands as three 16-byte words (LDS staging) and back; all-zero words give
    // operands that contribute exactly zero.
    __device__ static void to_words(const Act &a, uint4 &xa, uint4 &xb, uint4 &sc)
    {
        xa = a.xa;
        xb = a.xb;
        sc = make_uint4(__builtin_bit_cast(uint32_t, a.da), __builtin_bit_cast(uint32_t, a.db),
                        __builtin_bit_cast(uint32_t, a.dsa), __builtin_bit_cast(uint32_t, a.dsb));
    }
    __device__ static Act from_words(const uint4 &xa, const uint4 &xb, const uint4 &sc)
    {
        const uint32_t s0 = sc.x, s1 = sc.y, s2 = sc.z, s3 = sc.w;
        Act a;
        a.xa = xa;
        a.xb = xb;
        a.da = __builtin_bit_cast(float, s0);
        a.db = __builtin_bit_cast(float, s1);
        a.dsa = __builtin_bit_cast(float, s2);
        a.dsb = __builtin_bit_cast(float, s3);
        return a;
    }
};

using FmtQ4K = FmtKq<false>;
using FmtQ5K = FmtKq<true>;

}  // namespace q6k
