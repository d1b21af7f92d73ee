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
    int sa, sb;     // sums of xa, xb
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

__device__ __forceinline__ KqAct kq_load_act(const int8_t *__restrict__ qs_t,
                                             const uint16_t *__restrict__ d8_t, uint32_t Q)
{
    const uint32_t k = 64u * (Q >> 1) + 16u * (Q & 1u);
    const uint32_t blk = 2u * (Q >> 1);
    KqAct a;
    a.xa = *reinterpret_cast<const uint4 *>(qs_t + k);
    a.xb = *reinterpret_cast<const uint4 *>(qs_t + k + 32);
    a.da = f16_bits_to_f32(d8_t[blk]);
    a.db = f16_bits_to_f32(d8_t[blk + 1]);
    a.sa = sum16_i8(a.xa);
    a.sb = sum16_i8(a.xb);
    return a;
}

// 6-bit scale and min of sub-block s (0..7) from the 12 packed bytes (words p0:
// bytes 0..3, p1: 4..7, p2: 8..11): for s < 4, sc = byte s & 63, m = byte s+4 & 63;
// for s >= 4 (i = s - 4), sc = (byte i+8 & 15) | (byte i >> 6) << 4 and
// m = (byte i+8 >> 4) | (byte i+4 >> 6) << 4. s is the same for every chunk of a
// lane, so the selects below take per-lane constant conditions.
__device__ __forceinline__ void kq_scale_min(uint3 p, uint32_t s, int &sc, int &m)
{
    const uint32_t sh = 8u * (s & 3u);
    const uint32_t lo_sc = (p.x >> sh) & 63u, lo_m = (p.y >> sh) & 63u;
    const uint32_t hi_sc = ((p.z >> sh) & 15u) | (((p.x >> (sh + 6u)) & 3u) << 4);
    const uint32_t hi_m = ((p.z >> (sh + 4u)) & 15u) | (((p.y >> (sh + 6u)) & 3u) << 4);
    const bool hi = s >= 4u;
    sc = (int)(hi ? hi_sc : lo_sc);
    m = (int)(hi ? hi_m : lo_m);
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
    int da = 0, db = 0;
    uint32_t h;
    h = Q5 ? w.qh.x >> sh : 0u;
    da = __builtin_amdgcn_sdot4((int)kq_codes_lo<Q5>(w.qs.x, h), (int)a.xa.x, da, false);
    db = __builtin_amdgcn_sdot4((int)kq_codes_hi<Q5>(w.qs.x, h), (int)a.xb.x, db, false);
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
// d and dmin passed in (zero drops the chunk). sc*Dq (|Dq| <= 16*31*128) and m*Sx are
// exact integers below 2^23, so their f32 conversions are exact; every multiply-add
// is written out.
template <bool Q5>
__device__ __forceinline__ float kq_chunk_accumulate(float acc, const KqW &w, const KqAct &a,
                                                     uint32_t Q, float d, float dmin)
{
    int Da, Db, sca, ma, scb, mb;
    kq_chunk_dots<Q5>(w, a, Q, Da, Db);
    const uint32_t s = 2u * ((Q >> 1) & 3u);
    kq_scale_min(w.sc, s, sca, ma);
    kq_scale_min(w.sc, s + 1u, scb, mb);
    const float pd = __builtin_fmaf(a.da, (float)__mul24(sca, Da), a.db * (float)__mul24(scb, Db));
    const float pm = __builtin_fmaf(a.da, (float)__mul24(ma, a.sa), a.db * (float)__mul24(mb, a.sb));
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

    __device__ static float accumulate(float acc, const W &w, const Act &a, uint32_t Q, bool live)
    {
        const float d = live ? f16_bits_to_f32(w.dm & 0xFFFFu) : 0.0f;
        const float dmin = live ? f16_bits_to_f32(w.dm >> 16) : 0.0f;
        return kq_chunk_accumulate<Q5>(acc, w, a, Q, d, dmin);
    }
};

using FmtQ4K = FmtKq<false>;
using FmtQ5K = FmtKq<true>;

}  // namespace q6k
