// q6k_unit.h -- per-lane work on one 16-byte low-bit chunk of a dpl row (gfx950).
//
// A dpl row is [ql: nbe*128][qh: nbe*64][sc: nbe*16][d: nbe*2] (D4-4 §3.2 Excerpt B
// gives the section bases). The ql plane is cut into 16-byte chunks, chunk Q holding
// the low bits of 32 codes; a wave64 takes 64 consecutive chunks per instruction,
// so every low-bit load is one contiguous, 16 B-per-lane, 1 KB request.
//
// Chunk Q = 8*kbx + 4*c + 2*s + h (kbx the super-block, c its 128-element half,
// s = g & 1 of the 32-element unit, h the 16-byte half of the unit's 32-byte
// window). By the unit-load address formulas of D4-4 §3.2 Excerpt B (low bits of
// unit (c, g) at kbx*128 + c*64 + (g&1)*32, high bits at kbx*64 + c*32, 2-bit field
// at shift 2g), the chunk's low nibbles are codes of unit g = s and its high
// nibbles codes of unit g = s + 2, positions l = 16h .. 16h+15 of both units:
//   - high bits: the 16 qh bytes at qh plane + 16*(2*(Q>>2) + h); field 2s (low
//     nibble codes) and 2s + 4 (high nibble codes);
//   - scales: sub-blocks j = 8c + 2s + h and j + 4 of the block, i.e. bytes (Q & 3)
//     and (Q & 3) + 4 of the 8-byte scale group at sc plane + 8*(Q>>2);
//   - activations: the 16 int8 at k = 16*(Q + 4*(Q>>2)) and k + 64, in q8 blocks
//     4*(Q>>2) + s and that + 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bufload.h"
#include "kq_format.h"

namespace q6k {

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Activation operands of one chunk for one token.
struct ChunkAct {
    uint4 xa, xb;   // the 16 int8 activations of each of the chunk's two sub-blocks
    float da, db;   // their q8 block scales (fp16 values, exact in f32)
    int na, nb;     // -32 * (sum of the 16 activations): folds the code offset -32 in
};

// Weight operands of one chunk.
struct ChunkW {
    uint4 ql;       // 16 bytes of low bits (32 codes)
    uint4 qh;       // 16 bytes of high-bit fields
    uint2 sc;       // the 8-byte scale group
    uint32_t d;     // fp16 super-block scale bits
};

__device__ __forceinline__ int sum16_i8(uint4 v)
{
    int s = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, 0, false);
    s = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, s, false);
    return __builtin_amdgcn_sdot4((int)v.w, 0x01010101, s, false);
}

// c + the signed int8 dot of a and b, as the three-address v_dot4_i32_i8. The
// builtin selects the two-address accumulate-in-place form, which needs a copy of c
// first whenever c lives on (a hoisted activation sum, a zero).
__device__ __forceinline__ int sdot4_to(int a, int b, int c)
{
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ int sdot4_from0(int a, int b)
{
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// A chunk's activation bytes as loaded, before any arithmetic on them: the two
// 16-byte halves and the fp16 bits of their two q8 block scales.
struct ActRaw {
    uint4 xa, xb;
    uint32_t ha, hb;
};

// qs_t: int8 activations of one token (K entries); d8_t: its fp16 block scales.
__device__ __forceinline__ ActRaw load_act_raw(const int8_t *__restrict__ qs_t,
                                               const uint16_t *__restrict__ d8_t, uint32_t Q)
{
    const uint32_t G = Q >> 2;
    const uint32_t k = 16u * (Q + 4u * G);
    const uint32_t blk = 4u * G + ((Q >> 1) & 1u);
    ActRaw r;
    r.xa = *reinterpret_cast<const uint4 *>(qs_t + k);
    r.xb = *reinterpret_cast<const uint4 *>(qs_t + k + 64);
    r.ha = d8_t[blk];
    r.hb = d8_t[blk + 2];
    return r;
}

__device__ __forceinline__ ChunkAct act_from_raw(const ActRaw &r)
{
    ChunkAct a;
    a.xa = r.xa;
    a.xb = r.xb;
    a.da = f16_bits_to_f32(r.ha);
    a.db = f16_bits_to_f32(r.hb);
    a.na = -32 * sum16_i8(a.xa);
    a.nb = -32 * sum16_i8(a.xb);
    return a;
}

__device__ __forceinline__ ChunkAct load_act(const int8_t *__restrict__ qs_t,
                                             const uint16_t *__restrict__ d8_t, uint32_t Q)
{
    return act_from_raw(load_act_raw(qs_t, d8_t, Q));
}

// row: start of a dpl row; nbe: super-blocks per row.
__device__ __forceinline__ ChunkW load_w(const uint8_t *__restrict__ row, uint32_t nbe, uint32_t Q)
{
    const uint32_t G = Q >> 2;
    ChunkW w;
    w.ql = *reinterpret_cast<const uint4 *>(row + 16u * Q);
    w.qh = *reinterpret_cast<const uint4 *>(row + 128u * nbe + 16u * (2u * G + (Q & 1u)));
    w.sc = *reinterpret_cast<const uint2 *>(row + 192u * nbe + 8u * G);
    w.d = *reinterpret_cast<const uint16_t *>(row + 208u * nbe + 2u * (Q >> 3));
    return w;
}

// Four codes per 32-bit word: low nibbles (unit s) or high nibbles (unit s + 2) of
// the low-bit word l, with the matching 2-bit fields at bits 4..5 of each byte. hm is
// the high-bit word masked to this chunk's two fields (bits 2s..2s+1 and 2s+4..2s+5
// of each byte); up = 4 - 2s moves the first to bits 4..5, 2s the second. Each is
// one bitfield insert: bits 0..3 of every byte from l (or l >> 4), bits 4..7 from the
// shifted fields, whose other bits are zero there.
__device__ __forceinline__ uint32_t codes_lo(uint32_t l, uint32_t hm, uint32_t up)
{
    return (l & 0x0F0F0F0Fu) | ((hm << up) & 0xF0F0F0F0u);
}
__device__ __forceinline__ uint32_t codes_hi(uint32_t l, uint32_t hm, uint32_t sh)
{
    return ((l >> 4) & 0x0F0F0F0Fu) | ((hm >> sh) & 0xF0F0F0F0u);
}

// The chunk's two exact sub-block dots sum (q - 32) * x8: the dot of the unsigned
// codes with the activations, started from -32 * sum(x8).
__device__ __forceinline__ void chunk_dots(const ChunkW &w, const ChunkAct &a, uint32_t Q,
                                           int &Da, int &Db)
{
    const uint32_t sh = 2u * ((Q >> 1) & 1u), up = 4u - sh;
    const uint32_t M = 0x33333333u << sh;
    uint32_t hm = w.qh.x & M;
    int da = sdot4_to((int)codes_lo(w.ql.x, hm, up), (int)a.xa.x, a.na);
    int db = sdot4_to((int)codes_hi(w.ql.x, hm, sh), (int)a.xb.x, a.nb);
    hm = w.qh.y & M;
    da = __builtin_amdgcn_sdot4((int)codes_lo(w.ql.y, hm, up), (int)a.xa.y, da, false);
    db = __builtin_amdgcn_sdot4((int)codes_hi(w.ql.y, hm, sh), (int)a.xb.y, db, false);
    hm = w.qh.z & M;
    da = __builtin_amdgcn_sdot4((int)codes_lo(w.ql.z, hm, up), (int)a.xa.z, da, false);
    db = __builtin_amdgcn_sdot4((int)codes_hi(w.ql.z, hm, sh), (int)a.xb.z, db, false);
    hm = w.qh.w & M;
    da = __builtin_amdgcn_sdot4((int)codes_lo(w.ql.w, hm, up), (int)a.xa.w, da, false);
    db = __builtin_amdgcn_sdot4((int)codes_hi(w.ql.w, hm, sh), (int)a.xb.w, db, false);
    Da = da;
    Db = db;
}

// The chunk's int8 scales of its two sub-blocks.
__device__ __forceinline__ void chunk_scales(const ChunkW &w, uint32_t Q, int &sa, int &sb)
{
    const uint32_t bit = 8u * (Q & 3u);
    sa = (int)(int8_t)(uint8_t)(w.sc.x >> bit);
    sb = (int)(int8_t)(uint8_t)(w.sc.y >> bit);
}

// The chunk's contribution before its super-block scale, d8a * (sa*Da) + d8b * (sb*Db):
// one rounded product, then one fused multiply-add. |sa| <= 128 and |D| <= 2^16 fit
// the 24-bit multiplier, and sa*Da, sb*Db are exact integers below 2^23, so their
// f32 conversion is exact. Every multiply-add here and in the callers is written out
// (the library is built without implicit contraction), so all kernels round alike.
__device__ __forceinline__ float chunk_partial_nod(const ChunkW &w, const ChunkAct &a, uint32_t Q)
{
    int Da, Db, sa, sb;
    chunk_dots(w, a, Q, Da, Db);
    chunk_scales(w, Q, sa, sb);
    const float fa = (float)__mul24(sa, Da);
    const float fb = (float)__mul24(sb, Db);
    return __builtin_fmaf(a.da, fa, a.db * fb);
}

// acc + d * (the chunk's contribution), d passed in (the caller may zero it to drop
// the chunk).
__device__ __forceinline__ float chunk_accumulate(float acc, const ChunkW &w, const ChunkAct &a,
                                                  uint32_t Q, float d)
{
    return __builtin_fmaf(d, chunk_partial_nod(w, a, Q), acc);
}

// Byte offsets of one chunk's operands inside a dpl row.
struct ChunkOffs {
    uint32_t ql, qh, sc, d;
};

// Format policy for q6_K dpl rows, the interface the GEMV kernels are written
// against (offsets, loads, activation operands, the chunk's contribution).
struct FmtQ6K {
    static constexpr int TYPE = KQT_Q6_K;
    using W = ChunkW;
    using Act = ChunkAct;
    using Offs = ChunkOffs;

    __device__ static Offs offsets(uint32_t Q, uint32_t nbe)
    {
        const uint32_t G = Q >> 2;
        Offs o;
        o.ql = 16u * Q;
        o.qh = 128u * nbe + 16u * (2u * G + (Q & 1u));
        o.sc = 192u * nbe + 8u * G;
        o.d = 208u * nbe + 2u * (Q >> 3);
        return o;
    }

    // The same chunk `b` bytes further (a later row under one descriptor).
    __device__ static Offs shifted(const Offs &o, uint32_t b)
    {
        Offs r;
        r.ql = o.ql + b;
        r.qh = o.qh + b;
        r.sc = o.sc + b;
        r.d = o.d + b;
        return r;
    }

    // Low/high bits are streamed (non-temporal); the scale group and d keep the
    // default policy (each 64-byte line of them is touched by three load
    // instructions of the same row).
    __device__ static W load(__amdgpu_buffer_rsrc_t r, const Offs &o)
    {
        W w;
        w.ql = load_b128<POLICY_STREAM>(r, o.ql);
        w.qh = load_b128<POLICY_STREAM>(r, o.qh);
        w.sc = load_b64<POLICY_DEFAULT>(r, o.sc);
        w.d = load_b16<POLICY_DEFAULT>(r, o.d);
        return w;
    }

    __device__ static Act act(const int8_t *qs_t, const uint16_t *d8_t, uint32_t Q)
    {
        return load_act(qs_t, d8_t, Q);
    }

    // act() in two steps: the loads, then the arithmetic on what they returned
    __device__ static ActRaw act_raw(const int8_t *qs_t, const uint16_t *d8_t, uint32_t Q)
    {
        return load_act_raw(qs_t, d8_t, Q);
    }
    __device__ static Act act_finish(const ActRaw &r) { return act_from_raw(r); }

    // live = false drops the chunk (d = 0); callers whose operands were dropped
    // already pass true
    __device__ static float accumulate(float acc, const W &w, const Act &a, uint32_t Q, bool live)
    {
        const float d = live ? f16_bits_to_f32(w.d) : 0.0f;
        return chunk_accumulate(acc, w, a, Q, d);
    }

    // Operands that make the chunk contribute exactly zero: the block scales, which
    // multiply everything else, set to 0 (the weights are finite).
    __device__ static void drop(Act &a)
    {
        a.da = 0.0f;
        a.db = 0.0f;
    }

    // The operands as three 16-byte words (LDS staging) and back; all-zero words give
    // operands that contribute exactly zero.
    __device__ static void to_words(const Act &a, uint4 &xa, uint4 &xb, uint4 &sc)
    {
        xa = a.xa;
        xb = a.xb;
        sc = make_uint4(__builtin_bit_cast(uint32_t, a.da), __builtin_bit_cast(uint32_t, a.db),
                        (uint32_t)a.na, (uint32_t)a.nb);
    }
    __device__ static Act from_words(const uint4 &xa, const uint4 &xb, const uint4 &sc)
    {
        const uint32_t s0 = sc.x, s1 = sc.y, s2 = sc.z, s3 = sc.w;
        Act a;
        a.xa = xa;
        a.xb = xb;
        a.da = __builtin_bit_cast(float, s0);
        a.db = __builtin_bit_cast(float, s1);
        a.na = (int)s2;
        a.nb = (int)s3;
        return a;
    }
};

}  // namespace q6k
