// tern_tile.h — per-lane plane-tile loads and decode + MFMA steps shared by
// the ternary GEMV kernels (one launch per linear, and the persistent chain).
//
// A k-tile is 4 blocks of 128 weights of one 16-row tile.  Lane (r, g) of a
// wave holds plane word g (32 weights) of each of the 4 blocks of row r, and
// the four fp16 block scales of row r.
#pragma once

#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

struct PlaneTile {
    u32x4 nz, sg;   // word g of the (up to) 4 blocks of the k-tile
    u32x2 sc;       // fp16 scales of the 4 blocks for row r
};

// Load the plane words and scales a lane (row r, word g) needs from k-tile kt
// of row tile rt.  nbq = blocks in this k-tile (4 except a narrower last tile).
template <typename WordPtr, typename ScalePtr>
__device__ __forceinline__ PlaneTile load_plane_tile(WordPtr words, ScalePtr scales, int64_t rt, int kt, int nb,
                                                     int r, int g)
{
    PlaneTile p;
    const int64_t wb = tile_word_base(rt, kt, nb);
    const int64_t sb = tile_scale_base(rt, kt, nb);
    const int nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
    if (nbq == 4) {
        p.nz = ld_nt16(words + wb + (int64_t)((0 * 4 + g) * 16 + r) * 4);
        p.sg = ld_nt16(words + wb + (int64_t)((1 * 4 + g) * 16 + r) * 4);
        p.sc = ld_nt8(scales + sb + r * 4);
    } else {
        p.nz = u32x4{0, 0, 0, 0};
        p.sg = u32x4{0, 0, 0, 0};
        uint32_t s01 = 0, s23 = 0;
        for (int bq = 0; bq < nbq; ++bq) {
            p.nz[bq] = words[wb + (int64_t)((0 * 4 + g) * 16 + r) * nbq + bq];
            p.sg[bq] = words[wb + (int64_t)((1 * 4 + g) * 16 + r) * nbq + bq];
            const uint32_t h = scales[sb + r * nbq + bq];
            if (bq < 2) s01 |= h << (16 * bq);
            else s23 |= h << (16 * (bq - 2));
        }
        p.sc = u32x2{s01, s23};
    }
    return p;
}

__device__ __forceinline__ float tile_scale(const PlaneTile& p, int bq)
{
    const uint32_t w = p.sc[bq >> 1];
    return half_bits_to_float((w >> (16 * (bq & 1))) & 0xFFFFu);
}

// 64-bit left shift by S.  The amount reaches the shift through an SGPR the
// compiler cannot see into: with a constant amount it splits the shift into
// two 32-bit operations (only the masked bits of each half are used), while
// v_lshlrev_b64 issues at the full VALU rate.  The shift itself stays a
// compiler-visible instruction, so the hazard recognizer still inserts the
// wait states for a destination an in-flight MFMA is about to write (which it
// cannot do for a hand-written VALU instruction).
template <int S>
__device__ __forceinline__ uint64_t shl64(uint64_t v)
{
    uint32_t s;
    asm("s_mov_b32 %0, %1" : "=s"(s) : "i"(S));
    return v << s;
}

// Decode word pair (N, S) into the four B operands of the block's four MFMA
// steps (step c = weights 8c .. 8c+7 of the word).  Output dword j holds
// weights 2j (low half) and 2j+1 (high half) as bf16 2*t: 0x4000 = +2,
// 0xC000 = -2, 0 = 0 (a non-canonical sign bit without a nonzero bit would
// give -0).  c2 rotated right by one bit puts both code words' pairs at even
// bit positions, so one 64-bit shift of {c2', c1} aligns pair j of both words
// at bits (14, 15) / (30, 31): 7 shifts + 16 masks per 32 weights.
__device__ __forceinline__ void decode_bf16(uint32_t N, uint32_t S, u32x4 (&B)[4])
{
    const CodeWords c = interleave(N, S);
    const uint32_t c2r = __builtin_amdgcn_alignbit(c.c2, c.c2, 1);
    const uint64_t d = ((uint64_t)c2r << 32) | c.c1;
    const uint64_t sh[8] = {shl64<14>(d), shl64<12>(d), shl64<10>(d), shl64<8>(d),
                            shl64<6>(d),  shl64<4>(d),  shl64<2>(d),  d};
    uint32_t o[16];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        o[2 * p] = (uint32_t)sh[p] & 0xC000C000u;              // weights (4p, 4p+1)
        o[2 * p + 1] = (uint32_t)(sh[p] >> 32) & 0xC000C000u;  // weights (4p+2, 4p+3)
    }
    B[0] = u32x4{o[0], o[1], o[2], o[3]};
    B[1] = u32x4{o[4], o[5], o[6], o[7]};
    B[2] = u32x4{o[8], o[9], o[10], o[11]};
    B[3] = u32x4{o[12], o[13], o[14], o[15]};
}

// Decode word pair (N, S) into the two int8 B operands of the block's two
// MFMA 16x16x64 steps (bytes 64*t in the i8_quad order).
__device__ __forceinline__ void decode_i8(uint32_t N, uint32_t S, u32x4 (&B)[2])
{
    const CodeWords c = interleave(N, S);
    B[0] = u32x4{i8_quad<0>(c), i8_quad<1>(c), i8_quad<2>(c), i8_quad<3>(c)};
    B[1] = u32x4{i8_quad<4>(c), i8_quad<5>(c), i8_quad<6>(c), i8_quad<7>(c)};
}

// Two blocks of one k-tile with their MFMA chains interleaved.  xa points at
// the staged activations of this lane's row at the first block's k + 32*g.
template <int MT>
__device__ __forceinline__ void bf16_block_pair(uint32_t n0, uint32_t s0, uint32_t n1, uint32_t s1, float sc0,
                                                float sc1, const uint16_t* xa, f32x4& acc)
{
    u32x4 B0[4], B1[4];
    decode_bf16(n0, s0, B0);
    decode_bf16(n1, s1, B1);
    f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        d0 = mfma_bf16(*(const u32x4*)(xa + 8 * c), B0[c], d0);
        d1 = mfma_bf16(*(const u32x4*)(xa + kBlockK + 8 * c), B1[c], d1);
    }
#pragma unroll
    for (int i = 0; i < (MT < 4 ? MT : 4); ++i) {
        acc[i] = __builtin_fmaf(sc0, d0[i], acc[i]);
        acc[i] = __builtin_fmaf(sc1, d1[i], acc[i]);
    }
}

template <int MT>
__device__ __forceinline__ void bf16_block(uint32_t n0, uint32_t s0, float sc0, const uint16_t* xa, f32x4& acc)
{
    u32x4 B0[4];
    decode_bf16(n0, s0, B0);
    f32x4 d0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) d0 = mfma_bf16(*(const u32x4*)(xa + 8 * c), B0[c], d0);
#pragma unroll
    for (int i = 0; i < (MT < 4 ? MT : 4); ++i) acc[i] = __builtin_fmaf(sc0, d0[i], acc[i]);
}

// One k-tile of a lane's row: xt points at the staged activations of this
// lane's row at k = 512*kt + 32*g.  Scales are halved because decoded
// weights are 2*t.
template <int MT>
__device__ __forceinline__ void bf16_tile(const PlaneTile& t, const uint16_t* xt, int nbq, f32x4& acc)
{
    if (nbq == 4) {
        bf16_block_pair<MT>(t.nz[0], t.sg[0], t.nz[1], t.sg[1], 0.5f * tile_scale(t, 0), 0.5f * tile_scale(t, 1),
                            xt, acc);
        bf16_block_pair<MT>(t.nz[2], t.sg[2], t.nz[3], t.sg[3], 0.5f * tile_scale(t, 2), 0.5f * tile_scale(t, 3),
                            xt + 2 * kBlockK, acc);
    } else {
        for (int bq = 0; bq < nbq; ++bq)
            bf16_block<MT>(t.nz[bq], t.sg[bq], 0.5f * tile_scale(t, bq), xt + bq * kBlockK, acc);
    }
}

}  // namespace tern
