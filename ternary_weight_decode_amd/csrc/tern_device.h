// tern_device.h — device-side building blocks for the gfx950 ternary kernels.
//
// Packed layout (defined in include/tern.h): 16-row tiles, 4-block (512-k)
// k-tiles; inside a tile, plane-major, then word w (32 weights of a block),
// then row r, then block bq.  A lane that owns (row r, word w) of a tile
// therefore reads its nonzero words of the four blocks as one 16-byte load and
// its sign words as another, and a wave's load covers 1 KiB contiguously.
//
// Decoding targets the matrix cores.  For a 16x16xK MFMA the B operand of
// lane l holds column n = l % 16 and k-slot group g = l / 16; the A operand
// of lane l holds row m = l % 16 of the same slot group.  A lane (r, g) thus
// decodes word g of block b for weight row r and multiplies it against
// activations x[m = r][128b + 32g + ...] — every MFMA contracts 32 (bf16) or
// 64 (int8) k values from a single 128-weight block, so one fp16 block scale
// applies to the whole MFMA result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 16;     // rows per packed tile (= MFMA N)
constexpr int kBlockK = 128;      // weights per block (one fp16 scale)
constexpr int kTileBlocks = 4;    // blocks per k-tile
constexpr int kTileK = 512;       // k per k-tile

__device__ __forceinline__ uint32_t rotl32(uint32_t x, int r)
{
    // funnel shift of {x, x}: rotate left by r (r may be negative)
    return __builtin_amdgcn_alignbit(x, x, (uint32_t)(32 - r) & 31u);
}

__device__ __forceinline__ uint32_t bfi32(uint32_t mask, uint32_t a, uint32_t b)
{
    return (a & mask) | (b & ~mask);
}

// Row q and column r of the chunks u = first + c * stride (c = 0, 1, ...) of
// rows of `per_row` chunks, without a division per chunk: one division for
// the first chunk, the stride's quotient and remainder (uniform), then one
// add with a carry per step.  Activation staging runs 2..16 chunks per
// thread, and a division by a run-time value costs about 25 VALU
// instructions (four of them quarter-rate multiplies).
struct ChunkWalk {
    int q, r, dq, dr, per_row;
    __device__ __forceinline__ ChunkWalk(int first, int stride, int per_row_) : per_row(per_row_)
    {
        q = first / per_row;
        r = first - q * per_row;
        dq = stride / per_row;
        dr = stride - dq * per_row;
    }
    __device__ __forceinline__ void next()
    {
        r += dr;
        q += dq;
        if (r >= per_row) {
            r -= per_row;
            ++q;
        }
    }
};

// Interleave one nonzero word N and sign word S (weight i at bit
// 16*(i&1) + (i>>1) in both) into two code words whose adjacent bit pairs are
// (nonzero, sign) of one weight:
//   c1: pair at bits (2p, 2p+1)   = weight at plane position 2p
//   c2: pair at bits (2p+1, 2p+2) = weight at plane position 2p+1 (mod 32)
struct CodeWords {
    uint32_t c1, c2;
};

__device__ __forceinline__ CodeWords interleave(uint32_t N, uint32_t S)
{
    uint32_t R = rotl32(S, 1);
    CodeWords c;
    c.c1 = bfi32(0x55555555u, N, R);
    c.c2 = bfi32(0xAAAAAAAAu, N, R);
    return c;
}

// int8 quad d (d = 0..7) of a 32-weight word: bytes are 64*t of weights
// (2d, 2d+16, 2d+1, 2d+17).  Requires canonical planes.
template <int D>
__device__ __forceinline__ uint32_t i8_quad(const CodeWords& c)
{
    const uint32_t src = (D & 1) ? c.c2 : c.c1;
    return rotl32(src, 6 - D) & 0xC0C0C0C0u;
}

// Byte permutation applied to int8 activations so that their quad d matches
// i8_quad<d>: from natural dwords lo = q[4(d/2) .. +4), hi = q[16 + 4(d/2) .. +4)
// of a 32-byte word, bytes (q[2d], q[2d+16], q[2d+1], q[2d+17]).
__device__ __forceinline__ uint32_t i8_act_quad(uint32_t lo, uint32_t hi, int d)
{
    return __builtin_amdgcn_perm(hi, lo, (d & 1) ? 0x07030602u : 0x05010400u);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0,
                                                 0, 0);
}

// ---- packed-layout addressing (word / element indices, see include/tern.h)

__host__ __device__ inline int64_t tile_word_base(int64_t rt, int64_t kt, int64_t nb)
{
    return (rt * nb + 4 * kt) * 128;
}

__host__ __device__ inline int64_t tile_scale_base(int64_t rt, int64_t kt, int64_t nb)
{
    return (rt * nb + 4 * kt) * 16;
}

// streaming loads for data read once per call (weights): non-temporal so the
// weight stream does not evict the activations from the caches
__device__ __forceinline__ u32x4 ld_nt16(const void* p)
{
    return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ u32x2 ld_nt8(const void* p)
{
    return __builtin_nontemporal_load((const u32x2*)p);
}

// Pointers known to address global memory.  Loads through them compile to
// global (not flat) instructions, which count only against the vector-memory
// counter, so waiting for LDS traffic never waits for them.
#define TERN_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ u32x4 ld_nt16(const TERN_GLOBAL void* p)
{
    return __builtin_nontemporal_load((const TERN_GLOBAL u32x4*)p);
}

__device__ __forceinline__ u32x2 ld_nt8(const TERN_GLOBAL void* p)
{
    return __builtin_nontemporal_load((const TERN_GLOBAL u32x2*)p);
}

}  // namespace tern
