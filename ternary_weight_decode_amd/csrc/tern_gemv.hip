// tern_gemv.hip — ternary GEMV / small-M GEMM on the gfx950 matrix cores.
//
//   y[m][n] = sum_b scale[n][b] * sum_{k in block b} t[n][k] * x[m][k]
//
// The weights stay packed in HBM (2.125 bits per weight) and are decoded in
// registers: each lane turns one 32-weight word pair (nonzero, sign) into 16
// bf16 pairs (2*t) with two bit-field inserts and a rotate+mask per pair, and
// the matrix core does the multiply-add against the activations.  One MFMA
// 16x16x32 covers 16 weight rows x 32 k of one block, so the block scale is
// applied once per 4 MFMAs on the fp32 result; activation rows m < M ride in
// the 16 MFMA rows for free (M = 1 decode and up to 16 verify positions).
//
// Work split: one workgroup per 16-row tile; its waves split the k-tiles
// (512 k each) round-robin and their fp32 partials are summed in LDS in a
// fixed order (deterministic).  Activations are staged in LDS (in k-chunks
// when M*K is large); weight tiles are prefetched one k-tile ahead with
// non-temporal 16-byte loads.
#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

struct PlaneTile {
    u32x4 nz, sg;   // word g of the (up to) 4 blocks of the k-tile
    u32x2 sc;       // fp16 scales of the 4 blocks for row r
};

// Load the plane words and scales a lane (row r, word g) needs from k-tile kt
// of row tile rt.  nbq = blocks in this k-tile (4 except a narrower last tile).
__device__ __forceinline__ PlaneTile load_plane_tile(const uint32_t* __restrict__ words,
                                                     const uint16_t* __restrict__ scales, int64_t rt, int kt,
                                                     int nb, int r, int g)
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

// Decode word pair (N, S) into the four B operands of the block's four MFMA
// steps (step c = weights 8c .. 8c+7 of the word, as bf16 2*t).
__device__ __forceinline__ void decode_bf16(uint32_t N, uint32_t S, u32x4 (&B)[4])
{
    const CodeWords c = interleave(N, S);
    B[0] = u32x4{bf16_pair<0>(c), bf16_pair<1>(c), bf16_pair<2>(c), bf16_pair<3>(c)};
    B[1] = u32x4{bf16_pair<4>(c), bf16_pair<5>(c), bf16_pair<6>(c), bf16_pair<7>(c)};
    B[2] = u32x4{bf16_pair<8>(c), bf16_pair<9>(c), bf16_pair<10>(c), bf16_pair<11>(c)};
    B[3] = u32x4{bf16_pair<12>(c), bf16_pair<13>(c), bf16_pair<14>(c), bf16_pair<15>(c)};
}

// Decode word pair (N, S) into the two int8 B operands of the block's two
// MFMA 16x16x64 steps (bytes 64*t in the i8_quad order).
__device__ __forceinline__ void decode_i8(uint32_t N, uint32_t S, u32x4 (&B)[2])
{
    const CodeWords c = interleave(N, S);
    B[0] = u32x4{i8_quad<0>(c), i8_quad<1>(c), i8_quad<2>(c), i8_quad<3>(c)};
    B[1] = u32x4{i8_quad<4>(c), i8_quad<5>(c), i8_quad<6>(c), i8_quad<7>(c)};
}

// Sum the per-wave 16x16 accumulators (lane l, element i = output
// (m = 4*(l/16) + i, n = l % 16)) over the workgroup's waves in wave order and
// return the total for output element e = i*64 + lane, e < 256.
__device__ __forceinline__ void wave_partials_to_lds(float* red, int wave, int lane, const f32x4& acc)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave * 256 + i * 64 + lane] = acc[i];
}

// ------------------------------------------------------------------ bf16

template <int MT>
__global__ __launch_bounds__(512) void gemv_bf16_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                        const uint16_t* __restrict__ x, int M,
                                                        float* __restrict__ y, int kc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int nw = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int64_t rt = blockIdx.x;
    const int64_t nb = K / kBlockK, nkt = (nb + 3) / 4;
    const uint32_t* words = (const uint32_t*)packed;
    const uint16_t* scales = (const uint16_t*)(packed + scale_region_offset(N, K));

    const int xstride = kc + 8;                    // bf16 elements per staged row (16-byte pad)
    uint16_t* xs = (uint16_t*)smem;
    float* red = (float*)(smem + (size_t)M * xstride * 2);
    const int mrow = r < M ? r : M - 1;             // A rows >= M duplicate row M-1 (their outputs are dropped)

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int64_t kt = wave;
    PlaneTile cur;
    if (kt < nkt) cur = load_plane_tile(words, scales, rt, kt, nb, r, g);

    const int64_t tpc = kc / kTileK;                // k-tiles per chunk
    const int64_t nchunks = (nkt + tpc - 1) / tpc;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t kc0 = c * kc;
        const int64_t kcl = (K - kc0) < kc ? (K - kc0) : kc;
        if (c > 0) __syncthreads();
        {   // stage x[0..M)[kc0 .. kc0+kcl) into LDS, 16 bytes per thread-iteration
            const int64_t units = (int64_t)M * (kcl / 8);
            for (int64_t u = threadIdx.x; u < units; u += blockDim.x) {
                const int64_t m = u / (kcl / 8), c8 = u % (kcl / 8);
                *(u32x4*)(xs + m * xstride + 8 * c8) = *(const u32x4*)(x + m * K + kc0 + 8 * c8);
            }
        }
        __syncthreads();
        const int64_t t_end = (c + 1) * tpc < nkt ? (c + 1) * tpc : nkt;
        while (kt < t_end) {
            const int64_t kt_next = kt + nw;
            PlaneTile nxt;
            if (kt_next < nkt) nxt = load_plane_tile(words, scales, rt, kt_next, nb, r, g);
            const int nbq = (int)(nb - 4 * kt < 4 ? nb - 4 * kt : 4);
            const uint16_t* xt = xs + mrow * xstride + (4 * kt * kBlockK - kc0) + 32 * g;
            auto block = [&](int bq) {
                u32x4 B[4];
                decode_bf16(cur.nz[bq], cur.sg[bq], B);
                const uint16_t* xa = xt + bq * kBlockK;
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) d = mfma_bf16(*(const u32x4*)(xa + 8 * s), B[s], d);
                const float sh = 0.5f * tile_scale(cur, bq);   // decoded weights are 2*t
#pragma unroll
                for (int i = 0; i < (MT < 4 ? MT : 4); ++i) acc[i] = __builtin_fmaf(sh, d[i], acc[i]);
            };
            if (nbq == 4) {
#pragma unroll
                for (int bq = 0; bq < 4; ++bq) block(bq);
            } else {
                for (int bq = 0; bq < nbq; ++bq) block(bq);
            }
            cur = nxt;
            kt = kt_next;
        }
    }

    __syncthreads();
    wave_partials_to_lds(red, wave, lane, acc);
    __syncthreads();
    const int64_t n0 = rt * kTileRows;
    for (int e = threadIdx.x; e < 256; e += blockDim.x) {
        const int i = e >> 6, l = e & 63;
        const int m = 4 * (l >> 4) + i, n = l & 15;
        if (m < M && n0 + n < N) {
            float s = 0.f;
            for (int w = 0; w < nw; ++w) s += red[w * 256 + e];
            y[(int64_t)m * N + n0 + n] = s;
        }
    }
}

// Decode with 64-bit shifts: c2 rotated right by one bit puts both code words'
// pairs at even bit positions, so one 64-bit shift of {c2', c1} aligns pair j
// of both words at bits (14, 15) / (30, 31): 7 shifts + 16 masks per 32
// weights instead of 15 rotates + 16 masks.
__device__ __forceinline__ void decode_bf16_x2(uint32_t N, uint32_t S, u32x4 (&B)[4])
{
    const CodeWords c = interleave(N, S);
    const uint32_t c2r = __builtin_amdgcn_alignbit(c.c2, c.c2, 1);
    const uint64_t d = ((uint64_t)c2r << 32) | c.c1;
    uint32_t o[16];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint64_t sh = d << (14 - 2 * p);
        o[2 * p] = (uint32_t)sh & 0xC000C000u;          // weights (4p, 4p+1)
        o[2 * p + 1] = (uint32_t)(sh >> 32) & 0xC000C000u;  // weights (4p+2, 4p+3)
    }
    B[0] = u32x4{o[0], o[1], o[2], o[3]};
    B[1] = u32x4{o[4], o[5], o[6], o[7]};
    B[2] = u32x4{o[8], o[9], o[10], o[11]};
    B[3] = u32x4{o[12], o[13], o[14], o[15]};
}

// Two blocks of one k-tile with their MFMA chains interleaved.  xa points at
// the staged activations of this lane's row at the first block's k + 32*g.
template <int MT>
__device__ __forceinline__ void bf16_block_pair(uint32_t n0, uint32_t s0, uint32_t n1, uint32_t s1, float sc0,
                                                float sc1, const uint16_t* xa, f32x4& acc)
{
    u32x4 B0[4], B1[4];
    decode_bf16_x2(n0, s0, B0);
    decode_bf16_x2(n1, s1, B1);
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
    decode_bf16_x2(n0, s0, B0);
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

// Fast path: all of x[0..M)[0..K) fits in LDS.  Persistent workgroups: the
// grid is sized to what stays resident, and workgroup b handles row tiles
// b, b + G, b + 2G, ...  Within a row tile, wave w takes k-tiles w, w+nw, ...
// (nw <= number of k-tiles, so every wave has work in every row tile).  Each
// wave runs a ring of TPW plane tiles over its whole (row tile, k-tile)
// sequence, so loads for the next row tile are in flight while the current
// one is reduced.  Activations are staged once per workgroup after the first
// loads are issued.  Per row tile the waves' fp32 partials meet in LDS
// (double-buffered, one barrier per row tile) and are summed in wave order.
// Index arithmetic stays in 32 bits (64-bit divisions are emulated).
template <int MT, int TPW>
__global__ __launch_bounds__(512) void gemv_bf16_fast_kernel(const uint8_t* __restrict__ packed, int64_t N,
                                                             int64_t K, const uint16_t* __restrict__ x, int M,
                                                             float* __restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NI = MT < 4 ? MT : 4;            // accumulator rows in use per lane
    const int nw = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nb = (int)(K / kBlockK), nkt = (nb + 3) >> 2;
    const int nrt = (int)((N + 15) >> 4);
    const uint32_t* words = (const uint32_t*)packed;
    const uint16_t* scales = (const uint16_t*)(packed + scale_region_offset(N, K));
    const int xstride = (int)K + 8;
    uint16_t* xs = (uint16_t*)smem;
    float* red = (float*)(smem + (size_t)M * xstride * 2);   // [2][nw][NI][64]
    const int mrow = r < M ? r : M - 1;
    const int lanes_used = M <= 4 ? 16 : (M <= 8 ? 32 : 64);

    const int rt0 = blockIdx.x, rstep = gridDim.x;
    const int nmy = rt0 < nrt ? (nrt - 1 - rt0) / rstep + 1 : 0;
    const int Jw = (nkt - 1 - wave) / nw + 1;                 // k-tiles per row tile for this wave
    const int U = nmy * Jw;

    PlaneTile slot[TPW];
    int li = 0, lj = 0;                                       // next (row tile, k-tile) to load
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        if (s < U) {
            slot[s] = load_plane_tile(words, scales, rt0 + li * rstep, wave + lj * nw, nb, r, g);
            if (++lj == Jw) { lj = 0; ++li; }
        }
    }

    {
        const int per_row = (int)(K >> 3);
        const int units = M * per_row;
        for (int u = threadIdx.x; u < units; u += blockDim.x) {
            const int m = u / per_row, c8 = u - m * per_row;
            *(u32x4*)(xs + m * xstride + 8 * c8) = *(const u32x4*)(x + (int64_t)m * K + 8 * c8);
        }
    }
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xrow = xs + mrow * xstride + 32 * g;
    int pi = 0, pj = 0;                                       // (row tile, k-tile) being processed
    for (int u0 = 0; u0 < U; u0 += TPW) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            if (u0 + s < U) {
                const int kt = wave + pj * nw;
                const int nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
                bf16_tile<MT>(slot[s], xrow + kt * kTileK, nbq, acc);
                if (u0 + s + TPW < U) {
                    slot[s] = load_plane_tile(words, scales, rt0 + li * rstep, wave + lj * nw, nb, r, g);
                    if (++lj == Jw) { lj = 0; ++li; }
                }
                if (++pj == Jw) {                             // row tile pi complete in this wave
                    float* rb = red + (pi & 1) * nw * NI * 64;
                    if (lane < lanes_used) {
#pragma unroll
                        for (int i = 0; i < NI; ++i) rb[(wave * NI + i) * 64 + lane] = acc[i];
                    }
                    __syncthreads();
                    const int64_t n0 = (int64_t)(rt0 + pi * rstep) * kTileRows;
                    for (int e = threadIdx.x; e < NI * 64; e += blockDim.x) {
                        const int i = e >> 6, l = e & 63;
                        const int m = 4 * (l >> 4) + i, n = l & 15;
                        if (l < lanes_used && m < M && n0 + n < N) {
                            float sum = 0.f;
                            for (int w = 0; w < nw; ++w) sum += rb[(w * NI + i) * 64 + l];
                            y[(int64_t)m * N + n0 + n] = sum;
                        }
                    }
                    acc = f32x4{0.f, 0.f, 0.f, 0.f};
                    pj = 0;
                    ++pi;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ int8

template <int MT>
__global__ __launch_bounds__(512) void gemv_i8_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                      const int8_t* __restrict__ q, const float* __restrict__ s_x,
                                                      int M, float* __restrict__ y, int32_t* __restrict__ acc_dbg,
                                                      int kc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int nw = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int64_t rt = blockIdx.x;
    const int64_t nb = K / kBlockK, nkt = (nb + 3) / 4;
    const int64_t n0 = rt * kTileRows;
    const uint32_t* words = (const uint32_t*)packed;
    const uint16_t* scales = (const uint16_t*)(packed + scale_region_offset(N, K));

    const int qstride = kc + 16;                   // bytes per staged row
    uint8_t* qs = smem;
    float* red = (float*)(smem + (size_t)M * qstride);
    const int mrow = r < M ? r : M - 1;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int64_t kt = wave;
    PlaneTile cur;
    if (kt < nkt) cur = load_plane_tile(words, scales, rt, kt, nb, r, g);

    const int64_t tpc = kc / kTileK;
    const int64_t nchunks = (nkt + tpc - 1) / tpc;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t kc0 = c * kc;
        const int64_t kcl = (K - kc0) < kc ? (K - kc0) : kc;
        if (c > 0) __syncthreads();
        {   // stage q with the byte order of i8_quad, 32 bytes per thread-iteration
            const int64_t units = (int64_t)M * (kcl / 32);
            for (int64_t u = threadIdx.x; u < units; u += blockDim.x) {
                const int64_t m = u / (kcl / 32), c32 = u % (kcl / 32);
                const u32x4* src = (const u32x4*)(q + m * K + kc0 + 32 * c32);
                const u32x4 lo = src[0], hi = src[1];
                const uint32_t Q[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                u32x4 o0, o1;
#pragma unroll
                for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
                for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
                u32x4* dst = (u32x4*)(qs + m * qstride + 32 * c32);
                dst[0] = o0;
                dst[1] = o1;
            }
        }
        __syncthreads();
        const int64_t t_end = (c + 1) * tpc < nkt ? (c + 1) * tpc : nkt;
        while (kt < t_end) {
            const int64_t kt_next = kt + nw;
            PlaneTile nxt;
            if (kt_next < nkt) nxt = load_plane_tile(words, scales, rt, kt_next, nb, r, g);
            const int nbq = (int)(nb - 4 * kt < 4 ? nb - 4 * kt : 4);
            auto block = [&](int bq) {
                u32x4 B[2];
                decode_i8(cur.nz[bq], cur.sg[bq], B);
                const int64_t b = 4 * kt + bq;
                const uint8_t* qa = qs + mrow * qstride + (b * kBlockK - kc0) + 32 * g;
                i32x4 d = {0, 0, 0, 0};
                d = mfma_i8(*(const u32x4*)(qa), B[0], d);
                d = mfma_i8(*(const u32x4*)(qa + 16), B[1], d);
                const float sc = tile_scale(cur, bq) * (1.0f / 64.0f);   // decoded weights are 64*t
#pragma unroll
                for (int i = 0; i < (MT < 4 ? MT : 4); ++i) acc[i] = __builtin_fmaf(sc, (float)d[i], acc[i]);
                if (acc_dbg) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * g + i;
                        if (m < M && n0 + r < N) acc_dbg[((int64_t)m * N + n0 + r) * nb + b] = d[i] >> 6;
                    }
                }
            };
            if (nbq == 4) {
#pragma unroll
                for (int bq = 0; bq < 4; ++bq) block(bq);
            } else {
                for (int bq = 0; bq < nbq; ++bq) block(bq);
            }
            cur = nxt;
            kt = kt_next;
        }
    }

    __syncthreads();
    wave_partials_to_lds(red, wave, lane, acc);
    __syncthreads();
    for (int e = threadIdx.x; e < 256; e += blockDim.x) {
        const int i = e >> 6, l = e & 63;
        const int m = 4 * (l >> 4) + i, n = l & 15;
        if (m < M && n0 + n < N) {
            float s = 0.f;
            for (int w = 0; w < nw; ++w) s += red[w * 256 + e];
            y[(int64_t)m * N + n0 + n] = s_x[m] * s;
        }
    }
}

// ------------------------------------------------------------ launchers

static constexpr int64_t kStageBudget = 48 * 1024;   // LDS bytes for staged activations

static int pick_waves(int64_t nkt) { return nkt >= 8 ? 8 : 4; }

static int pick_chunk(int64_t K, int64_t M, int64_t bytes_per_elem)
{
    int64_t kr = (K + kTileK - 1) / kTileK * kTileK;
    int64_t cap = kStageBudget / (M * bytes_per_elem) / kTileK * kTileK;
    if (cap < kTileK) cap = kTileK;
    return (int)(kr < cap ? kr : cap);
}

static constexpr int64_t kFastLds = 64 * 1024;      // LDS budget of the fast path

// waves per workgroup and k-tiles in flight per wave for the fast path
// (nw never exceeds the number of k-tiles, so every wave works on every row tile)
static void pick_fast(int64_t nkt, int& nw, int& tpw)
{
    nw = nkt >= 8 ? 8 : (nkt >= 4 ? 4 : (int)(nkt < 1 ? 1 : nkt));
    const int64_t per = (nkt + nw - 1) / nw;
    tpw = per >= 3 ? 3 : (int)(per < 1 ? 1 : per);
}

static int device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    return cus;
}

// Workgroups that stay resident at once for this kernel instance (the grid of
// the persistent fast path); falls back to one per row tile on any error.
template <typename F>
static int64_t resident_grid(F kern, int block, size_t lds, int64_t nrt)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, block, lds) != hipSuccess || per_cu <= 0)
        return nrt;
    const int64_t cap = (int64_t)per_cu * device_cus();
    return nrt < cap ? nrt : cap;
}

template <int MT, int TPW>
static hipError_t launch_fast(int nw, size_t lds, hipStream_t stream, const uint8_t* packed, int64_t N, int64_t K,
                              const uint16_t* x, int M, float* y)
{
    const int64_t nrt = (N + 15) / 16;
    const int block = 64 * nw;
    const int64_t grid = resident_grid(gemv_bf16_fast_kernel<MT, TPW>, block, lds, nrt);
    gemv_bf16_fast_kernel<MT, TPW><<<dim3((unsigned)grid), dim3(block), lds, stream>>>(packed, N, K, x, M, y);
    return hipGetLastError();
}

template <int MT>
static hipError_t launch_fast_mt(int tpw, int nw, size_t lds, hipStream_t stream, const uint8_t* packed, int64_t N,
                                 int64_t K, const uint16_t* x, int M, float* y)
{
    if (tpw == 1) return launch_fast<MT, 1>(nw, lds, stream, packed, N, K, x, M, y);
    if (tpw == 2) return launch_fast<MT, 2>(nw, lds, stream, packed, N, K, x, M, y);
    return launch_fast<MT, 3>(nw, lds, stream, packed, N, K, x, M, y);
}

hipError_t launch_gemv_bf16(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                            hipStream_t stream)
{
    const int64_t nkt = (K / kBlockK + 3) / 4;
    int nw, tpw;
    pick_fast(nkt, nw, tpw);
    const int ni = M == 1 ? 1 : (M == 2 ? 2 : 4);   // accumulator rows of the instance (NI)
    const size_t fast_lds = (size_t)M * (K + 8) * 2 + (size_t)2 * nw * ni * 64 * 4;
    if (fast_lds <= (size_t)kFastLds) {
        if (M == 1) return launch_fast_mt<1>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
        if (M == 2) return launch_fast_mt<2>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
        if (M <= 4) return launch_fast_mt<4>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
        return launch_fast_mt<16>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
    }
    // general path: activations staged in k-chunks
    const dim3 grid((unsigned)((N + 15) / 16));
    const int nwc = pick_waves(nkt);
    const int kc = pick_chunk(K, M, 2);
    const size_t lds = (size_t)M * (kc + 8) * 2 + (size_t)nwc * 256 * 4;
    const dim3 block(64 * nwc);
    if (M == 1) gemv_bf16_kernel<1><<<grid, block, lds, stream>>>(packed, N, K, x, (int)M, y, kc);
    else if (M == 2) gemv_bf16_kernel<2><<<grid, block, lds, stream>>>(packed, N, K, x, (int)M, y, kc);
    else if (M <= 4) gemv_bf16_kernel<4><<<grid, block, lds, stream>>>(packed, N, K, x, (int)M, y, kc);
    else gemv_bf16_kernel<16><<<grid, block, lds, stream>>>(packed, N, K, x, (int)M, y, kc);
    return hipGetLastError();
}

hipError_t launch_gemv_i8(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                          int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    const int64_t nkt = (K / kBlockK + 3) / 4;
    const int nw = pick_waves(nkt);
    const int kc = pick_chunk(K, M, 1);
    const size_t lds = (size_t)M * (kc + 16) + (size_t)nw * 256 * 4;
    const dim3 grid((unsigned)((N + 15) / 16)), block(64 * nw);
    if (M == 1) gemv_i8_kernel<1><<<grid, block, lds, stream>>>(packed, N, K, q, s_x, (int)M, y, acc, kc);
    else if (M == 2) gemv_i8_kernel<2><<<grid, block, lds, stream>>>(packed, N, K, q, s_x, (int)M, y, acc, kc);
    else if (M <= 4) gemv_i8_kernel<4><<<grid, block, lds, stream>>>(packed, N, K, q, s_x, (int)M, y, acc, kc);
    else gemv_i8_kernel<16><<<grid, block, lds, stream>>>(packed, N, K, q, s_x, (int)M, y, acc, kc);
    return hipGetLastError();
}

}  // namespace tern
