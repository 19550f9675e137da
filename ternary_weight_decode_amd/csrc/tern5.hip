// tern5.hip — five-level (FV5-style) weights: load-time packing and the
// GEMV / small-M GEMM (bf16 or int8 activations) on the gfx950 matrix cores.
//
// Format (block structure from the FV5 row of the block-format table on the
// discuss.pytorch.kr Neutrino-1 page, section "FV5와 FV5B"): 256-weight
// blocks with two f32 scales s_lo, s_hi and three bit-planes (nonzero, sign,
// high); the weight is  sign * (high ? s_hi : s_lo)  where nonzero is set.
// The bit-level layout is this library's own (include/tern.h): 16-row tiles,
// 512-k tiles; inside a tile plane-major, then word group g (words g and
// g + 4 of the two blocks), then row r, then slot j = 2*block + word/4.  Slot
// j of lane (r, g) thus covers k = 128 j + 32 g .. +31 of the k-tile, the
// same k positions as block j, word g of the ternary tile, so the ternary
// decode and activation addressing carry over.
//
// The two magnitudes need separate sums (s_hi / s_lo is arbitrary), so each
// word yields two B operands: (nonzero & ~high, sign) and (nonzero & high,
// sign), both decoded to bf16 2*sign, on two MFMA chains per block; the block
// epilogue is  0.5 s_lo * d_lo + 0.5 s_hi * d_hi  in fp32.
#include "tern_device.h"
#include "tern_launch.h"
#include "tern_oneshot.h"
#include "tern_tile.h"

namespace tern {

constexpr int kT5TileWords = 768;   // 3 planes x 256 words per (row tile, k-tile)

__host__ __device__ inline int64_t t5_plane_bytes(int64_t N, int64_t K) { return npad16(N) * K * 3 / 8; }

struct Tile5 {
    u32x4 nz, sg, hi;   // slots j = 0..3 of the lane's word group
    f32x4 sc;           // s_lo, s_hi of block 0, then of block 1 (row r)
};

template <typename WordPtr, typename ScalePtr>
__device__ __forceinline__ Tile5 load_tile5(WordPtr words, ScalePtr scales, int64_t rt, int kt, int nkt, int r, int g)
{
    const int64_t tb = rt * nkt + kt;
    const int64_t wb = tb * kT5TileWords + (g * 16 + r) * 4;
    Tile5 t;
    t.nz = ld_nt16(words + wb);
    t.sg = ld_nt16(words + wb + 256);
    t.hi = ld_nt16(words + wb + 512);
    t.sc = __builtin_bit_cast(f32x4, ld_nt16(scales + tb * 64 + r * 4));
    return t;
}

// One k-tile of a lane's row: xt points at the activations of this lane's
// row at k = 512*kt + 32*g (LDS or global).
template <int MT>
__device__ __forceinline__ void tile5_bf16(const Tile5& t, const uint16_t* xt, f32x4& acc)
{
    f32x4 d[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int bh = j >> 1;
        u32x4 BL[4], BH[4];
        decode_bf16(t.nz[j] & ~t.hi[j], t.sg[j], BL);
        decode_bf16(t.nz[j] & t.hi[j], t.sg[j], BH);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 a = *(const u32x4*)(xt + kBlockK * j + 8 * c);
            d[2 * bh] = mfma_bf16(a, BL[c], d[2 * bh]);
            d[2 * bh + 1] = mfma_bf16(a, BH[c], d[2 * bh + 1]);
        }
    }
#pragma unroll
    for (int q = 0; q < (MT < 4 ? MT : 4); ++q) {
        acc[q] = __builtin_fmaf(0.5f * t.sc[0], d[0][q], acc[q]);
        acc[q] = __builtin_fmaf(0.5f * t.sc[1], d[1][q], acc[q]);
        acc[q] = __builtin_fmaf(0.5f * t.sc[2], d[2][q], acc[q]);
        acc[q] = __builtin_fmaf(0.5f * t.sc[3], d[3][q], acc[q]);
    }
}

// int8 activations: qa(j, h) gives the 16-byte A operand h of slot j (q of
// this lane's row at k = 512*kt + 128*j + 32*g, in the decoded byte order).  Each magnitude's words decode
// to bytes 64*sign with their own sign bits (the int8 decode needs the sign
// bit clear where the magnitude bit is clear), the matrix core sums each
// 256-block exactly in int32, and the block sums are scaled in fp32.  dbg,
// when given, receives the exact sums [m][n][block][lo, hi] of this unit.
template <int MT, typename QA>
__device__ __forceinline__ void tile5_i8(const Tile5& t, QA qa, f32x4& acc, int32_t* dbg, int64_t N, int M,
                                         int64_t n, int nb256, int b0, int g)
{
    i32x4 dl[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, dh[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int bh = j >> 1;
        const uint32_t L = t.nz[j] & ~t.hi[j], H = t.nz[j] & t.hi[j];
        u32x4 BL[2], BH[2];
        decode_i8(L, t.sg[j] & L, BL);
        decode_i8(H, t.sg[j] & H, BH);
        const u32x4 a0 = qa(j, 0), a1 = qa(j, 1);
        dl[bh] = mfma_i8(a0, BL[0], dl[bh]);
        dh[bh] = mfma_i8(a0, BH[0], dh[bh]);
        dl[bh] = mfma_i8(a1, BL[1], dl[bh]);
        dh[bh] = mfma_i8(a1, BH[1], dh[bh]);
    }
#pragma unroll
    for (int q = 0; q < (MT < 4 ? MT : 4); ++q) {
        // decoded weights are 64*sign: |sums| < 2^22, exact in fp32
        acc[q] = __builtin_fmaf(t.sc[0] * (1.0f / 64.0f), (float)dl[0][q], acc[q]);
        acc[q] = __builtin_fmaf(t.sc[1] * (1.0f / 64.0f), (float)dh[0][q], acc[q]);
        acc[q] = __builtin_fmaf(t.sc[2] * (1.0f / 64.0f), (float)dl[1][q], acc[q]);
        acc[q] = __builtin_fmaf(t.sc[3] * (1.0f / 64.0f), (float)dh[1][q], acc[q]);
    }
    if (dbg != nullptr) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * g + q;
            if (m < M && n < N) {
#pragma unroll
                for (int bh = 0; bh < 2; ++bh) {
                    int32_t* d = dbg + (((int64_t)m * N + n) * nb256 + b0 + bh) * 2;
                    d[0] = dl[bh][q] >> 6;
                    d[1] = dh[bh][q] >> 6;
                }
            }
        }
    }
}

// 32 bytes of q (natural order, lo = bytes 0..15, hi = 16..31) -> the two
// 16-byte A operands in the decoded byte order
__device__ __forceinline__ void q_decoded_order(const u32x4& lo, const u32x4& hi, u32x4& o0, u32x4& o1)
{
    const uint32_t Q[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
    for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
}

// ------------------------------------------------------------------ pack

// One thread per (row n < Np, block b, word w): reads the 32 levels of the
// word and writes its three plane words; threads with w == 0 also write the
// block's two scales.  |level| >= 2 sets the high bit (levels are clamped to
// [-2, 2]); rows n >= N are padding, written as zeros.
__global__ void pack5_kernel(const int8_t* __restrict__ lv, const float* __restrict__ s_lo,
                             const float* __restrict__ s_hi, int64_t N, int64_t K, uint32_t* __restrict__ words,
                             float* __restrict__ scales)
{
    const int64_t nb = K / 256, nkt = K / 512;
    const int64_t total = npad16(N) * nb * 8;
    for (int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tid < total;
         tid += (int64_t)gridDim.x * blockDim.x) {
        const int w = (int)(tid & 7);
        const int64_t b = (tid >> 3) % nb;
        const int64_t n = (tid >> 3) / nb;
        uint32_t nz = 0, sg = 0, hh = 0;
        if (n < N) {
            const u32x4* src = (const u32x4*)(lv + n * K + b * 256 + 32 * w);
            const u32x4 lo = src[0], hi = src[1];
            const uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int v = (int)(int8_t)(d[i >> 2] >> (8 * (i & 3)));
                const int pos = 16 * (i & 1) + (i >> 1);
                nz |= (uint32_t)(v != 0) << pos;
                sg |= (uint32_t)(v < 0) << pos;
                hh |= (uint32_t)(v >= 2 || v <= -2) << pos;
            }
        }
        const int64_t rt = n >> 4, r = n & 15, kt = b >> 1, bh = b & 1;
        const int64_t g = w & 3, j = 2 * bh + (w >> 2);
        const int64_t base = (rt * nkt + kt) * kT5TileWords + (g * 16 + r) * 4 + j;
        words[base] = nz;
        words[base + 256] = sg;
        words[base + 512] = hh;
        if (w == 0) {
            const int64_t e = ((rt * nkt + kt) * 16 + r) * 4 + 2 * bh;
            scales[e] = n < N ? s_lo[n * nb + b] : 0.f;
            scales[e + 1] = n < N ? s_hi[n * nb + b] : 0.f;
        }
    }
}

// ------------------------------------------------------------------ GEMV

// One pass over the weights (the configuration of tern_oneshot.h): x is
// staged in LDS once per workgroup, every wave's units are requested up front
// (the first before x is staged, the rest right after), partials are summed
// in LDS in k-tile order.  kI8: int8 activations q with row scales s_x (staged
// in the decoded byte order), y = s_x * sum.  XC = activation chunks per
// thread (16 bytes of bf16, or 32 bytes of int8).  kReuse: the partials
// overwrite x's LDS once every wave has computed (a second barrier).
template <bool kI8, int MT, int U, int XC, bool kReuse = false>
__global__ __launch_bounds__(1024) void gemv5_oneshot_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                             const void* __restrict__ x,
                                                             const float* __restrict__ s_x, int M,
                                                             float* __restrict__ y, int32_t* __restrict__ acc_dbg)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NI = MT < 4 ? MT : 4;
    constexpr int kChunkBytes = kI8 ? 32 : 16;
    constexpr int kLoadsPerChunk = kChunkBytes / 16;
    const int nthreads = blockDim.x, nw = nthreads >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nkt = (int)(K >> 9);
    const int nrt = (int)((N + 15) >> 4);
    const int rt0 = (int)blockIdx.x, G = (int)gridDim.x;
    const int rn = (nrt - 1 - rt0) / G + 1;                 // row tiles b, b + G, ...
    const int units = rn * nkt;
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL uint32_t* scales = (const TERN_GLOBAL uint32_t*)(packed + t5_plane_bytes(N, K));
    const TERN_GLOBAL u32x4* xg = (const TERN_GLOBAL u32x4*)x;
    const int xrow_bytes = kI8 ? (int)K + 16 : ((int)K + 8) * 2;   // staged bytes per activation row
    float* red = (float*)(smem + (kReuse ? 0 : (size_t)M * xrow_bytes));   // [unit + 1 spare][NI][64]

    // activations first; a chunk index past the end re-loads the last chunk
    // and stores it to a dummy slot (the start of the partials, written only
    // after the barrier), so every load is issued and used unconditionally
    const int per_row = (int)(K * (kI8 ? 1 : 2) / kChunkBytes), chunks = M * per_row;
    u32x4 xv[XC][kLoadsPerChunk];
    int xdst[XC];
    ChunkWalk cw((int)threadIdx.x, nthreads, per_row);
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const int u = threadIdx.x + c * nthreads;
        const int uc = u < chunks ? u : chunks - 1;
#pragma unroll
        for (int h = 0; h < kLoadsPerChunk; ++h) xv[c][h] = xg[(int64_t)uc * kLoadsPerChunk + h];
        xdst[c] = u < chunks ? cw.q * xrow_bytes + kChunkBytes * cw.r : M * xrow_bytes;
        cw.next();
    }
    __builtin_amdgcn_sched_barrier(0);
    Tile5 t[U];
    auto load_unit = [&](int i) {
        int j = wave + i * nw;
        j = j < units ? j : units - 1;
        const int lrt = j / nkt, kt = j - lrt * nkt;
        t[i] = load_tile5(words, scales, rt0 + lrt * G, kt, nkt, r, g);
    };
    // only the first unit is requested ahead of the activations, which every
    // unit needs and which would otherwise queue behind all of the weights
    load_unit(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        if constexpr (kI8) {
            u32x4 o0, o1;
            q_decoded_order(xv[c][0], xv[c][kLoadsPerChunk - 1], o0, o1);
            *(u32x4*)(smem + xdst[c]) = o0;
            *(u32x4*)(smem + xdst[c] + 16) = o1;
        } else {
            *(u32x4*)(smem + xdst[c]) = xv[c][0];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 1; i < U; ++i) {
        load_unit(i);
        __builtin_amdgcn_sched_barrier(0);
    }

    const int mrow = r < M ? r : M - 1;
    const uint8_t* xrow = smem + mrow * xrow_bytes + (kI8 ? 32 : 64) * g;
    f32x4 keep[kReuse ? U : 1];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int j = wave + i * nw;
        const int jc = j < units ? j : units - 1;
        const int lrt = jc / nkt, kt = jc - lrt * nkt;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kI8) {
            const int64_t n = (int64_t)(rt0 + lrt * G) * kTileRows + r;
            const uint8_t* qt = xrow + kt * kTileK;
            tile5_i8<MT>(t[i], [&](int jj, int h) { return *(const u32x4*)(qt + kBlockK * jj + 16 * h); }, acc,
                         j < units ? acc_dbg : nullptr, N, M, n, (int)(K >> 8), 2 * kt, g);
        } else {
            tile5_bf16<MT>(t[i], (const uint16_t*)xrow + kt * kTileK, acc);
        }
        if constexpr (kReuse) {
            keep[i] = acc;
        } else {
            const int slot = j < units ? j : units;
#pragma unroll
            for (int q = 0; q < NI; ++q) red[(slot * NI + q) * 64 + lane] = acc[q];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kReuse) {
        __syncthreads();                     // every wave is done with x
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int j = wave + i * nw;
            const int slot = j < units ? j : units;
#pragma unroll
            for (int q = 0; q < NI; ++q) red[(slot * NI + q) * 64 + lane] = keep[i][q];
        }
    }
    __syncthreads();

    const int lanes_used = M <= 4 ? 16 : (M <= 8 ? 32 : 64);
    const int nout = rn * NI * 64;
    for (int e = threadIdx.x; e < nout; e += nthreads) {
        const int l = e & 63, q = (e >> 6) % NI, lrt = (e >> 6) / NI;
        const int m = 4 * (l >> 4) + q, n = l & 15;
        const int64_t row = (int64_t)(rt0 + lrt * G) * kTileRows + n;
        if (l < lanes_used && m < M && row < N) {
            const float* pr = red + ((int64_t)lrt * nkt * NI + q) * 64 + l;
            float sum = 0.f;
            for (int kt = 0; kt < nkt; ++kt) sum += pr[kt * NI * 64];
            y[(int64_t)m * N + row] = kI8 ? s_x[m] * sum : sum;
        }
    }
}

// Two-phase variant for activations larger than LDS (large K at bf16
// M >= 6, int8 M >= 13): RT row tiles per workgroup (1, or 2 for bf16 when
// one tile's waves would each stage more than 8 chunks), nkt / 2 waves per
// row tile with two units each, unit i of every wave in half i of K; both
// halves of x loaded into registers up front, staged one half at a time (as
// the ternary two-phase kernel).  16 MFMA activation rows.
template <bool kI8, int XC, int RT>
__global__ __launch_bounds__(1024) void gemv5_phased_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                            const void* __restrict__ x, const float* __restrict__ s_x,
                                                            int M, float* __restrict__ y, int32_t* __restrict__ acc_dbg)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NI = 4;
    constexpr int kChunkBytes = kI8 ? 32 : 16;
    constexpr int kLoadsPerChunk = kChunkBytes / 16;
    const int nthreads = blockDim.x, nw = nthreads >> 6;   // nw = RT * nkt / 2
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nkt = (int)(K >> 9);
    const int nwh = nw / RT;                                          // waves per row tile (nkt / 2)
    const int lrt = wave / nwh, lw = wave - lrt * nwh;               // this wave's row tile and local wave
    // a row tile past the last one loads the workgroup's first tile and stores nothing
    const int64_t rt_out = (int64_t)blockIdx.x * RT + lrt;
    const int64_t rt = rt_out < (N + 15) / 16 ? rt_out : (int64_t)blockIdx.x * RT;
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL uint32_t* scales = (const TERN_GLOBAL uint32_t*)(packed + t5_plane_bytes(N, K));
    const TERN_GLOBAL u32x4* xg = (const TERN_GLOBAL u32x4*)x;
    const int pk = nwh * kTileK;                                     // k per half
    const int xrow_bytes = kI8 ? pk + 16 : (pk + 8) * 2;
    float* red = (float*)(smem + (size_t)M * xrow_bytes);           // [RT * nkt][NI][64]
    // chunk indices past the end store to a slot after the partials (the
    // second half is staged after the first units' partials are written)
    const int dummy = M * xrow_bytes + RT * nkt * NI * 64 * 4;

    const int row_chunks = (int)(K * (kI8 ? 1 : 2) / kChunkBytes);
    const int per_row = pk * (kI8 ? 1 : 2) / kChunkBytes;
    u32x4 xv[2][XC][kLoadsPerChunk];
    int xdst[XC];
    ChunkWalk cw((int)threadIdx.x, nthreads, per_row);
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const bool in = cw.q < M;                                    // chunk u = threadIdx.x + c * nthreads
        const int m = in ? cw.q : M - 1, cc = in ? cw.r : per_row - 1;
#pragma unroll
        for (int ph = 0; ph < 2; ++ph)
#pragma unroll
            for (int h = 0; h < kLoadsPerChunk; ++h)
                xv[ph][c][h] = xg[((int64_t)m * row_chunks + ph * per_row + cc) * kLoadsPerChunk + h];
        xdst[c] = in ? m * xrow_bytes + kChunkBytes * cc : dummy;
        cw.next();
    }
    __builtin_amdgcn_sched_barrier(0);
    Tile5 t[2];
    auto stage = [&](int ph) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            if constexpr (kI8) {
                u32x4 o0, o1;
                q_decoded_order(xv[ph][c][0], xv[ph][c][kLoadsPerChunk - 1], o0, o1);
                *(u32x4*)(smem + xdst[c]) = o0;
                *(u32x4*)(smem + xdst[c] + 16) = o1;
            } else {
                *(u32x4*)(smem + xdst[c]) = xv[ph][c][0];
            }
        }
    };
    const int mrow = r < M ? r : M - 1;
    const uint8_t* xrow = smem + mrow * xrow_bytes + (kI8 ? 32 : 64) * g;
    auto compute = [&](int i) {
        const int kt = lw + i * nwh;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kI8) {
            const uint8_t* qt = xrow + lw * kTileK;
            tile5_i8<16>(t[i], [&](int jj, int h) { return *(const u32x4*)(qt + kBlockK * jj + 16 * h); }, acc,
                         acc_dbg, N, M, rt_out * kTileRows + r, (int)(K >> 8), 2 * kt, g);
        } else {
            tile5_bf16<16>(t[i], (const uint16_t*)xrow + lw * kTileK, acc);
        }
#pragma unroll
        for (int q = 0; q < NI; ++q) red[((lrt * nkt + kt) * NI + q) * 64 + lane] = acc[q];
    };

    t[0] = load_tile5(words, scales, rt, lw, nkt, r, g);
    __builtin_amdgcn_sched_barrier(0);
    stage(0);
    __syncthreads();
    t[1] = load_tile5(words, scales, rt, lw + nwh, nkt, r, g);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __syncthreads();                       // every wave has read half 0
    stage(1);
    __syncthreads();
    compute(1);
    __syncthreads();

    const int lanes_used = M <= 4 ? 16 : (M <= 8 ? 32 : 64);
    for (int e = threadIdx.x; e < RT * NI * 64; e += nthreads) {
        const int l = e & 63, q = (e >> 6) % NI, et = (e >> 6) / NI;
        const int m = 4 * (l >> 4) + q, n = l & 15;
        const int64_t row = ((int64_t)blockIdx.x * RT + et) * kTileRows + n;
        if (l < lanes_used && m < M && row < N) {
            const float* pr = red + ((int64_t)et * nkt * NI + q) * 64 + l;
            float sum = 0.f;
            for (int kt = 0; kt < nkt; ++kt) sum += pr[kt * NI * 64];
            y[(int64_t)m * N + row] = kI8 ? s_x[m] * sum : sum;
        }
    }
}

// Any shape: one workgroup per row tile, its waves split the k-tiles
// round-robin, activations read from global memory (cached; int8 q is put
// in the decoded byte order in registers), partials summed in LDS in wave
// order.
template <bool kI8, int MT>
__global__ __launch_bounds__(512) void gemv5_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                    const void* __restrict__ x, const float* __restrict__ s_x,
                                                    int M, float* __restrict__ y, int32_t* __restrict__ acc_dbg)
{
    constexpr int NI = MT < 4 ? MT : 4;
    __shared__ float red[8 * NI * 64];
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nkt = (int)(K >> 9);
    const int64_t rt = blockIdx.x;
    const uint32_t* words = (const uint32_t*)packed;
    const uint32_t* scales = (const uint32_t*)(packed + t5_plane_bytes(N, K));
    const int mrow = r < M ? r : M - 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kt = wave; kt < nkt; kt += nw) {
        const Tile5 t = load_tile5(words, scales, rt, kt, nkt, r, g);
        if constexpr (kI8) {
            // this lane's four 32-byte slots of q, put in the decoded byte order in registers
            const int8_t* qr = (const int8_t*)x + (int64_t)mrow * K + (int64_t)kt * kTileK + 32 * g;
            u32x4 A[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                q_decoded_order(*(const u32x4*)(qr + kBlockK * j), *(const u32x4*)(qr + kBlockK * j + 16), A[j][0],
                                A[j][1]);
            tile5_i8<MT>(t, [&](int jj, int h) { return A[jj][h]; }, acc, acc_dbg, N, M, rt * kTileRows + r,
                         (int)(K >> 8), 2 * kt, g);
        } else {
            const uint16_t* xr = (const uint16_t*)x + (int64_t)mrow * K + 32 * g;
            tile5_bf16<MT>(t, xr + (int64_t)kt * kTileK, acc);
        }
    }
#pragma unroll
    for (int q = 0; q < NI; ++q) red[(wave * NI + q) * 64 + lane] = acc[q];
    __syncthreads();
    const int lanes_used = M <= 4 ? 16 : (M <= 8 ? 32 : 64);
    for (int e = threadIdx.x; e < NI * 64; e += blockDim.x) {
        const int l = e & 63, q = e >> 6;
        const int m = 4 * (l >> 4) + q, n = l & 15;
        const int64_t row = rt * kTileRows + n;
        if (l < lanes_used && m < M && row < N) {
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += red[(w * NI + q) * 64 + l];
            y[(int64_t)m * N + row] = kI8 ? s_x[m] * sum : sum;
        }
    }
}

// ------------------------------------------------------------------ launch

static unsigned t5_grid_for(int64_t items, int threads, int64_t cap)
{
    int64_t g = (items + threads - 1) / threads;
    if (g < 1) g = 1;
    return (unsigned)(g < cap ? g : cap);
}

hipError_t launch_pack5(const int8_t* lv, const float* s_lo, const float* s_hi, int64_t N, int64_t K,
                        uint8_t* packed, hipStream_t stream)
{
    const int64_t items = npad16(N) * (K / 256) * 8;
    pack5_kernel<<<t5_grid_for(items, 256, 65536), 256, 0, stream>>>(
        lv, s_lo, s_hi, N, K, (uint32_t*)packed, (float*)(packed + t5_plane_bytes(N, K)));
    return hipGetLastError();
}

template <bool kI8, int MT>
static hipError_t gemv5_oneshot_dispatch(const OneShot& c, hipStream_t stream, const uint8_t* packed, int64_t N,
                                         int64_t K, const void* x, const float* s_x, int M, float* y, int32_t* acc)
{
#define TERN5_CASE(UU, XX)                                                                                     \
    if (c.U == UU && c.XC == XX) {                                                                             \
        if (!oneshot_resident(gemv5_oneshot_kernel<kI8, MT, UU, XX>, c)) return hipErrorNotSupported;         \
        gemv5_oneshot_kernel<kI8, MT, UU, XX><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(     \
            packed, N, K, x, s_x, M, y, acc);                                                                  \
        return hipGetLastError();                                                                              \
    }
    TERN5_CASE(1, 1) TERN5_CASE(2, 1) TERN5_CASE(3, 1) TERN5_CASE(4, 1)
    TERN5_CASE(1, 2) TERN5_CASE(2, 2) TERN5_CASE(3, 2) TERN5_CASE(4, 2)
    TERN5_CASE(1, 4) TERN5_CASE(2, 4) TERN5_CASE(3, 4) TERN5_CASE(4, 4)
    if constexpr (MT == 16) {
        TERN5_CASE(1, 8) TERN5_CASE(2, 8) TERN5_CASE(3, 8) TERN5_CASE(4, 8)
    }
    if constexpr (MT == 16 && !kI8) {
        TERN5_CASE(1, 16) TERN5_CASE(2, 16) TERN5_CASE(3, 16)
    }
#undef TERN5_CASE
    return hipErrorNotSupported;
}

// the partials-over-x instances (bf16 rows above 8 whose x and partials do not fit side by side)
static hipError_t gemv5_reuse_dispatch(const OneShot& c, hipStream_t stream, const uint8_t* packed, int64_t N,
                                       int64_t K, const void* x, int M, float* y)
{
#define TERN5_REUSE_CASE(UU, XX)                                                                                \
    if (c.U == UU && c.XC == XX) {                                                                              \
        if (!oneshot_resident(gemv5_oneshot_kernel<false, 16, UU, XX, true>, c)) return hipErrorNotSupported;   \
        gemv5_oneshot_kernel<false, 16, UU, XX, true><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds,         \
                                                        stream>>>(packed, N, K, x, nullptr, M, y, nullptr);    \
        return hipGetLastError();                                                                               \
    }
    TERN5_REUSE_CASE(2, 8) TERN5_REUSE_CASE(3, 8) TERN5_REUSE_CASE(4, 8)
    TERN5_REUSE_CASE(2, 16) TERN5_REUSE_CASE(3, 16)
#undef TERN5_REUSE_CASE
    return hipErrorNotSupported;
}

// waves of U = 1..4 units per SIMD (registers: bf16 60, 77, 95-99 and
// 111-115 VGPRs, int8 68, 74, 90 and 106; the occupancy query has the last
// word)
bool gemv5_oneshot_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c)
{
    const OneShotShape s = i8 ? OneShotShape{K + 16, K, 32, {0, 7, 6, 5, 4}, 0, false}
                              : OneShotShape{(K + 8) * 2, 2 * K, 16, {0, 8, 6, 4, 4}, 0, true};
    return pick_oneshot(N, K, M, s, c);
}

// two-phase configuration (gemv5_phased_kernel); false when it does not
// apply.  One row tile per workgroup, two (bf16) when one tile's waves would
// each stage more than 8 chunks of a half of x (the 8B fused gate|up at
// M = 9..16, whose x leaves no room for a one-pass split).
bool gemv5_phased_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c)
{
    if (K % kTileK != 0 || M < 1 || M > 16 || N < 1) return false;
    const int64_t nkt = K / kTileK;
    if (nkt % 2 != 0 || nkt / 2 > 16 || nkt < 2) return false;
    const int64_t pk = nkt / 2 * kTileK;
    const int64_t chunks = M * pk * (i8 ? 1 : 2) / (i8 ? 32 : 16);
    for (int R = 1; R <= (i8 ? 1 : 2); ++R) {
        const int64_t nw = R * nkt / 2;
        if (nw > 16) break;
        const int64_t xc = (chunks + 64 * nw - 1) / (64 * nw);   // M / R (bf16) or M / 4 (int8)
        if (xc > (i8 ? 4 : 8)) continue;
        c.R = R;
        c.U = 2;
        c.nw = (int)nw;
        c.grid = ((N + 15) / 16 + R - 1) / R;
        c.rounds = true;
        c.XC = xc <= 1 ? 1 : (xc <= 2 ? 2 : (xc <= 4 ? 4 : 8));
        c.lds = (size_t)(M * (i8 ? pk + 16 : (pk + 8) * 2)) + (size_t)R * nkt * 4 * 64 * 4 + 32;   // + dummy
        return c.lds <= (size_t)kCuLds;
    }
    return false;
}

template <bool kI8>
static hipError_t launch_gemv5_phased(const uint8_t* packed, int64_t N, int64_t K, const void* x, const float* s_x,
                                      int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    OneShot c;
    if (!gemv5_phased_config(N, K, M, kI8, c)) return hipErrorNotSupported;
#define TERN5_PHASED_CASE(XX, RR)                                                                              \
    if (c.XC == XX && c.R == RR) {                                                                             \
        if (!oneshot_resident(gemv5_phased_kernel<kI8, XX, RR>, c)) return hipErrorNotSupported;              \
        gemv5_phased_kernel<kI8, XX, RR><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(          \
            packed, N, K, x, s_x, (int)M, y, acc);                                                             \
        return hipGetLastError();                                                                              \
    }
    TERN5_PHASED_CASE(1, 1) TERN5_PHASED_CASE(2, 1) TERN5_PHASED_CASE(4, 1)
    if constexpr (!kI8) {
        TERN5_PHASED_CASE(8, 1)
        TERN5_PHASED_CASE(8, 2)   // two row tiles: only above 8 chunks for one
    }
#undef TERN5_PHASED_CASE
    return hipErrorNotSupported;
}

template <bool kI8>
static hipError_t launch_gemv5(const uint8_t* packed, int64_t N, int64_t K, const void* x, const float* s_x,
                               int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    OneShot c;
    if (gemv5_oneshot_config(N, K, M, kI8, c)) {
        const int m = (int)M;
        // 8 activation chunks per thread are instantiated for MT = 16 only
        const bool wide = M > 4 || c.XC == 8;
        hipError_t e;
        // a partials-over-x configuration sized its LDS for that layout only
        if (c.reuse) e = gemv5_reuse_dispatch(c, stream, packed, N, K, x, m, y);
        else if (wide) e = gemv5_oneshot_dispatch<kI8, 16>(c, stream, packed, N, K, x, s_x, m, y, acc);
        else if (M == 1) e = gemv5_oneshot_dispatch<kI8, 1>(c, stream, packed, N, K, x, s_x, m, y, acc);
        else if (M == 2) e = gemv5_oneshot_dispatch<kI8, 2>(c, stream, packed, N, K, x, s_x, m, y, acc);
        else e = gemv5_oneshot_dispatch<kI8, 4>(c, stream, packed, N, K, x, s_x, m, y, acc);
        if (e != hipErrorNotSupported) return e;
    }
    {
        const hipError_t e = launch_gemv5_phased<kI8>(packed, N, K, x, s_x, M, y, acc, stream);
        if (e != hipErrorNotSupported) return e;
    }
    const int64_t nkt = K / kTileK;
    const int nw = nkt >= 8 ? 8 : (int)nkt;
    const dim3 grid((unsigned)((N + 15) / 16)), block(64 * nw);
    if (M == 1) gemv5_kernel<kI8, 1><<<grid, block, 0, stream>>>(packed, N, K, x, s_x, (int)M, y, acc);
    else if (M == 2) gemv5_kernel<kI8, 2><<<grid, block, 0, stream>>>(packed, N, K, x, s_x, (int)M, y, acc);
    else if (M <= 4) gemv5_kernel<kI8, 4><<<grid, block, 0, stream>>>(packed, N, K, x, s_x, (int)M, y, acc);
    else gemv5_kernel<kI8, 16><<<grid, block, 0, stream>>>(packed, N, K, x, s_x, (int)M, y, acc);
    return hipGetLastError();
}

hipError_t launch_gemv5_bf16(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                             hipStream_t stream)
{
    return launch_gemv5<false>(packed, N, K, x, nullptr, M, y, nullptr, stream);
}

hipError_t launch_gemv5_i8(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M,
                           float* y, int32_t* acc, hipStream_t stream)
{
    return launch_gemv5<true>(packed, N, K, q, s_x, M, y, acc, stream);
}

}  // namespace tern
