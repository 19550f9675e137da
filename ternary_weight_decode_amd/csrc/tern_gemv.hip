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
#include "tern_oneshot.h"
#include "tern_tile.h"

namespace tern {

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
__global__ __launch_bounds__(1024) void gemv_bf16_fast_kernel(const uint8_t* __restrict__ packed, int64_t N,
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
        ChunkWalk cw((int)threadIdx.x, (int)blockDim.x, per_row);
        for (int u = threadIdx.x; u < units; u += blockDim.x, cw.next())
            *(u32x4*)(xs + cw.q * xstride + 8 * cw.r) = *(const u32x4*)(x + (int64_t)cw.q * K + 8 * cw.r);
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

// One-pass path (K a multiple of 512, x in LDS, every workgroup resident at
// once): workgroup b owns R row tiles (b, b + G, ...) and its waves take the
// R*nkt (row tile, k-tile) units round-robin, U <= 4 per wave.  A wave
// requests its activations and its first unit, stages x, and then requests
// its remaining units before computing any, so no second memory latency is
// exposed.  Units are computed in order as they arrive; each leaves its fp32
// partial in LDS, and after one barrier every output is the sum of its row
// tile's partials in k-tile order (the result does not depend on the wave
// split).
//
// kI8 = false: bf16 activations, bf16 MFMA on weights decoded to 2t.
// kI8 = true:  int8 activations q with row scales s_x, int8 MFMA on weights
//              decoded to 64t; every block's exact int32 sum is scaled in
//              fp32 (and written to acc_dbg when it is given); y = s_x * sum.
// XC = activation chunks per thread (16 bytes of bf16, or 32 bytes of int8
// staged in the decoded byte order); the launcher checks that they cover x.
// kReuse: the partials overwrite x's LDS once every wave has computed (a
// second barrier; x and the partials need not fit side by side).
template <bool kI8, int MT, int U, int XC, bool kReuse = false>
__global__ __launch_bounds__(1024) void gemv_oneshot_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                            const void* __restrict__ x, const float* __restrict__ s_x,
                                                            int M, float* __restrict__ y,
                                                            int32_t* __restrict__ acc_dbg)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NI = MT < 4 ? MT : 4;
    constexpr int kChunkBytes = kI8 ? 32 : 16;
    constexpr int kLoadsPerChunk = kChunkBytes / 16;
    const int nthreads = blockDim.x, nw = nthreads >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nb = (int)(K >> 7), nkt = nb >> 2;
    const int nrt = (int)((N + 15) >> 4);
    // row tiles b, b + G, b + 2G, ... (G = grid): at any moment the
    // workgroups read neighbouring tiles, spread over all memory channels
    const int rt0 = (int)blockIdx.x;
    int G = (int)gridDim.x;
    // G comes from the dispatch's implicit arguments: read it together with
    // the kernel arguments, not after the unit search below needs it
    asm volatile("" : "+s"(G));
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
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
    // keep the activation loads ahead of the unit loads: waiting for them
    // must not wait for the weights
    __builtin_amdgcn_sched_barrier(0);
    // Unit j = wave + i*nw of this wave is (row tile lrt, k-tile kt) with
    // j = lrt*nkt + kt, found by subtraction (j < 64: at most R - 1 steps, in
    // scalar registers) so that no division sits between the kernel's start
    // and its first loads.  A unit past the workgroup's last row tile loads
    // k-tile nkt - 1 of its first row tile; its partial goes to the spare slot.
    int ulrt[U], ukt[U];
    bool uok[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        int lrt = 0, kt = wave + i * nw;
        while (kt >= nkt) {
            kt -= nkt;
            ++lrt;
        }
        uok[i] = rt0 + lrt * G < nrt;
        ulrt[i] = uok[i] ? lrt : 0;
        ukt[i] = uok[i] ? kt : nkt - 1;
    }
    PlaneTile t[U];
    // plane words first: the scale region's offset is computed after they are requested
    auto load_words = [&](int i) {
        const int64_t wb = tile_word_base(rt0 + ulrt[i] * G, ukt[i], nb);
        t[i].nz = ld_nt16(words + wb + (int64_t)(g * 16 + r) * 4);
        t[i].sg = ld_nt16(words + wb + (int64_t)((4 + g) * 16 + r) * 4);
    };
    auto load_scales = [&](int i) {
        const TERN_GLOBAL uint16_t* scales = (const TERN_GLOBAL uint16_t*)(packed + scale_region_offset(N, K));
        t[i].sc = ld_nt8(scales + tile_scale_base(rt0 + ulrt[i] * G, ukt[i], nb) + r * 4);
    };
    auto load_unit = [&](int i) {
        load_words(i);
        load_scales(i);
    };
    // Only the first unit is requested before the activations are staged:
    // requests queue in the memory system in issue order, and x (needed by
    // every unit) would otherwise wait behind all of the weights.  The
    // other units are requested right after the barrier and stream in while
    // the first one is computed.
    load_words(0);
    __builtin_amdgcn_sched_barrier(0);
    load_scales(0);
    __builtin_amdgcn_sched_barrier(0);
    int rn = 0;                                             // row tiles of this workgroup (at most R)
    for (int rt = rt0; rt < nrt; rt += G) ++rn;
    const int units = rn * nkt;
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        if constexpr (kI8) {
            // 32 bytes of q in the byte order of the decoded weights
            const uint32_t Q[8] = {xv[c][0][0], xv[c][0][1], xv[c][0][2], xv[c][0][3],
                                   xv[c][1][0], xv[c][1][1], xv[c][1][2], xv[c][1][3]};
            u32x4 o0, o1;
#pragma unroll
            for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
            for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
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
        __builtin_amdgcn_sched_barrier(0);   // unit i's loads complete before unit i+1's
    }

    const int mrow = r < M ? r : M - 1;
    const uint8_t* xrow = smem + mrow * xrow_bytes + (kI8 ? 32 : 64) * g;
    // every unit is computed (a unit past the end repeats a real one and
    // leaves its partial in the spare slot after the real ones), so no load
    // is consumed behind a branch
    f32x4 keep[kReuse ? U : 1];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int lrt = ulrt[i], kt = ukt[i];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kI8) {
            const int64_t n = (int64_t)(rt0 + lrt * G) * kTileRows + r;
#pragma unroll
            for (int bq = 0; bq < 4; ++bq) {
                u32x4 B[2];
                decode_i8(t[i].nz[bq], t[i].sg[bq], B);
                const uint8_t* qa = xrow + (kt * 4 + bq) * kBlockK;
                i32x4 d = {0, 0, 0, 0};
                d = mfma_i8(*(const u32x4*)(qa), B[0], d);
                d = mfma_i8(*(const u32x4*)(qa + 16), B[1], d);
                const float sc = tile_scale(t[i], bq) * (1.0f / 64.0f);   // decoded weights are 64*t
#pragma unroll
                for (int q = 0; q < NI; ++q) acc[q] = __builtin_fmaf(sc, (float)d[q], acc[q]);
                if (acc_dbg != nullptr && uok[i]) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int m = 4 * g + q;
                        if (m < M && n < N) acc_dbg[((int64_t)m * N + n) * nb + kt * 4 + bq] = d[q] >> 6;
                    }
                }
            }
        } else {
            bf16_tile<MT>(t[i], (const uint16_t*)xrow + kt * kTileK, 4, acc);
        }
        if constexpr (kReuse) {
            keep[i] = acc;
        } else {
            const int slot = uok[i] ? lrt * nkt + kt : units;
#pragma unroll
            for (int q = 0; q < NI; ++q) red[(slot * NI + q) * 64 + lane] = acc[q];   // all lanes: no branch
        }
        __builtin_amdgcn_sched_barrier(0);   // unit i+1's decode waits for its own loads only
    }
    if constexpr (kReuse) {
        __syncthreads();                     // every wave is done with x
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int slot = uok[i] ? ulrt[i] * nkt + ukt[i] : units;
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

// M = 1, bf16 activations: the one-pass split (units of 16 rows x 512 k, R
// row tiles per workgroup, U units per wave, partials summed in k-tile
// order), but every wave stages only the activations of its own units.  A
// unit's 512 bf16 of x are one 16-byte chunk per lane, requested just before
// the unit's plane words and written to the wave's own LDS slot, so no
// workgroup barrier stands between the loads and the compute: a wave
// computes a unit as soon as its own slice and planes have arrived.  Only
// the partial sums meet at a barrier.
template <int U>
__global__ __launch_bounds__(1024) void gemv_m1_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                       const uint16_t* __restrict__ x, float* __restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int kSlice = kTileK * 2;                                // bytes of x per unit
    const int nw = (int)(blockDim.x >> 6);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nb = (int)(K >> 7), nkt = nb >> 2;
    const int nrt = (int)((N + 15) >> 4);
    const int rt0 = (int)blockIdx.x;
    int G = (int)gridDim.x;
    asm volatile("" : "+s"(G));                                       // read with the kernel arguments
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL u32x4* xg = (const TERN_GLOBAL u32x4*)x;
    uint8_t* xs = smem + (size_t)wave * U * kSlice;                   // this wave's slices
    float* red = (float*)(smem + (size_t)nw * U * kSlice);            // [unit + 1 spare][64]

    // unit positions by subtraction, as in the one-pass kernel
    int ulrt[U], ukt[U];
    bool uok[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        int lrt = 0, kt = wave + i * nw;
        while (kt >= nkt) {
            kt -= nkt;
            ++lrt;
        }
        uok[i] = rt0 + lrt * G < nrt;
        ulrt[i] = uok[i] ? lrt : 0;
        ukt[i] = uok[i] ? kt : nkt - 1;
    }
    PlaneTile t[U];
    u32x4 xv[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        xv[i] = xg[ukt[i] * (kSlice / 16) + lane];
        const int64_t wb = tile_word_base(rt0 + ulrt[i] * G, ukt[i], nb);
        t[i].nz = ld_nt16(words + wb + (int64_t)(g * 16 + r) * 4);
        t[i].sg = ld_nt16(words + wb + (int64_t)((4 + g) * 16 + r) * 4);
        __builtin_amdgcn_sched_barrier(0);
    }
    const TERN_GLOBAL uint16_t* scales = (const TERN_GLOBAL uint16_t*)(packed + scale_region_offset(N, K));
#pragma unroll
    for (int i = 0; i < U; ++i)
        t[i].sc = ld_nt8(scales + tile_scale_base(rt0 + ulrt[i] * G, ukt[i], nb) + r * 4);
    __builtin_amdgcn_sched_barrier(0);
    int rn = 0;                                                       // row tiles of this workgroup
    for (int rt = rt0; rt < nrt; rt += G) ++rn;
    const int units = rn * nkt;

#pragma unroll
    for (int i = 0; i < U; ++i) {
        // a wave's LDS accesses run in order: its own write is seen by its reads below
        *(u32x4*)(xs + i * kSlice + 16 * lane) = xv[i];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        bf16_tile<1>(t[i], (const uint16_t*)(xs + i * kSlice + 64 * g), 4, acc);
        const int slot = uok[i] ? ulrt[i] * nkt + ukt[i] : units;
        red[slot * 64 + lane] = acc[0];
        __builtin_amdgcn_sched_barrier(0);   // unit i+1's work waits for its own loads only
    }
    __syncthreads();

    for (int e = threadIdx.x; e < rn * 16; e += (int)blockDim.x) {
        const int n = e & 15, lrt = e >> 4;
        const int64_t row = (int64_t)(rt0 + lrt * G) * kTileRows + n;
        if (row < N) {
            const float* pr = red + (int64_t)lrt * nkt * 64 + n;
            float sum = 0.f;
            for (int kt = 0; kt < nkt; ++kt) sum += pr[kt * 64];
            y[row] = sum;
        }
    }
}

// Small M (2..8), bf16 activations, one row tile per workgroup: the M = 1
// kernel's per-wave activation slices for MR rows (MR = 2, 4 or 8 >= M; a
// row past M repeats row M-1).  A unit's slice is MR rows of 512 bf16, one
// 16-byte chunk per lane and row, rows 1040 bytes apart in LDS so that the A
// reads of 16 rows fall in different banks.  With one row tile per workgroup
// every wave's k-tiles are its own: the slices load the bytes the workgroup
// staging did, and no workgroup barrier stands before the compute.
template <int MT, int U>
__global__ __launch_bounds__(1024) void gemv_slices_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                           const uint16_t* __restrict__ x, int M,
                                                           float* __restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NI = MT < 4 ? MT : 4;
    constexpr int MR = MT == 16 ? 8 : MT;                              // staged rows
    constexpr int kRowB = kTileK * 2 + 16;                            // bytes per staged row
    constexpr int kSlice = MR * kRowB;                                // bytes per unit
    const int nw = (int)(blockDim.x >> 6);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nb = (int)(K >> 7), nkt = nb >> 2;
    const int64_t rt = blockIdx.x;
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL u32x4* xg = (const TERN_GLOBAL u32x4*)x;
    uint8_t* xs = smem + (size_t)wave * U * kSlice;                   // this wave's slices
    float* red = (float*)(smem + (size_t)nw * U * kSlice);            // [nkt + 1 spare][NI][64]
    const int row_chunks = (int)(K >> 3);                              // 16-byte chunks per row of x

    int ukt[U];
    bool uok[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int kt = wave + i * nw;
        uok[i] = kt < nkt;
        ukt[i] = uok[i] ? kt : nkt - 1;
    }
    PlaneTile t[U];
    u32x4 xv[U][MR];
#pragma unroll
    for (int i = 0; i < U; ++i) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int mr = m < M ? m : M - 1;
            xv[i][m] = xg[mr * row_chunks + ukt[i] * (kTileK / 8) + lane];
        }
        const int64_t wb = tile_word_base(rt, ukt[i], nb);
        t[i].nz = ld_nt16(words + wb + (int64_t)(g * 16 + r) * 4);
        t[i].sg = ld_nt16(words + wb + (int64_t)((4 + g) * 16 + r) * 4);
        __builtin_amdgcn_sched_barrier(0);
    }
    const TERN_GLOBAL uint16_t* scales = (const TERN_GLOBAL uint16_t*)(packed + scale_region_offset(N, K));
#pragma unroll
    for (int i = 0; i < U; ++i) t[i].sc = ld_nt8(scales + tile_scale_base(rt, ukt[i], nb) + r * 4);
    __builtin_amdgcn_sched_barrier(0);

    const int mrow = r < M ? r : M - 1;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        // a wave's LDS accesses run in order: its own writes are seen by its reads below
#pragma unroll
        for (int m = 0; m < MR; ++m) *(u32x4*)(xs + i * kSlice + m * kRowB + 16 * lane) = xv[i][m];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        bf16_tile<MT>(t[i], (const uint16_t*)(xs + i * kSlice + mrow * kRowB + 64 * g), 4, acc);
        const int slot = uok[i] ? ukt[i] : nkt;
#pragma unroll
        for (int q = 0; q < NI; ++q) red[(slot * NI + q) * 64 + lane] = acc[q];
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    const int lanes_used = M <= 4 ? 16 : 32;
    for (int e = threadIdx.x; e < NI * 64; e += (int)blockDim.x) {
        const int l = e & 63, q = e >> 6;
        const int m = 4 * (l >> 4) + q, n = l & 15;
        const int64_t row = rt * kTileRows + n;
        if (l < lanes_used && m < M && row < N) {
            float sum = 0.f;
            for (int kt = 0; kt < nkt; ++kt) sum += red[(kt * NI + q) * 64 + l];
            y[(int64_t)m * N + row] = sum;
        }
    }
}

// Two-phase variant of the one-pass kernel for activations too large for
// LDS (large K at M >= 5 bf16, or M >= 13 int8): RT row tiles per workgroup
// (1, or 2 when one tile's waves would each stage more than 8 activation
// chunks), nkt / 2 waves per row tile with two units each, unit i of every
// wave in half i of K.  Both halves of x are loaded into registers up front
// (first in the memory queue, as in the one-pass kernel); half 0 is staged
// and its units computed, then half 1 replaces it in LDS.  Partials are summed
// in k-tile order (deterministic).  16 MFMA activation rows (any M <= 16).
template <bool kI8, int XC, int RT>
__global__ __launch_bounds__(1024) void gemv_phased_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
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
    const int nb = (int)(K >> 7), nkt = nb >> 2;
    const int nwh = nw / RT;                                          // waves per row tile (nkt / 2)
    const int lrt = wave / nwh, lw = wave - lrt * nwh;               // this wave's row tile and local wave
    // rows of row tile rt_out; a tile past the last one (odd row-tile count)
    // loads the workgroup's first tile and stores nothing
    const int64_t rt_out = (int64_t)blockIdx.x * RT + lrt;
    const int64_t rt = rt_out < (N + 15) / 16 ? rt_out : (int64_t)blockIdx.x * RT;
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL uint16_t* scales = (const TERN_GLOBAL uint16_t*)(packed + scale_region_offset(N, K));
    const TERN_GLOBAL u32x4* xg = (const TERN_GLOBAL u32x4*)x;
    const int pk = nwh * kTileK;                                     // k per half
    const int xrow_bytes = kI8 ? pk + 16 : (pk + 8) * 2;             // staged bytes per activation row
    float* red = (float*)(smem + (size_t)M * xrow_bytes);           // [RT * nkt + 1 spare][NI][64]
    // chunk indices past the end store to a dummy slot after the partials:
    // the second half is staged after the first units' partials are written
    const int dummy = M * xrow_bytes + (RT * nkt + 1) * NI * 64 * 4;

    const int row_chunks = (int)(K * (kI8 ? 1 : 2) / kChunkBytes);  // chunks per activation row in memory
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
    PlaneTile t[2];
    auto load_unit = [&](int i) {
        const int kt = lw + i * nwh;
        const int64_t wb = tile_word_base(rt, kt, nb);
        const int64_t sb = tile_scale_base(rt, kt, nb);
        t[i].nz = ld_nt16(words + wb + (int64_t)(g * 16 + r) * 4);
        t[i].sg = ld_nt16(words + wb + (int64_t)((4 + g) * 16 + r) * 4);
        t[i].sc = ld_nt8(scales + sb + r * 4);
    };
    auto stage = [&](int ph) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            if constexpr (kI8) {
                const uint32_t Q[8] = {xv[ph][c][0][0], xv[ph][c][0][1], xv[ph][c][0][2], xv[ph][c][0][3],
                                       xv[ph][c][1][0], xv[ph][c][1][1], xv[ph][c][1][2], xv[ph][c][1][3]};
                u32x4 o0, o1;
#pragma unroll
                for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
                for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
                *(u32x4*)(smem + xdst[c]) = o0;
                *(u32x4*)(smem + xdst[c] + 16) = o1;
            } else {
                *(u32x4*)(smem + xdst[c]) = xv[ph][c][0];
            }
        }
    };
    const int mrow = r < M ? r : M - 1;
    const uint8_t* xrow = smem + mrow * xrow_bytes + (kI8 ? 32 : 64) * g;
    // unit i of this wave: k-tile lw + i*nwh of its row tile, at local k-tile lw of half i
    auto compute = [&](int i) {
        const int kt = lw + i * nwh;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kI8) {
            const int64_t n = rt_out * kTileRows + r;
#pragma unroll
            for (int bq = 0; bq < 4; ++bq) {
                u32x4 B[2];
                decode_i8(t[i].nz[bq], t[i].sg[bq], B);
                const uint8_t* qa = xrow + (lw * 4 + bq) * kBlockK;
                i32x4 d = {0, 0, 0, 0};
                d = mfma_i8(*(const u32x4*)(qa), B[0], d);
                d = mfma_i8(*(const u32x4*)(qa + 16), B[1], d);
                const float sc = tile_scale(t[i], bq) * (1.0f / 64.0f);   // decoded weights are 64*t
#pragma unroll
                for (int q = 0; q < NI; ++q) acc[q] = __builtin_fmaf(sc, (float)d[q], acc[q]);
                if (acc_dbg != nullptr) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int m = 4 * g + q;
                        if (m < M && n < N) acc_dbg[((int64_t)m * N + n) * nb + kt * 4 + bq] = d[q] >> 6;
                    }
                }
            }
        } else {
            bf16_tile<16>(t[i], (const uint16_t*)xrow + lw * kTileK, 4, acc);
        }
#pragma unroll
        for (int q = 0; q < NI; ++q) red[((lrt * nkt + kt) * NI + q) * 64 + lane] = acc[q];
    };

    load_unit(0);
    __builtin_amdgcn_sched_barrier(0);
    stage(0);
    __syncthreads();
    load_unit(1);
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

// Three-phase variant for bf16 activations of up to 16 rows whose halves of K
// still exceed LDS (the 8B down projection, K = 12288, at M = 9..16): one row
// tile per workgroup and nkt / 3 waves with three units each, unit i of every
// wave in third i of K.  The first two thirds of x are loaded into two
// register sets up front; each third is staged into LDS in turn, and the set
// the first came from is refilled with the last third while the first is
// computed.  The weights stream once for all M rows.  Partials are summed in
// k-tile order (deterministic).
template <int XC>
__global__ __launch_bounds__(512) void gemv_phased3_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                           const uint16_t* __restrict__ x, int M,
                                                           float* __restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NI = 4;
    const int nthreads = blockDim.x, nw = nthreads >> 6;   // nw = nkt / 3
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nb = (int)(K >> 7), nkt = nb >> 2;
    const int64_t rt = blockIdx.x;
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL uint16_t* scales = (const TERN_GLOBAL uint16_t*)(packed + scale_region_offset(N, K));
    const TERN_GLOBAL u32x4* xg = (const TERN_GLOBAL u32x4*)x;
    const int pk = nw * kTileK;                                      // k per third
    const int xrow_bytes = (pk + 8) * 2;                             // staged bytes per activation row
    float* red = (float*)(smem + (size_t)M * xrow_bytes);            // [nkt][NI][64]
    // chunk indices past the end store to a dummy slot after the partials
    const int dummy = M * xrow_bytes + nkt * NI * 64 * 4;

    const int row_chunks = (int)(K * 2 / 16);                        // 16-byte chunks per activation row
    const int per_row = pk * 2 / 16;
    int xsrc[XC], xdst[XC];
    ChunkWalk cw((int)threadIdx.x, nthreads, per_row);
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const bool in = cw.q < M;                                    // chunk u = threadIdx.x + c * nthreads
        const int m = in ? cw.q : M - 1, cc = in ? cw.r : per_row - 1;
        xsrc[c] = m * row_chunks + cc;
        xdst[c] = in ? m * xrow_bytes + 16 * cc : dummy;
        cw.next();
    }
    u32x4 xa[XC], xb[XC];
    auto load_x = [&](int ph, u32x4 (&v)[XC]) {
#pragma unroll
        for (int c = 0; c < XC; ++c) v[c] = xg[xsrc[c] + ph * per_row];
    };
    auto stage = [&](const u32x4 (&v)[XC]) {
#pragma unroll
        for (int c = 0; c < XC; ++c) *(u32x4*)(smem + xdst[c]) = v[c];
    };
    PlaneTile t[3];
    auto load_unit = [&](int i) {
        const int kt = wave + i * nw;
        const int64_t wb = tile_word_base(rt, kt, nb);
        const int64_t sb = tile_scale_base(rt, kt, nb);
        t[i].nz = ld_nt16(words + wb + (int64_t)(g * 16 + r) * 4);
        t[i].sg = ld_nt16(words + wb + (int64_t)((4 + g) * 16 + r) * 4);
        t[i].sc = ld_nt8(scales + sb + r * 4);
    };
    const int mrow = r < M ? r : M - 1;
    const uint8_t* xrow = smem + mrow * xrow_bytes + 64 * g;
    auto compute = [&](int i) {
        const int kt = wave + i * nw;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        bf16_tile<16>(t[i], (const uint16_t*)xrow + wave * kTileK, 4, acc);
#pragma unroll
        for (int q = 0; q < NI; ++q) red[(kt * NI + q) * 64 + lane] = acc[q];
    };

    load_x(0, xa);
    load_x(1, xb);
    __builtin_amdgcn_sched_barrier(0);
    load_unit(0);
    __builtin_amdgcn_sched_barrier(0);
    stage(xa);
    __syncthreads();
    load_unit(1);
    __builtin_amdgcn_sched_barrier(0);
    load_unit(2);
    __builtin_amdgcn_sched_barrier(0);
    load_x(2, xa);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __syncthreads();                       // every wave has read the first third
    stage(xb);
    __syncthreads();
    compute(1);
    __syncthreads();
    stage(xa);
    __syncthreads();
    compute(2);
    __syncthreads();

    const int lanes_used = M <= 4 ? 16 : (M <= 8 ? 32 : 64);
    for (int e = threadIdx.x; e < NI * 64; e += nthreads) {
        const int l = e & 63, q = e >> 6;
        const int m = 4 * (l >> 4) + q, n = l & 15;
        const int64_t row = rt * kTileRows + n;
        if (l < lanes_used && m < M && row < N) {
            float sum = 0.f;
            for (int kt = 0; kt < nkt; ++kt) sum += red[(kt * NI + q) * 64 + l];
            y[(int64_t)m * N + row] = sum;
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

static constexpr int64_t kFastLds = kCuLds;     // LDS budget of the fast path (all of a CU's LDS)

// waves per workgroup and k-tiles in flight per wave for the fast path
// (nw never exceeds the number of k-tiles, so every wave works on every row
// tile).  Measured on the 8B shapes at M = 1 (hipGraph of 36 launches, cold
// weights): one tile in flight per wave beats deeper rings (fewer registers,
// more resident waves), and 16 waves per row tile beat 8 and 12 on the
// 24-k-tile down projection (6.4 us vs 6.9 / 7.5 us).
static void pick_fast(int64_t nkt, int& nw, int& tpw)
{
    nw = nkt >= 16 ? 16 : (nkt >= 8 ? 8 : (nkt >= 4 ? 4 : (int)(nkt < 1 ? 1 : nkt)));
    tpw = 1;
}

// LDS of the bf16 persistent fast path: all of x plus two partial rows per wave
static size_t fast_lds_bytes(int64_t K, int64_t M)
{
    int nw, tpw;
    pick_fast((K / kBlockK + 3) / 4, nw, tpw);
    const int ni = M == 1 ? 1 : (M == 2 ? 2 : 4);   // accumulator rows of the instance (NI)
    return (size_t)M * (K + 8) * 2 + (size_t)2 * nw * ni * 64 * 4;
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
    (void)tpw;   // one tile in flight per wave (pick_fast)
    return launch_fast<MT, 1>(nw, lds, stream, packed, N, K, x, M, y);
}

template <bool kI8, int MT>
static hipError_t oneshot_dispatch(const OneShot& c, hipStream_t stream, const uint8_t* packed, int64_t N, int64_t K,
                                   const void* x, const float* s_x, int M, float* y, int32_t* acc)
{
#define TERN_ONESHOT_CASE(UU, XX)                                                                              \
    if (c.U == UU && c.XC == XX) {                                                                             \
        if (!oneshot_resident(gemv_oneshot_kernel<kI8, MT, UU, XX>, c)) return hipErrorNotSupported;          \
        gemv_oneshot_kernel<kI8, MT, UU, XX><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(      \
            packed, N, K, x, s_x, M, y, acc);                                                                  \
        return hipGetLastError();                                                                              \
    }
    TERN_ONESHOT_CASE(1, 1) TERN_ONESHOT_CASE(2, 1) TERN_ONESHOT_CASE(3, 1) TERN_ONESHOT_CASE(4, 1)
    TERN_ONESHOT_CASE(1, 2) TERN_ONESHOT_CASE(2, 2) TERN_ONESHOT_CASE(3, 2) TERN_ONESHOT_CASE(4, 2)
    TERN_ONESHOT_CASE(1, 4) TERN_ONESHOT_CASE(2, 4) TERN_ONESHOT_CASE(3, 4) TERN_ONESHOT_CASE(4, 4)
    if constexpr (MT == 16) {
        TERN_ONESHOT_CASE(1, 8) TERN_ONESHOT_CASE(2, 8) TERN_ONESHOT_CASE(3, 8) TERN_ONESHOT_CASE(4, 8)
    }
    if constexpr (MT == 16 && !kI8) {
        TERN_ONESHOT_CASE(1, 16) TERN_ONESHOT_CASE(2, 16) TERN_ONESHOT_CASE(3, 16)
    }
#undef TERN_ONESHOT_CASE
    return hipErrorNotSupported;
}

// the partials-over-x instances: bf16 rows above 8 whose x and partials do not fit side by side
static hipError_t oneshot_reuse_dispatch(const OneShot& c, hipStream_t stream, const uint8_t* packed, int64_t N,
                                         int64_t K, const void* x, int M, float* y)
{
#define TERN_REUSE_CASE(UU, XX)                                                                                 \
    if (c.U == UU && c.XC == XX) {                                                                              \
        if (!oneshot_resident(gemv_oneshot_kernel<false, 16, UU, XX, true>, c)) return hipErrorNotSupported;    \
        gemv_oneshot_kernel<false, 16, UU, XX, true><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>( \
            packed, N, K, x, nullptr, M, y, nullptr);                                                           \
        return hipGetLastError();                                                                               \
    }
    TERN_REUSE_CASE(2, 8) TERN_REUSE_CASE(3, 8) TERN_REUSE_CASE(4, 8)
    TERN_REUSE_CASE(2, 16) TERN_REUSE_CASE(3, 16)
#undef TERN_REUSE_CASE
    return hipErrorNotSupported;
}

// The ternary instances with M <= 4 use 56-65, 62-70, 75-81 and 87-91 VGPRs
// for U = 1..4 (the occupancy query has the last word).
static OneShotShape oneshot_shape(int64_t K, bool i8)
{
    return OneShotShape{i8 ? K + 16 : (K + 8) * 2, i8 ? K : 2 * K, i8 ? 32 : 16, {0, 8, 7, 6, 5},
                        i8 ? 0 : kTileK * 2, !i8};
}

// the one-pass path for M <= 16 when it applies; hipErrorNotSupported otherwise
bool gemv_oneshot_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c)
{
    return pick_oneshot(N, K, M, oneshot_shape(K, i8), c);
}

static hipError_t m1_dispatch(const OneShot& c, hipStream_t stream, const uint8_t* packed, int64_t N, int64_t K,
                              const uint16_t* x, float* y)
{
#define TERN_M1_CASE(UU)                                                                                           \
    if (c.U == UU) {                                                                                               \
        if (!oneshot_resident(gemv_m1_kernel<UU>, c)) return hipErrorNotSupported;                                 \
        gemv_m1_kernel<UU><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(packed, N, K, x, y);        \
        return hipGetLastError();                                                                                  \
    }
    TERN_M1_CASE(1) TERN_M1_CASE(2) TERN_M1_CASE(3) TERN_M1_CASE(4)
#undef TERN_M1_CASE
    return hipErrorNotSupported;
}

template <int MT>
static hipError_t slices_dispatch(const OneShot& c, hipStream_t stream, const uint8_t* packed, int64_t N, int64_t K,
                                  const uint16_t* x, int M, float* y)
{
#define TERN_SLICES_CASE(UU)                                                                                       \
    if (c.U == UU) {                                                                                               \
        if (!oneshot_resident(gemv_slices_kernel<MT, UU>, c)) return hipErrorNotSupported;                         \
        gemv_slices_kernel<MT, UU><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(packed, N, K, x, M, \
                                                                                              y);                  \
        return hipGetLastError();                                                                                  \
    }
    TERN_SLICES_CASE(1) TERN_SLICES_CASE(2)
#undef TERN_SLICES_CASE
    return hipErrorNotSupported;
}

static hipError_t launch_oneshot(bool i8, const uint8_t* packed, int64_t N, int64_t K, const void* x, const float* s_x,
                                 int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    OneShot c;
    if (!pick_oneshot(N, K, M, oneshot_shape(K, i8), c)) return hipErrorNotSupported;
    if (c.reuse) return oneshot_reuse_dispatch(c, stream, packed, N, K, x, (int)M, y);
    if (!i8 && M == 1) return m1_dispatch(c, stream, packed, N, K, (const uint16_t*)x, y);
    if (!i8 && M <= 8 && c.R == 1 && c.U <= 2) {
        // per-wave slices (the picker sized LDS for them)
        const uint16_t* xb = (const uint16_t*)x;
        if (M == 2) return slices_dispatch<2>(c, stream, packed, N, K, xb, (int)M, y);
        if (M <= 4) return slices_dispatch<4>(c, stream, packed, N, K, xb, (int)M, y);
        return slices_dispatch<16>(c, stream, packed, N, K, xb, (int)M, y);
    }
    const int m = (int)M;
    // 8 activation chunks per thread are instantiated for the MT = 16 kernel
    // only, which computes the same rows as MT = 4 (4 per lane group)
    const bool wide = M > 4 || c.XC == 8;
    if (!i8) {
        if (wide) return oneshot_dispatch<false, 16>(c, stream, packed, N, K, x, s_x, m, y, acc);
        if (M == 1) return oneshot_dispatch<false, 1>(c, stream, packed, N, K, x, s_x, m, y, acc);
        if (M == 2) return oneshot_dispatch<false, 2>(c, stream, packed, N, K, x, s_x, m, y, acc);
        return oneshot_dispatch<false, 4>(c, stream, packed, N, K, x, s_x, m, y, acc);
    }
    if (wide) return oneshot_dispatch<true, 16>(c, stream, packed, N, K, x, s_x, m, y, acc);
    if (M == 1) return oneshot_dispatch<true, 1>(c, stream, packed, N, K, x, s_x, m, y, acc);
    if (M == 2) return oneshot_dispatch<true, 2>(c, stream, packed, N, K, x, s_x, m, y, acc);
    return oneshot_dispatch<true, 4>(c, stream, packed, N, K, x, s_x, m, y, acc);
}

// Two-phase configuration (gemv_phased_kernel): one row tile per workgroup,
// nkt / 2 waves, half of x in LDS at a time; false when it does not apply.
// R = 1 row tile per workgroup; R = 2 (bf16) when one tile's nkt / 2 waves
// would each stage more than 8 chunks of a half of x and x does not fit the
// persistent fast path either (K = 8192 at M = 9..15, which otherwise runs as
// two row-half calls that read the weights twice).  Where the fast path fits
// it is the faster one: 8B fused gate|up at M = 16, 14.1 us against 15.3 us
// with two row tiles.
static bool pick_phased(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c)
{
    if (K % kTileK != 0 || M < 1 || M > 16 || N < 1) return false;
    const int64_t nkt = K / kTileK;
    if (nkt % 2 != 0 || nkt / 2 > 16 || nkt < 2) return false;
    const int64_t pk = nkt / 2 * kTileK;
    const int64_t chunk = i8 ? 32 : 16;
    const int64_t chunks = M * pk * (i8 ? 1 : 2) / chunk;
    const int rmax = i8 || fast_lds_bytes(K, M) <= (size_t)kFastLds ? 1 : 2;
    for (int R = 1; R <= rmax; ++R) {
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
        c.lds = (size_t)(M * (i8 ? pk + 16 : (pk + 8) * 2)) + (size_t)(R * nkt + 1) * 4 * 64 * 4 + 32;   // + dummy
        return c.lds <= (size_t)kCuLds;
    }
    return false;
}

template <bool kI8>
static hipError_t launch_phased(const uint8_t* packed, int64_t N, int64_t K, const void* x, const float* s_x,
                                int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    OneShot c;
    if (!pick_phased(N, K, M, kI8, c)) return hipErrorNotSupported;
#define TERN_PHASED_CASE(XX, RR)                                                                      \
    if (c.XC == XX && c.R == RR) {                                                                    \
        if (!oneshot_resident(gemv_phased_kernel<kI8, XX, RR>, c)) return hipErrorNotSupported;       \
        gemv_phased_kernel<kI8, XX, RR><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(  \
            packed, N, K, x, s_x, (int)M, y, acc);                                                    \
        return hipGetLastError();                                                                     \
    }
    TERN_PHASED_CASE(1, 1) TERN_PHASED_CASE(2, 1) TERN_PHASED_CASE(4, 1)
    if constexpr (!kI8) {
        TERN_PHASED_CASE(8, 1)   // int8 needs M / 4 <= 4 chunks per thread
        TERN_PHASED_CASE(8, 2)   // two row tiles: only above 8 chunks for one
    }
#undef TERN_PHASED_CASE
    return hipErrorNotSupported;
}

bool gemv_phased_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c)
{
    return pick_phased(N, K, M, i8, c);
}

// Three-phase configuration (gemv_phased3_kernel, bf16): one row tile per
// workgroup, nkt / 3 waves of three units, a third of x in LDS at a time.
static bool pick_phased3(int64_t N, int64_t K, int64_t M, OneShot& c)
{
    if (K % kTileK != 0 || M < 1 || M > 16 || N < 1) return false;
    const int64_t nkt = K / kTileK;
    if (nkt % 3 != 0 || nkt / 3 > 8 || nkt < 3) return false;
    c.R = 1;
    c.U = 3;
    c.nw = (int)(nkt / 3);
    c.grid = (N + 15) / 16;
    c.rounds = true;
    const int64_t pk = c.nw * kTileK;
    const int64_t xc = (M * pk * 2 / 16 + 64 * c.nw - 1) / (64 * c.nw);
    if (xc > 16) return false;
    c.XC = xc <= 4 ? 4 : (xc <= 8 ? 8 : 16);
    c.lds = (size_t)(M * (pk + 8) * 2) + (size_t)nkt * 4 * 64 * 4 + 16;   // + dummy slot
    return c.lds <= (size_t)kCuLds;
}

bool gemv_phased3_config(int64_t N, int64_t K, int64_t M, OneShot& c) { return pick_phased3(N, K, M, c); }

static hipError_t launch_phased3(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                                 hipStream_t stream)
{
    OneShot c;
    if (!pick_phased3(N, K, M, c)) return hipErrorNotSupported;
#define TERN_PHASED3_CASE(XX)                                                                            \
    if (c.XC == XX) {                                                                                    \
        if (!oneshot_resident(gemv_phased3_kernel<XX>, c)) return hipErrorNotSupported;                  \
        gemv_phased3_kernel<XX><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(packed, N, K, x, \
                                                                                          (int)M, y);    \
        return hipGetLastError();                                                                        \
    }
    TERN_PHASED3_CASE(4) TERN_PHASED3_CASE(8) TERN_PHASED3_CASE(16)
#undef TERN_PHASED3_CASE
    return hipErrorNotSupported;
}


hipError_t launch_gemv_bf16(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                            hipStream_t stream)
{
    {
        hipError_t e = launch_oneshot(false, packed, N, K, x, nullptr, M, y, nullptr, stream);
        if (e != hipErrorNotSupported) return e;
        e = launch_phased<false>(packed, N, K, x, nullptr, M, y, nullptr, stream);
        if (e != hipErrorNotSupported) return e;
    }
    const int64_t nkt = (K / kBlockK + 3) / 4;
    int nw, tpw;
    pick_fast(nkt, nw, tpw);
    const size_t fast_lds = fast_lds_bytes(K, M);
    if (fast_lds <= (size_t)kFastLds) {
        if (M == 1) return launch_fast_mt<1>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
        if (M == 2) return launch_fast_mt<2>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
        if (M <= 4) return launch_fast_mt<4>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
        return launch_fast_mt<16>(tpw, nw, fast_lds, stream, packed, N, K, x, (int)M, y);
    }
    // Activation halves beyond LDS but thirds within it (8B down at M = 9..16):
    // the three-phase kernel reads the weights once for all rows.
    {
        const hipError_t e = launch_phased3(packed, N, K, x, M, y, stream);
        if (e != hipErrorNotSupported) return e;
    }
    // More than 8 activation rows that fit none of the kernels above: two
    // calls on row halves take the one-pass or two-phase kernels, which read
    // the weights twice but finish sooner than the k-chunked kernel (8B down
    // at M = 16: 20.9 us as one k-chunked launch, 2 x 7.5 us as two).
    if (M > 8 && K % kTileK == 0) {
        OneShot c;
        if (gemv_oneshot_config(N, K, 8, false, c) || gemv_phased_config(N, K, 8, false, c)) {
            const hipError_t e = launch_gemv_bf16(packed, N, K, x, 8, y, stream);
            if (e != hipSuccess) return e;
            return launch_gemv_bf16(packed, N, K, x + 8 * K, M - 8, y + 8 * N, stream);
        }
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
    {
        hipError_t e = launch_oneshot(true, packed, N, K, q, s_x, M, y, acc, stream);
        if (e != hipErrorNotSupported) return e;
        e = launch_phased<true>(packed, N, K, q, s_x, M, y, acc, stream);
        if (e != hipErrorNotSupported) return e;
    }
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
