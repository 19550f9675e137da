// tern_prefill.hip — prefill-size ternary GEMM on the int8 matrix cores.
//
//   acc[m][n][b] = sum_{k in block b} t[n][k] * q[m][k]   (exact int32)
//   y[m][n]      = s_x[m] * sum_b scale[n][b] * acc[m][n][b]
//
// Workgroup = NWAVE waves side by side along N; wave tile 16*WM (m) x 16*WN
// (n).  Each wave decodes the planes of its own weight tiles straight into
// MFMA B operands (bytes 64*t, one rotate + mask per 4 weights), reuses each
// decoded block across its WM activation tiles, and folds every block's int32
// result into fp32 with that block's scale (cvt + fma per output element per
// block).  Plane words arrive a whole k-tile (4 blocks) ahead in 16-byte
// loads; activations are loaded two blocks ahead into a 3-buffer LDS ring,
// permuted to the decoded byte order on the way in.  One barrier per block.
#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

template <int WN>
struct PfPlanes {
    u32x4 nz[WN], sg[WN];   // word g of the k-tile's 4 blocks, per weight tile
    u32x2 sc[WN];           // fp16 scales of the 4 blocks, row r
};

template <int WM, int WN, int NWAVE, bool kDbg>
__global__ __launch_bounds__(64 * NWAVE, 2) void prefill_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                             const int8_t* __restrict__ q,
                                                             const float* __restrict__ s_x, int64_t M,
                                                             float* __restrict__ y, int32_t* __restrict__ acc_dbg)
{
    constexpr int BM = 16 * WM;
    constexpr int kStride = kBlockK + 16;              // bytes per staged activation row
    constexpr int kUnits = BM * 4;                     // 32-byte staging units per block
    constexpr int kThreads = 64 * NWAVE;
    constexpr int kUpt = (kUnits + kThreads - 1) / kThreads;
    __shared__ __align__(16) uint8_t abuf[3][BM * kStride];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int nb = (int)(K / kBlockK), nkt = (nb + 3) >> 2;
    const int64_t nrt = (N + 15) >> 4;
    const uint32_t* words = (const uint32_t*)packed;
    const uint16_t* scales = (const uint16_t*)(packed + scale_region_offset(N, K));
    int64_t rts[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) rts[j] = (int64_t)blockIdx.x * (WN * NWAVE) + wave * WN + j;

    auto load_planes = [&](int kt, PfPlanes<WN>& P) {
        const int nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            P.nz[j] = u32x4{0, 0, 0, 0};
            P.sg[j] = u32x4{0, 0, 0, 0};
            P.sc[j] = u32x2{0, 0};
            if (rts[j] >= nrt) continue;
            const int64_t wb = tile_word_base(rts[j], kt, nb);
            const int64_t sb = tile_scale_base(rts[j], kt, nb);
            if (nbq == 4) {
                P.nz[j] = ld_nt16(words + wb + ((0 * 4 + g) * 16 + r) * 4);
                P.sg[j] = ld_nt16(words + wb + ((1 * 4 + g) * 16 + r) * 4);
                P.sc[j] = ld_nt8(scales + sb + r * 4);
            } else {
                uint32_t s01 = 0, s23 = 0;
                for (int e = 0; e < nbq; ++e) {
                    P.nz[j][e] = words[wb + ((0 * 4 + g) * 16 + r) * nbq + e];
                    P.sg[j][e] = words[wb + ((1 * 4 + g) * 16 + r) * nbq + e];
                    const uint32_t h = scales[sb + r * nbq + e];
                    if (e < 2) s01 |= h << (16 * e);
                    else s23 |= h << (16 * (e - 2));
                }
                P.sc[j] = u32x2{s01, s23};
            }
        }
    };
    auto load_act = [&](int b, u32x4 (&st)[2 * kUpt]) {
#pragma unroll
        for (int h = 0; h < kUpt; ++h) {
            const int unit = threadIdx.x + kThreads * h;
            if (unit < kUnits) {
                const int row = unit >> 2, c32 = unit & 3;
                const int64_t m = m0 + row < M ? m0 + row : M - 1;
                const u32x4* src = (const u32x4*)(q + m * K + (int64_t)b * kBlockK + 32 * c32);
                st[2 * h] = src[0];
                st[2 * h + 1] = src[1];
            }
        }
    };
    auto store_act = [&](int buf, const u32x4 (&st)[2 * kUpt]) {
#pragma unroll
        for (int h = 0; h < kUpt; ++h) {
            const int unit = threadIdx.x + kThreads * h;
            if (unit < kUnits) {
                const int row = unit >> 2, c32 = unit & 3;
                const uint32_t Q[8] = {st[2 * h][0], st[2 * h][1], st[2 * h][2], st[2 * h][3],
                                       st[2 * h + 1][0], st[2 * h + 1][1], st[2 * h + 1][2], st[2 * h + 1][3]};
                u32x4 o0, o1;
#pragma unroll
                for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
                for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
                u32x4* dst = (u32x4*)(&abuf[buf][row * kStride + 32 * c32]);
                dst[0] = o0;
                dst[1] = o1;
            }
        }
    };

    f32x4 facc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) facc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // block b of k-tile planes P (block bq of the tile): issue block b+2's
    // activation loads, compute from ring buffer b % 3, store block b+2 into
    // buffer (b+2) % 3 (last read by block b-1, before the previous barrier)
    auto block = [&](int b, const PfPlanes<WN>& P, int bq) {
        u32x4 st[2 * kUpt];
        const bool ahead = b + 2 < nb;
        if (ahead) load_act(b + 2, st);
        const uint8_t* ab = abuf[b % 3];
        u32x4 A[WM][2];
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            const uint8_t* arow = ab + (16 * i + r) * kStride + 32 * g;
            A[i][0] = *(const u32x4*)(arow);
            A[i][1] = *(const u32x4*)(arow + 16);
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const CodeWords c = interleave(P.nz[j][bq], P.sg[j][bq]);
            const u32x4 B0 = u32x4{i8_quad<0>(c), i8_quad<1>(c), i8_quad<2>(c), i8_quad<3>(c)};
            const u32x4 B1 = u32x4{i8_quad<4>(c), i8_quad<5>(c), i8_quad<6>(c), i8_quad<7>(c)};
            const uint32_t sw = P.sc[j][bq >> 1];
            const float sc = half_bits_to_float((sw >> (16 * (bq & 1))) & 0xFFFFu) * (1.0f / 64.0f);
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                i32x4 d = {0, 0, 0, 0};
                d = mfma_i8(A[i][0], B0, d);
                d = mfma_i8(A[i][1], B1, d);
#pragma unroll
                for (int e = 0; e < 4; ++e) facc[i][j][e] = __builtin_fmaf(sc, (float)d[e], facc[i][j][e]);
                if constexpr (kDbg) {
                    const int64_t n = (rts[j] << 4) + r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t m = m0 + 16 * i + 4 * g + e;
                        if (m < M && n < N) acc_dbg[(m * N + n) * nb + b] = d[e] >> 6;
                    }
                }
            }
        }
        if (ahead) store_act((b + 2) % 3, st);
        __syncthreads();
    };
    auto tile = [&](int kt, const PfPlanes<WN>& P) {
        const int nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
        if (nbq == 4) {
#pragma unroll
            for (int bq = 0; bq < 4; ++bq) block(4 * kt + bq, P, bq);
        } else {
            for (int bq = 0; bq < nbq; ++bq) block(4 * kt + bq, P, bq);
        }
    };

    // prologue: blocks 0 and 1 staged, planes of k-tile 0 requested
    PfPlanes<WN> Pa, Pb;
    load_planes(0, Pa);
    {
        u32x4 st[2 * kUpt];
        load_act(0, st);
        store_act(0, st);
        if (nb > 1) {
            load_act(1, st);
            store_act(1, st);
        }
    }
    __syncthreads();
    for (int kt = 0; kt < nkt; kt += 2) {
        if (kt + 1 < nkt) load_planes(kt + 1, Pb);
        tile(kt, Pa);
        if (kt + 1 < nkt) {
            if (kt + 2 < nkt) load_planes(kt + 2, Pa);
            tile(kt + 1, Pb);
        }
    }

#pragma unroll
    for (int j = 0; j < WN; ++j) {
        const int64_t n = (rts[j] << 4) + r;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + 16 * i + 4 * g + e;
                if (m < M) y[m * N + n] = s_x[m] * facc[i][j][e];
            }
    }
}

// ---------------------------------------------------------------------------
// Large-M kernel: each weight block is decoded once per workgroup into LDS and
// shared by all of its waves.
//
// Workgroup = 8 waves in a WGM (m) x WGN (n) grid, wave tile 16*TM x 16*TN, so
// a workgroup covers BM = 16*TM*WGM rows of M and BN = 16*TN*WGN rows of N.
// Per 128-k block, every thread decodes one plane word pair (32 weights of one
// row) into the two int8 B operands of its (row, word) lane and stores them in
// LDS in MFMA lane order, and stages part of the activation block (permuted to
// the decoded byte order); each wave then runs 2*TM*TN MFMAs from LDS and folds
// each block's int32 result into fp32 with that block's scale.  Two LDS stages:
// block b is computed while block b+1 is written.  Plane words are loaded a
// k-tile (4 blocks) ahead and activations two blocks ahead, all from fixed
// positions of a loop unrolled over two k-tiles, so the loads in flight are
// counted exactly.  Requires K % 512 == 0.  The occupancy hint of 2
// workgroups per CU is kept even for shapes that fit only one: the code it
// produces ran 10-14% faster (8B gate and down at M = 2048, same VGPR count).
template <int TM, int TN, int WGM, int WGN>
struct Pf2 {
    static constexpr int kWaves = WGM * WGN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 16 * TM * WGM;
    static constexpr int BN = 16 * TN * WGN;
    static constexpr int NRT = BN / 16;                     // row tiles per workgroup
    static constexpr int kAStride = kBlockK + 16;           // bytes per staged activation row
    static constexpr int kWBytes = NRT * 2 * 64 * 16;       // decoded B operands per block
    static constexpr int kABytes = BM * kAStride;
    static constexpr int kStage = kWBytes + kABytes + BN * 4;
    static constexpr int kActPerThread = BM * kBlockK / 16 / kThreads;   // 16-byte activation loads
    static constexpr size_t kLds = 2 * (size_t)kStage;
    static_assert(NRT * 64 == kThreads, "one plane word pair per thread and block");
    static_assert(kActPerThread >= 2 && kActPerThread % 2 == 0, "activations staged in 32-byte words");
};

template <int TM, int TN, int WGM, int WGN, bool kDbg>
__global__ __launch_bounds__(64 * WGM * WGN, 2) void prefill2_kernel(
    const uint8_t* __restrict__ packed, int64_t N, int64_t K, const int8_t* __restrict__ q,
    const float* __restrict__ s_x, int64_t M, float* __restrict__ y, int32_t* __restrict__ acc_dbg)
{
    using C = Pf2<TM, TN, WGM, WGN>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t m0 = (int64_t)blockIdx.y * C::BM;
    const int64_t rt0 = (int64_t)blockIdx.x * C::NRT;
    const int nb = (int)(K / kBlockK), nkt = nb >> 2;
    const int64_t nrt = (N + 15) >> 4;
    const uint32_t* words = (const uint32_t*)packed;
    const uint16_t* scales = (const uint16_t*)(packed + scale_region_offset(N, K));

    // this thread's decode assignment: row tile dt, lane (r, g) within it
    const int dt = tid >> 6;
    const int64_t drt = rt0 + dt;
    const bool drow_ok = drt < nrt;
    // this thread's activation staging assignment: row am, 32-byte words aw0 ..
    constexpr int kWordsPerThread = C::kActPerThread / 2;
    constexpr int kThreadsPerRow = (kBlockK / 32) / kWordsPerThread;
    const int am = tid / kThreadsPerRow, aw0 = (tid % kThreadsPerRow) * kWordsPerThread;
    const int64_t arow = m0 + am < M ? m0 + am : M - 1;
    const int8_t* asrc = q + arow * K + 32 * aw0;

    auto stage_w = [&](int st) { return smem + st * C::kStage; };
    auto stage_a = [&](int st) { return smem + st * C::kStage + C::kWBytes; };
    auto stage_s = [&](int st) { return (float*)(smem + st * C::kStage + C::kWBytes + C::kABytes); };

    // plane words of k-tile kt for this thread's (row tile, r, g); rows past N read tile 0 (outputs dropped)
    auto load_planes = [&](int kt, PfPlanes<1>& P) {
        const int ktc = kt < nkt ? kt : nkt - 1;
        const int64_t rt = drow_ok ? drt : 0;
        const int64_t wb = tile_word_base(rt, ktc, nb);
        P.nz[0] = ld_nt16(words + wb + ((0 * 4 + g) * 16 + r) * 4);
        P.sg[0] = ld_nt16(words + wb + ((1 * 4 + g) * 16 + r) * 4);
        P.sc[0] = ld_nt8(scales + tile_scale_base(rt, ktc, nb) + r * 4);
    };
    auto load_act = [&](int b, u32x4 (&v)[C::kActPerThread]) {
        const int bc = b < nb ? b : nb - 1;
        const u32x4* src = (const u32x4*)(asrc + (int64_t)bc * kBlockK);
#pragma unroll
        for (int i = 0; i < C::kActPerThread; ++i) v[i] = src[i];
    };
    // decode block bq of planes P and stage block activations v into stage st
    auto write_stage = [&](int st, const PfPlanes<1>& P, int bq, const u32x4 (&v)[C::kActPerThread]) {
        const CodeWords cw = interleave(P.nz[0][bq], P.sg[0][bq]);
        const u32x4 B0 = u32x4{i8_quad<0>(cw), i8_quad<1>(cw), i8_quad<2>(cw), i8_quad<3>(cw)};
        const u32x4 B1 = u32x4{i8_quad<4>(cw), i8_quad<5>(cw), i8_quad<6>(cw), i8_quad<7>(cw)};
        uint8_t* w = stage_w(st) + ((dt * 2 + 0) * 64 + lane) * 16;
        *(u32x4*)w = B0;
        *(u32x4*)(w + 64 * 16) = B1;
        if (g == 0) {
            const uint32_t sw = P.sc[0][bq >> 1];
            stage_s(st)[dt * 16 + r] = half_bits_to_float((sw >> (16 * (bq & 1))) & 0xFFFFu) * (1.0f / 64.0f);
        }
#pragma unroll
        for (int u = 0; u < kWordsPerThread; ++u) {
            const uint32_t Q[8] = {v[2 * u][0], v[2 * u][1], v[2 * u][2], v[2 * u][3],
                                   v[2 * u + 1][0], v[2 * u + 1][1], v[2 * u + 1][2], v[2 * u + 1][3]};
            u32x4 o0, o1;
#pragma unroll
            for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
            for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
            u32x4* dst = (u32x4*)(stage_a(st) + am * C::kAStride + 32 * (aw0 + u));
            dst[0] = o0;
            dst[1] = o1;
        }
    };

    f32x4 facc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) facc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The MFMAs of n-tile j are issued before the epilogue of n-tile j-1, so
    // the conversions never wait on the matrix core's latency.
    auto compute = [&](int st, int b) {
        const uint8_t* ab = stage_a(st);
        const uint8_t* wb = stage_w(st);
        const float* sb = stage_s(st);
        u32x4 A[TM][2];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint8_t* a = ab + (wm * 16 * TM + 16 * i + r) * C::kAStride + 32 * g;
            A[i][0] = *(const u32x4*)(a);
            A[i][1] = *(const u32x4*)(a + 16);
        }
        i32x4 dprev[TM], dcur[TM];
        float scprev = 0.f;
#pragma unroll
        for (int j = 0; j <= TN; ++j) {
            float sc = 0.f;
            if (j < TN) {
                const int t = wn * TN + j;
                const u32x4 B0 = *(const u32x4*)(wb + ((t * 2 + 0) * 64 + lane) * 16);
                const u32x4 B1 = *(const u32x4*)(wb + ((t * 2 + 1) * 64 + lane) * 16);
                sc = sb[t * 16 + r];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    dcur[i] = mfma_i8(A[i][0], B0, i32x4{0, 0, 0, 0});
                    dcur[i] = mfma_i8(A[i][1], B1, dcur[i]);
                }
            }
            if (j > 0) {
                const int jp = j - 1;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        facc[i][jp][e] = __builtin_fmaf(scprev, (float)dprev[i][e], facc[i][jp][e]);
                    if constexpr (kDbg) {
                        const int64_t n = ((rt0 + wn * TN + jp) << 4) + r;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int64_t m = m0 + wm * 16 * TM + 16 * i + 4 * g + e;
                            if (m < M && n < N) acc_dbg[(m * N + n) * nb + b] = dprev[i][e] >> 6;
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) dprev[i] = dcur[i];
            scprev = sc;
        }
    };

    // prologue: planes of k-tiles 0 and 1, activations of blocks 0 and 1; stage 0 = block 0
    PfPlanes<1> Pa, Pb;
    u32x4 va[C::kActPerThread], vb[C::kActPerThread];
    load_planes(0, Pa);
    load_act(0, va);
    load_act(1, vb);
    load_planes(1, Pb);
    write_stage(0, Pa, 0, va);
    load_act(2, va);
    __syncthreads();

    // block b = 4*kt + bq: compute b from stage b&1, write block b+1 into the
    // other stage (its activations sit in the register set loaded two blocks
    // earlier), then load block b+3's activations into that set.  Past the
    // last block, compute and writes are skipped but the (clamped) loads are
    // still issued, so every pass issues the same loads.
    auto block = [&](int b, const PfPlanes<1>& Pnext_src, int nbq_src, u32x4 (&vnext)[C::kActPerThread]) {
        if (b < nb) compute(b & 1, b);
        if (b + 1 < nb) write_stage((b + 1) & 1, Pnext_src, nbq_src, vnext);
        load_act(b + 3, vnext);
        __syncthreads();
    };
    for (int kt = 0; kt < nkt; kt += 2) {
        // k-tile kt has planes Pa, k-tile kt+1 has Pb
        block(4 * kt + 0, Pa, 1, vb);
        block(4 * kt + 1, Pa, 2, va);
        block(4 * kt + 2, Pa, 3, vb);
        block(4 * kt + 3, Pb, 0, va);
        load_planes(kt + 2, Pa);
        block(4 * kt + 4, Pb, 1, vb);
        block(4 * kt + 5, Pb, 2, va);
        block(4 * kt + 6, Pb, 3, vb);
        block(4 * kt + 7, Pa, 0, va);
        load_planes(kt + 3, Pb);
    }

#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = ((rt0 + wn * TN + j) << 4) + r;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + wm * 16 * TM + 16 * i + 4 * g + e;
                if (m < M) y[m * N + n] = s_x[m] * facc[i][j][e];
            }
    }
}

template <int TM, int TN, int WGM, int WGN>
static hipError_t launch_pf2(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                             int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    using C = Pf2<TM, TN, WGM, WGN>;
    const dim3 grid((unsigned)((N + C::BN - 1) / C::BN), (unsigned)((M + C::BM - 1) / C::BM));
    if (acc)
        prefill2_kernel<TM, TN, WGM, WGN, true><<<grid, C::kThreads, C::kLds, stream>>>(packed, N, K, q, s_x, M, y,
                                                                                      acc);
    else
        prefill2_kernel<TM, TN, WGM, WGN, false><<<grid, C::kThreads, C::kLds, stream>>>(packed, N, K, q, s_x, M, y,
                                                                                       acc);
    return hipGetLastError();
}

template <int WM, int WN, int NWAVE>
static hipError_t launch_pf(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M,
                            float* y, int32_t* acc, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + 16 * WN * NWAVE - 1) / (16 * WN * NWAVE)),
                    (unsigned)((M + 16 * WM - 1) / (16 * WM)));
    if (acc)
        prefill_kernel<WM, WN, NWAVE, true><<<grid, 64 * NWAVE, 0, stream>>>(packed, N, K, q, s_x, M, y, acc);
    else
        prefill_kernel<WM, WN, NWAVE, false><<<grid, 64 * NWAVE, 0, stream>>>(packed, N, K, q, s_x, M, y, acc);
    return hipGetLastError();
}

hipError_t launch_prefill(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                          int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    if (K % 512 == 0 && M >= 128) {
        // workgroup-shared decode.  256 x 128 workgroup tiles (8 waves of
        // 64 x 64) from M = 1024; below, 128 x 64 tiles (4 waves of 32 x 64,
        // three workgroups per CU).  Measured on the 8B shapes: gate M = 2048
        // 170 us vs 174 us, down M = 2048 141 us vs 167 us; gate M = 512
        // 51 us vs 59 us, down M = 512 65 us vs 132 us.
        if (M >= 1024) return launch_pf2<4, 4, 4, 2>(packed, N, K, q, s_x, M, y, acc, stream);
        return launch_pf2<2, 4, 4, 1>(packed, N, K, q, s_x, M, y, acc, stream);
    }
    // Below M = 128 the prefill kernel's time is set by its per-block latency
    // (about 0.62 us per 128-k block on the 8B shapes, nearly independent of
    // M and N), while the int8 GEMV reads the weights once per 16 activation
    // rows (about 4 us of fixed time plus the weight bytes at 5.3 TB/s per
    // launch).  Take the cheaper by that measured model: 8B down at M = 64
    // 61 us -> 31 us in four GEMV launches; 8B gate at M = 16/32/48 23-24 us
    // -> 7/13/19 us, at M = 64 a tie (the prefill kernel stays).
    {
        const double pf_us = 0.62 * (double)(K / kBlockK);
        const double gemv_us = 4.0 + (double)N * (double)K * (0.265625 / 5.3e6);
        const int64_t chunks = (M + 15) / 16;
        if ((double)chunks * gemv_us < pf_us) {
            for (int64_t m0 = 0; m0 < M; m0 += 16) {
                const int64_t mc = M - m0 < 16 ? M - m0 : 16;
                const hipError_t e = launch_gemv_i8(packed, N, K, q + m0 * K, s_x + m0, mc, y + m0 * N,
                                                    acc ? acc + m0 * N * (K / kBlockK) : nullptr, stream);
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }
    // wave tile 64 (m) x 16 (n), two workgroups per CU: measured best among the
    // tile shapes that fit 256 VGPRs without spills (8B gate, M = 2048: 259 us vs
    // 355-398 us for 32x32 and 64x16 at two waves per workgroup)
    return launch_pf<4, 1, 4>(packed, N, K, q, s_x, M, y, acc, stream);
}

}  // namespace tern
