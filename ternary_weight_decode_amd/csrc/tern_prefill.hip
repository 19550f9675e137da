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
#include "tern_tile.h"

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

template <int TM, int TN, int WGM, int WGN, bool kSplit, bool kDbg>
__global__ __launch_bounds__(64 * WGM * WGN, 2) void prefill2_kernel(
    const uint8_t* __restrict__ packed, int64_t N, int64_t K, const int8_t* __restrict__ q,
    const float* __restrict__ s_x, int64_t M, float* __restrict__ y, int32_t* __restrict__ acc_dbg, int kts)
{
    using C = Pf2<TM, TN, WGM, WGN>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t m0 = (int64_t)blockIdx.y * C::BM;
    const int64_t rt0 = (int64_t)blockIdx.x * C::NRT;
    const int nb = (int)(K / kBlockK);
    // this workgroup's k-tiles: [kt0, kt0 + nkt) of the row's K / 512 (all of them unless split)
    const int kt0 = kSplit ? (int)blockIdx.z * kts : 0;
    const int nkt = kSplit ? min(kts, (nb >> 2) - kt0) : nb >> 2;
    const int nbl = 4 * nkt;
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
        const int ktc = (kt < nkt ? kt : nkt - 1) + kt0;
        const int64_t rt = drow_ok ? drt : 0;
        const int64_t wb = tile_word_base(rt, ktc, nb);
        P.nz[0] = ld_nt16(words + wb + ((0 * 4 + g) * 16 + r) * 4);
        P.sg[0] = ld_nt16(words + wb + ((1 * 4 + g) * 16 + r) * 4);
        P.sc[0] = ld_nt8(scales + tile_scale_base(rt, ktc, nb) + r * 4);
    };
    auto load_act = [&](int b, u32x4 (&v)[C::kActPerThread]) {
        const int bc = (b < nbl ? b : nbl - 1) + 4 * kt0;
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
                            if (m < M && n < N) acc_dbg[(m * N + n) * nb + 4 * kt0 + b] = dprev[i][e] >> 6;
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
        if (b < nbl) compute(b & 1, b);
        if (b + 1 < nbl) write_stage((b + 1) & 1, Pnext_src, nbq_src, vnext);
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
                if (m < M) {
                    if constexpr (kSplit)
                        unsafeAtomicAdd(y + m * N + n, facc[i][j][e]);
                    else
                        y[m * N + n] = s_x[m] * facc[i][j][e];
                }
            }
    }
}

// K split in two halves (the reason and the measurements are at launch_pf2): nkt k-tiles
// of 512, `tiles` output tiles of the workgroup tile.
static bool pf2_split(int64_t nkt, int64_t tiles)
{
    return nkt >= 8 && 2 * tiles <= device_cus();
}

// The split prefill's first and last passes over y (M x N fp32, row-major): clear it, and
// multiply row m by s_x[m].  16-byte accesses where y is 16-byte aligned (and, for the
// row scaling, rows are too: N % 4 == 0); on 16 MB of y (8B down, M = 1024) they took 6.5 and
// 9.5 us with 4-byte accesses, 6.5 and 6.8 us with these.
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ y, int64_t n, bool vec)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n4 = vec ? n >> 2 : 0;
    for (int64_t i = i0; i < n4; i += stride) ((f32x4*)y)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t i = (n4 << 2) + i0; i < n; i += stride) y[i] = 0.f;
}

template <bool kVec>
__global__ __launch_bounds__(256) void scale_rows_kernel(float* __restrict__ y, const float* __restrict__ s_x,
                                                         int64_t M, int64_t N)
{
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const float s = s_x[m];
        if constexpr (kVec) {
            f32x4* row = (f32x4*)(y + m * N);
            for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < (N >> 2); j += (int64_t)gridDim.x * 256) {
                f32x4 v = row[j];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = s * v[e];
                row[j] = v;
            }
        } else {
            float* row = y + m * N;
            for (int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x; n < N; n += (int64_t)gridDim.x * 256)
                row[n] = s * row[n];
        }
    }
}

static hipError_t launch_zero_f32(float* y, int64_t n, hipStream_t stream)
{
    const bool vec = ((uintptr_t)y & 15) == 0;
    const int64_t items = vec ? (n + 3) / 4 : n;
    const int64_t g = (items + 255) / 256;
    zero_f32_kernel<<<(unsigned)(g < 4096 ? (g > 0 ? g : 1) : 4096), 256, 0, stream>>>(y, n, vec);
    return hipGetLastError();
}

static hipError_t launch_scale_rows(float* y, const float* s_x, int64_t M, int64_t N, hipStream_t stream)
{
    const bool vec = ((uintptr_t)y & 15) == 0 && N % 4 == 0;
    const int64_t gx = ((vec ? N / 4 : N) + 255) / 256;
    const dim3 grid((unsigned)(gx < 64 ? gx : 64), (unsigned)(M < 4096 ? M : 4096));
    if (vec)
        scale_rows_kernel<true><<<grid, 256, 0, stream>>>(y, s_x, M, N);
    else
        scale_rows_kernel<false><<<grid, 256, 0, stream>>>(y, s_x, M, N);
    return hipGetLastError();
}

template <int TM, int TN, int WGM, int WGN>
static hipError_t launch_pf2(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                             int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    using C = Pf2<TM, TN, WGM, WGN>;
    const int nkt = (int)(K / 512);
    const int64_t tiles = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
    // K split in two halves when both halves' workgroups still fit one per CU and each half
    // keeps at least 4 k-tiles.  A lone workgroup on a CU runs its blocks one after another
    // (about 0.65 us per 128-k block on the 8B down shape whatever the tile count), so the
    // split halves the time where CUs would otherwise idle: 8B down at M = 128 / 256 61.5 /
    // 61.8 us -> 38.1 / 41.7 us (128 x 64 tiles), at M = 1024 135.0 -> 98.9 us with the
    // 256 x 128 tile (which the tile model no longer picks there).  Two workgroups per CU gain nothing
    // (down at M = 512: 62.6 vs 63.7 us) and short K loses to the two extra passes (gate at
    // M = 128: 26.4 vs 31.8 us).  y is cleared first, each half adds its unscaled partial
    // with one atomic fp32 add per element (two addends onto zero give the same sum in
    // either order, so y is deterministic), and a last pass multiplies each row by s_x:
    // y = fl(s_x * fl(a + b)).
    const bool split = pf2_split(nkt, tiles);
    const int kts = split ? (nkt + 1) / 2 : nkt;
    const dim3 grid((unsigned)((N + C::BN - 1) / C::BN), (unsigned)((M + C::BM - 1) / C::BM), split ? 2u : 1u);
    if (split) {
        const hipError_t e = launch_zero_f32(y, M * N, stream);
        if (e != hipSuccess) return e;
        if (acc)
            prefill2_kernel<TM, TN, WGM, WGN, true, true><<<grid, C::kThreads, C::kLds, stream>>>(
                packed, N, K, q, s_x, M, y, acc, kts);
        else
            prefill2_kernel<TM, TN, WGM, WGN, true, false><<<grid, C::kThreads, C::kLds, stream>>>(
                packed, N, K, q, s_x, M, y, acc, kts);
        const hipError_t e2 = hipGetLastError();
        if (e2 != hipSuccess) return e2;
        return launch_scale_rows(y, s_x, M, N, stream);
    } else if (acc) {
        prefill2_kernel<TM, TN, WGM, WGN, false, true><<<grid, C::kThreads, C::kLds, stream>>>(
            packed, N, K, q, s_x, M, y, acc, kts);
    } else {
        prefill2_kernel<TM, TN, WGM, WGN, false, false><<<grid, C::kThreads, C::kLds, stream>>>(
            packed, N, K, q, s_x, M, y, acc, kts);
    }
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

// ---------------------------------------------------------------------------
// Small-M kernel (17 <= M <= 64, MG groups of 16 activation rows): the int8
// one-pass GEMV's split of K across the waves of a workgroup, instead of one
// serial pass over K per workgroup.  A workgroup owns R row tiles and R*nwr
// waves; wave (rr, kw) takes k-tile kw of row tile rr in every phase, and
// phase ph covers k-tiles [ph*nwr, (ph+1)*nwr), so unit ph of every wave lies
// in phase ph.  The activations of a phase (MG*16 rows x nwr*512 bytes) are
// staged in LDS in the decoded byte order, and the register set they came
// from is refilled with the next phase's at once; each wave decodes its unit
// once and reuses it
// across the MG row groups (two int8 MFMAs per group and 128-k block, exact
// int32 block sums folded in fp32 with the block scale).  Partials meet in
// LDS and are summed in k-tile order (deterministic).  Rows past M repeat row
// M-1 and rows past N a real row tile; their outputs are dropped.  The LDS
// of one phase allows one workgroup per CU, i.e. three waves per SIMD: the
// kernel is compiled for that occupancy (up to 168 VGPRs), so a block's A
// operands of every row group are read ahead of its MFMAs (gate M = 64
// 15.8 -> 15.1 us, down M = 64 26.2 -> 23.1 us against compiling for four
// waves per SIMD with the reads interleaved).
template <int MG, int XC, bool kDbg>
__global__ __launch_bounds__(768) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefill_small_kernel(const uint8_t* __restrict__ packed, int64_t N,
                                                             int64_t K, const int8_t* __restrict__ q,
                                                             const float* __restrict__ s_x, int M,
                                                             float* __restrict__ y, int32_t* __restrict__ acc_dbg,
                                                             int R)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int kRows = MG * 16;
    const int nthreads = blockDim.x, nw = nthreads >> 6, nwr = nw / R;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int rr = wave % R, kw = wave / R;
    const int nb = (int)(K >> 7), nkt = nb >> 2, nph = nkt / nwr;
    const int64_t nrt = (N + 15) >> 4;
    const int64_t rt_real = (int64_t)blockIdx.x * R + rr;
    const int64_t rt = rt_real < nrt ? rt_real : nrt - 1;
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL uint16_t* scales = (const TERN_GLOBAL uint16_t*)(packed + scale_region_offset(N, K));
    const int kp = nwr * kTileK;                                     // k per phase
    const int half = kp / 2;                                         // bytes of a row's first-half region
    const int xrow = kp + 16;                                        // staged bytes per activation row

    // Staging assignment: 32-byte word c of this thread is row (u / per_row), word (u % per_row)
    // of the phase.  A staged row holds the first 16 bytes (in the decoded order) of its words
    // in one region and their second 16 bytes in the next, so each staging write instruction
    // covers consecutive 16-byte slots.  per_row = 16*nwr is a power of two.
    const int per_row = kp / 32, lg = 31 - __builtin_clz((unsigned)per_row), chunks = kRows * per_row;
    int xsrc[XC], xdst[XC];
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const int u = threadIdx.x + c * nthreads;
        const int uc = u < chunks ? u : chunks - 1;
        const int m = uc >> lg, cc = uc & (per_row - 1);
        const int mr = m < M ? m : M - 1;
        xsrc[c] = (mr * (int)K + 32 * cc) >> 4;                      // in 16-byte units
        xdst[c] = u < chunks ? m * xrow + 16 * cc : kRows * xrow;   // past the end: a dummy slot
    }
    const TERN_GLOBAL u32x4* qg = (const TERN_GLOBAL u32x4*)q;
    auto load_x = [&](int ph, u32x4 (&v)[XC][2]) {
        const int p = (ph < nph ? ph : nph - 1) * (kp >> 4);
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            v[c][0] = qg[xsrc[c] + p];
            v[c][1] = qg[xsrc[c] + p + 1];
        }
    };
    auto stage = [&](const u32x4 (&v)[XC][2]) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const uint32_t Q[8] = {v[c][0][0], v[c][0][1], v[c][0][2], v[c][0][3],
                                   v[c][1][0], v[c][1][1], v[c][1][2], v[c][1][3]};
            u32x4 o0, o1;
#pragma unroll
            for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
            for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
            *(u32x4*)(smem + xdst[c]) = o0;
            *(u32x4*)(smem + xdst[c] + half) = o1;
        }
    };
    auto load_unit = [&](int ph, PlaneTile& t) {
        const int kt = (ph < nph ? ph : nph - 1) * nwr + kw;
        const int64_t wb = tile_word_base(rt, kt, nb);
        const int64_t sb = tile_scale_base(rt, kt, nb);
        t.nz = ld_nt16(words + wb + (int64_t)(g * 16 + r) * 4);
        t.sg = ld_nt16(words + wb + (int64_t)((4 + g) * 16 + r) * 4);
        t.sc = ld_nt8(scales + sb + r * 4);
    };

    f32x4 acc[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) acc[mg] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t* xw = smem + r * xrow + 16 * (kw * 16 + g);        // this lane's row r, the wave's k-tile
    auto compute = [&](int ph, const PlaneTile& t) {
        const int kt = ph * nwr + kw;
#pragma unroll
        for (int bq = 0; bq < 4; ++bq) {
            // the block's A operands of every row group first, then MG independent MFMA chains
            u32x4 A[MG][2];
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) {
                const uint8_t* qa = xw + mg * 16 * xrow + bq * 64;     // word kw*16 + bq*4 + g
                A[mg][0] = *(const u32x4*)(qa);
                A[mg][1] = *(const u32x4*)(qa + half);
            }
            u32x4 B[2];
            decode_i8(t.nz[bq], t.sg[bq], B);
            const float sc = tile_scale(t, bq) * (1.0f / 64.0f);     // decoded weights are 64*t
            i32x4 dd[MG];
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) dd[mg] = mfma_i8(A[mg][0], B[0], i32x4{0, 0, 0, 0});
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) dd[mg] = mfma_i8(A[mg][1], B[1], dd[mg]);
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) {
                const i32x4 d = dd[mg];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[mg][e] = __builtin_fmaf(sc, (float)d[e], acc[mg][e]);
                if constexpr (kDbg) {
                    const int64_t n = rt_real * kTileRows + r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = mg * 16 + 4 * g + e;
                        if (m < M && n < N) acc_dbg[((int64_t)m * N + n) * nb + kt * 4 + bq] = d[e] >> 6;
                    }
                }
            }
        }
    };

    // one activation register set, refilled with the next phase right after it is staged
    // (the next phase's load latency overlaps this phase's compute), and two unit slots.
    // The loop body is one phase with no branch inside, so the refill stays where it is
    // issued (its use is in the next iteration) instead of being sunk next to its use.
    u32x4 xa[XC][2];
    PlaneTile ta, tb;
    load_x(0, xa);
    __builtin_amdgcn_sched_barrier(0);
    load_unit(0, ta);
    load_unit(1, tb);
    __builtin_amdgcn_sched_barrier(0);
    for (int ph = 0; ph < nph; ++ph) {
        stage(xa);
        __syncthreads();
        load_x(ph + 1, xa);
        __builtin_amdgcn_sched_barrier(0);
        compute(ph, ta);
        ta = tb;                           // the next phase's unit, loaded a phase earlier
        load_unit(ph + 2, tb);
        __syncthreads();                   // every wave has read this phase
    }

    // partials [wave][MG][4][64] in the staging area, summed over the nwr waves of each row tile
    float* red = (float*)smem;
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((wave * MG + mg) * 4 + e) * 64 + lane] = acc[mg][e];
    __syncthreads();
    const int nout = R * MG * 4 * 64;
    for (int o = threadIdx.x; o < nout; o += nthreads) {
        const int l = o & 63, e = (o >> 6) & 3, mg = (o >> 8) % MG, orr = (o >> 8) / MG;
        const int m = mg * 16 + 4 * (l >> 4) + e;
        const int64_t n = ((int64_t)blockIdx.x * R + orr) * kTileRows + (l & 15);
        if (m < M && n < N) {
            float sum = 0.f;
            for (int w = 0; w < nwr; ++w) sum += red[(((w * R + orr) * MG + mg) * 4 + e) * 64 + l];
            y[(int64_t)m * N + n] = s_x[m] * sum;
        }
    }
}

// ---------------------------------------------------------------------------
// Register-resident activations (17 <= M <= 64, K % 512 == 0, K <= 4096): one
// wave per k-tile of K.  A wave loads its k-tile of all MG*16 activation rows
// once, straight into the int8 MFMA A operands (32-byte word 512*kw + 128*bq +
// 32*g of row mg*16 + r for lane (r, g) and block bq, gathered from two
// row-contiguous loads by a cross-lane swap and permuted in registers to the
// decoded byte order), and reuses them over the R consecutive row tiles
// of its workgroup, whose plane words it requests up front: no activation
// staging and no barrier before the compute.  Per row tile and 128-k block two
// MFMAs per row group give the exact int32 block sums, folded in fp32 with the
// block scale in block order; the nkt partials of each output meet in LDS once
// and are summed in k-tile order (deterministic).  Rows past M repeat row M-1
// and row tiles past N the last real one; their outputs are dropped.
template <int MG, int R, int KT, bool kDbg>
__global__ __launch_bounds__(512) void prefill_reg_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ s_x, int M,
                                                          float* __restrict__ y, int32_t* __restrict__ acc_dbg)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int nw = (int)(blockDim.x >> 6);                           // KT k-tiles per wave
    const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int nb = (int)(K >> 7);
    const int64_t nrt = (N + 15) >> 4;
    const int64_t rt0 = (int64_t)blockIdx.x * R;
    const int m0 = (int)blockIdx.y * (MG * 16);                     // this workgroup's activation rows
    const TERN_GLOBAL uint32_t* words = (const TERN_GLOBAL uint32_t*)packed;
    const TERN_GLOBAL uint16_t* scales = (const TERN_GLOBAL uint16_t*)(packed + scale_region_offset(N, K));

    // the plane words of this wave's R x KT units, then its activations, all requested up front
    PlaneTile t[R][KT];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t rt = rt0 + i < nrt ? rt0 + i : nrt - 1;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const int64_t wb = tile_word_base(rt, kw * KT + j, nb);
            t[i][j].nz = ld_nt16(words + wb + (int64_t)(g * 16 + r) * 4);
            t[i][j].sg = ld_nt16(words + wb + (int64_t)((4 + g) * 16 + r) * 4);
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t rt = rt0 + i < nrt ? rt0 + i : nrt - 1;
#pragma unroll
        for (int j = 0; j < KT; ++j) t[i][j].sc = ld_nt8(scales + tile_scale_base(rt, kw * KT + j, nb) + r * 4);
    }
    // Each load covers 64 contiguous bytes of every row (lane group g takes 16-byte piece
    // c(g) = 2(g & 1) + (g >> 1) of the block's first, then second, 64 bytes); one swap of
    // the upper 32 lanes of the first with the lower 32 lanes of the second then leaves
    // lane group g with pieces 2g and 2g + 1, its 32-byte word.
    const TERN_GLOBAL u32x4* qg = (const TERN_GLOBAL u32x4*)q;
    u32x4 A[MG][4 * KT][2];
    const int piece = 2 * (g & 1) + (g >> 1);
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        const int m = m0 + mg * 16 + r < M ? m0 + mg * 16 + r : M - 1;
        const int64_t base = (((int64_t)m * K + kTileK * KT * kw) >> 4) + piece;   // in 16-byte units
#pragma unroll
        for (int b = 0; b < 4 * KT; ++b) {
            A[mg][b][0] = qg[base + 8 * b];
            A[mg][b][1] = qg[base + 8 * b + 4];
        }
    }

    float* red = (float*)smem;                                       // [R][nw][MG][4][64]
#pragma unroll
    for (int i = 0; i < R; ++i) {
        f32x4 acc[MG];
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) acc[mg] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t n = (rt0 + i) * kTileRows + r;
#pragma unroll
        for (int b = 0; b < 4 * KT; ++b) {
            const int j = b >> 2, bq = b & 3;
            if (i == 0) {
                // pieces to words, then natural bytes -> the decoded order, once per activation word
#pragma unroll
                for (int mg = 0; mg < MG; ++mg) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(A[mg][b][0][d], A[mg][b][1][d], false,
                                                                         false);
                        A[mg][b][0][d] = sw[0];
                        A[mg][b][1][d] = sw[1];
                    }
                    const uint32_t Q[8] = {A[mg][b][0][0], A[mg][b][0][1], A[mg][b][0][2], A[mg][b][0][3],
                                           A[mg][b][1][0], A[mg][b][1][1], A[mg][b][1][2], A[mg][b][1][3]};
#pragma unroll
                    for (int d = 0; d < 4; ++d) A[mg][b][0][d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
                    for (int d = 4; d < 8; ++d) A[mg][b][1][d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
                }
            }
            u32x4 B[2];
            decode_i8(t[i][j].nz[bq], t[i][j].sg[bq], B);
            const float sc = tile_scale(t[i][j], bq) * (1.0f / 64.0f);    // decoded weights are 64*t
            i32x4 dd[MG];
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) dd[mg] = mfma_i8(A[mg][b][0], B[0], i32x4{0, 0, 0, 0});
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) dd[mg] = mfma_i8(A[mg][b][1], B[1], dd[mg]);
#pragma unroll
            for (int mg = 0; mg < MG; ++mg) {
                const i32x4 d = dd[mg];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[mg][e] = __builtin_fmaf(sc, (float)d[e], acc[mg][e]);
                if constexpr (kDbg) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = m0 + mg * 16 + 4 * g + e;
                        if (m < M && n < N) acc_dbg[((int64_t)m * N + n) * nb + kw * KT * 4 + b] = d[e] >> 6;
                    }
                }
            }
        }
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((((i * nw + kw) * MG + mg) * 4 + e) << 6) + lane] = acc[mg][e];
    }
    __syncthreads();
    const int nout = R * MG * 4 * 64;
    for (int o = threadIdx.x; o < nout; o += (int)blockDim.x) {
        const int l = o & 63, e = (o >> 6) & 3, mg = (o >> 8) % MG, i = (o >> 8) / MG;
        const int m = m0 + mg * 16 + 4 * (l >> 4) + e;
        const int64_t n = (rt0 + i) * kTileRows + (l & 15);
        if (m < M && n < N) {
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += red[((((i * nw + w) * MG + mg) * 4 + e) << 6) + l];
            y[(int64_t)m * N + n] = s_x[m] * sum;
        }
    }
}

// Launch configuration of prefill_reg_kernel, or false when it does not
// apply: nkt = K/512 waves (at most 8: two waves per SIMD keep the MG*32
// activation registers), the smallest R (1-4, 6 or 8 row tiles per workgroup)
// for which the grid fits the CUs at eight waves per CU.  Each CU reads the
// activations of its rows for all of K from L2, which sets the time (8B gate,
// M = 64: 14.3 us, 8.1 us with every activation row read from one row); at
// four row groups the workgroups take two rows of the grid, one per half of
// the activation rows, and read half as many activation bytes while every
// weight tile is read twice (the second time mostly from L2: the two halves'
// workgroups sit on the same XCD): 14.2 -> 12.8 us.  At three groups the
// split (16 rows wasted) measured 12.6 against 12.1 us, at M = 32 a split
// into single groups 9.4 against 9.5 us (decode work doubled), so those stay
// whole.
struct PfReg {
    int MG, R, nw, S, KT;
    int64_t grid;
    size_t lds;
};

static bool pick_pf_reg(int64_t N, int64_t K, int64_t M, PfReg& c)
{
    if (K % kTileK != 0 || M < 17 || M > 64 || N < 1) return false;
    const int64_t nkt = K / kTileK, groups = (M + 15) / 16;
    if (nkt <= 8) {
        // one k-tile per wave; two or three 16-row groups in one workgroup, four as two
        // halves in two grid rows
        c.KT = 1;
        c.MG = (int)(groups <= 3 ? groups : 2);
        c.S = (int)(groups <= 3 ? 1 : 2);
    } else if (nkt % 8 == 0 && nkt / 8 <= 3) {
        // eight waves of KT k-tiles each, every 16-row group in a grid row of its own
        // (K up to 12288: KT*32 activation registers per wave)
        c.KT = (int)(nkt / 8);
        c.MG = 1;
        c.S = (int)groups;
    } else {
        return false;
    }
    c.nw = (int)(nkt / c.KT);
    // the smallest R whose grid fits the CUs in one round (at most 8 row tiles, 4 with several
    // k-tiles per wave: the plane words of R*KT units stay in registers)
    const int64_t nrt = (N + 15) / 16, slots = device_cus() * (8 / c.nw);
    static const int kR1[] = {1, 2, 3, 4, 6, 8}, kR3[] = {1, 2, 3, 4};
    const int* rs = c.KT == 1 ? kR1 : kR3;
    const int nr = c.KT == 1 ? 6 : 4;
    c.R = rs[nr - 1];
    for (int i = 0; i < nr; ++i) {
        if ((nrt + rs[i] - 1) / rs[i] * c.S <= slots) {
            c.R = rs[i];
            break;
        }
    }
    c.grid = (nrt + c.R - 1) / c.R;
    c.lds = (size_t)c.R * c.nw * c.MG * 4 * 64 * 4;
    return c.lds <= (size_t)kCuLds;
}

template <int MG, int R, int KT>
static hipError_t launch_pf_reg_r(const PfReg& c, const uint8_t* packed, int64_t N, int64_t K, const int8_t* q,
                                  const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    const dim3 grid((unsigned)c.grid, (unsigned)c.S);
    if (acc)
        prefill_reg_kernel<MG, R, KT, true><<<grid, dim3(64 * c.nw), c.lds, stream>>>(packed, N, K, q, s_x, (int)M,
                                                                                        y, acc);
    else
        prefill_reg_kernel<MG, R, KT, false><<<grid, dim3(64 * c.nw), c.lds, stream>>>(packed, N, K, q, s_x, (int)M,
                                                                                         y, acc);
    return hipGetLastError();
}

template <int MG>
static hipError_t launch_pf_reg_mg(const PfReg& c, const uint8_t* packed, int64_t N, int64_t K, const int8_t* q,
                                   const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    switch (c.R) {
    case 1: return launch_pf_reg_r<MG, 1, 1>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 2: return launch_pf_reg_r<MG, 2, 1>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 3: return launch_pf_reg_r<MG, 3, 1>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 4: return launch_pf_reg_r<MG, 4, 1>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 6: return launch_pf_reg_r<MG, 6, 1>(c, packed, N, K, q, s_x, M, y, acc, stream);
    default: return launch_pf_reg_r<MG, 8, 1>(c, packed, N, K, q, s_x, M, y, acc, stream);
    }
}

template <int KT>
static hipError_t launch_pf_reg_kt(const PfReg& c, const uint8_t* packed, int64_t N, int64_t K, const int8_t* q,
                                   const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    switch (c.R) {
    case 1: return launch_pf_reg_r<1, 1, KT>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 2: return launch_pf_reg_r<1, 2, KT>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 3: return launch_pf_reg_r<1, 3, KT>(c, packed, N, K, q, s_x, M, y, acc, stream);
    default: return launch_pf_reg_r<1, 4, KT>(c, packed, N, K, q, s_x, M, y, acc, stream);
    }
}

static hipError_t launch_pf_reg(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                                int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    PfReg c;
    if (!pick_pf_reg(N, K, M, c)) return hipErrorNotSupported;
    if (c.KT == 2) return launch_pf_reg_kt<2>(c, packed, N, K, q, s_x, M, y, acc, stream);
    if (c.KT == 3) return launch_pf_reg_kt<3>(c, packed, N, K, q, s_x, M, y, acc, stream);
    if (c.MG == 2) return launch_pf_reg_mg<2>(c, packed, N, K, q, s_x, M, y, acc, stream);
    return launch_pf_reg_mg<3>(c, packed, N, K, q, s_x, M, y, acc, stream);
}

struct PfSmall {
    int MG, R, nw, XC;
    int64_t grid;
    size_t lds;
};

// Launch configuration of prefill_small_kernel, or false when it does not
// apply: nwr waves per row tile (the largest of 8, 4, 2 that divides the
// k-tiles and lets a phase of MG*16 activation rows fit in LDS), R row tiles
// per workgroup so that the grid covers the CUs about once (at most 12 waves,
// so that every instance keeps its registers without spills).
static bool pick_pf_small(int64_t N, int64_t K, int64_t M, PfSmall& c)
{
    if (K % kTileK != 0 || M < 17 || M > 64 || N < 1) return false;
    c.MG = (int)((M + 15) / 16);
    const int64_t nkt = K / kTileK, rows = 16 * c.MG;
    const int64_t nrt = (N + 15) / 16, cus = device_cus();
    for (int nwr : {8, 4, 2}) {
        if (nkt % nwr != 0) continue;
        const size_t stage_bytes = (size_t)rows * (nwr * kTileK + 16) + nwr * kTileK / 2 + 16;   // + dummy slot
        if (stage_bytes > (size_t)150 * 1024) continue;
        // about one workgroup per CU, and at least rows/32 row tiles per workgroup so that a
        // thread stages at most 8 activation chunks of a phase (rows/(4R) of them)
        int64_t R = (nrt + cus - 1) / cus;
        if (R < (rows + 31) / 32) R = (rows + 31) / 32;
        if (R * nwr > 12) continue;
        c.R = (int)R;
        c.nw = (int)(R * nwr);
        c.grid = (nrt + R - 1) / R;
        const int64_t chunks = rows * (nwr * kTileK / 32);
        const int64_t xc = (chunks + 64 * c.nw - 1) / (64 * c.nw);
        if (xc > 8) continue;
        c.XC = xc <= 2 ? 2 : (xc <= 4 ? 4 : (xc <= 6 ? 6 : 8));
        const size_t red_bytes = (size_t)c.nw * c.MG * 4 * 64 * 4;
        c.lds = stage_bytes > red_bytes ? stage_bytes : red_bytes;
        return c.lds <= (size_t)kCuLds;
    }
    return false;
}

template <int MG, int XC>
static hipError_t launch_pf_small_x(const PfSmall& c, const uint8_t* packed, int64_t N, int64_t K, const int8_t* q,
                                    const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    if (acc)
        prefill_small_kernel<MG, XC, true><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(
            packed, N, K, q, s_x, (int)M, y, acc, c.R);
    else
        prefill_small_kernel<MG, XC, false><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(
            packed, N, K, q, s_x, (int)M, y, acc, c.R);
    return hipGetLastError();
}

template <int MG>
static hipError_t launch_pf_small_mg(const PfSmall& c, const uint8_t* packed, int64_t N, int64_t K, const int8_t* q,
                                     const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    switch (c.XC) {
    case 2: return launch_pf_small_x<MG, 2>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 4: return launch_pf_small_x<MG, 4>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 6: return launch_pf_small_x<MG, 6>(c, packed, N, K, q, s_x, M, y, acc, stream);
    default: return launch_pf_small_x<MG, 8>(c, packed, N, K, q, s_x, M, y, acc, stream);
    }
}

static hipError_t launch_pf_small(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                                  int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    PfSmall c;
    if (!pick_pf_small(N, K, M, c)) return hipErrorNotSupported;
    switch (c.MG) {
    case 2: return launch_pf_small_mg<2>(c, packed, N, K, q, s_x, M, y, acc, stream);
    case 3: return launch_pf_small_mg<3>(c, packed, N, K, q, s_x, M, y, acc, stream);
    default: return launch_pf_small_mg<4>(c, packed, N, K, q, s_x, M, y, acc, stream);
    }
}

// The workgroup tile of the shared-decode kernel from the measured cost model described at
// its call in launch_prefill: true for 256 x 128, false for 128 x 64.
static bool pf2_big_tile(int64_t N, int64_t M)
{
    const int64_t cus = device_cus();
    const int64_t j_small = ((N + 63) / 64 * ((M + 127) / 128) + cus - 1) / cus;
    const int64_t j_big = ((N + 127) / 128 * ((M + 255) / 256) + cus - 1) / cus;
    const double small_us = j_small == 1 ? 0.65 : j_small == 2 ? 1.0 : j_small == 3 ? 1.5 : 0.48 * (double)j_small;
    return 1.6 * (double)j_big < small_us;
}

// Whether the shared-decode kernel takes the shape: from M = 128, and at 65 <= M < 128
// where a measured model puts it ahead of the other two paths there, the per-block kernel
// (about 0.62 us per 128-k block) and the int8 GEMV on 16-row slices (about 4 us plus the
// weight bytes at 5.3 TB/s per slice).  The shared-decode kernel alone on a CU takes about
// 0.65 us per block, and its K split in two adds about 5 us for the clear and the row
// scaling: 8B down at M = 96 / 112 / 127 42.8 / 49.9 / 56.9 us (GEMV slices) -> 36.5 / 37.2 /
// 37.6 us, down at M = 65 / 80 and gate at M = 65..127 keep their paths (33.1 / 35.9 us
// against 36.1 / 35.9 us, gate 24.0-25.2 us against 25.4-25.9 us).
static bool use_pf2(int64_t N, int64_t K, int64_t M)
{
    if (K % 512 != 0 || N < 1 || M < 65) return false;
    if (M >= 128) return true;
    const int64_t nb = K / kBlockK, cus = device_cus();
    const int64_t tiles = (N + 63) / 64;                        // 128 x 64 tiles, one row of them
    const int64_t j = (tiles + cus - 1) / cus;
    const double small_us = j == 1 ? 0.65 : j == 2 ? 1.0 : j == 3 ? 1.5 : 0.48 * (double)j;
    const double pf2_us = pf2_split(nb / 4, tiles) ? 0.65 * (double)(nb / 2) + 5.0 : small_us * (double)nb;
    const double pf_us = 0.62 * (double)nb;
    const double gemv_us = (double)((M + 15) / 16) * (4.0 + (double)N * (double)K * (0.265625 / 5.3e6));
    return pf2_us < pf_us && pf2_us < gemv_us;
}

bool prefill2_config(int64_t N, int64_t K, int64_t M, Pf2Config& c)
{
    if (!use_pf2(N, K, M)) return false;
    const bool big = pf2_big_tile(N, M);
    c.BM = big ? 256 : 128;
    c.BN = big ? 128 : 64;
    c.grid_x = (N + c.BN - 1) / c.BN;
    c.grid_y = (M + c.BM - 1) / c.BM;
    c.split = pf2_split(K / 512, c.grid_x * c.grid_y);
    c.grid_z = c.split ? 2 : 1;
    return true;
}

hipError_t launch_prefill(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                          int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    if (use_pf2(N, K, M)) {
        // workgroup-shared decode: 256 x 128 workgroup tiles (8 waves of 64 x 64, one
        // workgroup per CU) or 128 x 64 tiles (4 waves of 32 x 64, up to three per CU),
        // whichever a measured cost model favours.  Per 128-k block on the 8B shapes, a CU
        // with j tiles of 128 x 64 takes about 0.65, 1.0 and 1.5 us for j = 1, 2, 3 and
        // 0.48 j us beyond (they run three at a time); with j tiles of 256 x 128 (one at a
        // time) about 1.6 j us.  So the large tile wins where its tiles fill whole rounds
        // (gate M = 2048: 165 vs 184 us, down M = 2048: 139 vs 168 us, down M = 4096: 274
        // vs 314 us) and the small one elsewhere (gate M = 768 / 1024 / 1536: 76.8 / 91.2 /
        // 133.8 us against 106.8 / 108.1 / 159.8 us; down M = 1024 / 1536 / 3072: 90.6 /
        // 122.7 / 238.7 us against 99.5 / 136.3 / 269.3 us).
        if (pf2_big_tile(N, M)) return launch_pf2<4, 4, 4, 2>(packed, N, K, q, s_x, M, y, acc, stream);
        return launch_pf2<2, 4, 4, 1>(packed, N, K, q, s_x, M, y, acc, stream);
    }
    {   // 17 <= M <= 64, K <= 4096: activations held in registers, one wave per k-tile
        const hipError_t e = launch_pf_reg(packed, N, K, q, s_x, M, y, acc, stream);
        if (e != hipErrorNotSupported) return e;
    }
    {   // 17 <= M <= 64 above K = 4096: K split across the waves of a workgroup.  Measured
        // on the 8B shapes against the paths below (before the register-resident kernel took
        // K <= 4096): gate M = 64 16.2 us vs 24.6 us, down M = 64
        // 26.4 us vs 30.5 us, gate M = 32 10.6 us vs 12.5 us, gate M = 48 13.0 us vs 18.3 us.
        const hipError_t e = launch_pf_small(packed, N, K, q, s_x, M, y, acc, stream);
        if (e != hipErrorNotSupported) return e;
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
