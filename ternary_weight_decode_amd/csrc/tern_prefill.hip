// tern_prefill.hip — prefill-size ternary GEMM on the int8 matrix cores.
//
//   acc[m][n][b] = sum_{k in block b} t[n][k] * q[m][k]   (exact int32)
//   y[m][n]      = s_x[m] * sum_b scale[n][b] * acc[m][n][b]
//
// Workgroup tile 128 (m) x 128 (n), four waves of 64 x 64.  Each wave decodes
// the planes of its four 16-row weight tiles straight into MFMA B operands
// (bytes 64*t, one rotate+mask per 4 weights), reuses each decoded block
// across its four 16-row activation tiles, and folds every block's int32
// result into fp32 with that block's scale (cvt + fma per output element per
// block).  Activations are staged one 128-k block at a time in LDS (double
// buffered, byte order matching the decoded weights).
#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

constexpr int kPfBM = 128, kPfBN = 128;
constexpr int kPfAStride = kBlockK + 16;    // bytes per staged activation row (pad against bank conflicts)

__global__ __launch_bounds__(256) void prefill_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                      const int8_t* __restrict__ q, const float* __restrict__ s_x,
                                                      int64_t M, float* __restrict__ y,
                                                      int32_t* __restrict__ acc_dbg)
{
    __shared__ __align__(16) uint8_t abuf[2][kPfBM * kPfAStride];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t m0 = (int64_t)blockIdx.y * kPfBM, n0 = (int64_t)blockIdx.x * kPfBN;
    const int64_t nb = K / kBlockK;
    const int64_t nrt = (N + 15) / 16;
    const uint32_t* words = (const uint32_t*)packed;
    const uint16_t* scales = (const uint16_t*)(packed + scale_region_offset(N, K));

    // this wave's four weight row tiles
    int64_t rts[4];
    bool rt_ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        rts[j] = (n0 >> 4) + 4 * wn + j;
        rt_ok[j] = rts[j] < nrt;
    }

    // staging: thread -> (row, 32-byte unit): 128 rows x 4 units = 512 units, 2 per thread
    auto stage_load = [&](int64_t b, u32x4 (&st)[4]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int unit = threadIdx.x + 256 * h;
            const int row = unit >> 2, c32 = unit & 3;
            const int64_t m = m0 + row < M ? m0 + row : M - 1;
            const u32x4* src = (const u32x4*)(q + m * K + b * kBlockK + 32 * c32);
            st[2 * h] = src[0];
            st[2 * h + 1] = src[1];
        }
    };
    auto stage_store = [&](int buf, const u32x4 (&st)[4]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int unit = threadIdx.x + 256 * h;
            const int row = unit >> 2, c32 = unit & 3;
            const uint32_t Q[8] = {st[2 * h][0], st[2 * h][1], st[2 * h][2], st[2 * h][3],
                                   st[2 * h + 1][0], st[2 * h + 1][1], st[2 * h + 1][2], st[2 * h + 1][3]};
            u32x4 o0, o1;
#pragma unroll
            for (int d = 0; d < 4; ++d) o0[d] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
#pragma unroll
            for (int d = 4; d < 8; ++d) o1[d - 4] = i8_act_quad(Q[d >> 1], Q[4 + (d >> 1)], d);
            u32x4* dst = (u32x4*)(&abuf[buf][row * kPfAStride + 32 * c32]);
            dst[0] = o0;
            dst[1] = o1;
        }
    };

    f32x4 facc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) facc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 st[4];
    stage_load(0, st);
    stage_store(0, st);

    u32x4 pnz[4], psg[4];
    u32x2 psc[4];
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t kt = b >> 2;
        const int bq = (int)(b & 3);
        const int nbq = (int)(nb - 4 * kt < 4 ? nb - 4 * kt : 4);
        if (bq == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!rt_ok[j]) {
                    pnz[j] = u32x4{0, 0, 0, 0};
                    psg[j] = u32x4{0, 0, 0, 0};
                    psc[j] = u32x2{0, 0};
                    continue;
                }
                const int64_t wb = tile_word_base(rts[j], kt, nb);
                const int64_t sb = tile_scale_base(rts[j], kt, nb);
                if (nbq == 4) {
                    pnz[j] = ld_nt16(words + wb + (int64_t)((0 * 4 + g) * 16 + r) * 4);
                    psg[j] = ld_nt16(words + wb + (int64_t)((1 * 4 + g) * 16 + r) * 4);
                    psc[j] = ld_nt8(scales + sb + r * 4);
                } else {
                    uint32_t s01 = 0, s23 = 0;
                    for (int e = 0; e < 4; ++e) {
                        const bool in = e < nbq;
                        pnz[j][e] = in ? words[wb + (int64_t)((0 * 4 + g) * 16 + r) * nbq + e] : 0u;
                        psg[j][e] = in ? words[wb + (int64_t)((1 * 4 + g) * 16 + r) * nbq + e] : 0u;
                        const uint32_t h = in ? (uint32_t)scales[sb + r * nbq + e] : 0u;
                        if (e < 2) s01 |= h << (16 * e);
                        else s23 |= h << (16 * (e - 2));
                    }
                    psc[j] = u32x2{s01, s23};
                }
            }
        }
        const bool more = b + 1 < nb;
        if (more) stage_load(b + 1, st);
        __syncthreads();   // block b staged by every thread

        const int buf = (int)(b & 1);
        u32x4 A[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint8_t* arow = &abuf[buf][(64 * wm + 16 * i + r) * kPfAStride + 32 * g];
            A[i][0] = *(const u32x4*)(arow);
            A[i][1] = *(const u32x4*)(arow + 16);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 B0, B1;
            {
                const CodeWords c = interleave(pnz[j][bq], psg[j][bq]);
                B0 = u32x4{i8_quad<0>(c), i8_quad<1>(c), i8_quad<2>(c), i8_quad<3>(c)};
                B1 = u32x4{i8_quad<4>(c), i8_quad<5>(c), i8_quad<6>(c), i8_quad<7>(c)};
            }
            const uint32_t sw = psc[j][bq >> 1];
            const float sc = half_bits_to_float((sw >> (16 * (bq & 1))) & 0xFFFFu) * (1.0f / 64.0f);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                i32x4 d = {0, 0, 0, 0};
                d = mfma_i8(A[i][0], B0, d);
                d = mfma_i8(A[i][1], B1, d);
#pragma unroll
                for (int e = 0; e < 4; ++e) facc[i][j][e] = __builtin_fmaf(sc, (float)d[e], facc[i][j][e]);
                if (acc_dbg) {
                    const int64_t n = (rts[j] << 4) + r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t m = m0 + 64 * wm + 16 * i + 4 * g + e;
                        if (m < M && n < N) acc_dbg[(m * N + n) * nb + b] = d[e] >> 6;
                    }
                }
            }
        }
        if (more) stage_store((int)((b + 1) & 1), st);
        __syncthreads();   // next buffer complete; current buffer free for block b+2
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = (rts[j] << 4) + r;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + 64 * wm + 16 * i + 4 * g + e;
                if (m < M) y[m * N + n] = s_x[m] * facc[i][j][e];
            }
    }
}

hipError_t launch_prefill(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                          int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + kPfBN - 1) / kPfBN), (unsigned)((M + kPfBM - 1) / kPfBM));
    prefill_kernel<<<grid, 256, 0, stream>>>(packed, N, K, q, s_x, M, y, acc);
    return hipGetLastError();
}

}  // namespace tern
