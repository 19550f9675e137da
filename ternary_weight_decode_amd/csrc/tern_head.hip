// tern_head.hip — int8 output-head GEMV with a per-row fp32 scale.
//
//   bf16 activations: logits[m][v] = rs[v] * sum_k W[v][k] * x[m][k]
//   int8 activations: acc[m][v] = sum_k W[v][k] * q[m][k] (exact int32),
//                     logits[m][v] = rs[v] * s_x[m] * acc[m][v]
//
// One wave owns a 16-row tile of W over the whole K (no cross-wave
// reduction); a workgroup of 4 waves shares the activations staged in LDS.
// Each lane streams 32 contiguous bytes of its row per 128-k unit, so a
// wave's load pair covers 16 full 128-byte lines.  bf16 path: int8 -> f32 via
// the byte-select convert (exact) -> bf16 pair by taking the high halves
// (exact: |w| <= 127 has 7 significant bits), then MFMA 16x16x32 bf16.
// int8 path: bytes go straight into MFMA 16x16x64 i8.
#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

constexpr int kHeadWaves = 4;

__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int lo_byte)
{
    const float f0 = (float)(int8_t)(w >> (8 * lo_byte));
    const float f1 = (float)(int8_t)(w >> (8 * lo_byte + 8));
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0), 0x07060302u);
}

// 32 int8 weights (8 dwords) -> 4 bf16 B operands (step c = weights 8c .. 8c+7)
__device__ __forceinline__ void head_decode_bf16(const u32x4& lo, const u32x4& hi, u32x4 (&B)[4])
{
    const uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        B[c][0] = i8x2_to_bf16x2(d[2 * c], 0);
        B[c][1] = i8x2_to_bf16x2(d[2 * c], 2);
        B[c][2] = i8x2_to_bf16x2(d[2 * c + 1], 0);
        B[c][3] = i8x2_to_bf16x2(d[2 * c + 1], 2);
    }
}

template <bool kInt8>
__global__ __launch_bounds__(256) void head_kernel(const int8_t* __restrict__ W, const float* __restrict__ rs,
                                                   int64_t V, int64_t K, const void* __restrict__ act,
                                                   const float* __restrict__ s_x, int M, float* __restrict__ y,
                                                   int32_t* __restrict__ acc_dbg, int kc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int64_t v0 = ((int64_t)blockIdx.x * kHeadWaves + wave) * kTileRows;
    const int64_t vrow = v0 + r < V ? v0 + r : V - 1;       // rows past V re-read the last row (dropped)
    const int ebytes = kInt8 ? 1 : 2;
    const int astride = kc * ebytes + 16;                  // bytes per staged activation row
    const int mrow = r < M ? r : M - 1;
    const int8_t* wrow = W + vrow * K + 32 * g;
    const int64_t nunit = K / kBlockK;
    const int64_t upc = kc / kBlockK;                      // 128-k units per chunk

    f32x4 accf = {0.f, 0.f, 0.f, 0.f};
    i32x4 acci = {0, 0, 0, 0};
    u32x4 cl, ch, nl, nh;
    const bool active = v0 < V;
    if (active) {
        cl = ld_nt16(wrow);
        ch = ld_nt16(wrow + 16);
    }
    int64_t u = 0;
    const int64_t nchunks = (nunit + upc - 1) / upc;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t k0 = c * kc;
        const int64_t kcl = (K - k0) < kc ? (K - k0) : kc;
        if (c > 0) __syncthreads();
        {
            const int64_t per_row = kcl * ebytes / 16;
            const int64_t units = (int64_t)M * per_row;
            const uint8_t* src = (const uint8_t*)act;
            for (int64_t i = threadIdx.x; i < units; i += blockDim.x) {
                const int64_t m = i / per_row, c16 = i % per_row;
                *(u32x4*)(smem + m * astride + 16 * c16) = *(const u32x4*)(src + (m * K + k0) * ebytes + 16 * c16);
            }
        }
        __syncthreads();
        const int64_t u_end = (c + 1) * upc < nunit ? (c + 1) * upc : nunit;
        if (active) {
            for (; u < u_end; ++u) {
                if (u + 1 < nunit) {
                    nl = ld_nt16(wrow + (u + 1) * kBlockK);
                    nh = ld_nt16(wrow + (u + 1) * kBlockK + 16);
                }
                const uint8_t* arow = smem + mrow * astride + ((u * kBlockK - k0) + 32 * g) * ebytes;
                if constexpr (kInt8) {
                    acci = mfma_i8(*(const u32x4*)(arow), cl, acci);
                    acci = mfma_i8(*(const u32x4*)(arow + 16), ch, acci);
                } else {
                    u32x4 B[4];
                    head_decode_bf16(cl, ch, B);
#pragma unroll
                    for (int s = 0; s < 4; ++s) accf = mfma_bf16(*(const u32x4*)(arow + 16 * s), B[s], accf);
                }
                cl = nl;
                ch = nh;
            }
        }
    }
    if (!active) return;
    const int64_t v = v0 + r;
    if (v >= V) return;
    const float sv = rs[v];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < M) {
            if constexpr (kInt8) {
                y[(int64_t)m * V + v] = sv * s_x[m] * (float)acci[i];
                if (acc_dbg) acc_dbg[(int64_t)m * V + v] = acci[i];
            } else {
                y[(int64_t)m * V + v] = sv * accf[i];
            }
        }
    }
}

static int head_chunk(int64_t K, int64_t M, int ebytes)
{
    int64_t cap = (48 * 1024) / (M * ebytes) / kBlockK * kBlockK;
    if (cap < kBlockK) cap = kBlockK;
    return (int)(K < cap ? K : cap);
}

hipError_t launch_head_bf16(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                            float* y, hipStream_t stream)
{
    const int kc = head_chunk(K, M, 2);
    const size_t lds = (size_t)M * (kc * 2 + 16);
    const unsigned grid = (unsigned)((V + 16 * kHeadWaves - 1) / (16 * kHeadWaves));
    head_kernel<false><<<grid, 64 * kHeadWaves, lds, stream>>>(W, rs, V, K, x, nullptr, (int)M, y, nullptr, kc);
    return hipGetLastError();
}

hipError_t launch_head_i8(const int8_t* W, const float* rs, int64_t V, int64_t K, const int8_t* q,
                          const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    const int kc = head_chunk(K, M, 1);
    const size_t lds = (size_t)M * (kc + 16);
    const unsigned grid = (unsigned)((V + 16 * kHeadWaves - 1) / (16 * kHeadWaves));
    head_kernel<true><<<grid, 64 * kHeadWaves, lds, stream>>>(W, rs, V, K, q, s_x, (int)M, y, acc, kc);
    return hipGetLastError();
}

}  // namespace tern
