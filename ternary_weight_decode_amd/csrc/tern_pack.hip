// tern_pack.hip — load-time packing of ternary weights into the plane blob,
// occupancy statistics of a blob, and a zero-fill helper.
#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

// One thread per (row n < Np, block b, word w): reads the 32 int8 states of
// the word (32 contiguous bytes of t) and writes its nonzero word and sign word.
// Threads with w == 0 also write the block's fp16 scale.  Rows n >= N are
// padding and are written as zeros.
__global__ void pack_kernel(const int8_t* __restrict__ t, const uint16_t* __restrict__ scale, int64_t N, int64_t K,
                            uint32_t* __restrict__ words, uint16_t* __restrict__ scales)
{
    const int64_t nb = K / kBlockK;
    const int64_t total = npad16(N) * nb * 4;
    for (int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tid < total;
         tid += (int64_t)gridDim.x * blockDim.x) {
        const int w = (int)(tid & 3);
        const int64_t b = (tid >> 2) % nb;
        const int64_t n = (tid >> 2) / nb;
        uint32_t nz = 0, sg = 0;
        if (n < N) {
            const u32x4* src = (const u32x4*)(t + n * K + b * kBlockK + 32 * w);
            const u32x4 lo = src[0], hi = src[1];
            const uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int v = (int)(int8_t)(d[i >> 2] >> (8 * (i & 3)));
                const int pos = 16 * (i & 1) + (i >> 1);
                nz |= (uint32_t)(v != 0) << pos;
                sg |= (uint32_t)(v < 0) << pos;
            }
        }
        const int64_t rt = n >> 4, r = n & 15, kt = b >> 2, bq = b & 3;
        const int64_t nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
        const int64_t base = tile_word_base(rt, kt, nb);
        words[base + ((0 * 4 + w) * 16 + r) * nbq + bq] = nz;
        words[base + ((1 * 4 + w) * 16 + r) * nbq + bq] = sg;
        if (w == 0) scales[tile_scale_base(rt, kt, nb) + r * nbq + bq] = n < N ? scale[n * nb + b] : (uint16_t)0;
    }
}

__global__ void zero_u64_kernel(uint64_t* p, int n)
{
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

// Counts over the N real rows: nonzero bits, nonzero&sign bits, and sign bits
// without a nonzero bit (non-canonical).  Integer atomics: order-independent.
__global__ void stats_kernel(const uint32_t* __restrict__ words, int64_t N, int64_t K, uint64_t* __restrict__ counts)
{
    const int64_t nb = K / kBlockK;
    const int64_t total = N * nb * 4;
    uint64_t c0 = 0, c1 = 0, c2 = 0;
    for (int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tid < total;
         tid += (int64_t)gridDim.x * blockDim.x) {
        const int w = (int)(tid & 3);
        const int64_t b = (tid >> 2) % nb;
        const int64_t n = (tid >> 2) / nb;
        const int64_t rt = n >> 4, r = n & 15, kt = b >> 2, bq = b & 3;
        const int64_t nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
        const int64_t base = tile_word_base(rt, kt, nb);
        const uint32_t nz = words[base + ((0 * 4 + w) * 16 + r) * nbq + bq];
        const uint32_t sg = words[base + ((1 * 4 + w) * 16 + r) * nbq + bq];
        c0 += __builtin_popcount(nz);
        c1 += __builtin_popcount(nz & sg);
        c2 += __builtin_popcount(~nz & sg);
    }
    for (int off = 32; off > 0; off >>= 1) {
        c0 += __shfl_down(c0, off);
        c1 += __shfl_down(c1, off);
        c2 += __shfl_down(c2, off);
    }
    if ((threadIdx.x & 63) == 0) {
        atomicAdd((unsigned long long*)&counts[0], (unsigned long long)c0);
        atomicAdd((unsigned long long*)&counts[1], (unsigned long long)c1);
        atomicAdd((unsigned long long*)&counts[2], (unsigned long long)c2);
    }
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

static unsigned grid_for(int64_t items, int threads, int64_t cap = 65536)
{
    int64_t g = (items + threads - 1) / threads;
    if (g < 1) g = 1;
    return (unsigned)(g < cap ? g : cap);
}

hipError_t launch_fill_zero(void* dst, int64_t bytes, hipStream_t stream)
{
    const int64_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    fill_zero_kernel<<<grid_for(n, 256, 4096), 256, 0, stream>>>((uint32_t*)dst, n);
    return hipGetLastError();
}

hipError_t launch_pack(const int8_t* t, const uint16_t* scale, int64_t N, int64_t K, uint8_t* packed,
                       hipStream_t stream)
{
    const int64_t items = npad16(N) * (K / kBlockK) * 4;
    pack_kernel<<<grid_for(items, 256), 256, 0, stream>>>(t, scale, N, K, (uint32_t*)packed,
                                                          (uint16_t*)(packed + scale_region_offset(N, K)));
    return hipGetLastError();
}

hipError_t launch_stats(const uint8_t* packed, int64_t N, int64_t K, uint64_t* counts, hipStream_t stream)
{
    zero_u64_kernel<<<1, 64, 0, stream>>>(counts, 3);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = N * (K / kBlockK) * 4;
    if (items == 0) return hipSuccess;
    stats_kernel<<<grid_for(items, 256, 2048), 256, 0, stream>>>((const uint32_t*)packed, N, K, counts);
    return hipGetLastError();
}

}  // namespace tern
