// tern_peak.hip — measurement probes; they compute nothing of the method.
//
// Matrix-core throughput: independent MFMA chains on registers with no
// memory traffic inside the loop, so the achieved rate is the chip's
// sustained matrix-core rate for that instruction.  It is the denominator
// check for the prefill contraction (int8 16x16x64) and the GEMV's bf16
// 16x16x32 steps.
//
// Launch floor and read ceiling: the cost of one dependent launch of a
// kernel that does (almost) nothing, and the rate at which a plain streaming
// read moves bytes out of HBM; a GEMV launch at M = 1 costs about the floor
// of a launch with one cold load plus its bytes at the read ceiling.
#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

constexpr int kPeakChains = 8;      // independent accumulators per wave (covers the MFMA latency)
constexpr int kPeakWaves = 4;       // waves per workgroup

// Each wave runs kPeakChains dependent chains of `iters` MFMAs.  Operands
// depend on the lane and the loop counter stays opaque to the compiler, so
// no MFMA is folded away; every accumulator is stored at the end.
template <int kKind>
__global__ __launch_bounds__(64 * kPeakWaves) void mfma_peak_kernel(int64_t iters, int32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const uint32_t a0 = 0x01010101u * (uint32_t)(lane + 1), b0 = 0x02030405u ^ (uint32_t)lane;
    u32x4 a = {a0, a0 ^ 1u, a0 ^ 2u, a0 ^ 3u}, b = {b0, b0 + 1u, b0 + 2u, b0 + 3u};
    if constexpr (kKind == 0) {
        i32x4 c[kPeakChains];
#pragma unroll
        for (int j = 0; j < kPeakChains; ++j) c[j] = i32x4{lane + j, lane ^ j, 3 * lane + j, lane - j};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kPeakChains; ++j) c[j] = mfma_i8(a, b, c[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        i32x4 s = c[0];
#pragma unroll
        for (int j = 1; j < kPeakChains; ++j) s += c[j];
        *(i32x4*)(sink + ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4) = s;
    } else {
        // bf16 operands kept finite and small: exponent bits of 1.0 with lane-dependent mantissas
        a = (a & 0x007F007Fu) | 0x3F803F80u;
        b = (b & 0x007F007Fu) | 0x3F803F80u;
        f32x4 c[kPeakChains];
#pragma unroll
        for (int j = 0; j < kPeakChains; ++j)
            c[j] = f32x4{(float)(lane + j), (float)(lane ^ j), (float)(3 * lane + j), (float)(lane - j)};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kPeakChains; ++j) c[j] = mfma_bf16(a, b, c[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x4 s = c[0];
#pragma unroll
        for (int j = 1; j < kPeakChains; ++j) s += c[j];
        *(f32x4*)(sink + ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4) = s;
    }
}

double mfma_peak_ops(int kind, int64_t iters, int64_t grid)
{
    const double per_mfma = kind == 0 ? 2.0 * 16 * 16 * 64 : 2.0 * 16 * 16 * 32;
    return per_mfma * (double)iters * kPeakChains * kPeakWaves * (double)grid;
}

int64_t mfma_peak_sink_ints(int64_t grid) { return grid * 64 * kPeakWaves * 4; }

hipError_t launch_mfma_peak(int kind, int64_t iters, int64_t grid, int32_t* sink, hipStream_t stream)
{
    if (kind == 0) mfma_peak_kernel<0><<<dim3((unsigned)grid), dim3(64 * kPeakWaves), 0, stream>>>(iters, sink);
    else mfma_peak_kernel<1><<<dim3((unsigned)grid), dim3(64 * kPeakWaves), 0, stream>>>(iters, sink);
    return hipGetLastError();
}

// ---- launch floor / read ceiling -------------------------------------------

__global__ __launch_bounds__(64) void probe_empty_kernel() {}

// one float per workgroup
__global__ __launch_bounds__(512) void probe_store_kernel(float* __restrict__ sink)
{
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)blockIdx.x;
}

// one 16-byte load per thread (index clamped to the buffer), then one float per workgroup
__global__ __launch_bounds__(512) void probe_load_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         float* __restrict__ sink)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const u32x4 v = src[i < n16 ? i : n16 - 1];
    const uint32_t a = v[0] ^ v[1] ^ v[2] ^ v[3];
    // never true for the zero-filled buffers the probe is given; keeps the load
    if (a == 0x9E3779B9u) sink[blockIdx.x] = -1.0f;
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)blockIdx.x;
}

// the whole buffer read once: grid-stride 16-byte loads, eight in flight per thread
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         float* __restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t a = 0;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; base < n16; base += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t i = base + j * stride;
            v[j] = src[i < n16 ? i : n16 - 1];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) a ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    if (a == 0x9E3779B9u) sink[blockIdx.x] = -1.0f;
}

hipError_t launch_probe(int kind, int64_t grid, const void* src, int64_t src_bytes, float* sink, hipStream_t stream)
{
    const dim3 g((unsigned)grid);
    if (kind == 0) probe_empty_kernel<<<g, 64, 0, stream>>>();
    else if (kind == 1) probe_store_kernel<<<g, 512, 0, stream>>>(sink);
    else if (kind == 2) probe_load_kernel<<<g, 512, 0, stream>>>((const u32x4*)src, src_bytes / 16, sink);
    else probe_read_kernel<<<g, 256, 0, stream>>>((const u32x4*)src, src_bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace tern
