// tern_quant.hip — per-row absmax int8 quantization of bf16 activations.
//   a = max_k |x[m][k]|, s = a / 127 (IEEE fp32 division, nearest-even),
//   q = clamp(rint(x / s), -127, 127) with the IEEE fp32 quotient and ties to
//   even; a == 0 gives s = 0, q = 0.  Bit-exact with any correct IEEE
//   implementation: the max is order-independent, and the division and
//   rounding are correctly rounded single operations.
#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __builtin_bit_cast(float, d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __builtin_bit_cast(float, d & 0xFFFF0000u); }

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                       int8_t* __restrict__ q, float* __restrict__ s_out)
{
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const u32x4* row = (const u32x4*)(x + m * K);
    const int64_t nchunk = K / 8;   // 8 bf16 per 16-byte chunk
    float a = 0.0f;
    for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
        const u32x4 v = row[c];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a = fmaxf(a, fabsf(bf16_lo(v[j])));
            a = fmaxf(a, fabsf(bf16_hi(v[j])));
        }
    }
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = __fdiv_rn(a, 127.0f);
    if (threadIdx.x == 0) s_out[m] = a == 0.0f ? 0.0f : s;
    u32x2* qrow = (u32x2*)(q + m * K);
    for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
        const u32x4 v = row[c];
        uint32_t out[2] = {0u, 0u};
        if (a != 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f0 = fminf(fmaxf(__builtin_rintf(__fdiv_rn(bf16_lo(v[j]), s)), -127.0f), 127.0f);
                const float f1 = fminf(fmaxf(__builtin_rintf(__fdiv_rn(bf16_hi(v[j]), s)), -127.0f), 127.0f);
                const uint32_t b = ((uint32_t)(int)f0 & 0xFFu) | (((uint32_t)(int)f1 & 0xFFu) << 8);
                out[j >> 1] |= b << (16 * (j & 1));
            }
        }
        u32x2 o;
        o[0] = out[0];
        o[1] = out[1];
        qrow[c] = o;
    }
}

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t stream)
{
    quantize_kernel<<<(unsigned)M, 256, 0, stream>>>(x, K, q, s);
    return hipGetLastError();
}

}  // namespace tern
