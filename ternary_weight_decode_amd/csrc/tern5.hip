// tern5.hip — five-level (FV5-style) weights: load-time packing and the
// bf16 GEMV / small-M GEMM on the gfx950 matrix cores.
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
// in LDS in k-tile order.  XC = 16-byte activation chunks per thread.
template <int MT, int U, int XC>
__global__ __launch_bounds__(1024) void gemv5_oneshot_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                             const uint16_t* __restrict__ x, int M,
                                                             float* __restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NI = MT < 4 ? MT : 4;
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
    const int xrow_bytes = ((int)K + 8) * 2;
    float* red = (float*)(smem + (size_t)M * xrow_bytes);  // [unit + 1 spare][NI][64]

    // activations first; a chunk index past the end re-loads the last chunk
    // and stores it to a dummy slot (the start of the partials, written only
    // after the barrier), so every load is issued and used unconditionally
    const int per_row = (int)(K * 2 / 16), chunks = M * per_row;
    u32x4 xv[XC];
    int xdst[XC];
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const int u = threadIdx.x + c * nthreads;
        const int uc = u < chunks ? u : chunks - 1;
        const int m = uc / per_row, cc = uc - m * per_row;
        xv[c] = xg[(int64_t)m * per_row + cc];
        xdst[c] = u < chunks ? m * xrow_bytes + 16 * cc : M * xrow_bytes;
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
    for (int c = 0; c < XC; ++c) *(u32x4*)(smem + xdst[c]) = xv[c];
    __syncthreads();
#pragma unroll
    for (int i = 1; i < U; ++i) {
        load_unit(i);
        __builtin_amdgcn_sched_barrier(0);
    }

    const int mrow = r < M ? r : M - 1;
    const uint16_t* xrow = (const uint16_t*)(smem + mrow * xrow_bytes) + 32 * g;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int j = wave + i * nw;
        const int jc = j < units ? j : units - 1;
        const int kt = jc - (jc / nkt) * nkt;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile5_bf16<MT>(t[i], xrow + kt * kTileK, acc);
        const int slot = j < units ? j : units;
#pragma unroll
        for (int q = 0; q < NI; ++q) red[(slot * NI + q) * 64 + lane] = acc[q];
        __builtin_amdgcn_sched_barrier(0);
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
            y[(int64_t)m * N + row] = sum;
        }
    }
}

// Any shape: one workgroup per row tile, its waves split the k-tiles
// round-robin, activations read from global memory (cached), partials summed
// in LDS in wave order.
template <int MT>
__global__ __launch_bounds__(512) void gemv5_kernel(const uint8_t* __restrict__ packed, int64_t N, int64_t K,
                                                    const uint16_t* __restrict__ x, int M, float* __restrict__ y)
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
    const uint16_t* xr = x + (int64_t)mrow * K + 32 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kt = wave; kt < nkt; kt += nw) {
        const Tile5 t = load_tile5(words, scales, rt, kt, nkt, r, g);
        tile5_bf16<MT>(t, xr + (int64_t)kt * kTileK, acc);
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
            y[(int64_t)m * N + row] = sum;
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

template <int MT>
static hipError_t gemv5_oneshot_dispatch(const OneShot& c, hipStream_t stream, const uint8_t* packed, int64_t N,
                                         int64_t K, const uint16_t* x, int M, float* y)
{
#define TERN5_CASE(UU, XX)                                                                                     \
    if (c.U == UU && c.XC == XX) {                                                                             \
        if (!oneshot_resident(gemv5_oneshot_kernel<MT, UU, XX>, c)) return hipErrorNotSupported;              \
        gemv5_oneshot_kernel<MT, UU, XX><<<dim3((unsigned)c.grid), dim3(64 * c.nw), c.lds, stream>>>(          \
            packed, N, K, x, M, y);                                                                            \
        return hipGetLastError();                                                                              \
    }
    TERN5_CASE(1, 1) TERN5_CASE(2, 1) TERN5_CASE(3, 1) TERN5_CASE(4, 1)
    TERN5_CASE(1, 2) TERN5_CASE(2, 2) TERN5_CASE(3, 2) TERN5_CASE(4, 2)
    TERN5_CASE(1, 4) TERN5_CASE(2, 4) TERN5_CASE(3, 4) TERN5_CASE(4, 4)
    if constexpr (MT == 16) {
        TERN5_CASE(1, 8) TERN5_CASE(2, 8) TERN5_CASE(3, 8) TERN5_CASE(4, 8)
    }
#undef TERN5_CASE
    return hipErrorNotSupported;
}

// Waves of U = 1..4 units per SIMD (registers of the M <= 4 instances; the
// occupancy query has the last word).
static const OneShotShape kFiveShape = {0, 0, 16, {0, 8, 6, 4, 4}};

hipError_t launch_gemv5_bf16(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                             hipStream_t stream)
{
    OneShotShape s = kFiveShape;
    s.x_row_bytes = (K + 8) * 2;
    s.x_src_bytes = 2 * K;
    OneShot c;
    if (pick_oneshot(N, K, M, s, c)) {
        const int m = (int)M;
        const bool wide = M > 4 || c.XC == 8;
        hipError_t e;
        if (wide) e = gemv5_oneshot_dispatch<16>(c, stream, packed, N, K, x, m, y);
        else if (M == 1) e = gemv5_oneshot_dispatch<1>(c, stream, packed, N, K, x, m, y);
        else if (M == 2) e = gemv5_oneshot_dispatch<2>(c, stream, packed, N, K, x, m, y);
        else e = gemv5_oneshot_dispatch<4>(c, stream, packed, N, K, x, m, y);
        if (e != hipErrorNotSupported) return e;
    }
    const int64_t nkt = K / kTileK;
    const int nw = nkt >= 8 ? 8 : (int)nkt;
    const dim3 grid((unsigned)((N + 15) / 16)), block(64 * nw);
    if (M == 1) gemv5_kernel<1><<<grid, block, 0, stream>>>(packed, N, K, x, (int)M, y);
    else if (M == 2) gemv5_kernel<2><<<grid, block, 0, stream>>>(packed, N, K, x, (int)M, y);
    else if (M <= 4) gemv5_kernel<4><<<grid, block, 0, stream>>>(packed, N, K, x, (int)M, y);
    else gemv5_kernel<16><<<grid, block, 0, stream>>>(packed, N, K, x, (int)M, y);
    return hipGetLastError();
}

}  // namespace tern
