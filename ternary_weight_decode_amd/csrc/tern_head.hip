// tern_head.hip — int8 output-head GEMV with a per-row fp32 scale.
//
//   bf16 activations: logits[m][v] = rs[v] * sum_k W[v][k] * x[m][k]
//   int8 activations: acc[m][v] = sum_k W[v][k] * q[m][k] (exact int32),
//                     logits[m][v] = rs[v] * s_x[m] * acc[m][v]
//
// One wave owns a 16-row tile of W over the whole K (no cross-wave
// reduction); a workgroup of 4 waves shares the activations staged in LDS.
// Each wave keeps a ring of loads in flight (depth chosen by the launcher).
// Per 128-k unit, lane (row r, group g) loads bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of its row, so each of a wave's two loads covers whole
// 64-byte halves of 16 rows' lines (a line half is never requested twice);
// the activations are read at the matching k.  bf16 path: int8 -> f32 via
// the byte-select convert (exact) -> bf16 pair by taking the high halves
// (exact: |w| <= 127 has 7 significant bits), then MFMA 16x16x32 bf16.
// int8 path: bytes go straight into MFMA 16x16x64 i8.
#include <mutex>

#include "tern_device.h"
#include "tern_launch.h"

namespace tern {

constexpr int kHeadWaves = 4;
constexpr int kHeadUnitBytes = kTileRows * kBlockK;   // one wave's 128-k unit: 16 rows x 128 bytes
// byte offsets, within a lane's k range of a 128-k unit, of the four bf16 MFMA
// steps' activations: k = 16g + {0, 8} and 64 + 16g + {0, 8} (2 bytes each)
__device__ constexpr int kHalfOff[4] = {0, 16, 128, 144};
#ifndef TERN_HEAD_TPW
#define TERN_HEAD_TPW 4
#endif
constexpr int kHeadTpw = TERN_HEAD_TPW;   // 128-k units in flight per wave (single-chunk path)
#ifndef TERN_HEAD_PACKED_TPW
#define TERN_HEAD_PACKED_TPW 8
#endif
constexpr int kHeadPackedTpw = TERN_HEAD_PACKED_TPW;   // the same, packed layout
// 16-byte load of head weights.  Plain (cached) loads: with non-temporal ones
// the head fetched about 10% more bytes from HBM than it reads and ran ~13%
// slower at every ring depth measured (V = 151936, K = 4096).
__device__ __forceinline__ u32x4 head_ld16(const int8_t* p) { return *(const u32x4*)p; }

__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int lo_byte)
{
    const float f0 = (float)(int8_t)(w >> (8 * lo_byte));
    const float f1 = (float)(int8_t)(w >> (8 * lo_byte + 8));
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0), 0x07060302u);
}

// 32 int8 weights (lo then hi, 8 dwords) -> 4 bf16 B operands (step c = bytes 8c .. 8c+7 of lo, hi)
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

// Head kernel: wave q of the grid owns row tiles q, q + Q, q + 2Q, ...
// (Q = total waves; the launcher gives every wave one row tile) over the
// whole K and keeps a ring of TPW 128-k units (32 bytes per lane each) in
// flight, across row-tile boundaries when a wave has several.  Activations (all of K, or a chunk of it when
// M*K is large) are staged in LDS once per workgroup.
template <bool kInt8, int TPW>
__global__ __launch_bounds__(256) void head_kernel(const int8_t* __restrict__ W, const float* __restrict__ rs,
                                                   int64_t V, int64_t K, const void* __restrict__ act,
                                                   const float* __restrict__ s_x, int M, float* __restrict__ y,
                                                   int32_t* __restrict__ acc_dbg, int kc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int ebytes = kInt8 ? 1 : 2;
    const int astride = kc * ebytes + 16;                  // bytes per staged activation row
    const int mrow = r < M ? r : M - 1;
    const int nunit = (int)(K / kBlockK);                  // 128-k units per row
    const int upc = kc / kBlockK;                          // units per staged chunk
    const int nchunks = (nunit + upc - 1) / upc;
    const int64_t nrt = (V + 15) >> 4;
    const int64_t q0 = (int64_t)blockIdx.x * kHeadWaves + wave, qstep = (int64_t)gridDim.x * kHeadWaves;
    const int nmy = q0 < nrt ? (int)((nrt - 1 - q0) / qstep + 1) : 0;

    // units of this wave in order: (row tile i, unit j), j fastest; chunk c covers units [c*upc, (c+1)*upc)
    // With one chunk (kc >= K) the ring spans row tiles; with several chunks the
    // chunk loop is outermost and every row tile is revisited per chunk.
    for (int c = 0; c < nchunks; ++c) {
        const int j_lo = c * upc, j_hi = (c + 1) * upc < nunit ? (c + 1) * upc : nunit;
        const int Jc = j_hi - j_lo;
        const int U = nmy * Jc;
        u32x4 lo[TPW], hi[TPW];
        int li = 0, lj = 0;
        auto load = [&](int s) {
            int64_t v = (q0 + li * qstep) * kTileRows + r;
            v = v < V ? v : V - 1;                         // rows past V re-read the last row (outputs dropped)
            const int8_t* p = W + v * K + (int64_t)(j_lo + lj) * kBlockK + 16 * g;
            lo[s] = head_ld16(p);
            hi[s] = head_ld16(p + 64);
            if (++lj == Jc) { lj = 0; ++li; }
        };
#pragma unroll
        for (int s = 0; s < TPW; ++s)
            if (s < U) load(s);

        if (c > 0) __syncthreads();                        // previous chunk's activations no longer read
        {
            const int64_t k0 = (int64_t)j_lo * kBlockK;
            const int per_row = Jc * kBlockK * ebytes / 16;
            const int units = M * per_row;
            const uint8_t* src = (const uint8_t*)act;
            for (int i = threadIdx.x; i < units; i += blockDim.x) {
                const int m = i / per_row, c16 = i - m * per_row;
                *(u32x4*)(smem + m * astride + 16 * c16) = *(const u32x4*)(src + ((int64_t)m * K + k0) * ebytes + 16 * c16);
            }
        }
        __syncthreads();

        f32x4 accf = {0.f, 0.f, 0.f, 0.f};
        i32x4 acci = {0, 0, 0, 0};
        int pi = 0, pj = 0;
        for (int u0 = 0; u0 < U; u0 += TPW) {
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                if (u0 + s < U) {
                    const uint8_t* arow = smem + mrow * astride + (pj * kBlockK + 16 * g) * ebytes;
                    if constexpr (kInt8) {
                        acci = mfma_i8(*(const u32x4*)(arow), lo[s], acci);
                        acci = mfma_i8(*(const u32x4*)(arow + 64), hi[s], acci);
                    } else {
                        u32x4 B[4];
                        head_decode_bf16(lo[s], hi[s], B);
#pragma unroll
                        for (int t = 0; t < 4; ++t) accf = mfma_bf16(*(const u32x4*)(arow + kHalfOff[t]), B[t], accf);
                    }
                    if (u0 + s + TPW < U) load(s);
                    if (++pj == Jc) {                      // row tile pi: this chunk's part is complete
                        const int64_t v = (q0 + pi * qstep) * kTileRows + r;
                        if (v < V) {
                            const float sv = rs[v];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int m = 4 * g + i;
                                if (m < M) {
                                    float* yp = y + (int64_t)m * V + v;
                                    if constexpr (kInt8) {
                                        // with several chunks, logits add per-chunk products; acc_dbg adds exactly
                                        *yp = (c == 0 ? 0.0f : *yp) + sv * s_x[m] * (float)acci[i];
                                        if (acc_dbg) acc_dbg[(int64_t)m * V + v] = (c == 0 ? 0 : acc_dbg[(int64_t)m * V + v]) + acci[i];
                                    } else {
                                        *yp = (c == 0 ? 0.0f : *yp) + sv * accf[i];
                                    }
                                }
                            }
                        }
                        accf = f32x4{0.f, 0.f, 0.f, 0.f};
                        acci = i32x4{0, 0, 0, 0};
                        pj = 0;
                        ++pi;
                    }
                }
            }
        }
    }
}

// Greedy argmax fused into the head: per activation row m, the row v with the
// largest logit, the lowest v among equal logits (-0 counted as +0).  Each
// logit becomes a 64-bit key {order-preserving bits of the value, ~v}, so one
// unsigned maximum decides both.  Every wave reduces its 16 rows in
// registers and stores one key per m in its own slot of the workspace
// (row tile q, row m); a second kernel takes the maximum over the slots.  No
// atomics and no fences: the launch boundary makes the slots visible, and the
// result does not depend on the order in which waves finish.
struct HeadArgmax {
    unsigned long long* part;   // [row tiles][M] keys, or null: no argmax
};

__device__ __forceinline__ uint32_t order_bits(float f)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);   // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unorder_bits(uint32_t o)
{
    return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// The argmax epilogue of one wave (row tile q): lane (r, g) holds logits
// lv[i] of row v = q*16 + r for activation rows m = 4g + i (valid when ok[i]).
__device__ __forceinline__ void head_argmax_epilogue(const HeadArgmax& am, const float (&lv)[4], const bool (&ok)[4],
                                                     int64_t q, int64_t v, int M, int lane)
{
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint64_t key = ok[i] ? ((uint64_t)order_bits(lv[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)v) : 0;
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {   // the 16 lanes of group g
            const uint32_t lo = __shfl_xor((uint32_t)key, off), hi = __shfl_xor((uint32_t)(key >> 32), off);
            const uint64_t other = ((uint64_t)hi << 32) | lo;
            key = other > key ? other : key;
        }
        const int m = 4 * g + i;
        if (r == 0 && m < M) am.part[q * M + m] = key;
    }
}

// Rows of a block-scaled int8 table (FV5B-style: W int8 [V][K], S f32
// [V][K/256]) for token ids: out[m][k] = W[id][k] * S[id][k/256] (one fp32
// rounding) and out_bf16 its nearest-even bf16; an id outside [0, V) gives a
// zero row without reading W.  Either output may be null.
struct EmbedRows {
    const int8_t* W;
    const float* S;
    int64_t V, K;
    float* out;
    uint16_t* out_bf16;
};

// 16 weights (chunk c) of output row m for token id
__device__ __forceinline__ void embed_chunk(const EmbedRows& e, int64_t id, int64_t m, int64_t c)
{
    float f[16];
    if (id >= 0 && id < e.V) {
        const u32x4 w = *(const u32x4*)(e.W + id * e.K + 16 * c);
        const float sc = e.S[id * (e.K / 256) + (16 * c) / 256];
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = (float)(int8_t)(w[i >> 2] >> (8 * (i & 3))) * sc;
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = 0.f;
    }
    if (e.out) {
        f32x4* o = (f32x4*)(e.out + m * e.K + 16 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f32x4{f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]};
    }
    if (e.out_bf16) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // nearest-even bf16 of a finite fp32 value: add 0x7FFF plus the
            // lowest kept bit, keep the high half
            uint32_t b0 = __builtin_bit_cast(uint32_t, f[2 * i]);
            uint32_t b1 = __builtin_bit_cast(uint32_t, f[2 * i + 1]);
            b0 = (b0 + 0x7FFFu + ((b0 >> 16) & 1u)) >> 16;
            b1 = (b1 + 0x7FFFu + ((b1 >> 16) & 1u)) >> 16;
            h[i] = b0 | (b1 << 16);
        }
        u32x4* o = (u32x4*)(e.out_bf16 + m * e.K + 16 * c);
        o[0] = u32x4{h[0], h[1], h[2], h[3]};
        o[1] = u32x4{h[4], h[5], h[6], h[7]};
    }
}

// Maximum over the row tiles' keys of activation row m = blockIdx.x; with
// emb.W set, the workgroup then writes the embedding row of the chosen index
// (the next token's input) into row m of emb's outputs.
__global__ __launch_bounds__(1024) void head_argmax_finish_kernel(const unsigned long long* __restrict__ part,
                                                                  int64_t nrt, int M, int32_t* __restrict__ idx,
                                                                  float* __restrict__ val, EmbedRows emb)
{
    __shared__ int64_t chosen;
    __shared__ unsigned long long best_of_wave[16];
    const int m = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long best = 0;
    for (int64_t q = threadIdx.x; q < nrt; q += blockDim.x) {
        const unsigned long long k = part[q * M + m];
        best = k > best ? k : best;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, off), hi = __shfl_xor((uint32_t)(best >> 32), off);
        const unsigned long long other = ((unsigned long long)hi << 32) | lo;
        best = other > best ? other : best;
    }
    if (lane == 0) best_of_wave[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) best = best_of_wave[w] > best ? best_of_wave[w] : best;
        const uint32_t v = 0xFFFFFFFFu - (uint32_t)best;
        idx[m] = (int32_t)v;
        val[m] = unorder_bits((uint32_t)(best >> 32));
        chosen = v;
    }
    if (emb.W == nullptr) return;   // uniform across the workgroup
    __syncthreads();
    for (int64_t c = threadIdx.x; c < emb.K / 16; c += blockDim.x) embed_chunk(emb, chosen, m, c);
}

// Head kernel when all of x fits in LDS: one 16-row tile per wave over the
// whole K, a ring of TPW 128-k units per wave.  Every ring slot is refilled
// with the same two loads whether or not a unit is left (past the end they
// read 16 bytes at the start of W, unused), so the compiler can count the
// loads in flight exactly instead of waiting for all of them.
//
// kBlk: block-scaled weights (FV5B-style: one f32 scale per 256-weight block
// of a row, rs = S [V][K/256]).  Each block's MFMA sum (exact int32 with int8
// activations, fp32 with bf16) is folded into the row total with its scale
// (one FMA per element and block, in block order); the int8 block sums go
// to acc_dbg [M][V][K/256] on request; logits = total (bf16) or
// s_x[m] * total (int8).  Every slot also loads its block's scale (4 bytes
// per lane, shared by the 4 lanes of a row and the block's two units).
//
// kPacked: W is the head_pack layout (below): the workgroup's 64 rows are one
// block of memory in which 128-k unit j of all four waves is 8 KiB, read with
// non-temporal loads, so the workgroup streams one sequential region.
template <bool kInt8, int TPW, bool kBlk = false, bool kPacked = false>
__global__ __launch_bounds__(256) void head_fast_kernel(const int8_t* __restrict__ W, const float* __restrict__ rs,
                                                        int64_t V, int64_t K, const void* __restrict__ act,
                                                        const float* __restrict__ s_x, int M, float* __restrict__ y,
                                                        int32_t* __restrict__ acc_dbg, HeadArgmax am)
{
    static_assert(!kBlk || TPW % 2 == 0, "a block's two units share a ring parity");
    extern __shared__ __align__(16) uint8_t smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int ebytes = kInt8 ? 1 : 2;
    const int astride = (int)K * ebytes + 16;              // bytes per staged activation row
    const int mrow = r < M ? r : M - 1;
    const int nunit = (int)(K / kBlockK);                  // 128-k units per row
    const int64_t nrt = (V + 15) >> 4;
    const int64_t q = (int64_t)blockIdx.x * kHeadWaves + wave;
    const bool has = q < nrt;
    int64_t v = q * kTileRows + r;
    v = v < V ? v : V - 1;                                 // rows past V re-read the last row (outputs dropped)
    const int8_t* row = W + (has ? v : 0) * K + 16 * g;

    const int nblk = (int)(K >> 8);                        // 256-weight blocks per row (kBlk)
    u32x4 lo[TPW], hi[TPW];
    float bs[TPW];
    const int8_t* grp = W + (int64_t)blockIdx.x * (kHeadWaves * kTileRows) * K + wave * kHeadUnitBytes + 16 * lane;
    auto load = [&](int s, int j) {
        const bool valid = has && j < nunit;
        if constexpr (kPacked) {
            const int8_t* p = valid ? grp + (int64_t)j * (kHeadWaves * kHeadUnitBytes) : W;
            lo[s] = __builtin_nontemporal_load((const u32x4*)p);
            hi[s] = __builtin_nontemporal_load((const u32x4*)(valid ? p + kHeadUnitBytes / 2 : W));
        } else {
            const int8_t* p = valid ? row + (int64_t)j * kBlockK : W;
            lo[s] = head_ld16(p);
            hi[s] = head_ld16(valid ? p + 64 : W);
        }
        if constexpr (kBlk) bs[s] = rs[valid ? v * nblk + (j >> 1) : 0];
    };
#pragma unroll
    for (int s = 0; s < TPW; ++s) load(s, s);

    {
        const int per_row = (int)(K * ebytes / 16);
        const uint8_t* src = (const uint8_t*)act;
        for (int i = threadIdx.x; i < M * per_row; i += blockDim.x) {
            const int m = i / per_row, c16 = i - m * per_row;
            *(u32x4*)(smem + m * astride + 16 * c16) = *(const u32x4*)(src + (int64_t)m * K * ebytes + 16 * c16);
        }
    }
    __syncthreads();
    if (!has) return;

    f32x4 accf = {0.f, 0.f, 0.f, 0.f};
    i32x4 acci = {0, 0, 0, 0};
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};                      // kBlk: scaled block sums so far
    const int64_t vo = q * kTileRows + r;
    const uint8_t* arow = smem + mrow * astride + 16 * g * ebytes;
    for (int u0 = 0; u0 < nunit; u0 += TPW) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int j = u0 + s;
            if (j < nunit) {
                const uint8_t* a = arow + j * kBlockK * ebytes;
                if constexpr (kInt8) {
                    acci = mfma_i8(*(const u32x4*)(a), lo[s], acci);
                    acci = mfma_i8(*(const u32x4*)(a + 64), hi[s], acci);
                } else {
                    u32x4 B[4];
                    head_decode_bf16(lo[s], hi[s], B);
#pragma unroll
                    for (int t = 0; t < 4; ++t) accf = mfma_bf16(*(const u32x4*)(a + kHalfOff[t]), B[t], accf);
                }
                if constexpr (kBlk) {
                    if (s & 1) {                           // the second unit of block j / 2
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (kInt8) {
                                tot[i] = __builtin_fmaf(bs[s], (float)acci[i], tot[i]);
                                const int m = 4 * g + i;
                                if (acc_dbg && vo < V && m < M)
                                    acc_dbg[((int64_t)m * V + vo) * nblk + (j >> 1)] = acci[i];
                            } else {
                                tot[i] = __builtin_fmaf(bs[s], accf[i], tot[i]);
                            }
                        }
                        accf = f32x4{0.f, 0.f, 0.f, 0.f};
                        acci = i32x4{0, 0, 0, 0};
                    }
                }
            }
            load(s, j + TPW);
        }
    }
    float lv[4];
    bool ok[4];
    {
        const float sv = kBlk ? 1.0f : rs[vo < V ? vo : V - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            ok[i] = vo < V && m < M;
            if constexpr (kBlk) {
                if constexpr (kInt8) lv[i] = s_x[m < M ? m : M - 1] * tot[i];
                else lv[i] = tot[i];
            } else {
                if constexpr (kInt8) lv[i] = sv * s_x[m < M ? m : M - 1] * (float)acci[i];
                else lv[i] = sv * accf[i];
            }
            if (ok[i]) {
                if (y) y[(int64_t)m * V + vo] = lv[i];
                if constexpr (kInt8 && !kBlk) {
                    if (acc_dbg) acc_dbg[(int64_t)m * V + vo] = acci[i];
                }
            }
        }
    }
    if (am.part) head_argmax_epilogue(am, lv, ok, q, vo, M, lane);
}

static int head_chunk(int64_t K, int64_t M, int ebytes)
{
    int64_t cap = (48 * 1024) / (M * ebytes) / kBlockK * kBlockK;
    if (cap < kBlockK) cap = kBlockK;
    return (int)(K < cap ? K : cap);
}

template <bool kInt8, int TPW, bool kBlk = false, bool kPacked = false>
static hipError_t launch_head_fast(const int8_t* W, const float* rs, int64_t V, int64_t K, const void* act,
                                   const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream,
                                   HeadArgmax am = HeadArgmax{nullptr})
{
    const size_t lds = (size_t)M * (K * (kInt8 ? 1 : 2) + 16);
    const int64_t grid = ((V + 15) / 16 + kHeadWaves - 1) / kHeadWaves;
    head_fast_kernel<kInt8, TPW, kBlk, kPacked><<<dim3((unsigned)grid), dim3(64 * kHeadWaves), lds, stream>>>(
        W, rs, V, K, act, s_x, (int)M, y, acc, am);
    return hipGetLastError();
}

// ---- packed head layout ----------------------------------------------------
// Rows in groups of 64 (a workgroup's four 16-row tiles; V padded to a
// multiple of 64 with zero rows); inside a group, for 128-k unit j, for wave
// w (rows 16w .. 16w + 15 of the group), 2 KiB: the low half holds, for lane
// l = r + 16g, bytes 16g .. 16g + 15 of the unit's row 16w + r, the high half
// bytes 64 + 16g .. 64 + 16g + 15.  A lane thus loads the same 32 bytes as
// from the row-major matrix, and a workgroup reads 8 KiB contiguously per
// unit (size: head_packed_bytes).

__global__ __launch_bounds__(256) void head_pack_kernel(const int8_t* __restrict__ W, int64_t V, int64_t K,
                                                        int8_t* __restrict__ out)
{
    const int64_t n16 = head_packed_bytes(V, K) / 16;
    const int64_t per_group = 64 * K / 16;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n16; c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t grp = c / per_group;
        int64_t rem = c - grp * per_group;
        const int64_t j = rem / (kHeadWaves * kHeadUnitBytes / 16);
        rem -= j * (kHeadWaves * kHeadUnitBytes / 16);
        const int w = (int)(rem / (kHeadUnitBytes / 16));
        rem -= (int64_t)w * (kHeadUnitBytes / 16);
        const int h = (int)(rem / 64), l = (int)(rem % 64);
        const int64_t row = grp * 64 + w * kTileRows + (l & 15);
        const int64_t col = j * kBlockK + 64 * h + 16 * (l >> 4);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < V) v = *(const u32x4*)(W + row * K + col);
        *(u32x4*)(out + c * 16) = v;
    }
}

hipError_t launch_head_pack(const int8_t* W, int64_t V, int64_t K, int8_t* out, hipStream_t stream)
{
    const int64_t n16 = head_packed_bytes(V, K) / 16;
    const int64_t blocks = (n16 + 255) / 256;
    head_pack_kernel<<<dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream>>>(W, V, K, out);
    return hipGetLastError();
}

// packed head: the single-pass kernel only (x of all M rows in LDS)
bool head_packed_fits(int64_t K, int64_t M, bool int8_act) { return head_argmax_fits(K, M, int8_act); }

hipError_t launch_head_packed_bf16(const int8_t* Wp, const float* rs, int64_t V, int64_t K, const uint16_t* x,
                                   int64_t M, float* y, hipStream_t stream)
{
    return launch_head_fast<false, kHeadPackedTpw, false, true>(Wp, rs, V, K, x, nullptr, M, y, nullptr, stream);
}

hipError_t launch_head_packed_i8(const int8_t* Wp, const float* rs, int64_t V, int64_t K, const int8_t* q,
                                 const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    return launch_head_fast<true, kHeadPackedTpw, false, true>(Wp, rs, V, K, q, s_x, M, y, acc, stream);
}

template <bool kInt8>
static hipError_t launch_head(const int8_t* W, const float* rs, int64_t V, int64_t K, const void* act,
                              const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    const int kc = head_chunk(K, M, kInt8 ? 1 : 2);
    if (kc == K) return launch_head_fast<kInt8, kHeadTpw>(W, rs, V, K, act, s_x, M, y, acc, stream);
    constexpr int kTpw = 1;   // deeper rings cost more VGPRs than they win here
    const size_t lds = (size_t)M * (kc * (kInt8 ? 1 : 2) + 16);
    // one row tile per wave: a row tile is 16 x K bytes (64 KB at K = 4096), so
    // a static multi-tile assignment leaves a serial tail; retiring workgroups
    // balance the load instead
    const int64_t grid = ((V + 15) / 16 + kHeadWaves - 1) / kHeadWaves;
    head_kernel<kInt8, kTpw><<<dim3((unsigned)grid), dim3(64 * kHeadWaves), lds, stream>>>(W, rs, V, K, act, s_x,
                                                                                             (int)M, y, acc, kc);
    return hipGetLastError();
}

hipError_t launch_head_bf16(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                            float* y, hipStream_t stream)
{
    return launch_head<false>(W, rs, V, K, x, nullptr, M, y, nullptr, stream);
}

hipError_t launch_head_i8(const int8_t* W, const float* rs, int64_t V, int64_t K, const int8_t* q,
                          const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    return launch_head<true>(W, rs, V, K, q, s_x, M, y, acc, stream);
}

// fused head + argmax: x (all M rows) must fit in LDS, as the single-pass
// kernel stages it whole; the workspace holds one key per (row tile, m)
bool head_argmax_fits(int64_t K, int64_t M, bool int8_act)
{
    return (size_t)M * (K * (int8_act ? 1 : 2) + 16) <= (size_t)160 * 1024;
}

template <bool kInt8, bool kBlk = false, bool kPacked = false>
static hipError_t launch_head_argmax(const int8_t* W, const float* rs, int64_t V, int64_t K, const void* act,
                                     const float* s_x, int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                     hipStream_t stream, EmbedRows emb = EmbedRows{nullptr, nullptr, 0, 0, nullptr,
                                                                                  nullptr})
{
    const HeadArgmax am{(unsigned long long*)ws};
    hipError_t e = launch_head_fast<kInt8, kPacked ? kHeadPackedTpw : kHeadTpw, kBlk, kPacked>(W, rs, V, K, act, s_x,
                                                                                              M, y, nullptr, stream,
                                                                                              am);
    if (e != hipSuccess) return e;
    head_argmax_finish_kernel<<<dim3((unsigned)M), dim3(1024), 0, stream>>>((const unsigned long long*)ws,
                                                                           (V + 15) / 16, (int)M, idx, val, emb);
    return hipGetLastError();
}

hipError_t launch_head_argmax_bf16(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x,
                                   int64_t M, float* y, int32_t* idx, float* val, void* ws, hipStream_t stream)
{
    return launch_head_argmax<false>(W, rs, V, K, x, nullptr, M, y, idx, val, ws, stream);
}

hipError_t launch_head_argmax_i8(const int8_t* W, const float* rs, int64_t V, int64_t K, const int8_t* q,
                                 const float* s_x, int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                 hipStream_t stream)
{
    return launch_head_argmax<true>(W, rs, V, K, q, s_x, M, y, idx, val, ws, stream);
}

// the same over the packed copy (padding rows past V carry no key: their logits are never candidates)
hipError_t launch_head_argmax_packed_bf16(const int8_t* Wp, const float* rs, int64_t V, int64_t K,
                                          const uint16_t* x, int64_t M, float* y, int32_t* idx, float* val,
                                          void* ws, hipStream_t stream)
{
    return launch_head_argmax<false, false, true>(Wp, rs, V, K, x, nullptr, M, y, idx, val, ws, stream);
}

hipError_t launch_head_argmax_packed_i8(const int8_t* Wp, const float* rs, int64_t V, int64_t K, const int8_t* q,
                                        const float* s_x, int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                        hipStream_t stream)
{
    return launch_head_argmax<true, false, true>(Wp, rs, V, K, q, s_x, M, y, idx, val, ws, stream);
}

// ---- the argmax keys in a library-owned array (for callers that cannot
// allocate): every call on a device shares this array, which keeps the last
// call's keys.  Every slot the finish kernel reads is written by the head
// kernel of the same call first, so nothing needs clearing; calls that
// overlap in time on one device race on it.
static __device__ __align__(256) unsigned long long scratch[kHeadArgmaxScratchBytes / 8];

// Device address of `scratch` on the current device, looked up once per
// device (each device holds its own copy of the array at its own address).
// Host code uses only this address: the array's name on the host is a
// stand-in, not a device pointer.
static hipError_t head_argmax_scratch(void** out)
{
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void* addr[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_head_argmax_bf16_noalloc(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x,
                                           int64_t M, float* y, int32_t* idx, float* val, hipStream_t stream)
{
    if ((V + 15) / 16 * M * 8 > kHeadArgmaxScratchBytes) return hipErrorInvalidValue;   // the caller checked this
    void* ws = nullptr;
    const hipError_t e = head_argmax_scratch(&ws);
    if (e != hipSuccess) return e;
    return launch_head_argmax<false>(W, rs, V, K, x, nullptr, M, y, idx, val, ws, stream);
}

// ---- block-scaled (FV5B-style) head: x must fit in LDS (head_argmax_fits)

hipError_t launch_fv5b_head_bf16(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                 int64_t M, float* y, hipStream_t stream)
{
    return launch_head_fast<false, kHeadTpw, true>(W, S, V, K, x, nullptr, M, y, nullptr, stream);
}

hipError_t launch_fv5b_head_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q,
                               const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    return launch_head_fast<true, kHeadTpw, true>(W, S, V, K, q, s_x, M, y, acc, stream);
}

hipError_t launch_fv5b_head_argmax_bf16(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                        int64_t M, float* y, int32_t* idx, float* val, void* ws, hipStream_t stream)
{
    return launch_head_argmax<false, true>(W, S, V, K, x, nullptr, M, y, idx, val, ws, stream);
}

hipError_t launch_fv5b_head_argmax_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q,
                                      const float* s_x, int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                      hipStream_t stream)
{
    return launch_head_argmax<true, true>(W, S, V, K, q, s_x, M, y, idx, val, ws, stream);
}

// the block-scaled head over the packed copy of its int8 rows (the scales stay [V][K/256])
hipError_t launch_fv5b_head_packed_bf16(const int8_t* Wp, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                        int64_t M, float* y, hipStream_t stream)
{
    return launch_head_fast<false, kHeadPackedTpw, true, true>(Wp, S, V, K, x, nullptr, M, y, nullptr, stream);
}

hipError_t launch_fv5b_head_packed_i8(const int8_t* Wp, const float* S, int64_t V, int64_t K, const int8_t* q,
                                      const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream)
{
    return launch_head_fast<true, kHeadPackedTpw, true, true>(Wp, S, V, K, q, s_x, M, y, acc, stream);
}

hipError_t launch_fv5b_head_argmax_packed_bf16(const int8_t* Wp, const float* S, int64_t V, int64_t K,
                                               const uint16_t* x, int64_t M, float* y, int32_t* idx, float* val,
                                               void* ws, hipStream_t stream)
{
    return launch_head_argmax<false, true, true>(Wp, S, V, K, x, nullptr, M, y, idx, val, ws, stream);
}

hipError_t launch_fv5b_head_argmax_packed_i8(const int8_t* Wp, const float* S, int64_t V, int64_t K,
                                             const int8_t* q, const float* s_x, int64_t M, float* y, int32_t* idx,
                                             float* val, void* ws, hipStream_t stream)
{
    return launch_head_argmax<true, true, true>(Wp, S, V, K, q, s_x, M, y, idx, val, ws, stream);
}

// Embedding rows: one thread per 16 weights of an output row (embed_chunk).
__global__ void fv5b_embed_kernel(EmbedRows e, const int32_t* __restrict__ ids, int64_t M)
{
    const int64_t per_row = e.K / 16, total = M * per_row;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = t / per_row, c = t - m * per_row;
        embed_chunk(e, ids[m], m, c);
    }
}

hipError_t launch_fv5b_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const int32_t* ids, int64_t M,
                             float* out, uint16_t* out_bf16, hipStream_t stream)
{
    const int64_t items = M * (K / 16);
    int64_t grid = (items + 255) / 256;
    grid = grid < 1 ? 1 : (grid > 65536 ? 65536 : grid);
    fv5b_embed_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(EmbedRows{W, S, V, K, out, out_bf16}, ids, M);
    return hipGetLastError();
}

hipError_t launch_fv5b_head_argmax_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                         int64_t M, float* y, int32_t* idx, float* val, void* ws, const int8_t* E,
                                         const float* ES, int64_t Ve, int64_t Ke, float* emb, uint16_t* emb_bf16,
                                         hipStream_t stream)
{
    return launch_head_argmax<false, true>(W, S, V, K, x, nullptr, M, y, idx, val, ws, stream,
                                           EmbedRows{E, ES, Ve, Ke, emb, emb_bf16});
}

}  // namespace tern
