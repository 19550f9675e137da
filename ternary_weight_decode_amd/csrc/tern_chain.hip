// tern_chain.hip — a chain of ternary GEMVs (M = 1) in one persistent launch,
// the steps linked by their activations.
//
//   step p:  y_p[n] = sum_b scale_p[n][b] * sum_{k in b} t_p[n][k] * x_p[k]
//            x_p = an input vector, or bf16(y_q[0:K_p]) of an earlier step q
//
// This is single-stream decode with its dependent launches folded into one:
// on this chip a kernel boundary costs a few microseconds of launch, ramp and
// drain, and a token has one boundary per dependent linear.
//
// Work split.  One workgroup per CU stays resident for the whole chain (the
// launch is cooperative).  Workgroup b owns row tiles b, b+G, b+2G, ... of
// every step; its 15 compute waves split the step's (row tile, k-tile) units
// round-robin.  Each compute wave keeps a ring of plane tiles in registers
// whose loads run ahead of its compute, across step boundaries, so the next
// steps' weights stream in while the workgroup waits for its activations.
// Each unit's fp32 partial (16 rows) goes to LDS; a control wave sums them
// per output in fixed k-tile order (deterministic) and stores y.  All threads
// fetch the next activations.
//
// Hand-off.  A step whose output feeds a later step also writes it as 64-bit
// words {bf16 y[2i], bf16 y[2i+1], 32-bit tag} with device-coherent atomic
// stores, where the tag names the launch (an epoch counter in the workspace,
// bumped by the last workgroup to finish) and the step.  A consumer loads
// the words it needs (device-coherent) until every tag matches, so it waits
// for exactly the data it reads: no grid-wide barrier, no store
// acknowledgement on the producer's path.  Steps with an input vector do not
// wait for anything.  Every spin is bounded: a wait past the bound counts an
// error in the workspace and the workgroup leaves at the next step boundary;
// a workspace with a nonzero error count runs nothing until it is cleared.
#include "tern_device.h"
#include "tern_launch.h"
#include "tern_tile.h"

namespace tern {

constexpr int kChainIo = 1;                     // control wave: partial sums and outputs
constexpr int kChainCompute = kChainWaves - kChainIo;
constexpr int kChainTpw = 3;                    // plane tiles in flight per compute wave
constexpr unsigned kChainMaxPolls = 1u << 21;   // bound on every spin (seconds of polling)
constexpr int kBufferRsrcWord3 = 0x00020000;    // raw buffer resource, 32-bit data format
constexpr int kCachePolicySc1 = 16;             // sc1: device-coherent access
constexpr int kThreads = 64 * kChainWaves;
constexpr int kWordsPerThread = kChainMaxK / 2 / kThreads;      // hand-off words a thread polls at most
constexpr int kLoadsPerThread = kChainMaxK * 2 / 16 / kThreads;   // 16-byte input loads per thread
static_assert(kWordsPerThread == 8, "hand-off polling covers kChainMaxK with 8 words per thread");
static_assert(kLoadsPerThread == 2, "input staging covers kChainMaxK with 2 loads per thread");

struct ChainStepBatch {
    ChainStep s[kChainPlanBatch];
};

// Writes plan entries [first, first + count) and, with the last batch, the
// header's magic and step count.
__global__ void chain_plan_kernel(ChainStepBatch batch, int first, int count, int total, uint8_t* ws)
{
    ChainStep* plan = (ChainStep*)(ws + kChainPlanOffset);
    const int i = threadIdx.x;
    if (i < count) plan[first + i] = batch.s[i];
    if (i == 0 && first + count == total) {
        ChainHeader* h = (ChainHeader*)ws;
        h->magic = kChainMagic;
        h->nsteps = (uint32_t)total;
    }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;   // NaN stays NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Geometry of one step as seen by workgroup b.
struct StepGeo {
    const TERN_GLOBAL uint32_t* words;
    const TERN_GLOBAL uint16_t* scales;
    int nb, nkt, nmy;   // 128-blocks per row, k-tiles per row, row tiles of this workgroup
    int qd, qr;         // kChainCompute / nkt and kChainCompute % nkt (cursor stride)
};

// Plan entries are read with a wave-uniform index (scalar loads).
__device__ __forceinline__ ChainStep plan_entry(const ChainStep* __restrict__ plan, int p)
{
    return plan[__builtin_amdgcn_readfirstlane(p)];
}

__device__ __forceinline__ StepGeo step_geo(const ChainStep& st, int b, int G)
{
    StepGeo s;
    s.words = (const TERN_GLOBAL uint32_t*)st.packed;
    s.scales = (const TERN_GLOBAL uint16_t*)(st.packed + scale_region_offset(st.N, st.K));
    s.nb = (int)(st.K / kBlockK);
    s.nkt = (s.nb + 3) >> 2;
    const int nrt = (int)((st.N + 15) >> 4);
    s.nmy = b < nrt ? (nrt - 1 - b) / G + 1 : 0;
    s.qd = kChainCompute / s.nkt;
    s.qr = kChainCompute - s.qd * s.nkt;
    return s;
}

// Position of a wave in the unit sequence of the chain: step p, local row tile
// i (row tile b + i*G) and k-tile k.  Units of a step go round-robin over the
// compute waves in (row tile, k-tile) order.
struct Cursor {
    int p, i, k;
    StepGeo geo;
};

__device__ __forceinline__ void cursor_skip_empty(Cursor& c, const ChainStep* plan, int nsteps, int b, int G,
                                                  int cw)
{
    while (c.p < nsteps && c.i >= c.geo.nmy) {
        if (++c.p < nsteps) {
            c.geo = step_geo(plan_entry(plan, c.p), b, G);
            c.i = cw / c.geo.nkt;
            c.k = cw - c.i * c.geo.nkt;
        }
    }
}

__device__ __forceinline__ void cursor_next(Cursor& c, const ChainStep* plan, int nsteps, int b, int G, int cw)
{
    c.k += c.geo.qr;
    c.i += c.geo.qd;
    if (c.k >= c.geo.nkt) {
        c.k -= c.geo.nkt;
        ++c.i;
    }
    cursor_skip_empty(c, plan, nsteps, b, G, cw);
}

__global__ __launch_bounds__(kThreads) void chain_kernel(const ChainStep* __restrict__ plan,
                                                         ChainHeader* __restrict__ hdr, uint8_t* __restrict__ ws,
                                                         int nsteps_arg)
{
    extern __shared__ __align__(16) uint8_t smem[];
    uint16_t* xs = (uint16_t*)smem;                                    // [kChainMaxK] activations
    float* red = (float*)(smem + kChainMaxK * 2);                      // [kChainRedMax] unit partials
    int* flags = (int*)(smem + kChainMaxK * 2 + kChainRedMax * 4);     // abort, nsteps, epoch

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int b = blockIdx.x, G = gridDim.x;

    // one thread reads the header for the workgroup: a workspace that was never
    // planned, or that holds an aborted run, runs nothing
    if (threadIdx.x == 0) {
        const bool ok = hdr->magic == kChainMagic && hdr->errors == 0;
        flags[0] = 0;
        flags[1] = ok ? (nsteps_arg < (int)hdr->nsteps ? nsteps_arg : (int)hdr->nsteps) : 0;
        flags[2] = (int)hdr->epoch;
    }
    __syncthreads();
    const int nsteps = __builtin_amdgcn_readfirstlane(flags[1]);
    if (nsteps <= 0) return;
    const uint32_t epoch = (uint32_t)__builtin_amdgcn_readfirstlane(flags[2]);
    auto tag_of = [&](int p) -> uint32_t { return epoch * (uint32_t)kChainMaxSteps + (uint32_t)(p + 1); };

    // Activations of step p into LDS, by all threads (t = threadIdx.x).
    // An input vector: 16-byte buffer loads (loads past K return zeros, and
    // the LDS array holds kChainMaxK elements, so nothing needs a guard).  A
    // hand-off: each thread polls its words until their tags name (this
    // launch, step q).
    auto acquire_x = [&](int p, int t) {
        const ChainStep st = plan_entry(plan, p);
        if (st.x_from < 0) {
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)st.x, (short)0, (int)(st.K * 2), kBufferRsrcWord3);
            u32x4 v[kLoadsPerThread];
#pragma unroll
            for (int j = 0; j < kLoadsPerThread; ++j)
                v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (t + j * kThreads) * 16, 0, 0);
#pragma unroll
            for (int j = 0; j < kLoadsPerThread; ++j) ((u32x4*)xs)[t + j * kThreads] = v[j];
            return;
        }
        // 8-byte device-coherent buffer loads (one access each, so a word's tag
        // and values come from the same store); loads past K/2 words return 0
        const int nw = (int)(st.K >> 1);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(ws + st.x_hand_off), (short)0, nw * 8, kBufferRsrcWord3);
        const uint32_t want = tag_of((int)st.x_from);
        unsigned pend = 0;
#pragma unroll
        for (int j = 0; j < kWordsPerThread; ++j)
            if (t + j * kThreads < nw) pend |= 1u << j;
        unsigned polls = 0;
        while (pend) {
            // issue every pending word's load, then check them
            u32x2 v[kWordsPerThread];
#pragma unroll
            for (int j = 0; j < kWordsPerThread; ++j) {
                v[j] = u32x2{0, 0};
                if (pend & (1u << j))
                    v[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, (t + j * kThreads) * 8, 0, kCachePolicySc1);
            }
#pragma unroll
            for (int j = 0; j < kWordsPerThread; ++j) {
                if ((pend & (1u << j)) && v[j][1] == want) {
                    ((uint32_t*)xs)[t + j * kThreads] = v[j][0];
                    pend &= ~(1u << j);
                }
            }
            if (pend && ++polls > kChainMaxPolls) {
                __hip_atomic_fetch_add(&hdr->errors, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                flags[0] = 1;
                break;
            }
        }
    };

    const int t = (int)threadIdx.x;
    if (wave < kChainIo) {
        // ------------------------------------------------------ control wave
        acquire_x(0, t);
        __syncthreads();                                               // B_0: x_0 in LDS
        if (flags[0]) return;
        for (int p = 0; p < nsteps; ++p) {
            __syncthreads();                                           // A_p: partials of step p in LDS
            const ChainStep st = plan_entry(plan, p);
            const StepGeo geo = step_geo(st, b, G);
            TERN_GLOBAL float* y = (TERN_GLOBAL float*)st.y;
            TERN_GLOBAL unsigned long long* ho = (TERN_GLOBAL unsigned long long*)(ws + st.hand_off);
            const unsigned long long tag = (unsigned long long)tag_of(p) << 32;
            // outputs in pairs (n, n+1) of row tile i: sum the k-tile partials in order
            for (int o = t; o < geo.nmy * 8; o += 64 * kChainIo) {
                const int i = o >> 3, n = 2 * (o & 7);
                const float2* rp = (const float2*)(red + (i * geo.nkt) * 16 + n);
                float s0 = 0.f, s1 = 0.f;
                for (int k = 0; k < geo.nkt; ++k) {
                    const float2 v = rp[k * 8];
                    s0 += v.x;
                    s1 += v.y;
                }
                const int64_t row = ((int64_t)(b + i * G) << 4) + n;
                if (row < st.N) y[row] = s0;
                if (row + 1 < st.N) y[row + 1] = s1;
                if (st.feeds && row < st.N) {
                    const unsigned long long lo = f32_to_bf16_rne(s0);
                    const unsigned long long hi = row + 1 < st.N ? f32_to_bf16_rne(s1) : 0u;
                    __hip_atomic_store(&ho[row >> 1], tag | (hi << 16) | lo, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if (p + 1 == nsteps) break;
            acquire_x(p + 1, t);
            __syncthreads();                                           // B_{p+1}
            if (flags[0]) return;
        }
        // the last workgroup to finish moves the workspace to the next epoch
        if (t == 0) {
            const unsigned long long d = __hip_atomic_fetch_add(&hdr->done, 1ull, __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_AGENT);
            if (d % (unsigned long long)G == (unsigned long long)(G - 1))
                __hip_atomic_fetch_add(&hdr->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    // ---------------------------------------------------------- compute waves
    const int cw = wave - kChainIo;
    Cursor ld, cu;
    ld.p = 0;
    ld.geo = step_geo(plan_entry(plan, 0), b, G);
    ld.i = cw / ld.geo.nkt;
    ld.k = cw - ld.i * ld.geo.nkt;
    cursor_skip_empty(ld, plan, nsteps, b, G, cw);
    cu = ld;

    // unused ring slots (past the chain's end) read the first 16 bytes of step 0's planes
    const ChainStep st0 = plan_entry(plan, 0);
    const TERN_GLOBAL uint32_t* dummy_w = (const TERN_GLOBAL uint32_t*)st0.packed;
    const TERN_GLOBAL uint16_t* dummy_s = (const TERN_GLOBAL uint16_t*)st0.packed;
    // every k-tile is full (K % 512 == 0), so each refill is the same three loads
    auto refill = [&](PlaneTile& t) {
        const bool valid = ld.p < nsteps;
        const TERN_GLOBAL uint32_t* wn = dummy_w;
        const TERN_GLOBAL uint32_t* wsg = dummy_w;
        const TERN_GLOBAL uint16_t* sp = dummy_s;
        if (valid) {
            const int64_t rt = (int64_t)b + (int64_t)ld.i * G;
            const int64_t wb = tile_word_base(rt, ld.k, ld.geo.nb);
            wn = ld.geo.words + wb + ((0 * 4 + g) * 16 + r) * 4;
            wsg = ld.geo.words + wb + ((1 * 4 + g) * 16 + r) * 4;
            sp = ld.geo.scales + tile_scale_base(rt, ld.k, ld.geo.nb) + r * 4;
            cursor_next(ld, plan, nsteps, b, G, cw);
        }
        t.nz = ld_nt16(wn);
        t.sg = ld_nt16(wsg);
        t.sc = ld_nt8(sp);
    };

    PlaneTile slot[kChainTpw];
#pragma unroll
    for (int s = 0; s < kChainTpw; ++s) refill(slot[s]);
    acquire_x(0, t);

    int passed = 0;                                                    // step whose activations are staged
    __syncthreads();                                                   // B_0
    if (flags[0]) return;
    // step boundary: A (partials stored), the next activations, B
    auto next_step = [&]() -> bool {
        __syncthreads();                                               // A_passed
        ++passed;
        acquire_x(passed, t);
        __syncthreads();                                               // B_passed
        return flags[0] == 0;
    };
    while (cu.p < nsteps) {
#pragma unroll
        for (int s = 0; s < kChainTpw; ++s) {
            if (cu.p < nsteps) {
                while (passed < cu.p)
                    if (!next_step()) return;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                bf16_tile<1>(slot[s], xs + cu.k * kTileK + 32 * g, 4, acc);
                if (lane < 16) red[(cu.i * cu.geo.nkt + cu.k) * 16 + lane] = acc[0];
                cursor_next(cu, plan, nsteps, b, G, cw);
            }
            refill(slot[s]);
        }
    }
    while (passed < nsteps - 1)
        if (!next_step()) return;
    __syncthreads();                                                   // A_last
}

__global__ void chain_clear_kernel(unsigned long long* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

hipError_t launch_chain_plan(const ChainStep* steps, int nsteps, uint8_t* ws, int64_t hand_off_begin,
                             int64_t hand_off_end, hipStream_t stream)
{
    // stale hand-off words from an earlier plan must never carry a live tag
    const int64_t nclear = (hand_off_end - hand_off_begin) / 8;
    if (nclear > 0) {
        const int64_t blocks = (nclear + 255) / 256 < 1024 ? (nclear + 255) / 256 : 1024;
        chain_clear_kernel<<<(unsigned)blocks, 256, 0, stream>>>((unsigned long long*)(ws + hand_off_begin),
                                                                 nclear);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    for (int first = 0; first < nsteps; first += kChainPlanBatch) {
        const int count = nsteps - first < kChainPlanBatch ? nsteps - first : kChainPlanBatch;
        ChainStepBatch batch;
        for (int i = 0; i < count; ++i) batch.s[i] = steps[first + i];
        for (int i = count; i < kChainPlanBatch; ++i) batch.s[i] = ChainStep{};
        chain_plan_kernel<<<1, kChainPlanBatch, 0, stream>>>(batch, first, count, nsteps, ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t chain_grid(int* grid)
{
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel, kThreads, kChainLds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
    *grid = cus;   // exactly one workgroup per CU (the LDS request admits no second one)
    return hipSuccess;
}

hipError_t launch_chain(uint8_t* ws, int nsteps, hipStream_t stream)
{
    int grid = 0;
    hipError_t e = chain_grid(&grid);
    if (e != hipSuccess) return e;
    const ChainStep* plan = (const ChainStep*)(ws + kChainPlanOffset);
    ChainHeader* hdr = (ChainHeader*)ws;
    void* args[] = {&plan, &hdr, &ws, &nsteps};
    return hipLaunchCooperativeKernel((const void*)chain_kernel, dim3((unsigned)grid), dim3(kThreads), args,
                                      kChainLds, stream);
}

}  // namespace tern
