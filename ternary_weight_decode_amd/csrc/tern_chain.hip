// tern_chain.hip — a chain of dependent ternary GEMVs (M = 1) in one
// persistent launch.
//
//   step p:  y_p[n] = sum_b scale_p[n][b] * sum_{k in b} t_p[n][k] * x_p[k]
//            y_bf16_p = y_p rounded to bf16 (nearest-even), when requested
//
// x_p may be the bf16 output of an earlier step of the same chain.  This is
// single-stream decode with its dependent launches folded into one: on this
// chip a kernel boundary costs a few microseconds of launch, ramp and drain,
// and a token has one boundary per dependent linear.
//
// Work split.  One workgroup per CU stays resident for the whole chain (the
// launch is cooperative).  Workgroup b owns row tiles b, b+G, b+2G, ... of
// every step; its 15 compute waves split the step's (row tile, k-tile) units
// round-robin.  Each compute wave keeps a ring of plane tiles in registers
// whose loads run ahead of its compute, across step boundaries, so the next
// step's weights stream in while the workgroups synchronise.  Each unit's
// fp32 partial (16 rows) goes to LDS.
//
// Step boundary.  A control wave per workgroup sums the unit partials of each
// output in fixed k-tile order (deterministic), stores y (and y_bf16) with
// device-coherent stores, waits for them to complete, joins a grid-wide
// barrier, then loads the next step's activations (device-coherent loads when
// they were written earlier in the chain) into LDS.  Compute waves only wait
// on workgroup barriers, so their weight loads stay in flight meanwhile.
//
// Grid barrier: monotonic 64-bit counters, never reset, so the workspace needs
// no clearing between launches: eight group counters (workgroup b joins group
// b % 8), a top counter bumped by the last arrival of each group, and a
// generation counter bumped by the last top arrival.  Arrival number a in a
// group of size s belongs to barrier a / s; a waiter leaves when the
// generation exceeds that.  All spins are bounded: a wait past the bound
// counts an error in the workspace, and every workgroup leaves at the next
// step boundary; a workspace with a nonzero error count runs nothing until it
// is cleared.
#include "tern_device.h"
#include "tern_launch.h"
#include "tern_tile.h"

namespace tern {

constexpr int kChainCompute = kChainWaves - 1;
constexpr int kChainTpw = 3;                    // plane tiles in flight per compute wave
constexpr unsigned kChainMaxPolls = 1u << 22;   // bound on every spin (seconds of polling)
constexpr int kBufferRsrcWord3 = 0x00020000;    // raw buffer resource, 32-bit data format
constexpr int kCachePolicySc1 = 16;             // sc1: device-coherent access

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
        uint32_t* hdr = (uint32_t*)(ws + kChainHeaderOffset);
        hdr[0] = kChainMagic;
        hdr[1] = (uint32_t)total;
    }
}

struct ChainCounters {
    unsigned long long grp[8][16];   // one 128-byte line per group
    unsigned long long top[16];
    unsigned long long gen[16];
};

__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Grid-wide barrier among G workgroups (lane 0 of the control wave of each).
// Returns false when a spin exceeded its bound.
__device__ bool chain_grid_barrier(ChainCounters* c, uint32_t* errors, unsigned G)
{
    const unsigned grp = blockIdx.x & 7u;
    const unsigned gsize = G / 8 + (grp < (G & 7u) ? 1u : 0u);
    const unsigned ngroups = G < 8 ? G : 8;
    const unsigned long long a = __hip_atomic_fetch_add(&c->grp[grp][0], 1ull, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long done = a / gsize;   // barriers completed before this one
    if (a % gsize == gsize - 1) {
        const unsigned long long t = __hip_atomic_fetch_add(&c->top[0], 1ull, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
        if (t % ngroups == ngroups - 1)
            __hip_atomic_fetch_add(&c->gen[0], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    unsigned polls = 0;
    while (__hip_atomic_load(&c->gen[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= done) {
        if (++polls > kChainMaxPolls) {
            __hip_atomic_fetch_add(errors, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
    return true;
}

// Geometry of one step as seen by workgroup b and compute wave cw.
struct StepGeo {
    const TERN_GLOBAL uint32_t* words;
    const TERN_GLOBAL uint16_t* scales;
    int nb, nkt, nmy;   // 128-blocks per row, k-tiles per row, row tiles of this workgroup
    int qd, qr;         // kChainCompute / nkt and kChainCompute % nkt (cursor stride)
};

// Plan entries are read with a wave-uniform index (scalar loads), and their
// device pointers are global-memory pointers.
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

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;   // NaN stays NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(64 * kChainWaves) void chain_kernel(const ChainStep* __restrict__ plan,
                                                                ChainCounters* __restrict__ ctr,
                                                                uint32_t* __restrict__ hdr, int nsteps_arg)
{
    extern __shared__ __align__(16) uint8_t smem[];
    uint16_t* xs = (uint16_t*)smem;                                    // [kChainMaxK] activations
    float* red = (float*)(smem + kChainMaxK * 2);                      // [kChainRedMax] unit partials
    int* abort_flag = (int*)(smem + kChainMaxK * 2 + kChainRedMax * 4);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int b = blockIdx.x, G = gridDim.x;

    // one thread reads the header for the workgroup: a workspace that was never
    // planned, or that holds an aborted run, runs nothing
    int* nsteps_lds = abort_flag + 1;
    if (threadIdx.x == 0) {
        const bool ok = hdr[0] == kChainMagic && hdr[2] == 0;
        *nsteps_lds = ok ? (nsteps_arg < (int)hdr[1] ? nsteps_arg : (int)hdr[1]) : 0;
        *abort_flag = 0;
    }
    __syncthreads();
    const int nsteps = __builtin_amdgcn_readfirstlane(*nsteps_lds);
    if (nsteps <= 0) return;

    // Activations of a step into LDS: all threads, two 16-byte loads each
    // (K <= 16384).  Buffer loads past K return zeros and the LDS array holds
    // kChainMaxK elements, so loads and stores need no guards (and the
    // compiler's wait counts stay exact).  Loads of an x written earlier in
    // this chain bypass the non-coherent caches (sc1), as the stores did.
    auto load_x = [&](const ChainStep& st, u32x4 (&v)[2]) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)st.x, (short)0, (int)(st.K * 2), kBufferRsrcWord3);
        const int i0 = (int)threadIdx.x * 16, i1 = i0 + 64 * kChainWaves * 16;
        if (st.x_coherent) {
            v[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, i0, 0, kCachePolicySc1);
            v[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, i1, 0, kCachePolicySc1);
        } else {
            v[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, i0, 0, 0);
            v[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, i1, 0, 0);
        }
    };
    auto store_x = [&](const u32x4 (&v)[2]) {
        ((u32x4*)xs)[threadIdx.x] = v[0];
        ((u32x4*)xs)[threadIdx.x + 64 * kChainWaves] = v[1];
    };
    static_assert(kChainMaxK == 2 * 64 * kChainWaves * 8, "x staging covers kChainMaxK with two loads per thread");

    if (wave == 0) {
        // ------------------------------------------------------ control wave
        {
            u32x4 v[2];
            const ChainStep st = plan_entry(plan, 0);
            load_x(st, v);
            store_x(v);
        }
        __syncthreads();                                               // B_0
        for (int p = 0; p < nsteps; ++p) {
            __syncthreads();                                           // A_p: partials of step p in LDS
            const ChainStep st = plan_entry(plan, p);
            const StepGeo geo = step_geo(st, b, G);
            // outputs in pairs (n, n+1) of row tile i: sum the k-tile partials in order
            TERN_GLOBAL float* y = (TERN_GLOBAL float*)st.y;
            TERN_GLOBAL uint16_t* yb = (TERN_GLOBAL uint16_t*)st.y_bf16;
            for (int o = lane; o < geo.nmy * 8; o += 64) {
                const int i = o >> 3, n = 2 * (o & 7);
                const float2* rp = (const float2*)(red + (i * geo.nkt) * 16 + n);
                float s0 = 0.f, s1 = 0.f;
                for (int k = 0; k < geo.nkt; ++k) {
                    const float2 v = rp[k * 8];
                    s0 += v.x;
                    s1 += v.y;
                }
                const int64_t row = ((int64_t)(b + i * G) << 4) + n;
                if (row < st.N) {
                    __hip_atomic_store(&y[row], s0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (st.y_bf16)
                        __hip_atomic_store(&yb[row], (uint16_t)f32_to_bf16_rne(s0), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                if (row + 1 < st.N) {
                    __hip_atomic_store(&y[row + 1], s1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (st.y_bf16)
                        __hip_atomic_store(&yb[row + 1], (uint16_t)f32_to_bf16_rne(s1), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if (p + 1 == nsteps) break;
            // this workgroup's outputs are complete at the device's coherence point
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(0);
            compiler_fence();
            bool ok = true;
            if (lane == 0) ok = chain_grid_barrier(ctr, hdr + 2, (unsigned)G);
            ok = __builtin_amdgcn_readfirstlane((int)ok) != 0;
            if (!ok && lane == 0) *abort_flag = 1;
            compiler_fence();
            __syncthreads();                                           // C_p: every step-p output stored
            if (*abort_flag) return;
            u32x4 v[2];
            const ChainStep nx = plan_entry(plan, p + 1);
            load_x(nx, v);
            store_x(v);
            __syncthreads();                                           // B_{p+1}
        }
        return;
    }

    // ---------------------------------------------------------- compute waves
    const int cw = wave - 1;
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
    {
        // x of step 0 is requested before the first weight tiles, so waiting
        // for it does not wait for them
        u32x4 v[2];
        load_x(st0, v);
#pragma unroll
        for (int s = 0; s < kChainTpw; ++s) refill(slot[s]);
        store_x(v);
    }

    int passed = 0;                                                    // step whose activations are staged
    __syncthreads();                                                   // B_0
    // step boundary: A (partials stored), C (outputs stored device-wide), B (next x staged)
    auto next_step = [&]() -> bool {
        __syncthreads();                                               // A_passed
        __syncthreads();                                               // C_passed
        if (*abort_flag) return false;
        ++passed;
        u32x4 v[2];
        const ChainStep nx = plan_entry(plan, passed);
        load_x(nx, v);
        store_x(v);
        __syncthreads();                                               // B_passed
        return true;
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

hipError_t launch_chain_plan(const ChainStep* steps, int nsteps, uint8_t* ws, hipStream_t stream)
{
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
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel, 64 * kChainWaves, kChainLds);
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
    ChainCounters* ctr = (ChainCounters*)ws;
    uint32_t* hdr = (uint32_t*)(ws + kChainHeaderOffset);
    void* args[] = {&plan, &ctr, &hdr, &nsteps};
    return hipLaunchCooperativeKernel((const void*)chain_kernel, dim3((unsigned)grid), dim3(64 * kChainWaves), args,
                                      kChainLds, stream);
}

}  // namespace tern
