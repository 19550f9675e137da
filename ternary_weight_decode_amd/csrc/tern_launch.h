// tern_launch.h — host-side launchers of the gfx950 kernels.  Arguments are
// already validated by the C ABI layer (tern_api.cpp); each launcher enqueues
// on `stream` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_oneshot.h"

namespace tern {

__host__ __device__ inline int64_t npad16(int64_t n) { return (n + 15) / 16 * 16; }
__host__ __device__ inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }
__host__ __device__ inline int64_t scale_region_offset(int64_t N, int64_t K) { return align256(npad16(N) * K / 4); }

hipError_t launch_fill_zero(void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_pack(const int8_t* t, const uint16_t* scale, int64_t N, int64_t K, uint8_t* packed,
                       hipStream_t stream);
hipError_t launch_stats(const uint8_t* packed, int64_t N, int64_t K, uint64_t* counts, hipStream_t stream);
hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t stream);
hipError_t launch_gemv_bf16(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                            hipStream_t stream);
hipError_t launch_gemv_i8(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                          int64_t M, float* y, int32_t* acc, hipStream_t stream);
// the one-pass configuration the GEMV launchers would take (false: another path)
bool gemv_oneshot_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c);
bool gemv5_oneshot_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c);
bool gemv_phased_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c);
bool gemv5_phased_config(int64_t N, int64_t K, int64_t M, bool i8, OneShot& c);
bool gemv_phased3_config(int64_t N, int64_t K, int64_t M, OneShot& c);
hipError_t launch_head_bf16(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                            float* y, hipStream_t stream);
hipError_t launch_head_i8(const int8_t* W, const float* rs, int64_t V, int64_t K, const int8_t* q,
                          const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream);
bool head_argmax_fits(int64_t K, int64_t M, bool int8_act);
hipError_t launch_head_argmax_bf16(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x,
                                   int64_t M, float* y, int32_t* idx, float* val, void* ws, hipStream_t stream);
hipError_t launch_head_argmax_i8(const int8_t* W, const float* rs, int64_t V, int64_t K, const int8_t* q,
                                 const float* s_x, int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                 hipStream_t stream);
// the head over its packed layout (workgroup-contiguous row groups of 64)
__host__ __device__ inline int64_t head_packed_bytes(int64_t V, int64_t K) { return (V + 63) / 64 * 64 * K; }
hipError_t launch_head_pack(const int8_t* W, int64_t V, int64_t K, int8_t* out, hipStream_t stream);
bool head_packed_fits(int64_t K, int64_t M, bool int8_act);
hipError_t launch_head_packed_bf16(const int8_t* Wp, const float* rs, int64_t V, int64_t K, const uint16_t* x,
                                   int64_t M, float* y, hipStream_t stream);
hipError_t launch_head_packed_i8(const int8_t* Wp, const float* rs, int64_t V, int64_t K, const int8_t* q,
                                 const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream);
hipError_t launch_head_argmax_packed_bf16(const int8_t* Wp, const float* rs, int64_t V, int64_t K,
                                          const uint16_t* x, int64_t M, float* y, int32_t* idx, float* val,
                                          void* ws, hipStream_t stream);
hipError_t launch_head_argmax_packed_i8(const int8_t* Wp, const float* rs, int64_t V, int64_t K, const int8_t* q,
                                        const float* s_x, int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                        hipStream_t stream);
// the bf16 head + argmax with its keys in a library-owned device array of
// kHeadArgmaxScratchBytes (no workspace argument, nothing allocated)
constexpr int64_t kHeadArgmaxScratchBytes = 2 << 20;
hipError_t launch_head_argmax_bf16_noalloc(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x,
                                           int64_t M, float* y, int32_t* idx, float* val, hipStream_t stream);
// ---- block-scaled (FV5B-style) head and embedding rows ----
hipError_t launch_fv5b_head_bf16(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                 int64_t M, float* y, hipStream_t stream);
hipError_t launch_fv5b_head_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q,
                               const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream);
hipError_t launch_fv5b_head_argmax_bf16(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                        int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                        hipStream_t stream);
hipError_t launch_fv5b_head_argmax_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q,
                                      const float* s_x, int64_t M, float* y, int32_t* idx, float* val, void* ws,
                                      hipStream_t stream);
hipError_t launch_fv5b_head_packed_bf16(const int8_t* Wp, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                        int64_t M, float* y, hipStream_t stream);
hipError_t launch_fv5b_head_packed_i8(const int8_t* Wp, const float* S, int64_t V, int64_t K, const int8_t* q,
                                      const float* s_x, int64_t M, float* y, int32_t* acc, hipStream_t stream);
hipError_t launch_fv5b_head_argmax_packed_bf16(const int8_t* Wp, const float* S, int64_t V, int64_t K,
                                               const uint16_t* x, int64_t M, float* y, int32_t* idx, float* val,
                                               void* ws, hipStream_t stream);
hipError_t launch_fv5b_head_argmax_packed_i8(const int8_t* Wp, const float* S, int64_t V, int64_t K,
                                             const int8_t* q, const float* s_x, int64_t M, float* y, int32_t* idx,
                                             float* val, void* ws, hipStream_t stream);
hipError_t launch_fv5b_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const int32_t* ids, int64_t M,
                             float* out, uint16_t* out_bf16, hipStream_t stream);
hipError_t launch_fv5b_head_argmax_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x,
                                         int64_t M, float* y, int32_t* idx, float* val, void* ws, const int8_t* E,
                                         const float* ES, int64_t Ve, int64_t Ke, float* emb, uint16_t* emb_bf16,
                                         hipStream_t stream);
// ---- GEMV chain (persistent, one workgroup per CU) ----
// Workspace layout: header at 0, plan entries at kChainPlanOffset, then the
// hand-off words of every step that feeds a later one (offsets in the plan).
constexpr int kChainWaves = 16;                   // 1 control + 15 compute waves
constexpr int kChainMaxK = 16384;                 // activation elements staged per step
constexpr int kChainRedMax = 4096;                // unit partial floats per workgroup and step
constexpr int kChainMaxSteps = 4096;              // steps per chain (the hand-off tag counts them)
constexpr size_t kChainLds = 96 * 1024;           // more than half the CU's LDS: one workgroup per CU
constexpr int64_t kChainPlanOffset = 4096;
constexpr uint32_t kChainMagic = 0x7E4C3A12u;
constexpr int kChainPlanBatch = 16;

struct ChainHeader {
    uint32_t magic;                               // kChainMagic once a plan is written
    uint32_t nsteps;                              // planned steps
    uint32_t errors;                              // aborted waits (byte offset 8)
    uint32_t epoch;                               // launches completed on this workspace
    unsigned long long done;                      // workgroups that finished, over all launches
};

struct ChainStep {                                // 64 bytes
    const uint8_t* packed;
    const uint16_t* x;                            // input vector when x_from < 0
    float* y;
    int64_t N, K;
    int32_t x_from;                               // -1, or the step whose output is x
    uint32_t feeds;                               // a later step reads this step's output
    int64_t hand_off;                             // workspace offset of this step's hand-off words
    int64_t x_hand_off;                           // workspace offset of the producer's words
};
static_assert(sizeof(ChainStep) == 64, "plan entry layout");

hipError_t launch_chain_plan(const ChainStep* steps, int nsteps, uint8_t* ws, int64_t hand_off_begin,
                             int64_t hand_off_end, hipStream_t stream);
hipError_t launch_chain(uint8_t* ws, int nsteps, hipStream_t stream);
hipError_t chain_grid(int* grid);

// ---- five-level (FV5-style) weights ----
hipError_t launch_pack5(const int8_t* lv, const float* s_lo, const float* s_hi, int64_t N, int64_t K,
                        uint8_t* packed, hipStream_t stream);
hipError_t launch_gemv5_bf16(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                             hipStream_t stream);
hipError_t launch_gemv5_i8(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M,
                           float* y, int32_t* acc, hipStream_t stream);

// ---- matrix-core throughput probe (measurement aid) ----
double mfma_peak_ops(int kind, int64_t iters, int64_t grid);
int64_t mfma_peak_sink_ints(int64_t grid);
hipError_t launch_mfma_peak(int kind, int64_t iters, int64_t grid, int32_t* sink, hipStream_t stream);
hipError_t launch_probe(int kind, int64_t grid, const void* src, int64_t src_bytes, float* sink, hipStream_t stream);

hipError_t launch_prefill(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                          int64_t M, float* y, int32_t* acc, hipStream_t stream);

// Host-side view of the workgroup-shared-decode prefill's launch (M >= 128, K % 512 == 0):
// workgroup tile, whether K is split in two halves, and the grid; false when another
// kernel takes the shape.
struct Pf2Config {
    int BM, BN;
    bool split;
    int64_t grid_x, grid_y, grid_z;
};
bool prefill2_config(int64_t N, int64_t K, int64_t M, Pf2Config& c);

}  // namespace tern
