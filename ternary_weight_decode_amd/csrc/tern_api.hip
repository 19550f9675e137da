// tern_api.hip — the extern "C" surface declared in include/tern.h.
//
// Every entry point validates shapes, pointers and alignment on the host
// before any HIP call (so argument errors are testable without a device),
// checks once per device that it is a gfx950, and enqueues the launchers of
// tern_launch.h on the caller's stream.  Nothing here allocates, frees or
// synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/tern.h"
#include "tern_launch.h"

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e)
{
    const char* s = hipGetErrorString(e);
    std::strncpy(g_last_error, s ? s : "unknown HIP error", sizeof(g_last_error) - 1);
    g_last_error[sizeof(g_last_error) - 1] = 0;
    return TERN_E_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// per-device result of the gfx950 check: 0 unknown, 1 ok, 2 not gfx950
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];

int check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return TERN_E_DEVICE;
    int st = g_device_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? TERN_OK : TERN_E_DEVICE;
}

int finish(hipError_t e) { return e == hipSuccess ? TERN_OK : hip_fail(e); }

bool bad_nk(int64_t N, int64_t K) { return N < 0 || K < 0 || K % 128 != 0; }

}  // namespace

extern "C" {

const char* tern_strerror(int status)
{
    switch (status) {
    case TERN_OK: return "ok";
    case TERN_E_NULL: return "null pointer argument";
    case TERN_E_SHAPE: return "invalid shape (negative size, K not a multiple of 128, or M out of range)";
    case TERN_E_ALIGN: return "pointer not 16-byte aligned";
    case TERN_E_HIP: return "HIP error (see tern_last_error)";
    case TERN_E_DEVICE: return "current device is not a gfx950 (MI355X)";
    default: return "unknown tern status";
    }
}

const char* tern_last_error(void) { return g_last_error; }

int tern_abi_version(void) { return TERN_ABI_VERSION; }

int64_t tern_packed_bytes(int64_t N, int64_t K)
{
    if (bad_nk(N, K)) return -1;
    return tern::align256(tern::npad16(N) * K / 4) + tern::npad16(N) * (K / 128) * 2;
}

int tern_pack(const int8_t* t, const uint16_t* scale, int64_t N, int64_t K, void* packed, void* stream)
{
    if (bad_nk(N, K)) return TERN_E_SHAPE;
    if (N == 0 || K == 0) return TERN_OK;
    if (!t || !scale || !packed) return TERN_E_NULL;
    if (!aligned16(t) || !aligned16(packed) || ((uintptr_t)scale & 1u)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_pack(t, scale, N, K, (uint8_t*)packed, (hipStream_t)stream));
}

int tern_stats(const void* packed, int64_t N, int64_t K, uint64_t* counts, void* stream)
{
    if (bad_nk(N, K)) return TERN_E_SHAPE;
    if (!counts || (!packed && N > 0 && K > 0)) return TERN_E_NULL;
    if ((packed && !aligned16(packed)) || ((uintptr_t)counts & 7u)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_stats((const uint8_t*)packed, N, K, counts, (hipStream_t)stream));
}

int tern_quantize_i8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s_x, void* stream)
{
    if (M < 0 || K < 0 || K % 16 != 0) return TERN_E_SHAPE;
    if (M == 0) return TERN_OK;
    if (!s_x || (K > 0 && (!x || !q))) return TERN_E_NULL;
    if ((x && !aligned16(x)) || (q && !aligned16(q)) || !aligned4(s_x)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_quantize(x, M, K, q, s_x, (hipStream_t)stream));
}

int tern_gemv(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y, void* stream)
{
    if (bad_nk(N, K) || M < 0 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (N == 0 || M == 0) return TERN_OK;
    if (!y || (K > 0 && (!packed || !x))) return TERN_E_NULL;
    if ((packed && !aligned16(packed)) || (x && !aligned16(x)) || !aligned4(y)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    if (K == 0) return finish(tern::launch_fill_zero(y, M * N * 4, (hipStream_t)stream));
    return finish(tern::launch_gemv_bf16((const uint8_t*)packed, N, K, x, M, y, (hipStream_t)stream));
}

int tern_gemv_i8(const void* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M, float* y,
                 int32_t* acc_dbg, void* stream)
{
    if (bad_nk(N, K) || M < 0 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (N == 0 || M == 0) return TERN_OK;
    if (!y || !s_x || (K > 0 && (!packed || !q))) return TERN_E_NULL;
    if ((packed && !aligned16(packed)) || (q && !aligned16(q)) || !aligned4(y) || !aligned4(s_x) ||
        (acc_dbg && !aligned4(acc_dbg)))
        return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    if (K == 0) return finish(tern::launch_fill_zero(y, M * N * 4, (hipStream_t)stream));
    return finish(tern::launch_gemv_i8((const uint8_t*)packed, N, K, q, s_x, M, y, acc_dbg, (hipStream_t)stream));
}

int i8_head_gemv(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                 float* logits, void* stream)
{
    if (bad_nk(V, K) || M < 0 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (V == 0 || M == 0) return TERN_OK;
    if (!logits || !row_scale || (K > 0 && (!W || !x))) return TERN_E_NULL;
    if ((W && !aligned16(W)) || (x && !aligned16(x)) || !aligned4(logits) || !aligned4(row_scale))
        return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    if (K == 0) return finish(tern::launch_fill_zero(logits, M * V * 4, (hipStream_t)stream));
    return finish(tern::launch_head_bf16(W, row_scale, V, K, x, M, logits, (hipStream_t)stream));
}

int i8_head_gemv_i8(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                    const float* s_x, int64_t M, float* logits, int32_t* acc_dbg, void* stream)
{
    if (bad_nk(V, K) || M < 0 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (V == 0 || M == 0) return TERN_OK;
    if (!logits || !row_scale || !s_x || (K > 0 && (!W || !q))) return TERN_E_NULL;
    if ((W && !aligned16(W)) || (q && !aligned16(q)) || !aligned4(logits) || !aligned4(row_scale) ||
        !aligned4(s_x) || (acc_dbg && !aligned4(acc_dbg)))
        return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    if (K == 0) {
        rc = finish(tern::launch_fill_zero(logits, M * V * 4, (hipStream_t)stream));
        if (rc || !acc_dbg) return rc;
        return finish(tern::launch_fill_zero(acc_dbg, M * V * 4, (hipStream_t)stream));
    }
    return finish(tern::launch_head_i8(W, row_scale, V, K, q, s_x, M, logits, acc_dbg, (hipStream_t)stream));
}

int64_t i8_head_packed_bytes(int64_t V, int64_t K)
{
    if (V < 1 || V > 0xFFFFFFF0ll || K < 128 || K % 128 != 0 || K > (1ll << 20)) return -1;
    return tern::head_packed_bytes(V, K);
}

int i8_head_pack(const int8_t* W, int64_t V, int64_t K, int8_t* packed, void* stream)
{
    if (i8_head_packed_bytes(V, K) < 0) return TERN_E_SHAPE;
    if (!W || !packed) return TERN_E_NULL;
    if (!aligned16(W) || !aligned16(packed)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_head_pack(W, V, K, packed, (hipStream_t)stream));
}

int i8_head_gemv_packed(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const uint16_t* x,
                        int64_t M, float* logits, void* stream)
{
    if (i8_head_packed_bytes(V, K) < 0 || M < 1 || M > TERN_MAX_M_GEMV || !tern::head_packed_fits(K, M, false))
        return TERN_E_SHAPE;
    if (!packed || !row_scale || !x || !logits) return TERN_E_NULL;
    if (!aligned16(packed) || !aligned16(x) || !aligned4(logits) || !aligned4(row_scale)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_head_packed_bf16(packed, row_scale, V, K, x, M, logits, (hipStream_t)stream));
}

int i8_head_gemv_packed_i8(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                           const float* s_x, int64_t M, float* logits, int32_t* acc_dbg, void* stream)
{
    if (i8_head_packed_bytes(V, K) < 0 || M < 1 || M > TERN_MAX_M_GEMV || !tern::head_packed_fits(K, M, true))
        return TERN_E_SHAPE;
    if (!packed || !row_scale || !q || !s_x || !logits) return TERN_E_NULL;
    if (!aligned16(packed) || !aligned16(q) || !aligned4(logits) || !aligned4(row_scale) || !aligned4(s_x) ||
        (acc_dbg && !aligned4(acc_dbg)))
        return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_head_packed_i8(packed, row_scale, V, K, q, s_x, M, logits, acc_dbg,
                                              (hipStream_t)stream));
}

int64_t i8_head_argmax_workspace_bytes(int64_t V, int64_t M)
{
    if (V < 1 || V > 0xFFFFFFF0ll || M < 1 || M > TERN_MAX_M_GEMV) return -1;
    return (V + 15) / 16 * M * 8;
}

static int head_argmax_check(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const void* act,
                             const float* s_x, bool int8_act, int64_t M, int32_t* idx, float* val, float* logits,
                             void* workspace, bool need_workspace = true)
{
    if (bad_nk(V, K) || K == 0 || V < 1 || V > 0xFFFFFFF0ll || M < 1 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (!tern::head_argmax_fits(K, M, int8_act)) return TERN_E_SHAPE;
    if (!W || !row_scale || !act || !idx || !val || (need_workspace && !workspace) || (int8_act && !s_x))
        return TERN_E_NULL;
    if (!aligned16(W) || !aligned16(act) || !aligned4(row_scale) || !aligned4(idx) || !aligned4(val) ||
        (logits && !aligned4(logits)) || (s_x && !aligned4(s_x)) || ((uintptr_t)workspace & 7))
        return TERN_E_ALIGN;
    return check_device();
}

int i8_head_argmax(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                   int32_t* idx, float* val, float* logits, void* workspace, void* stream)
{
    const int rc = head_argmax_check(W, row_scale, V, K, x, nullptr, false, M, idx, val, logits, workspace);
    if (rc) return rc;
    return finish(tern::launch_head_argmax_bf16(W, row_scale, V, K, x, M, logits, idx, val, workspace,
                                                (hipStream_t)stream));
}

int i8_head_argmax_noalloc(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const uint16_t* x,
                           int64_t M, int32_t* idx, float* val, float* logits, void* stream)
{
    if (V >= 1 && M >= 1 && M <= TERN_MAX_M_GEMV && V <= 0xFFFFFFF0ll &&
        i8_head_argmax_workspace_bytes(V, M) > tern::kHeadArgmaxScratchBytes)
        return TERN_E_SHAPE;
    // the checks of i8_head_argmax, without a workspace (the library's array holds the keys)
    const int rc = head_argmax_check(W, row_scale, V, K, x, nullptr, false, M, idx, val, logits, nullptr, false);
    if (rc) return rc;
    return finish(tern::launch_head_argmax_bf16_noalloc(W, row_scale, V, K, x, M, logits, idx, val,
                                                        (hipStream_t)stream));
}

int i8_head_argmax_packed(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const uint16_t* x,
                          int64_t M, int32_t* idx, float* val, float* logits, void* workspace, void* stream)
{
    if (i8_head_packed_bytes(V, K) < 0) return TERN_E_SHAPE;
    const int rc = head_argmax_check(packed, row_scale, V, K, x, nullptr, false, M, idx, val, logits, workspace);
    if (rc) return rc;
    return finish(tern::launch_head_argmax_packed_bf16(packed, row_scale, V, K, x, M, logits, idx, val, workspace,
                                                       (hipStream_t)stream));
}

int i8_head_argmax_packed_i8(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                             const float* s_x, int64_t M, int32_t* idx, float* val, float* logits, void* workspace,
                             void* stream)
{
    if (i8_head_packed_bytes(V, K) < 0) return TERN_E_SHAPE;
    const int rc = head_argmax_check(packed, row_scale, V, K, q, s_x, true, M, idx, val, logits, workspace);
    if (rc) return rc;
    return finish(tern::launch_head_argmax_packed_i8(packed, row_scale, V, K, q, s_x, M, logits, idx, val, workspace,
                                                     (hipStream_t)stream));
}

int i8_head_argmax_i8(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                      const float* s_x, int64_t M, int32_t* idx, float* val, float* logits, void* workspace,
                      void* stream)
{
    const int rc = head_argmax_check(W, row_scale, V, K, q, s_x, true, M, idx, val, logits, workspace);
    if (rc) return rc;
    return finish(tern::launch_head_argmax_i8(W, row_scale, V, K, q, s_x, M, logits, idx, val, workspace,
                                              (hipStream_t)stream));
}

int tern_gemm_prefill(const void* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M,
                      float* y, int32_t* acc_dbg, void* stream)
{
    if (bad_nk(N, K) || M < 0) return TERN_E_SHAPE;
    if (N == 0 || M == 0) return TERN_OK;
    if (!y || !s_x || (K > 0 && (!packed || !q))) return TERN_E_NULL;
    if ((packed && !aligned16(packed)) || (q && !aligned16(q)) || !aligned4(y) || !aligned4(s_x) ||
        (acc_dbg && !aligned4(acc_dbg)))
        return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    if (K == 0) return finish(tern::launch_fill_zero(y, M * N * 4, (hipStream_t)stream));
    return finish(tern::launch_prefill((const uint8_t*)packed, N, K, q, s_x, M, y, acc_dbg, (hipStream_t)stream));
}

namespace {

// Byte offsets of the hand-off buffers of a chain (0 for steps that feed no
// later step) and the workspace size; -1 if the step links are invalid.
int64_t chain_layout(const tern_chain_step* steps, int64_t nsteps, std::vector<int64_t>* offs,
                     std::vector<char>* feeds, int64_t* begin)
{
    if (nsteps < 0 || nsteps >= tern::kChainMaxSteps || (nsteps > 0 && !steps)) return -1;
    std::vector<char> f((size_t)nsteps, 0);
    for (int64_t p = 0; p < nsteps; ++p) {
        const int64_t q = steps[p].x_from;
        if (q < -1 || q >= p) return -1;
        if (q >= 0) f[(size_t)q] = 1;
    }
    int64_t at = tern::align256(tern::kChainPlanOffset + nsteps * (int64_t)sizeof(tern::ChainStep));
    if (begin) *begin = at;
    if (offs) offs->assign((size_t)nsteps, 0);
    for (int64_t p = 0; p < nsteps; ++p) {
        if (!f[(size_t)p]) continue;
        if (steps[p].N < 1) return -1;
        if (offs) (*offs)[(size_t)p] = at;
        at += tern::align256((steps[p].N + 1) / 2 * 8);
    }
    if (feeds) *feeds = f;
    return at;
}

bool overlap(const void* a, int64_t na, const void* b, int64_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a && b && na > 0 && nb > 0 && a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

int64_t tern_chain_workspace_bytes(const tern_chain_step* steps, int64_t nsteps)
{
    return chain_layout(steps, nsteps, nullptr, nullptr, nullptr);
}

int tern_chain_plan(const tern_chain_step* steps, int64_t nsteps, void* workspace, int64_t workspace_bytes,
                    void* stream)
{
    if (nsteps < 0 || nsteps >= tern::kChainMaxSteps) return TERN_E_SHAPE;
    if (!workspace || (nsteps > 0 && !steps)) return TERN_E_NULL;
    if (((uintptr_t)workspace & 255u) != 0) return TERN_E_ALIGN;
    for (int64_t p = 0; p < nsteps; ++p) {
        const tern_chain_step& st = steps[p];
        if (st.N < 1 || st.K < 512 || st.K % 512 != 0 || st.K > tern::kChainMaxK) return TERN_E_SHAPE;
        if (st.x_from < -1 || st.x_from >= p) return TERN_E_SHAPE;
        if (st.x_from >= 0 && st.K > steps[st.x_from].N) return TERN_E_SHAPE;
        if (!st.packed || !st.y || (st.x_from < 0 && !st.x)) return TERN_E_NULL;
        if (!aligned16(st.packed) || !aligned4(st.y) || (st.x_from < 0 && !aligned16(st.x))) return TERN_E_ALIGN;
    }
    // steps without a hand-off between them may run at the same time, so no
    // output may overlap another output, an input vector or packed weights
    for (int64_t p = 0; p < nsteps; ++p) {
        const tern_chain_step& a = steps[p];
        for (int64_t q = 0; q < nsteps; ++q) {
            const tern_chain_step& c = steps[q];
            if (q != p && overlap(a.y, a.N * 4, c.y, c.N * 4)) return TERN_E_SHAPE;
            if (c.x_from < 0 && overlap(a.y, a.N * 4, c.x, c.K * 2)) return TERN_E_SHAPE;
            if (overlap(a.y, a.N * 4, c.packed, tern_packed_bytes(c.N, c.K))) return TERN_E_SHAPE;
        }
    }
    std::vector<int64_t> offs;
    std::vector<char> feeds;
    int64_t begin = 0;
    const int64_t need = chain_layout(steps, nsteps, &offs, &feeds, &begin);
    if (need < 0 || workspace_bytes < need) return TERN_E_SHAPE;
    std::vector<tern::ChainStep> plan((size_t)nsteps);
    for (int64_t p = 0; p < nsteps; ++p) {
        const tern_chain_step& st = steps[p];
        tern::ChainStep& d = plan[(size_t)p];
        d = tern::ChainStep{};
        d.packed = (const uint8_t*)st.packed;
        d.x = st.x_from < 0 ? st.x : nullptr;
        d.y = st.y;
        d.N = st.N;
        d.K = st.K;
        d.x_from = (int32_t)st.x_from;
        d.feeds = feeds[(size_t)p] ? 1u : 0u;
        d.hand_off = offs[(size_t)p];
        d.x_hand_off = st.x_from >= 0 ? offs[(size_t)st.x_from] : 0;
    }
    int rc = check_device();
    if (rc) return rc;
    int grid = 0;
    hipError_t e = tern::chain_grid(&grid);
    if (e != hipSuccess) return hip_fail(e);
    for (const tern::ChainStep& d : plan) {
        const int64_t nrt = (d.N + 15) / 16, nkt = d.K / 512;
        const int64_t per_cu = (nrt + grid - 1) / grid;
        if (per_cu * nkt * 16 > tern::kChainRedMax) return TERN_E_SHAPE;
    }
    return finish(tern::launch_chain_plan(plan.data(), (int)nsteps, (uint8_t*)workspace, begin, need,
                                          (hipStream_t)stream));
}

int tern_gemv_chain(void* workspace, int64_t nsteps, void* stream)
{
    if (nsteps < 0 || nsteps >= tern::kChainMaxSteps) return TERN_E_SHAPE;
    if (!workspace) return TERN_E_NULL;
    if (((uintptr_t)workspace & 255u) != 0) return TERN_E_ALIGN;
    if (nsteps == 0) return TERN_OK;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_chain((uint8_t*)workspace, (int)nsteps, (hipStream_t)stream));
}

}  // extern "C"

extern "C" {

int64_t tern5_packed_bytes(int64_t N, int64_t K)
{
    if (N < 0 || K < 0 || K % 512 != 0) return -1;
    return tern::npad16(N) * K * 3 / 8 + tern::npad16(N) * (K / 256) * 8;
}

int tern5_pack(const int8_t* levels, const float* s_lo, const float* s_hi, int64_t N, int64_t K, void* packed,
               void* stream)
{
    if (N < 0 || K < 0 || K % 512 != 0) return TERN_E_SHAPE;
    if (N == 0 || K == 0) return TERN_OK;
    if (!levels || !s_lo || !s_hi || !packed) return TERN_E_NULL;
    if (!aligned16(levels) || !aligned16(packed) || !aligned4(s_lo) || !aligned4(s_hi)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_pack5(levels, s_lo, s_hi, N, K, (uint8_t*)packed, (hipStream_t)stream));
}

int tern5_gemv_i8(const void* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M, float* y,
                  int32_t* acc_dbg, void* stream)
{
    if (N < 0 || K < 0 || K % 512 != 0 || M < 0 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (N == 0 || M == 0) return TERN_OK;
    if (!y || !s_x || (K > 0 && (!packed || !q))) return TERN_E_NULL;
    if ((packed && !aligned16(packed)) || (q && !aligned16(q)) || !aligned4(y) || !aligned4(s_x) ||
        (acc_dbg && !aligned4(acc_dbg)))
        return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    if (K == 0) return finish(tern::launch_fill_zero(y, M * N * 4, (hipStream_t)stream));
    return finish(tern::launch_gemv5_i8((const uint8_t*)packed, N, K, q, s_x, M, y, acc_dbg, (hipStream_t)stream));
}

int tern5_gemv(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y, void* stream)
{
    if (N < 0 || K < 0 || K % 512 != 0 || M < 0 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (N == 0 || M == 0) return TERN_OK;
    if (!y || (K > 0 && (!packed || !x))) return TERN_E_NULL;
    if ((packed && !aligned16(packed)) || (x && !aligned16(x)) || !aligned4(y)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    if (K == 0) return finish(tern::launch_fill_zero(y, M * N * 4, (hipStream_t)stream));
    return finish(tern::launch_gemv5_bf16((const uint8_t*)packed, N, K, x, M, y, (hipStream_t)stream));
}

}  // extern "C"

// ---- block-scaled (FV5B-style) head and embedding rows

namespace {

int fv5b_head_check(const int8_t* W, const float* S, int64_t V, int64_t K, const void* act, const float* s_x,
                    bool int8_act, int64_t M, const void* out, bool out_4)
{
    if (V < 1 || V > 0xFFFFFFF0ll || K < 256 || K % 256 != 0 || M < 1 || M > TERN_MAX_M_GEMV) return TERN_E_SHAPE;
    if (!tern::head_argmax_fits(K, M, int8_act)) return TERN_E_SHAPE;
    if (!W || !S || !act || !out || (int8_act && !s_x)) return TERN_E_NULL;
    if (!aligned16(W) || !aligned16(act) || !aligned4(S) || (s_x && !aligned4(s_x)) || (out_4 && !aligned4(out)))
        return TERN_E_ALIGN;
    return TERN_OK;
}

}  // namespace

extern "C" {

int fv5b_head_gemv(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                   float* logits, void* stream)
{
    int rc = fv5b_head_check(W, S, V, K, x, nullptr, false, M, logits, true);
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_bf16(W, S, V, K, x, M, logits, (hipStream_t)stream));
}

int fv5b_head_gemv_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q, const float* s_x,
                      int64_t M, float* logits, int32_t* acc_dbg, void* stream)
{
    int rc = fv5b_head_check(W, S, V, K, q, s_x, true, M, logits, true);
    if (rc) return rc;
    if (acc_dbg && !aligned4(acc_dbg)) return TERN_E_ALIGN;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_i8(W, S, V, K, q, s_x, M, logits, acc_dbg, (hipStream_t)stream));
}

int fv5b_head_argmax(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                     int32_t* idx, float* val, float* logits, void* workspace, void* stream)
{
    int rc = fv5b_head_check(W, S, V, K, x, nullptr, false, M, workspace, false);
    if (rc) return rc;
    if (!idx || !val) return TERN_E_NULL;
    if (!aligned4(idx) || !aligned4(val) || (logits && !aligned4(logits)) || ((uintptr_t)workspace & 7))
        return TERN_E_ALIGN;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_argmax_bf16(W, S, V, K, x, M, logits, idx, val, workspace,
                                                     (hipStream_t)stream));
}

int fv5b_head_argmax_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q, const float* s_x,
                        int64_t M, int32_t* idx, float* val, float* logits, void* workspace, void* stream)
{
    int rc = fv5b_head_check(W, S, V, K, q, s_x, true, M, workspace, false);
    if (rc) return rc;
    if (!idx || !val) return TERN_E_NULL;
    if (!aligned4(idx) || !aligned4(val) || (logits && !aligned4(logits)) || ((uintptr_t)workspace & 7))
        return TERN_E_ALIGN;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_argmax_i8(W, S, V, K, q, s_x, M, logits, idx, val, workspace,
                                                   (hipStream_t)stream));
}

int fv5b_head_gemv_packed(const int8_t* packed, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                          float* logits, void* stream)
{
    int rc = fv5b_head_check(packed, S, V, K, x, nullptr, false, M, logits, true);
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_packed_bf16(packed, S, V, K, x, M, logits, (hipStream_t)stream));
}

int fv5b_head_gemv_packed_i8(const int8_t* packed, const float* S, int64_t V, int64_t K, const int8_t* q,
                             const float* s_x, int64_t M, float* logits, int32_t* acc_dbg, void* stream)
{
    int rc = fv5b_head_check(packed, S, V, K, q, s_x, true, M, logits, true);
    if (rc) return rc;
    if (acc_dbg && !aligned4(acc_dbg)) return TERN_E_ALIGN;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_packed_i8(packed, S, V, K, q, s_x, M, logits, acc_dbg, (hipStream_t)stream));
}

int fv5b_head_argmax_packed(const int8_t* packed, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                            int32_t* idx, float* val, float* logits, void* workspace, void* stream)
{
    int rc = fv5b_head_check(packed, S, V, K, x, nullptr, false, M, workspace, false);
    if (rc) return rc;
    if (!idx || !val) return TERN_E_NULL;
    if (!aligned4(idx) || !aligned4(val) || (logits && !aligned4(logits)) || ((uintptr_t)workspace & 7))
        return TERN_E_ALIGN;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_argmax_packed_bf16(packed, S, V, K, x, M, logits, idx, val, workspace,
                                                            (hipStream_t)stream));
}

int fv5b_head_argmax_packed_i8(const int8_t* packed, const float* S, int64_t V, int64_t K, const int8_t* q,
                               const float* s_x, int64_t M, int32_t* idx, float* val, float* logits, void* workspace,
                               void* stream)
{
    int rc = fv5b_head_check(packed, S, V, K, q, s_x, true, M, workspace, false);
    if (rc) return rc;
    if (!idx || !val) return TERN_E_NULL;
    if (!aligned4(idx) || !aligned4(val) || (logits && !aligned4(logits)) || ((uintptr_t)workspace & 7))
        return TERN_E_ALIGN;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_argmax_packed_i8(packed, S, V, K, q, s_x, M, logits, idx, val, workspace,
                                                          (hipStream_t)stream));
}

int fv5b_head_argmax_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                           int32_t* idx, float* val, float* logits, void* workspace, const int8_t* E, const float* ES,
                           int64_t Ve, int64_t Ke, float* emb, uint16_t* emb_bf16, void* stream)
{
    int rc = fv5b_head_check(W, S, V, K, x, nullptr, false, M, workspace, false);
    if (rc) return rc;
    if (Ve < 1 || Ke < 256 || Ke % 256 != 0) return TERN_E_SHAPE;
    if (!idx || !val || !E || !ES || (!emb && !emb_bf16)) return TERN_E_NULL;
    if (!aligned4(idx) || !aligned4(val) || (logits && !aligned4(logits)) || ((uintptr_t)workspace & 7) ||
        !aligned16(E) || !aligned4(ES) || (emb && !aligned16(emb)) || (emb_bf16 && !aligned16(emb_bf16)))
        return TERN_E_ALIGN;
    if ((rc = check_device())) return rc;
    return finish(tern::launch_fv5b_head_argmax_embed(W, S, V, K, x, M, logits, idx, val, workspace, E, ES, Ve, Ke,
                                                      emb, emb_bf16, (hipStream_t)stream));
}

int fv5b_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const int32_t* ids, int64_t M, float* out,
               uint16_t* out_bf16, void* stream)
{
    if (V < 0 || K < 0 || K % 256 != 0 || M < 0) return TERN_E_SHAPE;
    if (M == 0 || K == 0) return TERN_OK;
    if (!ids || (!out && !out_bf16) || (V > 0 && (!W || !S))) return TERN_E_NULL;
    if ((W && !aligned16(W)) || (S && !aligned4(S)) || !aligned4(ids) || (out && !aligned16(out)) ||
        (out_bf16 && !aligned16(out_bf16)))
        return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_fv5b_embed(W, S, V, K, ids, M, out, out_bf16, (hipStream_t)stream));
}

}  // extern "C"

extern "C" {

int tern_gemv_config(int64_t N, int64_t K, int64_t M, int kind, int64_t* out)
{
    if (!out) return -TERN_E_NULL;
    if (kind < 0 || kind > 8 || N < 1 || K < 1 || M < 1 || M > TERN_MAX_M_GEMV) return -TERN_E_SHAPE;
    const bool i8 = (kind & 1) != 0;
    tern::OneShot c{};
    bool one;
    if (kind < 2) one = tern::gemv_oneshot_config(N, K, M, i8, c);
    else if (kind < 4) one = tern::gemv5_oneshot_config(N, K, M, i8, c);
    else if (kind < 6) one = !tern::gemv_oneshot_config(N, K, M, i8, c) && tern::gemv_phased_config(N, K, M, i8, c);
    else if (kind < 8) one = !tern::gemv5_oneshot_config(N, K, M, i8, c) && tern::gemv5_phased_config(N, K, M, i8, c);
    else one = !tern::gemv_oneshot_config(N, K, M, false, c) && !tern::gemv_phased_config(N, K, M, false, c) &&
               tern::gemv_phased3_config(N, K, M, c);
    if (!one) return 0;
    out[0] = c.R;
    out[1] = c.nw;
    out[2] = c.U;
    out[3] = c.XC;
    out[4] = c.grid;
    out[5] = (int64_t)c.lds;
    out[6] = c.rounds ? 1 : 0;
    out[7] = (kind >= 4 || M > 4 || c.XC == 8) ? 16 : (M == 1 ? 1 : (M == 2 ? 2 : 4));
    return 1;
}

int tern_prefill_config(int64_t N, int64_t K, int64_t M, int64_t* out)
{
    if (!out) return -TERN_E_NULL;
    if (N < 1 || K < 1 || M < 1 || K % 128 != 0) return -TERN_E_SHAPE;
    tern::Pf2Config c{};
    if (!tern::prefill2_config(N, K, M, c)) return 0;
    out[0] = c.BM;
    out[1] = c.BN;
    out[2] = c.split ? 1 : 0;
    out[3] = c.grid_x;
    out[4] = c.grid_y;
    out[5] = c.grid_z;
    return 1;
}

}  // extern "C"

extern "C" {

double tern_mfma_peak_ops(int kind, int64_t iters, int64_t grid)
{
    if ((kind != 0 && kind != 1) || iters < 0 || grid < 0) return -1.0;
    return tern::mfma_peak_ops(kind, iters, grid);
}

int64_t tern_mfma_peak_sink_bytes(int64_t grid)
{
    if (grid < 0) return -1;
    return tern::mfma_peak_sink_ints(grid) * 4;
}

int tern_mfma_peak(int kind, int64_t iters, int64_t grid, int32_t* sink, void* stream)
{
    if ((kind != 0 && kind != 1) || iters < 0 || grid < 1 || grid > 0x7FFFFFFF) return TERN_E_SHAPE;
    if (!sink) return TERN_E_NULL;
    if (!aligned16(sink)) return TERN_E_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_mfma_peak(kind, iters, grid, sink, (hipStream_t)stream));
}

int tern_launch_probe(int kind, int64_t grid, const void* src, int64_t src_bytes, float* sink, void* stream)
{
    if (kind < 0 || kind > 3 || grid < 1 || grid > 0x7FFFFFFF) return TERN_E_SHAPE;
    if (kind >= 1 && !sink) return TERN_E_NULL;
    if (kind >= 2) {
        if (!src) return TERN_E_NULL;
        if (!aligned16(src)) return TERN_E_ALIGN;
        if (src_bytes < 16 || src_bytes % 16 != 0) return TERN_E_SHAPE;
    }
    int rc = check_device();
    if (rc) return rc;
    return finish(tern::launch_probe(kind, grid, src, src_bytes, sink, (hipStream_t)stream));
}

}  // extern "C"
