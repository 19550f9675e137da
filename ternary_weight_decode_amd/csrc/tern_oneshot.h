// tern_oneshot.h — launch configuration of the one-pass GEMV kernels (the
// ternary and the five-level formats share it).
//
// A unit is one 16-row tile x one 512-k tile.  A workgroup owns R row tiles
// (every R-th of the grid) and its waves take U units each, all loads issued
// up front; activations are staged once in LDS (at M = 1 in bf16: each wave
// only the slices of its own units) and each unit leaves its fp32 partial in
// LDS, summed afterwards in k-tile order.  The whole grid must be resident in
// one round where a split allows it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

constexpr int64_t kCuLds = 160 * 1024;     // LDS of one gfx950 CU

inline int device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    return cus;
}

struct OneShot {
    int R, nw, U, XC;
    int64_t grid;
    size_t lds;
    bool rounds = false;   // the grid runs in several rounds (no split fits one)
    bool reuse = false;    // the partials overwrite x's LDS after the compute (x and partials exceed a CU side by side)
};

// units per wave for a workgroup of `units` units
inline int64_t oneshot_u(int64_t units)
{
    return units <= 8 ? 1 : ((units + 15) / 16 > 2 ? (units + 15) / 16 : 2);
}

// Activation staging and partials of one workgroup.
struct OneShotShape {
    int64_t x_row_bytes;      // staged LDS bytes per activation row
    int64_t x_src_bytes;      // bytes of one activation row in global memory
    int64_t chunk_bytes;      // activation bytes one thread loads per chunk
    int64_t waves_per_simd[5];// waves of U = 1..4 units that fit on a SIMD (registers)
    int64_t m1_slice_bytes;   // > 0: at M = 1 every wave stages only the activation slices of its
                              // own units (this many bytes per unit) instead of the whole row
    bool reuse_ok;            // bf16 rows above 8: partials may overwrite x after the compute
};

// R row tiles per workgroup is chosen to minimise the largest number of
// units any CU receives (the critical path), and among equals (at M > 1) to
// run one workgroup per CU, which stages x once, while a wave keeps at most
// two units (8B gate at M = 4: 6.32 -> 5.57 us with one workgroup of 12 waves
// per CU instead of three of 8; two workgroups per CU, or three units per
// wave, were slower on the fused gate|up), then to bring a workgroup
// closest to 16 units; waves take 2 units each (1 when a workgroup
// has at most 8), so the second unit's loads overlap the first unit's
// compute.  Measured on the 8B ternary shapes at M = 1 (hipGraph of 36
// launches, cold weights): 24576x4096 7.99 us with R = 2 / 8 waves vs 8.37 us
// (R = 3, 12 waves) and 9.17 us (R = 6, 16 waves); 6144x4096 4.58 us with
// R = 2 vs 4.87 us with R = 1; 4096x12288 5.64 us with 12 waves x 2 units vs
// 6.16 us with 8 x 3.  When no split fits one resident round (large N), the
// grid runs in several rounds with R chosen for about 16 units per
// workgroup: workgroups are independent, and on 49152..393216 x 4096 this
// streams 12-14% faster than the persistent kernel (up to 5.3 TB/s).
// Returns false when no configuration fits (another path runs then).
inline bool pick_oneshot(int64_t N, int64_t K, int64_t M, const OneShotShape& s, OneShot& c)
{
    if (K % 512 != 0 || M > 16) return false;
    const int64_t nkt = K / 512, nrt = (N + 15) / 16;
    const int64_t cus = device_cus();
    const int ni = M == 1 ? 1 : (M == 2 ? 2 : 4);
    // per-wave activation slices: at M = 1 (1 KiB per unit), and at M <= 8 with one row
    // tile per workgroup and at most two units per wave (2, 4 or 8 rows of 1040 bytes
    // per unit, held in registers until staged)
    const int64_t mr = M <= 2 ? 2 : (M <= 4 ? 4 : 8);
    auto slices_of = [&](int64_t R, int64_t U) {
        return s.m1_slice_bytes > 0 && (M == 1 || (M <= 8 && R == 1 && U <= 2));
    };
    auto lds_of = [&](int64_t units, int64_t R) {
        const int64_t U = oneshot_u(units), nw = (units + U - 1) / U;
        const size_t x_lds = !slices_of(R, U) ? (size_t)(M * s.x_row_bytes)
                             : M == 1      ? (size_t)(nw * U * s.m1_slice_bytes)
                                           : (size_t)(nw * U * mr * (s.m1_slice_bytes + 16));
        return x_lds + (size_t)(units + 1) * ni * 64 * 4;
    };
    // bf16 rows above 8 in one resident round: the partials may overwrite x after the compute
    // (x, the dummy slot of chunks past its end, and the partials, whichever is larger)
    auto reuse_lds_of = [&](int64_t units) {
        const size_t xs = (size_t)(M * s.x_row_bytes) + 16, ps = (size_t)(units + 1) * ni * 64 * 4;
        return xs > ps ? xs : ps;
    };
    // the partials over x only where no split fits one round side by side
    // (8B fused gate|up at M = 13..16, whose x alone is up to 128 KiB)
    const bool can_reuse = s.reuse_ok && s.chunk_bytes == 16 && M > 8;
    c.R = 0;
    c.reuse = false;
    for (int pass = 0; pass < (can_reuse ? 2 : 1) && c.R == 0; ++pass) {
        const bool reuse = pass == 1;
        int64_t best_max = -1, best_dist = 0, best_wg = 0;
        for (int R = 1; R <= 64 && R * nkt <= 64; ++R) {
            const int64_t units = R * nkt, U = oneshot_u(units);
            if (U > 4) break;
            const int64_t nw = (units + U - 1) / U;
            const int64_t grid = (nrt + R - 1) / R, per_cu = (grid + cus - 1) / cus;
            if (per_cu * nw > 4 * s.waves_per_simd[U]) continue;              // not resident in one round
            const size_t lds = reuse ? reuse_lds_of(units) : lds_of(units, R);
            if ((size_t)per_cu * lds > (size_t)kCuLds) continue;              // LDS of the workgroups on a CU
            const int64_t max_units = per_cu * units;
            const int64_t dist = units > 16 ? units - 16 : 16 - units;
            // among equal critical paths: at M > 1 one workgroup per CU first (x, M*K
            // elements, staged once per CU) as long as a wave keeps at most two units, then
            // the workgroup closest to 16 units
            const int64_t wg = M > 1 && per_cu == 1 && U <= 2 ? 0 : 1;
            if (best_max < 0 || max_units < best_max ||
                (max_units == best_max && (wg < best_wg || (wg == best_wg && dist < best_dist)))) {
                best_max = max_units;
                best_dist = dist;
                best_wg = wg;
                c.R = R;
                c.reuse = reuse;
            }
            if (grid == 1) break;
        }
    }
    c.rounds = false;
    if (c.R == 0) {
        // several rounds: the workgroup closest to 16 units whose LDS fits a CU
        int64_t best = -1;
        for (int R = 1; R <= 64 && R * nkt <= 64; ++R) {
            const int64_t units = R * nkt;
            if (oneshot_u(units) > 4 || lds_of(units, R) > (size_t)kCuLds) break;
            const int64_t dist = units > 16 ? units - 16 : 16 - units;
            if (best < 0 || dist < best) {
                best = dist;
                c.R = R;
            }
        }
        if (c.R == 0) return false;
        c.rounds = true;
    }
    const int64_t units = c.R * nkt;
    c.U = (int)oneshot_u(units);
    c.nw = (int)((units + c.U - 1) / c.U);
    c.grid = (nrt + c.R - 1) / c.R;
    const bool slices = slices_of(c.R, c.U);
    const int64_t xc = slices ? 1 : (M * (s.x_src_bytes / s.chunk_bytes) + 64 * c.nw - 1) / (64 * c.nw);
    // 8 chunks run on the MT = 16 kernels, whose partials hold 4 rows per
    // lane group: not for M <= 2, whose partial area is sized for 1 or 2;
    // 16 chunks (bf16 rows at M > 8, x up to 128 KiB) only in one resident
    // round, where every workgroup stages x once
    const int64_t xc_max = s.chunk_bytes == 16 && M > 8 && !c.rounds && c.U <= 3 ? 16 : 8;
    if (xc > xc_max || (xc > 4 && M <= 2)) return false;
    c.XC = xc <= 1 ? 1 : (xc <= 2 ? 2 : (xc <= 4 ? 4 : (xc <= 8 ? 8 : 16)));
    // the partials-over-x instances: two to four units per wave, 8 or 16 chunks
    if (c.reuse && (c.U < 2 || c.XC < 8 || (c.XC == 16 && c.U > 3))) return false;
    c.lds = c.reuse ? reuse_lds_of(units) : lds_of(units, c.R);
    return c.lds <= (size_t)kCuLds;
}

// true when `grid` workgroups of this kernel instance are resident at once
// (for a configuration that runs in rounds: when one workgroup fits a CU)
template <typename F>
inline bool oneshot_resident(F kern, const OneShot& c)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * c.nw, c.lds) != hipSuccess || per_cu <= 0)
        return false;
    return c.rounds || c.grid <= (int64_t)per_cu * device_cus();
}

}  // namespace tern
