/*
 * tern_oracle.c — TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, obviously-correct CPU implementation of everything the
 * ternary decode path computes, in fp64 where the method is floating point.
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load it.  It shares no code, header, table or helper with the HIP
 * library: the packed layout is re-implemented here from its written
 * definition, bit by bit.
 *
 * What each function follows (pages of the Neutrino-1 discussion, and the
 * reading taken where they are silent):
 *  - ternary linear: "Fermion Research, 3진 계열 포맷으로 직접 학습한 Neutrino-1
 *    모델군 3종 공개" (discuss.pytorch.kr), section "학습 중에 포맷이 있어야 하는
 *    이유", equation y_j = sum_i w_ij x_i; with w in {-1,0,+1} the product is
 *    add / skip / subtract (origotech.dev low-bit essay, Figure I).
 *  - one shared scale per small block of weights: origotech.dev essay,
 *    section "어떻게 작동하나" (block-wise scaling).
 *  - separate bit-planes per block (the FV5 table of the discuss.pytorch.kr
 *    page, section "FV5와 FV5B").  The exact plane layout is not published;
 *    the layout below is this project's own definition.
 *  - int8 output head: same page, section "3진 계열이라는 이름의 실체"
 *    (embedding and head stay int8) and the FV5B row of the FV5 table.
 *  - int8 activations: same page, section "토큰 동일성의 경계" (an int8
 *    activation runtime exists; no quantizer is described, so the plain
 *    absmax/127 reading is used).
 *
 * Packed layout (the definition this file implements):
 *   Weights W[N][K], K % 128 == 0.  Block (n, b) = row n, k in [128b, 128b+128),
 *   with one fp16 scale.  Rows are padded to Np = ceil(N/16)*16 (padding rows
 *   are zero with zero scales).  Each block has a nonzero plane and a sign
 *   plane of 128 bits each, stored as four little-endian 32-bit words per
 *   plane; word w of a plane holds the 32 weights k = 128b + 32w + i
 *   (i = 0..31) with weight i at bit 16*(i & 1) + (i >> 1).
 *   Word placement: row tile rt = n/16, r = n%16; k-tile kt = b/4, bq = b%4;
 *   nb = K/128; nbq = min(4, nb - 4kt) (the last k-tile may be narrower);
 *     word_index = (rt*nb + 4kt)*128 + ((plane*4 + w)*16 + r)*nbq + bq,
 *   plane 0 = nonzero, plane 1 = sign; byte offset = 4*word_index.
 *   Scales start at byte align256(Np*K/4); scale (n, b) is the fp16 at
 *   element (rt*nb + 4kt)*16 + r*nbq + bq.
 *   Total bytes = align256(Np*K/4) + Np*(K/128)*2.
 *   Decoding rule: t = nz ? (sign ? -1 : +1) : 0.  Canonical form has
 *   sign = 0 wherever nz = 0.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- layout */

static int64_t or_npad(int64_t N) { return (N + 15) / 16 * 16; }
static int64_t or_align256(int64_t v) { return (v + 255) / 256 * 256; }

int64_t oracle_packed_bytes(int64_t N, int64_t K)
{
    if (N < 0 || K < 0 || K % 128 != 0) return -1;
    int64_t np = or_npad(N);
    return or_align256(np * K / 4) + np * (K / 128) * 2;
}

static int64_t or_scale_region(int64_t N, int64_t K) { return or_align256(or_npad(N) * K / 4); }

/* word index of plane word (plane, w) of block (n, b) */
static int64_t or_word_index(int64_t n, int64_t b, int plane, int w, int64_t K)
{
    int64_t nb = K / 128, rt = n / 16, r = n % 16, kt = b / 4, bq = b % 4;
    int64_t nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
    return (rt * nb + 4 * kt) * 128 + (((int64_t)plane * 4 + w) * 16 + r) * nbq + bq;
}

static int64_t or_scale_index(int64_t n, int64_t b, int64_t K)
{
    int64_t nb = K / 128, rt = n / 16, r = n % 16, kt = b / 4, bq = b % 4;
    int64_t nbq = nb - 4 * kt < 4 ? nb - 4 * kt : 4;
    return (rt * nb + 4 * kt) * 16 + r * nbq + bq;
}

static int or_bitpos(int i) { return 16 * (i & 1) + (i >> 1); }

static uint32_t or_load_word(const uint8_t* p, int64_t wi)
{
    const uint8_t* q = p + 4 * wi;
    return (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
}

static void or_store_word(uint8_t* p, int64_t wi, uint32_t v)
{
    uint8_t* q = p + 4 * wi;
    q[0] = (uint8_t)v; q[1] = (uint8_t)(v >> 8); q[2] = (uint8_t)(v >> 16); q[3] = (uint8_t)(v >> 24);
}

static uint16_t or_load_u16(const uint8_t* p, int64_t idx)
{
    return (uint16_t)(p[2 * idx] | (p[2 * idx + 1] << 8));
}

/* decode weight (n, k) from the packed bytes */
static int or_weight(const uint8_t* packed, int64_t n, int64_t k, int64_t K)
{
    int64_t b = k / 128;
    int w = (int)((k % 128) / 32), i = (int)(k % 32);
    uint32_t nzw = or_load_word(packed, or_word_index(n, b, 0, w, K));
    uint32_t sgw = or_load_word(packed, or_word_index(n, b, 1, w, K));
    int nz = (nzw >> or_bitpos(i)) & 1, sg = (sgw >> or_bitpos(i)) & 1;
    return nz ? (sg ? -1 : 1) : 0;
}

/* ------------------------------------------------------ number formats */

/* IEEE binary16 bits -> double, including subnormals, inf and NaN */
double oracle_f16_to_f64(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* bfloat16 bits -> double (bfloat16 is the top half of an IEEE float) */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static float or_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ----------------------------------------------------------- pack/unpack */

/* t: int8 [N][K] in {-1,0,+1}; scale: fp16 bits [N][K/128]; out: packed bytes */
int oracle_pack(const int8_t* t, const uint16_t* scale, int64_t N, int64_t K, uint8_t* out)
{
    int64_t total = oracle_packed_bytes(N, K);
    if (total < 0) return 2;
    memset(out, 0, (size_t)total);
    int64_t nb = K / 128, s0 = or_scale_region(N, K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int v = t[n * K + k];
            if (v < -1 || v > 1) return 2;
            if (v == 0) continue;
            int64_t b = k / 128;
            int w = (int)((k % 128) / 32), i = (int)(k % 32);
            int64_t wn = or_word_index(n, b, 0, w, K);
            or_store_word(out, wn, or_load_word(out, wn) | (1u << or_bitpos(i)));
            if (v < 0) {
                int64_t ws = or_word_index(n, b, 1, w, K);
                or_store_word(out, ws, or_load_word(out, ws) | (1u << or_bitpos(i)));
            }
        }
        for (int64_t b = 0; b < nb; ++b) {
            uint16_t s = scale[n * nb + b];
            int64_t si = or_scale_index(n, b, K);
            out[s0 + 2 * si] = (uint8_t)(s & 255);
            out[s0 + 2 * si + 1] = (uint8_t)(s >> 8);
        }
    }
    return 0;
}

/* inverse of oracle_pack: t [N][K], scale [N][K/128] */
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* t, uint16_t* scale)
{
    if (oracle_packed_bytes(N, K) < 0) return 2;
    int64_t nb = K / 128, s0 = or_scale_region(N, K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) t[n * K + k] = (int8_t)or_weight(packed, n, k, K);
        for (int64_t b = 0; b < nb; ++b) scale[n * nb + b] = or_load_u16(packed + s0, or_scale_index(n, b, K));
    }
    return 0;
}

/* counts[0] = nonzero weights, counts[1] = -1 weights, counts[2] = sign bits
 * set where the nonzero bit is clear (non-canonical), over the N real rows */
int oracle_stats(const uint8_t* packed, int64_t N, int64_t K, uint64_t* counts)
{
    if (oracle_packed_bytes(N, K) < 0) return 2;
    uint64_t nz = 0, neg = 0, bad = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t b = k / 128;
            int w = (int)((k % 128) / 32), i = (int)(k % 32);
            int z = (or_load_word(packed, or_word_index(n, b, 0, w, K)) >> or_bitpos(i)) & 1;
            int s = (or_load_word(packed, or_word_index(n, b, 1, w, K)) >> or_bitpos(i)) & 1;
            nz += z; neg += z & s; bad += (!z) & s;
        }
    counts[0] = nz; counts[1] = neg; counts[2] = bad;
    return 0;
}

/* ------------------------------------------------------------ GEMV (bf16) */

/* y[m][n] = sum_b scale[n,b] * sum_{k in b} t[n,k] * x[m,k], exact in fp64
 * (every product is exact; only the fp64 sums round).  y64 gets the fp64
 * value, y32 (optional) the single rounding of it to fp32.  Rows n are those
 * listed in `rows` (or all N rows when rows == NULL); outputs are [M][nrows]. */
int oracle_gemv_bf16(const uint8_t* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                     const int64_t* rows, int64_t nrows, double* y64, float* y32)
{
    if (oracle_packed_bytes(N, K) < 0) return 2;
    if (rows == NULL) nrows = N;
    int64_t nb = K / 128, s0 = or_scale_region(N, K);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t n = rows ? rows[j] : j;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                double part = 0.0;
                for (int64_t k = 128 * b; k < 128 * b + 128; ++k) {
                    int v = or_weight(packed, n, k, K);
                    if (v) part += v * oracle_bf16_to_f64(x[m * K + k]);
                }
                acc += oracle_f16_to_f64(or_load_u16(packed + s0, or_scale_index(n, b, K))) * part;
            }
            y64[m * nrows + j] = acc;
            if (y32) y32[m * nrows + j] = (float)acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------- int8 activations */

/* Per row m: a = max_k |x[m,k]| (exact in fp32), s = a / 127 (fp32 IEEE
 * division, round-to-nearest-even), q = clamp(rint(x / s), -127, 127) with
 * the fp32 IEEE quotient and ties to even; a == 0 gives s = 0 and q = 0. */
int oracle_quantize_i8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s)
{
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(or_bf16_to_f32(x[m * K + k]));
            if (v > a) a = v;
        }
        float sv = a / 127.0f;
        s[m] = a == 0.0f ? 0.0f : sv;
        for (int64_t k = 0; k < K; ++k) {
            if (a == 0.0f) { q[m * K + k] = 0; continue; }
            float quot = or_bf16_to_f32(x[m * K + k]) / sv;
            float r = rintf(quot);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[m * K + k] = (int8_t)r;
        }
    }
    return 0;
}

/* int8-activation ternary contraction (GEMV for small M, prefill for large M):
 * acc[m][n][b] = sum_{k in b} t[n,k] * q[m,k]  (exact int32),
 * y[m][n] = s_x[m] * sum_b scale[n,b] * acc[m][n][b]  (fp64, one rounding to y32).
 * acc (optional) is [M][nrows][K/128]; y64 / y32 are [M][nrows]. */
int oracle_tern_i8(const uint8_t* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x,
                   int64_t M, const int64_t* rows, int64_t nrows, int32_t* acc, double* y64, float* y32)
{
    if (oracle_packed_bytes(N, K) < 0) return 2;
    if (rows == NULL) nrows = N;
    int64_t nb = K / 128, s0 = or_scale_region(N, K);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t n = rows ? rows[j] : j;
        for (int64_t m = 0; m < M; ++m) {
            double tot = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int32_t a = 0;
                for (int64_t k = 128 * b; k < 128 * b + 128; ++k) a += or_weight(packed, n, k, K) * q[m * K + k];
                if (acc) acc[(m * nrows + j) * nb + b] = a;
                tot += oracle_f16_to_f64(or_load_u16(packed + s0, or_scale_index(n, b, K))) * (double)a;
            }
            double y = (double)s_x[m] * tot;
            if (y64) y64[m * nrows + j] = y;
            if (y32) y32[m * nrows + j] = (float)y;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ head */

/* logits[m][v] = rs[v] * sum_k W[v,k] * x[m,k] in fp64 (W int8 row-major [V][K]) */
int oracle_head_bf16(const int8_t* W, const float* rs, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                     const int64_t* rows, int64_t nrows, double* y64, float* y32)
{
    if (rows == NULL) nrows = V;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t v = rows ? rows[j] : j;
        for (int64_t m = 0; m < M; ++m) {
            double a = 0.0;
            for (int64_t k = 0; k < K; ++k) a += (double)W[v * K + k] * oracle_bf16_to_f64(x[m * K + k]);
            double y = (double)rs[v] * a;
            y64[m * nrows + j] = y;
            if (y32) y32[m * nrows + j] = (float)y;
        }
    }
    return 0;
}

/* int8-activation head: acc[m][v] = sum_k W[v,k] * q[m,k] (exact int32),
 * logits = rs[v] * s_x[m] * acc in fp64 */
int oracle_head_i8(const int8_t* W, const float* rs, int64_t V, int64_t K, const int8_t* q, const float* s_x,
                   int64_t M, const int64_t* rows, int64_t nrows, int32_t* acc, double* y64, float* y32)
{
    if (rows == NULL) nrows = V;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t v = rows ? rows[j] : j;
        for (int64_t m = 0; m < M; ++m) {
            int32_t a = 0;
            for (int64_t k = 0; k < K; ++k) a += (int32_t)W[v * K + k] * (int32_t)q[m * K + k];
            if (acc) acc[m * nrows + j] = a;
            double y = (double)rs[v] * (double)s_x[m] * (double)a;
            if (y64) y64[m * nrows + j] = y;
            if (y32) y32[m * nrows + j] = (float)y;
        }
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* threads of the OpenMP loops from now on (n >= 1); returns the count in effect */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
