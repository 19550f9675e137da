/*
 * tern.h — C ABI of libtern.so: ternary-weight GEMV / GEMM kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * The decode step these calls implement: every transformer linear of a
 * single-stream decode is a matrix-vector product over weights in {-1, 0, +1}
 * (add, skip or subtract), kept packed in HBM and decoded inside the matrix
 * kernel, plus an int8 output head.  Sources (pages on the Neutrino-1
 * ternary-family models):
 *   [P2] "Fermion Research, 3진 계열 포맷으로 직접 학습한 Neutrino-1 모델군 3종
 *        공개" (discuss.pytorch.kr).  Sections cited by their headings.
 *   [P4] aiatolah.com article announcing Neutrino-1 8B (Portuguese), sections
 *        cited by their headings.
 *   [P5] origotech.dev low-bit essay ("더 적은 비트로 계산하기"), Figure I.
 *
 * Conventions for every call
 *  - All data pointers are DEVICE pointers allocated by the caller (for
 *    example torch tensors), row-major and contiguous.  The library never
 *    allocates, frees or synchronises; each call enqueues its kernels on
 *    `stream` (a hipStream_t; NULL = the null stream) and returns at once.
 *  - Outputs are fully overwritten.  Inputs are never written.
 *  - Shapes are validated on the host before any HIP call, so a bad shape
 *    returns TERN_E_SHAPE without touching the device.  Empty problems
 *    (N == 0 or M == 0) return TERN_OK and enqueue nothing; K == 0 writes
 *    zeros.
 *  - Alignment: packed blobs, x, q and head rows must be 16-byte aligned.
 *  - Errors: a non-zero tern_status; tern_last_error() gives the HIP error
 *    string of the calling thread's last TERN_E_HIP.  Faults inside a kernel
 *    surface at the caller's next synchronisation.
 *  - The library keeps no mutable global state; calls are thread-safe.
 *
 * Packed ternary layout ("plane blob"), this library's own definition (the
 * shipped FV5 internals are not published, [P2] section "FV5와 FV5B"):
 *   W[N][K] with K % 128 == 0.  Block (n, b) covers k in [128b, 128b+128) of
 *   row n and has one fp16 scale (block-wise scaling, [P5] section
 *   "어떻게 작동하나"), a 128-bit nonzero plane and a 128-bit sign plane
 *   (34 bytes per 128 weights = 2.125 bits per weight).  Each plane is four
 *   little-endian 32-bit words; word w holds weights k = 128b + 32w + i,
 *   i = 0..31, with weight i at bit 16*(i&1) + (i>>1).  Rows are padded to
 *   Np = 16*ceil(N/16).  With rt = n/16, r = n%16, kt = b/4, bq = b%4,
 *   nb = K/128, nbq = min(4, nb - 4kt):
 *     word index  = (rt*nb + 4kt)*128 + ((plane*4 + w)*16 + r)*nbq + bq
 *                   (plane 0 = nonzero, 1 = sign; byte offset = 4*index)
 *     scale index = (rt*nb + 4kt)*16 + r*nbq + bq, fp16, starting at byte
 *                   align256(Np*K/4)
 *   Decoding: t = nz ? (sign ? -1 : +1) : 0.  Canonical form has sign = 0
 *   wherever nz = 0; tern_pack emits it and the int8 kernels require it.
 *   Dequantized weight: W[n][k] = t[n][k] * scale[n][k/128].
 */
#ifndef TERN_H
#define TERN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TERN_OK = 0,
    TERN_E_NULL = 1,    /* a required pointer is NULL */
    TERN_E_SHAPE = 2,   /* negative size, K % 128 != 0, M out of range */
    TERN_E_ALIGN = 3,   /* a pointer is not 16-byte aligned */
    TERN_E_HIP = 4,     /* a HIP call or kernel launch failed */
    TERN_E_DEVICE = 5   /* the current device is not gfx950 */
} tern_status;

#define TERN_ABI_VERSION 10
#define TERN_MAX_M_GEMV 16   /* activation rows per tern_gemv / tern_gemv_i8 / i8_head_gemv call */

/* Human-readable name of a tern_status value (static string). */
const char* tern_strerror(int status);

/* HIP error text of this thread's last TERN_E_HIP ("" if none). */
const char* tern_last_error(void);

/* TERN_ABI_VERSION of the loaded library. */
int tern_abi_version(void);

/* Bytes of the packed blob for an N x K ternary matrix:
 * align256(Np*K/4) + Np*(K/128)*2, Np = 16*ceil(N/16).  -1 on a bad shape. */
int64_t tern_packed_bytes(int64_t N, int64_t K);

/* Pack ternary weights (load-time work: the loader resolves backend layout
 * once at load time with values unchanged, [P2] section "하나의 파일, 네 개의
 * 백엔드"; bit-planes per block after the FV5 table of [P2]).
 *   t      int8 [N][K], values in {-1, 0, +1} (other values are taken as
 *          their sign)
 *   scale  fp16 bit patterns [N][K/128]
 *   packed output, tern_packed_bytes(N, K) bytes, 16-byte aligned; padding
 *          rows are written as zeros. */
int tern_pack(const int8_t* t, const uint16_t* scale, int64_t N, int64_t K, void* packed, void* stream);

/* Occupancy of a packed matrix (the analogue of the container walk that
 * counts zero / +1 / -1 states, [P2] section "출하된 컨테이너를 직접 읽기: 62.63%의 침묵").
 *   counts  device uint64 [3]: nonzero weights, -1 weights, non-canonical
 *           bits (sign set where nonzero is clear), over the N real rows. */
int tern_stats(const void* packed, int64_t N, int64_t K, uint64_t* counts, void* stream);

/* Per-row absmax int8 quantization of bf16 activations (an int8-activation
 * runtime is mentioned in [P2] section "토큰 동일성의 경계: 그리디, float32,
 * 그리고 두 개의 근접 동점"; the quantizer is
 * not described there, so this plain reading is used):
 *   a = max_k |x[m][k]|, s_x[m] = a / 127 (fp32, IEEE division, nearest-even),
 *   q[m][k] = clamp(rint(x[m][k] / s_x[m]), -127, 127) (fp32 quotient, ties
 *   to even); a == 0 gives s_x = 0 and q = 0.
 *   x  bf16 bits [M][K] (K % 16 == 0);  q  int8 [M][K];  s_x  fp32 [M]. */
int tern_quantize_i8(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s_x, void* stream);

/* Ternary GEMV / small-M GEMM with bf16 activations and fp32 accumulation
 * (the linear y_j = sum_i w_ij x_i of [P2] section "학습 중에 포맷이 있어야
 * 하는 이유"; add / skip / subtract of [P5] Figure I; weights decoded inside
 * the matrix kernel, [P4] opening paragraphs; up to 7 speculative positions per
 * batched forward, [P2] section "검증된 추측 디코딩: 속도만 바꾸고 답은 바꾸지
 * 않는다"):
 *   y[m][n] = sum_b scale[n][b] * sum_{k in block b} t[n][k] * x[m][k]
 *   packed  plane blob of an N x K matrix
 *   x       bf16 bits [M][K], 1 <= M <= TERN_MAX_M_GEMV
 *   y       fp32 [M][N]
 * Accuracy: fp32 accumulation; relative L2 error against the exact value is
 * ~1e-7 (any summation order).  A call may enqueue more than one kernel (more
 * than 8 activation rows whose activations fit no one-pass or two-phase
 * split run as two calls on row halves); every kernel goes to `stream`. */
int tern_gemv(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y, void* stream);

/* Ternary GEMV / small-M GEMM with int8 activations (q, s_x from
 * tern_quantize_i8 or the caller):
 *   acc[m][n][b] = sum_{k in block b} t[n][k] * q[m][k]   (exact int32)
 *   y[m][n] = s_x[m] * sum_b scale[n][b] * acc[m][n][b]  (fp32)
 *   q        int8 [M][K];  s_x fp32 [M];  1 <= M <= TERN_MAX_M_GEMV
 *   acc_dbg  NULL or int32 [M][N][K/128]: the block accumulators (debug;
 *            for small shapes). */
int tern_gemv_i8(const void* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M,
                 float* y, int32_t* acc_dbg, void* stream);

/* int8 output-head GEMV with a per-row fp32 scale and bf16 activations
 * (embedding and head stay int8, [P2] section "3진 계열이라는 이름의 실체";
 * the unembedding runs on the DRAM roofline, [P2] section "뉴트리노 엔진:
 * 토큰 하나의 시간은 어디로 가는가"):
 *   logits[m][v] = row_scale[v] * sum_k W[v][k] * x[m][k]
 *   W  int8 [V][K] (K % 128 == 0, else TERN_E_SHAPE);  row_scale fp32 [V];
 *   x bf16 bits [M][K];  logits fp32 [M][V];  1 <= M <= TERN_MAX_M_GEMV. */
int i8_head_gemv(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                 float* logits, void* stream);

/* int8 output head with int8 activations:
 *   acc[m][v] = sum_k W[v][k] * q[m][k] (exact int32),
 *   logits[m][v] = row_scale[v] * s_x[m] * acc[m][v]
 *   W int8 [V][K] (K % 128 == 0, else TERN_E_SHAPE);  q int8 [M][K];
 *   s_x fp32 [M];  acc_dbg NULL or int32 [M][V]. */
int i8_head_gemv_i8(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                    const float* s_x, int64_t M, float* logits, int32_t* acc_dbg, void* stream);

/* The int8 head over a packed copy of W, for the logits of i8_head_gemv /
 * i8_head_gemv_i8 (bit for bit those of the row-major single-pass kernel,
 * which i8_head_argmax[_i8] and, up to 48 KiB of activations, i8_head_gemv
 * run: every lane multiplies the same weights in the same order; the same
 * accuracy otherwise) at a higher read rate: the head is the
 * largest tensor of a decode step and runs on the DRAM roofline ([P2]
 * section "뉴트리노 엔진: 토큰 하나의 시간은 어디로 가는가").
 *
 * i8_head_packed_bytes: bytes of the packed copy, ceil(V/64)*64*K, or -1
 * when 1 <= V <= 0xFFFFFFF0 and 128 <= K <= 2^20 with K % 128 == 0 fail.
 *
 * i8_head_pack: W int8 [V][K] row-major -> packed (caller-allocated, 16-byte
 * aligned, i8_head_packed_bytes long).  Layout: row groups of 64 (rows past V
 * are zero); within a group, for each 128-k unit j, for each 16-row tile w of
 * the group, 2048 bytes: at 16*l (l = r + 16*g, r < 16, g < 4) bytes
 * 128j + 16g .. +15 of row 16w + r, at 1024 + 16*l bytes 128j + 64 + 16g ..
 * +15.  Byte-exact; the packed copy is read-only afterwards and owned by the
 * caller.
 *
 * i8_head_gemv_packed / i8_head_gemv_packed_i8: as i8_head_gemv /
 * i8_head_gemv_i8 with W replaced by its packed copy; 1 <= M <=
 * TERN_MAX_M_GEMV and the activations of all M rows must fit one CU's LDS
 * (M*(2K+16) bytes for bf16, M*(K+16) for int8, at most 160 KiB), else
 * TERN_E_SHAPE; the same shape errors as i8_head_packed_bytes. */
int64_t i8_head_packed_bytes(int64_t V, int64_t K);
int i8_head_pack(const int8_t* W, int64_t V, int64_t K, int8_t* packed, void* stream);
int i8_head_gemv_packed(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const uint16_t* x,
                        int64_t M, float* logits, void* stream);
int i8_head_gemv_packed_i8(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                           const float* s_x, int64_t M, float* logits, int32_t* acc_dbg, void* stream);

/* Greedy decode on the output head: the int8 head GEMV fused with an argmax
 * over the vocabulary (token identity is decided greedily on float32 logits,
 * [P2] section "토큰 동일성의 경계: 그리디, float32, 그리고 두 개의 근접
 * 동점", which also documents near ties; the unembedding is the largest
 * tensor of the step, section "뉴트리노 엔진: 토큰 하나의 시간은 어디로
 * 가는가").  For each activation row m:
 *   idx[m] = the v with the largest logits[m][v], the lowest such v among
 *            equal values (-0 counts as +0);  val[m] = that logit.
 * logits are those of i8_head_gemv (bf16 x) or i8_head_gemv_i8 (int8 q, s_x:
 * logits[m][v] = (row_scale[v] * s_x[m]) * acc[m][v], rounded to fp32 in
 * that order); logits must be finite.
 *   W int8 [V][K] (K % 128 == 0, 1 <= V < 2^32 - 16);  x bf16 bits / q int8
 *   [M][K] with M*(2K+16) (bf16) or M*(K+16) (int8) <= 163840 bytes;
 *   1 <= M <= TERN_MAX_M_GEMV;  idx int32 [M];  val fp32 [M];
 *   logits NULL or fp32 [M][V] (written when given);
 *   workspace: i8_head_argmax_workspace_bytes(V, M) bytes of device memory
 *   (8 bytes per 16 rows of W and activation row), 8-byte aligned, owned by
 *   the caller; the call overwrites it, so calls that share a workspace must
 *   not overlap in time.  Two kernels run: the head, whose waves leave one
 *   key per 16 rows, and a reduction over those keys.
 * Errors: TERN_E_SHAPE for a shape outside these limits, TERN_E_NULL /
 * TERN_E_ALIGN for pointers; nothing is launched then. */
int64_t i8_head_argmax_workspace_bytes(int64_t V, int64_t M);
int i8_head_argmax(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                   int32_t* idx, float* val, float* logits, void* workspace, void* stream);
int i8_head_argmax_i8(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                      const float* s_x, int64_t M, int32_t* idx, float* val, float* logits, void* workspace,
                      void* stream);

/* i8_head_argmax / i8_head_argmax_i8 over the packed copy of W written by
 * i8_head_pack (same arguments with W replaced by it, same limits, errors
 * and workspace): idx, val and logits bit for bit those of the row-major
 * calls; the copy's padding rows (V up to a multiple of 64) are never
 * candidates.  The head is the largest tensor of the step ([P2] section
 * "뉴트리노 엔진: 토큰 하나의 시간은 어디로 가는가"); the packed copy is
 * read at a higher rate. */
int i8_head_argmax_packed(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const uint16_t* x,
                          int64_t M, int32_t* idx, float* val, float* logits, void* workspace, void* stream);
int i8_head_argmax_packed_i8(const int8_t* packed, const float* row_scale, int64_t V, int64_t K, const int8_t* q,
                             const float* s_x, int64_t M, int32_t* idx, float* val, float* logits, void* workspace,
                             void* stream);

/* i8_head_argmax without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same inputs, outputs, limits and result
 * as i8_head_argmax (bf16 x); the argmax keys live in a device array the
 * library owns, 2 MiB per device (held until the process ends):
 * i8_head_argmax_workspace_bytes(V, M) must not exceed 2097152 bytes, i.e.
 * ceil(V/16) * M <= 262144 (V = 151936 allows every M up to
 * TERN_MAX_M_GEMV), else TERN_E_SHAPE and nothing is launched.  Nothing is
 * allocated or freed.  Every call on a device shares that array: calls that
 * overlap in time on one device (other streams, other threads) race and
 * must be ordered by the caller. */
int i8_head_argmax_noalloc(const int8_t* W, const float* row_scale, int64_t V, int64_t K, const uint16_t* x,
                           int64_t M, int32_t* idx, float* val, float* logits, void* stream);

/* Prefill-size ternary GEMM with int8 activations (batched prefill, [P2]
 * section "실행해보기: pip부터 llama.cpp 포크까지"; batched verify is
 * compute-bound, section "노트북에서는 이야기가 다르다"),
 * same arithmetic as tern_gemv_i8 for any M >= 1, with kernels of its own
 * from M = 17: planes are decoded to int8 and fed to the int8 matrix cores.
 * Outside 17 <= M <= 64 and below M = 128, where the contraction's time is
 * set by its per-block latency, the call may run the int8 GEMV on 16-row
 * slices of q instead (chosen on the host from the shape); the result is the
 * same contraction (fp32 y may differ in the last bits with the kernel: the
 * block sums are added in a kernel-specific order).  The workgroup-shared
 * decode kernel runs from M = 128, and at 65 <= M < 128 where a measured model
 * puts it ahead of the other two (see tern_prefill_config).  When its output
 * tiles leave most CUs idle and K >= 4096, K is split in two halves:
 * the call then enqueues three kernels (y cleared, the two halves' unscaled
 * fp32 partials added with atomics, rows scaled by s_x), so y is
 * fl(s_x * fl(a + b)) and the same on every run.
 *   q int8 [M][K]; s_x fp32 [M]; y fp32 [M][N];
 *   acc_dbg NULL or int32 [M][N][K/128] (debug; small shapes). */
int tern_gemm_prefill(const void* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M,
                      float* y, int32_t* acc_dbg, void* stream);

/* ---- GEMV chain (single-stream decode in one launch) ----
 *
 * A token runs its linears one after another, each reading an activation
 * that the previous ones produced; per token the time above the pure DRAM
 * bound sits at the roughly one hundred kernel boundaries and in the
 * dependency chain inside each small kernel ([P2] section "뉴트리노 엔진:
 * 토큰 하나의 시간은 어디로 가는가").  tern_gemv_chain runs a whole chain
 * of M = 1 ternary GEMVs in one persistent launch: each step waits only for
 * the activations it reads, and later steps' weights stream in meanwhile.
 *
 * Step p computes, with the arithmetic of tern_gemv at M = 1:
 *   y[n] = sum_b scale[n][b] * sum_{k in block b} t[n][k] * x[k]
 * where x is either the step's own input vector, or (x_from = q, an earlier
 * step with N_q >= K) the first K outputs of step q rounded to bf16
 * (nearest-even); the rounded copy travels through the workspace, y_q itself
 * is the fp32 result.  Steps without such a link may run concurrently, so no
 * y may overlap another y, an input vector or a packed blob of the chain. */
typedef struct tern_chain_step {
    const void* packed;   /* tern_pack blob of W [N][K], 16-byte aligned              */
    int64_t N;            /* output rows, >= 1                                         */
    int64_t K;            /* input features, 512 <= K <= 16384, K % 512 == 0           */
    const uint16_t* x;    /* bf16 bits [K], 16-byte aligned; unused when x_from >= 0  */
    int64_t x_from;       /* -1, or the earlier step whose output is x                 */
    float* y;             /* fp32 [N], 4-byte aligned                                  */
} tern_chain_step;

/* Workspace bytes for this chain, or -1 if nsteps is outside [0, 4095], steps
 * is NULL or an x_from does not name an earlier step.  The workspace holds the
 * plan and the rounded copies of the outputs that later steps read.  The
 * caller allocates it (256-byte aligned), fills it with zeros once before its
 * first use and then leaves it to the library; it may be re-planned (with a
 * chain that fits) and run any number of times.  Runs that share a workspace
 * must not overlap in time.  A 32-bit count of aborted waits sits at byte
 * offset 8 (0 in normal operation; a workspace with a nonzero count runs
 * nothing until it is zero-filled again). */
int64_t tern_chain_workspace_bytes(const tern_chain_step* steps, int64_t nsteps);

/* Validate nsteps host-side step descriptors and enqueue the write of their
 * device plan into the workspace.  Errors: TERN_E_NULL / TERN_E_ALIGN /
 * TERN_E_SHAPE for a bad step or link, overlapping outputs, a workspace
 * smaller than tern_chain_workspace_bytes, or a step with more than 256 (row
 * tile, 512-k tile) units per CU.  The steps array is read before the call
 * returns. */
int tern_chain_plan(const tern_chain_step* steps, int64_t nsteps, void* workspace, int64_t workspace_bytes,
                    void* stream);

/* Run the first nsteps steps of the plan in the workspace (no more than were
 * planned).  One workgroup per CU stays resident for the whole launch
 * (cooperative launch); the call fails with TERN_E_HIP if the device cannot
 * hold them.  Every wait inside is bounded (a stalled run ends after seconds
 * and counts an error, see tern_chain_workspace_bytes). */
int tern_gemv_chain(void* workspace, int64_t nsteps, void* stream);

/* ---- five-level weights (FV5-style) ----
 *
 * The GGUF pack of the pages stores every attention and MLP linear as FV5:
 * blocks of 256 weights with two f32 scales (s_lo, s_hi) and three 32-byte
 * bit-planes, 3.25 bits per weight ([P2] section "FV5와 FV5B", the block
 * table); the page reads the planes as sign, zero and two magnitude steps.
 * This library takes that reading as five levels l in {-2, -1, 0, +1, +2}:
 *   W[n][k] = sign(l) * (|l| == 2 ? s_hi[n][b] : s_lo[n][b]),  b = k/256,
 * and W = 0 where l = 0.  Its bit layout ("five-level blob") is its own:
 *   K % 512 == 0; rows padded to Np = 16*ceil(N/16); planes p = 0 nonzero
 *   (l != 0), 1 sign (l < 0), 2 high (|l| == 2), each 256 bits of a block
 *   as eight little-endian 32-bit words, word w holding weights
 *   k = 256b + 32w + i with weight i at bit 16*(i&1) + (i>>1).  With
 *   rt = n/16, r = n%16, kt = b/2, bh = b%2, nkt = K/512, g = w%4,
 *   j = 2*bh + w/4:
 *     word index = ((rt*nkt + kt)*3 + p)*256 + (g*16 + r)*4 + j
 *     (byte offset = 4*index; Np*K*3/8 bytes of planes)
 *   then f32 scales from byte Np*K*3/8: s_lo of (n, b) at element
 *   ((rt*nkt + kt)*16 + r)*4 + 2*bh, s_hi at the next element.
 *   Canonical form: sign = high = 0 wherever nonzero = 0 (tern5_pack emits
 *   it; the GEMV reads a high or sign bit only where nonzero is set). */

/* Bytes of the five-level blob of W[N][K]: Np*K*3/8 + Np*(K/256)*8, or -1
 * for N < 0, K < 0 or K % 512 != 0. */
int64_t tern5_packed_bytes(int64_t N, int64_t K);

/* Pack levels int8 [N][K] (values in [-2, 2]; others are clamped to that
 * range) and f32 scales s_lo, s_hi [N][K/256] into a blob of
 * tern5_packed_bytes(N, K) bytes (every byte written, padding rows as zeros).
 * levels and packed 16-byte aligned, scales 4-byte aligned. */
int tern5_pack(const int8_t* levels, const float* s_lo, const float* s_hi, int64_t N, int64_t K, void* packed,
               void* stream);

/* y[m][n] = sum_k W[n][k] * x[m][k] for the five-level W, fp32 accumulation
 * on the matrix cores (bf16 x times 2*sign(l) exactly, the two scales of a
 * block applied once to their fp32 sums).
 *   packed  tern5_pack blob of W[N][K], K % 512 == 0
 *   x       bf16 bits [M][K], 1 <= M <= TERN_MAX_M_GEMV, 16-byte aligned
 *   y       fp32 [M][N], 4-byte aligned */
int tern5_gemv(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y, void* stream);

/* int8 activations (tern_quantize_i8 output) for the five-level W:
 *   acc[m][n][b][0] = sum_{k in block b, |l| = 1} sign(l) * q[m][k],
 *   acc[m][n][b][1] = the same over |l| = 2 (exact int32, 256-weight blocks),
 *   y[m][n] = s_x[m] * sum_b (s_lo[n][b] * acc[..][0] + s_hi[n][b] * acc[..][1])
 * with the block sums scaled in fp32.
 *   q int8 [M][K] (16-byte aligned), s_x fp32 [M], 1 <= M <= TERN_MAX_M_GEMV;
 *   y fp32 [M][N];  acc_dbg NULL or int32 [M][N][K/256][2] (debug). */
int tern5_gemv_i8(const void* packed, int64_t N, int64_t K, const int8_t* q, const float* s_x, int64_t M, float* y,
                  int32_t* acc_dbg, void* stream);

/* ---- block-scaled int8 tensors (FV5B-style) ----
 *
 * The GGUF pack of the pages stores the token embedding and the output head
 * as FV5B: blocks of 256 int8 weights with one f32 scale, 8.125 bits per
 * weight ([P2] section "FV5와 FV5B", the block table); embedding and head
 * stay int8 ([P2] section "3진 계열이라는 이름의 실체").  Storage here:
 * W int8 [V][K] row-major (16-byte aligned) and S f32 [V][K/256]; the
 * weight is W[v][k] * S[v][k/256].  The head calls stage all of x in LDS:
 * they need K % 256 == 0, 1 <= M <= TERN_MAX_M_GEMV and M*(K*e + 16) <=
 * 160 KiB (e = 2 for bf16 x, 1 for int8 q), else TERN_E_SHAPE; V <= 2^32-16. */

/* logits[m][v] = sum_b S[v][b] * sum_{k in block b} W[v][k] * x[m][k], each
 * block's sum in fp32 on the matrix cores, folded into the row total in
 * block order.  x bf16 bits [M][K]; logits fp32 [M][V]. */
int fv5b_head_gemv(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                   float* logits, void* stream);

/* int8 activations: acc[m][v][b] = sum_{k in block b} W[v][k] * q[m][k]
 * (exact int32), logits[m][v] = s_x[m] * sum_b S[v][b] * acc[m][v][b] (fp32).
 * acc_dbg NULL or int32 [M][V][K/256]. */
int fv5b_head_gemv_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q, const float* s_x,
                      int64_t M, float* logits, int32_t* acc_dbg, void* stream);

/* The block-scaled head fused with greedy argmax, as i8_head_argmax: idx /
 * val of the largest logit per activation row (lowest v among equal
 * logits, -0 as +0); logits optional; the workspace is the one
 * i8_head_argmax_workspace_bytes(V, M) sizes (8-byte aligned). */
int fv5b_head_argmax(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                     int32_t* idx, float* val, float* logits, void* workspace, void* stream);
int fv5b_head_argmax_i8(const int8_t* W, const float* S, int64_t V, int64_t K, const int8_t* q, const float* s_x,
                        int64_t M, int32_t* idx, float* val, float* logits, void* workspace, void* stream);

/* The block-scaled head calls above over the packed copy of W's int8 rows
 * (i8_head_pack; the scales S stay [V][K/256] row-major): same arguments
 * with W replaced by the copy, same limits and errors, results bit for bit
 * those of the row-major calls; the copy's padding rows are never argmax
 * candidates.  The head is the step's largest tensor ([P2] section
 * "뉴트리노 엔진: 토큰 하나의 시간은 어디로 가는가"); the copy is read at a
 * higher rate. */
int fv5b_head_gemv_packed(const int8_t* packed, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                          float* logits, void* stream);
int fv5b_head_gemv_packed_i8(const int8_t* packed, const float* S, int64_t V, int64_t K, const int8_t* q,
                             const float* s_x, int64_t M, float* logits, int32_t* acc_dbg, void* stream);
int fv5b_head_argmax_packed(const int8_t* packed, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                            int32_t* idx, float* val, float* logits, void* workspace, void* stream);
int fv5b_head_argmax_packed_i8(const int8_t* packed, const float* S, int64_t V, int64_t K, const int8_t* q,
                               const float* s_x, int64_t M, int32_t* idx, float* val, float* logits, void* workspace,
                               void* stream);

/* The end of one decode token and the start of the next in one call:
 * fv5b_head_argmax (bf16 x), then the embedding row of each chosen index
 * idx[m] from the block-scaled table E int8 [Ve][Ke] with scales ES f32
 * [Ve][Ke/256], written as fv5b_embed writes it (emb fp32 [M][Ke], emb_bf16
 * [M][Ke]; either may be NULL, not both; an index outside [0, Ve) gives a
 * zero row).  The gather runs inside the argmax's final kernel, so the index
 * never travels through memory first.  Ke % 256 == 0; E, emb and emb_bf16
 * 16-byte aligned. */
int fv5b_head_argmax_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const uint16_t* x, int64_t M,
                           int32_t* idx, float* val, float* logits, void* workspace, const int8_t* E, const float* ES,
                           int64_t Ve, int64_t Ke, float* emb, uint16_t* emb_bf16, void* stream);

/* Embedding rows for M token ids (the step before the first linear):
 *   out[m][k] = W[ids[m]][k] * S[ids[m]][k/256], one fp32 rounding;
 *   out_bf16[m][k] = that value rounded to bf16, nearest-even (the
 *   activation format of tern_gemv).
 * ids int32 [M]; an id outside [0, V) gives a zero row (W is not read).
 * out fp32 [M][K] and out_bf16 [M][K]: either may be NULL, not both; both
 * 16-byte aligned.  K % 256 == 0; M >= 0 (M == 0 or K == 0: nothing). */
int fv5b_embed(const int8_t* W, const float* S, int64_t V, int64_t K, const int32_t* ids, int64_t M, float* out,
               uint16_t* out_bf16, void* stream);

/* ---- launch-configuration introspection (no operation of the method) ----
 *
 * The one-pass GEMV configuration that tern_gemv (kind 0), tern_gemv_i8 (1),
 * tern5_gemv (2) or tern5_gemv_i8 (3) takes for this shape, or the two-phase
 * configuration that tern_gemv / tern_gemv_i8 (kinds 4 and 5) or tern5_gemv /
 * tern5_gemv_i8 (6 and 7) take when no one-pass one fits (activations staged
 * in LDS one half of K at a time), or the three-phase configuration that
 * tern_gemv takes when neither fits (kind 8: a third of K at a time),
 * computed on the host exactly as the launchers do (the CU count is the current device's, or
 * 256 without one; the launchers also confirm residency with the occupancy
 * query).  Returns 1 and fills out[8] = {row tiles per workgroup R, waves per
 * workgroup, 512-k units per wave U, activation chunks per thread (1 where
 * every wave stages only its own units' activation slices: kind 0 at M = 1,
 * and at M <= 8 with R = 1 and U <= 2), grid, dynamic LDS bytes, runs in
 * several rounds (0/1), MFMA activation rows of the kernel instance}; 0 when
 * another kernel takes the shape; -TERN_E_NULL or
 * -TERN_E_SHAPE for a NULL out or a shape outside 1 <= M <= TERN_MAX_M_GEMV,
 * N, K >= 1, kind 0..8.  Touches no device memory. */
int tern_gemv_config(int64_t N, int64_t K, int64_t M, int kind, int64_t* out);

/* The launch of tern_gemm_prefill's workgroup-shared-decode kernel (K % 512 == 0,
 * from M = 128 and, where a measured model favours it, at 65 <= M < 128),
 * computed on the host exactly as the launcher does (CU count
 * of the current device, or 256 without one): returns 1 and fills out[6] =
 * {workgroup rows of M (256 or 128), workgroup rows of N (128 or 64), K split in
 * two halves (0/1; three kernels then), grid x (tiles over N), grid y (tiles over
 * M), grid z (2 when split, else 1)}; 0 when another kernel takes the shape;
 * -TERN_E_NULL for a NULL out, -TERN_E_SHAPE for N, K or M below 1 or
 * K % 128 != 0.  Touches no device memory. */
int tern_prefill_config(int64_t N, int64_t K, int64_t M, int64_t* out);

/* ---- matrix-core throughput probe (a measurement aid; no operation of the method) ----
 *
 * The contraction of tern_gemm_prefill runs on the int8 matrix cores and the
 * GEMVs on the bf16 ones; their throughput targets are fractions of the
 * chip's dense matrix-core peak.  This probe measures what the chip
 * sustains: `grid` workgroups of 4 waves, each wave running 8 independent
 * chains of `iters` MFMAs on registers (no memory traffic in the loop).
 *   kind 0: v_mfma_i32_16x16x64_i8 (2*16*16*64 operations each)
 *   kind 1: v_mfma_f32_16x16x32_bf16 (2*16*16*32 operations each)
 * tern_mfma_peak_ops gives the operations one launch executes (-1 for a bad
 * argument); the caller times the launch.  sink: device memory of
 * tern_mfma_peak_sink_bytes(grid) bytes, 16-byte aligned, overwritten with
 * the final accumulators (so no MFMA is optimised away).
 * Errors: TERN_E_SHAPE for kind outside {0, 1}, iters < 0 or grid outside
 * [1, 2^31 - 1]; TERN_E_NULL / TERN_E_ALIGN for sink. */
double tern_mfma_peak_ops(int kind, int64_t iters, int64_t grid);
int64_t tern_mfma_peak_sink_bytes(int64_t grid);
int tern_mfma_peak(int kind, int64_t iters, int64_t grid, int32_t* sink, void* stream);

/* ---- launch floor and read ceiling probe (a measurement aid; no operation of the method) ----
 *
 * A GEMV launch at M = 1 costs about what a launch that does almost nothing
 * costs, plus its bytes at the rate a plain streaming read reaches.  This
 * probe enqueues one launch of:
 *   kind 0: an empty kernel (`grid` workgroups of 64 threads);
 *   kind 1: `grid` workgroups of 512 threads, each storing one float of sink;
 *   kind 2: as kind 1, every thread first loading 16 bytes of src (thread i
 *           reads bytes [16i, 16i + 16), clamped to the last 16 bytes);
 *   kind 3: `grid` workgroups of 256 threads reading all src_bytes of src once
 *           (16-byte loads, eight in flight per thread).
 * The caller times the launches (in a graph, one after another, for the
 * floor; one large src for the read rate).  sink: device memory of at least
 * `grid` floats (kinds 1-3; kind 3 writes it only if the bytes it read XOR
 * to 0x9E3779B9, so pass zero-filled src); src: device memory, 16-byte
 * aligned, src_bytes a positive multiple of 16 (kinds 2 and 3).
 * Errors: TERN_E_SHAPE for kind outside [0, 3], grid outside [1, 2^31 - 1]
 * or a bad src_bytes; TERN_E_NULL / TERN_E_ALIGN for sink and src. */
int tern_launch_probe(int kind, int64_t grid, const void* src, int64_t src_bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TERN_H */
