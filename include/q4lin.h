/*
 * q4lin.h -- C ABI of the Q4_G64_FP16 weight-only Linear for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation ("q4-linear.md", setup table; "linear-benchmark.md", section 0,
 * the public call linear(x, w, out, policy, workspace, stream)):
 *
 *     Y[N,T] = W[N,K] x X[K,T]
 *
 *   W   Q4_G64_FP16: every 64 consecutive weights of a row share one FP16
 *       scale; a weight is (q - 8) * scale with q a 4-bit code in 0..15
 *       ("linear-benchmark.md", section 4 table: 32 code bytes + 2 scale
 *       bytes = 34 bytes per group).
 *   X   bfloat16 activations, Y bfloat16 outputs; products are summed in
 *       binary32 and Y is rounded to nearest even ("q4-linear.md", setup
 *       table: BF16 input and output; the note under the metric definitions:
 *       BF16 inputs with FP32 accumulation).  Only the A16 policy exists, so
 *       the call carries no policy argument.
 *
 * Memory layout (all buffers are device memory owned by the caller):
 *   codes   uint8  [N][K/2], row-major.  Byte j of a row holds the code of
 *           k = 2j in its low nibble and of k = 2j+1 in its high nibble.
 *           16-byte aligned.
 *   scales  fp16   [N][K/64], row-major (IEEE binary16 bit patterns); scale g
 *           of a row covers k in [64g, 64g+64).  2-byte aligned.
 *   x       bf16   token-major [T][K]: element (k, t) at x[t*K + k].
 *           16-byte aligned.
 *   y       bf16   token-major [T][N]: element (n, t) at y[t*N + n].
 *           2-byte aligned.  Fully overwritten; nothing outside it is written.
 *   workspace  device scratch of at least q4lin_workspace_bytes(N, K, T)
 *           bytes, 256-byte aligned; contents on entry are ignored and are not
 *           preserved.  May be NULL when that size is 0.
 *
 * Shapes: N >= 0, T >= 0, K a positive multiple of 64.  N == 0 or T == 0 is an
 * empty product: the call returns Q4LIN_OK and touches no memory (pointers may
 * then be NULL).  The largest accepted values are N <= 2^24, T <= 2^21 and
 * K <= 2^20, with every buffer under 2^40 bytes.
 *
 * Behaviour: the call only validates its arguments on the host and enqueues
 * one or more kernels on `stream` (a hipStream_t; NULL is the null stream).  It
 * never allocates, frees or synchronizes, keeps no pointer after it returns,
 * and keeps no state between calls (the library's only process-wide records
 * are set once per kernel and device -- the dynamic-LDS limit -- and, for
 * q4lin_linear_noalloc, the scratch array's address per device, both behind
 * a lock), so it is thread-safe and may be captured in a HIP graph.  x,
 * codes and scales are only read.  Every argument error is reported before
 * anything is enqueued, leaving y untouched.  Calls that share a workspace
 * must not overlap in time.
 */
#ifndef Q4LIN_H
#define Q4LIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef Q4LIN_API
#define Q4LIN_API __attribute__((visibility("default")))
#endif

/* Status codes. */
#define Q4LIN_OK 0
#define Q4LIN_E_NULL 1      /* a required pointer is NULL                         */
#define Q4LIN_E_SHAPE 2     /* N, K or T out of contract (K % 64 != 0, sizes...)  */
#define Q4LIN_E_ALIGN 3     /* a pointer is not aligned as stated above           */
#define Q4LIN_E_WORKSPACE 4 /* workspace smaller than q4lin_workspace_bytes()     */
#define Q4LIN_E_LAUNCH 5    /* the HIP runtime refused a kernel launch (e.g. the
                               current device is not a gfx950 GPU)               */
#define Q4LIN_E_FORMAT 6    /* unknown weight format (q4lin_linear_fmt)          */

/* Bytes of workspace q4lin_linear needs for this shape (0 when none), or a
 * negative status (-Q4LIN_E_SHAPE) for a shape outside the contract.  Pure
 * host function; the pages ask for a public capacity query answered before
 * any timed call ("linear-benchmark.md", section 1.1). */
Q4LIN_API int64_t q4lin_workspace_bytes(int64_t n, int64_t k, int64_t t);

/* Y = W x X as described above.  Returns Q4LIN_OK or a status code. */
Q4LIN_API int q4lin_linear(const void *x, const void *codes, const void *scales, void *y,
                 int64_t n, int64_t k, int64_t t,
                 void *workspace, size_t workspace_bytes, void *stream);

/* LinearAdd, the pages' fused Linear variant with a residual ("q4-linear.md"
 * and "linear-benchmark.md" name LinearAdd beside LinearSwiGLU and LinearPair
 * without defining it; the plain reading taken here):
 *
 *     Y[N,T] = W[N,K] x X[K,T] + R[N,T]
 *
 * with the residual R in bfloat16, token-major like Y (element (n, t) at
 * residual[t*N + n]), 2-byte aligned.  R joins the binary32 result before
 * its single rounding to bfloat16, so the sum is rounded once (not the
 * product first).  residual may be the same buffer as y (in place, element
 * for element); any other overlap with y is outside the contract.  Every
 * other argument, the workspace size (q4lin_workspace_bytes), the routes and
 * the errors are those of q4lin_linear; residual NULL with a non-empty
 * product is Q4LIN_E_NULL. */
Q4LIN_API int q4lin_linear_add(const void *x, const void *codes, const void *scales, const void *residual,
                     void *y, int64_t n, int64_t k, int64_t t,
                     void *workspace, size_t workspace_bytes, void *stream);

/* LinearPair, the third fused Linear variant the pages name beside LinearAdd
 * and LinearSwiGLU ("q4-linear.md" and "linear-benchmark.md", without a
 * definition; the plain reading taken here): two weights of the same K over
 * one activation X, two outputs,
 *
 *     Y1[N1,T] = W1[N1,K] x X[K,T]      Y2[N2,T] = W2[N2,K] x X[K,T]
 *
 * each element equal to what q4lin_linear gives for that weight alone.  Each
 * (codes, scales, y) triple follows q4lin_linear's layout and alignment with
 * its own row count.  Up to 128 tokens the route chosen for N1 + N2 rows runs
 * both weights in a single launch, the second weight's rows as further row
 * blocks; beyond that the many-token route runs both weights' tiles in one
 * launch after one activation preparation; the wide-K routes run one launch
 * sequence per weight, one after the other on `stream`.  workspace
 * must hold q4lin_pair_workspace_bytes(n1, n2, k, t) bytes.  N1 or N2 = 0
 * reduces to q4lin_linear on the other weight (whose pointers alone are then
 * checked).  y1 and y2 must not overlap each other or any input. */
Q4LIN_API int q4lin_linear_pair(const void *x, const void *codes1, const void *scales1, void *y1, int64_t n1,
                      const void *codes2, const void *scales2, void *y2, int64_t n2, int64_t k, int64_t t,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace q4lin_linear_pair needs (0 when none), or
 * -Q4LIN_E_SHAPE for a shape outside the contract.  Pure host function. */
Q4LIN_API int64_t q4lin_pair_workspace_bytes(int64_t n1, int64_t n2, int64_t k, int64_t t);

/* LinearSwiGLU, the gate/up variant the pages name beside LinearAdd and
 * LinearPair ("q4-linear.md" and "linear-benchmark.md", without a
 * definition; the plain reading taken here, the gated linear unit with the
 * SiLU gate):
 *
 *     Y[N,T] = silu(Wg[N,K] x X[K,T]) * (Wu[N,K] x X[K,T]),  silu(g) = g / (1 + e^-g)
 *
 * elementwise, both products taken as unrounded sums (binary32 on the GPU,
 * never bf16), the gate formed in binary64 and the result rounded once to
 * bfloat16.  The gate weight (codes_gate, scales_gate) and the up weight
 * (codes_up, scales_up) both have N rows and q4lin_linear's layout and
 * alignment; y is bf16 [T][N] like q4lin_linear's.  workspace must hold
 * q4lin_swiglu_workspace_bytes(n, k, t) bytes, 256-byte aligned: 0 where one
 * pass takes the same rows of both weights and applies the gate before its
 * store (1 to 128 tokens, where the rows' scales fit the kernel's tables);
 * from 129 tokens, where the 2N-row problem takes the many-token route's
 * 96 x 256 tiles without a K split, one tiled launch whose tiles take 48
 * rows of each weight applies the gate in its epilogue and the workspace
 * holds only the activation preparation (q4lin_workspace_bytes' layout with
 * both weights' row exponents); else room for the two binary32 sums (or the
 * many-token route's activation copy and partials) and a combine pass.  y
 * must not overlap any input or the workspace.  Errors as for
 * q4lin_linear. */
Q4LIN_API int q4lin_linear_swiglu(const void *x, const void *codes_gate, const void *scales_gate,
                      const void *codes_up, const void *scales_up, void *y, int64_t n, int64_t k, int64_t t,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace q4lin_linear_swiglu needs (0 for an empty product), or
 * -Q4LIN_E_SHAPE for a shape outside the contract.  Pure host function. */
Q4LIN_API int64_t q4lin_swiglu_workspace_bytes(int64_t n, int64_t k, int64_t t);

/* The op without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Y = W x X with every argument, layout, route and
 * error of q4lin_linear; where the route needs scratch memory it uses a
 * static array inside the library instead of a caller's workspace.  Each GPU
 * the library runs on holds its own copy of that array
 * (q4lin_noalloc_scratch_bytes() bytes) from the first call that needs it
 * until the process ends; the call looks up its address once per device
 * (with that device current) and never calls hipMalloc, hipFree or any
 * allocating routine.  A shape whose route needs more scratch than the array
 * holds returns Q4LIN_E_WORKSPACE before anything is enqueued.  Every call on
 * one GPU shares that GPU's array and leaves its contents behind (the kernels
 * write every scratch byte they later read, so nothing needs clearing): calls
 * that overlap in time on one GPU -- on different streams, or from different
 * threads -- race on it and must be serialized by the caller. */
Q4LIN_API int q4lin_linear_noalloc(const void *x, const void *codes, const void *scales, void *y,
                 int64_t n, int64_t k, int64_t t, void *stream);

/* Size in bytes of the static scratch array q4lin_linear_noalloc uses
 * (64 MiB): the largest q4lin_workspace_bytes() it accepts.  Pure host
 * function. */
Q4LIN_API int64_t q4lin_noalloc_scratch_bytes(void);

/* The other weight formats of the same A16 Linear ("linear-benchmark.md",
 * section 0: the Q4/Q5/Q6/W8 and BF16_CTRL formats use the A16 routes, and
 * NVFP4 supports A16; section 4, weight-format table: bytes per group).  The
 * table gives only byte counts; the packing read here is the plainest one
 * that matches them:
 *
 *   Q4LIN_FMT_Q4G64_F16S  q4lin_linear's weight (w = codes, w_hi unused).
 *   Q4LIN_FMT_Q5G64_F16S  w: uint8 [N][K/2] low nibbles as Q4 (even k in the
 *           low nibble); w_hi: uint8 [N][K/8], bit i of byte b is the high
 *           bit of k = 8b + i; scales: fp16 [N][K/64].  q = low | high << 4
 *           in 0..31, weight (q - 16) * scale.  42 bytes per 64 weights.
 *   Q4LIN_FMT_Q6G64_F16S  w as Q5; w_hi: uint8 [N][K/4], bits 2i and 2i+1 of
 *           byte b are the high pair of k = 4b + i; scales fp16 [N][K/64];
 *           q in 0..63, weight (q - 32) * scale.  50 bytes per 64 weights.
 *   Q4LIN_FMT_W8G32_F16S  w: int8 [N][K] (two's complement); scales: fp16
 *           [N][K/32]; weight c * scale.  34 bytes per 32 weights.
 *   Q4LIN_FMT_NVFP4  w: uint8 [N][K/2] of E2M1 codes (even k in the low
 *           nibble); scales: uint8 [N][K/16] of E4M3 values (bias 7, no
 *           infinities); weight E2M1 * E4M3.  9 bytes per 16 weights.  The
 *           A4 policy (activations quantized to FP4 in the call) is not
 *           offered.
 *   Q4LIN_FMT_BF16  w: bf16 [N][K], the weights themselves (BF16_CTRL, the
 *           dense control of the pages' bench); w_hi and scales unused.
 *
 * Alignment: x and w 16 bytes, y 2, w_hi 4 (Q5) or 8 (Q6), scales 2 (NVFP4
 * included).  x and y as for q4lin_linear.  The sum is taken in binary32 and
 * rounded once to bf16 (an output whose binary32 sums leave the range is
 * formed again in binary64).
 * Routes: Q4 as q4lin_linear; the others stream their weight once per
 * 128 tokens (64 where a block of rows needs three or four 16-row column
 * tiles) on one workgroup per block of rows with K split across its waves
 * (matrix cores on exact bf16 code values, the scale applied per group in
 * binary32); at one token with K up to 8192 a streaming GEMV (whole rows per
 * wave, bf16 dot products on the same exact values); no workspace (NULL and
 * 0 are accepted).  Errors as for
 * q4lin_linear, plus Q4LIN_E_FORMAT for an unknown format. */
#define Q4LIN_FMT_Q4G64_F16S 0
#define Q4LIN_FMT_Q5G64_F16S 1
#define Q4LIN_FMT_Q6G64_F16S 2
#define Q4LIN_FMT_W8G32_F16S 3
#define Q4LIN_FMT_NVFP4 4
#define Q4LIN_FMT_BF16 5
Q4LIN_API int q4lin_linear_fmt(int fmt, const void *x, const void *w, const void *w_hi, const void *scales,
                 void *y, int64_t n, int64_t k, int64_t t,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Weight bytes of an N x K matrix in format fmt, the pages' closed forms
 * ("linear-benchmark.md", section 4: groups * bytes per group; 2 N K for
 * BF16), or a negative status.  Pure host function. */
Q4LIN_API int64_t q4lin_fmt_weight_bytes(int fmt, int64_t n, int64_t k);

/* Workspace bytes q4lin_linear_fmt needs (q4lin_workspace_bytes for Q4, 0
 * for the others), or a negative status.  Pure host function. */
Q4LIN_API int64_t q4lin_fmt_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t t);

/* Static, human-readable text for a status code (never NULL). */
Q4LIN_API const char *q4lin_status_string(int status);

/* Introspection for tests and reports: the kernel route the host dispatch
 * picks for this shape (one of the Q4LIN_ROUTE_* values), or a negative status
 * for a shape outside the contract.  The product call never needs it. */
#define Q4LIN_ROUTE_NONE 0   /* empty product, nothing launched */
#define Q4LIN_ROUTE_GEMV 1   /* few tokens: vector-ALU dot products            */
#define Q4LIN_ROUTE_SKINNY 2 /* small T: W streamed once, matrix cores, K split */
#define Q4LIN_ROUTE_TILED 3  /* large T: LDS-tiled matrix-core GEMM            */
#define Q4LIN_ROUTE_DECODE 4 /* one token: one weight stream per CU, K split   */
#define Q4LIN_ROUTE_MID 5    /* medium T: row blocks x K slices, matrix cores  */
Q4LIN_API int q4lin_route(int64_t n, int64_t k, int64_t t);

/* Library version as major*10000 + minor*100 + patch. */
Q4LIN_API int q4lin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4LIN_H */
