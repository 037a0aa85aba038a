/*
 * dora.h - C ABI of the MI355X (gfx950) DoRA hot-path library, libdora.so.
 *
 * DoRA rescales every output row of an adapted weight to a learned magnitude:
 *
 *     V' = W0 + s * B A            (adapted direction, [d_out, d_in])
 *     n_i = || V'_i ||             (row norm, one per output feature)
 *     y   = x (diag(m / n) V')^T   (layer output)
 *
 * (DoRA reading notes, zhongzhuzhou.org: Sec. 3.1 eq. (6) and Sec. 3.2
 * Algorithm 1; Scaling DoRA summary page, gptget.net, arXiv
 * 2603.22276, abstract, for the row-wise norm of W + sBA and the scale s.)
 *
 * The library never forms the d_out x d_in product B A.  The norm is
 * evaluated in factored form from ||W0_i||^2, 2s B_i.(W0 A^T)_i and
 * s^2 B_i (A A^T) B_i^T (Scaling DoRA abstract: base, cross and Gram terms),
 * and the output is composed in one pass in the near-unity form
 * y = base + ((g - 1) base + g s lora) with g - 1 = (m - n) / n
 * (Scaling DoRA abstract: numerically stable form for the near-unity regime).
 *
 * Conventions for every entry point
 *   Layout     Row-major and contiguous, nn.Linear convention:
 *                W0 [d_out, d_in]   A [r, d_in]   B [d_out, r]   m [d_out]
 *                x  [T, d_in]       y [T, d_out]  xs [T, r]      (T = tokens)
 *   Types      Every tensor has the layer dtype (DORA_F32 or DORA_BF16), except
 *              norm and grad_m, which are always float32.  Accumulation is
 *              float32; each output is rounded once, to nearest even.
 *   Memory     All tensor pointers are DEVICE pointers, 16-byte aligned.  The
 *              caller owns every buffer, including the workspace `ws`; the
 *              library allocates no device memory and keeps no data between
 *              calls.  Inputs are read only.  Outputs must not overlap inputs
 *              or each other.
 *   Streams    Work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 *              null stream) and the call returns without synchronising.
 *              dora_forward and dora_backward may fork independent parts to a
 *              second stream of the library's own (default priority, one per
 *              host thread and device, created on the first call and kept
 *              until the process ends) and join it back through events before
 *              returning: all work of a call is ordered before anything the
 *              caller enqueues on `hip_stream` afterwards, and the pattern is
 *              valid under stream capture.  Calls on distinct buffers may be
 *              made from several host threads.
 *   Errors     Arguments are validated before anything is enqueued; on a
 *              validation error nothing is written.  Return value 0 = enqueued,
 *              negative = DORA_ERR_* below.  DORA_ERR_HIP means the HIP runtime
 *              rejected a launch (hipGetLastError is checked after each one);
 *              kernels already enqueued may then have run.
 *   Sizes      1 <= d_out, d_in < 2^22; 0 <= r < 2^22; 0 <= tokens < 2^31.
 *              d_out, d_in and r must be multiples of 8 (16-byte rows for both
 *              dtypes).
 */
#ifndef DORA_H
#define DORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DORA_API __attribute__((visibility("default")))

typedef enum { DORA_F32 = 0, DORA_BF16 = 1 } dora_dtype;

/* Layer description shared by every call. */
typedef struct {
    int64_t  d_out;     /* output features (rows of W0, B; entries of m)        */
    int64_t  d_in;      /* input features (columns of W0, A; columns of x)      */
    int64_t  r;         /* LoRA rank (rows of A, columns of B); 0 = no LoRA     */
    int64_t  tokens;    /* T, rows of x and y; 0 allowed                        */
    int32_t  dtype;     /* dora_dtype of every tensor except norm / grad_m      */
    float    s;         /* LoRA scale multiplying B A (any finite value)        */
    uint32_t flags;     /* DORA_FLAG_* bits, 0 for the default path             */
    uint32_t reserved;  /* must be 0                                            */
} dora_shape;

/* flags */
#define DORA_FLAG_EXACT_NORM_GRAD   (1u << 0)  /* backward: undetached norm gradient (DoRA reading notes, Appendix A.1); needs the matching workspace size */
#define DORA_FLAG_SEPARATE_COMPOSE  (1u << 1)  /* forward/backward: run the standalone compose kernels instead of the GEMM-fused ones */

/* op ids for dora_workspace_bytes */
#define DORA_OP_NORM      0
#define DORA_OP_FORWARD   1
#define DORA_OP_BACKWARD  2
#define DORA_OP_MERGE     3
#define DORA_OP_VERA_GRADS 4

/* return codes */
#define DORA_OK              0
#define DORA_ERR_NULL       -1  /* a required pointer is NULL                          */
#define DORA_ERR_SHAPE      -2  /* a dimension is out of range or not a multiple of 8   */
#define DORA_ERR_DTYPE      -3  /* dtype is not DORA_F32 / DORA_BF16                    */
#define DORA_ERR_ALIGN      -4  /* a pointer is not 16-byte aligned                     */
#define DORA_ERR_WORKSPACE  -5  /* ws_bytes < dora_workspace_bytes(shape, op)           */
#define DORA_ERR_HIP        -6  /* the HIP runtime reported an error                    */
#define DORA_ERR_FLAGS      -7  /* unknown flag bits, reserved != 0, or s not finite    */

/*
 * Bytes of device workspace `op` needs for `shape`: O(d_out*r + r*r + T*r)
 * for the norm, merge and GEMM-fused paths, plus one [T, d_out] buffer for the
 * DORA_FLAG_SEPARATE_COMPOSE forward and for the backward; never d_out*d_in.
 * Returns 0 if the shape is invalid (the calls then fail with DORA_ERR_SHAPE).
 */
DORA_API size_t dora_workspace_bytes(const dora_shape* shape, int op);

/*
 * Row norms n_i = || W0_i + s (B A)_i ||, in factored form (Scaling DoRA
 * abstract: base, cross and Gram terms through O(d_out r + r^2)
 * intermediates; DoRA reading notes Algorithm 1, per output row).
 *   W0, A, B   inputs (layer dtype); A and B may be NULL when r == 0
 *   norm_out   output, float32 [d_out]
 *   ws         workspace of at least dora_workspace_bytes(shape, DORA_OP_NORM)
 */
DORA_API int dora_norm(const dora_shape* shape, const void* W0, const void* A, const void* B,
                       float* norm_out, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Forward of a DoRA linear layer (DoRA reading notes Algorithm 1):
 *   norm_out = n (float32 [d_out], as dora_norm),
 *   xs_out   = s * (x A^T)                  [T, r], layer dtype; NULL = not kept,
 *   y        = g * (x W0^T + xs B^T) with g = m / max(n, 1e-8),
 *              composed as base + ((g - 1) base + g s lora) in float32
 *              and rounded once (Scaling DoRA abstract).
 *   x, W0, A, B, m   inputs; y, norm_out required outputs; xs_out optional.
 * y, norm and xs are what dora_backward consumes.
 */
DORA_API int dora_forward(const dora_shape* shape, const void* x, const void* W0, const void* A,
                          const void* B, const void* m, void* y, float* norm_out, void* xs_out,
                          void* ws, size_t ws_bytes, void* hip_stream);

/*
 * dora_forward for callers that cannot allocate device memory (code under HIP
 * stream capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and validation as dora_forward, without ws / ws_bytes:
 * the workspace is a static device array of DORA_NOALLOC_SCRATCH_BYTES inside
 * the library, one copy on every GPU the library runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no stream or event
 * creation): every launch goes on hip_stream, without the side stream.
 *   Limit     shapes whose dora_workspace_bytes(shape, DORA_OP_FORWARD) exceeds
 *             DORA_NOALLOC_SCRATCH_BYTES return DORA_ERR_WORKSPACE (nothing is
 *             enqueued); every configuration up to d_out 27648, d_in 8192,
 *             r 384 and 8192 tokens fits.
 *   Sharing   all calls on one GPU use that GPU's one array, which keeps the last
 *             call's contents (nothing in it needs to start at zero).  Calls that
 *             overlap on one GPU (concurrent streams, or host threads) race on
 *             it: order them on one stream, or use dora_forward.
 *   Errors    as dora_forward; DORA_ERR_HIP also if the array's device address
 *             cannot be looked up.
 */
#define DORA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
DORA_API int dora_forward_noalloc(const dora_shape* shape, const void* x, const void* W0,
                                  const void* A, const void* B, const void* m, void* y,
                                  float* norm_out, void* xs_out, void* hip_stream);

/*
 * Backward of dora_forward for L with dL/dy = grad_y.  By default the norm is
 * detached, i.e. held constant (DoRA reading notes Sec. 3.4, the default
 * implementation there):
 *   grad_m_i = sum_t grad_y[t,i] y[t,i] / m_i          (eq. (8); needs m_i != 0)
 *   gz       = g * grad_y                               (eq. (7): dV' = (m/n) dW')
 *   grad_x   = gz W0 + s (gz B) A
 *   grad_B   = s gz^T (x A^T)      = gz^T xs
 *   grad_A   = s (gz B)^T x
 * With DORA_FLAG_EXACT_NORM_GRAD the norm is not detached: dV'_i is projected
 * off V'_i (Appendix A.1 of the notes), which adds, with
 * k'_i = -s m_i grad_m_i / n_i^2 and Bk' = diag(k') B,
 *   grad_B += diag(k') (W0 A^T + s B A A^T)
 *   grad_A += Bk'^T W0 + s (Bk'^T B) A
 * (grad_x and grad_m are the same in both modes).  W0 receives no gradient
 * (it is frozen).
 *   grad_y, x, W0, A, B, m, norm, y   inputs (norm and y as written by
 *                                     dora_forward for the same layer)
 *   xs        s * (x A^T) as written by dora_forward, or NULL to recompute it
 *   grad_x [T, d_in], grad_A [r, d_in], grad_B [d_out, r] (layer dtype) and
 *   grad_m [d_out] (float32): outputs; each may be NULL to skip it.
 */
DORA_API int dora_backward(const dora_shape* shape, const void* grad_y, const void* x,
                           const void* W0, const void* A, const void* B, const void* m,
                           const float* norm, const void* xs, const void* y,
                           void* grad_x, void* grad_A, void* grad_B, float* grad_m,
                           void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Merged weight for deployment (DoRA reading notes, Algorithm 1;
 * Sec. 3.1 eq. (6)): the dense layer that replaces the adapted one,
 *   W_out_i = g_i * (W0_i + s (B A)_i),  g_i = m_i / max(n_i, 1e-8),
 * so that x W_out^T equals dora_forward's y.  One GEMM, B . A over K = r, whose
 * epilogue adds W0 and scales each row; computed in float32, rounded once.
 *   W0, A, B, m   inputs (layer dtype)
 *   norm          float32 [d_out] as written by dora_norm / dora_forward, or NULL to
 *                 compute it here (in the workspace)
 *   W_out         output [d_out, d_in], layer dtype (the output is d_out x d_in by
 *                 definition; it must not overlap any input)
 *   ws            workspace of at least dora_workspace_bytes(shape, DORA_OP_MERGE)
 * shape->tokens is not used.
 */
DORA_API int dora_merge(const dora_shape* shape, const void* W0, const void* A, const void* B,
                        const void* m, const float* norm, void* W_out, void* ws, size_t ws_bytes,
                        void* hip_stream);

/*
 * DVoRA (DoRA reading notes, Sec. 3.5): DoRA whose direction update is VeRA's
 * diag(b) B_sh diag(d) A_sh, with A_sh [r, d_in] and B_sh [d_out, r] frozen
 * random matrices shared by all layers and b [d_out], d [r] the trainable
 * vectors of one layer.  It runs on the DoRA entry points with A = A_sh and
 * B = B_eff = diag(b) B_sh diag(d):
 *   dora_vera_scale    B_eff_ij = b_i B_sh_ij d_j   [d_out, r], layer dtype, rounded once
 *   dora_forward / dora_backward with B = B_eff (grad_A may be NULL: A_sh is frozen;
 *                      DORA_FLAG_EXACT_NORM_GRAD works unchanged)
 *   dora_vera_grads    grad_b_i = sum_j grad_B_eff_ij B_sh_ij d_j   [d_out]
 *                      grad_d_j = sum_i grad_B_eff_ij b_i B_sh_ij   [r]
 *                      (layer dtype; float32 accumulation in a fixed order; either
 *                      output may be NULL)
 * Only d_out, r and dtype of `shape` are used (the rest must still be valid).
 * dora_vera_grads needs dora_workspace_bytes(shape, DORA_OP_VERA_GRADS) bytes of ws.
 */
DORA_API int dora_vera_scale(const dora_shape* shape, const void* B_shared, const void* b,
                             const void* d, void* B_eff, void* hip_stream);
DORA_API int dora_vera_grads(const dora_shape* shape, const void* grad_B_eff,
                             const void* B_shared, const void* b, const void* d, void* grad_b,
                             void* grad_d, void* ws, size_t ws_bytes, void* hip_stream);

/* Static text for a DORA_* return code. */
DORA_API const char* dora_strerror(int code);

/*
 * Per-kernel timing, for measurement.  While enabled, every kernel the
 * library launches is bracketed by a pair of hipEvents recorded on its launch
 * stream.  dora_timing_collect waits for the recorded events, writes
 * {"<kernel label>": [launch count, total milliseconds], ...} as JSON text into
 * buf (NUL-terminated, truncated to buflen), clears the record and returns the
 * number of launches it covered, or DORA_ERR_HIP.  Enabling/disabling applies
 * to calls made afterwards, from any thread.
 */
DORA_API int dora_timing_enable(int enable);
DORA_API int dora_timing_collect(char* buf, size_t buflen);

/*
 * Measurement probe: the sustained dense bf16 MFMA rate.  Launches `blocks`
 * workgroups of four waves on hip_stream; each wave runs four independent
 * chains of `iters` v_mfma_f32_32x32x16_bf16 on register operands and writes
 * one checksum per thread to out (device, blocks * 256 floats, caller-owned).
 * Time it with events on the same stream; dora_probe_mfma_flops gives the
 * flops one such launch performs.  Returns DORA_ERR_SHAPE for iters < 1,
 * blocks < 1 or a NULL out, DORA_ERR_HIP if the launch fails.
 */
DORA_API int dora_probe_mfma(int64_t iters, int blocks, float* out, void* hip_stream);
DORA_API double dora_probe_mfma_flops(int64_t iters, int blocks);

/*
 * Measurement probe: the streaming HBM rate.  c = a + b elementwise over
 * `bytes` bytes of float32 (two streams read, one written: 3 * bytes of
 * traffic), device pointers, caller-owned, 16-byte aligned, c not aliasing a
 * or b.  Returns DORA_ERR_NULL, DORA_ERR_SHAPE (bytes not a positive multiple
 * of 16), DORA_ERR_ALIGN or DORA_ERR_HIP.
 */
DORA_API int dora_probe_stream(const void* a, const void* b, void* c, int64_t bytes,
                               void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DORA_H */
