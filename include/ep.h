/*
 * ep.h - C ABI of the MI355X (gfx950) MoE dispatch / combine library.
 *
 * One GPU's share of DeepEP-style expert-parallel dispatch and combine,
 * without the inter-GPU exchange.  The "ranks" here are segments of one
 * expert-major receive buffer in HBM.  Three stages:
 *
 *   ep_layout    top-k expert ids -> per-expert / per-rank counts, prefix
 *                offsets and the token->slot map (the routing handle).
 *   ep_dispatch  scatter BF16 tokens into the receive buffer, as BF16 or as
 *                FP8 E4M3 with one fp32 scale per 128 columns.
 *   ep_combine   gather expert outputs back to token order as the gate-
 *                weighted fp32 sum of the top-k rows, written as BF16.
 *
 * and the backward pair over the same routing handle:
 *
 *   ep_dispatch_backward  gradient of the tokens: the unit-weight combine of
 *                         the received rows' gradients.
 *   ep_combine_backward   gradients of the expert outputs (a dispatch of the
 *                         output gradient, scaled per copy) and of the gate
 *                         weights.
 *
 * Sources for what the operations are (the pages print no code):
 *   [GN]  GeekNews "DeepSeek publica DeepEP, una biblioteca open source para
 *         entrenamiento e inferencia MoE" (es.news.hada.io), sections
 *         "Resultados de medición de rendimiento", "Interfaz centrada en
 *         ElasticBuffer", "Patrones de uso en entrenamiento, prefill y
 *         decoding".
 *   [DOC] "DeepEP (DeepEveryParallel) Documentation" (docsearch.algolia.com),
 *         items 3 ("... for Inference Decoding") and 10 ("... for Training
 *         or Prefilling").
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (hipMalloc / torch CUDA
 *     tensors), row-major and contiguous; `shape` is a HOST pointer.
 *   - The caller owns every buffer, including the layout workspace.  The
 *     library allocates nothing, keeps no state between calls and may be
 *     called from several host threads at once.
 *   - Work is only enqueued on `stream` (0 = the null stream); nothing
 *     synchronises the host.  Results are valid in stream order.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error nothing is launched and the status says why.
 *   - Bad data on the device (an expert id outside [-1, E), a pair beyond
 *     a padded expert's capacity) is never fatal: such pairs get slot -1
 *     and are counted in diag.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 6

/* Limits checked by every entry point (EP_ERR_UNSUPPORTED beyond them). */
#define EP_MAX_EXPERTS 2048
#define EP_MAX_TOPK 64
#define EP_MAX_NUM_CUS 65535

/*
 * Problem shape.  T tokens of hidden size H, each routed to k experts out of
 * E; the E experts are split into R contiguous groups of E/R ("ranks").
 * The arguments mirror DeepEP's buffer and dispatch parameters (maximum
 * tokens, hidden, num_topk, num_experts, expert_alignment: [GN] "Interfaz
 * centrada en ElasticBuffer"; [DOC] item 10).
 *
 *   num_tokens        T >= 0
 *   hidden            H > 0, a multiple of 8 (of 128 for FP8 dispatch)
 *   num_topk          k in [1, EP_MAX_TOPK], k <= E
 *   num_experts       E in [1, EP_MAX_EXPERTS]
 *   num_ranks         R >= 1, R divides E
 *   expert_alignment  A >= 1: each expert's segment of the flat layout is
 *                     padded to a multiple of A rows (for grouped GEMMs)
 *   capacity          C >= 0: 0 = flat expert-major layout; C > 0 = padded
 *                     per-expert layout [E, C] (low-latency decode form),
 *                     requires A == 1
 *   num_cus           launch budget of dispatch, combine and the backward
 *                     pair, the analog of DeepEP's num_sms argument ([GN]
 *                     "Interfaz centrada en ElasticBuffer": a caller-given
 *                     SM count overrides the computed one).  0 = the whole
 *                     GPU: one wavefront per work item.  n in
 *                     [1, EP_MAX_NUM_CUS] = n persistent workgroups of up to
 *                     1024 threads that loop over the work; the hardware
 *                     dispatcher spreads them over the CUs (on an idle
 *                     MI355X the bandwidth grows linearly with n up to
 *                     ~96), leaving the rest of the chip to kernels on
 *                     other streams.  Results do not depend on it.  ep_layout
 *                     ignores it (its launch is latency-bound and small).
 */
typedef struct ep_shape_t {
    int32_t num_tokens;
    int32_t hidden;
    int32_t num_topk;
    int32_t num_experts;
    int32_t num_ranks;
    int32_t expert_alignment;
    int32_t capacity;
    int32_t num_cus;
} ep_shape_t;

typedef enum ep_dtype_t {
    EP_BF16 = 0,        /* receive rows are BF16 copies of the tokens            */
    EP_FP8_E4M3 = 1,    /* OCP E4M3FN codes + one fp32 scale per 128 columns     */
    EP_MXFP8_E4M3 = 2,  /* OCP MX: E4M3 codes + one E8M0 scale per 32 columns    */
    EP_MXFP4_E2M1 = 3   /* OCP MX: E2M1 codes, 2 per byte, + E8M0 per 32 columns */
} ep_dtype_t;

typedef enum ep_status_t {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,  /* null pointer or inconsistent shape           */
    EP_ERR_UNSUPPORTED = 2,  /* shape outside the supported limits           */
    EP_ERR_MISALIGNED = 3,   /* a row pointer is not 16-byte aligned         */
    EP_ERR_WORKSPACE = 4,    /* workspace missing or too small               */
    EP_ERR_HIP = 5           /* a HIP launch failed; see ep_last_hip_error() */
} ep_status_t;

/*
 * Rows of the receive buffer (recv_x, recv_scale, y, src_pair) for `shape`:
 * T*k + E*(A-1) for the flat layout, E*C for the padded one.  This is the
 * worst case over all routings, so buffers of this size never overflow and
 * no device->host count read is needed (the analog of sizing DeepEP's buffer
 * from its maximum token count: [GN] "Interfaz centrada en ElasticBuffer").
 * Host only.
 */
ep_status_t ep_recv_rows(const ep_shape_t *shape, int64_t *rows);

/*
 * Bytes of device workspace ep_layout needs for `shape` (per-tile counts;
 * no initial contents required).  Host only.  One workspace must not be
 * used by two ep_layout calls that may overlap in time.
 */
ep_status_t ep_layout_workspace_bytes(const ep_shape_t *shape, size_t *bytes);

/*
 * Routing layout: the per-expert counts the expert GEMM needs and the
 * routing metadata combine needs ([GN] "Patrones de uso en entrenamiento,
 * prefill y decoding"; [DOC] item 10).  The outputs are the reusable
 * handle: calling ep_dispatch / ep_combine again with the same `slot` is
 * the cached-handle path that skips the layout ([DOC] item 3).
 *
 *   topk_idx      int32 [T, k]  expert of pair (t, j); -1 = masked pair
 *   expert_count  int32 [E]     pairs routed to each expert (true count,
 *                               also when the padded layout drops pairs)
 *   expert_offset int32 [E+1]   first receive row of each expert; [E] is
 *                               the end of the flat layout (e*C if padded)
 *   rank_count    int32 [R]     distinct tokens with >= 1 expert in rank r
 *                               (rank r owns experts [r*E/R, (r+1)*E/R))
 *   rank_offset   int32 [R+1]   expert_offset[r*E/R]
 *   slot          int32 [T, k]  receive row of pair (t, j), or -1
 *   src_pair      int32 [ep_recv_rows] or NULL: pair t*k+j held by each
 *                               receive row, -1 for padding rows
 *   diag          int32 [2] or NULL: [0] ids outside [-1, E), [1] pairs
 *                               dropped by the padded layout's capacity
 *   workspace     device buffer of ep_layout_workspace_bytes (see there)
 *
 * Slot order inside an expert is ascending (t, j): the layout is a stable
 * counting sort of the pairs by expert, deterministic bit for bit.
 */
ep_status_t ep_layout(const ep_shape_t *shape, const int32_t *topk_idx,
                      int32_t *expert_count, int32_t *expert_offset,
                      int32_t *rank_count, int32_t *rank_offset,
                      int32_t *slot, int32_t *src_pair, int32_t *diag,
                      void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Dispatch: every pair (t, j) with slot >= 0 receives token t
 * ([DOC] item 10: dispatch routes tokens to their experts, in BF16 or FP8).
 *
 *   x          BF16 [T, H]      tokens (bit patterns, 16-byte aligned)
 *   slot       int32 [T, k]     from ep_layout
 *   recv_dtype EP_BF16:     recv_x is BF16 [rows, H], a bit copy of x[t];
 *              EP_FP8_E4M3: recv_x is uint8 [rows, H] OCP E4M3FN codes and
 *                           recv_scale fp32 [rows, H/128]: per 128-column
 *                           block b, s = max(amax_b, 1e-4) / 448 and
 *                           code = E4M3_RNE_SAT(x / s), both in fp32, with
 *                           a correctly rounded division
 *              EP_MXFP8_E4M3, EP_MXFP4_E2M1: the OCP Microscaling (MX v1.0)
 *                           formats MI355X's matrix cores read, the
 *                           counterpart of the 4-bit dispatch of DeepEP's
 *                           Hybrid-EP branch ([GN] "Ramas experimentales y
 *                           forks de la comunidad").  Per 32-column block b:
 *                           e = floor(log2 amax_b) - emax (8 for E4M3, 2 for
 *                           E2M1), clamped to [-127, 127], -127 for an
 *                           all-zero block; element = RNE(x * 2^-e)
 *                           saturated to the largest normal (448 / 6), sign
 *                           kept; recv_scale[row, b] = e + 127 (E8M0 byte).
 *                           MXFP8 rows are [H] bytes, MXFP4 rows [H/2] bytes
 *                           with column 2i in the low nibble of byte i.
 *                           H must be a multiple of 32.
 *   recv_x     [ep_recv_rows, H] (BF16, E4M3, MXFP8) or [ep_recv_rows, H/2]
 *              bytes (MXFP4), 16-byte aligned; rows that no pair maps to
 *              are left untouched
 *   recv_scale fp32 [ep_recv_rows, H/128] for EP_FP8_E4M3, uint8
 *              [ep_recv_rows, H/32] for the MX formats; ignored (may be
 *              NULL) for EP_BF16
 *
 * Non-finite x: BF16 copies any bits.  An EP_FP8_E4M3 block holding an Inf
 * gets an Inf scale, its finite elements code to +-0 and the Inf to a NaN
 * code; the codes and scale of a block holding a NaN are unspecified.
 */
ep_status_t ep_dispatch(const ep_shape_t *shape, const void *x, const int32_t *slot,
                        ep_dtype_t recv_dtype, void *recv_x, void *recv_scale,
                        hipStream_t stream);

/*
 * ep_layout followed by ep_dispatch, with the same arguments and bit for bit
 * the same results.  It is one launch when recv_dtype is EP_BF16 or
 * EP_FP8_E4M3, num_cus is 0 and the batch holds at most 1024 pairs
 * (T * k <= 1024; the decode shape) with either a padded layout (capacity
 * > 0, E <= 2048) or expert_alignment 1 (E <= 1024), or fits one layout tile
 * (E <= 256): the dispatch works the slots out itself instead of waiting for
 * a layout launch and reading them back (the per-step layout of the decode
 * path: [DOC] item 3; [GN] "Patrones de uso en entrenamiento, prefill y
 * decoding").  Otherwise it enqueues the two calls.  Argument checks are
 * those of the two calls.
 */
ep_status_t ep_layout_dispatch(const ep_shape_t *shape, const int32_t *topk_idx,
                               int32_t *expert_count, int32_t *expert_offset,
                               int32_t *rank_count, int32_t *rank_offset,
                               int32_t *slot, int32_t *src_pair, int32_t *diag,
                               void *workspace, size_t workspace_bytes,
                               const void *x, ep_dtype_t recv_dtype, void *recv_x,
                               void *recv_scale, hipStream_t stream);

/*
 * Dispatch of tokens the caller has already quantised: DeepEP's dispatch
 * takes FP8 input as a (data, scale factors) pair ([DOC] item 10).  Every
 * valid pair (t, j) receives the codes and scales of token t unchanged (a
 * byte scatter): recv_x[slot[t, j], :] = x_q[t, :] and
 * recv_scale[slot[t, j], :] = x_scale[t, :].  Feeding it the output of an
 * EP_FP8_E4M3 ep_dispatch to rows 0..T-1 reproduces ep_dispatch's result.
 *
 *   x_q         uint8 [T, H]          E4M3 codes (any bytes), 16-byte aligned
 *   x_scale     fp32 [T, H/128]       block scales
 *   slot        int32 [T, k]          from ep_layout
 *   recv_x      uint8 [ep_recv_rows, H], 16-byte aligned; unmapped rows untouched
 *   recv_scale  fp32 [ep_recv_rows, H/128]
 * H must be a multiple of 128.
 */
ep_status_t ep_dispatch_prequantized(const ep_shape_t *shape, const void *x_q,
                                     const float *x_scale, const int32_t *slot,
                                     void *recv_x, float *recv_scale, hipStream_t stream);

/*
 * Combine: the expert outputs are reduced back to token order
 * ([DOC] item 10; [GN] "Patrones de uso ..."):
 *   out[t, h] = BF16_RNE( acc ),  acc = +0, then for j = 0..k-1 with
 *               slot[t, j] >= 0:  acc = fmaf(w[t, j], y[slot[t, j], h], acc)
 * The fixed order makes the result deterministic and identical to a scalar
 * evaluation of the same chain.  Non-finite y follows IEEE arithmetic; a
 * NaN result's bit pattern is not specified.
 *
 *   y             BF16 [ep_recv_rows, H]   expert outputs in receive layout
 *   slot          int32 [T, k]             from ep_layout
 *   topk_weights  fp32 [T, k]              gate weights (no renormalisation)
 *   out           BF16 [T, H]
 */
ep_status_t ep_combine(const ep_shape_t *shape, const void *y, const int32_t *slot,
                       const float *topk_weights, void *out, hipStream_t stream);

/*
 * Backward of dispatch.  DeepEP runs it as a combine over the same handle
 * ([DOC] item 10, "Backward Pass"; [GN] "Patrones de uso ...").  Forward,
 * every valid pair's row is a copy of x[t], so the gradient of x[t] is the
 * sum of its copies' gradients:
 *   grad_x[t, h] = BF16_RNE( acc ),  acc = +0, then for j = 0..k-1 with
 *                  slot[t, j] >= 0:  acc = acc + grad_recv_x[slot[t, j], h]
 * (fp32, ascending j): ep_combine with every weight 1, bit for bit.  Pairs
 * that are masked or were dropped by a padded layout contribute nothing.
 * For FP8 dispatch the quantisation is passed through as the identity.
 *
 *   grad_recv_x  BF16 [ep_recv_rows, H]  gradient of the received rows
 *   slot         int32 [T, k]            from ep_layout
 *   grad_x       BF16 [T, H]
 */
ep_status_t ep_dispatch_backward(const ep_shape_t *shape, const void *grad_recv_x,
                                 const int32_t *slot, void *grad_x, hipStream_t stream);

/*
 * Backward of combine.  DeepEP runs it as a dispatch over the same handle
 * ([DOC] item 10, "Backward Pass"; [GN] "Patrones de uso ...").  Forward,
 * out[t] = sum over valid j of w[t, j] * y[slot[t, j]] (its BF16 rounding is
 * passed through as the identity), so for g = d loss / d out:
 *   grad_y[slot[t, j], h] = BF16_RNE( w[t, j] * g[t, h] )  (fp32 product)
 *   grad_weights[t, j]    = sum over h of g[t, h] * y[slot[t, j], h]  (fp32)
 * grad_y rows that no valid pair maps to are left untouched;
 * grad_weights of a masked or dropped pair is 0.  grad_y is exact to the
 * definition.  grad_weights is summed in a fixed, deterministic tree; it
 * lies within (H/64 + 16) * 2^-24 * sum_h |g[t, h] * y[slot[t, j], h]| of
 * the exact dot product (every BF16 x BF16 product is exact in fp32).
 *
 *   grad_out      BF16 [T, H]             g
 *   y             BF16 [ep_recv_rows, H]  the expert outputs combine read;
 *                                         may be NULL if grad_weights is NULL
 *   slot          int32 [T, k]            from ep_layout
 *   topk_weights  fp32 [T, k]             the gate weights combine used
 *   grad_y        BF16 [ep_recv_rows, H]
 *   grad_weights  fp32 [T, k], or NULL to skip the weight gradient (then y
 *                 is not read)
 */
ep_status_t ep_combine_backward(const ep_shape_t *shape, const void *grad_out, const void *y,
                                const int32_t *slot, const float *topk_weights, void *grad_y,
                                float *grad_weights, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *ep_status_string(ep_status_t status);

/* EP_ABI_VERSION of the loaded library. */
int ep_abi_version(void);

/* hipError_t of the last EP_ERR_HIP returned on the calling thread, else 0. */
int ep_last_hip_error(void);

/*
 * Conversion check helpers.  They run, element by element, the exact device
 * routines ep_dispatch and ep_combine use for their final rounding steps, so
 * a test can sweep whole input ranges:
 *   ep_check_cvt_e4m3: out[i] = E4M3 code of in[i], round to nearest even;
 *                      defined for |in[i]| <= 464 (E4M3FN's top code 448 and
 *                      its rounding half-step), which covers every quotient
 *                      FP8 dispatch produces (|x / s| <= 448 plus one ulp)
 *   ep_check_cvt_bf16: out[i] = BF16_RNE(in[i]) for finite in[i]
 *   ep_check_cvt_e2m1: out[i] = E2M1 code (low 4 bits) of in[i], nearest
 *                      with ties to even, saturating at +-6, sign kept
 *   ep_check_quant_e4m3: out[i] = the E4M3 code FP8 dispatch stores for the
 *                      BF16 value x[i] (bit pattern) under block scale s[i]:
 *                      the code of the correctly rounded quotient x / s,
 *                      through the dispatch kernels' own quantiser; defined
 *                      for |x| <= 448 * s (every value a block with that
 *                      scale holds)
 * in is a device fp32 array of n elements (x: n BF16 bit patterns and s: n
 * fp32 scales), out a device array of n codes (uint8) or BF16 bit patterns
 * (uint16); n >= 0.
 */
ep_status_t ep_check_cvt_e4m3(const float *in, uint8_t *out, int64_t n, hipStream_t stream);
ep_status_t ep_check_cvt_bf16(const float *in, uint16_t *out, int64_t n, hipStream_t stream);
ep_status_t ep_check_cvt_e2m1(const float *in, uint8_t *out, int64_t n, hipStream_t stream);
ep_status_t ep_check_quant_e4m3(const uint16_t *x, const float *s, uint8_t *out, int64_t n,
                                hipStream_t stream);

/*
 * Streaming probe, for measurement only (not part of the method): the
 * practical memory ceiling of a read:write mix.  Unit u of `units` reads
 * read_chunks contiguous 1 KiB chunks of src at byte offset
 * u * read_chunks * 1024, XORs them (16-byte lanes), and writes the result
 * to write_chunks contiguous 1 KiB chunks of dst at byte offset
 * u * write_chunks * 1024.  Cache policy: 0 non-temporal loads and
 * stores, 1 default loads and stores, 2 non-temporal loads and device-scope
 * (sc1) stores, 3 default loads and non-temporal stores; policy + 4 takes the
 * units in XCD-contiguous order (each of the 8 XCDs one contiguous eighth)
 * instead of round robin.  src must hold
 * units * read_chunks KiB and dst units * write_chunks KiB, both device
 * memory, 16-byte aligned.  read_chunks is 1, 2, 4, 8 or 16; write_chunks
 * is 1..64; policy 0..7; units >= 0.
 */
ep_status_t ep_probe_stream(const void *src, void *dst, int64_t units, int read_chunks,
                            int write_chunks, int policy, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
