/*
 * Reference (oracle) implementation of MoE routing layout, dispatch and
 * combine: plain, scalar, single-threaded C99.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the HIP library is
 * compared against.  Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant generator with the HIP path under
 * combine_ep_layout_02_amd/csrc, and it includes nothing from there.
 *
 * What is computed, and where the pages describe it:
 *   - layout: per-expert received-token counts, the prefix offsets of an
 *     expert-major receive buffer, and the token->slot map that combine
 *     later needs.  DeepEP's dispatch returns a handle holding the routing
 *     metadata combine needs, and the per-expert received counts the expert
 *     GEMM needs (GeekNews "DeepSeek publica DeepEP ...", section "Patrones
 *     de uso en entrenamiento, prefill y decoding"; DeepEP documentation,
 *     item 10 "Perform MoE Dispatch and Combine for Training or
 *     Prefilling").  Re-using that handle skips recomputing the layout
 *     (same GeekNews section; documentation item 3).
 *   - dispatch: each token is sent to each of its top-k experts, in BF16 or
 *     FP8 (documentation item 10; GeekNews section "Resultados de medición
 *     de rendimiento" names FP8 dispatch with BF16 combine).
 *   - combine: the expert outputs are reduced back to the token's origin
 *     (documentation item 10; GeekNews "Patrones de uso ...").
 *
 * The pages do not fix the slot order, the FP8 encoding, the scale rule or
 * the summation order.  This file takes one reading of each and states it
 * where it is used:
 *   R1  slots inside an expert segment are in ascending (token, k-index)
 *       order (a stable counting sort);
 *   R2  rank r owns the contiguous experts [r*E/R, (r+1)*E/R);
 *   R3  rank_count[r] is the number of distinct tokens with at least one
 *       valid expert on rank r;
 *   R4  expert_alignment A pads each expert segment to a multiple of A;
 *   R5  capacity C > 0 selects a padded [E, C] layout, pairs past C dropped;
 *   R6  id -1 is a masked pair; ids outside [-1, E) count as invalid and
 *       are treated as -1;
 *   R7  FP8 is OCP E4M3FN, round-to-nearest-even, saturating to +-448;
 *   R8  one fp32 scale per (row, 128-column block):
 *       s = max(amax, 1e-4) / 448, code = E4M3(x / s), all in fp32;
 *   R9  combine: acc = +0; for j ascending over valid slots
 *       acc = fmaf(w[t,j], y[slot[t,j], h], acc); out = BF16_RNE(acc);
 *   R10 the scales are row-major fp32 [rows, H/128], on the same row index
 *       as the receive row they scale;
 *   R11 dispatch backward: acc = +0; for j ascending over valid slots
 *       acc = acc + grad_recv[slot[t,j], h] (fp32); grad_x = BF16_RNE(acc);
 *   R12 combine backward: grad_y[slot[t,j], h] = BF16_RNE(w[t,j] * g[t,h])
 *       with the product rounded to fp32 first; grad_w[t,j] = the exact dot
 *       product of g[t] and y[slot[t,j]] (returned in double); the BF16
 *       rounding of the forward output passes the gradient through as is;
 *   R13 pre-quantised dispatch: the caller's E4M3 codes and 1x128 fp32
 *       scales are copied to every valid slot unchanged;
 *   R14 MX dispatch (MXFP8 = E4M3 elements, MXFP4 = E2M1 elements, one
 *       E8M0 scale per 32 columns) follows the OCP Microscaling Formats
 *       v1.0 conversion: e = floor(log2(amax)) - emax(element), clamped to
 *       [-127, 127] (an all-zero block takes -127), X = 2^e, element =
 *       RNE(x / X) saturated to the element's largest normal; the scale is
 *       stored as the biased byte e + 127; two E2M1 codes share a byte,
 *       the even column in the low nibble.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fPIC -shared oracle.c -lm
 * (no fast-math: every float operation below is one IEEE-754 binary32
 * operation rounded to nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ABI 1

int oracle_abi(void) { return ORACLE_ABI; }

/* ------------------------------------------------------------------ */
/* Layout                                                              */
/* ------------------------------------------------------------------ */

/* Worst-case number of receive rows: every pair valid and every expert
 * segment carrying A-1 padding rows (flat), or E*C (padded). */
int64_t oracle_recv_rows(int64_t T, int64_t k, int64_t E, int64_t A, int64_t C)
{
    if (C > 0) return E * C;
    return T * k + E * (A - 1);
}

/*
 * Routing layout (readings R1..R6 above).  Returns 0, or -1 if scratch
 * memory could not be allocated.
 *
 * idx          [T*k]  expert id of pair (t, j) at t*k + j
 * expert_count [E]    pairs routed to each expert (the true count, also in
 *                     padded mode)
 * expert_offset[E+1]  start row of each expert's segment; [E] = end
 * rank_count   [R]    distinct tokens sent to each rank
 * rank_offset  [R+1]  expert_offset[r*E/R]
 * slot         [T*k]  receive row of pair (t, j), -1 if masked or dropped
 * src_pair     [rows] pair t*k+j held by each receive row, -1 if none
 *                     (may be NULL)
 * diag         [2]    [0] invalid ids seen, [1] pairs dropped (may be NULL)
 */
int oracle_layout(int64_t T, int64_t k, int64_t E, int64_t R, int64_t A, int64_t C,
                  const int32_t *idx,
                  int32_t *expert_count, int32_t *expert_offset,
                  int32_t *rank_count, int32_t *rank_offset,
                  int32_t *slot, int32_t *src_pair, int64_t rows,
                  int32_t *diag)
{
    int64_t e, r, t, j, i;
    int64_t per_rank = E / R;
    int32_t invalid = 0, dropped = 0;
    int32_t *next;

    /* counts (R6: an id outside [-1, E) is treated as masked) */
    for (e = 0; e < E; ++e) expert_count[e] = 0;
    for (i = 0; i < T * k; ++i) {
        int32_t v = idx[i];
        if (v >= 0 && v < E) expert_count[v] += 1;
        else if (v != -1) invalid += 1;
    }

    /* offsets: flat segments padded to a multiple of A (R4), or e*C (R5) */
    expert_offset[0] = 0;
    for (e = 0; e < E; ++e) {
        if (C > 0) {
            expert_offset[e + 1] = (int32_t)((e + 1) * C);
        } else {
            int64_t padded = ((expert_count[e] + A - 1) / A) * A;
            expert_offset[e + 1] = (int32_t)(expert_offset[e] + padded);
        }
    }

    /* ranks (R2, R3) */
    for (r = 0; r <= R; ++r) rank_offset[r] = expert_offset[r * per_rank];
    for (r = 0; r < R; ++r) rank_count[r] = 0;
    for (t = 0; t < T; ++t) {
        for (r = 0; r < R; ++r) {
            int hit = 0;
            for (j = 0; j < k; ++j) {
                int32_t v = idx[t * k + j];
                if (v >= 0 && v < E && v / per_rank == r) hit = 1;
            }
            rank_count[r] += hit;
        }
    }

    /* slots: a stable counting sort, pairs visited in (t, j) order (R1).
     * next[e] is the position the next pair of expert e takes inside its
     * segment. */
    next = (int32_t *)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
    if (!next) return -1;
    if (src_pair)
        for (i = 0; i < rows; ++i) src_pair[i] = -1;
    for (i = 0; i < T * k; ++i) {
        int32_t v = idx[i];
        int32_t p;
        slot[i] = -1;
        if (!(v >= 0 && v < E)) continue;
        p = next[v]++;
        if (C > 0) {
            if (p >= C) { dropped += 1; continue; }
            slot[i] = (int32_t)(v * C + p);
        } else {
            slot[i] = expert_offset[v] + p;
        }
        if (src_pair) src_pair[slot[i]] = (int32_t)i;
    }
    free(next);

    if (diag) { diag[0] = invalid; diag[1] = dropped; }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/*
 * float32 -> BF16, round to nearest, ties to even.  BF16 values are the
 * float32 values whose low 16 bits are zero; the two candidates are the
 * truncation `lo` and the next BF16 away from zero `hi`.  The distances are
 * compared exactly in double.  NaN maps to the canonical quiet NaN.
 */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u, lo_u, hi_u;
    float lo, hi;
    double dlo, dhi;
    if (isnan(f)) return 0x7FC0;
    memcpy(&u, &f, 4);
    lo_u = u & 0xFFFF0000u;
    hi_u = lo_u + 0x10000u;  /* next magnitude up; may become +-Inf */
    memcpy(&lo, &lo_u, 4);
    memcpy(&hi, &hi_u, 4);
    if (isinf(f)) return (uint16_t)(lo_u >> 16);
    dlo = fabs((double)f - (double)lo);
    /* past the largest finite BF16 the next step up is Inf; for rounding
     * it stands at 2^128, where the exponent range would continue */
    if (isinf(hi)) dhi = fabs(ldexp(1.0, 128) - fabs((double)f));
    else dhi = fabs((double)hi - (double)f);
    if (dlo < dhi) return (uint16_t)(lo_u >> 16);
    if (dhi < dlo) return (uint16_t)(hi_u >> 16);
    return ((lo_u >> 16) & 1u) ? (uint16_t)(hi_u >> 16) : (uint16_t)(lo_u >> 16);
}

void oracle_bf16_rne_array(const float *in, uint16_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = oracle_bf16_rne(in[i]);
}

/*
 * OCP 8-bit floating point, E4M3FN flavour (reading R7): 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, the single
 * NaN pattern S.1111.111, largest finite magnitude 1.75 * 2^8 = 448.
 * Exponent field 0 is subnormal: m/8 * 2^-6.
 */
double oracle_e4m3_decode(uint8_t c)
{
    int e = (c >> 3) & 0xF, m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);            /* m/8 * 2^-6     */
    else mag = ldexp((double)(8 + m), e - 10);         /* (1+m/8)*2^(e-7) */
    return (c & 0x80) ? -mag : mag;
}

/*
 * float32 -> E4M3FN with round-to-nearest-even and saturation to +-448.
 * The non-negative finite codes 0x00..0x7E are ordered by value, so the
 * encoder finds the largest code whose value does not exceed |v| by a
 * binary search, then compares |v| with the midpoint to the next code:
 * below -> lower code, above -> upper code, exactly on it -> the code with
 * an even mantissa (its last bit is 0).  The sign is kept, so a negative
 * value that rounds to zero gives 0x80.  NaN gives 0x7F (with sign).
 */
static double e4m3_mag[127];  /* values of codes 0x00..0x7E, filled once */
static int e4m3_mag_ready = 0;

uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    int lo = 0, hi = 0x7E, code;
    double mid;
    if (!e4m3_mag_ready) {
        int c;
        for (c = 0; c < 127; ++c) e4m3_mag[c] = oracle_e4m3_decode((uint8_t)c);
        e4m3_mag_ready = 1;
    }
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);   /* saturate */
    /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int m = (lo + hi) / 2;
        int below = e4m3_mag[m] <= a;
        lo = below ? m : lo;
        hi = below ? hi : m;
    }
    mid = 0.5 * (e4m3_mag[lo] + e4m3_mag[hi]);  /* exact: short dyadic rationals */
    if (a < mid) code = lo;
    else if (a > mid) code = hi;
    else code = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | code);
}

void oracle_e4m3_encode_array(const float *in, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(in[i]);
}

/* The FP8 dispatch's per-element step (R8) on its own: code of the BF16
 * value x[i] divided by the block scale s[i] (one fp32 division). */
void oracle_fp8_quantize_array(const uint16_t *x, const float *s, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(bf16_to_f32(x[i]) / s[i]);
}

/* ------------------------------------------------------------------ */
/* Dispatch                                                            */
/* ------------------------------------------------------------------ */

/* BF16 dispatch: receive row slot[t,j] is a bit copy of token row t. */
void oracle_dispatch_bf16(int64_t T, int64_t H, int64_t k,
                          const uint16_t *x, const int32_t *slot,
                          uint16_t *recv_x)
{
    int64_t t, j;
    for (t = 0; t < T; ++t)
        for (j = 0; j < k; ++j) {
            int32_t s = slot[t * k + j];
            if (s < 0) continue;
            memcpy(recv_x + (int64_t)s * H, x + t * H, (size_t)H * sizeof(uint16_t));
        }
}

/*
 * FP8 dispatch (readings R7, R8).  For each token t and each 128-column
 * block b:
 *   amax = max |x[t, 128b + i]|            (exact, in fp32)
 *   s    = max(amax, 1e-4f) / 448.0f       (one fp32 division)
 *   q_i  = E4M3(x[t, 128b + i] / s)        (one fp32 division each)
 * and every valid slot of t receives the codes q and the scale s at
 * recv_scale[slot, b].  H must be a multiple of 128.
 */
void oracle_dispatch_fp8(int64_t T, int64_t H, int64_t k,
                         const uint16_t *x, const int32_t *slot,
                         uint8_t *recv_x, float *recv_scale)
{
    int64_t t, b, i, j;
    int64_t nb = H / 128;
    uint8_t codes[128];
    for (t = 0; t < T; ++t) {
        for (b = 0; b < nb; ++b) {
            const uint16_t *xb = x + t * H + b * 128;
            float amax = 0.0f, s;
            /* a NaN never compares greater, so it takes no part in amax (a
             * block holding one is outside the GPU path's contract); an Inf
             * makes the scale Inf */
            for (i = 0; i < 128; ++i) {
                float a = fabsf(bf16_to_f32(xb[i]));
                if (a > amax) amax = a;
            }
            s = (amax > 1e-4f ? amax : 1e-4f) / 448.0f;
            for (i = 0; i < 128; ++i) codes[i] = oracle_e4m3_encode(bf16_to_f32(xb[i]) / s);
            for (j = 0; j < k; ++j) {
                int32_t sl = slot[t * k + j];
                if (sl < 0) continue;
                memcpy(recv_x + (int64_t)sl * H + b * 128, codes, 128);
                recv_scale[(int64_t)sl * nb + b] = s;
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Combine                                                             */
/* ------------------------------------------------------------------ */

/*
 * Gate-weighted combine (reading R9): for each token t and column h,
 *   acc = +0.0f
 *   for j = 0..k-1 with slot[t,j] >= 0:  acc = fmaf(w[t,j], y[slot,h], acc)
 *   out[t,h] = BF16_RNE(acc)
 */
void oracle_combine(int64_t T, int64_t H, int64_t k,
                    const uint16_t *y, const int32_t *slot, const float *w,
                    uint16_t *out)
{
    int64_t t, h, j;
    for (t = 0; t < T; ++t) {
        for (h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (j = 0; j < k; ++j) {
                int32_t s = slot[t * k + j];
                if (s < 0) continue;
                acc = fmaf(w[t * k + j], bf16_to_f32(y[(int64_t)s * H + h]), acc);
            }
            out[t * H + h] = oracle_bf16_rne(acc);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Backward pair                                                       */
/* ------------------------------------------------------------------ */
/*
 * DeepEP runs the backward of dispatch as a combine and the backward of
 * combine as a dispatch, over the same routing handle (GeekNews "DeepSeek
 * publica DeepEP ...", section "Patrones de uso en entrenamiento, prefill y
 * decoding"; DeepEP documentation, item 10, "Backward Pass").  The two
 * functions below are the gradients of the forward definitions above.
 */

/*
 * Dispatch backward (R11).  Forward, recv[slot[t,j]] = x[t] for each valid
 * pair, so the gradient of x[t] is the sum of the gradients of its received
 * copies.  Copies that were masked or dropped (slot -1) carry none.  The sum
 * runs in fp32 from +0 in ascending j, rounded once to BF16; it is the
 * combine of R9 with every weight 1 (fmaf(1, v, acc) == acc + v).
 *
 * grad_recv [rows, H] BF16 bits; slot [T, k]; grad_x [T, H] BF16 bits.
 */
void oracle_dispatch_backward(int64_t T, int64_t H, int64_t k,
                              const uint16_t *grad_recv, const int32_t *slot,
                              uint16_t *grad_x)
{
    int64_t t, h, j;
    for (t = 0; t < T; ++t) {
        for (h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (j = 0; j < k; ++j) {
                int32_t s = slot[t * k + j];
                if (s < 0) continue;
                acc = acc + bf16_to_f32(grad_recv[(int64_t)s * H + h]);
            }
            grad_x[t * H + h] = oracle_bf16_rne(acc);
        }
    }
}

/*
 * Combine backward (R12).  Forward, out[t] = sum over valid j of
 * w[t,j] * y[slot[t,j]], so for the gradient g = d loss / d out:
 *   d/dy[slot[t,j]] = w[t,j] * g[t]      (a dispatch of g, scaled per copy)
 *   d/dw[t,j]       = <g[t], y[slot[t,j]]>
 * grad_y rows: the fp32 product w * g (one IEEE multiply, nearest-even),
 * then BF16 nearest-even.  Rows that no valid pair maps to are not written.
 * grad_w: every product of two BF16 values is exact in double (8 + 8
 * significant bits), and the double sum over h carries a relative error of
 * at most H * 2^-53, so grad_w here is the exact dot product for all
 * practical purposes; the GPU's fp32 sum is compared to it within the
 * fp32 summation bound.  A masked or dropped pair gets grad_w = 0.
 *
 * g [T, H], y [rows, H] BF16 bits; slot, w [T, k]; grad_y [rows, H] BF16
 * bits (only valid rows written); grad_w [T, k] double.
 */
void oracle_combine_backward(int64_t T, int64_t H, int64_t k,
                             const uint16_t *g, const uint16_t *y,
                             const int32_t *slot, const float *w,
                             uint16_t *grad_y, double *grad_w)
{
    int64_t t, h, j;
    for (t = 0; t < T; ++t) {
        for (j = 0; j < k; ++j) {
            int32_t s = slot[t * k + j];
            double dot = 0.0;
            if (s < 0) {
                grad_w[t * k + j] = 0.0;
                continue;
            }
            for (h = 0; h < H; ++h) {
                float gv = bf16_to_f32(g[t * H + h]);
                float prod = w[t * k + j] * gv;
                grad_y[(int64_t)s * H + h] = oracle_bf16_rne(prod);
                dot += (double)gv * (double)bf16_to_f32(y[(int64_t)s * H + h]);
            }
            grad_w[t * k + j] = dot;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Other dispatch precisions                                           */
/* ------------------------------------------------------------------ */
/*
 * DeepEP's dispatch also takes its FP8 input already quantised, as a
 * (data, scale factors) pair (DeepEP documentation item 10), and the
 * Hybrid-EP branch adds a 4-bit format (GeekNews "DeepSeek publica DeepEP
 * ...", section "Ramas experimentales y forks de la comunidad").
 */

/*
 * Pre-quantised FP8 dispatch (R13): every valid slot of token t receives
 * the token's E4M3 codes x_q[t, :] and its block scales x_s[t, :] as they
 * are (a byte copy).  x_q [T, H] bytes, x_s [T, H/128] fp32.
 */
void oracle_dispatch_prequantized(int64_t T, int64_t H, int64_t k,
                                  const uint8_t *x_q, const float *x_s,
                                  const int32_t *slot, uint8_t *recv_x,
                                  float *recv_scale)
{
    int64_t t, j;
    int64_t nb = H / 128;
    for (t = 0; t < T; ++t)
        for (j = 0; j < k; ++j) {
            int32_t sl = slot[t * k + j];
            if (sl < 0) continue;
            memcpy(recv_x + (int64_t)sl * H, x_q + t * H, (size_t)H);
            memcpy(recv_scale + (int64_t)sl * nb, x_s + t * nb, (size_t)nb * sizeof(float));
        }
}

/*
 * OCP FP4 E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
 * magnitudes 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6; no Inf or NaN.
 */
double oracle_e2m1_decode(uint8_t c)
{
    int e = (c >> 1) & 3, m = c & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (c & 0x8) ? -mag : mag;
}

/*
 * float32 -> E2M1 code (low 4 bits), nearest with ties to the even code,
 * saturating to +-6; the sign is kept (a negative value that rounds to zero
 * gives 0x8).  Same search as the E4M3 encoder, over the 8 magnitudes.
 */
uint8_t oracle_e2m1_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs((double)v), mid;
    int lo = 0, hi = 7, code;
    if (a >= 6.0) return (uint8_t)(sign | 7);
    while (hi - lo > 1) {
        int m = (lo + hi) / 2;
        int below = oracle_e2m1_decode((uint8_t)m) <= a;
        lo = below ? m : lo;
        hi = below ? hi : m;
    }
    mid = 0.5 * (oracle_e2m1_decode((uint8_t)lo) + oracle_e2m1_decode((uint8_t)hi));
    if (a < mid) code = lo;
    else if (a > mid) code = hi;
    else code = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | code);
}

void oracle_e2m1_encode_array(const float *in, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(in[i]);
}

/*
 * MX block scale exponent (R14): e = floor(log2(amax)) - emax, clamped to
 * [-127, 127]; amax == 0 gives -127.  emax is the element format's largest
 * exponent: 8 for E4M3 (448 = 1.75 * 2^8), 2 for E2M1 (6 = 1.5 * 2^2).
 * floor(log2(a)) is frexp's exponent minus one (exact for every finite a).
 */
int oracle_mx_exponent(float amax, int emax)
{
    int fe, e;
    if (!(amax > 0.0f)) return -127;
    (void)frexp((double)amax, &fe);   /* amax = f * 2^fe, f in [0.5, 1) */
    e = (fe - 1) - emax;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/*
 * MX dispatch (R14).  elem_bits 8: MXFP8, recv_x [rows, H] E4M3 codes;
 * elem_bits 4: MXFP4, recv_x [rows, H/2] bytes, column 2i in the low nibble
 * of byte i.  recv_scale [rows, H/32] biased exponents (e + 127).  x / X is
 * a division by a power of two, exact in double and in float for every
 * BF16 x; the quotient is saturated to the element's largest normal and
 * then rounded to the nearest element (a value at or below the largest
 * normal never rounds past it).  H must be a multiple of 32.
 */
void oracle_dispatch_mx(int64_t T, int64_t H, int64_t k, int elem_bits,
                        const uint16_t *x, const int32_t *slot,
                        uint8_t *recv_x, uint8_t *recv_scale)
{
    int64_t t, b, i, j;
    int64_t nb = H / 32;
    int64_t row_bytes = elem_bits == 8 ? H : H / 2;
    int emax = elem_bits == 8 ? 8 : 2;
    double maxnorm = elem_bits == 8 ? 448.0 : 6.0;
    uint8_t *row = (uint8_t *)malloc((size_t)(row_bytes > 0 ? row_bytes : 1));
    uint8_t *scales = (uint8_t *)malloc((size_t)(nb > 0 ? nb : 1));
    if (!row || !scales) { free(row); free(scales); return; }
    for (t = 0; t < T; ++t) {
        for (b = 0; b < nb; ++b) {
            const uint16_t *xb = x + t * H + b * 32;
            float amax = 0.0f;
            int e;
            for (i = 0; i < 32; ++i) {
                float a = fabsf(bf16_to_f32(xb[i]));
                if (a > amax) amax = a;
            }
            e = oracle_mx_exponent(amax, emax);
            scales[b] = (uint8_t)(e + 127);
            for (i = 0; i < 32; ++i) {
                double q = ldexp((double)bf16_to_f32(xb[i]), -e);   /* x / 2^e, exact */
                float qf;
                if (q > maxnorm) q = maxnorm;
                if (q < -maxnorm) q = -maxnorm;
                qf = (float)q;                                       /* exact: a BF16 times 2^-e */
                if (elem_bits == 8) {
                    row[b * 32 + i] = oracle_e4m3_encode(qf);
                } else {
                    uint8_t c = oracle_e2m1_encode(qf);
                    int64_t col = b * 32 + i;
                    if (col % 2 == 0) row[col / 2] = c;
                    else row[col / 2] = (uint8_t)(row[col / 2] | (c << 4));
                }
            }
        }
        for (j = 0; j < k; ++j) {
            int32_t sl = slot[t * k + j];
            if (sl < 0) continue;
            memcpy(recv_x + (int64_t)sl * row_bytes, row, (size_t)row_bytes);
            memcpy(recv_scale + (int64_t)sl * nb, scales, (size_t)nb);
        }
    }
    free(row);
    free(scales);
}
