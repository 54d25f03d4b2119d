/*
 * verify_attn_oracle.c -- plain fp64 CPU oracle for split-KV target-verify
 * attention (speculative decoding, topk = 1).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library and never includes anything from it.
 *
 * What it computes (sglang "verify_splitkv.py", module docstring and the
 * kernels _verify_prefix_stage1 / _verify_combine_stage2): for every sequence
 * b, query head h and draft row i, one softmax over the union of
 *   - every prefix token j < n_b of the paged pool, reached through
 *     kv_indices[kv_indptr[b] + j]; no mask ("full prefix is visible");
 *     score = sm_scale * k_scale * <q_hat, K_pool[t_j, g]>, where q_hat is q
 *     rounded to the pool element type (q cast to the buffer dtype before the
 *     dot), and the value row enters multiplied by v_scale;
 *   - the draft keys j <= i of the same sequence (causal among the drafts);
 *     score = sm_scale * <q, K_ext[j, g]>, no cast and no k/v scale.
 * g = h / (H_Q / H_KV): query heads are grouped contiguously per KV head.
 *
 * The split into ranges, the per-range log-sum-exp and the two-way merge on
 * the pages are a re-association of this single softmax; the oracle does not
 * split.  Everything is evaluated in fp64 from the exact stored bf16 / fp8
 * values.  Readings where the pages are silent:
 *   - fp8 pool format is OCP E4M3FN (bias 7, max 448, no infinities, one NaN
 *     code per sign, subnormals kept);
 *   - the q -> fp8 cast rounds to nearest, ties to even, and saturates to
 *     +-448 (the pages only say the query is converted to the buffer dtype);
 *   - an empty prefix (n_b = 0) gives the draft-only softmax.
 *
 * Tree verify (topk > 1; sglang aiter_backend.py passes custom_mask and
 * mask_indptr with skip_prefix_custom_mask): each sequence's mask is a
 * row-major [n_draft x (n_b + n_draft)] byte array at mask_indptr[b]; the
 * prefix columns are not consulted (the prefix stays fully visible) and draft
 * key j is visible to draft row i where the byte at column n_b + j is nonzero.
 * Without a mask the draft block is causal.  A row that sees no key at all
 * gives output 0 (reading: the pages never build such a row).
 *
 * Also here: the draft K/V append into the pool (aiter_backend.py,
 * set_kv_buffer / launch_reshape_and_cache_flash) and the kv_indices build
 * from req_to_token (create_flashinfer_kv_indices_triton as called there).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Decoded from the format definition, not by reinterpreting a float. */
double oracle_bf16_to_f64(uint16_t bits)
{
    int s = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double v;
    if (e == 0xFF)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m / 128.0, -126);
    else
        v = ldexp(1.0 + (double)m / 128.0, e - 127);
    return s ? -v : v;
}

/* OCP 8-bit floating point, E4M3FN: bias 7; exponent field 0 is subnormal
 * (2^-6 * m/8); field 15 with mantissa 7 is NaN; no infinities. */
double oracle_e4m3fn_to_f64(uint8_t bits)
{
    int s = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round a real to the nearest E4M3FN value, ties to even, saturating at
 * +-448; returns the 8-bit code.  Grid spacing is 2^(k-3) in the binade
 * [2^k, 2^(k+1)) for k >= -6 and 2^-9 below 2^-6 (subnormals). */
uint8_t oracle_f64_to_e4m3fn(double x)
{
    if (isnan(x))
        return 0x7F;
    int s = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint8_t code;
    if (a >= 448.0) {
        code = 0x7E; /* 448 = 2^8 * 1.75 */
    } else if (a == 0.0) {
        code = 0;
    } else {
        int ex;
        frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
        int k = ex - 1;         /* a in [2^k, 2^(k+1)) */
        if (k < -6)
            k = -6;
        double spacing = ldexp(1.0, k - 3);
        double q = a / spacing; /* exact: power-of-two divisor */
        double r = nearbyint(q); /* default rounding mode: ties to even */
        double val = r * spacing;
        if (val >= 448.0) {
            code = 0x7E;
        } else if (val < ldexp(1.0, -6)) {
            code = (uint8_t)(int)(val / ldexp(1.0, -9)); /* subnormal */
        } else {
            int ev;
            double f = frexp(val, &ev); /* val = f * 2^ev */
            int E = ev - 1;             /* val = (2f) * 2^E, 2f in [1,2) */
            int mant = (int)((2.0 * f - 1.0) * 8.0);
            code = (uint8_t)(((E + 7) << 3) | mant);
        }
    }
    return (uint8_t)(code | (s << 7));
}

/* Draft key j visible to draft row i: the row's mask bytes (columns of the
 * draft keys) when a tree mask is given, else causal. */
static int draft_visible(const uint8_t *mask_row, int i, int j)
{
    return mask_row ? mask_row[j] != 0 : j <= i;
}

static double pool_elem(const void *buf, int is_fp8, int64_t off)
{
    if (is_fp8)
        return oracle_e4m3fn_to_f64(((const uint8_t *)buf)[off]);
    return oracle_bf16_to_f64(((const uint16_t *)buf)[off]);
}

/*
 * Full problem.  All strides are in elements; the last dimension of every
 * tensor is contiguous.  q/k_ext/v_ext are bf16 bit patterns; k_buf/v_buf are
 * bf16 bit patterns (kv_is_fp8 = 0) or E4M3FN bytes (kv_is_fp8 = 1).
 *
 * Work is restricted to the (b, h) pairs listed in sel_b/sel_h (n_sel of
 * them) or to all pairs when n_sel <= 0.  Output rows of pairs not selected
 * are left untouched.  out is fp64 [rows, h_q, dv] with strides o_s0, o_s1.
 * Returns 0, or -1 on an argument error or allocation failure.
 */
static int verify_core(
    int bs, int h_q, int h_kv, int d, int dv, int kv_is_fp8,
    const uint16_t *q, int64_t q_s0, int64_t q_s1,
    const uint16_t *k_ext, int64_t ke_s0, int64_t ke_s1,
    const uint16_t *v_ext, int64_t ve_s0, int64_t ve_s1,
    const void *k_buf, int64_t kb_s0, int64_t kb_s1,
    const void *v_buf, int64_t vb_s0, int64_t vb_s1,
    const int32_t *qo_indptr, const int32_t *kv_indptr,
    const int64_t *kv_indices,
    const uint8_t *mask, const int64_t *mask_indptr,
    double sm_scale, double k_scale, double v_scale,
    int n_sel, const int32_t *sel_b, const int32_t *sel_h,
    double *out, int64_t o_s0, int64_t o_s1)
{
    if (bs < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv != 0 || d < 1 || dv < 1)
        return -1;
    const int group = h_q / h_kv;
    const int n_units = (n_sel > 0) ? n_sel : bs * h_q;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int u = 0; u < n_units; ++u) {
        const int b = (n_sel > 0) ? sel_b[u] : u / h_q;
        const int h = (n_sel > 0) ? sel_h[u] : u % h_q;
        const int g = h / group;
        const int64_t row0 = qo_indptr[b];
        const int n_draft = qo_indptr[b + 1] - qo_indptr[b];
        const int64_t kv0 = kv_indptr[b];
        const int64_t n_pre = (int64_t)kv_indptr[b + 1] - kv0;

        double *qv = (double *)malloc(sizeof(double) * (size_t)d);
        double *qh = (double *)malloc(sizeof(double) * (size_t)d);
        double *sc = (double *)malloc(sizeof(double) * (size_t)(n_pre + n_draft + 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!qv || !qh || !sc || !acc) {
            free(qv); free(qh); free(sc); free(acc);
            failed |= 1;
            continue;
        }

        for (int i = 0; i < n_draft; ++i) {
            const int64_t r = row0 + i;
            const uint8_t *mrow =
                mask ? mask + mask_indptr[b] + (int64_t)i * (n_pre + n_draft) + n_pre : NULL;
            /* query row, and its copy rounded to the pool element type */
            for (int c = 0; c < d; ++c) {
                qv[c] = oracle_bf16_to_f64(q[r * q_s0 + (int64_t)h * q_s1 + c]);
                qh[c] = kv_is_fp8 ? oracle_e4m3fn_to_f64(oracle_f64_to_e4m3fn(qv[c])) : qv[c];
            }
            /* prefix scores: unmasked, k_scale on the score */
            double mx = -INFINITY;
            for (int64_t j = 0; j < n_pre; ++j) {
                const int64_t t = kv_indices[kv0 + j];
                double dot = 0.0;
                for (int c = 0; c < d; ++c)
                    dot += qh[c] * pool_elem(k_buf, kv_is_fp8, t * kb_s0 + (int64_t)g * kb_s1 + c);
                sc[j] = sm_scale * k_scale * dot;
                if (sc[j] > mx) mx = sc[j];
            }
            /* draft scores: visible draft keys (causal: j <= i), unscaled, uncast */
            for (int j = 0; j < n_draft; ++j) {
                if (!draft_visible(mrow, i, j))
                    continue;
                double dot = 0.0;
                for (int c = 0; c < d; ++c)
                    dot += qv[c] * oracle_bf16_to_f64(k_ext[(row0 + j) * ke_s0 + (int64_t)g * ke_s1 + c]);
                sc[n_pre + j] = sm_scale * dot;
                if (sc[n_pre + j] > mx) mx = sc[n_pre + j];
            }
            /* one softmax over prefix and draft keys */
            double z = 0.0;
            for (int c = 0; c < dv; ++c) acc[c] = 0.0;
            for (int64_t j = 0; j < n_pre; ++j) {
                const int64_t t = kv_indices[kv0 + j];
                const double w = exp(sc[j] - mx);
                z += w;
                for (int c = 0; c < dv; ++c)
                    acc[c] += w * v_scale * pool_elem(v_buf, kv_is_fp8, t * vb_s0 + (int64_t)g * vb_s1 + c);
            }
            for (int j = 0; j < n_draft; ++j) {
                if (!draft_visible(mrow, i, j))
                    continue;
                const double w = exp(sc[n_pre + j] - mx);
                z += w;
                for (int c = 0; c < dv; ++c)
                    acc[c] += w * oracle_bf16_to_f64(v_ext[(row0 + j) * ve_s0 + (int64_t)g * ve_s1 + c]);
            }
            for (int c = 0; c < dv; ++c)
                out[r * o_s0 + (int64_t)h * o_s1 + c] = z > 0.0 ? acc[c] / z : 0.0;
        }
        free(qv); free(qh); free(sc); free(acc);
    }
    return failed ? -1 : 0;
}

/* Causal draft block (topk = 1). */
int oracle_verify_attn(
    int bs, int h_q, int h_kv, int d, int dv, int kv_is_fp8,
    const uint16_t *q, int64_t q_s0, int64_t q_s1,
    const uint16_t *k_ext, int64_t ke_s0, int64_t ke_s1,
    const uint16_t *v_ext, int64_t ve_s0, int64_t ve_s1,
    const void *k_buf, int64_t kb_s0, int64_t kb_s1,
    const void *v_buf, int64_t vb_s0, int64_t vb_s1,
    const int32_t *qo_indptr, const int32_t *kv_indptr,
    const int64_t *kv_indices,
    double sm_scale, double k_scale, double v_scale,
    int n_sel, const int32_t *sel_b, const int32_t *sel_h,
    double *out, int64_t o_s0, int64_t o_s1)
{
    return verify_core(bs, h_q, h_kv, d, dv, kv_is_fp8, q, q_s0, q_s1, k_ext, ke_s0, ke_s1,
                       v_ext, ve_s0, ve_s1, k_buf, kb_s0, kb_s1, v_buf, vb_s0, vb_s1,
                       qo_indptr, kv_indptr, kv_indices, NULL, NULL, sm_scale, k_scale, v_scale,
                       n_sel, sel_b, sel_h, out, o_s0, o_s1);
}

/* Tree-masked draft block: mask / mask_indptr as described at the top. */
int oracle_verify_attn_masked(
    int bs, int h_q, int h_kv, int d, int dv, int kv_is_fp8,
    const uint16_t *q, int64_t q_s0, int64_t q_s1,
    const uint16_t *k_ext, int64_t ke_s0, int64_t ke_s1,
    const uint16_t *v_ext, int64_t ve_s0, int64_t ve_s1,
    const void *k_buf, int64_t kb_s0, int64_t kb_s1,
    const void *v_buf, int64_t vb_s0, int64_t vb_s1,
    const int32_t *qo_indptr, const int32_t *kv_indptr,
    const int64_t *kv_indices,
    const uint8_t *mask, const int64_t *mask_indptr,
    double sm_scale, double k_scale, double v_scale,
    int n_sel, const int32_t *sel_b, const int32_t *sel_h,
    double *out, int64_t o_s0, int64_t o_s1)
{
    if (!mask || !mask_indptr)
        return -1;
    return verify_core(bs, h_q, h_kv, d, dv, kv_is_fp8, q, q_s0, q_s1, k_ext, ke_s0, ke_s1,
                       v_ext, ve_s0, ve_s1, k_buf, kb_s0, kb_s1, v_buf, vb_s0, vb_s1,
                       qo_indptr, kv_indptr, kv_indices, mask, mask_indptr, sm_scale, k_scale,
                       v_scale, n_sel, sel_b, sel_h, out, o_s0, o_s1);
}

/*
 * Draft K/V append (aiter_backend.py: set_kv_buffer, and
 * launch_reshape_and_cache_flash, which fuses the bf16 -> fp8 cast with the
 * paged write): row i of k [n, h_kv, d] / v [n, h_kv, dv] (bf16) goes to pool
 * row loc[i] of every head.  A bf16 pool receives the bits unchanged; an fp8
 * pool receives the E4M3FN code of x / scale, the quotient formed in fp32
 * (x and scale as fp32, one correctly rounded division), then rounded to
 * nearest, ties to even, saturating at +-448 (reading: the pages give the cast
 * but not its overflow rule; saturation keeps a NaN out of the cache).  Rows
 * of the pool not named by loc are untouched; a row named twice keeps the
 * last write (i order).  Strides are in elements.  Returns 0.
 */
int oracle_append_kv(
    int64_t n, int h_kv, int d, int dv, int kv_is_fp8,
    const uint16_t *k, int64_t k_s0, int64_t k_s1,
    const uint16_t *v, int64_t v_s0, int64_t v_s1,
    const int64_t *loc, float k_scale, float v_scale,
    void *k_buf, int64_t kb_s0, int64_t kb_s1,
    void *v_buf, int64_t vb_s0, int64_t vb_s1)
{
    for (int64_t i = 0; i < n; ++i) {
        const int64_t t = loc[i];
        for (int g = 0; g < h_kv; ++g) {
            for (int c = 0; c < d; ++c) {
                const uint16_t x = k[i * k_s0 + (int64_t)g * k_s1 + c];
                const int64_t off = t * kb_s0 + (int64_t)g * kb_s1 + c;
                if (kv_is_fp8) {
                    const float y = (float)oracle_bf16_to_f64(x) / k_scale;
                    ((uint8_t *)k_buf)[off] = oracle_f64_to_e4m3fn((double)y);
                } else {
                    ((uint16_t *)k_buf)[off] = x;
                }
            }
            for (int c = 0; c < dv; ++c) {
                const uint16_t x = v[i * v_s0 + (int64_t)g * v_s1 + c];
                const int64_t off = t * vb_s0 + (int64_t)g * vb_s1 + c;
                if (kv_is_fp8) {
                    const float y = (float)oracle_bf16_to_f64(x) / v_scale;
                    ((uint8_t *)v_buf)[off] = oracle_f64_to_e4m3fn((double)y);
                } else {
                    ((uint16_t *)v_buf)[off] = x;
                }
            }
        }
    }
    return 0;
}

/*
 * kv_indices from the request-to-token table (aiter_backend.py builds
 * kv_indptr as the running sum of the per-request lengths and then calls
 * create_flashinfer_kv_indices_triton with them): for request b and
 * i < seq_lens[b],
 *   kv_indices[kv_indptr[b] + i] = req_to_token[req_pool_indices[b] * stride
 *                                               + start_b + i],
 * start_b = kv_start_idx[b], or 0 when kv_start_idx is NULL.  kv_indptr
 * (bs + 1 entries, kv_indptr[0] = 0) is written too.  Returns 0.
 */
int oracle_build_kv_indices(
    int bs, const int32_t *req_to_token, int64_t stride, const int64_t *req_pool_indices,
    const int32_t *seq_lens, const int32_t *kv_start_idx, int32_t *kv_indptr, int64_t *kv_indices)
{
    kv_indptr[0] = 0;
    for (int b = 0; b < bs; ++b)
        kv_indptr[b + 1] = kv_indptr[b] + seq_lens[b];
    for (int b = 0; b < bs; ++b) {
        const int64_t base = req_pool_indices[b] * stride + (kv_start_idx ? kv_start_idx[b] : 0);
        for (int32_t i = 0; i < seq_lens[b]; ++i)
            kv_indices[kv_indptr[b] + i] = req_to_token[base + i];
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n <= 0: all processors); returns the count
 * now in effect.  Only the timing of the oracle changes. */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
