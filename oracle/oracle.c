/*
 * CPU oracle for the MoE indirect matrix multiplication (mul_mat_id).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file or the library built from it; only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg do. It shares no code, header, table or
 * helper with the GPU library.
 *
 * What it computes is the plain definition of the operation, in float64, with a
 * fixed summation order and nothing blocked, fused or reordered:
 *
 *  - The op has three inputs: stacked expert weights, activations, and an integer
 *    ids table naming which experts each token uses; each token is multiplied only
 *    by the weight matrices of the experts the ids name for it
 *    ("CUDA: better MoE implementation" (ik_llama.cpp PR #283 write-up), section 1.2).
 *  - The fast path first builds three maps from ids -- a reordering of the
 *    flattened src1 rows so rows are grouped by expert, the same reordering
 *    applied to dst, and each expert's bounds in the reordered buffer -- and then
 *    does the reorder and reduction by those maps (same page, section 2.1 and
 *    the summary in section 6). Here the maps are built by plain enumeration.
 *  - Experts may be Q8_0-quantized (section 2.1 names Q8_0): blocks of 32 int8
 *    values sharing one fp16 scale, value = d * q. Dequantization is exact in
 *    float64 (an 11-bit by 8-bit product).
 *  - Experts may be MXFP4 (the TensorSharp MoE-offload page lists GPT-OSS 20B as
 *    "Q8_0 / MXFP4"; the pages do not define the format, so it is taken from the
 *    OCP Microscaling (MX) v1.0 specification): blocks of 32 FP4 E2M1 elements
 *    sharing one E8M0 scale, value = fp4(code) * 2^(scale - 127). Exact in float64.
 *  - Experts may be IQ4_NL, the 4-bit member of the IQ series the pages name (the
 *    TensorSharp MoE-offload page's models ship as UD-IQ4_XS, whose 4-bit codes are
 *    IQ4_NL's; the ik_llama.cpp write-up, section 3.2, runs IQ2_K_R4). The pages do
 *    not define the format, so it is taken from ggml's definition of IQ4_NL: blocks
 *    of 32 4-bit indices into a fixed non-uniform table of 16 signed integers, one
 *    fp16 scale per block, value = d * table[code]. Exact in float64.
 *  - Experts may be IQ4_XS (the type of those UD-IQ4_XS models), also from ggml's
 *    definition: IQ4_NL's codes and levels in super-blocks of 256 weights that share
 *    one fp16 scale d, each block of 32 carrying a 6-bit sub-scale ls (its low 4 bits
 *    in a nibble of scales_l, its high 2 bits in scales_h); value = d * (ls - 32) *
 *    level[code]. Exact in float64.
 *  - The fused MoE FFN applies gate and up projections, SiLU(gate) * up, then the
 *    down projection (section 4.2 names the fused up/gate MoE forward), weights each
 *    routed slot's result by its routing weight and adds always-on shared experts,
 *    which are computed in the same operation ("CUDA: fuse shared experts into
 *    MMVQ", release b11370; the TensorSharp MoE-offload page lists the shared
 *    expert among the tensors that stay on the accelerator).
 *
 * Readings where the pages are silent (stated once here, used below):
 *  - Weights are row-major W[E][rows][cols] (ggml ne order, fastest dimension last
 *    here); Q8_0 scales are a separate fp16 array d[E][rows][cols/32].
 *  - src1 is [T][B][K] with B = 1 (every slot reads the token's row) or B = k (one
 *    row per slot); ids is [T][k].
 *  - Inside an expert segment, rows are ordered by token index then slot index.
 *  - An id outside [0, E) selects no expert: that slot's output row is zero and it
 *    contributes nothing; its map entries go after all expert segments, in
 *    (token, slot) order, so the maps stay a permutation.
 *  - SiLU(z) = z / (1 + exp(-z)); shared experts have weight 1 and are added after
 *    the routed slots, in index order.
 *
 * Types: 0 = float32, 1 = bfloat16 (uint16 bit pattern), 2 = Q8_0 (int8 + fp16),
 * 3 = MXFP4 (two 4-bit codes per byte + one uint8 E8M0 scale per 32 elements). MXFP4
 * storage (a reading; the pages fix none): codes [E][rows][cols/2] bytes, element 2i
 * of a row in bits 0-3 of byte i and element 2i+1 in bits 4-7; scales [E][rows][cols/32].
 * 4 = IQ4_NL: codes packed exactly as MXFP4's (a reading: ggml's own block packs the
 * low nibbles of a block's 16 bytes first; only the values are the format's), with
 * fp16 scales d[E][rows][cols/32] as for Q8_0.
 * 5 = IQ4_XS: codes as IQ4_NL's; per super-block of 256 columns one 8-byte record in
 * scales[E][rows][cols/256][8]: fp16 d (bytes 0-1), uint16 scales_h (bytes 2-3; bits
 * 2j, 2j+1 are the high bits of block j's ls), uint8 scales_l[4] (bytes 4-7; byte j/2,
 * nibble j%2 (low first) holds the low 4 bits of block j's ls), ggml's field order
 * without the codes. cols % 256 == 0.
 * All entry points return 0 on success and a negative value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_Q8_0 2
#define OR_MXFP4 3
#define OR_IQ4_NL 4
#define OR_IQ4_XS 5

/* IQ4_NL's 16 levels, index = the 4-bit code: ggml's non-linear table for the type
 * (kvalues_iq4nl in ggml-common.h). */
static const int8_t iq4nl_levels[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                        1,    13,   25,  38,  53,  69,  89,  113};

/* Level of one IQ4_NL code (0..15), as a double; other inputs return NaN. */
double oracle_iq4nl_level(int code) {
    if (code < 0 || code > 15) return NAN;
    return (double)iq4nl_levels[code];
}

/* IEEE binary16 -> double, written from the format's definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits). */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24); /* subnormal: fr * 2^-14 * 2^-10 */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr + 1024), ex - 25); /* (1 + fr/1024) * 2^(ex-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double: the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* FP4 E2M1 code -> double, from the format's definition: bit 3 sign, bits 2-1 exponent
 * with bias 1, bit 0 mantissa; exponent 0 is subnormal (mantissa * 2^-1), otherwise
 * (1 + mantissa/2) * 2^(exponent - 1). No infinities or NaN. */
double oracle_e2m1_to_double(int code) {
    int sign = (code >> 3) & 1;
    int ex = (code >> 1) & 3;
    int m = code & 1;
    double v = ex == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, ex - 1);
    return sign ? -v : v;
}

/* E8M0 scale -> double: 2^(x - 127); x = 255 encodes NaN. */
double oracle_e8m0_to_double(int x) {
    if ((x & 0xff) == 255) return NAN;
    return ldexp(1.0, (x & 0xff) - 127);
}

static int is_quant(int type) {
    return type == OR_Q8_0 || type == OR_MXFP4 || type == OR_IQ4_NL || type == OR_IQ4_XS;
}
/* columns per scale unit of a quantized type (IQ4_XS: its super-block) */
static int64_t quant_cols(int type) { return type == OR_IQ4_XS ? 256 : 32; }

/* IQ4_XS: the scale of block j (0..7) of one super-block record, as a double. */
double oracle_iq4xs_block_scale(const uint8_t *rec, int j) {
    uint16_t d = (uint16_t)(rec[0] | (rec[1] << 8));
    unsigned sh = (unsigned)(rec[2] | (rec[3] << 8));
    int lo = (rec[4 + j / 2] >> (4 * (j % 2))) & 15;
    int hi = (sh >> (2 * j)) & 3;
    return oracle_half_to_double(d) * (double)((lo | (hi << 4)) - 32);
}

/* One weight element w(e, n, c) of a stacked matrix, as a double. */
static double weight_at(int type, const void *data, const void *scales, int64_t rows,
                        int64_t cols, int64_t e, int64_t n, int64_t c) {
    int64_t idx = (e * rows + n) * cols + c;
    if (type == OR_F32) return (double)((const float *)data)[idx];
    if (type == OR_MXFP4) {
        /* two codes per byte, the even column in the low nibble; one E8M0 scale per
         * 32 consecutive columns of a row */
        uint8_t b = ((const uint8_t *)data)[(e * rows + n) * (cols / 2) + c / 2];
        int code = (c & 1) ? (b >> 4) : (b & 15);
        uint8_t x = ((const uint8_t *)scales)[(e * rows + n) * (cols / 32) + c / 32];
        return oracle_e2m1_to_double(code) * oracle_e8m0_to_double(x);
    }
    if (type == OR_IQ4_NL) {
        /* codes packed as MXFP4's; value = d * level, one fp16 d per 32 columns */
        uint8_t b = ((const uint8_t *)data)[(e * rows + n) * (cols / 2) + c / 2];
        int code = (c & 1) ? (b >> 4) : (b & 15);
        uint16_t d = ((const uint16_t *)scales)[(e * rows + n) * (cols / 32) + c / 32];
        return oracle_half_to_double(d) * oracle_iq4nl_level(code);
    }
    if (type == OR_IQ4_XS) {
        /* codes packed as MXFP4's; value = (block scale) * level */
        uint8_t b = ((const uint8_t *)data)[(e * rows + n) * (cols / 2) + c / 2];
        int code = (c & 1) ? (b >> 4) : (b & 15);
        const uint8_t *rec = (const uint8_t *)scales + ((e * rows + n) * (cols / 256) + c / 256) * 8;
        return oracle_iq4xs_block_scale(rec, (int)((c % 256) / 32)) * oracle_iq4nl_level(code);
    }
    /* Q8_0: value = d * q, one fp16 scale per 32 consecutive columns of a row. */
    int8_t q = ((const int8_t *)data)[idx];
    uint16_t d = ((const uint16_t *)scales)[(e * rows + n) * (cols / 32) + c / 32];
    return oracle_half_to_double(d) * (double)q;
}

/* Activation element as a double. */
static double act_at(int type, const void *src, int64_t idx) {
    if (type == OR_F32) return (double)((const float *)src)[idx];
    return oracle_bf16_to_double(((const uint16_t *)src)[idx]);
}

/* Dequantize (or widen) a whole stack of matrices into out[n_mat*rows*cols]. */
int oracle_dequant(int type, const void *data, const void *scales, int64_t n_mat, int64_t rows,
                   int64_t cols, double *out) {
    if (!data || !out || (type != OR_F32 && !is_quant(type))) return -1;
    if (is_quant(type) && (!scales || cols % quant_cols(type))) return -1;
    for (int64_t e = 0; e < n_mat; e++)
        for (int64_t n = 0; n < rows; n++)
            for (int64_t c = 0; c < cols; c++)
                out[(e * rows + n) * cols + c] = weight_at(type, data, scales, rows, cols, e, n, c);
    return 0;
}

/*
 * The three maps of section 2.1, built by enumeration:
 *   for each expert e ascending: bounds[e] = running count; then every (t, s) with
 *   ids[t][s] == e, t ascending then s ascending, takes the next slot j, with
 *   ids_src1[j] = t*B + (s mod B) (the src1 row it reads) and ids_dst[j] = t*k + s
 *   (the dst row it writes).
 *   bounds[E] = number of valid entries; entries with ids outside [0, E) follow.
 */
int oracle_row_ids(const int32_t *ids, int64_t T, int32_t k, int32_t E, int32_t B,
                   int32_t *ids_src1, int32_t *ids_dst, int32_t *bounds) {
    if (!ids || !ids_src1 || !ids_dst || !bounds || T < 0 || k <= 0 || E <= 0) return -1;
    if (B != 1 && B != k) return -1;
    int64_t j = 0;
    for (int32_t e = 0; e < E; e++) {
        bounds[e] = (int32_t)j;
        for (int64_t t = 0; t < T; t++)
            for (int32_t s = 0; s < k; s++)
                if (ids[t * k + s] == e) {
                    ids_src1[j] = (int32_t)(t * B + s % B);
                    ids_dst[j] = (int32_t)(t * k + s);
                    j++;
                }
    }
    bounds[E] = (int32_t)j;
    for (int64_t t = 0; t < T; t++)
        for (int32_t s = 0; s < k; s++) {
            int32_t e = ids[t * k + s];
            if (e < 0 || e >= E) {
                ids_src1[j] = (int32_t)(t * B + s % B);
                ids_dst[j] = (int32_t)(t * k + s);
                j++;
            }
        }
    return 0;
}

/*
 * y[n] = sum over c ascending of w(e, n, c) * a[c], for n in [0, rows).
 * Each weight is formed as d * q (exact) before it multiplies a[c]; four rows are
 * accumulated side by side only to keep the CPU busy -- every row still has its
 * own accumulator and its own ascending-c order.
 */
static void matvec(int type, const void *data, const void *scales, int64_t rows, int64_t cols,
                   int64_t e, const double *a, double *y) {
    int64_t n = 0;
    if (type == OR_F32) {
        const float *w = (const float *)data + e * rows * cols;
        for (; n < rows; n++) {
            const float *wr = w + n * cols;
            double acc = 0.0;
            for (int64_t c = 0; c < cols; c++) acc += (double)wr[c] * a[c];
            y[n] = acc;
        }
        return;
    }
    if (type == OR_MXFP4 || type == OR_IQ4_NL || type == OR_IQ4_XS) {
        for (; n < rows; n++) {
            double acc = 0.0;
            for (int64_t c = 0; c < cols; c++) acc += weight_at(type, data, scales, rows, cols, e, n, c) * a[c];
            y[n] = acc;
        }
        return;
    }
    const int8_t *q = (const int8_t *)data + e * rows * cols;
    const uint16_t *ds = (const uint16_t *)scales + e * rows * (cols / 32);
    int64_t nb = cols / 32;
    for (; n + 4 <= rows; n += 4) {
        const int8_t *q0 = q + n * cols, *q1 = q0 + cols, *q2 = q1 + cols, *q3 = q2 + cols;
        const uint16_t *d0 = ds + n * nb, *d1 = d0 + nb, *d2 = d1 + nb, *d3 = d2 + nb;
        double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            double s0 = oracle_half_to_double(d0[b]), s1 = oracle_half_to_double(d1[b]);
            double s2 = oracle_half_to_double(d2[b]), s3 = oracle_half_to_double(d3[b]);
            for (int64_t c = b * 32; c < b * 32 + 32; c++) {
                acc0 += (s0 * (double)q0[c]) * a[c];
                acc1 += (s1 * (double)q1[c]) * a[c];
                acc2 += (s2 * (double)q2[c]) * a[c];
                acc3 += (s3 * (double)q3[c]) * a[c];
            }
        }
        y[n] = acc0;
        y[n + 1] = acc1;
        y[n + 2] = acc2;
        y[n + 3] = acc3;
    }
    for (; n < rows; n++) {
        const int8_t *qr = q + n * cols;
        const uint16_t *dr = ds + n * nb;
        double acc = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            double sc = oracle_half_to_double(dr[b]);
            for (int64_t c = b * 32; c < b * 32 + 32; c++) acc += (sc * (double)qr[c]) * a[c];
        }
        y[n] = acc;
    }
}

/*
 * mul_mat_id (section 1.2): dst[t][s][n] = sum_c W[ids[t][s]][n][c] * src1[t][s mod B][c],
 * c ascending, in float64; a slot whose id is outside [0, E) gives a zero row.
 * With route_w, the per-slot rows are combined: dst[t][n] = sum over s ascending of
 * route_w[t][s] * (per-slot row).
 * Weights: n_mat = E, rows = N, cols = K.
 */
int oracle_mul_mat_id(int w_type, const void *w_data, const void *w_scales, int64_t E, int64_t N,
                      int64_t K, const void *src1, int src1_type, int32_t B, const int32_t *ids,
                      int64_t T, int32_t k, const float *route_w, double *dst) {
    if (!w_data || !src1 || !ids || !dst || E <= 0 || N <= 0 || K <= 0 || T < 0 || k <= 0) return -1;
    if (w_type != OR_F32 && !is_quant(w_type)) return -1;
    if (is_quant(w_type) && (!w_scales || K % quant_cols(w_type))) return -1;
    if (src1_type != OR_F32 && src1_type != OR_BF16) return -1;
    if (B != 1 && B != k) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < T; t++) {
        double *a = (double *)malloc(sizeof(double) * (size_t)K);
        double *y = (double *)malloc(sizeof(double) * (size_t)N);
        if (!a || !y) {
            bad = 1;
            free(a);
            free(y);
            continue;
        }
        double *out_t = dst + t * (route_w ? N : (int64_t)k * N);
        if (route_w)
            for (int64_t n = 0; n < N; n++) out_t[n] = 0.0;
        for (int32_t s = 0; s < k; s++) {
            int32_t e = ids[t * k + s];
            double *row = route_w ? y : out_t + (int64_t)s * N;
            if (e < 0 || e >= E) {
                if (!route_w)
                    for (int64_t n = 0; n < N; n++) row[n] = 0.0;
                continue;
            }
            int64_t r = t * B + s % B;
            for (int64_t c = 0; c < K; c++) a[c] = act_at(src1_type, src1, r * K + c);
            matvec(w_type, w_data, w_scales, N, K, e, a, row);
            if (route_w) {
                double wt = (double)route_w[t * k + s];
                for (int64_t n = 0; n < N; n++) out_t[n] += wt * y[n];
            }
        }
        free(a);
        free(y);
    }
    return bad ? -2 : 0;
}

/* One expert's FFN on one activation vector: y = Wd (silu(Wg x) * (Wu x)). */
static void expert_ffn(int type, const void *g_data, const void *g_scales, const void *u_data,
                       const void *u_scales, const void *d_data, const void *d_scales, int64_t n_ff,
                       int64_t n_embd, int64_t e, const double *x, double *g, double *u,
                       double *y) {
    matvec(type, g_data, g_scales, n_ff, n_embd, e, x, g);
    matvec(type, u_data, u_scales, n_ff, n_embd, e, x, u);
    for (int64_t i = 0; i < n_ff; i++) g[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
    matvec(type, d_data, d_scales, n_embd, n_ff, e, g, y);
}

/*
 * Fused MoE FFN: for each token t, for s ascending with e = ids[t][s] in [0, E):
 *   out[t] += route_w[t][s] * Wd_e (silu(Wg_e x_t) * (Wu_e x_t));
 * then for each shared expert j ascending: out[t] += Sd_j (silu(Sg_j x_t) * (Su_j x_t)).
 * Routed gate/up: [E][n_ff][n_embd]; routed down: [E][n_embd][n_ff].
 * Shared gate/up: [S][n_ff_sh][n_embd]; shared down: [S][n_embd][n_ff_sh]. S may be 0.
 */
int oracle_ffn(int w_type, const void *g_data, const void *g_scales, const void *u_data,
               const void *u_scales, const void *d_data, const void *d_scales, int64_t E,
               int64_t n_ff, int64_t n_embd, const void *sg_data, const void *sg_scales,
               const void *su_data, const void *su_scales, const void *sd_data,
               const void *sd_scales, int64_t S, int64_t n_ff_sh, const void *x, int x_type,
               const int32_t *ids, const float *route_w, int64_t T, int32_t k, double *out) {
    if (!g_data || !u_data || !d_data || !x || !ids || !route_w || !out) return -1;
    if (E <= 0 || n_ff <= 0 || n_embd <= 0 || T < 0 || k <= 0 || S < 0) return -1;
    if (w_type != OR_F32 && !is_quant(w_type)) return -1;
    if (x_type != OR_F32 && x_type != OR_BF16) return -1;
    if (is_quant(w_type) && (!g_scales || !u_scales || !d_scales || n_embd % quant_cols(w_type) ||
                              n_ff % quant_cols(w_type)))
        return -1;
    if (S > 0 && (!sg_data || !su_data || !sd_data || n_ff_sh <= 0)) return -1;
    if (S > 0 && is_quant(w_type) && (!sg_scales || !su_scales || !sd_scales || n_ff_sh % quant_cols(w_type)))
        return -1;
    int64_t ffmax = n_ff > n_ff_sh ? n_ff : n_ff_sh;
    int bad = 0;
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < T; t++) {
        double *xv = (double *)malloc(sizeof(double) * (size_t)n_embd);
        double *g = (double *)malloc(sizeof(double) * (size_t)ffmax);
        double *u = (double *)malloc(sizeof(double) * (size_t)ffmax);
        double *y = (double *)malloc(sizeof(double) * (size_t)n_embd);
        if (!xv || !g || !u || !y) {
            bad = 1;
            free(xv);
            free(g);
            free(u);
            free(y);
            continue;
        }
        double *o = out + t * n_embd;
        for (int64_t c = 0; c < n_embd; c++) {
            xv[c] = act_at(x_type, x, t * n_embd + c);
            o[c] = 0.0;
        }
        for (int32_t s = 0; s < k; s++) {
            int32_t e = ids[t * k + s];
            if (e < 0 || e >= E) continue;
            expert_ffn(w_type, g_data, g_scales, u_data, u_scales, d_data, d_scales, n_ff, n_embd,
                       e, xv, g, u, y);
            double wt = (double)route_w[t * k + s];
            for (int64_t c = 0; c < n_embd; c++) o[c] += wt * y[c];
        }
        for (int64_t j = 0; j < S; j++) {
            expert_ffn(w_type, sg_data, sg_scales, su_data, su_scales, sd_data, sd_scales, n_ff_sh,
                       n_embd, j, xv, g, u, y);
            for (int64_t c = 0; c < n_embd; c++) o[c] += y[c];
        }
        free(xv);
        free(g);
        free(u);
        free(y);
    }
    return bad ? -2 : 0;
}

/* Router (the step ahead of the indirect matmul): for each token pick the n_used
 * experts with the largest logits and weight them by a softmax over the picked
 * logits alone. The pages' op takes ids as given ("CUDA: better MoE implementation",
 * section 1.2: ids names the experts each token uses); the weights follow the
 * softmax renormalised over the picks.
 *
 * Order: picks are made one at a time, each the largest remaining logit, equal
 * logits going to the lower expert index, so the order inside a token is descending
 * logit. NaN ranks strictly below every number, -inf included; NaNs among
 * themselves go lower index first.
 *
 * Weights (a reading: the pages define no weights for non-finite logits): a NaN pick
 * counts as -inf. With v_0 the first (largest) pick:
 *   v_0 finite:   w_r = exp(v_r - v_0) / sum_q exp(v_q - v_0)   (-inf picks get 0);
 *   v_0 = +-inf:  the softmax's limit -- the c picks equal to v_0 get 1/c each, the
 *                 rest 0 (all picks -inf or NaN: every pick gets 1/k).
 * ids int32[T][k], w float64[T][k]. */

/* Rank key of a logit: 0 for NaN, 1 for every number (compared first). */
static int router_rank_class(float x) { return isnan(x) ? 0 : 1; }

int oracle_router_topk(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *ids,
                       double *w) {
    if (!logits || !ids || !w || T < 0 || E <= 0 || k <= 0 || k > E) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        double *v = (double *)malloc(sizeof(double) * (size_t)k);
        for (int32_t r = 0; r < k; r++) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0) {
                    best = e;
                    continue;
                }
                /* strictly better only: ties keep the lower index (found first) */
                int ce = router_rank_class(l[e]), cb = router_rank_class(l[best]);
                if (ce > cb || (ce == 1 && cb == 1 && l[e] > l[best])) best = e;
            }
            taken[best] = 1;
            ids[t * k + r] = best;
            v[r] = isnan(l[best]) ? -INFINITY : (double)l[best];
        }
        double m = v[0];
        if (isfinite(m)) {
            double sum = 0.0;
            for (int32_t r = 0; r < k; r++) sum += exp(v[r] - m);
            for (int32_t r = 0; r < k; r++) w[t * k + r] = exp(v[r] - m) / sum;
        } else {
            int32_t c = 0;
            for (int32_t r = 0; r < k; r++) c += v[r] == m;
            for (int32_t r = 0; r < k; r++) w[t * k + r] = v[r] == m ? 1.0 / c : 0.0;
        }
        free(taken);
        free(v);
    }
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Quantized-activation path (the MMQ-style path: "CUDA: better MoE implementation",
 * section 2.1, names mmq_id, the grouped product of quantized experts with quantized
 * activations; the pages do not define the activation format, so it is a reading):
 *
 *   Each activation row is cut into blocks of 32 consecutive columns. A block's values
 *   x (bf16 or fp32, widened exactly to fp32) get one float32 scale
 *       d = max|x| / 127            (fp32 division, rounded to nearest-even)
 *   and int8 codes
 *       q = rint(x / d)             (fp32 division, then round to the nearest integer,
 *                                    ties to even; clamped to [-127, 127])
 *   A block of zeros has d = 0 and q = 0. The block's value is d * q.
 *
 *   The decisions are taken in float32 (the precision stated above), so any side that
 *   follows the same float32 operations reaches the same codes. Activations must be
 *   finite.
 */

/* bf16 RNE of a double, in one rounding: keep 8 significant bits. */
static double round_to_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    double m = frexp(v, &e);           /* v = m * 2^e, 0.5 <= |m| < 1 */
    double r = nearbyint(ldexp(m, 8)); /* 8 significant bits, ties to even */
    return ldexp(r, e - 8);
}

/* One block of n <= 32 float32 values -> codes and scale, as defined above. */
static void quantize_block(const float *x, int n, int8_t *q, float *d) {
    float amax = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    volatile float dv = amax / 127.0f; /* float32 division, not contracted or widened */
    float dd = dv;
    *d = dd;
    for (int i = 0; i < n; i++) {
        if (dd == 0.0f) {
            q[i] = 0;
            continue;
        }
        volatile float t = x[i] / dd;
        float r = rintf(t);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
}

/* Quantize rows x[rows][K] (type 0 float32, 1 bf16 bits) into q int8 [rows][K] and
 * d float32 [rows][K/32]. K % 32 == 0. */
int oracle_quantize_act(int type, const void *x, int64_t rows, int64_t K, int8_t *q, float *d) {
    if (!x || !q || !d || rows < 0 || K <= 0 || K % 32) return -1;
    if (type != OR_F32 && type != OR_BF16) return -1;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < K / 32; b++) {
            float blk[32];
            for (int i = 0; i < 32; i++) blk[i] = (float)act_at(type, x, r * K + b * 32 + i);
            quantize_block(blk, 32, q + r * K + b * 32, d + r * (K / 32) + b);
        }
    return 0;
}

/* Dequantized quantized-activation row: out[c] = d[c/32] * q[c], exact in float64. */
static void q8act_row(const int8_t *q, const float *d, int64_t K, double *out) {
    for (int64_t c = 0; c < K; c++) out[c] = (double)d[c / 32] * (double)q[c];
}

/*
 * mul_mat_id on quantized activations: as oracle_mul_mat_id (section 1.2 of the same
 * page), with slot (t, s) reading the quantized row t*B + (s mod B) of (q, d):
 *   dst[t][s][n] = sum_c w(ids[t][s], n, c) * d[row][c/32] * q[row][c], c ascending.
 */
int oracle_mul_mat_id_q8act(int w_type, const void *w_data, const void *w_scales, int64_t E,
                            int64_t N, int64_t K, const int8_t *q, const float *d, int32_t B,
                            const int32_t *ids, int64_t T, int32_t k, const float *route_w,
                            double *dst) {
    if (!w_data || !q || !d || !ids || !dst || E <= 0 || N <= 0 || K <= 0 || T < 0 || k <= 0)
        return -1;
    if (!is_quant(w_type) || !w_scales || K % quant_cols(w_type)) return -1;
    if (B != 1 && B != k) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < T; t++) {
        double *a = (double *)malloc(sizeof(double) * (size_t)K);
        double *y = (double *)malloc(sizeof(double) * (size_t)N);
        if (!a || !y) {
            bad = 1;
            free(a);
            free(y);
            continue;
        }
        double *out_t = dst + t * (route_w ? N : (int64_t)k * N);
        if (route_w)
            for (int64_t n = 0; n < N; n++) out_t[n] = 0.0;
        for (int32_t s = 0; s < k; s++) {
            int32_t e = ids[t * k + s];
            double *row = route_w ? y : out_t + (int64_t)s * N;
            if (e < 0 || e >= E) {
                if (!route_w)
                    for (int64_t n = 0; n < N; n++) row[n] = 0.0;
                continue;
            }
            int64_t r = t * B + s % B;
            q8act_row(q + r * K, d + r * (K / 32), K, a);
            matvec(w_type, w_data, w_scales, N, K, e, a, row);
            if (route_w) {
                double wt = (double)route_w[t * k + s];
                for (int64_t n = 0; n < N; n++) out_t[n] += wt * y[n];
            }
        }
        free(a);
        free(y);
    }
    return bad ? -2 : 0;
}

/* One expert's FFN on a quantized activation row: g = Wg xq, u = Wu xq, h = silu(g)*u,
 * h rounded to bf16 (the intermediate's storage type) and quantized as above, then
 * y = Wd hq. */
static void expert_ffn_q8act(int type, const void *g_data, const void *g_scales, const void *u_data,
                             const void *u_scales, const void *d_data, const void *d_scales,
                             int64_t n_ff, int64_t n_embd, int64_t e, const double *xq, double *g,
                             double *u, float *hf, int8_t *hq, float *hd, double *y) {
    matvec(type, g_data, g_scales, n_ff, n_embd, e, xq, g);
    matvec(type, u_data, u_scales, n_ff, n_embd, e, xq, u);
    for (int64_t i = 0; i < n_ff; i++) hf[i] = (float)round_to_bf16(g[i] / (1.0 + exp(-g[i])) * u[i]);
    for (int64_t b = 0; b < n_ff / 32; b++) quantize_block(hf + b * 32, 32, hq + b * 32, hd + b);
    q8act_row(hq, hd, n_ff, g);
    matvec(type, d_data, d_scales, n_embd, n_ff, e, g, y);
}

/*
 * Fused MoE FFN on the quantized-activation path: as oracle_ffn, with each token's x
 * quantized (definition above) before the gate and up projections, and each expert's
 * h rounded to bf16 and quantized before the down projection.
 */
int oracle_ffn_q8act(int w_type, const void *g_data, const void *g_scales, const void *u_data,
                     const void *u_scales, const void *d_data, const void *d_scales, int64_t E,
                     int64_t n_ff, int64_t n_embd, const void *sg_data, const void *sg_scales,
                     const void *su_data, const void *su_scales, const void *sd_data,
                     const void *sd_scales, int64_t S, int64_t n_ff_sh, const void *x, int x_type,
                     const int32_t *ids, const float *route_w, int64_t T, int32_t k, double *out) {
    if (!g_data || !u_data || !d_data || !x || !ids || !route_w || !out) return -1;
    if (E <= 0 || n_ff <= 0 || n_embd <= 0 || T < 0 || k <= 0 || S < 0) return -1;
    if (!is_quant(w_type) || x_type != OR_BF16) return -1;
    const int64_t qc = quant_cols(w_type);
    if (!g_scales || !u_scales || !d_scales || n_embd % qc || n_ff % qc) return -1;
    if (S > 0 && (!sg_data || !su_data || !sd_data || !sg_scales || !su_scales || !sd_scales ||
                  n_ff_sh <= 0 || n_ff_sh % qc))
        return -1;
    int64_t ffmax = n_ff > n_ff_sh ? n_ff : n_ff_sh;
    int bad = 0;
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < T; t++) {
        double *xq = (double *)malloc(sizeof(double) * (size_t)n_embd);
        int8_t *xc = (int8_t *)malloc((size_t)n_embd);
        float *xd = (float *)malloc(sizeof(float) * (size_t)(n_embd / 32));
        double *g = (double *)malloc(sizeof(double) * (size_t)ffmax);
        double *u = (double *)malloc(sizeof(double) * (size_t)ffmax);
        float *hf = (float *)malloc(sizeof(float) * (size_t)ffmax);
        int8_t *hq = (int8_t *)malloc((size_t)ffmax);
        float *hd = (float *)malloc(sizeof(float) * (size_t)(ffmax / 32 + 1));
        double *y = (double *)malloc(sizeof(double) * (size_t)n_embd);
        if (!xq || !xc || !xd || !g || !u || !hf || !hq || !hd || !y) {
            bad = 1;
        } else {
            double *o = out + t * n_embd;
            oracle_quantize_act(x_type, (const uint16_t *)x + t * n_embd, 1, n_embd, xc, xd);
            q8act_row(xc, xd, n_embd, xq);
            for (int64_t c = 0; c < n_embd; c++) o[c] = 0.0;
            for (int32_t s = 0; s < k; s++) {
                int32_t e = ids[t * k + s];
                if (e < 0 || e >= E) continue;
                expert_ffn_q8act(w_type, g_data, g_scales, u_data, u_scales, d_data, d_scales, n_ff,
                                 n_embd, e, xq, g, u, hf, hq, hd, y);
                double wt = (double)route_w[t * k + s];
                for (int64_t c = 0; c < n_embd; c++) o[c] += wt * y[c];
            }
            for (int64_t j = 0; j < S; j++) {
                expert_ffn_q8act(w_type, sg_data, sg_scales, su_data, su_scales, sd_data, sd_scales,
                                 n_ff_sh, n_embd, j, xq, g, u, hf, hq, hd, y);
                for (int64_t c = 0; c < n_embd; c++) o[c] += y[c];
            }
        }
        free(xq);
        free(xc);
        free(xd);
        free(g);
        free(u);
        free(hf);
        free(hq);
        free(hd);
        free(y);
    }
    return bad ? -2 : 0;
}
