/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) Mixture-of-Experts indirect
 * matrix multiplication (mul_mat_id) library.
 *
 * The operation. mul_mat_id takes stacked expert weights, activations and an
 * integer ids table; every token is multiplied only by the weight matrices of the
 * experts its ids row names ("CUDA: better MoE implementation", the ik_llama.cpp
 * PR #283 write-up, section 1.2). The deterministic fast path first turns ids into
 * three maps -- the src1 rows reordered so each expert's rows are contiguous, the
 * same reordering for dst, and each expert's bounds in that order -- and then
 * reorders and reduces by those maps with no atomic slot counters (same page,
 * sections 2 and 2.1; summary in section 6). The fused MoE FFN adds gate/up with
 * SiLU(gate) * up (section 4.2 names the fused up/gate forward) and always-on
 * shared experts computed in the same operation ("CUDA: fuse shared experts into
 * MMVQ", llama.cpp release b11370: fused shared experts, optional buffers checked
 * for null).
 *
 * Layouts (row-major, last index contiguous):
 *   weights  W[n_mat][rows][cols]; Q8_0: int8 qs[n_mat][rows][cols] plus fp16
 *            scales d[n_mat][rows][cols/32], value = d * q (32 values per scale).
 *            MXFP4 (the format the TensorSharp page lists for GPT-OSS 20B experts;
 *            defined by the OCP Microscaling v1.0 specification): uint8
 *            codes[n_mat][rows][cols/2], two FP4 E2M1 codes per byte, column 2i in
 *            bits 0-3 and column 2i+1 in bits 4-7, plus uint8 E8M0 scales
 *            x[n_mat][rows][cols/32], value = e2m1(code) * 2^(x - 127) (x = 255: NaN).
 *            IQ4_NL (the 4-bit codes of the IQ-series types the pages name: IQ2_K_R4
 *            in the PR #283 write-up, section 3.2, UD-IQ4_XS models on the TensorSharp
 *            page; defined by ggml): uint8 codes[n_mat][rows][cols/2] packed as MXFP4's,
 *            plus fp16 scales d[n_mat][rows][cols/32] as Q8_0's, value = d * level(code)
 *            with ggml's 16 IQ4_NL levels (-127 -104 -83 -65 -49 -35 -22 -10 1 13 25
 *            38 53 69 89 113).
 *            IQ4_XS (ggml's super-block form of those codes): codes as IQ4_NL's, plus one
 *            8-byte record per 256 columns, uint8 scales[n_mat][rows][cols/256][8] (8-byte
 *            aligned): fp16 d (bytes 0-1), uint16 scales_h (bytes 2-3), uint8 scales_l[4]
 *            (bytes 4-7); block j (0..7) of the 256 has the 6-bit sub-scale ls = (nibble
 *            j%2 of scales_l[j/2], low nibble first) | ((scales_h >> 2j) & 3) << 4, and
 *            value = d * (ls - 32) * level(code). cols % 256 == 0.
 *   ids      int32 [n_tokens][n_used]; route_w float32 [n_tokens][n_used].
 *   src1     [n_tokens][B][K] with B = src1_rows_per_token in {1, n_used}:
 *            slot s of token t reads row t*B + (s mod B).
 *   x        [n_tokens][n_embd]; bf16 tensors are raw 16-bit patterns.
 *
 * Ownership and ordering. Every tensor pointer is a caller-owned DEVICE pointer;
 * the library never allocates, frees or keeps one. Structs passed by pointer
 * (moe_weights, moe_options) are read before the call returns, so host memory is
 * never touched after return. Work is enqueued on `stream` (a hipStream_t; NULL =
 * the default stream) and the call returns without synchronising. The workspace
 * `ws` is caller-owned device memory of at least the size the matching
 * *_workspace_size function reports; its contents are undefined on entry and on
 * exit, and two calls in flight at once must not share one.
 *
 * Errors. Arguments are validated before anything is enqueued; on any status other
 * than MOE_OK nothing was enqueued and outputs are untouched (MOE_EHIP: a launch
 * failed; earlier launches of the same call may have run). moe_last_error()
 * returns a thread-local description of the last failure.
 *
 * Determinism. No floating-point or placement atomics are used: for identical
 * inputs, shapes, options and device, outputs are bitwise identical run to run.
 *
 * Ids outside [0, n_experts) are a caller error that does not fault: such an entry
 * joins no expert segment (expert_bounds[n_experts] counts valid entries only),
 * its per-slot output row is zero and it contributes nothing to weighted sums.
 * Duplicate ids within a token are legal; every (token, slot) is its own row.
 *
 * Limits (MOE_ELIMIT): n_tokens < 2^22 and n_used < 2^10 (the bounds the page
 * above quotes for safe 32-bit packing, section 2.1), n_tokens * n_used < 2^31,
 * n_experts <= 1024, Q8_0, MXFP4 and IQ4_NL cols % 32 == 0, IQ4_XS cols % 256 == 0. On the grouped GEMM path the
 * activation tensor whose rows are gathered through the row map (moe_ffn_fused: x;
 * moe_mul_mat_id: src1) must be under 4 GiB, and each GEMM launch must hold fewer
 * than 2^32 work-items; float32 moe_mul_mat_id needs n_tokens * n_used * N < 2^32.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,     /* null pointer, bad size, unsupported dtype combination */
    MOE_ELIMIT = -2,     /* a size limit above is exceeded                         */
    MOE_EWORKSPACE = -3, /* ws_bytes smaller than the required workspace           */
    MOE_EHIP = -4        /* a HIP launch failed                                    */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_Q8_0 = 2, MOE_MXFP4 = 3, MOE_IQ4_NL = 4, MOE_IQ4_XS = 5 } moe_dtype;

/* n_mat stacked matrices of rows x cols. */
typedef struct {
    moe_dtype type;     /* MOE_F32, MOE_Q8_0, MOE_MXFP4, MOE_IQ4_NL, MOE_IQ4_XS  */
    const void *data;   /* F32: float[n_mat][rows][cols]; Q8_0: int8 qs[...];    */
                        /* MXFP4, IQ4_NL, IQ4_XS: uint8 codes[n_mat][rows][cols/2] */
    const void *scales; /* Q8_0, IQ4_NL: uint16 (fp16) d[n_mat][rows][cols/32];  */
                        /* MXFP4: uint8 E8M0 x[n_mat][rows][cols/32];            */
                        /* IQ4_XS: uint8 records[n_mat][rows][cols/256][8]; F32: NULL */
    int64_t n_mat, rows, cols;
} moe_weights;

/* Path selection (the pages' backend picks its quantized grouped path by comparing
 * the token count with a threshold times the expert count, section 2.1):
 * GEMM when n_tokens >= tau * n_experts, else the GEMV (decode) path within the
 * bounds that moe_select_path states.
 * Optional per-kernel timing: when timing_events is non-NULL it points to
 * n_timing_events hipEvent_t handles; the call records events[2i] before and
 * events[2i+1] after its i-th kernel launch on `stream` (while 2i+1 <
 * n_timing_events). Kernel order -- moe_ffn_fused GEMM path: row ids, gate/up
 * grouped GEMM, down grouped GEMM, reduce; GEMV path: gate/up GEMV, down GEMV,
 * reduce, where small batches (the distinct experts plus the shared ones fit two per
 * wave) do the reduce inside the down GEMV and time two kernels only.
 * moe_mul_mat_id GEMM path: row ids, grouped GEMM, fix-up/reduce; GEMV path: GEMV,
 * fix-up/reduce (weighted calls of small batches: the GEMV alone).
 * moe_last_stage_count() tells how many kernels the last call timed. */
typedef struct {
    int32_t path; /* 0 auto, 1 force grouped GEMM, 2 force GEMV (decode)        */
    float tau;    /* <= 0 means the default, 1.0                                 */
    /* 1: quantized activations (the MMQ-style path; Q8_0 experts only): activation
     * rows are quantized (moe_quantize_act's format) and the grouped GEMM runs int8
     * MFMA with per-block scales, for every batch size (path must be 0 or 1). The
     * fused FFN quantizes x before gate/up and h (rounded to bf16) before down.
     * Kernel order for timing: row ids, quantize, grouped GEMM[, quantize h, down
     * grouped GEMM], reduce / fix-up. 0 (default): bf16 activations. */
    int32_t act_quant;
    int32_t reserved[5];
    void *const *timing_events;
    int32_t n_timing_events;
    int32_t reserved2;
} moe_options;

/*
 * moe_row_ids -- the three maps of section 2.1 of the PR #283 write-up.
 *   ids              device int32 [n_tokens][n_used]
 *   ids_src1, ids_dst device int32 [n_tokens * n_used] (written)
 *   expert_bounds    device int32 [n_experts + 1] (written)
 * Position j enumerates experts ascending, and inside an expert its entries by
 * token then slot (a stable counting sort): ids_src1[j] = t*B + (s mod B) is the
 * src1 row entry j reads, ids_dst[j] = t*n_used + s the dst row it writes, and
 * expert e owns [expert_bounds[e], expert_bounds[e+1]). Entries with invalid ids
 * follow position expert_bounds[n_experts], in (t, s) order.
 * n_tokens = 0 is allowed (all bounds 0). Workspace: moe_row_ids_workspace_size.
 */
moe_status moe_row_ids(const int32_t *ids, int64_t n_tokens, int32_t n_used, int32_t n_experts,
                       int32_t src1_rows_per_token, int32_t *ids_src1, int32_t *ids_dst,
                       int32_t *expert_bounds, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_gather_rows -- the src1 rows copied into expert order by the first map of
 * moe_row_ids (section 2.1 of the PR #283 write-up: ids_src1 names the src1 row each
 * position of the expert-grouped buffer reads; section 2 shows the atomic-slot copy
 * k_copy_src1_to_contiguous this replaces): dst[j][:] = src1[ids_src1[j]][:].
 *   src1      device BF16 or F32 [src1_rows][K]
 *   ids_src1  device int32 [n] (moe_row_ids' ids_src1 with n = n_tokens * n_used)
 *   dst       device [n][K] of src1's type (written; a position whose index is outside
 *             [0, src1_rows) gets a zero row)
 * The fused calls never need it (their grouped GEMM gathers the rows into LDS itself);
 * it is for callers that want the expert-contiguous copy. No workspace. n = 0 is a
 * no-op. MOE_ELIMIT: src1_rows >= 2^31 or n >= 2^33.
 */
moe_status moe_gather_rows(const void *src1, moe_dtype src1_type, int64_t src1_rows, int64_t K,
                           const int32_t *ids_src1, int64_t n, void *dst, void *stream);

/*
 * moe_mul_mat_id -- GGML_OP_MUL_MAT_ID (section 1.2 of the PR #283 write-up).
 *   w        n_mat = n_experts, rows = N, cols = K. Supported pairs: (Q8_0 w, BF16
 *            src1), (MXFP4, IQ4_NL or IQ4_XS w, BF16 src1) on the MFMA grouped
 *            GEMM or the GEMV path (the 4-bit types on the GEMV path: n_tokens *
 *            n_used <= 64 and K <= 4096, else the GEMM path is taken, and forcing the
 *            GEMV path is MOE_EINVAL); (F32 w, F32
 *            src1), which has one path, the fp32 grouped product: opt->path must be
 *            0 or 1 (else MOE_EINVAL).
 *   src1     device [n_tokens][B][K], B = src1_rows_per_token in {1, n_used}
 *   ids      device int32 [n_tokens][n_used]
 *   route_w  NULL: dst = float32 [n_tokens][n_used][N], dst[t][s] = W_{ids[t][s]} src1_row;
 *            else device float32 [n_tokens][n_used] and dst = float32 [n_tokens][N],
 *            dst[t] = sum over s ascending of route_w[t][s] * (slot s's row).
 * Outputs are overwritten, never accumulated into. n_tokens = 0 is a no-op.
 */
moe_status moe_mul_mat_id(const moe_weights *w, const void *src1, moe_dtype src1_type,
                          int32_t src1_rows_per_token, const int32_t *ids, int64_t n_tokens,
                          int32_t n_used, const float *route_w, float *dst, const moe_options *opt,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * moe_ffn_fused -- MoE FFN layer on the indirect matmul: the gate and up projections
 * with the fused up/gate forward SiLU(gate) * up ("CUDA: better MoE implementation",
 * section 4.2), the down projection, and the deterministic reorder and fixed-order
 * reduction of the routed slots (sections 2.1 and 6), plus the always-on shared
 * experts computed in the same operation ("CUDA: fuse shared experts into MMVQ",
 * llama.cpp release b11370; optional, so checked for null):
 *   out[t] = sum_{s ascending, valid} route_w[t][s] * Wd_e (silu(Wg_e x_t) * (Wu_e x_t)),
 *            e = ids[t][s];  then + sum_{j ascending} Sd_j (silu(Sg_j x_t) * (Su_j x_t)).
 *   gate, up  Q8_0 [n_experts][n_ff][n_embd]; down Q8_0 [n_experts][n_embd][n_ff]
 *   sh_gate, sh_up Q8_0 [S][n_ff_sh][n_embd]; sh_down Q8_0 [S][n_embd][n_ff_sh];
 *             or all of them MXFP4, all IQ4_NL or all IQ4_XS (their GEMV path needs n_tokens *
 *             n_used <= 64 and n_embd, n_ff, n_ff_sh <= 4096; larger calls take the
 *             grouped GEMM);
 *             all three NULL (or n_mat == 0) = no shared experts; giving only some of
 *             them is MOE_EINVAL.
 *   x         device BF16 [n_tokens][n_embd]; ids, route_w as above.
 *   out       device float32 [n_tokens][n_embd] (overwritten).
 * silu(z) = z / (1 + exp(-z)). Intermediates: GEMM path -- bf16 weights (Q8_0: d*q
 * rounded to nearest-even; MXFP4: exact; IQ4_NL, IQ4_XS: scale*level rounded to nearest-even), bf16 activations, fp32 accumulate, bf16 SiLU*up, fp32 down
 * results; GEMV path -- weights exact, fp32 accumulate throughout.
 */
moe_status moe_ffn_fused(const moe_weights *gate, const moe_weights *up, const moe_weights *down,
                         const moe_weights *sh_gate, const moe_weights *sh_up,
                         const moe_weights *sh_down, const void *x, moe_dtype x_type,
                         const int32_t *ids, const float *route_w, int64_t n_tokens, int32_t n_used,
                         float *out, const moe_options *opt, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * moe_ffn_fused_noalloc -- moe_ffn_fused for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * arguments and results as moe_ffn_fused, without ws / ws_bytes: the workspace is a
 * fixed array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every
 * device it runs on, from the first call there until the process ends. Enough for a
 * DeepSeek-Lite-shaped PP512 layer and any decode batch; a call needing more
 * (moe_ffn_fused_workspace_size) is MOE_ELIMIT, with nothing enqueued. The call itself
 * allocates nothing. All calls on one device share that device's array, so calls that
 * overlap in time on one device (different streams, or different host threads) race
 * and give undefined results: serialise them, e.g. on one stream. Its contents need no
 * clearing between calls (the kernels overwrite what they read).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_ffn_fused_noalloc(const moe_weights *gate, const moe_weights *up,
                                 const moe_weights *down, const moe_weights *sh_gate,
                                 const moe_weights *sh_up, const moe_weights *sh_down,
                                 const void *x, moe_dtype x_type, const int32_t *ids,
                                 const float *route_w, int64_t n_tokens, int32_t n_used, float *out,
                                 const moe_options *opt, void *stream);

/*
 * moe_quantize_act -- the activation format of the quantized-activation path (the
 * pages' mmq_id multiplies quantized experts with quantized activations, "CUDA: better
 * MoE implementation", section 2.1; they do not define the format, so it is a
 * reading): each row of x is cut into blocks of 32 columns; a block gets the float32
 * scale d = max|x| / 127 and int8 codes q = x / d rounded to the nearest integer, ties
 * to even (float32 division and rounding; clamped to [-127, 127]); a block of zeros has
 * d = 0 and q = 0. Value = d * q. x must be finite.
 *   x   device BF16 or F32 [rows][K], K % 32 == 0 (MOE_ELIMIT otherwise), 16-byte aligned
 *   q   device int8 [rows][K] (written, 16-byte aligned); d device float32 [rows][K/32]
 *       (written)
 * rows = 0 is a no-op. No workspace. Deterministic.
 */
moe_status moe_quantize_act(const void *x, moe_dtype x_type, int64_t rows, int64_t K, int8_t *q,
                            float *d, void *stream);

/*
 * moe_router_topk -- the step ahead of the op: the ids table the op consumes (section
 * 1.2 of the PR #283 write-up: ids names the experts each token uses) and routing
 * weights, from router logits.
 *   logits   device float32 [n_tokens][n_experts]
 *   ids      device int32 [n_tokens][n_used] (written): the n_used largest logits of
 *            each token in descending order, equal logits taken lower index first;
 *            NaN logits rank strictly below every number, -inf included (NaNs among
 *            themselves: lower index first)
 *   route_w  device float32 [n_tokens][n_used] (written): softmax over the picked
 *            logits only (exp(v_r - v_0) / sum_r exp(v_r - v_0)), the weighting the
 *            DeepSeek-V3-shaped configuration calls softmax renormalised over the
 *            picks. A NaN pick is weighted as -inf (weight 0). When the largest pick
 *            v_0 is +inf or -inf the softmax's limit is used: the c picks equal to v_0
 *            get 1/c each and the others 0 (a token whose picks are all -inf or NaN
 *            gets 1/n_used on every pick)
 * Requires 1 <= n_used <= n_experts <= 1024 (MOE_EINVAL / MOE_ELIMIT otherwise) and
 * n_tokens < 2^22. No workspace. Deterministic. n_tokens = 0 is a no-op.
 */
moe_status moe_router_topk(const float *logits, int64_t n_tokens, int32_t n_experts, int32_t n_used,
                           int32_t *ids, float *route_w, void *stream);

/* Workspace sizes in bytes for the calls above with the same arguments (0 if the
 * arguments are invalid; a valid call may also need 0 bytes, then ws may be NULL). */
size_t moe_row_ids_workspace_size(int64_t n_tokens, int32_t n_used, int32_t n_experts);
size_t moe_mul_mat_id_workspace_size(const moe_weights *w, moe_dtype src1_type,
                                     int32_t src1_rows_per_token, int64_t n_tokens,
                                     int32_t n_used, const moe_options *opt);
size_t moe_ffn_fused_workspace_size(const moe_weights *gate, const moe_weights *sh_gate,
                                    moe_dtype x_type, int64_t n_tokens, int32_t n_used,
                                    const moe_options *opt);

/* Which path a call with these sizes takes: 1 grouped GEMM, 2 GEMV (decode), or a
 * negative moe_status for invalid arguments. act_width is the widest activation
 * row a GEMV kernel would stage (mul_mat_id: K; FFN: max(n_embd, n_ff, n_ff_sh)).
 * Auto (Q8_0): GEMV when n_tokens < tau * n_experts and either n_tokens * n_used <= 48
 * with act_width <= 4096, or n_tokens == 1 with n_used <= 256 and act_width <= 16384;
 * else GEMM. 4-bit experts: GEMV when n_tokens < tau * n_experts, n_tokens * n_used
 * <= 64 (MXFP4: 32) and act_width <= 4096. Forcing GEMV is allowed up to n_tokens * n_used <= 256
 * and act_width <= 16384 (Q8_0; 64 and 4096 for 4-bit), else MOE_EINVAL.
 * Pure host function. */
int32_t moe_select_path(int64_t n_tokens, int32_t n_used, int32_t n_experts, int64_t act_width,
                        const moe_options *opt);

/* The path moe_mul_mat_id / moe_ffn_fused take for experts of weight_type (MOE_Q8_0,
 * MOE_MXFP4, MOE_IQ4_NL or MOE_IQ4_XS) under opt: 1 grouped GEMM, 2 GEMV, 3 the grouped
 * GEMM over quantized activations (opt->act_quant = 1, Q8_0 only), or a negative
 * moe_status (MOE_EINVAL for other weight types, or for options the call would reject).
 * Q8_0 gives the same answer as moe_select_path. Pure host function. */
int32_t moe_select_path_typed(int64_t n_tokens, int32_t n_used, int32_t n_experts, int64_t act_width,
                              moe_dtype weight_type, const moe_options *opt);

const char *moe_status_string(moe_status s);
const char *moe_last_error(void); /* thread-local detail of the last failure ("" if none) */
/* Kernels (timing-event pairs, see moe_options) enqueued by the last successful
 * moe_mul_mat_id or moe_ffn_fused call on this thread; 0 before any such call. */
int32_t moe_last_stage_count(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
