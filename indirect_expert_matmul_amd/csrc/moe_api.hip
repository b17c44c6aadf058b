// libmoe C ABI: argument validation, limits, workspace carving, path selection and
// the launch sequence of each entry point (declared and documented in moe.h).
//
// Host-side rules taken from the pages' account of the CUDA implementation
// ("CUDA: better MoE implementation"):
//   * the three row maps are built on the device, so no host buffer has to outlive
//     an asynchronous copy (section 5 discusses exactly that hazard with host-side
//     mapping buffers) -- this file never copies host data to the device and never
//     synchronises;
//   * the grouped (GEMM) path serves batches whose token count is large relative to
//     the expert count, the mat-vec path the small ones (section 2.1's threshold
//     test, read here as n_tokens >= tau * n_experts);
//   * the packing limits n_tokens < 2^22 and n_used < 2^10 (section 2.1).
#include <cstdarg>
#include <cstdio>
#include <string>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_err;
thread_local int32_t g_stages = 0;   // kernels timed by the last call

moe_status fail(moe_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base((char*)b) {}
    void* take(size_t bytes) {
        off = (off + kAlign - 1) / kAlign * kAlign;
        void* p = base ? base + off : nullptr;
        off += bytes;
        return p;
    }
};

struct Timer {
    void* const* ev;
    int n;
    int stage = 0;
    hipStream_t st;
    Timer(const moe_options* o, hipStream_t s)
        : ev(o ? o->timing_events : nullptr), n(o ? o->n_timing_events : 0), st(s) {}
    void begin() {
        if (ev && 2 * stage + 1 < n) (void)hipEventRecord((hipEvent_t)ev[2 * stage], st);
    }
    void end() {
        if (ev && 2 * stage + 1 < n) (void)hipEventRecord((hipEvent_t)ev[2 * stage + 1], st);
        stage++;
    }
};

moe_status hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

moe_status check_tokens(int64_t T, int32_t k) {
    if (T < 0) return fail(MOE_EINVAL, "n_tokens must be >= 0 (got %lld)", (long long)T);
    if (k <= 0) return fail(MOE_EINVAL, "n_used must be > 0 (got %d)", k);
    if (T >= (1LL << 22)) return fail(MOE_ELIMIT, "n_tokens must be < 2^22 (got %lld)", (long long)T);
    if (k >= (1 << 10)) return fail(MOE_ELIMIT, "n_used must be < 2^10 (got %d)", k);
    if (T * (int64_t)k >= (1LL << 31))
        return fail(MOE_ELIMIT, "n_tokens * n_used must be < 2^31");
    return MOE_OK;
}

moe_status check_experts(int64_t E) {
    if (E <= 0) return fail(MOE_EINVAL, "n_experts must be > 0 (got %lld)", (long long)E);
    if (E > kMaxExperts) return fail(MOE_ELIMIT, "n_experts must be <= %d (got %lld)", kMaxExperts, (long long)E);
    return MOE_OK;
}

moe_status check_weights(const moe_weights* w, const char* name, bool allow_f32) {
    if (!w) return fail(MOE_EINVAL, "%s: weights struct is NULL", name);
    if (!w->data) return fail(MOE_EINVAL, "%s: data is NULL", name);
    if (w->n_mat <= 0 || w->rows <= 0 || w->cols <= 0)
        return fail(MOE_EINVAL, "%s: sizes must be > 0", name);
    if (w->rows > INT32_MAX || w->cols > INT32_MAX)
        return fail(MOE_ELIMIT, "%s: rows and cols must fit in int32", name);
    if (w->type == MOE_Q8_0 || w->type == MOE_MXFP4 || w->type == MOE_IQ4_NL || w->type == MOE_IQ4_XS) {
        const char* fmt = w->type == MOE_Q8_0 ? "Q8_0"
                          : w->type == MOE_MXFP4 ? "MXFP4" : w->type == MOE_IQ4_NL ? "IQ4_NL" : "IQ4_XS";
        const int64_t unit = w->type == MOE_IQ4_XS ? 256 : 32;   // columns per scale unit
        if (!w->scales) return fail(MOE_EINVAL, "%s: %s scales are NULL", name, fmt);
        if (w->cols % unit)
            return fail(MOE_ELIMIT, "%s: %s needs cols %% %lld == 0 (got %lld)", name, fmt, (long long)unit,
                        (long long)w->cols);
        if (w->type == MOE_IQ4_XS && ((uintptr_t)w->scales & 7))
            return fail(MOE_EINVAL, "%s: IQ4_XS super-block records must be 8-byte aligned", name);
    } else if (w->type == MOE_F32) {
        if (!allow_f32) return fail(MOE_EINVAL, "%s: float32 weights are not supported here", name);
    } else {
        return fail(MOE_EINVAL, "%s: unsupported weight type %d", name, (int)w->type);
    }
    return MOE_OK;
}

// Weight format code of the kernels: 0 Q8_0, 1 MXFP4, 2 IQ4_NL, 3 IQ4_XS.
int32_t kernel_fmt(moe_dtype t) {
    return t == MOE_MXFP4 ? 1 : t == MOE_IQ4_NL ? 2 : t == MOE_IQ4_XS ? 3 : 0;
}

float tau_of(const moe_options* o) { return (o && o->tau > 0.f) ? o->tau : 1.0f; }

// 1 = GEMM, 2 = GEMV, or a negative status.
int select_path(int64_t T, int32_t k, int32_t E, int64_t act_width, const moe_options* o) {
    const int32_t force = o ? o->path : 0;
    const bool dec_ok = T * (int64_t)k <= kDecMaxSlots && act_width <= kDecMaxWidth;
    if (force == 1) return 1;
    if (force == 2) {
        if (!dec_ok)
            return fail(MOE_EINVAL, "GEMV path needs n_tokens*n_used <= %d and activation width <= %lld",
                        kDecMaxSlots, (long long)kDecMaxWidth);
        return 2;
    }
    if (force != 0) return fail(MOE_EINVAL, "options.path must be 0, 1 or 2 (got %d)", force);
    // Automatic choice: the GEMV's wave-level kernels up to kDecAutoSlots slots, its block
    // kernel (wider rows, more slots) for a single token only. Past those the block kernel
    // streams an expert's rows once per slot and the grouped GEMM wins (measured on one
    // MI355X, Q8_0, GEMV against GEMM per layer call: V3-shaped T = 2 155 / 156 us, T = 16
    // 2,868 / 941 us; Lite-shaped T = 10 126 / 106 us, T = 42 1,249 / 149 us; GPT-OSS-shaped
    // T = 16 235 / 225 us; T = 8 127 / 153 us).
    const bool wave_ok = T * (int64_t)k <= kDecAutoSlots && act_width <= 4096;
    return ((double)T < (double)tau_of(o) * (double)E && dec_ok && (wave_ok || T == 1)) ? 2 : 1;
}

// 4-bit experts (MXFP4, IQ4_NL, IQ4_XS): the GEMV path only through its wave-level kernels
// (n_tokens * n_used <= 64 and every activation width <= 4096); otherwise the grouped GEMM.
// Automatically up to auto_slots slots: MXFP4 32 (GPT-OSS-shaped, GEMV against GEMM per layer
// call on one MI355X: 16 slots 79 / 91 us, 32 slots 119 / 112, 48 slots 165 / 141, 64 slots
// 200 / 162), the IQ formats 64 (IQ4_XS E128 k8 at 64 slots 70 / 77 us; IQ4_NL
// GPT-OSS-shaped at 48 and 64 slots 189 / 189 and 227 / 219, Lite-shaped at 48 84 / 93).
int select_path_fmt(int64_t T, int32_t k, int32_t E, int64_t act_width, bool fp4, const moe_options* o,
                    int auto_slots = 64) {
    if (!fp4) return select_path(T, k, E, act_width, o);
    const int32_t force = o ? o->path : 0;
    const bool dec_ok = T * (int64_t)k <= 64 && act_width <= 4096;
    if (force == 1) return 1;
    if (force == 2) {
        if (!dec_ok)
            return fail(MOE_EINVAL, "GEMV path with 4-bit (MXFP4, IQ4_NL, IQ4_XS) experts needs n_tokens*n_used <= 64 "
                        "and widths <= 4096");
        return 2;
    }
    if (force != 0) return fail(MOE_EINVAL, "options.path must be 0, 1 or 2 (got %d)", force);
    return ((double)T < (double)tau_of(o) * (double)E && dec_ok && T * (int64_t)k <= auto_slots) ? 2 : 1;
}

// With options.act_quant = 1: 3 (the quantized-activation grouped GEMM, Q8_0 experts
// only, whatever the batch size), else the choice above; or a negative status.
int select_path_aq(int64_t T, int32_t k, int32_t E, int64_t act_width, int32_t wtype,
                   const moe_options* o) {
    const int32_t aq = o ? o->act_quant : 0;
    if (aq != 0 && aq != 1) return fail(MOE_EINVAL, "options.act_quant must be 0 or 1 (got %d)", aq);
    if (!aq)
        return select_path_fmt(T, k, E, act_width,
                               wtype == MOE_MXFP4 || wtype == MOE_IQ4_NL || wtype == MOE_IQ4_XS, o,
                               wtype == MOE_MXFP4 ? 32 : 64);
    if (wtype != MOE_Q8_0) return fail(MOE_EINVAL, "quantized activations (act_quant = 1) need Q8_0 experts");
    if (o->path != 0 && o->path != 1)
        return fail(MOE_EINVAL, "quantized activations run on the grouped GEMM only: options.path must "
                    "be 0 or 1 (got %d)", o->path);
    return 3;
}

int64_t m_tiles_bound(int64_t n, int64_t E, int bm) { return n / bm + (n < E ? n : E); }

// ---------------------------------------------------------------- workspace plans
struct RowIdsPlan {
    int32_t *ids_src1, *ids_dst, *bounds, *tile_a, *tile_tab;
    void* scratch;   // multi-block scratch of the row-id pass (row_ids_scratch_bytes)
    int32_t tile_cap;
};
// tile_m > 0: also room for the GEMM's M-tile prefix and per-tile table (tiles of
// tile_m rows)
RowIdsPlan carve_row_ids(Carve& c, int64_t n, int32_t E, bool maps, int tile_m) {
    RowIdsPlan p{};
    const bool tiles = tile_m > 0;
    if (maps) {
        p.ids_src1 = (int32_t*)c.take(sizeof(int32_t) * n);
        p.ids_dst = (int32_t*)c.take(sizeof(int32_t) * n);
        p.bounds = (int32_t*)c.take(sizeof(int32_t) * (E + 1));
    }
    if (tiles) {
        p.tile_a = (int32_t*)c.take(sizeof(int32_t) * (E + 1));
        p.tile_cap = (int32_t)m_tiles_bound(n, E, tile_m);
        p.tile_tab = (int32_t*)c.take(sizeof(int32_t) * 4 * (size_t)p.tile_cap);
    }
    const size_t sb = row_ids_scratch_bytes(n, E);
    if (sb) p.scratch = c.take(sb);
    return p;
}

struct FfnDims {
    int64_t T;
    int32_t k, E, n_embd, n_ff, S, n_ff_sh;
    int32_t fmt;   // kernel weight format: 0 Q8_0, 1 MXFP4, 2 IQ4_NL, 3 IQ4_XS
};

struct FfnPlan {
    int path;
    int msub;
    RowIdsPlan r;
    void *h, *hsh, *y, *ysh;
    // quantized-activation path: codes and block scales of x, h and the shared h
    int8_t *xq, *hq, *hshq;
    float *xd, *hd, *hshd;
};

FfnPlan carve_ffn(Carve& c, const FfnDims& d, int path) {
    FfnPlan p{};
    p.path = path;
    const int64_t n = d.T * d.k;
    if (path == 3) {
        p.r = carve_row_ids(c, n, d.E, true, kQ8aTileM);
        p.xq = (int8_t*)c.take((size_t)d.T * d.n_embd);
        p.xd = (float*)c.take((size_t)d.T * (d.n_embd / 32) * 4);
        p.h = c.take((size_t)n * d.n_ff * 2);
        p.hsh = c.take((size_t)d.S * d.T * d.n_ff_sh * 2);
        p.hq = (int8_t*)c.take((size_t)n * d.n_ff);
        p.hd = (float*)c.take((size_t)n * (d.n_ff / 32) * 4);
        p.hshq = (int8_t*)c.take((size_t)d.S * d.T * d.n_ff_sh);
        p.hshd = (float*)c.take((size_t)d.S * d.T * (d.n_ff_sh / 32) * 4);
    } else if (path == 1) {
        p.msub = gemm_pick_msub((double)n / d.E);
        p.r = carve_row_ids(c, n, d.E, true, gemm_tile_m(p.msub));
        p.h = c.take((size_t)n * d.n_ff * 2);
        p.hsh = c.take((size_t)d.S * d.T * d.n_ff_sh * 2);
    } else {
        p.h = c.take((size_t)n * d.n_ff * 4);
        p.hsh = c.take((size_t)d.S * d.T * d.n_ff_sh * 4);
    }
    p.y = c.take((size_t)n * d.n_embd * 4);
    p.ysh = c.take((size_t)d.S * d.T * d.n_embd * 4);
    return p;
}

struct MmidPlan {
    int path;
    int msub;
    RowIdsPlan r;
    void* y;
    int8_t* aq;   // quantized-activation path: src1 codes [T*B][K] and block scales
    float* ad;
};

MmidPlan carve_mmid(Carve& c, int64_t T, int32_t k, int32_t E, int64_t N, bool weighted, bool q8, int path,
                    int32_t B = 1, int64_t K = 0) {
    MmidPlan p{};
    p.path = path;
    const int64_t n = T * k;
    if (path == 3) {
        p.r = carve_row_ids(c, n, E, true, kQ8aTileM);
        p.aq = (int8_t*)c.take((size_t)(T * B) * K);
        p.ad = (float*)c.take((size_t)(T * B) * (K / 32) * 4);
    } else if (!q8 || path == 1) {
        p.msub = gemm_pick_msub((double)n / E);
        p.r = carve_row_ids(c, n, E, true, q8 ? gemm_tile_m(p.msub) : 0);
    }
    if (weighted) p.y = c.take((size_t)n * N * 4);
    return p;
}

moe_status validate_ffn(const moe_weights* gate, const moe_weights* up, const moe_weights* down,
                        const moe_weights* sg, const moe_weights* su, const moe_weights* sd,
                        moe_dtype x_type, int64_t T, int32_t k, FfnDims* d) {
    moe_status s;
    if ((s = check_tokens(T, k))) return s;
    if ((s = check_weights(gate, "gate", false))) return s;
    if ((s = check_weights(up, "up", false))) return s;
    if ((s = check_weights(down, "down", false))) return s;
    if ((s = check_experts(gate->n_mat))) return s;
    if (x_type != MOE_BF16) return fail(MOE_EINVAL, "x must be BF16 (Q8_0 experts run bf16 activations)");
    if (up->type != gate->type || down->type != gate->type)
        return fail(MOE_EINVAL, "gate, up and down must have the same weight type");
    if (up->n_mat != gate->n_mat || down->n_mat != gate->n_mat || up->rows != gate->rows ||
        up->cols != gate->cols || down->rows != gate->cols || down->cols != gate->rows)
        return fail(MOE_EINVAL, "gate/up must be [E][n_ff][n_embd] and down [E][n_embd][n_ff]");
    d->T = T;
    d->k = k;
    d->E = (int32_t)gate->n_mat;
    d->n_ff = (int32_t)gate->rows;
    d->n_embd = (int32_t)gate->cols;
    d->fmt = kernel_fmt(gate->type);
    const bool any_sh = (sg && sg->n_mat) || (su && su->n_mat) || (sd && sd->n_mat);
    d->S = 0;
    d->n_ff_sh = 0;
    if (any_sh) {
        if (!sg || !su || !sd || !sg->n_mat || !su->n_mat || !sd->n_mat)
            return fail(MOE_EINVAL, "shared experts: give all of sh_gate, sh_up and sh_down, or none");
        if ((s = check_weights(sg, "sh_gate", false))) return s;
        if ((s = check_weights(su, "sh_up", false))) return s;
        if ((s = check_weights(sd, "sh_down", false))) return s;
        if (sg->type != gate->type || su->type != gate->type || sd->type != gate->type)
            return fail(MOE_EINVAL, "shared experts must have the routed experts' weight type");
        if (su->n_mat != sg->n_mat || sd->n_mat != sg->n_mat || su->rows != sg->rows ||
            su->cols != sg->cols || sg->cols != gate->cols || sd->rows != gate->cols ||
            sd->cols != sg->rows)
            return fail(MOE_EINVAL, "shared gate/up must be [S][n_ff_sh][n_embd], shared down [S][n_embd][n_ff_sh]");
        if (sg->n_mat > 64) return fail(MOE_ELIMIT, "at most 64 shared experts");
        d->S = (int32_t)sg->n_mat;
        d->n_ff_sh = (int32_t)sg->rows;
    }
    return MOE_OK;
}

int64_t ffn_act_width(const FfnDims& d) {
    int64_t w = d.n_embd > d.n_ff ? d.n_embd : d.n_ff;
    return w > d.n_ff_sh ? w : d.n_ff_sh;
}

moe_status validate_mmid(const moe_weights* w, moe_dtype st, int32_t B, int64_t T, int32_t k) {
    moe_status s;
    if ((s = check_tokens(T, k))) return s;
    if ((s = check_weights(w, "w", true))) return s;
    if ((s = check_experts(w->n_mat))) return s;
    if (B != 1 && B != k) return fail(MOE_EINVAL, "src1_rows_per_token must be 1 or n_used (got %d)", B);
    if (w->type == MOE_Q8_0 && st != MOE_BF16) return fail(MOE_EINVAL, "Q8_0 weights need BF16 src1");
    if (w->type == MOE_MXFP4 && st != MOE_BF16) return fail(MOE_EINVAL, "MXFP4 weights need BF16 src1");
    if (w->type == MOE_IQ4_NL && st != MOE_BF16) return fail(MOE_EINVAL, "IQ4_NL weights need BF16 src1");
    if (w->type == MOE_IQ4_XS && st != MOE_BF16) return fail(MOE_EINVAL, "IQ4_XS weights need BF16 src1");
    if (w->type == MOE_F32 && st != MOE_F32) return fail(MOE_EINVAL, "F32 weights need F32 src1");
    return MOE_OK;
}

RowIdsArgs row_ids_args(const int32_t* ids, int64_t n, int32_t k, int32_t E, int32_t B,
                        const RowIdsPlan& p) {
    RowIdsArgs a{};
    a.ids = ids;
    a.n = n;
    a.k = k;
    a.E = E;
    a.B = B;
    a.ids_src1 = p.ids_src1;
    a.ids_dst = p.ids_dst;
    a.bounds = p.bounds;
    if (p.scratch) row_ids_carve_scratch(a, p.scratch);
    return a;
}

constexpr int64_t k4GiB = 1LL << 32;

// Launch limits of the grouped GEMM path, checked before anything is enqueued:
// activation rows gathered through the row map are addressed by 32-bit byte offsets
// from the tensor's start, and one dispatch holds fewer than 2^32 work-items.
moe_status check_gemm_limits(const GemmArgs& g, int msub, int64_t gathered_rows, int64_t lda,
                             const char* what) {
    if (gathered_rows * lda * 2 > k4GiB - 256)
        return fail(MOE_ELIMIT, "%s: the gathered bf16 activation tensor must be under 4 GiB "
                    "(%lld rows x %lld columns)", what, (long long)gathered_rows, (long long)lda);
    if (gemm_q8_max_threads(g, msub) >= k4GiB)
        return fail(MOE_ELIMIT, "%s: the grouped GEMM grid exceeds 2^32 work-items", what);
    return MOE_OK;
}

moe_status check_q8a_limits(const GemmArgs& g, int64_t gathered_rows, int64_t K, const char* what) {
    if (gathered_rows * K > k4GiB - 256)
        return fail(MOE_ELIMIT, "%s: the gathered int8 activation tensor must be under 4 GiB "
                    "(%lld rows x %lld columns)", what, (long long)gathered_rows, (long long)K);
    if (gemm_q8a_max_threads(g) >= k4GiB)
        return fail(MOE_ELIMIT, "%s: the grouped GEMM grid exceeds 2^32 work-items", what);
    return MOE_OK;
}

// One activation quantization part: rows x K of bf16 -> codes and block scales.
QuantPart qpart(const void* src, int64_t rows, int64_t K, int8_t* q, float* d) {
    QuantPart p{};
    p.src = src;
    p.rows = rows;
    p.K = K;
    p.q = q;
    p.d = d;
    return p;
}

}  // namespace

void moe::set_last_error(const char* msg) { g_err = msg; }

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
        case MOE_ELIMIT: return "MOE_ELIMIT: size limit exceeded";
        case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
        case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
    }
    return "unknown moe_status";
}

const char* moe_last_error(void) { return g_err.c_str(); }
int32_t moe_last_stage_count(void) { return g_stages; }

int32_t moe_select_path(int64_t n_tokens, int32_t n_used, int32_t n_experts, int64_t act_width,
                        const moe_options* opt) {
    moe_status s;
    if ((s = check_tokens(n_tokens, n_used))) return s;
    if ((s = check_experts(n_experts))) return s;
    if (act_width <= 0) return fail(MOE_EINVAL, "act_width must be > 0");
    return select_path(n_tokens, n_used, n_experts, act_width, opt);
}

int32_t moe_select_path_typed(int64_t n_tokens, int32_t n_used, int32_t n_experts, int64_t act_width,
                              moe_dtype weight_type, const moe_options* opt) {
    moe_status s;
    if ((s = check_tokens(n_tokens, n_used))) return s;
    if ((s = check_experts(n_experts))) return s;
    if (act_width <= 0) return fail(MOE_EINVAL, "act_width must be > 0");
    if (weight_type != MOE_Q8_0 && weight_type != MOE_MXFP4 && weight_type != MOE_IQ4_NL &&
        weight_type != MOE_IQ4_XS)
        return fail(MOE_EINVAL, "weight_type must be Q8_0, MXFP4, IQ4_NL or IQ4_XS (got %d)", (int)weight_type);
    return select_path_aq(n_tokens, n_used, n_experts, act_width, weight_type, opt);
}

size_t moe_row_ids_workspace_size(int64_t n_tokens, int32_t n_used, int32_t n_experts) {
    if (check_tokens(n_tokens, n_used) || check_experts(n_experts)) return 0;
    Carve c(nullptr);
    carve_row_ids(c, n_tokens * n_used, n_experts, false, 0);
    return c.off;
}

moe_status moe_gather_rows(const void* src1, moe_dtype src1_type, int64_t src1_rows, int64_t K,
                           const int32_t* ids_src1, int64_t n, void* dst, void* stream) {
    g_err.clear();
    if (src1_type != MOE_BF16 && src1_type != MOE_F32)
        return fail(MOE_EINVAL, "gather: src1_type must be BF16 or F32");
    if (src1_rows <= 0 || K <= 0 || n < 0) return fail(MOE_EINVAL, "gather: sizes must be > 0 (n >= 0)");
    if (src1_rows > INT32_MAX) return fail(MOE_ELIMIT, "gather: src1_rows must fit in int32");
    if (n > (int64_t)INT32_MAX * 4) return fail(MOE_ELIMIT, "gather: too many rows for one launch");
    if (n == 0) return MOE_OK;
    if (!src1 || !ids_src1 || !dst) return fail(MOE_EINVAL, "NULL pointer argument");
    GatherArgs a{src1, src1_rows, K * (src1_type == MOE_BF16 ? 2 : 4), ids_src1, n, dst};
    return hip_check(launch_gather(a, (hipStream_t)stream), "gather");
}

moe_status moe_row_ids(const int32_t* ids, int64_t n_tokens, int32_t n_used, int32_t n_experts,
                       int32_t src1_rows_per_token, int32_t* ids_src1, int32_t* ids_dst,
                       int32_t* expert_bounds, void* ws, size_t ws_bytes, void* stream) {
    moe_status s;
    g_err.clear();
    if ((s = check_tokens(n_tokens, n_used))) return s;
    if ((s = check_experts(n_experts))) return s;
    if (src1_rows_per_token != 1 && src1_rows_per_token != n_used)
        return fail(MOE_EINVAL, "src1_rows_per_token must be 1 or n_used");
    if (!expert_bounds || (n_tokens > 0 && (!ids || !ids_src1 || !ids_dst)))
        return fail(MOE_EINVAL, "NULL pointer argument");
    const size_t need = moe_row_ids_workspace_size(n_tokens, n_used, n_experts);
    if (need > ws_bytes || (need && !ws)) return fail(MOE_EWORKSPACE, "workspace needs %zu bytes", need);
    Carve c(ws);
    RowIdsPlan p = carve_row_ids(c, n_tokens * n_used, n_experts, false, 0);
    p.ids_src1 = ids_src1;
    p.ids_dst = ids_dst;
    p.bounds = expert_bounds;
    const RowIdsArgs a = row_ids_args(ids, n_tokens * n_used, n_used, n_experts, src1_rows_per_token, p);
    return hip_check(launch_row_ids(a, (hipStream_t)stream, nullptr), "row ids");
}

size_t moe_ffn_fused_workspace_size(const moe_weights* gate, const moe_weights* sh_gate,
                                    moe_dtype x_type, int64_t n_tokens, int32_t n_used,
                                    const moe_options* opt) {
    if (!gate) return 0;
    FfnDims d{};
    const moe_weights up = *gate;
    moe_weights down = *gate;
    down.rows = gate->cols;
    down.cols = gate->rows;
    const moe_weights* su = nullptr;
    moe_weights sup{}, sdown{};
    if (sh_gate && sh_gate->n_mat) {
        sup = *sh_gate;
        sdown = *sh_gate;
        sdown.rows = sh_gate->cols;
        sdown.cols = sh_gate->rows;
        su = &sup;
    }
    if (validate_ffn(gate, &up, &down, (su ? sh_gate : nullptr), su, (su ? &sdown : nullptr),
                     x_type, n_tokens, n_used, &d))
        return 0;
    const int path = select_path_aq(d.T, d.k, d.E, ffn_act_width(d), gate->type, opt);
    if (path < 0) return 0;
    Carve c(nullptr);
    carve_ffn(c, d, path);
    return c.off;
}

moe_status moe_ffn_fused(const moe_weights* gate, const moe_weights* up, const moe_weights* down,
                         const moe_weights* sh_gate, const moe_weights* sh_up,
                         const moe_weights* sh_down, const void* x, moe_dtype x_type,
                         const int32_t* ids, const float* route_w, int64_t n_tokens, int32_t n_used,
                         float* out, const moe_options* opt, void* ws, size_t ws_bytes,
                         void* stream) {
    g_err.clear();
    FfnDims d{};
    moe_status s = validate_ffn(gate, up, down, sh_gate, sh_up, sh_down, x_type, n_tokens, n_used, &d);
    if (s) return s;
    if (n_tokens == 0) {
        g_stages = 0;
        return MOE_OK;
    }
    if (!x || !ids || !route_w || !out) return fail(MOE_EINVAL, "NULL pointer argument");
    const int path = select_path_aq(d.T, d.k, d.E, ffn_act_width(d), gate->type, opt);
    if (path < 0) return (moe_status)path;
    Carve sz(nullptr);
    carve_ffn(sz, d, path);
    if (sz.off > ws_bytes || !ws) return fail(MOE_EWORKSPACE, "workspace needs %zu bytes", sz.off);
    Carve c(ws);
    const FfnPlan p = carve_ffn(c, d, path);
    const hipStream_t st = (hipStream_t)stream;
    Timer tm(opt, st);
    const int64_t n = d.T * d.k;
    const bool shared = d.S > 0;
    bool reduced = false;

    if (path == 3) {
        // quantized activations: row ids, x -> codes, gate/up int8 GEMM (h in bf16),
        // h -> codes, down int8 GEMM, then the reduce below
        const int bm = kQ8aTileM;
        RowIdsArgs ra = row_ids_args(ids, n, d.k, d.E, 1, p.r);
        ra.tile_off[0] = p.r.tile_a;
        ra.tile_m[0] = bm;
        ra.tile_tab[0] = p.r.tile_tab;
        ra.tile_cap[0] = p.r.tile_cap;
        QuantArgs qx{};
        qx.src_bf16 = 1;
        qx.n_part = 1;
        qx.part[0] = qpart(x, d.T, d.n_embd, p.xq, p.xd);
        GemmArgs g{};
        g.mode = 1;
        g.n_prob = shared ? 2 : 1;
        GemmProblem& r = g.p[0];
        r.qs1 = (const int8_t*)gate->data;
        r.d1 = (const uint16_t*)gate->scales;
        r.qs2 = (const int8_t*)up->data;
        r.d2 = (const uint16_t*)up->scales;
        r.N = d.n_ff;
        r.K = d.n_embd;
        r.bounds = p.r.bounds;
        r.tile_off = p.r.tile_a;
        r.tile_tab = p.r.tile_tab;
        r.n_seg = d.E;
        r.m_tiles_max = (int32_t)m_tiles_bound(n, d.E, bm);
        r.Aq = p.xq;
        r.Ad = p.xd;
        r.a_rows = p.r.ids_src1;
        r.out = p.h;
        r.ldo = d.n_ff;
        if (shared) {
            GemmProblem& q = g.p[1];
            q.qs1 = (const int8_t*)sh_gate->data;
            q.d1 = (const uint16_t*)sh_gate->scales;
            q.qs2 = (const int8_t*)sh_up->data;
            q.d2 = (const uint16_t*)sh_up->scales;
            q.N = d.n_ff_sh;
            q.K = d.n_embd;
            q.n_seg = d.S;
            q.seg_len = (int32_t)d.T;
            q.m_tiles_max = (int32_t)(d.S * ((d.T + bm - 1) / bm));
            q.Aq = p.xq;
            q.Ad = p.xd;
            q.a_row_mod = (int32_t)d.T;
            q.out = p.hsh;
            q.ldo = d.n_ff_sh;
        }
        QuantArgs qh{};
        qh.src_bf16 = 1;
        qh.n_part = shared ? 2 : 1;
        qh.part[0] = qpart(p.h, n, d.n_ff, p.hq, p.hd);
        if (shared) qh.part[1] = qpart(p.hsh, (int64_t)d.S * d.T, d.n_ff_sh, p.hshq, p.hshd);
        GemmArgs g2{};
        g2.mode = 0;
        g2.n_prob = shared ? 2 : 1;
        GemmProblem& r2 = g2.p[0];
        r2.qs1 = (const int8_t*)down->data;
        r2.d1 = (const uint16_t*)down->scales;
        r2.N = d.n_embd;
        r2.K = d.n_ff;
        r2.bounds = p.r.bounds;
        r2.tile_off = p.r.tile_a;
        r2.tile_tab = p.r.tile_tab;
        r2.n_seg = d.E;
        r2.m_tiles_max = r.m_tiles_max;
        r2.Aq = p.hq;
        r2.Ad = p.hd;
        r2.out = p.y;
        r2.ldo = d.n_embd;
        r2.out_rows = p.r.ids_dst;
        if (shared) {
            GemmProblem& q = g2.p[1];
            q.qs1 = (const int8_t*)sh_down->data;
            q.d1 = (const uint16_t*)sh_down->scales;
            q.N = d.n_embd;
            q.K = d.n_ff_sh;
            q.n_seg = d.S;
            q.seg_len = (int32_t)d.T;
            q.m_tiles_max = g.p[1].m_tiles_max;
            q.Aq = p.hshq;
            q.Ad = p.hshd;
            q.out = p.ysh;
            q.ldo = d.n_embd;
        }
        if ((uintptr_t)x % 16) return fail(MOE_EINVAL, "quantized activations: x must be 16-byte aligned");
        if ((s = check_q8a_limits(g, d.T, d.n_embd, "gate/up"))) return s;
        if ((s = check_q8a_limits(g2, 0, d.n_ff, "down"))) return s;
        tm.begin();
        if ((s = hip_check(launch_row_ids(ra, st, nullptr), "row ids"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_quant_act(qx, st), "quantize x"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_gemm_q8a(g, st), "gate/up grouped GEMM (int8)"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_quant_act(qh, st), "quantize h"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_gemm_q8a(g2, st), "down grouped GEMM (int8)"))) return s;
        tm.end();
    } else if (path == 1) {
        const int bm = gemm_tile_m(p.msub);
        RowIdsArgs ra = row_ids_args(ids, n, d.k, d.E, 1, p.r);
        ra.tile_off[0] = p.r.tile_a;
        ra.tile_m[0] = bm;
        ra.tile_tab[0] = p.r.tile_tab;
        ra.tile_cap[0] = p.r.tile_cap;

        GemmArgs g{};
        g.mode = 1;
        g.fmt = d.fmt;
        g.n_prob = shared ? 2 : 1;
        GemmProblem& r = g.p[0];
        r.qs1 = (const int8_t*)gate->data;
        r.d1 = (const uint16_t*)gate->scales;
        r.qs2 = (const int8_t*)up->data;
        r.d2 = (const uint16_t*)up->scales;
        r.N = d.n_ff;
        r.K = d.n_embd;
        r.bounds = p.r.bounds;
        r.tile_off = p.r.tile_a;
        r.tile_tab = p.r.tile_tab;
        r.n_seg = d.E;
        r.m_tiles_max = (int32_t)m_tiles_bound(n, d.E, bm);
        r.A = (const uint16_t*)x;
        r.lda = d.n_embd;
        r.a_rows = p.r.ids_src1;
        r.out = p.h;
        r.ldo = d.n_ff;
        r.w_once = n <= (int64_t)d.E * bm;   // at most one M tile per expert on average
        if (shared) {
            GemmProblem& q = g.p[1];
            q.qs1 = (const int8_t*)sh_gate->data;
            q.d1 = (const uint16_t*)sh_gate->scales;
            q.qs2 = (const int8_t*)sh_up->data;
            q.d2 = (const uint16_t*)sh_up->scales;
            q.N = d.n_ff_sh;
            q.K = d.n_embd;
            q.n_seg = d.S;
            q.seg_len = (int32_t)d.T;
            q.m_tiles_max = (int32_t)(d.S * ((d.T + bm - 1) / bm));
            q.A = (const uint16_t*)x;
            q.lda = d.n_embd;
            q.a_row_mod = (int32_t)d.T;
            q.out = p.hsh;
            q.ldo = d.n_ff_sh;
            q.w_once = d.T <= bm;
        }

        GemmArgs g2{};
        g2.mode = 0;
        g2.fmt = g.fmt;
        g2.n_prob = shared ? 2 : 1;
        GemmProblem& r2 = g2.p[0];
        r2.qs1 = (const int8_t*)down->data;
        r2.d1 = (const uint16_t*)down->scales;
        r2.N = d.n_embd;
        r2.K = d.n_ff;
        r2.bounds = p.r.bounds;
        r2.tile_off = p.r.tile_a;
        r2.tile_tab = p.r.tile_tab;
        r2.n_seg = d.E;
        r2.m_tiles_max = r.m_tiles_max;
        r2.A = (const uint16_t*)p.h;
        r2.lda = d.n_ff;
        r2.out = p.y;
        r2.ldo = d.n_embd;
        r2.out_rows = p.r.ids_dst;
        r2.w_once = r.w_once;
        if (shared) {
            GemmProblem& q = g2.p[1];
            q.qs1 = (const int8_t*)sh_down->data;
            q.d1 = (const uint16_t*)sh_down->scales;
            q.N = d.n_embd;
            q.K = d.n_ff_sh;
            q.n_seg = d.S;
            q.seg_len = (int32_t)d.T;
            q.m_tiles_max = g.p[1].m_tiles_max;
            q.A = (const uint16_t*)p.hsh;
            q.lda = d.n_ff_sh;
            q.out = p.ysh;
            q.ldo = d.n_embd;
            q.w_once = d.T <= bm;
        }
        // segment-last tiles of up to 160 rows where both GEMMs (and the shared ones they
        // launch with) run the wide kernel: the two share the row-id pass's tile table
        // MXFP4: every scale tensor at an even address; IQ4_NL: 4-byte, IQ4_XS: 8-byte aligned
        const uintptr_t smask = g.fmt == 3 ? 7 : (g.fmt == 2 ? 3 : 1);
        bool even = true;
        for (const moe_weights* w : {gate, up, down, sh_gate, sh_up, sh_down})
            if (w && ((uintptr_t)w->scales & smask)) even = false;
        int tx = gemm_tile_x(p.msub, g.fmt, d.n_embd, even);
        if (gemm_tile_x(p.msub, g.fmt, d.n_ff, even) == 0 ||
            (shared && gemm_tile_x(p.msub, g.fmt, d.n_ff_sh, even) == 0))
            tx = 0;
        if (tx) {
            gemm_set_tall(r, ra, 0);
            gemm_set_tall(r2, ra, 0);
        }
        // x is gathered through the row map; h and the shared rows are read in order
        if ((s = check_gemm_limits(g, p.msub, d.T, d.n_embd, "gate/up"))) return s;
        if ((s = check_gemm_limits(g2, p.msub, 0, d.n_ff, "down"))) return s;

        tm.begin();
        if ((s = hip_check(launch_row_ids(ra, st, nullptr), "row ids"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_gemm_q8(g, p.msub, st), "gate/up grouped GEMM"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_gemm_q8(g2, p.msub, st), "down grouped GEMM"))) return s;
        tm.end();
    } else {
        DecArgs a{};
        a.ids = ids;
        a.T = (int32_t)d.T;
        a.k = d.k;
        a.E = d.E;
        const int32_t fmt = d.fmt;
        a.rw = DecWeights{(const int8_t*)gate->data, (const uint16_t*)gate->scales,
                          (const int8_t*)up->data, (const uint16_t*)up->scales, d.E, d.n_ff, d.n_embd, fmt};
        if (shared)
            a.sw = DecWeights{(const int8_t*)sh_gate->data, (const uint16_t*)sh_gate->scales,
                              (const int8_t*)sh_up->data, (const uint16_t*)sh_up->scales, d.S,
                              d.n_ff_sh, d.n_embd, fmt};
        a.act = x;
        a.act_type = 1;
        a.act_B = 1;
        a.sact = x;
        a.sact_type = 1;
        a.sact_jstride = 0;
        a.out = (float*)p.h;
        a.sout = (float*)p.hsh;
        a.mode = 1;
        a.d_max = (int32_t)(n < d.E ? n : d.E);
        a.rows_per_block = 32;
        tm.begin();
        if ((s = hip_check(launch_decode(a, st), "gate/up GEMV"))) return s;
        tm.end();

        DecArgs b{};
        b.ids = ids;
        b.T = (int32_t)d.T;
        b.k = d.k;
        b.E = d.E;
        b.rw = DecWeights{(const int8_t*)down->data, (const uint16_t*)down->scales, nullptr, nullptr,
                          d.E, d.n_embd, d.n_ff, fmt};
        if (shared)
            b.sw = DecWeights{(const int8_t*)sh_down->data, (const uint16_t*)sh_down->scales, nullptr,
                              nullptr, d.S, d.n_embd, d.n_ff_sh, fmt};
        b.act = p.h;
        b.act_type = 0;
        b.act_B = d.k;
        b.sact = p.hsh;
        b.sact_type = 0;
        b.sact_jstride = d.T;
        b.out = (float*)p.y;
        b.sout = (float*)p.ysh;
        b.mode = 0;
        b.d_max = a.d_max;
        b.rows_per_block = 32;
        b.route_w = route_w;
        b.out_tok = out;
        tm.begin();
        if ((s = hip_check(launch_decode(b, st, &reduced), "down GEMV"))) return s;
        tm.end();
    }
    if (reduced) {   // the down GEMV wrote out itself
        g_stages = tm.stage;
        return MOE_OK;
    }
    ReduceArgs rd{};
    rd.ids = ids;
    rd.route_w = route_w;
    rd.T = (int32_t)d.T;
    rd.k = d.k;
    rd.E = d.E;
    rd.N = d.n_embd;
    rd.y = (const float*)p.y;
    rd.ysh = (const float*)p.ysh;
    rd.S = d.S;
    rd.out = out;
    rd.mode = 0;
    tm.begin();
    if ((s = hip_check(launch_reduce(rd, st), "reduce"))) return s;
    tm.end();
    g_stages = tm.stage;
    return MOE_OK;
}

size_t moe_mul_mat_id_workspace_size(const moe_weights* w, moe_dtype src1_type,
                                     int32_t src1_rows_per_token, int64_t n_tokens,
                                     int32_t n_used, const moe_options* opt) {
    if (validate_mmid(w, src1_type, src1_rows_per_token, n_tokens, n_used)) return 0;
    const bool q8 = w->type != MOE_F32;   // quantized experts
    if (!q8 && opt && ((opt->path != 0 && opt->path != 1) || opt->act_quant)) return 0;
    const int path = q8 ? select_path_aq(n_tokens, n_used, (int32_t)w->n_mat, w->cols, w->type, opt) : 1;
    if (path < 0) return 0;
    // the weighted and unweighted calls use the same plan size when weighted
    Carve c(nullptr);
    carve_mmid(c, n_tokens, n_used, (int32_t)w->n_mat, w->rows, true, q8, path, src1_rows_per_token,
               w->cols);
    return c.off;
}

moe_status moe_mul_mat_id(const moe_weights* w, const void* src1, moe_dtype src1_type,
                          int32_t src1_rows_per_token, const int32_t* ids, int64_t n_tokens,
                          int32_t n_used, const float* route_w, float* dst, const moe_options* opt,
                          void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    moe_status s = validate_mmid(w, src1_type, src1_rows_per_token, n_tokens, n_used);
    if (s) return s;
    if (n_tokens == 0) {
        g_stages = 0;
        return MOE_OK;
    }
    if (!src1 || !ids || !dst) return fail(MOE_EINVAL, "NULL pointer argument");
    const bool q8 = w->type != MOE_F32;   // quantized experts
    const int32_t E = (int32_t)w->n_mat, N = (int32_t)w->rows, K = (int32_t)w->cols;
    const int32_t B = src1_rows_per_token, k = n_used;
    if (!q8 && opt && opt->path != 0 && opt->path != 1)
        return fail(MOE_EINVAL, "float32 experts run the grouped fp32 product only: options.path "
                    "must be 0 or 1 (got %d)", opt->path);
    if (!q8 && opt && opt->act_quant)
        return fail(MOE_EINVAL, "quantized activations (act_quant = 1) need Q8_0 experts");
    if (!q8 && n_tokens * k * (int64_t)N >= k4GiB - 256)
        return fail(MOE_ELIMIT, "float32 mul_mat_id: n_tokens * n_used * N must be under 2^32");
    const int path = q8 ? select_path_aq(n_tokens, k, E, K, w->type, opt) : 1;
    if (path < 0) return (moe_status)path;
    const bool weighted = route_w != nullptr;
    Carve sz(nullptr);
    carve_mmid(sz, n_tokens, k, E, N, weighted, q8, path, B, K);
    if (sz.off > ws_bytes || (sz.off && !ws)) return fail(MOE_EWORKSPACE, "workspace needs %zu bytes", sz.off);
    Carve c(ws);
    const MmidPlan p = carve_mmid(c, n_tokens, k, E, N, weighted, q8, path, B, K);
    const hipStream_t st = (hipStream_t)stream;
    Timer tm(opt, st);
    const int64_t n = n_tokens * k;
    float* slot_out = weighted ? (float*)p.y : dst;  // per-slot rows [T*k][N]

    if (path == 3) {
        // quantized activations: row ids, src1 -> codes, int8 grouped GEMM, then the
        // reduce / zero fix-up below
        const int bm = kQ8aTileM;
        RowIdsArgs ra = row_ids_args(ids, n, k, E, B, p.r);
        ra.tile_off[0] = p.r.tile_a;
        ra.tile_m[0] = bm;
        ra.tile_tab[0] = p.r.tile_tab;
        ra.tile_cap[0] = p.r.tile_cap;
        QuantArgs qa{};
        qa.src_bf16 = 1;
        qa.n_part = 1;
        qa.part[0] = qpart(src1, n_tokens * B, K, p.aq, p.ad);
        GemmArgs g{};
        g.mode = 0;
        g.n_prob = 1;
        GemmProblem& r = g.p[0];
        r.qs1 = (const int8_t*)w->data;
        r.d1 = (const uint16_t*)w->scales;
        r.N = N;
        r.K = K;
        r.bounds = p.r.bounds;
        r.tile_off = p.r.tile_a;
        r.tile_tab = p.r.tile_tab;
        r.n_seg = E;
        r.m_tiles_max = (int32_t)m_tiles_bound(n, E, bm);
        r.Aq = p.aq;
        r.Ad = p.ad;
        r.a_rows = p.r.ids_src1;
        r.out = slot_out;
        r.ldo = N;
        r.out_rows = p.r.ids_dst;
        if ((uintptr_t)src1 % 16) return fail(MOE_EINVAL, "quantized activations: src1 must be 16-byte aligned");
        if ((s = check_q8a_limits(g, n_tokens * B, K, "mul_mat_id"))) return s;
        if (n_tokens * B * (K / 32) >= k4GiB) return fail(MOE_ELIMIT, "mul_mat_id: too many activation blocks");
        tm.begin();
        if ((s = hip_check(launch_row_ids(ra, st, nullptr), "row ids"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_quant_act(qa, st), "quantize src1"))) return s;
        tm.end();
        tm.begin();
        if ((s = hip_check(launch_gemm_q8a(g, st), "grouped GEMM (int8)"))) return s;
        tm.end();
    } else if (!q8 || path == 1) {
        const int bm = gemm_tile_m(p.msub);
        RowIdsArgs ra = row_ids_args(ids, n, k, E, B, p.r);
        GemmArgs g{};
        if (q8) {
            ra.tile_off[0] = p.r.tile_a;
            ra.tile_m[0] = bm;
            ra.tile_tab[0] = p.r.tile_tab;
            ra.tile_cap[0] = p.r.tile_cap;
            g.mode = 0;
            g.fmt = kernel_fmt(w->type);
            g.n_prob = 1;
            GemmProblem& r = g.p[0];
            r.qs1 = (const int8_t*)w->data;
            r.d1 = (const uint16_t*)w->scales;
            r.N = N;
            r.K = K;
            r.bounds = p.r.bounds;
            r.tile_off = p.r.tile_a;
            r.tile_tab = p.r.tile_tab;
            r.n_seg = E;
            r.m_tiles_max = (int32_t)m_tiles_bound(n, E, bm);
            r.A = (const uint16_t*)src1;
            r.lda = K;
            r.a_rows = p.r.ids_src1;
            r.out = slot_out;
            r.ldo = N;
            r.out_rows = p.r.ids_dst;
            r.w_once = n <= (int64_t)E * bm;   // at most one M tile per expert on average
            if (gemm_tile_x(p.msub, g.fmt, K, ((uintptr_t)w->scales & (g.fmt == 3 ? 7 : (g.fmt == 2 ? 3 : 1))) == 0))
                gemm_set_tall(r, ra, 0);
            if ((s = check_gemm_limits(g, p.msub, n_tokens * B, K, "mul_mat_id"))) return s;
        }
        tm.begin();
        if ((s = hip_check(launch_row_ids(ra, st, nullptr), "row ids"))) return s;
        tm.end();
        if (q8) {
            tm.begin();
            if ((s = hip_check(launch_gemm_q8(g, p.msub, st), "grouped GEMM"))) return s;
            tm.end();
        } else {
            GemmF32Args gf{};
            gf.W = (const float*)w->data;
            gf.A = (const float*)src1;
            gf.ids = ids;
            gf.ids_src1 = p.r.ids_src1;
            gf.ids_dst = p.r.ids_dst;
            gf.bounds = p.r.bounds;
            gf.n_slots = n;
            gf.E = E;
            gf.N = N;
            gf.K = K;
            gf.out = slot_out;
            tm.begin();
            if ((s = hip_check(launch_gemm_f32(gf, st), "fp32 grouped matmul"))) return s;
            tm.end();
        }
    } else {
        DecArgs a{};
        a.ids = ids;
        a.T = (int32_t)n_tokens;
        a.k = k;
        a.E = E;
        a.rw = DecWeights{(const int8_t*)w->data, (const uint16_t*)w->scales, nullptr, nullptr, E, N, K,
                          kernel_fmt(w->type)};
        a.act = src1;
        a.act_type = 1;
        a.act_B = B;
        a.out = slot_out;
        a.mode = 0;
        a.d_max = (int32_t)(n < E ? n : E);
        a.rows_per_block = 32;
        if (weighted) {
            a.route_w = route_w;
            a.out_tok = dst;
        }
        bool reduced = false;
        tm.begin();
        if ((s = hip_check(launch_decode(a, st, &reduced), "GEMV"))) return s;
        tm.end();
        if (reduced) {   // the GEMV wrote the weighted sum itself
            g_stages = tm.stage;
            return MOE_OK;
        }
    }
    ReduceArgs rd{};
    rd.ids = ids;
    rd.route_w = route_w;
    rd.T = (int32_t)n_tokens;
    rd.k = k;
    rd.E = E;
    rd.N = N;
    rd.y = slot_out;
    rd.out = dst;
    rd.mode = weighted ? 0 : 1;
    tm.begin();
    if ((s = hip_check(launch_reduce(rd, st), weighted ? "reduce" : "zero invalid slots"))) return s;
    tm.end();
    g_stages = tm.stage;
    return MOE_OK;
}

moe_status moe_quantize_act(const void* x, moe_dtype x_type, int64_t rows, int64_t K, int8_t* q,
                            float* d, void* stream) {
    g_err.clear();
    if (x_type != MOE_BF16 && x_type != MOE_F32) return fail(MOE_EINVAL, "x must be BF16 or F32");
    if (rows < 0 || K <= 0) return fail(MOE_EINVAL, "rows must be >= 0 and K > 0");
    if (K % 32) return fail(MOE_ELIMIT, "K must be a multiple of 32 (got %lld)", (long long)K);
    if (rows > 0 && (!x || !q || !d)) return fail(MOE_EINVAL, "NULL pointer argument");
    if (((uintptr_t)x | (uintptr_t)q) % 16 || (uintptr_t)d % 4)
        return fail(MOE_EINVAL, "x and q must be 16-byte aligned, d 4-byte aligned");
    if (rows > 0 && rows * (K / 32) >= k4GiB - 256)
        return fail(MOE_ELIMIT, "rows * K / 32 must be under 2^32");
    QuantArgs a{};
    a.n_part = 1;
    a.src_bf16 = x_type == MOE_BF16;
    a.part[0] = qpart(x, rows, K, q, d);
    return hip_check(launch_quant_act(a, (hipStream_t)stream), "quantize activations");
}

moe_status moe_router_topk(const float* logits, int64_t n_tokens, int32_t n_experts, int32_t n_used,
                           int32_t* ids, float* route_w, void* stream) {
    moe_status s;
    g_err.clear();
    if ((s = check_tokens(n_tokens, n_used))) return s;
    if ((s = check_experts(n_experts))) return s;
    if (n_used > n_experts)
        return fail(MOE_EINVAL, "n_used (%d) must not exceed n_experts (%d) for top-k", n_used, n_experts);
    if (n_tokens > 0 && (!logits || !ids || !route_w)) return fail(MOE_EINVAL, "NULL pointer argument");
    RouterArgs a{};
    a.logits = logits;
    a.T = n_tokens;
    a.E = n_experts;
    a.k = n_used;
    a.ids = ids;
    a.w = route_w;
    return hip_check(launch_router(a, (hipStream_t)stream), "router top-k");
}

}  // extern "C"
