// GEMV (decode) path for small batches: D1 = gate/up with silu(gate) * up,
// D2 = down projection, each over the selected experts only, with the always-on
// shared experts computed in the same launch (the pages' decode-side design fuses
// the shared experts into the quantized mat-vec kernel and checks the optional
// shared buffers for null -- "CUDA: fuse shared experts into MMVQ", llama.cpp
// release b11370).
//
// gfx950 design. Decode is a weight stream: every selected expert's Q8_0 rows are
// read from HBM exactly once per launch and applied to every token slot that uses
// that expert.
//   * Block = 4 wavefronts; a block owns (one distinct expert, a chunk of rows).
//     The distinct experts are found inside the block from ids (n_tokens * n_used
//     <= 256 entries): no separate row-id launch on the latency-critical path.
//   * The expert's activation rows (bf16 x, or fp32 h for the down projection) are
//     staged once per block into LDS as fp32, padded by 16 bytes per 64 so the
//     lanes' 16-float reads hit distinct banks.
//   * A wave streams one weight row per step: each lane loads 16 contiguous int8
//     (a half Q8_0 block) and its fp16 scale, converts q exactly to fp32 and does
//     fp32 FMAs against every staged slot; the per-block scale multiplies the
//     16-term partial sum. Cross-lane sums use shuffles. All arithmetic is fp32.
//   * Results are written per slot; the fixed-order weighted reduction runs in
//     the reduce kernel.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kR = 8;    // weight rows (row pairs for gate/up) per block
constexpr int kSP = 1;   // token slots per pass

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Sum over the 64 lanes of a wave with DPP moves (no LDS traffic), in a fixed
// tree: within each row of 16 lanes by shifts of 1, 2, 4, 8, then across rows by
// the row broadcasts of lanes 15 and 31. The total lands in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_term(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xf, true));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_term(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, true);
}
// Bitwise OR over the 64 lanes (same DPP tree as the sum), returned to every lane.
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
    v |= dpp_or_term<0x111, 0xf>(v);
    v |= dpp_or_term<0x112, 0xf>(v);
    v |= dpp_or_term<0x114, 0xf>(v);
    v |= dpp_or_term<0x118, 0xf>(v);
    v |= dpp_or_term<0x142, 0xa>(v);
    v |= dpp_or_term<0x143, 0xc>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float wave_sum_lane63(float v) {
    v += dpp_term<0x111, 0xf>(v);  // row_shr:1
    v += dpp_term<0x112, 0xf>(v);  // row_shr:2
    v += dpp_term<0x114, 0xf>(v);  // row_shr:4
    v += dpp_term<0x118, 0xf>(v);  // row_shr:8
    v += dpp_term<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_term<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// 16 int8 in q (four dwords) dotted with 16 floats.
__device__ __forceinline__ float dot16(const i32x4& q, const f32x4& x0, const f32x4& x1,
                                       const f32x4& x2, const f32x4& x3) {
    float s = 0.f;
    s = fmaf((float)(int8_t)(q[0]), x0[0], s);
    s = fmaf((float)(int8_t)(q[0] >> 8), x0[1], s);
    s = fmaf((float)(int8_t)(q[0] >> 16), x0[2], s);
    s = fmaf((float)(int8_t)(q[0] >> 24), x0[3], s);
    s = fmaf((float)(int8_t)(q[1]), x1[0], s);
    s = fmaf((float)(int8_t)(q[1] >> 8), x1[1], s);
    s = fmaf((float)(int8_t)(q[1] >> 16), x1[2], s);
    s = fmaf((float)(int8_t)(q[1] >> 24), x1[3], s);
    s = fmaf((float)(int8_t)(q[2]), x2[0], s);
    s = fmaf((float)(int8_t)(q[2] >> 8), x2[1], s);
    s = fmaf((float)(int8_t)(q[2] >> 16), x2[2], s);
    s = fmaf((float)(int8_t)(q[2] >> 24), x2[3], s);
    s = fmaf((float)(int8_t)(q[3]), x3[0], s);
    s = fmaf((float)(int8_t)(q[3] >> 8), x3[1], s);
    s = fmaf((float)(int8_t)(q[3] >> 16), x3[2], s);
    s = fmaf((float)(int8_t)(q[3] >> 24), x3[3], s);
    return s;
}

// Block = 4 waves; it owns kR rows (row pairs in gate/up mode) of one expert and
// every token slot routed to that expert. Wave w covers the 1024-wide K slices
// w, w+4, ...: per slice each lane loads 16 int8 of each of the block's rows, their
// fp16 scales, and 16 activation values of each slot, all issued back to back, then
// accumulates in fp32. Lane sums use DPP; the 4 waves' partial sums are added in
// wave order through LDS.
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_decode(DecArgs a) {
    constexpr int M = MODE == 1 ? 2 : 1;  // weight matrices per row (gate and up)
    __shared__ int32_t s_ids[kDecMaxSlots];
    __shared__ int32_t s_first[kDecMaxSlots];
    __shared__ int32_t s_slots[kDecMaxSlots];
    __shared__ int32_t s_wcnt[kThreads / 64];
    __shared__ int32_t s_e;
    __shared__ float s_red[kThreads / 64][kR][M][kSP];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nch_r = (a.rw.N + kR - 1) / kR;
    const int nb_r = a.d_max * nch_r;
    const bool routed = (int)blockIdx.x < nb_r;
    const DecWeights& W = routed ? a.rw : a.sw;
    const int N = W.N, K = W.K;
    int e, chunk, cnt;
    if (routed) {
        const int d = blockIdx.x / nch_r;
        chunk = blockIdx.x - d * nch_r;
        const int n = a.T * a.k;
        if (tid < n) {
            const int32_t v = a.ids[tid];
            s_ids[tid] = (v >= 0 && v < a.E) ? v : -1;
        }
        if (tid == 0) s_e = -1;
        __syncthreads();
        if (tid < n) {
            const int32_t v = s_ids[tid];
            bool first = v >= 0;
            for (int j = 0; j < tid && first; j++) first = s_ids[j] != v;
            s_first[tid] = first;
        }
        __syncthreads();
        if (tid < n && s_first[tid]) {
            const int32_t v = s_ids[tid];
            int rank = 0;
            for (int j = 0; j < n; j++) rank += (s_first[j] && s_ids[j] < v) ? 1 : 0;
            if (rank == d) s_e = v;
        }
        __syncthreads();
        e = s_e;
        if (e < 0) return;  // fewer distinct experts than the grid allows for
        // slots of expert e in ascending (t, s) order
        const bool m = tid < n && s_ids[tid] == e;
        const uint64_t bal = __ballot(m);
        if (lane == 0) s_wcnt[wv] = __popcll(bal);
        __syncthreads();
        int pre = 0;
        cnt = 0;
        for (int w = 0; w < kThreads / 64; w++) {
            if (w < wv) pre += s_wcnt[w];
            cnt += s_wcnt[w];
        }
        if (m) {
            const int r = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            s_slots[pre + r] = tid;
        }
        __syncthreads();
    } else {
        const int nch_s = (a.sw.N + kR - 1) / kR;
        const int b = blockIdx.x - nb_r;
        e = b / nch_s;
        chunk = b - e * nch_s;
        cnt = a.T;
    }

    const int n_lo = chunk * kR;
    const int n_it = (K + 1023) >> 10;
    const int64_t KB = K >> 5;
    const void* src = routed ? a.act : a.sact;
    const int atype = routed ? a.act_type : a.sact_type;
    // source activation row of slot p of this block
    auto src_row = [&](int p) -> int64_t {
        if (routed) {
            const int slot = s_slots[p];
            const int t = slot / a.k, s = slot - t * a.k;
            return (int64_t)t * a.act_B + s % a.act_B;
        }
        return (int64_t)e * a.sact_jstride + p;
    };

    for (int p0 = 0; p0 < cnt; p0 += kSP) {
        const int pc = min(kSP, cnt - p0);
        float acc[kR][M][kSP];
#pragma unroll
        for (int r = 0; r < kR; r++)
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int p = 0; p < kSP; p++) acc[r][m][p] = 0.f;
        for (int it = wv; it < n_it; it += kThreads / 64) {
            const int k = (it << 10) + (lane << 4);
            const int kc = k < K ? k : 0;  // past K: a valid address, result unused
            i32x4 q[kR][M];
            uint32_t dsc[kR][M];
#pragma unroll
            for (int r = 0; r < kR; r++) {
                const int64_t wr = (int64_t)e * N + min(n_lo + r, N - 1);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    q[r][m] = *(const i32x4*)((m == 0 ? W.qs1 : W.qs2) + wr * K + kc);
                    dsc[r][m] = (m == 0 ? W.d1 : W.d2)[wr * KB + (kc >> 5)];
                }
            }
            f32x4 xv[kSP][4];
#pragma unroll
            for (int p = 0; p < kSP; p++) {
                const int64_t off = src_row(p0 + min(p, pc - 1)) * K + kc;
                if (atype == 1) {
                    const i32x4 r0 = *(const i32x4*)((const uint16_t*)src + off);
                    const i32x4 r1 = *(const i32x4*)((const uint16_t*)src + off + 8);
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        const i32x4& rr = h ? r1 : r0;
                        xv[p][2 * h] = f32x4{__builtin_bit_cast(float, (uint32_t)rr[0] << 16),
                                             __builtin_bit_cast(float, (uint32_t)rr[0] & 0xffff0000u),
                                             __builtin_bit_cast(float, (uint32_t)rr[1] << 16),
                                             __builtin_bit_cast(float, (uint32_t)rr[1] & 0xffff0000u)};
                        xv[p][2 * h + 1] = f32x4{__builtin_bit_cast(float, (uint32_t)rr[2] << 16),
                                                 __builtin_bit_cast(float, (uint32_t)rr[2] & 0xffff0000u),
                                                 __builtin_bit_cast(float, (uint32_t)rr[3] << 16),
                                                 __builtin_bit_cast(float, (uint32_t)rr[3] & 0xffff0000u)};
                    }
                } else {
                    const float* xp = (const float*)src + off;
#pragma unroll
                    for (int c = 0; c < 4; c++) xv[p][c] = *(const f32x4*)(xp + 4 * c);
                }
            }
            {
#pragma unroll
                for (int r = 0; r < kR; r++)
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        const float d = k < K ? half_bits_to_float((uint16_t)dsc[r][m]) : 0.f;
#pragma unroll
                        for (int p = 0; p < kSP; p++)
                            if (p < pc)
                                acc[r][m][p] = fmaf(d, dot16(q[r][m], xv[p][0], xv[p][1], xv[p][2], xv[p][3]),
                                                    acc[r][m][p]);
                    }
            }
        }
#pragma unroll
        for (int r = 0; r < kR; r++)
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int p = 0; p < kSP; p++) {
                    if (p < pc) {
                        const float v = wave_sum_lane63(acc[r][m][p]);
                        if (lane == 63) s_red[wv][r][m][p] = v;
                    }
                }
        __syncthreads();
        if (tid < kR * pc) {
            const int r = tid / pc, p = tid - r * pc;
            const int nrow = n_lo + r;
            float g = 0.f, u = 0.f;
            for (int w = 0; w < kThreads / 64; w++) {
                g += s_red[w][r][0][p];
                if (MODE == 1) u += s_red[w][r][M - 1][p];
            }
            const float res = MODE == 1 ? g / (1.0f + __expf(-g)) * u : g;
            if (nrow < N) {
                if (routed) a.out[(int64_t)s_slots[p0 + p] * N + nrow] = res;
                else a.sout[((int64_t)e * a.T + p0 + p) * N + nrow] = res;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- wave-level fast path
// For n_tokens * n_used <= 64 and K <= 4096: every wave is an independent unit (no
// LDS, no barriers). Wave g of the grid owns R consecutive rows (row pairs in gate/up
// mode) of one expert. It loads the ids table (one entry per lane), finds the distinct
// experts present with a wave OR of per-word bitmaps, takes the d-th, and collects
// that expert's slots as a lane mask. It then loads the activation rows of up to P of
// those slots into registers once (lane l holds k = 1024i + 16l .. +15 of each), and
// streams its R weight rows against them: per row all NIT 16-byte pieces and scales
// are loaded back to back, converted exactly to fp32 and accumulated per slot in fp32;
// lanes are summed with DPP and lane 63 writes. The activations are read once per R
// rows instead of once per row.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
    for (int i = 0; i < n; i++) m &= m - 1;
    return __ffsll((unsigned long long)m) - 1;
}

template <int MODE, int P, bool XBF16, int NIT>
__global__ __launch_bounds__(256) void k_decode_wave(DecArgs a) {
    constexpr int M = MODE == 1 ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int gw = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));  // global wave
    const int R = a.rows_per_block;  // rows per wave
    const int nch_r = (a.rw.N + R - 1) / R;
    const int nw_r = a.d_max * nch_r;
    const int nw_s = a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + R - 1) / R) : 0;
    if (gw >= nw_r + nw_s) return;
    const bool routed = gw < nw_r;
    const DecWeights& W = routed ? a.rw : a.sw;
    const int N = W.N, K = W.K;
    int e, chunk, cnt;
    uint64_t smask = 0;  // routed: lanes (entries t*k+s) of this expert
    if (routed) {
        const int d = gw / nch_r;
        chunk = gw - d * nch_r;
        const int n = a.T * a.k;
        int v = lane < n ? a.ids[lane] : -1;
        if (v >= a.E) v = -1;
        // distinct experts present: a 64-expert bitmap word at a time (wave OR), the
        // d-th set bit over the words in ascending order is this wave's expert
        e = -1;
        int seen = 0;
        for (int w0 = 0; w0 < a.E && e < 0; w0 += 64) {
            const int rel = v - w0;
            const bool in = v >= 0 && rel >= 0 && rel < 64;
            const uint32_t lo = wave_or_u32(in && rel < 32 ? 1u << rel : 0u);
            const uint32_t hi = wave_or_u32(in && rel >= 32 ? 1u << (rel - 32) : 0u);
            const uint64_t present = ((uint64_t)hi << 32) | lo;
            const int c = __popcll(present);
            if (d < seen + c) e = w0 + nth_set_bit(present, d - seen);
            seen += c;
        }
        if (e < 0) return;  // fewer distinct experts than the grid allows for
        smask = __ballot(v == e);
        cnt = __popcll(smask);
    } else {
        const int nch_s = (a.sw.N + R - 1) / R;
        const int b = gw - nw_r;
        e = b / nch_s;
        chunk = b - e * nch_s;
        cnt = a.T;
    }
    const int n_lo = chunk * R;
    const int n_hi = min(n_lo + R, N);
    const int64_t KB = K >> 5;
    const void* src = routed ? a.act : a.sact;
    auto slot_of = [&](int p) -> int { return routed ? nth_set_bit(smask, p) : p; };
    auto src_row = [&](int p) -> int64_t {
        if (routed) {
            const int slot = slot_of(p);
            const int t = slot / a.k, s = slot - t * a.k;
            return (int64_t)t * a.act_B + s % a.act_B;
        }
        return (int64_t)e * a.sact_jstride + p;
    };
    // lane's K pieces: k = 1024*i + 16*lane; pieces past K read column 0 (a valid
    // address) and get a zero scale
    int kc[NIT];
    bool kin[NIT];
#pragma unroll
    for (int i = 0; i < NIT; i++) {
        const int k = (i << 10) + (lane << 4);
        kin[i] = k < K;
        kc[i] = kin[i] ? k : 0;
    }
    const int8_t* q1 = W.qs1 + (int64_t)e * N * K;
    const int8_t* q2 = MODE == 1 ? W.qs2 + (int64_t)e * N * K : q1;
    const uint16_t* d1 = W.d1 + (int64_t)e * N * KB;
    const uint16_t* d2 = MODE == 1 ? W.d2 + (int64_t)e * N * KB : d1;

    // one weight row (pair): NIT 16-byte pieces per matrix and their scales
    struct Row {
        i32x4 q[M][NIT];
        uint32_t d[M][NIT];
    };
    auto load_row = [&](int n, Row& w) {
#pragma unroll
        for (int m = 0; m < M; m++) {
            const int8_t* qr = (m == 0 ? q1 : q2) + (int64_t)n * K;
            const uint16_t* dr = (m == 0 ? d1 : d2) + (int64_t)n * KB;
#pragma unroll
            for (int i = 0; i < NIT; i++) {
                w.q[m][i] = *(const i32x4*)(qr + kc[i]);
                w.d[m][i] = dr[kc[i] >> 5];
            }
        }
    };

    for (int p0 = 0; p0 < cnt; p0 += P) {
        const int pc = min(P, cnt - p0);
        // activations of this pass's slots, exact fp32
        float x[P][NIT][16];
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int64_t row = src_row(p0 + min(p, pc - 1));
#pragma unroll
            for (int i = 0; i < NIT; i++) {
                if constexpr (XBF16) {
                    const uint16_t* xp = (const uint16_t*)src + row * K + kc[i];
                    const i32x4 r0 = *(const i32x4*)(xp);
                    const i32x4 r1 = *(const i32x4*)(xp + 8);
#pragma unroll
                    for (int c = 0; c < 8; c++) {
                        const uint32_t w = (uint32_t)(c < 4 ? r0[c] : r1[c - 4]);
                        x[p][i][2 * c] = __builtin_bit_cast(float, w << 16);
                        x[p][i][2 * c + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
                    }
                } else {
                    const float* xp = (const float*)src + row * K + kc[i];
#pragma unroll
                    for (int c = 0; c < 4; c++) {
                        const f32x4 v = *(const f32x4*)(xp + 4 * c);
#pragma unroll
                        for (int j = 0; j < 4; j++) x[p][i][4 * c + j] = v[j];
                    }
                }
            }
        }
        auto compute_row = [&](int n, const Row& w) {
            float acc[M][P];
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int p = 0; p < P; p++) acc[m][p] = 0.f;
#pragma unroll
            for (int i = 0; i < NIT; i++)
#pragma unroll
                for (int m = 0; m < M; m++) {
                    // lanes past K add 0 through a zero scale instead of branching
                    const float dd = kin[i] ? half_bits_to_float((uint16_t)w.d[m][i]) : 0.f;
#pragma unroll
                    for (int p = 0; p < P; p++) {
                        const float* xv = x[p][i];
                        acc[m][p] = fmaf(dd, dot16(w.q[m][i], f32x4{xv[0], xv[1], xv[2], xv[3]},
                                                   f32x4{xv[4], xv[5], xv[6], xv[7]},
                                                   f32x4{xv[8], xv[9], xv[10], xv[11]},
                                                   f32x4{xv[12], xv[13], xv[14], xv[15]}),
                                         acc[m][p]);
                    }
                }
#pragma unroll
            for (int p = 0; p < P; p++) {
                if (p >= pc) continue;
                const float g = wave_sum_lane63(acc[0][p]);
                float res = g;
                if (MODE == 1) {
                    const float u = wave_sum_lane63(acc[M - 1][p]);
                    res = g / (1.0f + __expf(-g)) * u;
                }
                if (lane == 63) {
                    if (routed) a.out[(int64_t)slot_of(p0 + p) * N + n] = res;
                    else a.sout[((int64_t)e * a.T + p0 + p) * N + n] = res;
                }
            }
        };
        // rows in pairs, the next row's loads in flight while one computes; loads past
        // the last row re-read the last row (unconditional, so the waits stay exact)
        Row wa, wb;
        load_row(n_lo, wa);
        for (int n = n_lo; n < n_hi; n += 2) {
            load_row(min(n + 1, n_hi - 1), wb);
            compute_row(n, wa);
            if (n + 1 >= n_hi) break;
            load_row(min(n + 2, n_hi - 1), wa);
            compute_row(n + 1, wb);
        }
    }
}

// Waves of a kernel that fit on the chip at once (queried once per kernel).
template <class Kern>
int resident_waves(Kern kern, int& cache) {
    if (cache == 0) {
        int dev = 0, n_cu = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
            n_cu <= 0 || per_cu <= 0) {
            n_cu = 256;
            per_cu = 2;
        }
        cache = n_cu * per_cu * 4;
    }
    return cache;
}

// Rows per wave, at least 4 so the per-wave start (ids, expert search, activation
// loads) is amortised. When one resident round of waves covers the grid's upper bound
// on rows with at most 8 rows per wave, use exactly one round (no partial second
// round); otherwise aim at about 8 waves per SIMD over the chip, several rounds, so
// that grids sized for more experts than the batch uses still fill the chip.
int rows_per_wave(const DecArgs& a, int waves) {
    const int64_t rows = (int64_t)a.d_max * a.rw.N + (a.sw.n_mat > 0 ? (int64_t)a.sw.n_mat * a.sw.N : 0);
    const int64_t one_round = (rows + waves - 1) / waves;
    int64_t r = one_round <= 8 ? one_round : (rows + 256 * 4 * 8 - 1) / (256 * 4 * 8);
    return (int)(r < 4 ? 4 : (r > 32 ? 32 : r));
}

template <int MODE, bool XBF16, int NIT>
hipError_t launch_wave_nit(DecArgs a, int slots_max, hipStream_t st) {
    static int cache1 = 0, cache2 = 0;
    const int waves = slots_max <= 1 ? resident_waves(k_decode_wave<MODE, 1, XBF16, NIT>, cache1)
                                     : resident_waves(k_decode_wave<MODE, 2, XBF16, NIT>, cache2);
    a.rows_per_block = rows_per_wave(a, waves);
    const int R = a.rows_per_block;
    const int nw = a.d_max * ((a.rw.N + R - 1) / R) +
                   (a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + R - 1) / R) : 0);
    if (nw <= 0) return hipSuccess;
    const int grid = (nw + 3) / 4;
    if (slots_max <= 1) k_decode_wave<MODE, 1, XBF16, NIT><<<grid, 256, 0, st>>>(a);
    else k_decode_wave<MODE, 2, XBF16, NIT><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

template <int MODE, bool XBF16>
hipError_t launch_wave(const DecArgs& a, int slots_max, hipStream_t st) {
    const int kmax = max(a.rw.K, a.sw.n_mat > 0 ? a.sw.K : 0);
    if (kmax <= 1024) return launch_wave_nit<MODE, XBF16, 1>(a, slots_max, st);
    if (kmax <= 2048) return launch_wave_nit<MODE, XBF16, 2>(a, slots_max, st);
    if (kmax <= 3072) return launch_wave_nit<MODE, XBF16, 3>(a, slots_max, st);
    return launch_wave_nit<MODE, XBF16, 4>(a, slots_max, st);
}

}  // namespace

hipError_t launch_decode(const DecArgs& a, hipStream_t st) {
    if ((int64_t)a.T * a.k <= 64 && a.rw.K <= 4096 && (a.sw.n_mat == 0 || a.sw.K <= 4096)) {
        // activation rows per pass: an expert usually serves each token at most once,
        // so up to n_tokens rows; more (repeated ids) take further passes. Two rows per
        // pass keep the register budget at two or more waves per SIMD.
        const int slots = a.T;
        const bool same_type = a.sw.n_mat == 0 || a.sact_type == a.act_type;
        if (same_type) {
            if (a.mode == 1) return a.act_type == 1 ? launch_wave<1, true>(a, slots, st)
                                                    : launch_wave<1, false>(a, slots, st);
            return a.act_type == 1 ? launch_wave<0, true>(a, slots, st) : launch_wave<0, false>(a, slots, st);
        }
    }
    const int nb_r = a.d_max * ((a.rw.N + kR - 1) / kR);
    const int nb_s = a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + kR - 1) / kR) : 0;
    const int grid = nb_r + nb_s;
    if (grid <= 0) return hipSuccess;
    if (a.mode == 1) k_decode<1><<<grid, kThreads, 0, st>>>(a);
    else k_decode<0><<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
