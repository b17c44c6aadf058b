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
constexpr int kMaxP = 8;               // activation rows staged per pass
constexpr int kActLds = 48 * 1024;     // LDS bytes for staged activations

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// padded LDS index of element k of a staged row (16 floats + 4 pad per group)
__device__ __forceinline__ int xpad(int k) { return (k >> 4) * 20 + (k & 15); }
__host__ __device__ __forceinline__ int padded_width(int K) { return ((K + 15) >> 4) * 20; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// 16 int8 in q (four dwords) dotted with 16 staged floats at xs.
__device__ __forceinline__ float dot16(const i32x4& q, const float* xs) {
    const f32x4 x0 = *(const f32x4*)(xs + 0);
    const f32x4 x1 = *(const f32x4*)(xs + 4);
    const f32x4 x2 = *(const f32x4*)(xs + 8);
    const f32x4 x3 = *(const f32x4*)(xs + 12);
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

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_decode(DecArgs a, int P) {
    extern __shared__ __attribute__((aligned(16))) float xs[];
    __shared__ int32_t s_ids[kDecMaxSlots];
    __shared__ int32_t s_first[kDecMaxSlots];
    __shared__ int32_t s_slots[kDecMaxSlots];
    __shared__ int32_t s_wcnt[kThreads / 64];
    __shared__ int32_t s_e;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int RB = a.rows_per_block;
    const int nch_r = (a.rw.N + RB - 1) / RB;
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
        const int nch_s = (a.sw.N + RB - 1) / RB;
        const int b = blockIdx.x - nb_r;
        e = b / nch_s;
        chunk = b - e * nch_s;
        cnt = a.T;
    }

    const int KP = padded_width(K);
    const int n_lo = chunk * RB, n_hi = min(n_lo + RB, N);
    const int n_it = (K + 1023) >> 10;
    const int64_t KB = K >> 5;
    for (int p0 = 0; p0 < cnt; p0 += P) {
        const int pc = min(P, cnt - p0);
        // ---- stage activation rows p0 .. p0+pc-1 (fp32, padded)
        for (int idx = tid; idx < pc * (K >> 2); idx += kThreads) {
            const int p = idx / (K >> 2);
            const int k = (idx - p * (K >> 2)) << 2;
            const int slot = routed ? s_slots[p0 + p] : (p0 + p);
            f32x4 v;
            if (routed) {
                const int t = slot / a.k, s = slot - t * a.k;
                const int64_t row = (int64_t)t * a.act_B + s % a.act_B;
                if (a.act_type == 1) {
                    const uint16_t* src = (const uint16_t*)a.act + row * K + k;
                    v = f32x4{bf16_bits_to_float(src[0]), bf16_bits_to_float(src[1]),
                              bf16_bits_to_float(src[2]), bf16_bits_to_float(src[3])};
                } else {
                    v = *(const f32x4*)((const float*)a.act + row * K + k);
                }
            } else {
                const int64_t row = (int64_t)e * a.sact_jstride + slot;
                if (a.sact_type == 1) {
                    const uint16_t* src = (const uint16_t*)a.sact + row * K + k;
                    v = f32x4{bf16_bits_to_float(src[0]), bf16_bits_to_float(src[1]),
                              bf16_bits_to_float(src[2]), bf16_bits_to_float(src[3])};
                } else {
                    v = *(const f32x4*)((const float*)a.sact + row * K + k);
                }
            }
            *(f32x4*)(xs + p * KP + xpad(k)) = v;
        }
        __syncthreads();
        // ---- stream weight rows
        for (int nrow = n_lo + wv; nrow < n_hi; nrow += kThreads / 64) {
            float acc1[kMaxP], acc2[kMaxP];
#pragma unroll
            for (int p = 0; p < kMaxP; p++) acc1[p] = acc2[p] = 0.f;
            const int64_t wrow = (int64_t)e * N + nrow;
            const int8_t* q1 = W.qs1 + wrow * K;
            const uint16_t* d1 = W.d1 + wrow * KB;
            const int8_t* q2 = MODE == 1 ? W.qs2 + wrow * K : nullptr;
            const uint16_t* d2 = MODE == 1 ? W.d2 + wrow * KB : nullptr;
            for (int it = 0; it < n_it; it++) {
                const int k = (it << 10) + (lane << 4);
                if (k < K) {
                    const i32x4 qa = *(const i32x4*)(q1 + k);
                    const float da = half_bits_to_float(d1[k >> 5]);
                    i32x4 qb;
                    float db = 0.f;
                    if (MODE == 1) {
                        qb = *(const i32x4*)(q2 + k);
                        db = half_bits_to_float(d2[k >> 5]);
                    }
                    const float* xk = xs + xpad(k);
#pragma unroll
                    for (int p = 0; p < kMaxP; p++) {
                        if (p < pc) {
                            acc1[p] = fmaf(da, dot16(qa, xk + p * KP), acc1[p]);
                            if (MODE == 1) acc2[p] = fmaf(db, dot16(qb, xk + p * KP), acc2[p]);
                        }
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < kMaxP; p++) {
                if (p < pc) {
                    const float g = wave_sum(acc1[p]);
                    float r = g;
                    if (MODE == 1) {
                        const float u = wave_sum(acc2[p]);
                        r = g / (1.0f + __expf(-g)) * u;
                    }
                    if (lane == 0) {
                        if (routed) a.out[(int64_t)s_slots[p0 + p] * N + nrow] = r;
                        else a.sout[((int64_t)e * a.T + p0 + p) * N + nrow] = r;
                    }
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_decode(const DecArgs& a, hipStream_t st) {
    const int RB = a.rows_per_block;
    const int nb_r = a.d_max * ((a.rw.N + RB - 1) / RB);
    const int nb_s = a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + RB - 1) / RB) : 0;
    const int grid = nb_r + nb_s;
    if (grid <= 0) return hipSuccess;
    // rows staged per pass: enough for every slot of an expert when it fits
    int P = a.act_B == 1 ? a.T : a.T * a.k;
    if (nb_s && a.T > P) P = a.T;
    if (P > kMaxP) P = kMaxP;
    const int64_t wmax = (nb_s && a.sw.K > a.rw.K) ? a.sw.K : a.rw.K;
    const int64_t row_bytes = (int64_t)padded_width((int)wmax) * 4;
    while (P > 1 && P * row_bytes > kActLds) P--;
    const size_t lds = (size_t)(P * row_bytes);
    if (a.mode == 1) k_decode<1><<<grid, kThreads, lds, st>>>(a, P);
    else k_decode<0><<<grid, kThreads, lds, st>>>(a, P);
    return hipGetLastError();
}

}  // namespace moe
