// Router top-k: the step ahead of the indirect matmul, turning router logits into
// the ids table the op consumes ("CUDA: better MoE implementation", section 1.2:
// ids names, per token, the experts it uses) and the routing weights, a softmax
// renormalised over each token's picks.
//
// gfx950 design: one wavefront per token. Lane l holds logits l, l+64, ... (up to
// 64*NC experts) in registers. Each of the k rounds takes the largest remaining logit
// with a wave max, breaks ties towards the lower expert index with a wave min over
// the tied candidates, and clears that entry in its owner lane; the round's value is
// parked in lane r%64 of slot r/64. The weights are exp(v_r - v_0) over their sum,
// summed by slot in a fixed butterfly order, so every run gives the same bits. No
// atomics, no LDS.
//
// Non-finite logits. Candidates are compared by an unsigned key that orders floats
// as numbers (sign-magnitude flipped to two's-complement order, -0 taken as +0) and
// puts NaN at 0, strictly below -inf. For the weights a NaN pick counts as -inf; when
// the largest pick v_0 is itself infinite the softmax is replaced by its limit: the
// picks equal to v_0 share the weight equally and the rest get 0.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;  // tokens per block

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m));
    return v;
}
// Order key of a logit: larger numbers give larger keys; NaN gives 0, below -inf
// (whose key is 0x007fffff).
__device__ __forceinline__ uint32_t rank_key(float x) {
    if (x != x) return 0u;
    const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m));
    return v;
}
// Butterfly sum: lanes i and i^m add the same two values, so every lane ends with
// the same bits and the order is fixed.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

template <int NC>
__global__ __launch_bounds__(64 * kWaves) void k_router_topk(RouterArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int E = a.E, k = a.k;
    const float* l = a.logits + t * E;
    uint32_t key[NC];
    float v[NC];   // the logit, NaN taken as -inf (the value a NaN pick is weighted by)
    uint32_t avail = 0;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int e = lane + 64 * c;
        const float x = e < E ? l[e] : -INFINITY;
        key[c] = rank_key(x);
        v[c] = x != x ? -INFINITY : x;
        if (e < E) avail |= 1u << c;
    }
    float pv[NC];   // picked value of round r in lane r%64, slot r/64
#pragma unroll
    for (int c = 0; c < NC; c++) pv[c] = -INFINITY;
    for (int r = 0; r < k; r++) {
        uint32_t bk = 0;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int e = lane + 64 * c;
            // indices grow with c, so a strictly larger key or the first available
            // entry replaces the running best
            if (((avail >> c) & 1) && (key[c] > bk || bi == 0x7fffffff)) {
                bk = key[c];
                bv = v[c];
                bi = e;
            }
        }
        const uint32_t mk = wave_max(bi != 0x7fffffff ? bk : 0u);
        const int win = wave_min(bi != 0x7fffffff && bk == mk ? bi : 0x7fffffff);
        const float m = __shfl(bv, win & 63);
        if (lane == (win & 63)) avail &= ~(1u << (win >> 6));
        if (lane == 0) a.ids[t * k + r] = win;
#pragma unroll
        for (int c = 0; c < NC; c++)
            if (c == (r >> 6) && lane == (r & 63)) pv[c] = m;
    }
    const float m0 = __shfl(pv[0], 0);   // round 0 holds the largest logit
    const bool fin = __builtin_isfinite(m0);
    float ex[NC];
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const bool live = lane + 64 * c < k;
        ex[c] = !live ? 0.f : fin ? expf(pv[c] - m0) : (pv[c] == m0 ? 1.f : 0.f);
        sum += wave_sum(ex[c]);
    }
#pragma unroll
    for (int c = 0; c < NC; c++)
        if (lane + 64 * c < k) a.w[t * k + lane + 64 * c] = ex[c] / sum;
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((a.T + kWaves - 1) / kWaves);
    const int nc = (a.E + 63) / 64;
    if (nc <= 1) k_router_topk<1><<<grid, 64 * kWaves, 0, st>>>(a);
    else if (nc <= 2) k_router_topk<2><<<grid, 64 * kWaves, 0, st>>>(a);
    else if (nc <= 4) k_router_topk<4><<<grid, 64 * kWaves, 0, st>>>(a);
    else if (nc <= 8) k_router_topk<8><<<grid, 64 * kWaves, 0, st>>>(a);
    else k_router_topk<16><<<grid, 64 * kWaves, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
