// Deterministic scatter / reduction (K5): the step that writes results back in
// token order after the expert-grouped products ("CUDA: better MoE implementation",
// sections 2.1 and 5: reorder and reduce by a precomputed map, device pointers
// only, no atomics).
//
// One thread owns one output element and sums its token's slots in ascending slot
// order, then the shared experts in index order, in fp32 -- the same order on every
// run, so results are bitwise repeatable. Per-slot rows arrive already in slot
// order (the grouped GEMM and the GEMV write row ids_dst[j] = t*k + s), so the
// reads of one token are k consecutive rows.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_reduce_weighted(ReduceArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (int64_t)a.T * a.N) return;
    const int t = (int)(idx / a.N), c = (int)(idx - (int64_t)t * a.N);
    float acc = 0.f;
    for (int s = 0; s < a.k; s++) {
        const int32_t e = a.ids[(int64_t)t * a.k + s];
        if (e < 0 || e >= a.E) continue;
        const float w = a.route_w ? a.route_w[(int64_t)t * a.k + s] : 1.0f;
        acc = fmaf(w, a.y[((int64_t)t * a.k + s) * a.N + c], acc);
    }
    for (int j = 0; j < a.S; j++) acc += a.ysh[((int64_t)j * a.T + t) * a.N + c];
    a.out[idx] = acc;
}

// Per-slot output: rows of slots whose id is out of range are zero.
__global__ __launch_bounds__(kThreads) void k_zero_invalid(ReduceArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t n = (int64_t)a.T * a.k * a.N;
    if (idx >= n) return;
    const int64_t slot = idx / a.N;
    const int32_t e = a.ids[slot];
    if (e < 0 || e >= a.E) a.out[idx] = 0.f;
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st) {
    if (a.mode == 0) {
        const int64_t n = (int64_t)a.T * a.N;
        if (n == 0) return hipSuccess;
        k_reduce_weighted<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
    } else {
        const int64_t n = (int64_t)a.T * a.k * a.N;
        if (n == 0) return hipSuccess;
        k_zero_invalid<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
