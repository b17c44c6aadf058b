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

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kU = 8;   // slots whose rows are loaded together
constexpr int kSh = 2;  // shared-expert rows loaded together with the first slots

// Block = one token x 1024 columns; each thread owns 4 consecutive columns. The
// token's ids and weights are block-uniform; the k slot rows are loaded kU at a
// time before they are summed in slot order, and the first kSh shared-expert rows
// are loaded with the first of those batches. Every row is read once and every
// output written once, so both go through non-temporal accesses: they do not
// displace lines that other kernels will read again (V3-shaped layer, 2.35 GB
// moved: 453 -> 379 us).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_reduce_weighted(ReduceArgs a) {
    const int ncb = (a.N + 4 * kThreads - 1) / (4 * kThreads);
    const int t = blockIdx.x / ncb;
    const int c = ((blockIdx.x - t * ncb) * kThreads + threadIdx.x) * 4;
    if (c >= a.N) return;
    const int64_t tk = (int64_t)t * a.k;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f32x4 vsh[kSh];
    if (VEC) {
#pragma unroll
        for (int j = 0; j < kSh; j++)
            vsh[j] = j < a.S ? __builtin_nontemporal_load((const f32x4*)(a.ysh + ((int64_t)j * a.T + t) * a.N + c))
                             : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < a.k; s0 += kU) {
        f32x4 v[kU];
        float w[kU];
        bool okv[kU];
        // Every slot row of the batch is loaded at once, whatever its id (rows past k
        // re-read slot k-1, rows of invalid ids are read and not used): the loads do not
        // wait for the ids, and no load sits under a condition whose join would make the
        // compiler wait for it there.
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int s = min(s0 + u, a.k - 1);
            const float* y = a.y + (tk + s) * a.N + c;
            if (VEC) {
                v[u] = __builtin_nontemporal_load((const f32x4*)y);
            } else {
                for (int q = 0; q < 4; q++) v[u][q] = y[min(q, a.N - 1 - c)];
            }
        }
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int s = s0 + u;
            const int32_t e = s < a.k ? a.ids[tk + s] : -1;
            const bool ok = e >= 0 && e < a.E;
            okv[u] = ok;
            w[u] = ok ? (a.route_w ? a.route_w[tk + s] : 1.0f) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kU; u++) {
            if (okv[u]) {
                acc[0] = fmaf(w[u], v[u][0], acc[0]);
                acc[1] = fmaf(w[u], v[u][1], acc[1]);
                acc[2] = fmaf(w[u], v[u][2], acc[2]);
                acc[3] = fmaf(w[u], v[u][3], acc[3]);
            }
        }
    }
    for (int j = 0; j < a.S; j++) {
        const float* y = a.ysh + ((int64_t)j * a.T + t) * a.N + c;
        if (VEC) {
            const f32x4 v = j < kSh ? vsh[j] : __builtin_nontemporal_load((const f32x4*)y);
            acc[0] += v[0];
            acc[1] += v[1];
            acc[2] += v[2];
            acc[3] += v[3];
        } else {
            for (int q = 0; q < 4; q++)
                if (c + q < a.N) acc[q] += y[q];
        }
    }
    float* o = a.out + (int64_t)t * a.N + c;
    if (VEC) {
        __builtin_nontemporal_store(acc, (f32x4*)o);
    } else {
        for (int q = 0; q < 4; q++)
            if (c + q < a.N) o[q] = acc[q];
    }
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
        if ((int64_t)a.T * a.N == 0) return hipSuccess;
        const int64_t ncb = (a.N + 4 * kThreads - 1) / (4 * kThreads);
        const unsigned grid = (unsigned)(ncb * a.T);
        const bool vec = (a.N % 4) == 0;  // 16-byte aligned rows (buffers are 256-byte aligned)
        if (vec) k_reduce_weighted<true><<<grid, kThreads, 0, st>>>(a);
        else k_reduce_weighted<false><<<grid, kThreads, 0, st>>>(a);
    } else {
        const int64_t n = (int64_t)a.T * a.k * a.N;
        if (n == 0) return hipSuccess;
        k_zero_invalid<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
