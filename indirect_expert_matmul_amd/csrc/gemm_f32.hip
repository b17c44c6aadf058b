// fp32 grouped product over expert segments (mul_mat_id with float32 experts and
// activations, section 1.2 of "CUDA: better MoE implementation"): one thread per
// (sorted row j, output column n) runs the K-long dot product in ascending order and
// writes dst row ids_dst[j]. It serves small fp32 layers, where launch latency,
// not arithmetic, sets the time.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_gemm_f32(GemmF32Args a) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t j = idx / a.N;
    const int n = (int)(idx - j * a.N);
    if (j >= a.n_slots || j >= a.bounds[a.E]) return;  // invalid-id rows sit past bounds[E]
    const int32_t slot = a.ids_dst[j];
    const int32_t e = a.ids[slot];
    const float* w = a.W + ((int64_t)e * a.N + n) * a.K;
    const float* x = a.A + (int64_t)a.ids_src1[j] * a.K;
    float acc = 0.f;
    for (int c = 0; c < a.K; c++) acc = fmaf(w[c], x[c], acc);
    a.out[(int64_t)slot * a.N + n] = acc;
}

}  // namespace

hipError_t launch_gemm_f32(const GemmF32Args& a, hipStream_t st) {
    const int64_t n = a.n_slots * a.N;
    if (n == 0) return hipSuccess;
    k_gemm_f32<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
