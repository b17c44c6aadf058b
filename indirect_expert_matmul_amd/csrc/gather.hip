// Row gather into expert order (K2): dst[j][:] = src1[ids_src1[j]][:], the copy of the
// src1 rows into the order the row-id maps give ("CUDA: better MoE implementation",
// section 2.1: ids_src1 names the src1 row each position of the expert-grouped buffer
// reads; section 2 describes the old atomic-slot copy, k_copy_src1_to_contiguous, that
// this gather replaces with a plain indexed copy).
//
// The library's own grouped GEMM does not call this: it reads the gathered rows through
// the same map straight into LDS. The standalone form serves callers that want the
// expert-contiguous copy itself, and measures what the gather costs on its own.
//
// gfx950: one wave per destination row, 16-byte vector loads and stores (a row of n_embd
// bf16 is n_embd/8 chunks; each lane keeps four chunks in flight), four rows per block of
// 256 threads. Positions whose index falls outside [0, src1_rows) get a zero row.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Gathered rows are written once: non-temporal stores keep them from evicting the source
// rows, which every one of a token's k positions reads again, from the last-level cache
// (V3-shaped input: 283 -> 267 us per gather).
__device__ __forceinline__ void st16(i32x4* p, const i32x4& v) { __builtin_nontemporal_store(v, p); }

// rows of 16-byte chunks (row bytes % 16 == 0, both bases 16-byte aligned)
__global__ __launch_bounds__(256) void k_gather_vec(GatherArgs a) {
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= a.n) return;
    const int lane = threadIdx.x & 63;
    const int64_t nc = a.row_bytes >> 4;
    const int32_t r = a.idx[j];
    i32x4* d = (i32x4*)((uint8_t*)a.dst + j * a.row_bytes);
    if ((uint32_t)r >= (uint64_t)a.src_rows) {
        for (int64_t c = lane; c < nc; c += 64) d[c] = i32x4{0, 0, 0, 0};
        return;
    }
    const i32x4* s = (const i32x4*)((const uint8_t*)a.src + (int64_t)r * a.row_bytes);
    int64_t c = lane;
    for (; c + 192 < nc; c += 256) {
        const i32x4 v0 = s[c], v1 = s[c + 64], v2 = s[c + 128], v3 = s[c + 192];
        st16(d + c, v0);
        st16(d + c + 64, v1);
        st16(d + c + 128, v2);
        st16(d + c + 192, v3);
    }
    for (; c < nc; c += 64) st16(d + c, s[c]);
}

// any row size: 2-byte elements
__global__ __launch_bounds__(256) void k_gather_u16(GatherArgs a) {
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= a.n) return;
    const int lane = threadIdx.x & 63;
    const int64_t ne = a.row_bytes >> 1;
    const int32_t r = a.idx[j];
    uint16_t* d = (uint16_t*)((uint8_t*)a.dst + j * a.row_bytes);
    const bool ok = (uint32_t)r < (uint64_t)a.src_rows;
    const uint16_t* s = (const uint16_t*)((const uint8_t*)a.src + (int64_t)(ok ? r : 0) * a.row_bytes);
    for (int64_t c = lane; c < ne; c += 64) d[c] = ok ? s[c] : (uint16_t)0;
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t st) {
    if (a.n <= 0) return hipSuccess;
    const int64_t grid = (a.n + 3) / 4;
    const bool vec = a.row_bytes % 16 == 0 && ((uintptr_t)a.src & 15) == 0 && ((uintptr_t)a.dst & 15) == 0;
    if (vec) k_gather_vec<<<(unsigned)grid, 256, 0, st>>>(a);
    else k_gather_u16<<<(unsigned)grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
