// IQ4_NL codes -> levels on gfx950, shared by the GEMV and grouped-GEMM kernels.
//
// IQ4_NL (ggml's 4-bit member of the IQ series; the pages name IQ-series experts,
// "CUDA: better MoE implementation" section 3.2 and the TensorSharp MoE-offload page's
// UD-IQ4_XS models, without defining the formats): blocks of 32 4-bit codes share one
// fp16 scale d, and a code c stands for d * level[c], the 16 levels being ggml's fixed
// non-uniform table of signed integers. Storage here: two codes per byte, the even
// column in the low nibble (the MXFP4 packing), scales as Q8_0's.
//
// The table lives in four dwords of signed bytes; v_perm_b32 picks bytes out of a pair
// of dwords by 3-bit selectors, so one lookup of four codes is two picks (levels 0-7
// and 8-15) and a third pick choosing between them by bit 3 of each code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr uint32_t nl_pack(int a, int b, int c, int d) {
    return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
           ((uint32_t)(uint8_t)d << 24);
}
constexpr uint32_t kNL0 = nl_pack(-127, -104, -83, -65);
constexpr uint32_t kNL1 = nl_pack(-49, -35, -22, -10);
constexpr uint32_t kNL2 = nl_pack(1, 13, 25, 38);
constexpr uint32_t kNL3 = nl_pack(53, 69, 89, 113);

// Four codes (one per byte, 0..15) -> their four levels as signed bytes.
__device__ __forceinline__ uint32_t nl_levels4(uint32_t c) {
    const uint32_t s = c & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(kNL1, kNL0, s);   // levels 0..7
    const uint32_t hi = __builtin_amdgcn_perm(kNL3, kNL2, s);   // levels 8..15
    // byte i comes from hi (selector i + 4) when bit 3 of code i is set, else lo (i)
    return __builtin_amdgcn_perm(hi, lo, ((c >> 1) & 0x04040404u) | 0x03020100u);
}

// Eight codes (one dword, column 2i in the low nibble of byte i) -> the levels of
// columns 0-3 (c03) and 4-7 (c47) as signed bytes in column order.
__device__ __forceinline__ void nl_levels8(uint32_t w, uint32_t& c03, uint32_t& c47) {
    const uint32_t ev = nl_levels4(w & 0x0F0F0F0Fu);          // columns 0, 2, 4, 6
    const uint32_t od = nl_levels4((w >> 4) & 0x0F0F0F0Fu);   // columns 1, 3, 5, 7
    c03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);
    c47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);
}

}  // namespace moe
