// GEMV (decode) path for small batches: D1 = gate/up with silu(gate) * up,
// D2 = down projection, each over the selected experts only, with the always-on
// shared experts computed in the same launch (the pages' decode-side design fuses
// the shared experts into the quantized mat-vec kernel and checks the optional
// shared buffers for null -- "CUDA: fuse shared experts into MMVQ", llama.cpp
// release b11370).
//
// gfx950 design. Decode is a weight stream: every selected expert's Q8_0 rows are
// read from HBM exactly once per launch and applied to every token slot that uses
// that expert. The distinct experts are found on the device from ids (a wave-wide
// bitmap OR), so no row-id launch sits on the latency-critical path, and the grid is
// sized for an upper bound on them.
//   * One wave owns (one distinct expert, a chunk of R rows); R comes from the
//     kernel's resident-wave count. Each lane takes 16 contiguous int8 of a row per
//     1024-wide K piece and multiplies them exactly with the slot's activations held in
//     registers: bf16 activations as packed pairs against exact bf16 weight pairs
//     (dot2, fp32 accumulate), fp32 ones (the down projection's h) with fp32 FMAs. The
//     per-block scale multiplies the 16-term partial sum. Lane sums use DPP; lane 63
//     writes the result.
//   * One activation row per pass (single-token decode): rows are double-buffered in
//     registers, which leaves room for two or more waves per SIMD.
//   * Two per pass: the activations fill the register file, so the rows stream
//     through a per-wave ring in LDS with direct global-to-LDS copies (the bytes in
//     flight cost no registers).
//   * 4-bit experts (MXFP4, IQ4_NL, IQ4_XS): a lane takes one whole block of 32 codes (16
//     bytes) per 2048-wide K piece; MXFP4 codes convert in hardware, IQ4_NL / IQ4_XS code
//     pairs through 256-entry tables of level pairs in LDS.
//   * For larger batches or K a block kernel (4 waves per chunk of rows, activations
//     staged in LDS) takes over (Q8_0 only).
//   * Results are written per slot; the fixed-order weighted reduction runs in the
//     reduce kernel.
#include <type_traits>

#include "iq4nl.h"
#include "lds_dma.h"
#include "moe_internal.h"

// Weight loads carry the non-temporal hint: every weight row is read once per launch,
// while the activation rows are read by every wave of their expert (measured on
// single-token decode: 27.4 -> 26.1 us per layer; eight tokens: 122.7 -> 117.9 us).
#ifndef MOE_DEC_W_NT
#define MOE_DEC_W_NT 1
#endif

namespace moe {
namespace {

// weight loads carry the non-temporal hint
constexpr bool kDecWeightsNT = MOE_DEC_W_NT != 0;

constexpr int kThreads = 256;
constexpr int kR = 8;    // weight rows (row pairs for gate/up) per block
#ifndef MOE_DEC_SP
#define MOE_DEC_SP 1
#endif
constexpr int kSP = MOE_DEC_SP;   // token slots per pass

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
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

// Weight formats of the wave-level GEMV. In both, lane l of K piece i reads bytes
// 1024*i + 16*l .. +15 of a weight row: 16 Q8_0 values (k = 1024*i + 16*l ..) or 32 MXFP4
// values (k = 2048*i + 32*l .., exactly one block of 32 with one scale byte).
template <int FMT> struct Fmt;
template <> struct Fmt<0> {   // Q8_0: int8 codes, one fp16 scale per 32
    static constexpr int VPL = 16, PIECE = 1024, SB = 2;
};
template <> struct Fmt<1> {   // MXFP4: two E2M1 codes per byte (even column low), one E8M0 byte per 32
    static constexpr int VPL = 32, PIECE = 2048, SB = 1;
};
template <> struct Fmt<2> {   // IQ4_NL: two codes per byte (even column low), one fp16 scale per 32
    static constexpr int VPL = 32, PIECE = 2048, SB = 2;
};
// IQ4_XS: IQ4_NL's codes; per 256 columns one 8-byte record (fp16 d, scales_h, scales_l[4]),
// i.e. one scale byte per 32 columns. Lane l's block is block l % 8 of its super-block.
template <> struct Fmt<3> {
    static constexpr int VPL = 32, PIECE = 2048, SB = 1;
};

// IQ4_XS: the scale of block j (0..7) of a super-block from its 8-byte record r (bytes
// 0-1 fp16 d, 2-3 scales_h with block j's high sub-scale bits at 2j, 4-7 scales_l with its
// low four at 4j): d * (ls - 32), exact in fp32.
__device__ __forceinline__ float iq4xs_scale(uint64_t r, int j) {
    const uint32_t lo = (uint32_t)(r >> (32 + 4 * j)) & 15u;
    const uint32_t hi = (uint32_t)(r >> (16 + 2 * j)) & 3u;
    return (float)__builtin_bit_cast(_Float16, (uint16_t)r) * (float)((int)(lo | (hi << 4)) - 32);
}

// E8M0 scale byte -> 2^(x - 127) (x = 0 is the subnormal 2^-127; x = 255 is NaN).
__device__ __forceinline__ float e8m0_to_float(uint32_t x) {
    const uint32_t bits = x == 0 ? 0x00400000u : (x == 255 ? 0x7fc00000u : x << 23);
    return __builtin_bit_cast(float, bits);
}

// 32 MXFP4 codes (16 bytes) dotted with 32 floats. The hardware conversion turns the
// two codes of a byte into exact fp32 values (scale 1; the low nibble is the first);
// the caller multiplies the sum by the block's power-of-two scale.
__device__ __forceinline__ float dot32_fp4(const i32x4& q, const float* x) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const uint32_t u = (uint32_t)q[w];
        const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 0);
        const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 1);
        const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 2);
        const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, 3);
        s = fmaf(v0[0], x[8 * w + 0], s);
        s = fmaf(v0[1], x[8 * w + 1], s);
        s = fmaf(v1[0], x[8 * w + 2], s);
        s = fmaf(v1[1], x[8 * w + 3], s);
        s = fmaf(v2[0], x[8 * w + 4], s);
        s = fmaf(v2[1], x[8 * w + 5], s);
        s = fmaf(v3[0], x[8 * w + 6], s);
        s = fmaf(v3[1], x[8 * w + 7], s);
    }
    return s;
}

// 32 MXFP4 codes (16 bytes) dotted with 32 bf16 activations held as 16 packed pairs (raw
// dwords): each byte's two codes become an exact bf16 pair and one dot2 instruction
// multiplies it with the matching activation pair, accumulating in fp32. The caller
// multiplies the sum by the block's scale. (The pairs are kept in integer registers: held
// in float slots and bit-cast to bf16 pairs, the compiler merged distinct pairs into one.)
__device__ __forceinline__ float dot32_fp4_bf16(const i32x4& q, const uint32_t* xv) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const uint32_t u = (uint32_t)q[w];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 0),
                                            __builtin_bit_cast(bf16x2, xv[4 * w + 0]), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 1),
                                            __builtin_bit_cast(bf16x2, xv[4 * w + 1]), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 2),
                                            __builtin_bit_cast(bf16x2, xv[4 * w + 2]), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, 1.0f, 3),
                                            __builtin_bit_cast(bf16x2, xv[4 * w + 3]), s, false);
    }
    return s;
}

// IQ4_NL lookup tables in LDS, format constants each block builds at its start
// (nl_tables_init): for every byte value b (two codes; b & 15 is the even column's) the
// levels of its two codes as an exact bf16 pair (one dword) and as two fp32. A lane then
// turns two codes into operands with one LDS read (about two VALU instructions for the
// address) instead of picking levels out of registers and converting them.
__shared__ uint32_t nl_tab_bf16[256];
__shared__ __attribute__((aligned(8))) float nl_tab_f32[512];

__device__ __forceinline__ int nl_level(int c) {
    const uint32_t w = c < 4 ? kNL0 : (c < 8 ? kNL1 : (c < 12 ? kNL2 : kNL3));
    return (int8_t)(w >> (8 * (c & 3)));
}

// Fills the tables (blocks of 256 threads; IQ4_NL and IQ4_XS only) and waits for the whole block.
template <int FMT>
__device__ __forceinline__ void nl_tables_init() {
    if constexpr (FMT == 2 || FMT == 3) {
        const int t = threadIdx.x;
        const float lo = (float)nl_level(t & 15), hi = (float)nl_level(t >> 4);
        // a level has at most 7 significant bits: the top half of its fp32 form is exact
        nl_tab_bf16[t] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xffff0000u);
        nl_tab_f32[2 * t] = lo;
        nl_tab_f32[2 * t + 1] = hi;
        __syncthreads();
    }
}

// 32 IQ4_NL codes (16 bytes) dotted with 32 floats, fp32 FMAs on the exact levels; the
// caller multiplies the sum by the block's fp16 scale.
__device__ __forceinline__ float dot32_nl(const i32x4& q, const float* x) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const uint32_t u = (uint32_t)q[w];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f32x2 v = *(const f32x2*)&nl_tab_f32[2 * ((u >> (8 * i)) & 255u)];
            s = fmaf(v[0], x[8 * w + 2 * i], s);
            s = fmaf(v[1], x[8 * w + 2 * i + 1], s);
        }
    }
    return s;
}

// 32 IQ4_NL codes dotted with 32 bf16 activations held as 16 packed pairs: byte j of the
// codes is columns 2j and 2j+1, whose bf16 level pair meets activation pair j in one dot2
// instruction (fp32 accumulate).
__device__ __forceinline__ float dot32_nl_bf16(const i32x4& q, const uint32_t* xv) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const uint32_t u = (uint32_t)q[w];
#pragma unroll
        for (int i = 0; i < 4; i++)
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, nl_tab_bf16[(u >> (8 * i)) & 255u]),
                                                __builtin_bit_cast(bf16x2, xv[4 * w + i]), s, false);
    }
    return s;
}

// 16 int8 in q (four dwords) dotted with 16 bf16 activations held as 8 packed pairs:
// each pair of int8 becomes an exact bf16 pair (two conversions and one pick; |q| <= 127
// has at most 7 significant bits) for one dot2 instruction, fp32 accumulate.
__device__ __forceinline__ float dot16_bf16(const i32x4& q, const uint32_t* xv) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const uint32_t u = (uint32_t)q[w];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint32_t f0 = __builtin_bit_cast(uint32_t, (float)(int8_t)(u >> (16 * i)));
            const uint32_t f1 = __builtin_bit_cast(uint32_t, (float)(int8_t)(u >> (16 * i + 8)));
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(f1, f0, 0x07060302u)),
                                                __builtin_bit_cast(bf16x2, xv[2 * w + i]), s, false);
        }
    }
    return s;
}

// bf16 activations of Q8_0 rows kept as packed pairs too (half the registers of fp32
// copies, so more waves fit a SIMD)
#ifndef MOE_DEC_Q8_PACKED
#define MOE_DEC_Q8_PACKED 1
#endif

// Activations of one lane's piece in registers: bf16 activations are kept as packed
// pairs (VPL / 2 dwords); fp32 ones (the down projection's h) as VPL values.
template <int FMT, bool XBF16>
struct XRegs {
    static constexpr bool PACKED = (FMT != 0 || MOE_DEC_Q8_PACKED) && XBF16;
    static constexpr int N = PACKED ? Fmt<FMT>::VPL / 2 : Fmt<FMT>::VPL;
    using T = std::conditional_t<PACKED, uint32_t, float>;
};

// One lane's share of a row piece: acc + scale * (codes q . activations xv), with one
// rounding for the scaling add (fma). sb holds the raw scale bits (fp16 for Q8_0, E8M0
// for MXFP4, fp16 for IQ4_NL, the super-block record for IQ4_XS); pieces past K get a zero
// scale.
template <int FMT, bool PACKED, class XT>
__device__ __forceinline__ float piece_fma(const i32x4& q, const XT* xv, uint64_t sb, bool in, float acc) {
    if constexpr (FMT == 2 || FMT == 3) {
        const float dd = in ? (FMT == 2 ? half_bits_to_float((uint16_t)sb) : iq4xs_scale(sb, threadIdx.x & 7)) : 0.f;
        if constexpr (PACKED) return fmaf(dd, dot32_nl_bf16(q, xv), acc);
        else return fmaf(dd, dot32_nl(q, xv), acc);
    } else if constexpr (FMT == 1 && PACKED) {
        const float sc = in ? e8m0_to_float(sb & 255u) : 0.f;
        return fmaf(sc, dot32_fp4_bf16(q, xv), acc);
    } else if constexpr (FMT == 0 && PACKED) {
        const float dd = in ? half_bits_to_float((uint16_t)sb) : 0.f;
        return fmaf(dd, dot16_bf16(q, xv), acc);
    } else if constexpr (FMT == 0) {
        const float dd = in ? half_bits_to_float((uint16_t)sb) : 0.f;
        return fmaf(dd, dot16(q, f32x4{xv[0], xv[1], xv[2], xv[3]}, f32x4{xv[4], xv[5], xv[6], xv[7]},
                              f32x4{xv[8], xv[9], xv[10], xv[11]}, f32x4{xv[12], xv[13], xv[14], xv[15]}),
                    acc);
    } else {
        const float sc = in ? e8m0_to_float(sb & 255u) : 0.f;
        return fmaf(sc, dot32_fp4(q, xv), acc);
    }
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
// For n_tokens * n_used <= 64 and K <= 4096 the work is cut into units: one distinct
// routed expert with the slots routed to it, or one shared expert with every token,
// over a chunk of rows. A wave loads the ids table (one entry per lane), finds the
// distinct experts present with a wave OR of per-word bitmaps, and collects an
// expert's slots as a lane mask. It loads the activation rows of up to P of those
// slots once (lane l holds k = 1024i + 16l .. +15 of each, exact fp32) and streams the
// unit's weight rows against them: per row all NIT 16-byte pieces and scales, converted
// exactly to fp32 and accumulated per slot in fp32; lanes are summed with DPP and lane
// 63 hands each result to the caller. The activations are read once per chunk of rows
// instead of once per row.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
    for (int i = 0; i < n; i++) m &= m - 1;
    return __ffsll((unsigned long long)m) - 1;
}

// This lane's entry of the ids table; lanes past n_tokens * n_used and ids outside
// [0, E) hold -1.
__device__ __forceinline__ int lane_expert(const DecArgs& a, int lane) {
    const int v = lane < a.T * a.k ? a.ids[lane] : -1;
    return (v >= 0 && v < a.E) ? v : -1;
}

// Experts w0 .. w0+63 present in the ids table, as a bitmap (the same on every lane).
__device__ __forceinline__ uint64_t present_word(int v, int w0) {
    const int rel = v - w0;
    const bool in = v >= 0 && rel >= 0 && rel < 64;
    const uint32_t lo = wave_or_u32(in && rel < 32 ? 1u << rel : 0u);
    const uint32_t hi = wave_or_u32(in && rel >= 32 ? 1u << (rel - 32) : 0u);
    return ((uint64_t)hi << 32) | lo;
}

// The d-th distinct expert present, in ascending order; -1 if fewer are present.
__device__ __forceinline__ int nth_expert(int v, int E, int d) {
    int e = -1, seen = 0;
    for (int w0 = 0; w0 < E && e < 0; w0 += 64) {
        const uint64_t present = present_word(v, w0);
        const int c = __popcll(present);
        if (d < seen + c) e = w0 + nth_set_bit(present, d - seen);
        seen += c;
    }
    return e;
}

// Number of distinct experts present.
__device__ __forceinline__ int count_experts(int v, int E) {
    int seen = 0;
    for (int w0 = 0; w0 < E; w0 += 64) seen += __popcll(present_word(v, w0));
    return seen;
}

// The unit of global wave gw when every wave owns one unit of R rows: routed units
// first (distinct expert d = gw / chunks), then the shared ones. Returns false for waves
// past the last unit.
#ifndef MOE_DEC_SHARED_FIRST
#define MOE_DEC_SHARED_FIRST 1
#endif
__device__ __forceinline__ bool wave_unit(const DecArgs& a, int gw, int R, bool& routed, int& e,
                                          uint64_t& smask, int& cnt, int& n_lo, int& n_hi) {
    const int lane = threadIdx.x & 63;
    const int Rs = a.rows_shared > 0 ? a.rows_shared : R;
    const int nch_r = (a.rw.N + R - 1) / R;
    const int nw_r = a.d_max * nch_r;
    const int nw_s = a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + Rs - 1) / Rs) : 0;
    if (gw >= nw_r + nw_s) return false;
    // shared-expert units (several passes each) take the first waves, so they start in
    // the first round instead of forming the launch's tail. Measured per layer call on
    // one MI355X: Lite-shaped T = 8 107 -> 95 us, GPT-OSS-shaped with a shared expert T = 8
    // 162 -> 155 us, but T = 10 and 16 slower (126 -> 134, 262 -> 286 us), so only up to 8.
    const bool sh_first = MOE_DEC_SHARED_FIRST && a.T > 1 && a.T <= 8;
    const int gr = sh_first ? gw - nw_s : gw;   // index among the routed units
    routed = sh_first ? gw >= nw_s : gw < nw_r;
    int chunk;
    if (routed) {
        const int d = gr / nch_r;
        chunk = gr - d * nch_r;
        const int v = lane_expert(a, lane);
        e = nth_expert(v, a.E, d);
        if (e < 0) return false;  // fewer distinct experts than the grid allows for
        smask = __ballot(v == e);
        cnt = __popcll(smask);
    } else {
        const int nch_s = (a.sw.N + Rs - 1) / Rs;
        const int b = sh_first ? gw : gw - nw_r;
        e = b / nch_s;
        chunk = b - e * nch_s;
        smask = 0;
        cnt = a.T;
    }
    const int N = routed ? a.rw.N : a.sw.N;
    const int Ru = routed ? R : Rs;
    n_lo = chunk * Ru;
    n_hi = min(n_lo + Ru, N);
    return true;
}

// Register-staged unit: rows [n_lo, n_hi) of routed expert e (slots in smask, cnt of
// them) or of shared expert e (all tokens), streamed two at a time through registers (the
// next row's loads in flight while one computes). With one activation row per pass it
// needs few registers and keeps two or more waves per SIMD, which beats staging through
// LDS for single-token decode. emit(idx, n, res) runs on lane 63; idx is the slot t*k+s
// (routed) or the token (shared).
template <int MODE, int P, bool XBF16, int NIT, int FMT, class Emit>
__device__ __forceinline__ void unit_regs(const DecArgs& a, bool routed, int e, uint64_t smask, int cnt,
                                          int n_lo, int n_hi, Emit&& emit) {
    constexpr int M = MODE == 1 ? 2 : 1;
    using F = Fmt<FMT>;
    const int lane = threadIdx.x & 63;
    const DecWeights& W = routed ? a.rw : a.sw;
    const int N = W.N, K = W.K;
    const int64_t KB = K >> 5;
    const int64_t RB = (int64_t)K * 16 / F::VPL;   // bytes per weight row
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
    // lane's K pieces: first value k = PIECE*i + VPL*lane (bytes 1024*i + 16*lane of the
    // row); pieces past K read column 0 (a valid address) and get a zero scale
    int kc[NIT];
    bool kin[NIT];
#pragma unroll
    for (int i = 0; i < NIT; i++) {
        const int k = i * F::PIECE + lane * F::VPL;
        kin[i] = k < K;
        kc[i] = kin[i] ? k : 0;
    }
    const int8_t* q1 = W.qs1 + (int64_t)e * N * RB;
    const int8_t* q2 = MODE == 1 ? W.qs2 + (int64_t)e * N * RB : q1;
    const uint8_t* d1 = (const uint8_t*)W.d1 + (int64_t)e * N * KB * F::SB;
    const uint8_t* d2 = MODE == 1 ? (const uint8_t*)W.d2 + (int64_t)e * N * KB * F::SB : d1;

    // one weight row (pair): NIT 16-byte pieces per matrix and their scales
    struct Row {
        i32x4 q[M][NIT];
        std::conditional_t<FMT == 3, uint64_t, uint32_t> d[M][NIT];
    };
    auto load_row = [&](int n, Row& w) {
#pragma unroll
        for (int m = 0; m < M; m++) {
            const int8_t* qr = (m == 0 ? q1 : q2) + (int64_t)n * RB;
            const uint8_t* dr = (m == 0 ? d1 : d2) + (int64_t)n * KB * F::SB;
#pragma unroll
            for (int i = 0; i < NIT; i++) {
                const i32x4* qp = (const i32x4*)(qr + kc[i] * 16 / F::VPL);
                if constexpr (kDecWeightsNT) w.q[m][i] = __builtin_nontemporal_load(qp);
                else w.q[m][i] = *qp;
                if constexpr (FMT == 3) w.d[m][i] = *(const uint64_t*)(dr + 8 * (kc[i] >> 8));
                else if constexpr (FMT != 1) w.d[m][i] = *(const uint16_t*)(dr + 2 * (kc[i] >> 5));
                else w.d[m][i] = dr[kc[i] >> 5];
            }
        }
    };

    for (int p0 = 0; p0 < cnt; p0 += P) {
        const int pc = min(P, cnt - p0);
        // activations of this pass's slots: bf16 ones as packed pairs, fp32 ones as they are
        using XR = XRegs<FMT, XBF16>;
        typename XR::T x[P][NIT][XR::N];
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int64_t row = src_row(p0 + min(p, pc - 1));
#pragma unroll
            for (int i = 0; i < NIT; i++) {
                if constexpr (XR::PACKED) {
                    const uint16_t* xp = (const uint16_t*)src + row * K + kc[i];
#pragma unroll
                    for (int h = 0; h < F::VPL / 8; h++) {
                        const i32x4 r = *(const i32x4*)(xp + 8 * h);
#pragma unroll
                        for (int c = 0; c < 4; c++) x[p][i][4 * h + c] = (uint32_t)r[c];
                    }
                } else if constexpr (XBF16) {
                    const uint16_t* xp = (const uint16_t*)src + row * K + kc[i];
                    i32x4 r[F::VPL / 8];
#pragma unroll
                    for (int h = 0; h < F::VPL / 8; h++) r[h] = *(const i32x4*)(xp + 8 * h);
#pragma unroll
                    for (int c = 0; c < F::VPL / 2; c++) {
                        const uint32_t w = (uint32_t)r[c >> 2][c & 3];
                        x[p][i][2 * c] = __builtin_bit_cast(float, w << 16);
                        x[p][i][2 * c + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
                    }
                } else {
                    const float* xp = (const float*)src + row * K + kc[i];
#pragma unroll
                    for (int c = 0; c < F::VPL / 4; c++) {
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
                for (int m = 0; m < M; m++)
#pragma unroll
                    for (int p = 0; p < P; p++)   // lanes past K add 0 through a zero scale
                        acc[m][p] = piece_fma<FMT, XR::PACKED>(w.q[m][i], x[p][i], w.d[m][i], kin[i], acc[m][p]);
#pragma unroll
            for (int p = 0; p < P; p++) {
                if (p >= pc) continue;
                const float g = wave_sum_lane63(acc[0][p]);
                float res = g;
                if (MODE == 1) {
                    const float u = wave_sum_lane63(acc[M - 1][p]);
                    res = g / (1.0f + __expf(-g)) * u;
                }
                if (lane == 63) emit(slot_of(p0 + p), n, res);
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

// Per-slot results: routed rows [n_tokens * n_used][N], shared rows [n_mat][T][N].
struct EmitGlobal {
    const DecArgs& a;
    bool routed;
    int e, N;
    __device__ void operator()(int idx, int n, float res) const {
        if (routed) a.out[(int64_t)idx * N + n] = res;
        else a.sout[((int64_t)e * a.T + idx) * N + n] = res;
    }
};

// One wave per unit, register-staged rows.
template <int MODE, int P, bool XBF16, int NIT, int FMT>
__global__ __launch_bounds__(256) void k_decode_wave(DecArgs a) {
    nl_tables_init<FMT>();
    const int gw = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));  // global wave
    bool routed;
    int e, cnt, n_lo, n_hi;
    uint64_t smask;
    if (!wave_unit(a, gw, a.rows_per_block, routed, e, smask, cnt, n_lo, n_hi)) return;
    unit_regs<MODE, P, XBF16, NIT, FMT>(a, routed, e, smask, cnt, n_lo, n_hi,
                                   EmitGlobal{a, routed, e, routed ? a.rw.N : a.sw.N});
}

// ring slots per wave (gate/up pairs, single rows) and blocks per CU the registers
// are budgeted for
#ifndef MOE_DEC_NR1
#define MOE_DEC_NR1 3
#endif
#ifndef MOE_DEC_NR0
#define MOE_DEC_NR0 5
#endif
#ifndef MOE_DEC_MINB
#define MOE_DEC_MINB 2
#endif

// s_waitcnt vmcnt(after * D) for a run-time after in [0, MAXA].
template <int D, int MAXA>
__device__ __forceinline__ void wait_rows(int after) {
    if constexpr (MAXA == 0) {
        wait_vm<0>();
    } else {
        if (after >= MAXA) wait_vm<MAXA * D>();
        else wait_rows<D, MAXA - 1>(after);
    }
}

template <int MODE, int NIT>
struct StreamSlot {
    static constexpr int MAT = NIT * 1024 + 256;
    static constexpr int BYTES = (MODE == 1 ? 2 : 1) * MAT;
    static constexpr int NR_CFG = MODE == 1 ? MOE_DEC_NR1 : MOE_DEC_NR0;
    static constexpr int NR_FIT = 150 * 1024 / (4 * BYTES);
    static constexpr int NR = NR_CFG < NR_FIT ? NR_CFG : NR_FIT;   // ring slots per wave
    static constexpr int LDS = 4 * NR * BYTES;       // 4 waves per block
};

// Streaming unit (same work as unit_regs): the wave copies its weight rows (a gate/up
// pair in gate/up mode) straight from global memory into a ring of NR row slots in its
// own part of LDS, keeping NR-1 rows in flight while it multiplies the oldest: the bytes
// in flight cost no registers, so the occupancy is set by LDS, not by the row buffers. A
// wave only reads slots its own copies wrote, so no barrier is needed; its vmcnt says
// when a row has landed. Every copy has landed when the unit returns.
//
// Slot layout per matrix: NIT KB of int8 (piece i at 1024*i, lane l's 16 bytes at
// 16*l, the row's byte k at offset k) and 256 bytes for the row's fp16 scales (the
// aligned dwords holding them; the row's first scale sits at byte (row offset & 3)).
template <int MODE, int P, bool XBF16, int NIT, int FMT, class Emit>
__device__ __forceinline__ void unit_stream(const DecArgs& a, bool routed, int e, uint64_t smask,
                                            int cnt, int n_lo, int n_hi, uint8_t* ring, Emit&& emit) {
    constexpr int M = MODE == 1 ? 2 : 1;
    using F = Fmt<FMT>;
    using G = StreamSlot<MODE, NIT>;
    constexpr int MAT = G::MAT, SLOT = G::BYTES, NR = G::NR;
    constexpr int D = M * (NIT + 1);   // copies per row (pair)
    static_assert((NR - 1) * D <= 63, "vmcnt counts to 63");
    const int lane = threadIdx.x & 63;
    const DecWeights& W = routed ? a.rw : a.sw;
    const int N = W.N, K = W.K;
    const int nrows = n_hi - n_lo;
    const int KB = K >> 5;
    const int RB = K * 16 / F::VPL;   // bytes per weight row
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
    // lane's K pieces: first value k = PIECE*i + VPL*lane, bytes 1024*i + 16*lane of the
    // row. Pieces past K copy the row's last 16 bytes (a valid address), read column 0 of
    // the activations and get a zero scale.
    int kc[NIT];
    bool kin[NIT];
    uint32_t qoff[NIT];
#pragma unroll
    for (int i = 0; i < NIT; i++) {
        const int k = i * F::PIECE + lane * F::VPL;
        kin[i] = k < K;
        kc[i] = kin[i] ? k : 0;
        qoff[i] = (uint32_t)(kin[i] ? (i << 10) + (lane << 4) : RB - 16);
    }
    const int8_t* q1 = W.qs1 + (int64_t)e * N * RB;
    const int8_t* q2 = MODE == 1 ? W.qs2 + (int64_t)e * N * RB : q1;
    const uint8_t* d1 = (const uint8_t*)W.d1 + (int64_t)e * N * KB * F::SB;
    const uint8_t* d2 = MODE == 1 ? (const uint8_t*)W.d2 + (int64_t)e * N * KB * F::SB : d1;
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));

    // copies of row n into slot j: per matrix NIT 16-byte pieces and one word per lane
    // of scales (lanes past the row's last word re-read it)
    auto issue_row = [&](int n, int j) {
#pragma unroll
        for (int m = 0; m < M; m++) {
            const uint32_t dst = ring_lds + (uint32_t)(j * SLOT + m * MAT);
            const int8_t* qrow = (const int8_t*)uniform_ptr((m == 0 ? q1 : q2) + (int64_t)n * RB);
#pragma unroll
            for (int i = 0; i < NIT; i++) dma16<kDecWeightsNT>(qrow, qoff[i], dst + i * 1024);
            const uintptr_t sa = (uintptr_t)((m == 0 ? d1 : d2) + (int64_t)n * KB * F::SB);  // first scale
            const uint8_t* srow = (const uint8_t*)uniform_ptr((const void*)(sa & ~(uintptr_t)3));
            const int last = ((int)(sa & 3) + F::SB * KB - 1) >> 2;
            dma4(srow, (uint32_t)(min(lane, last) * 4), dst + NIT * 1024);
        }
    };
    // wait until row j of this pass has landed, given how many rows were sent after it
    auto wait_row = [&](int after) { wait_rows<D, NR - 1>(after); };

    for (int p0 = 0; p0 < cnt; p0 += P) {
        const int pc = min(P, cnt - p0);
        // activations of this pass's slots: bf16 ones as packed pairs, fp32 ones as they are
        using XR = XRegs<FMT, XBF16>;
        typename XR::T x[P][NIT][XR::N];
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int64_t row = src_row(p0 + min(p, pc - 1));
#pragma unroll
            for (int i = 0; i < NIT; i++) {
                if constexpr (XR::PACKED) {
                    const uint16_t* xp = (const uint16_t*)src + row * K + kc[i];
#pragma unroll
                    for (int h = 0; h < F::VPL / 8; h++) {
                        const i32x4 r = *(const i32x4*)(xp + 8 * h);
#pragma unroll
                        for (int c = 0; c < 4; c++) x[p][i][4 * h + c] = (uint32_t)r[c];
                    }
                } else if constexpr (XBF16) {
                    const uint16_t* xp = (const uint16_t*)src + row * K + kc[i];
                    i32x4 r[F::VPL / 8];
#pragma unroll
                    for (int h = 0; h < F::VPL / 8; h++) r[h] = *(const i32x4*)(xp + 8 * h);
#pragma unroll
                    for (int c = 0; c < F::VPL / 2; c++) {
                        const uint32_t w = (uint32_t)r[c >> 2][c & 3];
                        x[p][i][2 * c] = __builtin_bit_cast(float, w << 16);
                        x[p][i][2 * c + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
                    }
                } else {
                    const float* xp = (const float*)src + row * K + kc[i];
#pragma unroll
                    for (int c = 0; c < F::VPL / 4; c++) {
                        const f32x4 v = *(const f32x4*)(xp + 4 * c);
#pragma unroll
                        for (int j = 0; j < 4; j++) x[p][i][4 * c + j] = v[j];
                    }
                }
            }
        }
        auto compute_row = [&](int n, int j) {
            const uint8_t* sl = ring + j * SLOT;
            float acc[M][P];
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int p = 0; p < P; p++) acc[m][p] = 0.f;
#pragma unroll
            for (int i = 0; i < NIT; i++)
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const uint8_t* mp = sl + m * MAT;
                    const int s0 = (int)((uintptr_t)((m == 0 ? d1 : d2) + (int64_t)n * KB * F::SB) & 3);
                    const i32x4 q = *(const i32x4*)(mp + (i << 10) + (lane << 4));
                    const uint8_t* sp = mp + NIT * 1024 + s0 + (FMT == 3 ? 8 * (kc[i] >> 8) : F::SB * (kc[i] >> 5));
                    const uint64_t sb = FMT == 3 ? *(const uint64_t*)sp
                                                 : (FMT != 1 ? (uint64_t)*(const uint16_t*)sp : (uint64_t)*sp);
#pragma unroll
                    for (int p = 0; p < P; p++)   // lanes past K add 0 through a zero scale
                        acc[m][p] = piece_fma<FMT, XR::PACKED>(q, x[p][i], sb, kin[i], acc[m][p]);
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
                if (lane == 63) emit(slot_of(p0 + p), n, res);
            }
        };
        // ring: rows 0 .. NR-2 in flight before the first multiply; row j+NR-1 goes
        // into the slot row j-1 used (read completely before this point)
        for (int j = 0; j < NR - 1 && j < nrows; j++) issue_row(n_lo + j, j);
        for (int j = 0; j < nrows; j++) {
            if (j + NR - 1 < nrows) issue_row(n_lo + j + NR - 1, (j + NR - 1) % NR);
            wait_row(min(NR - 1, nrows - 1 - j));
            compute_row(n_lo + j, j % NR);
        }
    }
}

// One wave per unit, rows streamed through a per-wave LDS ring.
template <int MODE, int P, bool XBF16, int NIT, int FMT>
__global__ __launch_bounds__(256, MOE_DEC_MINB) void k_decode_stream(DecArgs a) {
    using G = StreamSlot<MODE, NIT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    nl_tables_init<FMT>();
    const int gw = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));  // global wave
    bool routed;
    int e, cnt, n_lo, n_hi;
    uint64_t smask;
    if (!wave_unit(a, gw, a.rows_per_block, routed, e, smask, cnt, n_lo, n_hi)) return;
    uint8_t* ring = smem + (threadIdx.x >> 6) * (G::NR * G::BYTES);
    unit_stream<MODE, P, XBF16, NIT, FMT>(a, routed, e, smask, cnt, n_lo, n_hi, ring,
                                     EmitGlobal{a, routed, e, routed ? a.rw.N : a.sw.N});
}

// ---------------------------------------------------------------- down with the reduce
// D2 with the weighted reduction fused in (down mode, n_tokens * n_used <= 64): a block
// owns a chunk of R output rows for every unit, the distinct routed experts and the
// shared experts, which its 4 waves take in turn (unit u on wave u mod 4). Each result
// (slot or shared token, row) goes to LDS; after one barrier, one thread per (token, row)
// sums the token's slots in ascending slot order with their routing weights, then the
// shared experts in index order, in fp32, and writes the output row once. The order and
// the operations are those of the standalone reduce, so both give identical bits.
constexpr int kFuseRows = 16;    // R, at most
constexpr int kFuseSlots = 64;   // routed slots, and shared (expert, token) pairs, at most

template <int P, bool XBF16, int NIT, bool STREAM, int FMT>
__global__ __launch_bounds__(256, STREAM ? MOE_DEC_MINB : 1) void k_decode_down_reduce(DecArgs a) {
    using G = StreamSlot<0, NIT>;
    nl_tables_init<FMT>();
    __shared__ float s_part[kFuseSlots * kFuseRows];   // routed slot s, row r at s*kFuseRows + r
    __shared__ float s_shp[kFuseSlots * kFuseRows];    // shared j, token t at (j*T + t)*kFuseRows + r
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int R = a.rows_per_block;
    const int N = a.rw.N;
    const int n_lo = (int)blockIdx.x * R, n_hi = min(n_lo + R, N);
    const int v = lane_expert(a, lane);
    const int D = count_experts(v, a.E);
    const int S = a.sw.n_mat;
    // route weight of slot `lane`: loaded now, so its round trip runs under the units'
    // work, and parked in LDS by wave 0 for the weighted sum at the end (loading the
    // weights there, slot after slot, put one round trip per slot after the units)
    __shared__ float s_w[kFuseSlots];
    __shared__ int32_t s_ok[kFuseSlots];
    const float w_l = (wv == 0 && lane < a.T * a.k && a.route_w) ? a.route_w[lane] : 1.0f;
    uint8_t* ring = smem + wv * (G::NR * G::BYTES);
    for (int u = wv; u < D + S; u += 4) {
        if (u < D) {
            const int e = nth_expert(v, a.E, u);
            const uint64_t sm = __ballot(v == e);
            auto emit = [&](int slot, int n, float res) { s_part[slot * kFuseRows + (n - n_lo)] = res; };
            if constexpr (STREAM)
                unit_stream<0, P, XBF16, NIT, FMT>(a, true, e, sm, __popcll(sm), n_lo, n_hi, ring, emit);
            else
                unit_regs<0, P, XBF16, NIT, FMT>(a, true, e, sm, __popcll(sm), n_lo, n_hi, emit);
        } else {
            const int j = u - D;
            auto emit = [&](int t, int n, float res) { s_shp[(j * a.T + t) * kFuseRows + (n - n_lo)] = res; };
            if constexpr (STREAM)
                unit_stream<0, P, XBF16, NIT, FMT>(a, false, j, 0, a.T, n_lo, n_hi, ring, emit);
            else
                unit_regs<0, P, XBF16, NIT, FMT>(a, false, j, 0, a.T, n_lo, n_hi, emit);
        }
    }
    if (wv == 0) {
        s_w[lane] = w_l;
        s_ok[lane] = v >= 0;   // slot `lane` names an expert in [0, E)
    }
    __syncthreads();
    for (int i = tid; i < a.T * R; i += 256) {
        const int t = i / R, r = i - t * R, n = n_lo + r;
        if (n >= N) continue;
        float acc = 0.f;
        for (int s = 0; s < a.k; s++) {
            const int slot = t * a.k + s;
            if (s_ok[slot]) acc = fmaf(s_w[slot], s_part[slot * kFuseRows + r], acc);
        }
        for (int j = 0; j < S; j++) acc += s_shp[(j * a.T + t) * kFuseRows + r];
        a.out_tok[(int64_t)t * N + n] = acc;
    }
}

// Waves of a kernel that fit on the chip at once (queried once per kernel and device).
template <class Kern>
hipError_t resident_waves(Kern kern, size_t lds, PerDeviceOnce& cache, int* waves) {
    return once_per_device(cache, [&](int& v) {
        int dev = 0, n_cu = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess ||
            n_cu <= 0 || per_cu <= 0) {
            n_cu = 256;
            per_cu = 2;
        }
        v = n_cu * per_cu * 4;
        return hipSuccess;
    }, waves);
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

// Rows per shared-expert unit. A routed unit usually serves one pass of slots; a shared
// unit serves all T tokens in ceil(T / P) passes over its rows, so its rows are cut by
// that many passes (at least one row) to keep it about as long as a routed unit.
#ifndef MOE_DEC_SHARED_SPLIT
#define MOE_DEC_SHARED_SPLIT 1
#endif
int shared_rows(int R, int T, int P) {
    if (!MOE_DEC_SHARED_SPLIT) return R;
    const int passes = (T + P - 1) / P;
    const int r = (R + passes - 1) / passes;
    return r < 1 ? 1 : r;
}

// Units per wave (routed experts plus shared experts over 4 waves) up to which the fused
// down + reduce kernel is used; beyond it each wave would restart its row stream too often
// and the per-unit kernels with the standalone reduce are faster.
#ifndef MOE_DEC_FUSE_UPW
#define MOE_DEC_FUSE_UPW 2
#endif
// Blocks the fused kernel aims at (R = N / blocks rows each, 1 <= R <= kFuseRows).
#ifndef MOE_DEC_FUSE_BLOCKS
#define MOE_DEC_FUSE_BLOCKS 512
#endif

template <int MODE, int P, bool XBF16, int NIT, int FMT>
hipError_t launch_stream(DecArgs a, hipStream_t st) {
    constexpr int lds = StreamSlot<MODE, NIT>::LDS;
    static_assert(lds <= 150 * 1024, "ring exceeds LDS");
    static PerDeviceOnce lds_cap, occ;   // dynamic LDS cap, resident waves: once per device
    const void* kern = (const void*)k_decode_stream<MODE, P, XBF16, NIT, FMT>;
    if (hipError_t e = set_lds_cap(lds_cap, kern, lds)) return e;
    int waves = 0;
    if (hipError_t e = resident_waves(k_decode_stream<MODE, P, XBF16, NIT, FMT>, lds, occ, &waves)) return e;
    a.rows_per_block = rows_per_wave(a, waves);
    a.rows_shared = shared_rows(a.rows_per_block, a.T, P);
    const int R = a.rows_per_block, Rs = a.rows_shared;
    const int nw = a.d_max * ((a.rw.N + R - 1) / R) +
                   (a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + Rs - 1) / Rs) : 0);
    if (nw <= 0) return hipSuccess;
    const int grid = (nw + 3) / 4;
    k_decode_stream<MODE, P, XBF16, NIT, FMT><<<grid, 256, lds, st>>>(a);
    return hipGetLastError();
}

template <int MODE, bool XBF16, int NIT, int FMT>
hipError_t launch_regs(DecArgs a, hipStream_t st) {
    static PerDeviceOnce occ;
    int waves = 0;
    if (hipError_t e = resident_waves(k_decode_wave<MODE, 1, XBF16, NIT, FMT>, 0, occ, &waves)) return e;
    a.rows_per_block = rows_per_wave(a, waves);
    a.rows_shared = shared_rows(a.rows_per_block, a.T, 1);
    const int R = a.rows_per_block, Rs = a.rows_shared;
    const int nw = a.d_max * ((a.rw.N + R - 1) / R) +
                   (a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + Rs - 1) / Rs) : 0);
    if (nw <= 0) return hipSuccess;
    k_decode_wave<MODE, 1, XBF16, NIT, FMT><<<(nw + 3) / 4, 256, 0, st>>>(a);
    return hipGetLastError();
}

template <bool XBF16, int NIT, bool STREAM, int FMT>
hipError_t launch_down_reduce(DecArgs a, hipStream_t st) {
    constexpr int lds = STREAM ? StreamSlot<0, NIT>::LDS : 0;
    constexpr int P = STREAM ? 2 : 1;
    if constexpr (STREAM) {
        static PerDeviceOnce lds_cap;
        if (hipError_t e = set_lds_cap(lds_cap, (const void*)k_decode_down_reduce<P, XBF16, NIT, STREAM, FMT>, lds))
            return e;
    }
    const int N = a.rw.N;
    int R = (N + MOE_DEC_FUSE_BLOCKS - 1) / MOE_DEC_FUSE_BLOCKS;
    R = R < 1 ? 1 : (R > kFuseRows ? kFuseRows : R);
    a.rows_per_block = R;
    const int grid = (N + R - 1) / R;
    if (grid <= 0) return hipSuccess;
    k_decode_down_reduce<P, XBF16, NIT, STREAM, FMT><<<grid, 256, lds, st>>>(a);
    return hipGetLastError();
}

// One activation row per pass: register staging. Two per pass: the two rows' fp32
// activations take too many registers to also hold rows in flight, so the rows stream
// through LDS.
template <int MODE, bool XBF16, int NIT, int FMT>
hipError_t launch_wave_nit(const DecArgs& a, int slots_max, bool fuse, hipStream_t st) {
    if constexpr (MODE == 0) {
        if (fuse) return slots_max <= 1 ? launch_down_reduce<XBF16, NIT, false, FMT>(a, st)
                                        : launch_down_reduce<XBF16, NIT, true, FMT>(a, st);
    }
    return slots_max <= 1 ? launch_regs<MODE, XBF16, NIT, FMT>(a, st)
                          : launch_stream<MODE, 2, XBF16, NIT, FMT>(a, st);
}

// K pieces per lane: ceil(K / 1024) for Q8_0, ceil(K / 2048) for MXFP4 (K <= 4096).
template <int MODE, bool XBF16, int FMT>
hipError_t launch_wave(const DecArgs& a, int slots_max, bool fuse, hipStream_t st) {
    const int kmax = max(a.rw.K, a.sw.n_mat > 0 ? a.sw.K : 0);
    const int pieces = (kmax + Fmt<FMT>::PIECE - 1) / Fmt<FMT>::PIECE;
    if constexpr (FMT != 0) {   // 2048-column pieces: K <= 4096 takes two
        return pieces <= 1 ? launch_wave_nit<MODE, XBF16, 1, FMT>(a, slots_max, fuse, st)
                           : launch_wave_nit<MODE, XBF16, 2, FMT>(a, slots_max, fuse, st);
    } else {
        if (pieces <= 1) return launch_wave_nit<MODE, XBF16, 1, FMT>(a, slots_max, fuse, st);
        if (pieces <= 2) return launch_wave_nit<MODE, XBF16, 2, FMT>(a, slots_max, fuse, st);
        if (pieces <= 3) return launch_wave_nit<MODE, XBF16, 3, FMT>(a, slots_max, fuse, st);
        return launch_wave_nit<MODE, XBF16, 4, FMT>(a, slots_max, fuse, st);
    }
}

// Gate/up mode always reads the bf16 layer input; down mode reads the fp32 h (or, for
// mul_mat_id, bf16 src1).
template <int FMT>
hipError_t launch_wave_fmt(const DecArgs& a, int slots, bool fuse, hipStream_t st) {
    if (a.mode == 1) return a.act_type == 1 ? launch_wave<1, true, FMT>(a, slots, false, st) : hipErrorInvalidValue;
    return a.act_type == 1 ? launch_wave<0, true, FMT>(a, slots, fuse, st)
                           : launch_wave<0, false, FMT>(a, slots, fuse, st);
}

}  // namespace

hipError_t launch_decode(const DecArgs& a, hipStream_t st, bool* reduced) {
    if (reduced) *reduced = false;
    if ((int64_t)a.T * a.k <= 64 && a.rw.K <= 4096 && (a.sw.n_mat == 0 || a.sw.K <= 4096)) {
        // activation rows per pass: an expert usually serves each token at most once,
        // so up to n_tokens rows; more (repeated ids) take further passes. Two rows per
        // pass keep the register budget at two or more waves per SIMD.
        const int slots = a.T;
        const bool same_type = a.sw.n_mat == 0 || a.sact_type == a.act_type;
        const int S = a.sw.n_mat > 0 ? a.sw.n_mat : 0;
        const bool fuse = a.mode == 0 && a.out_tok != nullptr && same_type &&
                          (S == 0 || a.sw.N == a.rw.N) && (int64_t)S * a.T <= kFuseSlots &&
                          a.d_max + S <= 4 * MOE_DEC_FUSE_UPW;
        if (same_type) {
            if (reduced) *reduced = fuse;
            if (a.rw.fmt == 2) return launch_wave_fmt<2>(a, slots, fuse, st);
            if (a.rw.fmt == 3) return launch_wave_fmt<3>(a, slots, fuse, st);
            return a.rw.fmt == 1 ? launch_wave_fmt<1>(a, slots, fuse, st) : launch_wave_fmt<0>(a, slots, fuse, st);
        }
    }
    if (a.rw.fmt != 0) return hipErrorInvalidValue;   // MXFP4, IQ4_NL, IQ4_XS: the wave kernels only
    const int nb_r = a.d_max * ((a.rw.N + kR - 1) / kR);
    const int nb_s = a.sw.n_mat > 0 ? a.sw.n_mat * ((a.sw.N + kR - 1) / kR) : 0;
    const int grid = nb_r + nb_s;
    if (grid <= 0) return hipSuccess;
    if (a.mode == 1) k_decode<1><<<grid, kThreads, 0, st>>>(a);
    else k_decode<0><<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
