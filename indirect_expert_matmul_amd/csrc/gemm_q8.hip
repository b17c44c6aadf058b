// Grouped GEMM over expert segments (K3 gate/up, K4 down) for Q8_0 experts and
// bf16 activations on gfx950 MFMA.
//
// What it computes: for every expert segment, out_rows = A_rows x W_e^T, where the
// segment's rows are the src1 rows the row-id pass grouped under expert e (the
// quantized grouped product over expert-sorted rows that the pages' mmq_id path
// runs, "CUDA: better MoE implementation", section 2.1). In gate/up mode the block
// also applies the fused up/gate epilogue silu(gate) * up (section 4.2 names the
// fused up/gate MoE forward). Shared experts ride in the same launch as a second
// "problem" whose segments are all tokens in order.
//
// gfx950 design (not the pages' CUDA tiling):
//   * Block = W wavefronts (4 or 8). Block tile = BM activation rows (BM = 32*MSUB,
//     all inside one expert segment) x 32*W weight rows; wave w owns 32 weight rows
//     (one MFMA column group) and all BM rows, so every weight is dequantized once
//     per block and the activation tile is shared through LDS.
//   * One pipeline stage = 128 columns of K (four Q8_0 blocks). Every operand of a
//     stage goes global -> LDS with direct copies (global_load_lds): activations
//     (gathered row by row through the row map), the int8 weights (a whole 128-byte
//     line per weight row, so no line is fetched twice) and the fp16 scales. NS
//     stages are in flight; the waits are explicit vmcnt counts, one barrier per
//     stage. Two 4-wave blocks per CU (64-row tiles) keep independent pipelines
//     going; measured on gfx950 this beats one block with a deeper ring.
//   * Dequant: each lane turns 32 int8 of its weight row (one Q8_0 block) into
//     bf16(d*q) (d*q exact in fp32, one rounding to bf16, nearest-even) straight
//     into MFMA B-operand registers.
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulate. Inside a 64-wide half of a stage,
//     lane half h and element e of MFMA sub-step ss stand for k = 32h + 8ss + e on
//     BOTH operands, so A and B agree on k whatever order the unit sums in.
//   * LDS tiles use XOR swizzles of the 16-byte chunk index so MFMA operand reads
//     and dequant reads are free of bank conflicts.
//   * Gate/up mode: a wave's 32 weight rows are 16 gate rows and the 16 up rows of
//     the same outputs; lane l (l%32 < 16) meets its up partner l+16 in the
//     epilogue through a lane exchange.
//   * Block index -> tile is XCD-aware (see k_gemm_q8). Tiles are located on device
//     from the row-id pass's M-tile prefix (no host readback); blocks past the real
//     tile count exit at once.
#include <type_traits>

#include "iq4nl.h"
#include "lds_dma.h"

#include "moe_internal.h"

// Wave priority (s_setprio) while a step issues its MFMAs, so that of the two waves on a
// SIMD the one in its multiply phase issues first. Measured (same box, A/B, two runs):
// Q8_0 on the wide kernel V3-shaped gate/up 4,763 -> 4,440 us, Skew gate/up 294 -> 285 us
// (priority 3; 1 gives nearly the same); the narrow kernel's Q8_0 down (Lite) 64.5 -> 62.2
// us with priority 1, but its gate/up 117.8 -> 121.5 us, and MXFP4 on the wide kernel
// 0.7-1% slower, so only those two forms raise it.
template <bool WIDE, int MODE, int FMT>
constexpr int mfma_prio() {
    if constexpr (FMT != 0) return 0;
    else return WIDE ? 3 : (MODE == 0 ? 1 : 0);
}
#ifndef MOE_GEMM_CFG2
#define MOE_GEMM_CFG2 4, 2   // waves, pipeline stages: 64-row tiles
#endif
#ifndef MOE_GEMM_CFG4
#define MOE_GEMM_CFG4 8, 2   // the same for 128-row tiles
#endif

namespace moe {
namespace {

// A weight copy, with the non-temporal hint when the slab is read once (wave-uniform).
__device__ __forceinline__ void dma16_w(bool once, const void* base, uint32_t voff, uint32_t lds_base) {
    if (once) dma16<true>(base, voff, lds_base);
    else dma16<false>(base, voff, lds_base);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// 8 int8 (two dwords) * d -> 8 bf16 (RNE).
__device__ __forceinline__ bf16x8 dequant8(int lo, int hi, float d) {
    bf16x8 r;
    r[0] = (__bf16)((float)(int8_t)(lo) * d);
    r[1] = (__bf16)((float)(int8_t)(lo >> 8) * d);
    r[2] = (__bf16)((float)(int8_t)(lo >> 16) * d);
    r[3] = (__bf16)((float)(int8_t)(lo >> 24) * d);
    r[4] = (__bf16)((float)(int8_t)(hi) * d);
    r[5] = (__bf16)((float)(int8_t)(hi >> 8) * d);
    r[6] = (__bf16)((float)(int8_t)(hi >> 16) * d);
    r[7] = (__bf16)((float)(int8_t)(hi >> 24) * d);
    return r;
}

// Chunk swizzles. Activation rows are 256 bytes (16 chunks): chunk c of row r sits at
// c ^ (r & 15), so the 16 rows of one read phase cover all 64 banks once. Weight rows
// are 128 bytes (8 chunks): c ^ ((r & 7) ^ ((r >> 3) & 1)) keeps rows r and r+8 apart.
__device__ __forceinline__ int swz_a(int r) { return r & 15; }
__device__ __forceinline__ int swz_b(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// MXFP4 weight rows are 64 bytes per stage (4 chunks, 4 rows per 256-byte bank row):
// chunk c of row r sits at c ^ ((r >> 2) & 3), so 16 rows reading the same logical
// chunk hit 16 different bank groups.
__device__ __forceinline__ int swz_b4(int r) { return (r >> 2) & 3; }

// 8 MXFP4 codes (one dword, even value in each low nibble) -> 8 bf16. The E8M0 scale
// byte x goes into the exponent field of the conversion's scale operand, which the
// hardware applies as 2^(x - 127); fp4 times a power of two is exact in bf16.
__device__ __forceinline__ bf16x8 dequant8_fp4(uint32_t w, float sc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int MODE, int W>
constexpr int out_cols() { return MODE == 1 ? 16 * W : 32 * W; }

#ifndef MOE_GEMM_MCHUNK
#define MOE_GEMM_MCHUNK 4
#endif
constexpr int kMChunk = MOE_GEMM_MCHUNK;   // M tiles sharing each weight slab in turn

// Per stage, in LDS (NS stages in a ring):
//   A  BM rows x 256 B of bf16 activations (128 K columns)
//   B  32*W weight rows x 128 B of int8
//   S  32*W rows x 4 aligned 4-byte words, word i holding the fp16 scale of block i
// SG = 1: each stage carries its rows' scales (one aligned word per block). SG = 4 (when
// K % 512 == 0 and the scale rows are 16-byte aligned): the scales of four stages come
// as 32 bytes per row into a two-slot ring, a quarter of the memory requests; one word
// per row per stage costs as many requests as the weight rows themselves.
// FMT = 1: MXFP4 experts (64-byte weight rows per stage, E8M0 scale bytes, SG = 1).
// FMT = 2: IQ4_NL experts (the same 64-byte rows of 4-bit codes, fp16 scales, SG = 1):
// the codes become their levels (signed bytes) and then take the Q8_0 dequant.
// FMT = 3: IQ4_XS experts (IQ4_NL's codes; a stage is half of a 256-column super-block,
// whose 8-byte record of scales comes as two words per row; K % 256 == 0, two slots).
template <int MSUB, int MODE, int W, int NS, int SG, int FMT>
__global__ __launch_bounds__(64 * W) void k_gemm_q8(GemmArgs args) {
    constexpr int BM = 32 * MSUB;
    constexpr int NTW = out_cols<MODE, W>();     // output columns per block
    constexpr int A_BYTES = BM * 256;
    constexpr int WROW = FMT != 0 ? 64 : 128;    // weight bytes per row per stage
    constexpr int B_BYTES = W * 32 * WROW;
    static_assert(FMT == 0 || SG == 1, "4-bit formats' scales come one word per block per stage");
    static_assert(FMT != 3 || NS == 2, "IQ4_XS: a stage's half of the super-block follows from s % 2");
    constexpr int S_BYTES = SG == 1 ? W * 32 * 16 : 0;
    constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    constexpr int SGROUP = W * 32 * 32;          // SG = 4: one group, 32 bytes per row
    static_assert(SG == 1 || SG == 4, "scale groups of one or four stages");
    constexpr int NA = BM / (4 * W);             // activation copies (1 KB) per wave per stage
    // copies per wave per stage with per-stage scales: NA activation, the weight copies
    // and two scale-word copies
    constexpr int VM_STAGE = NA + (FMT != 0 ? 2 : 4) + 2;
    static_assert(NS == 2 || (NS == 3 && SG == 1),
                  "a two-slot ring, or a three-slot one with a fixed copy count per stage");
    static_assert(NA * 4 * W == BM, "activation rows must split evenly over the waves");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int32_t s_orow[BM];

    // ---- tile of this block. The grid holds, per problem, 8 equal parts sized by an
    // upper bound on the tile count; part x runs on XCD x (the dispatcher deals block b
    // to XCD b mod 8). The problem's real tiles are ordered by expert, then by chunk of
    // up to kMChunk M tiles, then N tile, then M tile inside the chunk, and cut into 8
    // contiguous ranges, one per XCD: the M tiles of a chunk, which share each slab of
    // weights, are dispatched back to back on one XCD, so the slab comes from HBM once
    // per chunk, while the chunk's activation tiles stay in that XCD's L2 across the
    // N tiles.
    int b = (int)blockIdx.x, pi = 0;
    {
        const GemmProblem& P0 = args.p[0];
        const int reg0 = ((P0.m_tiles_max * ((P0.N + NTW - 1) / NTW) + 7) >> 3) * 8;
        if (b >= reg0) {
            pi = 1;
            b -= reg0;
        }
    }
    const GemmProblem& P = args.p[pi];
    const int N = P.N, K = P.K;
    const int n_nt = (N + NTW - 1) / NTW;
    int e, m0, m_len, nt;
    {
        const int m_tiles = P.bounds ? P.tile_off[P.n_seg] : P.n_seg * ((P.seg_len + BM - 1) / BM);
        const int total = m_tiles * n_nt;
        const int part = (total + 7) >> 3;
        const int q = b >> 3;
        const int t = (b & 7) * part + q;
        if (q >= part || t >= total) return;
        // expert e owns tiles [n_nt * first_e, n_nt * (first_e + tiles_e)), so the
        // M tile index t / n_nt falls inside e's M-tile range
        int first, tiles, row0, rows;
        if (P.bounds) {
            const int mt = t / n_nt;
            if (P.tile_tab) {
                const int4 ti = *(const int4*)(P.tile_tab + 4 * (int64_t)mt);
                e = ti.x;
                first = ti.y;
                row0 = ti.z;
                rows = ti.w;
            } else {
                int lo = 0, hi = P.n_seg;  // tile_off[lo] <= mt < tile_off[hi]
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (P.tile_off[mid] <= mt) lo = mid; else hi = mid;
                }
                e = lo;
                first = P.tile_off[e];
                row0 = P.bounds[e];
                rows = P.bounds[e + 1] - row0;
            }
            tiles = (rows + BM - 1) / BM;
        } else {
            tiles = (P.seg_len + BM - 1) / BM;
            e = t / (n_nt * tiles);
            first = e * tiles;
            row0 = e * P.seg_len;
            rows = P.seg_len;
        }
        // position inside the expert: M tiles in chunks of kMChunk; a chunk runs its N
        // tiles in turn, each across the chunk's M tiles
        const int r = t - n_nt * first;
        const int c = r / (kMChunk * n_nt);
        const int g = min(kMChunk, tiles - c * kMChunk);
        const int rr = r - c * kMChunk * n_nt;
        nt = rr / g;
        const int j = c * kMChunk + (rr - nt * g);
        m0 = row0 + j * BM;
        m_len = min(BM, rows - j * BM);
    }

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR
    const int nsteps = (K + 127) >> 7;
    const int KB = K >> 5;
    const bool w_once = P.w_once != 0;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    if (tid < BM) {
        const int j = m0 + min(tid, m_len - 1);
        s_orow[tid] = P.out_rows ? P.out_rows[j] : j;
    }

    // weight row (within the expert) of local row l (0..31) of this wave. Gate/up
    // mode: rows 0..15 are gate rows, 16..31 the up rows of the same outputs.
    auto wrow = [&](int l) -> int {
        const int n = MODE == 1 ? nt * NTW + wv * 16 + (l & 15) : nt * NTW + wv * 32 + l;
        return min(n, N - 1);
    };

    // ---- copy geometry: wave-uniform bases, per-lane 32-bit byte offsets (stage 0).
    // Rows that are not gathered sit next to each other inside the tile and are
    // addressed from the tile's first row, so their offsets stay small whatever the
    // size of A; gathered rows are addressed from A itself (the host keeps a gathered
    // A under 4 GiB).
    const int64_t a_row0 = P.a_rows ? 0 : (P.a_row_mod ? m0 % P.a_row_mod : m0);
    const uint8_t* a_base = (const uint8_t*)uniform_ptr((const uint8_t*)P.A + a_row0 * P.lda * 2);
    uint32_t a_off[NA];
    int a_lc[NA];
#pragma unroll
    for (int i = 0; i < NA; i++) {
        const int R = (wv * NA + i) * 4 + (lane >> 4);  // tile row this lane fetches
        const int lc = (lane & 15) ^ swz_a(R);           // logical 16-byte chunk
        const int j = m0 + min(R, m_len - 1);
        const int64_t src = P.a_rows ? (int64_t)P.a_rows[j] : (int64_t)(j - m0);
        a_off[i] = (uint32_t)(src * P.lda * 2 + lc * 16);
        a_lc[i] = lc;
    }
    // weights: copy i covers local rows 8i..8i+7 (8 lanes x 16 B per row); in gate/up
    // mode copies 0-1 read gate rows and 2-3 up rows
    // (4-bit codes: copy i covers local rows 16i..16i+15, 4 lanes x 16 B per row; copy 0
    // the gate rows and 1 the up rows)
    constexpr int NB = FMT != 0 ? 2 : 4;           // weight copies per wave per stage
    const int64_t RB = FMT != 0 ? K / 2 : K;       // bytes per weight row
    const int8_t* b_base1 = (const int8_t*)uniform_ptr(P.qs1 + (int64_t)e * N * RB);
    const int8_t* b_base2 = MODE == 1 ? (const int8_t*)uniform_ptr(P.qs2 + (int64_t)e * N * RB) : b_base1;
    uint32_t b_off[NB];
    int b_lc[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const int l = FMT != 0 ? 16 * i + (lane >> 2) : 8 * i + (lane >> 3);
        const int lc = FMT != 0 ? (lane & 3) ^ swz_b4(wv * 32 + l) : (lane & 7) ^ swz_b(wv * 32 + l);
        b_off[i] = (uint32_t)((int64_t)wrow(l) * RB + lc * 16);
        b_lc[i] = lc;
    }
    // scales: copy t covers local rows 16t..16t+15, lane -> (row 16t + lane/4, block
    // lane%4 of the stage); the copy fetches the aligned word holding that fp16
    constexpr int SB = (FMT == 1 || FMT == 3) ? 1 : 2;   // scale bytes per block
    const uint8_t* s_base1 = (const uint8_t*)uniform_ptr((const uint8_t*)P.d1 + (int64_t)e * N * KB * SB);
    const uint8_t* s_base2 =
        MODE == 1 ? (const uint8_t*)uniform_ptr((const uint8_t*)P.d2 + (int64_t)e * N * KB * SB) : s_base1;
    int s_row[2];
    uint32_t s_word[2];  // aligned word of the scale at stage 0; stage s adds 4*SB*s bytes
    const int s_blk = lane & 3;
#pragma unroll
    for (int t = 0; t < 2; t++) {
        s_row[t] = wrow(16 * t + (lane >> 2));
        s_word[t] = (uint32_t)(((int64_t)s_row[t] * KB + s_blk) * SB) & ~3u;
        // IQ4_XS: word s_blk & 1 of the super-block record (stage s adds 8 * (s / 2) bytes)
        if constexpr (FMT == 3) s_word[t] = (uint32_t)((int64_t)s_row[t] * KB + 4 * (s_blk & 1));
    }
    // SG = 4: lane l fetches 16 bytes (half l&1 of the group's 32) of local row l>>1,
    // from the row's own tensor (gate and up rows sit in different tensors)
    const uint8_t* sg_ptr;
    {
        const int l = lane >> 1;
        const uint16_t* dt = (MODE == 1 && l >= 16) ? P.d2 : P.d1;
        sg_ptr = FMT != 0 ? nullptr : (const uint8_t*)(dt + ((int64_t)e * N + wrow(l)) * KB) + 16 * (lane & 1);
    }
    const uint32_t sring = lds0 + (uint32_t)(NS * STAGE);

    // Issue the copies of stage s into LDS slot s % NS. The last stage may end inside
    // K: activation chunks past K re-read chunk 0 of the stage, weight chunks past K
    // re-read the stage's first 16 bytes, scales past K re-read block KB-1 (all zeroed
    // at use), so every address stays inside its row.
    auto issue = [&](int s, int slot) {
        const uint32_t st = lds0 + (uint32_t)(slot * STAGE);
        const int k0 = s * 128;
        if (k0 + 128 <= K) {   // wave-uniform: every stage but a partial last one
#pragma unroll
            for (int i = 0; i < NA; i++)
                dma16(a_base + (int64_t)k0 * 2, a_off[i], st + (wv * NA + i) * 1024);
#pragma unroll
            for (int i = 0; i < NB; i++)
                dma16_w(w_once, ((MODE == 1 && i >= NB / 2) ? b_base2 : b_base1) + k0 * WROW / 128, b_off[i],
                        st + A_BYTES + wv * 32 * WROW + i * 1024);
            if (SG == 1) {
#pragma unroll
                for (int t = 0; t < 2; t++)
                    dma4((MODE == 1 && t == 1) ? s_base2 : s_base1,
                         s_word[t] + (FMT == 3 ? 8 * (s >> 1) : 4 * SB * s),
                         st + A_BYTES + B_BYTES + wv * 512 + t * 256);
            } else if ((s & 3) == 0) {
                dma16v(sg_ptr + 8 * s, sring + (uint32_t)(((s >> 2) & 1) * SGROUP) + wv * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NA; i++) {
                const uint32_t adj = (k0 + a_lc[i] * 8 >= K) ? (uint32_t)(a_lc[i] * 16) : 0u;
                dma16(a_base + (int64_t)k0 * 2, a_off[i] - adj, st + (wv * NA + i) * 1024);
            }
#pragma unroll
            for (int i = 0; i < NB; i++) {
                // chunk lc holds columns k0 + lc*16 (Q8_0) or k0 + lc*32 (4-bit codes) on
                const uint32_t adj = (k0 + b_lc[i] * (FMT != 0 ? 32 : 16) >= K) ? (uint32_t)(b_lc[i] * 16) : 0u;
                dma16_w(w_once, ((MODE == 1 && i >= NB / 2) ? b_base2 : b_base1) + k0 * WROW / 128, b_off[i] - adj,
                        st + A_BYTES + wv * 32 * WROW + i * 1024);
            }
            if (SG == 1) {   // (SG = 4 needs K % 512 == 0, IQ4_XS K % 256 == 0: no partial stage)
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const int blk = FMT == 3 ? 0 : min(4 * s + s_blk, KB - 1);
                    const uint32_t byte = (uint32_t)(((int64_t)s_row[t] * KB + blk) * SB);
                    dma4((MODE == 1 && t == 1) ? s_base2 : s_base1, byte & ~3u,
                         st + A_BYTES + B_BYTES + wv * 512 + t * 256);
                }
            }
        }
    };

    f32x16 acc[MSUB];
#pragma unroll
    for (int i = 0; i < MSUB; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][v] = 0.f;

    // dequant geometry of this lane: local weight row l32; in half u it takes the
    // 32-byte block 2u + h of the stage = chunks 4u + 2h and 4u + 2h + 1
    const int lrow = wv * 32 + l32;
    const int b_rd = A_BYTES + lrow * WROW;
    const int s_rd = A_BYTES + B_BYTES + wv * 512 + l32 * 16;
    // where in each aligned scale word the scale sits (constant over stages: stages
    // start at a multiple of 4 blocks): the half (fp16) or the byte (E8M0)
    int s_sh[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int64_t sidx = (int64_t)wrow(l32) * KB + 2 * u + h;
        s_sh[u] = FMT == 1 ? (int)(sidx & 3) * 8 : ((sidx & 1) ? 16 : 0);
    }

    // One step: wait for stage s, send stage s+1 into the other slot, dequantize and
    // multiply. SLOT is s % 2 as a constant, so the LDS offsets become immediates;
    // CHECK_K zeroes the scales of blocks past K and is only needed on the last stage.
    auto step = [&](int s, auto slot_c, auto check_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr bool CHECK_K = decltype(check_c)::value;
        if constexpr (NS == 2) {
            wait_stage_and_barrier<0>();   // stage s landed; nobody still reads the other slot
            if (s + 1 < nsteps) issue(s + 1, SLOT ^ 1);
        } else {
            // stage s landed (stage s+1 may still be in flight: its copies are the last
            // VM_STAGE of this wave); nobody still reads slot (s+2) % 3, used by stage s-1
            if (s + 1 < nsteps) wait_stage_and_barrier<VM_STAGE>();
            else wait_stage_and_barrier<0>();
            if (s + 2 < nsteps) issue(s + 2, (SLOT + 2) % 3);
        }
        const uint8_t* st = smem + SLOT * STAGE;
        const int k0 = s * 128;
        // the stage's weights (both 64-column halves) and scales; both halves always
        // run (a half past K has zero scales): a conditional MFMA would make the
        // compiler copy the accumulators between register files each step
        i32x4 q[2][2];
        float d[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            if constexpr (FMT == 1) {
                // one 16-byte chunk = this lane's block of 32 codes; blocks past K get zero
                // codes (a zero scale operand would still mean 2^-127)
                q[u][0] = *(const i32x4*)(st + b_rd + (((2 * u + h) ^ swz_b4(lrow)) << 4));
                const uint32_t sw = *(const uint32_t*)(st + s_rd + (2 * u + h) * 4);
                d[u] = __builtin_bit_cast(float, ((sw >> s_sh[u]) & 255u) << 23);
                if constexpr (CHECK_K)
                    if (!(k0 + 64 * u + 32 * h < K)) q[u][0] = i32x4{0, 0, 0, 0};
            } else if constexpr (FMT == 2) {
                // one 16-byte chunk = this lane's block of 32 codes; the block's fp16 scale
                // from the stage's scale words as for Q8_0 (zero past K)
                q[u][0] = *(const i32x4*)(st + b_rd + (((2 * u + h) ^ swz_b4(lrow)) << 4));
                const uint32_t sw = *(const uint32_t*)(st + s_rd + (2 * u + h) * 4);
                d[u] = half_bits_to_float((uint16_t)(sw >> s_sh[u]));
                if constexpr (CHECK_K) d[u] = (k0 + 64 * u + 32 * h < K) ? d[u] : 0.f;
            } else if constexpr (FMT == 3) {
                // the codes as for IQ4_NL; block j = 4 (s % 2) + 2u + h of the super-block:
                // d * (ls - 32), ls's low four bits at bit 4j of scales_l (word 1), its high
                // two at bit 16 + 2j of word 0 (after the fp16 d)
                q[u][0] = *(const i32x4*)(st + b_rd + (((2 * u + h) ^ swz_b4(lrow)) << 4));
                const uint32_t w0 = *(const uint32_t*)(st + s_rd);
                const uint32_t w1 = *(const uint32_t*)(st + s_rd + 4);
                const int j = 4 * (s & 1) + 2 * u + h;
                const uint32_t ls = ((w1 >> (4 * j)) & 15u) | (((w0 >> (16 + 2 * j)) & 3u) << 4);
                d[u] = half_bits_to_float((uint16_t)w0) * (float)((int)ls - 32);
            } else {
                q[u][0] = *(const i32x4*)(st + b_rd + (((4 * u + 2 * h) ^ swz_b(lrow)) << 4));
                q[u][1] = *(const i32x4*)(st + b_rd + (((4 * u + 2 * h + 1) ^ swz_b(lrow)) << 4));
                if constexpr (SG == 1) {
                    const uint32_t sw = *(const uint32_t*)(st + s_rd + (2 * u + h) * 4);
                    d[u] = half_bits_to_float((uint16_t)(sw >> s_sh[u]));
                } else {
                    d[u] = half_bits_to_float(*(const uint16_t*)(smem + NS * STAGE + ((s >> 2) & 1) * SGROUP +
                                                                 lrow * 32 + (4 * (s & 3) + 2 * u + h) * 2));
                }
                if constexpr (CHECK_K) d[u] = (k0 + 64 * u + 32 * h < K) ? d[u] : 0.f;
            }
        }
        // 8 k sub-steps (half u = t/4, ss = t%4): the MSUB MFMAs of sub-step t run while
        // sub-step t+1's weights are dequantized and its activation fragments read;
        // each sub-step is a scheduling region with that interleave pinned (left alone,
        // the compiler issues all of a stage's dequant work before its MFMAs)
        auto deq = [&](int t) -> bf16x8 {
            if constexpr (FMT == 1) return dequant8_fp4((uint32_t)q[t >> 2][0][t & 3], d[t >> 2]);
            if constexpr (FMT == 2 || FMT == 3) {
                uint32_t c03, c47;
                nl_levels8((uint32_t)q[t >> 2][0][t & 3], c03, c47);
                return dequant8((int)c03, (int)c47, d[t >> 2]);
            }
            const i32x4& v = q[t >> 2][(t & 3) >> 1];
            return (t & 1) ? dequant8(v[2], v[3], d[t >> 2]) : dequant8(v[0], v[1], d[t >> 2]);
        };
        auto afrag = [&](int i, int t) -> bf16x8 {
            const int r = i * 32 + l32;
            const int chunk = (8 * (t >> 2) + 4 * h + (t & 3)) ^ swz_a(r);
            return *(const bf16x8*)(st + r * 256 + (chunk << 4));
        };
        bf16x8 bf[2], af[2][MSUB];
        bf[0] = deq(0);
#pragma unroll
        for (int i = 0; i < MSUB; i++) af[0][i] = afrag(i, 0);
#ifndef MOE_GEMM_NO_SCHED
        __builtin_amdgcn_sched_barrier(0);
#endif
        if constexpr (mfma_prio<false, MODE, FMT>() > 0) __builtin_amdgcn_s_setprio(mfma_prio<false, MODE, FMT>());
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t < 7) {
                bf[nxt] = deq(t + 1);
#pragma unroll
                for (int i = 0; i < MSUB; i++) af[nxt][i] = afrag(i, t + 1);
            }
#pragma unroll
            for (int i = 0; i < MSUB; i++)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bf[cur], acc[i], 0, 0, 0);
#ifndef MOE_GEMM_NO_SCHED
            if (t < 7) {
                constexpr int VPM = ((FMT == 1 ? 4 : FMT >= 2 ? 36 : 20) + MSUB - 1) / MSUB;   // dequant VALU per MFMA
#pragma unroll
                for (int m = 0; m < MSUB; m++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
        if constexpr (mfma_prio<false, MODE, FMT>() > 0) __builtin_amdgcn_s_setprio(0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using NoCheck = std::integral_constant<bool, false>;
    using Check = std::integral_constant<bool, true>;

    const int last = nsteps - 1;   // only this stage can end inside K
    int s = 0;
    if constexpr (NS == 2) {
        issue(0, 0);
        for (; s + 1 < last; s += 2) {
            step(s, S0{}, NoCheck{});
            step(s + 1, S1{}, NoCheck{});
        }
        if (s < last) {
            step(s, S0{}, NoCheck{});
            step(s + 1, S1{}, Check{});
        } else {
            step(s, S0{}, Check{});
        }
    } else {
        using S2 = std::integral_constant<int, 2>;
        issue(0, 0);
        if (nsteps > 1) issue(1, 1);
        for (; s + 2 < last; s += 3) {
            step(s, S0{}, NoCheck{});
            step(s + 1, S1{}, NoCheck{});
            step(s + 2, S2{}, NoCheck{});
        }
        // stages s .. last (one to three), slots 0, 1, 2 in turn
        if (s == last) {
            step(s, S0{}, Check{});
        } else if (s + 1 == last) {
            step(s, S0{}, NoCheck{});
            step(s + 1, S1{}, Check{});
        } else {
            step(s, S0{}, NoCheck{});
            step(s + 1, S1{}, NoCheck{});
            step(s + 2, S2{}, Check{});
        }
    }

    // ---- epilogue. Accumulator v of lane l holds row 8*(v/4) + 4*(l/32) + v%4 of
    // the 32x32 sub-tile and column l%32.
    if (MODE == 1) {
        const int n = nt * NTW + wv * 16 + (l32 & 15);
        const bool writer = l32 < 16 && n < N;
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            if (i * 32 >= m_len) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const float up = __shfl_xor(acc[i][v], 16);
                const int row = i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                if (writer && row < m_len) {
                    const float g = acc[i][v];
                    const float hv = g / (1.0f + __expf(-g)) * up;
                    ((__bf16*)P.out)[(int64_t)s_orow[row] * P.ldo + n] = (__bf16)hv;
                }
            }
        }
    } else {
        // fp32 rows, read once by the reduce: non-temporal stores (Lite-shaped layer:
        // down 67.5 -> 64.9 us, reduce 7.3 -> 8.1 us). The wide kernel keeps plain
        // stores: there the reduce lost more than the GEMM gained.
        const int n = nt * NTW + wv * 32 + l32;
        if (n < N) {
#pragma unroll
            for (int i = 0; i < MSUB; i++) {
                if (i * 32 >= m_len) continue;
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int row = i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (row < m_len) {
                        float* o = &((float*)P.out)[(int64_t)s_orow[row] * P.ldo + n];
                        __builtin_nontemporal_store(acc[i][v], o);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- wide-N variant
// Same product as k_gemm_q8 for 128-row tiles and K % 64 == 0, with a block tile of
// 128 activation rows x 64*W weight rows. Each wave owns 64 weight rows (two MFMA column
// groups) and all 128 rows, so every activation fragment read from LDS feeds two MFMAs.
// A stage is 64 K columns: 16 KB of activations and, for 4 waves, 16 KB of int8 weights
// (8 KB of MXFP4 codes). It is dispatched with 4 waves and a two-slot ring, so two
// independent blocks share a CU and one block's barrier waits, prologue and epilogue
// overlap the other's multiplies.
//
// Scales (SG): with one word per row per stage (SG = 1) every stage touches one cache
// line per weight row just for 4 bytes, which costs as many memory requests as the
// weights themselves. When K % 256 == 0 and the scale rows are 16-byte aligned, SG = 4
// fetches 16 bytes per row (the blocks of four stages) into a two-slot ring instead.
namespace wide {
constexpr int KS = 64;
__device__ __forceinline__ int swz_wa(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_wb(int r) { return (r >> 2) & 3; }
// Block tile 32*MSUB activation rows x 64*W weight rows, W waves, NS ring slots; FMT = 1
// for MXFP4 weights (32-byte rows per stage, two E8M0 scale bytes per row per stage);
// FMT = 2 for IQ4_NL (the same 32-byte rows of codes, the stage's two fp16 scales in one
// aligned word as for Q8_0).
template <int MSUB, int W, int NS, int FMT = 0>
struct Cfg {
    static constexpr int BM = 32 * MSUB;
    static constexpr int BN = 64 * W;                 // weight rows per block
    static constexpr int A_BYTES = BM * KS * 2;       // 128-byte rows, 8 chunks
    static constexpr int WROW = FMT != 0 ? KS / 2 : KS;   // weight bytes per row per stage
    static constexpr int B_BYTES = BN * WROW;         // 64-byte rows, 4 chunks (MXFP4: 32, 2)
    static constexpr int NA = BM / (8 * W);           // activation copies (8 rows) per wave
    static constexpr int SGROUP = BN * 16;            // SG = 4: one group of scales
    template <int SG>
    static constexpr int stage_bytes() { return A_BYTES + B_BYTES + (SG == 1 ? BN * (FMT == 3 ? 8 : 4) : 0); }
    template <int SG>
    static constexpr int lds_bytes() { return NS * stage_bytes<SG>() + (SG == 4 ? 2 * SGROUP : 0); }
    template <int MODE>
    static constexpr int out_cols() { return MODE == 1 ? BN / 2 : BN; }
};
}  // namespace wide

template <int MODE, int SG, int MSUB, int W, int NS, int FMT>
__global__ __launch_bounds__(64 * W, W == 4 ? 2 : 1) void k_gemm_q8w(GemmArgs args) {
    using namespace wide;
    using C = Cfg<MSUB, W, NS, FMT>;
    static_assert(NS == 2 || NS == 3, "two- or three-slot ring");
    static_assert(FMT == 0 || (SG == 1 && NS == 2), "4-bit codes: per-stage scale words, two slots");
    constexpr int BM = C::BM, A_BYTES = C::A_BYTES, B_BYTES = C::B_BYTES, NA = C::NA;
    constexpr int SGROUP = C::SGROUP;
    constexpr int NTW = C::template out_cols<MODE>();
    constexpr int STAGE = C::template stage_bytes<SG>();
    static_assert(NA * 8 * W == BM, "activation rows must split evenly over the waves");
    // copies per wave per stage: NA activation + 4 weight (+ 1 scale word if SG = 1);
    // with SG = 4 every fourth stage also carries one scale-group copy
    constexpr int VM_STAGE = NA + (FMT != 0 ? 2 : 4) + (SG == 1 ? (FMT == 3 ? 2 : 1) : 0);
    static_assert(SG == 1 || SG == 4, "scale groups of one or four stages");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    // ---- tile of this block: the same XCD-aware order as k_gemm_q8
    int b = (int)blockIdx.x, pi = 0;
    {
        const GemmProblem& P0 = args.p[0];
        const int reg0 = ((P0.m_tiles_max * ((P0.N + NTW - 1) / NTW) + 7) >> 3) * 8;
        if (b >= reg0) {
            pi = 1;
            b -= reg0;
        }
    }
    const GemmProblem& P = args.p[pi];
    const int N = P.N, K = P.K;
    const int n_nt = (N + NTW - 1) / NTW;
    // tile height TM: the 160-row form (MSUB = 5) runs tiles of P.tile_m rows (128 or
    // 160) whose segment-last tile may hold up to tile_x rows more (0 or 32; never past
    // 160); the row-id pass counts tiles the same way
    const int TM = MSUB == 5 ? (P.tile_m ? P.tile_m : 128) : BM;
    const int tx = MSUB == 5 ? P.tile_x : 0;
    int e, m0, m_len, nt;
    {
        const int m_tiles = P.bounds ? P.tile_off[P.n_seg] : P.n_seg * tiles_of(P.seg_len, TM, tx);
        const int total = m_tiles * n_nt;
        const int part = (total + 7) >> 3;
        const int q = b >> 3;
        const int t = (b & 7) * part + q;
        if (q >= part || t >= total) return;
        int first, tiles, row0, rows;
        if (P.bounds) {
            const int mt = t / n_nt;
            if (P.tile_tab) {
                const int4 ti = *(const int4*)(P.tile_tab + 4 * (int64_t)mt);
                e = ti.x;
                first = ti.y;
                row0 = ti.z;
                rows = ti.w;
            } else {
                int lo = 0, hi = P.n_seg;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (P.tile_off[mid] <= mt) lo = mid; else hi = mid;
                }
                e = lo;
                first = P.tile_off[e];
                row0 = P.bounds[e];
                rows = P.bounds[e + 1] - row0;
            }
            tiles = tiles_of(rows, TM, tx);
        } else {
            tiles = tiles_of(P.seg_len, TM, tx);
            e = t / (n_nt * tiles);
            first = e * tiles;
            row0 = e * P.seg_len;
            rows = P.seg_len;
        }
        const int r = t - n_nt * first;
        const int c = r / (kMChunk * n_nt);
        const int g = min(kMChunk, tiles - c * kMChunk);
        const int rr = r - c * kMChunk * n_nt;
        nt = rr / g;
        const int j = c * kMChunk + (rr - nt * g);
        m0 = row0 + j * TM;
        m_len = j == tiles - 1 ? rows - j * TM : TM;
    }

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nsteps = K / KS;
    const int KB = K >> 5;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // output column of block-local weight row R (0..BN-1). Gate/up mode: the rows of
    // each 32-row column group are 16 gate rows then the 16 up rows of the same outputs.
    auto wrow = [&](int R) -> int {
        const int n = MODE == 1 ? nt * NTW + (R >> 5) * 16 + (R & 15) : nt * NTW + R;
        return min(n, N - 1);
    };

    // ---- copy geometry (stage 0); rows that are not gathered are addressed from the
    // tile's first row, as in k_gemm_q8
    const int64_t a_row0 = P.a_rows ? 0 : (P.a_row_mod ? m0 % P.a_row_mod : m0);
    const uint8_t* a_base = (const uint8_t*)uniform_ptr((const uint8_t*)P.A + a_row0 * P.lda * 2);
    uint32_t a_off[NA];
#pragma unroll
    for (int i = 0; i < NA; i++) {
        const int R = (wv * NA + i) * 8 + (lane >> 3);    // tile row this lane fetches
        const int lc = (lane & 7) ^ swz_wa(R);
        const int j = m0 + min(R, m_len - 1);
        const int64_t src = P.a_rows ? (int64_t)P.a_rows[j] : (int64_t)(j - m0);
        a_off[i] = (uint32_t)(src * P.lda * 2 + lc * 16);
    }
    // weights: copy i of wave w covers rows 64w + 16i .. +15 (4 lanes x 16 B per row);
    // in gate/up mode odd copies hold up rows
    const int64_t RB = FMT != 0 ? K / 2 : K;   // bytes per weight row
    const int8_t* qg = (const int8_t*)uniform_ptr(P.qs1 + (int64_t)e * N * RB);
    const int8_t* qu = MODE == 1 ? (const int8_t*)uniform_ptr(P.qs2 + (int64_t)e * N * RB) : qg;
    uint32_t b_off[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int R = wv * 64 + 16 * i + (lane >> 2);
        const int lc = (lane & 3) ^ swz_wb(R);
        b_off[i] = (uint32_t)((int64_t)wrow(R) * K + lc * 16);
    }
    // MXFP4: copy i of wave w covers rows 64w + 32i .. +31 (2 lanes x 16 B per row, no
    // swizzle). Its lanes 0-31 and 32-63 read rows of different matrices in gate/up
    // mode, so each lane carries its own 64-bit address.
    const int8_t* b_ptr[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int R = wv * 64 + 32 * i + (lane >> 1);
        b_ptr[i] = ((MODE == 1 && (R & 16)) ? qu : qg) + (int64_t)wrow(R) * RB + (lane & 1) * 16;
    }
    // scales: lane l of wave w fetches for row 64w + l, from a per-lane address (gate
    // and up rows sit in different tensors). SG = 1: the word of blocks 2s, 2s+1 at
    // stage s (K % 64 == 0 keeps the pair inside one aligned word); SG = 4: the 16
    // bytes of blocks 8g .. 8g+7 for stages 4g .. 4g+3.
    // MXFP4: the aligned word holding the row's two scale bytes of stage s (blocks 2s,
    // 2s + 1: an even byte offset, since K % 64 == 0 makes KB even, so both bytes sit in
    // one aligned word)
    const uint8_t* s_ptr;
    {
        const int R = wv * 64 + lane;
        const uint16_t* dt = (MODE == 1 && (R & 16)) ? P.d2 : P.d1;
        s_ptr = (FMT == 1 || FMT == 3) ? (const uint8_t*)dt + ((int64_t)e * N + wrow(R)) * KB
                         : (const uint8_t*)(dt + ((int64_t)e * N + wrow(R)) * KB);
    }
    // MXFP4: where the scale row of this lane's weight row in column group c sits
    // within its aligned word (0 or 2); stage s's bytes start at that + 2s, mod 4
    int s_al[2] = {0, 0};
    if constexpr (FMT == 1) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int lr = wv * 64 + c * 32 + l32;
            const uint16_t* dt = (MODE == 1 && (lr & 16)) ? P.d2 : P.d1;
            s_al[c] = (int)((uintptr_t)((const uint8_t*)dt + ((int64_t)e * N + wrow(lr)) * KB) & 3);
        }
    }
    const uint32_t sring = lds0 + (uint32_t)(NS * STAGE);

    auto issue = [&](int s, int slot) __attribute__((always_inline)) {
        const uint32_t st = lds0 + (uint32_t)(slot * STAGE);
        const int k0 = s * KS;
#pragma unroll
        for (int i = 0; i < NA; i++) dma16(a_base + (int64_t)k0 * 2, a_off[i], st + (wv * NA + i) * 1024);
        if constexpr (FMT != 0) {
#pragma unroll
            for (int i = 0; i < 2; i++) dma16v(b_ptr[i] + k0 / 2, st + A_BYTES + (wv * 2 + i) * 1024);
            if constexpr (FMT == 1)
                dma4v((const void*)((uintptr_t)(s_ptr + 2 * s) & ~(uintptr_t)3), st + A_BYTES + B_BYTES + wv * 256);
            if constexpr (FMT == 3) {   // both words of the row's super-block record (stage s: record s / 4)
                dma4v(s_ptr + 8 * (s >> 2), st + A_BYTES + B_BYTES + wv * 256);
                dma4v(s_ptr + 8 * (s >> 2) + 4, st + A_BYTES + B_BYTES + C::BN * 4 + wv * 256);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                dma16(((MODE == 1 && (i & 1)) ? qu : qg) + k0, b_off[i], st + A_BYTES + (wv * 4 + i) * 1024);
        }
        if (FMT == 1 || FMT == 3) {
        } else if (SG == 1) {
            dma4v(s_ptr + 4 * s, st + A_BYTES + B_BYTES + wv * 256);
        } else if ((s & 3) == 0) {
            dma16v(s_ptr + 4 * s, sring + (uint32_t)(((s >> 2) & 1) * SGROUP) + wv * 1024);
        }
    };

    f32x16 acc[MSUB][2];
#pragma unroll
    for (int i = 0; i < MSUB; i++)
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][c][v] = 0.f;

    // One step: wait for stage s (stage s+1 may stay in flight), send stage s+2 into
    // the slot that step s-1 read, dequantize and multiply. MACT = 32-row sub-tiles
    // that hold rows of the tile: the last tile of an expert is often mostly empty,
    // and its empty sub-tiles skip their fragment reads and MFMAs.
    auto step = [&](int s, auto slot_c, auto mact_c) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr int MACT = decltype(mact_c)::value;
        // copies still allowed in flight: those of stage s+1 with three slots (sent one
        // step ago), none with two (stage s+1 is sent after this wait)
        if (NS == 2 || s + 1 >= nsteps) wait_stage_and_barrier<0>();
        else if (SG == 4 && ((s + 1) & 3) == 0) wait_stage_and_barrier<VM_STAGE + 1>();
        else wait_stage_and_barrier<VM_STAGE>();
        if (s + NS - 1 < nsteps) issue(s + NS - 1, (SLOT + NS - 1) % NS);
        const uint8_t* st = smem + SLOT * STAGE;
        const uint8_t* sg = SG == 1 ? st + A_BYTES + B_BYTES
                                    : smem + NS * STAGE + ((s >> 2) & 1) * SGROUP + (s & 3) * 4;
        // operands of the stage: both column groups' 32 int8 weights and scale, and
        // the activation fragments of k sub-step 0
        // The lane's k columns: half h of the stage (k 32h .. 32h + 31, block 2s + h),
        // 8 of them per k sub-step ss (k 32h + 8ss ..), as the activation fragments
        // below take them.
        i32x4 q[2][2];
        float d[2];
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int lr = wv * 64 + c * 32 + l32;
            if constexpr (FMT == 1) {
                // chunk h of the row holds the 32 codes; sub-step ss takes its dword ss
                q[c][0] = *(const i32x4*)(st + A_BYTES + lr * 32 + 16 * h);
                const uint32_t sw = *(const uint32_t*)(sg + lr * 4);
                const int sh = ((s_al[c] + 2 * s) & 3) * 8 + 8 * h;
                d[c] = __builtin_bit_cast(float, ((sw >> sh) & 255u) << 23);
            } else if constexpr (FMT == 2) {
                // the 32 codes as for MXFP4; block 2s + h's fp16 scale from the stage's word
                q[c][0] = *(const i32x4*)(st + A_BYTES + lr * 32 + 16 * h);
                const uint32_t sw = *(const uint32_t*)(sg + lr * 4);
                d[c] = half_bits_to_float((uint16_t)(sw >> (16 * h)));
            } else if constexpr (FMT == 3) {
                // IQ4_XS: the codes as for IQ4_NL; block j = 2 (s % 4) + h of the super-block
                // takes d * (ls - 32) from the record's words (word 0: fp16 d, scales_h;
                // word 1: scales_l)
                q[c][0] = *(const i32x4*)(st + A_BYTES + lr * 32 + 16 * h);
                const uint32_t w0 = *(const uint32_t*)(sg + lr * 4);
                const uint32_t w1 = *(const uint32_t*)(sg + C::BN * 4 + lr * 4);
                const int j = 2 * (s & 3) + h;
                const uint32_t ls = ((w1 >> (4 * j)) & 15u) | (((w0 >> (16 + 2 * j)) & 3u) << 4);
                d[c] = half_bits_to_float((uint16_t)w0) * (float)((int)ls - 32);
            } else {
                const uint8_t* rowp = st + A_BYTES + lr * 64;
                q[c][0] = *(const i32x4*)(rowp + (((2 * h) ^ swz_wb(lr)) << 4));
                q[c][1] = *(const i32x4*)(rowp + (((2 * h + 1) ^ swz_wb(lr)) << 4));
                const uint32_t sw = *(const uint32_t*)(sg + lr * (SG == 1 ? 4 : 16));
                d[c] = half_bits_to_float((uint16_t)(sw >> (16 * h)));
            }
        }
        auto afrag = [&](int i, int ss) -> bf16x8 {
            const int r = i * 32 + l32;
            return *(const bf16x8*)(st + r * 128 + (((4 * h + ss) ^ swz_wa(r)) << 4));
        };
        auto deq = [&](int c, int ss) -> bf16x8 {
            if constexpr (FMT == 1) return dequant8_fp4((uint32_t)q[c][0][ss], d[c]);
            if constexpr (FMT == 2 || FMT == 3) {
                uint32_t c03, c47;
                nl_levels8((uint32_t)q[c][0][ss], c03, c47);
                return dequant8((int)c03, (int)c47, d[c]);
            }
            const i32x4& v = q[c][ss >> 1];
            return (ss & 1) ? dequant8(v[2], v[3], d[c]) : dequant8(v[0], v[1], d[c]);
        };
        bf16x8 af[2][MSUB], bf[2][2];
#pragma unroll
        for (int i = 0; i < MACT; i++) af[0][i] = afrag(i, 0);
        bf[0][0] = deq(0, 0);
        bf[0][1] = deq(1, 0);
        // k sub-step ss: its 8 MFMAs run while the next sub-step's weights are
        // dequantized and its activation fragments read. Each sub-step is a
        // scheduling region of its own, with the interleave pinned inside it; left
        // alone the compiler runs all dequant work of the stage first, and the two
        // waves of a SIMD, kept in step by the stage barrier, then contend for the
        // vector ALU and the matrix unit at the same time instead of overlapping.
#ifndef MOE_GEMM_NO_SCHED
        __builtin_amdgcn_sched_barrier(0);
#endif
        if constexpr (mfma_prio<true, MODE, FMT>() > 0) __builtin_amdgcn_s_setprio(mfma_prio<true, MODE, FMT>());
#pragma unroll
        for (int ss = 0; ss < 4; ss++) {
            const int cur = ss & 1, nxt = cur ^ 1;
            if (ss < 3) {
#pragma unroll
                for (int i = 0; i < MACT; i++) af[nxt][i] = afrag(i, ss + 1);
                bf[nxt][0] = deq(0, ss + 1);
                bf[nxt][1] = deq(1, ss + 1);
            }
#pragma unroll
            for (int i = 0; i < MACT; i++)
#pragma unroll
                for (int c = 0; c < 2; c++)
                    acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bf[cur][c], acc[i][c], 0, 0, 0);
#ifndef MOE_GEMM_NO_SCHED
            if (ss < 3) {
                // 2*MACT MFMAs share the sub-step's dequant instructions (Q8_0: 40,
                // MXFP4: 8, IQ4_NL: about 72)
                constexpr int VPM = ((FMT == 1 ? 8 : FMT >= 2 ? 72 : 40) + 2 * MACT - 1) / (2 * MACT);
#pragma unroll
                for (int m = 0; m < 2 * MACT; m++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
                    if ((m & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
        if constexpr (mfma_prio<true, MODE, FMT>() > 0) __builtin_amdgcn_s_setprio(0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    auto k_loop = [&](auto mact_c) __attribute__((always_inline)) {
        issue(0, 0);
        int s = 0;
        if constexpr (NS == 3) {
            if (nsteps > 1) issue(1, 1);
            for (; s + 3 <= nsteps; s += 3) {
                step(s, S0{}, mact_c);
                step(s + 1, S1{}, mact_c);
                step(s + 2, S2{}, mact_c);
            }
            if (s < nsteps) step(s, S0{}, mact_c);
            if (s + 1 < nsteps) step(s + 1, S1{}, mact_c);
        } else {
            for (; s + 2 <= nsteps; s += 2) {
                step(s, S0{}, mact_c);
                step(s + 1, S1{}, mact_c);
            }
            if (s < nsteps) step(s, S0{}, mact_c);
        }
    };
    const int mact = (m_len + 31) >> 5;   // block-uniform
    if (mact >= MSUB) k_loop(std::integral_constant<int, MSUB>{});
    else if (MSUB > 4 && mact == 4) k_loop(std::integral_constant<int, (MSUB > 4 ? 4 : 1)>{});
    else if (MSUB > 3 && mact == 3) k_loop(std::integral_constant<int, (MSUB > 3 ? 3 : 1)>{});
    else if (MSUB > 2 && mact == 2) k_loop(std::integral_constant<int, (MSUB > 2 ? 2 : 1)>{});
    else k_loop(std::integral_constant<int, 1>{});

    // ---- output rows into the (now idle) ring: every copy has landed (the last step
    // waited for all of them) and the barrier ends every wave's reads of the ring
    int32_t* s_orow = (int32_t*)smem;
    __syncthreads();
    if (tid < BM) {
        const int j = m0 + min(tid, m_len - 1);
        s_orow[tid] = P.out_rows ? P.out_rows[j] : j;
    }
    __syncthreads();

    // ---- epilogue. Accumulator v of lane l holds row 8*(v/4) + 4*(l/32) + v%4 of
    // the 32x32 sub-tile and column l%32 of the column group.
    if (MODE == 1) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int n = nt * NTW + wv * 32 + c * 16 + (l32 & 15);
            const bool writer = l32 < 16 && n < N;
#pragma unroll
            for (int i = 0; i < MSUB; i++) {
                if (i * 32 >= m_len) continue;
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const float up = __shfl_xor(acc[i][c][v], 16);
                    const int row = i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (writer && row < m_len) {
                        const float g = acc[i][c][v];
                        const float hv = g / (1.0f + __expf(-g)) * up;
                        ((__bf16*)P.out)[(int64_t)s_orow[row] * P.ldo + n] = (__bf16)hv;
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int n = nt * NTW + wv * 64 + c * 32 + l32;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < MSUB; i++) {
                if (i * 32 >= m_len) continue;
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int row = i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (row < m_len) ((float*)P.out)[(int64_t)s_orow[row] * P.ldo + n] = acc[i][c][v];
                }
            }
        }
    }
}

template <int MODE, int SG, int MSUB, int W, int NS, int FMT = 0>
hipError_t launch_wide_sg(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr int lds = wide::Cfg<MSUB, W, NS, FMT>::template lds_bytes<SG>();
    static_assert(lds <= 160 * 1024, "LDS ring exceeds 160 KB");
    static PerDeviceOnce lds_cap;
    if (const hipError_t e = set_lds_cap(lds_cap, (const void*)k_gemm_q8w<MODE, SG, MSUB, W, NS, FMT>, lds))
        return e;
    k_gemm_q8w<MODE, SG, MSUB, W, NS, FMT><<<grid, 64 * W, lds, st>>>(a);
    return hipGetLastError();
}

// MXFP4 (FMT = 1) or IQ4_NL (FMT = 2) experts on the wide kernel (per-stage scale words only).
template <int MODE, int MSUB, int W, int NS, int FMT = 1>
hipError_t launch_wide_fp4(const GemmArgs& a, hipStream_t st) {
    constexpr int ntw = wide::Cfg<MSUB, W, NS, FMT>::template out_cols<MODE>();
    int64_t total = 0;
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        total += ((int64_t)p.m_tiles_max * ((p.N + ntw - 1) / ntw) + 7) / 8 * 8;
    }
    if (total <= 0) return hipSuccess;
    GemmArgs g = a;
    g.grid_real = (int32_t)total;
    return launch_wide_sg<MODE, 1, MSUB, W, NS, FMT>(g, (int)total, st);
}

template <int MODE, int MSUB, int W, int NS>
hipError_t launch_wide(const GemmArgs& a, hipStream_t st) {
    constexpr int ntw = wide::Cfg<MSUB, W, NS>::template out_cols<MODE>();
    int64_t total = 0;
    bool groups = true;   // scale groups of four stages for every problem
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        total += ((int64_t)p.m_tiles_max * ((p.N + ntw - 1) / ntw) + 7) / 8 * 8;
        groups = groups && p.K % 256 == 0 && ((uintptr_t)p.d1 & 15) == 0 &&
                 (MODE == 0 || ((uintptr_t)p.d2 & 15) == 0);
    }
    if (total <= 0) return hipSuccess;
    GemmArgs g = a;
    g.grid_real = (int32_t)total;
    return groups ? launch_wide_sg<MODE, 4, MSUB, W, NS, 0>(g, (int)total, st)
                  : launch_wide_sg<MODE, 1, MSUB, W, NS, 0>(g, (int)total, st);
}

template <int MSUB, int W, int NS, int SG, int FMT>
constexpr int stage_lds() {
    return NS * (32 * MSUB * 256 + W * 32 * (FMT != 0 ? 64 : 128) + (SG == 1 ? W * 32 * 16 : 0)) +
           (SG == 4 ? 2 * W * 32 * 32 : 0);
}

template <int MSUB, int MODE, int W, int NS, int SG, int FMT>
hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr int lds = stage_lds<MSUB, W, NS, SG, FMT>();
    static_assert(lds + 32 * MSUB * 4 <= 160 * 1024, "LDS rings exceed 160 KB");
    static PerDeviceOnce lds_cap;   // raise the dynamic LDS cap once per device
    if (const hipError_t e = set_lds_cap(lds_cap, (const void*)k_gemm_q8<MSUB, MODE, W, NS, SG, FMT>, lds))
        return e;
    k_gemm_q8<MSUB, MODE, W, NS, SG, FMT><<<grid, 64 * W, lds, st>>>(a);
    return hipGetLastError();
}

// Grid of the narrow kernel with W waves: per problem, an upper bound on its tiles,
// rounded up to a multiple of 8 (one part per XCD).
template <int W>
int64_t narrow_grid(const GemmArgs& a) {
    const int ntw = a.mode == 1 ? out_cols<1, W>() : out_cols<0, W>();
    int64_t total = 0;
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        total += ((int64_t)p.m_tiles_max * ((p.N + ntw - 1) / ntw) + 7) / 8 * 8;
    }
    return total;
}

// MXFP4 experts: the same kernel with 64-byte weight rows and per-stage scale words.
// An MXFP4 stage is small enough for a three-slot ring at two 4-wave blocks per CU.
// IQ4_NL experts (FMT = 2) take the same launch shapes.
template <int MSUB, int W, int NS, int FMT = 1>
hipError_t launch_cfg_fp4(const GemmArgs& a, hipStream_t st) {
    const int64_t total = narrow_grid<W>(a);
    if (total <= 0) return hipSuccess;
    GemmArgs g = a;
    g.grid_real = (int32_t)total;
    return a.mode == 1 ? launch_one<MSUB, 1, W, NS, 1, FMT>(g, (int)total, st)
                       : launch_one<MSUB, 0, W, NS, 1, FMT>(g, (int)total, st);
}

template <int MSUB, int W, int NS>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
    const int ntw = a.mode == 1 ? out_cols<1, W>() : out_cols<0, W>();
    int64_t total = 0;
    bool groups = true;   // scale groups of four stages for every problem
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        total += ((int64_t)p.m_tiles_max * ((p.N + ntw - 1) / ntw) + 7) / 8 * 8;
        groups = groups && p.K % 512 == 0 && ((uintptr_t)p.d1 & 15) == 0 &&
                 (a.mode == 0 || ((uintptr_t)p.d2 & 15) == 0);
    }
    if (total <= 0) return hipSuccess;
    GemmArgs g = a;
    g.grid_real = (int32_t)total;
    if (a.mode == 1)
        return groups ? launch_one<MSUB, 1, W, NS, 4, 0>(g, (int)total, st)
                      : launch_one<MSUB, 1, W, NS, 1, 0>(g, (int)total, st);
    return groups ? launch_one<MSUB, 0, W, NS, 4, 0>(g, (int)total, st)
                  : launch_one<MSUB, 0, W, NS, 1, 0>(g, (int)total, st);
}

}  // namespace

int64_t gemm_q8_max_threads(const GemmArgs& a0, int msub) {
    GemmArgs a = a0;
    if (a.n_prob < 2) a.p[1] = GemmProblem{};
    // every kernel variant the dispatch below may pick for this tile height
    int64_t wide = 0;
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        const int ntw = a.mode == 1 ? 128 : 256;   // the wide kernel's 256 weight rows
        wide += ((int64_t)p.m_tiles_max * ((p.N + ntw - 1) / ntw) + 7) / 8 * 8;
    }
    int64_t t = narrow_grid<8>(a) * 512;
    if (msub == 2) t = t > narrow_grid<4>(a) * 256 ? t : narrow_grid<4>(a) * 256;
    else t = t > wide * 256 ? t : wide * 256;
    return t;
}

int gemm_pick_msub(double avg_rows) {
    if (avg_rows <= 64) return 2;
    return 4;
}
int gemm_tile_m(int msub) { return 32 * msub; }

#ifndef MOE_GEMM_TALL_LAST
#define MOE_GEMM_TALL_LAST 1   // 0: 128-row tiles only (no 160-row segment-last tiles)
#endif
int gemm_tile_x(int msub, int fmt, int64_t K, bool scales_aligned) {
    // MXFP4 takes the wide kernel only with its scale rows at even addresses, IQ4_NL
    // only with its scale tensors 4-byte aligned
    return (MOE_GEMM_TALL_LAST && msub == 4 && K % wide::KS == 0 && (fmt == 0 || scales_aligned)) ? 32 : 0;
}
#ifndef MOE_GEMM_TILE160
#define MOE_GEMM_TILE160 0   // 1: the 160-row kernel runs 160-row tiles instead of 128 + 32
#endif
void gemm_set_tall(GemmProblem& p, RowIdsArgs& r, int q) {
    p.tile_m = MOE_GEMM_TILE160 ? 160 : 128;
    p.tile_x = MOE_GEMM_TILE160 ? 0 : 32;
    r.tile_m[q] = p.tile_m;
    r.tile_x[q] = p.tile_x;
}

// Every problem's scale tensors start at an address with (address & mask) == 0.
static bool scales_aligned(const GemmArgs& a, uintptr_t mask) {
    for (int i = 0; i < a.n_prob; i++)
        if (((uintptr_t)a.p[i].d1 & mask) || (a.mode == 1 && ((uintptr_t)a.p[i].d2 & mask))) return false;
    return true;
}

hipError_t launch_gemm_q8(const GemmArgs& a0, int msub, hipStream_t st) {
    GemmArgs a = a0;
    if (a.n_prob < 2) a.p[1] = GemmProblem{};
    bool wide_ok = true;   // the wide kernels need whole 64-column stages
    for (int i = 0; i < a.n_prob; i++) wide_ok = wide_ok && a.p[i].K % wide::KS == 0;
#ifdef MOE_GEMM_NO_WIDE
    wide_ok = false;
#endif
    // segment-last tiles of 128 + 32 rows: only the 160-row wide kernel takes them, and
    // the tile tables were built for them, so any other choice is a caller error
    bool tall = false;
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        if ((p.tile_x != 0 && p.tile_x != 32) || (p.tile_m != 0 && p.tile_m != 128 && p.tile_m != 160) ||
            (p.tile_m ? p.tile_m : 128) + p.tile_x > 160)
            return hipErrorInvalidValue;
        tall = tall || p.tile_x != 0 || p.tile_m == 160;
    }
    if (tall) {
        if (msub != 4 || !wide_ok) return hipErrorInvalidValue;
        if (a.fmt == 3) {
            if (!scales_aligned(a, 7)) return hipErrorInvalidValue;
            return a.mode == 1 ? launch_wide_fp4<1, 5, 4, 2, 3>(a, st) : launch_wide_fp4<0, 5, 4, 2, 3>(a, st);
        }
        if (a.fmt == 2) {
            if (!scales_aligned(a, 3)) return hipErrorInvalidValue;
            return a.mode == 1 ? launch_wide_fp4<1, 5, 4, 2, 2>(a, st) : launch_wide_fp4<0, 5, 4, 2, 2>(a, st);
        }
        if (a.fmt == 1) {
            for (int i = 0; i < a.n_prob; i++)
                if (((uintptr_t)a.p[i].d1 & 1) || (a.mode == 1 && ((uintptr_t)a.p[i].d2 & 1)))
                    return hipErrorInvalidValue;
            return a.mode == 1 ? launch_wide_fp4<1, 5, 4, 2>(a, st) : launch_wide_fp4<0, 5, 4, 2>(a, st);
        }
        return a.mode == 1 ? launch_wide<1, 5, 4, 2>(a, st) : launch_wide<0, 5, 4, 2>(a, st);
    }
    if (a.fmt == 3) {   // IQ4_XS experts: 64-row tiles on the narrow kernel, 128-row on the wide one
        switch (msub) {
            case 2:
                if (narrow_grid<8>(a) >= 2048) return launch_cfg_fp4<2, 8, 2, 3>(a, st);
                return launch_cfg_fp4<2, 4, 2, 3>(a, st);
            case 4:
                if (wide_ok && scales_aligned(a, 7))
                    return a.mode == 1 ? launch_wide_fp4<1, 4, 4, 2, 3>(a, st) : launch_wide_fp4<0, 4, 4, 2, 3>(a, st);
                return launch_cfg_fp4<4, 8, 2, 3>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (a.fmt == 2) {   // IQ4_NL experts: MXFP4's launch shapes
        switch (msub) {
            case 2:
                if (narrow_grid<8>(a) >= 2048) return launch_cfg_fp4<2, 8, 3, 2>(a, st);
                return launch_cfg_fp4<2, 4, 3, 2>(a, st);
            case 4:
                // the wide kernel reads each stage's two fp16 scales as one aligned word
                if (wide_ok && scales_aligned(a, 3))
                    return a.mode == 1 ? launch_wide_fp4<1, 4, 4, 2, 2>(a, st) : launch_wide_fp4<0, 4, 4, 2, 2>(a, st);
                return launch_cfg_fp4<4, 8, 2, 2>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (a.fmt == 1) {   // MXFP4 experts: 64-row tiles on the narrow kernel, 128-row on the wide one
        switch (msub) {
            case 2:
                // 64-row tiles: 8 waves (256 weight rows) with three slots, one block per
                // CU, when that still leaves some 8 rounds of blocks (V3-shaped layers);
                // otherwise 4 waves with three slots, two blocks per CU. Measured on
                // MXFP4 layers: V3-shaped T=2048 step 3708 -> 3205 us with 8 waves,
                // Lite- and GPT-OSS-shaped PP512 1-3% better with 4.
                if (narrow_grid<8>(a) >= 2048) return launch_cfg_fp4<2, 8, 3>(a, st);
                return launch_cfg_fp4<2, 4, 3>(a, st);
            case 4: {
                // 128-row tiles: the wide kernel, two blocks per CU. Its per-stage scale
                // word holds both scale bytes of the stage when the scale rows start at
                // even addresses. Otherwise the narrow kernel with 8 waves (three slots
                // measured no better than two there).
                bool even = true;
                for (int i = 0; i < a.n_prob; i++)
                    even = even && ((uintptr_t)a.p[i].d1 & 1) == 0 &&
                           (a.mode == 0 || ((uintptr_t)a.p[i].d2 & 1) == 0);
                if (wide_ok && even) return a.mode == 1 ? launch_wide_fp4<1, 4, 4, 2>(a, st)
                                                        : launch_wide_fp4<0, 4, 4, 2>(a, st);
                return launch_cfg_fp4<4, 8, 2>(a, st);
            }
            default: return hipErrorInvalidValue;
        }
    }
    switch (msub) {
        case 2:
            // 64-row tiles stay on the narrow kernel: on segments of about 50 rows the
            // wide one (Cfg<2, 4>) gives too few blocks per CU and was measured slower
            return launch_cfg<2, MOE_GEMM_CFG2>(a, st);
        case 4:
#ifndef MOE_GEMM_WIDE_CFG
#define MOE_GEMM_WIDE_CFG 4, 2   // waves, ring slots of the 128-row wide kernel (2 blocks per CU)
#endif
            if (wide_ok) return a.mode == 1 ? launch_wide<1, 4, MOE_GEMM_WIDE_CFG>(a, st)
                                            : launch_wide<0, 4, MOE_GEMM_WIDE_CFG>(a, st);
            return launch_cfg<4, MOE_GEMM_CFG4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
