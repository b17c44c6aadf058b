// Quantized-activation grouped GEMM (the MMQ-style path) for Q8_0 experts on gfx950.
//
// What it computes: the grouped product over expert segments of the pages' mmq_id
// path, where quantized experts meet quantized activations ("CUDA: better MoE
// implementation", section 2.1). Activation rows come quantized in 32-column blocks
// (int8 codes q_a and one float32 scale d_a per block, written by k_quant_act); expert
// rows are Q8_0 (int8 codes q_w, one fp16 scale d_w per 32 columns). For output
// (row m, column n):
//     out[m][n] = sum over blocks b of  d_a[m][b] * d_w[n][b] * S_b[m][n],
//     S_b[m][n] = sum over the 32 columns of block b of q_a * q_w   (exact int32).
// Gate/up mode applies silu(gate) * up and writes bf16; down mode writes fp32 rows
// through the output row map, as the bf16 grouped GEMM does.
//
// gfx950 design:
//   * v_mfma_i32_32x32x32_i8: one instruction covers one 32-column block of a 32x32
//     output tile, so S_b comes out exactly in int32 and each block is scaled on its
//     own: 16 conversions, 16 scale products and 16 FMAs per lane per instruction.
//     That vector work, not the matrix unit, bounds the kernel (the weights need no
//     dequantization at all).
//   * Block tile: 128 activation rows x 256 weight rows, 4 waves; wave w owns 64 weight
//     rows (two 32-row column groups) and all 128 rows. A stage is 64 K columns (two
//     blocks): 8 KB of int8 activations gathered row by row through the row map,
//     16 KB of int8 weights, the activation scales and the weight scales, all copied
//     global -> LDS with direct copies; two ring slots, two blocks per CU.
//   * LDS rows are 64 bytes; 16-byte chunk c of row r sits at c ^ ((r >> 2) & 3), so the
//     8 lanes of a ds_read_b128 phase hit 8 different bank groups.
//   * Lane half h and byte e of an MFMA operand stand for column 16h + e of the block on
//     both operands, so A and B agree on k whatever order the unit sums in.
//   * Tiles are placed as in the bf16 grouped GEMM: per problem 8 equal parts of the
//     grid, one per XCD, over tiles ordered by expert, chunk of M tiles, N tile.
#include <type_traits>

#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQBM = 128;             // activation rows per block tile
constexpr int kQW = 4;                // waves
constexpr int kQBN = 64 * kQW;        // weight rows per block tile
constexpr int kQKS = 64;              // K columns per stage
constexpr int kQA = kQBM * kQKS;      // activation bytes per stage
constexpr int kQB = kQBN * kQKS;      // weight bytes per stage
constexpr int kQSA = kQBM * 2 * 4;    // activation scales per stage (fp32, two blocks)
constexpr int kQSW = kQBN * 2 * 4;    // weight-scale words per stage (two per row)
constexpr int kQStage = kQA + kQB + kQSA + kQSW;
constexpr int kQNS = 2;               // ring slots
constexpr int kQLds = kQNS * kQStage;
constexpr int kQMChunk = 4;           // M tiles sharing each weight slab in turn

__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

template <int MODE>
constexpr int q_out_cols() { return MODE == 1 ? kQBN / 2 : kQBN; }

// ---------------------------------------------------------------- activation quantizer
// One thread per 32-column block: d = max|x| / 127 and q = rint(x / d) in float32 (IEEE
// division, rounded to nearest-even; rint ties to even), clamped to [-127, 127]; a block
// of zeros gets d = 0 and q = 0.
template <bool BF16>
__global__ __launch_bounds__(256) void k_quant_act(QuantArgs args) {
    const bool second = (int64_t)blockIdx.x >= args.blocks0;
    const QuantPart& a = args.part[second ? 1 : 0];
    const int64_t blk = ((int64_t)blockIdx.x - (second ? args.blocks0 : 0)) * 256 + threadIdx.x;
    const int64_t KB = a.K >> 5;
    if (blk >= a.rows * KB) return;
    const int64_t r = blk / KB;
    const int64_t b = blk - r * KB;
    float v[32];
    if constexpr (BF16) {
        const i32x4* src = (const i32x4*)((const uint16_t*)a.src + r * a.K + b * 32);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const i32x4 w = src[i];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[8 * i + 2 * j] = __builtin_bit_cast(float, (uint32_t)w[j] << 16);
                v[8 * i + 2 * j + 1] = __builtin_bit_cast(float, (uint32_t)w[j] & 0xffff0000u);
            }
        }
    } else {
        const f32x4* src = (const f32x4*)((const float*)a.src + r * a.K + b * 32);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const f32x4 w = src[i];
#pragma unroll
            for (int j = 0; j < 4; j++) v[4 * i + j] = w[j];
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
    const float d = amax / 127.0f;
    uint32_t packed[8];
#pragma unroll
    for (int i = 0; i < 8; i++) packed[i] = 0;
    if (d != 0.f) {
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const float t = fminf(fmaxf(rintf(v[i] / d), -127.f), 127.f);
            packed[i >> 2] |= ((uint32_t)(int)t & 255u) << (8 * (i & 3));
        }
    }
    i32x4* dq = (i32x4*)(a.q + r * a.K + b * 32);
    dq[0] = i32x4{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
    dq[1] = i32x4{(int)packed[4], (int)packed[5], (int)packed[6], (int)packed[7]};
    a.d[r * KB + b] = d;
}

// ---------------------------------------------------------------- grouped GEMM
template <int MODE>
__global__ __launch_bounds__(64 * kQW, 2) void k_gemm_q8a(GemmArgs args) {
    constexpr int NTW = q_out_cols<MODE>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    // ---- tile of this block (the same XCD-aware order as the bf16 grouped GEMM)
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
        const int m_tiles = P.bounds ? P.tile_off[P.n_seg] : P.n_seg * ((P.seg_len + kQBM - 1) / kQBM);
        const int total = m_tiles * n_nt;
        const int part = (total + 7) >> 3;
        const int q = b >> 3;
        const int t = (b & 7) * part + q;
        if (q >= part || t >= total) return;
        int first, tiles, row0, rows;
        if (P.bounds) {
            const int mt = t / n_nt;
            const int4 ti = *(const int4*)(P.tile_tab + 4 * (int64_t)mt);
            e = ti.x;
            first = ti.y;
            row0 = ti.z;
            rows = ti.w;
            tiles = (rows + kQBM - 1) / kQBM;
        } else {
            tiles = (P.seg_len + kQBM - 1) / kQBM;
            e = t / (n_nt * tiles);
            first = e * tiles;
            row0 = e * P.seg_len;
            rows = P.seg_len;
        }
        const int r = t - n_nt * first;
        const int c = r / (kQMChunk * n_nt);
        const int g = min(kQMChunk, tiles - c * kQMChunk);
        const int rr = r - c * kQMChunk * n_nt;
        nt = rr / g;
        const int j = c * kQMChunk + (rr - nt * g);
        m0 = row0 + j * kQBM;
        m_len = min(kQBM, rows - j * kQBM);
    }

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KB = K >> 5;                  // blocks per row
    const int nsteps = (K + kQKS - 1) / kQKS;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // output column of block-local weight row R (0..255); gate/up mode: each 32-row
    // column group holds 16 gate rows, then the 16 up rows of the same outputs
    auto wrow = [&](int R) -> int {
        const int n = MODE == 1 ? nt * NTW + (R >> 5) * 16 + (R & 15) : nt * NTW + R;
        return min(n, N - 1);
    };

    // ---- copy geometry (stage 0). Activation rows: rows that are not gathered are
    // addressed from the tile's first row; gathered ones from the tensor's start (the
    // host keeps a gathered tensor under 4 GiB).
    const int64_t a_row0 = P.a_rows ? 0 : (P.a_row_mod ? m0 % P.a_row_mod : m0);
    const uint8_t* aq_base = (const uint8_t*)uniform_ptr(P.Aq + a_row0 * (int64_t)K);
    const uint8_t* ad_base = (const uint8_t*)uniform_ptr(P.Ad + a_row0 * (int64_t)KB);
    uint32_t a_off[2];
    int a_lc[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int R = (wv * 2 + i) * 16 + (lane >> 2);   // tile row this lane fetches
        const int lc = (lane & 3) ^ swz64(R);
        const int j = m0 + min(R, m_len - 1);
        const int64_t src = P.a_rows ? (int64_t)P.a_rows[j] : (int64_t)(j - m0);
        a_off[i] = (uint32_t)(src * K + lc * 16);
        a_lc[i] = lc;
    }
    // activation scales: lane -> (block lane / 32 of the stage, tile row 32w + lane % 32)
    uint32_t sa_off;
    {
        const int R = wv * 32 + l32;
        const int j = m0 + min(R, m_len - 1);
        const int64_t src = P.a_rows ? (int64_t)P.a_rows[j] : (int64_t)(j - m0);
        sa_off = (uint32_t)((src * KB + h) * 4);
    }
    // weights: copy i of wave w covers rows 64w + 16i .. +15 (4 lanes x 16 B per row)
    const int8_t* qg = (const int8_t*)uniform_ptr(P.qs1 + (int64_t)e * N * K);
    const int8_t* qu = MODE == 1 ? (const int8_t*)uniform_ptr(P.qs2 + (int64_t)e * N * K) : qg;
    uint32_t b_off[4];
    int b_lc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int R = wv * 64 + 16 * i + (lane >> 2);
        const int lc = (lane & 3) ^ swz64(R);
        b_off[i] = (uint32_t)((int64_t)wrow(R) * K + lc * 16);
        b_lc[i] = lc;
    }
    // weight scales: copy j (block 2s + j) of wave w: lane -> row 64w + lane, the aligned
    // word holding that fp16, from the row's own tensor (gate and up rows sit apart)
    const uint16_t* sw_row;
    {
        const int R = wv * 64 + lane;
        const uint16_t* dt = (MODE == 1 && (R & 16)) ? P.d2 : P.d1;
        sw_row = dt + ((int64_t)e * N + wrow(R)) * KB;
    }
    // where in its aligned word the scale of (this lane's row in column group c, block
    // 2s + j) sits: odd element -> upper half (same for every stage)
    int sw_sh[2][2];
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int R = wv * 64 + c * 32 + l32;
        const uint16_t* dt = (MODE == 1 && (R & 16)) ? P.d2 : P.d1;
        const uint64_t idx = (uint64_t)(((uintptr_t)(dt + ((int64_t)e * N + wrow(R)) * KB)) >> 1);
#pragma unroll
        for (int j = 0; j < 2; j++) sw_sh[c][j] = ((idx + j) & 1) ? 16 : 0;
    }

    auto issue = [&](int s, int slot) __attribute__((always_inline)) {
        const uint32_t st = lds0 + (uint32_t)(slot * kQStage);
        const int k0 = s * kQKS;
        const bool full = k0 + kQKS <= K;   // wave-uniform: every stage but a half last one
#pragma unroll
        for (int i = 0; i < 2; i++) {
            // chunks past K (columns k0 + 16 lc ..) re-read the stage's first chunk
            const uint32_t adj = (!full && k0 + a_lc[i] * 16 >= K) ? (uint32_t)(a_lc[i] * 16) : 0u;
            dma16(aq_base + k0, a_off[i] - adj, st + (wv * 2 + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t adj = (!full && k0 + b_lc[i] * 16 >= K) ? (uint32_t)(b_lc[i] * 16) : 0u;
            dma16(((MODE == 1 && (i & 1)) ? qu : qg) + k0, b_off[i] - adj, st + kQA + (wv * 4 + i) * 1024);
        }
        {
            // block 2s + h, or the row's last block when that is past K
            const uint32_t adj = (!full && h == 1) ? 4u : 0u;
            dma4(ad_base + (int64_t)k0 / 8, sa_off - adj, st + kQA + kQB + wv * 256);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int blk = min(2 * s + j, KB - 1);
            dma4v((const void*)((uintptr_t)(sw_row + blk) & ~(uintptr_t)3),
                  st + kQA + kQB + kQSA + (wv * 2 + j) * 256);
        }
    };

    float acc[4][2][16];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][c][v] = 0.f;

    // one stage: the blocks of the stage (the second only if it lies inside K), each
    // through all occupied 32-row sub-tiles and both column groups
    auto step = [&](int s, auto slot_c, auto mact_c) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr int MACT = decltype(mact_c)::value;
        wait_stage_and_barrier<0>();   // stage s landed; nobody still reads the other slot
        if (s + 1 < nsteps) issue(s + 1, SLOT ^ 1);
        const uint8_t* st = smem + SLOT * kQStage;
        const bool two = s * kQKS + 32 < K;   // block-uniform: the stage's second block is inside K
#pragma unroll
        for (int j = 0; j < 2; j++) {
            if (j == 1 && !two) break;
            i32x4 bq[2];
            float dw[2];
#pragma unroll
            for (int c = 0; c < 2; c++) {
                const int lr = wv * 64 + c * 32 + l32;
                bq[c] = *(const i32x4*)(st + kQA + lr * 64 + (((2 * j + h) ^ swz64(lr)) << 4));
                const uint32_t w = *(const uint32_t*)(st + kQA + kQB + kQSA + (wv * 2 + j) * 256 +
                                                      (c * 32 + l32) * 4);
                dw[c] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> sw_sh[c][j]));
            }
            // sub-tile i: its two MFMAs, then the scaling of their int32 results
#pragma unroll
            for (int i = 0; i < MACT; i++) {
                const int r = i * 32 + l32;
                const i32x4 aq = *(const i32x4*)(st + r * 64 + (((2 * j + h) ^ swz64(r)) << 4));
                // activation scales of this lane's 16 accumulator rows 8g + 4h + (0..3)
                float da[16];
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const f32x4 v = *(const f32x4*)(st + kQA + kQB + i * 256 + j * 128 + (8 * g + 4 * h) * 4);
#pragma unroll
                    for (int u = 0; u < 4; u++) da[4 * g + u] = v[u];
                }
                const i32x16 S0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq, bq[0], i32x16{}, 0, 0, 0);
                const i32x16 S1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aq, bq[1], i32x16{}, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    acc[i][0][v] = fmaf(da[v] * dw[0], (float)S0[v], acc[i][0][v]);
                    acc[i][1][v] = fmaf(da[v] * dw[1], (float)S1[v], acc[i][1][v]);
                }
            }
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    auto k_loop = [&](auto mact_c) __attribute__((always_inline)) {
        issue(0, 0);
        int s = 0;
        for (; s + 2 <= nsteps; s += 2) {
            step(s, S0{}, mact_c);
            step(s + 1, S1{}, mact_c);
        }
        if (s < nsteps) step(s, S0{}, mact_c);
    };
    const int mact = (m_len + 31) >> 5;   // occupied 32-row sub-tiles (block-uniform)
    if (mact >= 4) k_loop(std::integral_constant<int, 4>{});
    else if (mact == 3) k_loop(std::integral_constant<int, 3>{});
    else if (mact == 2) k_loop(std::integral_constant<int, 2>{});
    else k_loop(std::integral_constant<int, 1>{});

    // ---- output rows into the (now idle) ring
    int32_t* s_orow = (int32_t*)smem;
    __syncthreads();
    if (tid < kQBM) {
        const int j = m0 + min(tid, m_len - 1);
        s_orow[tid] = P.out_rows ? P.out_rows[j] : j;
    }
    __syncthreads();

    // ---- epilogue: accumulator (g, u) of lane l holds row 8g + 4(l/32) + u of the
    // 32x32 sub-tile and column l%32 of the column group
    if (MODE == 1) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int n = nt * NTW + wv * 32 + c * 16 + (l32 & 15);
            const bool writer = l32 < 16 && n < N;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (i * 32 >= m_len) continue;
#pragma unroll
                for (int g = 0; g < 4; g++)
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const float up = __shfl_xor(acc[i][c][4 * g + u], 16);
                        const int row = i * 32 + 8 * g + 4 * h + u;
                        if (writer && row < m_len) {
                            const float gv = acc[i][c][4 * g + u];
                            const float hv = gv / (1.0f + __expf(-gv)) * up;
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
            for (int i = 0; i < 4; i++) {
                if (i * 32 >= m_len) continue;
#pragma unroll
                for (int g = 0; g < 4; g++)
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const int row = i * 32 + 8 * g + 4 * h + u;
                        if (row < m_len) ((float*)P.out)[(int64_t)s_orow[row] * P.ldo + n] = acc[i][c][4 * g + u];
                    }
            }
        }
    }
}

template <int MODE>
hipError_t launch_q8a(const GemmArgs& a0, hipStream_t st) {
    GemmArgs a = a0;
    if (a.n_prob < 2) a.p[1] = GemmProblem{};
    constexpr int ntw = q_out_cols<MODE>();
    int64_t total = 0;
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        total += ((int64_t)p.m_tiles_max * ((p.N + ntw - 1) / ntw) + 7) / 8 * 8;
    }
    if (total <= 0) return hipSuccess;
    static PerDeviceOnce lds_cap;
    if (const hipError_t e = set_lds_cap(lds_cap, (const void*)k_gemm_q8a<MODE>, kQLds)) return e;
    a.grid_real = (int32_t)total;
    k_gemm_q8a<MODE><<<(unsigned)total, 64 * kQW, kQLds, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_act(const QuantArgs& a0, hipStream_t st) {
    QuantArgs a = a0;
    int64_t grid[2] = {0, 0};
    for (int i = 0; i < a.n_part; i++) grid[i] = (a.part[i].rows * (a.part[i].K >> 5) + 255) / 256;
    a.blocks0 = grid[0];
    const int64_t total = grid[0] + grid[1];
    if (total <= 0) return hipSuccess;
    if (a.src_bf16) k_quant_act<true><<<(unsigned)total, 256, 0, st>>>(a);
    else k_quant_act<false><<<(unsigned)total, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemm_q8a(const GemmArgs& a, hipStream_t st) {
    return a.mode == 1 ? launch_q8a<1>(a, st) : launch_q8a<0>(a, st);
}

int64_t gemm_q8a_max_threads(const GemmArgs& a) {
    int64_t total = 0;
    for (int i = 0; i < a.n_prob; i++) {
        const GemmProblem& p = a.p[i];
        const int ntw = a.mode == 1 ? kQBN / 2 : kQBN;
        total += ((int64_t)p.m_tiles_max * ((p.N + ntw - 1) / ntw) + 7) / 8 * 8;
    }
    return total * 64 * kQW;
}

}  // namespace moe
