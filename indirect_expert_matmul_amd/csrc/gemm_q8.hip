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
//   * Block = 4 wavefronts. Block tile = BM rows (BM = 32*MSUB, all inside one
//     expert segment) x 4 waves x 64 weight rows. Waves split N, so every wave
//     dequantizes only its own weight rows and the tile's activation rows are
//     shared through LDS.
//   * K advances 64 at a time = two Q8_0 blocks. Lane half h = lane/32 owns Q8_0
//     block (2*step + h) of its weight row: one 32-byte contiguous load and one
//     fp16 scale per lane. It dequantizes d*q in fp32 (exact) and rounds to bf16
//     (v_cvt_pk_bf16_f32, nearest-even) straight into MFMA B-operand registers --
//     the weights never pass through LDS.
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulate. Inside a 64-wide K step, lane
//     half h and element e of MFMA sub-step ss stand for k = 32h + 8ss + e on BOTH
//     operands, so A and B agree on k whatever order the unit sums in.
//   * Activation rows are gathered (indirect rows through ids_src1) into a
//     double-buffered LDS tile with an XOR swizzle of the 16-byte chunk index by
//     (row & 7), so the 32 rows an MFMA A-read touches hit distinct banks.
//   * Loads for step s+1 are in flight while step s runs its MFMAs; one barrier
//     per step.
//   * Block index -> tile is XCD-aware: consecutive logical tiles (the N tiles of
//     one M tile, then the M tiles of the same expert) go to the same XCD, so they
//     share that XCD's L2 for activations and weights.
//   * Tiles are located on device from the row-id pass's M-tile prefix (no host
//     readback); blocks past the real tile count exit at once.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

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

// LDS byte address of a shared-memory pointer (the M0 operand of an LDS DMA).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS copies. Lane i of the wave reads base + voff (a per-lane
// 32-bit byte offset from a wave-uniform 64-bit base) and writes LDS
// [lds_base + size*i, +size). Issued as inline asm so that the waits are ours: the
// compiler would otherwise drain every outstanding load at each barrier. M0 is saved
// and restored around the copy.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
    uint32_t tmp;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(tmp)
        : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(base)
        : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds_base) {
    uint32_t tmp;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dword %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(tmp)
        : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(base)
        : "memory");
}
// Wait until at most N of this wave's vector-memory operations are outstanding,
// and until this wave's LDS reads returned, then meet the other waves at the barrier
// (LDS DMA data of every wave landed; no wave still reads a buffer about to be refilled).
template <int N>
__device__ __forceinline__ void wait_stage_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// LDS swizzles (16-byte chunk index XOR a function of the row), chosen so the 8 / 16
// rows one ds_read_b128 phase touches fall on distinct banks (measured on gfx950).
__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }   // 8 chunks/row
__device__ __forceinline__ int swz_b(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }  // 4 chunks/row

// Block tile: BM = 32*MSUB activation rows (one expert segment) x 256 weight rows
// (4 waves x 2 column groups x 32). One pipeline stage = one 64-wide K step:
//   A  BM rows x 128 B (bf16), 16-byte chunk c of row r stored at chunk c ^ swz_a(r)
//   B  256 weight rows x 64 B (int8), chunk c of local row r stored at c ^ swz_b(r)
//   S  256 rows x 2 half-steps: the 4-byte aligned word holding that fp16 scale
// NS stages live in LDS at once; stage s+NS-1 is being fetched while s computes.
// Block -> tile: XCD x (= block index mod 8, how the dispatcher deals blocks) owns
// the M tiles congruent to x mod 8 and runs all N tiles of one M tile back to back,
// so they share the XCD's L2 for the activation rows, and real tiles spread evenly
// over the 8 XCDs even though the grid is sized by an upper bound.
template <int MSUB, int MODE, int NS>
__global__ __launch_bounds__(kThreads) void k_gemm_q8(GemmArgs args) {
    constexpr int BM = 32 * MSUB;
    constexpr int NTW = MODE == 1 ? 128 : 256;  // output columns per block
    constexpr int A_BYTES = BM * 128;
    constexpr int B_BYTES = 256 * 64;
    constexpr int S_BYTES = 512 * 4;
    constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    constexpr int L = MSUB + 4 + 2;  // DMA instructions per wave per stage
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int32_t s_orow[BM];

    // ---- tile of this block
    int b = (int)blockIdx.x, pi = 0;
    {
        const GemmProblem& P0 = args.p[0];
        const int reg0 = ((P0.m_tiles_max + 7) >> 3) * 8 * ((P0.N + NTW - 1) / NTW);
        if (b >= reg0) {
            pi = 1;
            b -= reg0;
        }
    }
    const GemmProblem& P = args.p[pi];
    const int N = P.N, K = P.K;
    const int n_nt = (N + NTW - 1) / NTW;
    const int jx = b >> 3;
    const int mt = (jx / n_nt) * 8 + (b & 7), nt = jx - (jx / n_nt) * n_nt;
    if (mt >= P.m_tiles_max) return;
    int e, m0, m_len;
    if (P.bounds) {
        if (mt >= P.tile_off[P.n_seg]) return;
        int lo = 0, hi = P.n_seg;  // tile_off[lo] <= mt < tile_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (P.tile_off[mid] <= mt) lo = mid; else hi = mid;
        }
        e = lo;
        m0 = P.bounds[e] + (mt - P.tile_off[e]) * BM;
        m_len = min(BM, P.bounds[e + 1] - m0);
    } else {
        const int tps = (P.seg_len + BM - 1) / BM;
        e = mt / tps;
        if (e >= P.n_seg) return;
        m0 = e * P.seg_len + (mt - e * tps) * BM;
        m_len = min(BM, (e + 1) * P.seg_len - m0);
    }

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR
    const int nsteps = (K + 63) >> 6;
    const int nfull = K >> 6;  // steps with all 64 columns inside K
    const int64_t KB = K >> 5;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    if (tid < BM) {
        const int j = m0 + min(tid, m_len - 1);
        s_orow[tid] = P.out_rows ? P.out_rows[j] : j;
    }

    // weight row (within the expert) of local row lr (0..63) of wave w
    auto wrow = [&](int w, int lr) -> int {
        const int c = lr >> 5, r = lr & 31;
        const int n = MODE == 1 ? nt * 128 + w * 32 + r : nt * 256 + w * 64 + c * 32 + r;
        return min(n, N - 1);
    };

    // ---- DMA geometry: wave-uniform bases, per-lane 32-bit byte offsets (step 0)
    const uint8_t* a_base = (const uint8_t*)uniform_ptr(P.A);
    uint32_t a_off[MSUB];
    int a_lc[MSUB];
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
        const int R = (wv * MSUB + i) * 8 + (lane >> 3);  // tile row this lane fetches
        const int lc = (lane & 7) ^ swz_a(R);              // logical 16-byte chunk
        const int j = m0 + min(R, m_len - 1);
        const int64_t src = P.a_rows ? (int64_t)P.a_rows[j]
                                     : (int64_t)(P.a_row_mod ? j % P.a_row_mod : j);
        a_off[i] = (uint32_t)(src * P.lda * 2 + lc * 16);
        a_lc[i] = lc;
    }
    const int8_t* b_base1 = (const int8_t*)uniform_ptr(P.qs1 + (int64_t)e * N * K);
    const int8_t* b_base2 = MODE == 1 ? (const int8_t*)uniform_ptr(P.qs2 + (int64_t)e * N * K) : b_base1;
    uint32_t b_off[4];
    int b_lc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int lr = 16 * i + (lane >> 2);
        const int lc = (lane & 3) ^ swz_b(lr);
        b_off[i] = (uint32_t)((int64_t)wrow(wv, lr) * K + lc * 16);
        b_lc[i] = lc;
    }
    const uint8_t* s_base1 = (const uint8_t*)uniform_ptr(P.d1 + (int64_t)e * N * KB);
    const uint8_t* s_base2 = MODE == 1 ? (const uint8_t*)uniform_ptr(P.d2 + (int64_t)e * N * KB) : s_base1;
    uint32_t s_offw[2];
    int s_h[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int pl = 64 * i + lane;  // pair within this wave: local row pl/2, half pl&1
        const int lr = pl >> 1, hh = pl & 1;
        // byte offset of the scale; the DMA fetches the aligned word holding it
        s_offw[i] = (uint32_t)(((int64_t)wrow(wv, lr) * KB + hh) * 2);
        s_h[i] = hh;
    }
    // In gate/up mode waves 0..3 own gate rows in local rows 0..31 and up rows in 32..63:
    // DMA instruction i covers local rows 16i..16i+15, so i < 2 reads gate, i >= 2 up.

    // Issue stage s. Full steps use the constant offsets; the half step past a K that
    // is an odd multiple of 32 pulls its upper half back inside the row (those weights
    // are zeroed at dequant time), so every address stays in bounds.
    auto issue = [&](int s) {
        const uint32_t st = lds0 + (uint32_t)((s % NS) * STAGE);
        const int k0 = s * 64;
        const bool full = s < nfull;
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            const uint32_t adj = (!full && k0 + a_lc[i] * 8 >= K) ? 64u : 0u;
            dma16(a_base + (int64_t)k0 * 2, a_off[i] - adj, st + (wv * MSUB + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t adj = (!full && k0 + b_lc[i] * 16 >= K) ? 32u : 0u;
            const int8_t* bb = (MODE == 1 && i >= 2) ? b_base2 : b_base1;
            dma16(bb + k0, b_off[i] - adj, st + A_BYTES + wv * 4096 + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            // the aligned 4-byte word holding the scale (its other half is the
            // neighbouring scale, or at most 2 bytes past the end of the array, inside
            // the allocation's page); past K one block back (that weight is zeroed)
            const uint32_t adj = (!full && k0 + 32 * s_h[i] >= K) ? 2u : 0u;
            const uint8_t* sb = (MODE == 1 && i >= 1) ? s_base2 : s_base1;
            dma4(sb + 4 * s, (s_offw[i] - adj) & ~3u, st + A_BYTES + B_BYTES + (wv * 2 + i) * 256);
        }
    };

    f32x16 acc[MSUB][2];
#pragma unroll
    for (int i = 0; i < MSUB; i++)
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][c][v] = 0.f;

    // dequant geometry of this lane: column group c holds local row c*32 + l32, half h
    int bq_off[2][2];
    int sc_off[2];
    int sc_shift[2];
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int lr = c * 32 + l32;
        bq_off[c][0] = A_BYTES + wv * 4096 + lr * 64 + (((2 * h) ^ swz_b(lr)) << 4);
        bq_off[c][1] = A_BYTES + wv * 4096 + lr * 64 + (((2 * h + 1) ^ swz_b(lr)) << 4);
        sc_off[c] = A_BYTES + B_BYTES + wv * 512 + (lr * 2 + h) * 4;
        const uint32_t sbyte = (uint32_t)(((int64_t)wrow(wv, lr) * KB + h) * 2);
        sc_shift[c] = (sbyte & 2) ? 16 : 0;  // which half of the aligned word holds it
    }

    // dequantize B of stage s (already in LDS) into MFMA operand registers
    auto dequant = [&](int s, bf16x8 (&bf)[2][4]) {
        const uint8_t* st = smem + (s % NS) * STAGE;
        const bool in_k = s * 64 + 32 * h < K;   // false only for the upper half past K
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const i32x4 q0 = *(const i32x4*)(st + bq_off[c][0]);
            const i32x4 q1 = *(const i32x4*)(st + bq_off[c][1]);
            const uint32_t sw = *(const uint32_t*)(st + sc_off[c]);
            float d = half_bits_to_float((uint16_t)(sw >> sc_shift[c]));
            d = in_k ? d : 0.f;
            bf[c][0] = dequant8(q0[0], q0[1], d);
            bf[c][1] = dequant8(q0[2], q0[3], d);
            bf[c][2] = dequant8(q1[0], q1[1], d);
            bf[c][3] = dequant8(q1[2], q1[3], d);
        }
    };
    auto mfma_step = [&](int s, const bf16x8 (&bf)[2][4]) {
        const uint8_t* st = smem + (s % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            const int r = i * 32 + l32;
#pragma unroll
            for (int ss = 0; ss < 4; ss++) {
                const int chunk = (4 * h + ss) ^ swz_a(r);
                const bf16x8 af = *(const bf16x8*)(st + r * 128 + (chunk << 4));
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[0][ss], acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[1][ss], acc[i][1], 0, 0, 0);
            }
        }
    };
    for (int s = 0; s < NS - 1 && s < nsteps; s++) issue(s);
    for (int s = 0; s < nsteps; s++) {
        const int ahead = min(NS - 2, nsteps - 1 - s);  // stages after s already issued
        if (ahead >= 2) wait_stage_and_barrier<2 * L>();
        else if (ahead == 1) wait_stage_and_barrier<L>();
        else wait_stage_and_barrier<0>();
        // the buffer refilled here held step s-1, which every wave finished
        if (s + NS - 1 < nsteps) issue(s + NS - 1);
        bf16x8 bf[2][4];
        dequant(s, bf);
        mfma_step(s, bf);
    }

    // ---- epilogue. Accumulator v of lane l holds row 8*(v/4) + 4*(l/32) + v%4 of
    // the 32x32 sub-tile and column l%32.
    const int nB0 = MODE == 1 ? nt * 128 + wv * 32 + l32 : nt * 256 + wv * 64 + l32;
    const int nB1 = MODE == 1 ? nB0 : nB0 + 32;
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
        if (i * 32 >= m_len) continue;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int row = i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (row >= m_len) continue;
            const int64_t orow = s_orow[row];
            if (MODE == 1) {
                if (nB0 < N) {
                    const float g = acc[i][0][v], u = acc[i][1][v];
                    const float hv = g / (1.0f + __expf(-g)) * u;
                    ((__bf16*)P.out)[orow * P.ldo + nB0] = (__bf16)hv;
                }
            } else {
                float* o = (float*)P.out + orow * P.ldo;
                if (nB0 < N) o[nB0] = acc[i][0][v];
                if (nB1 < N) o[nB1] = acc[i][1][v];
            }
        }
    }
}

template <int MSUB, int NS>
constexpr int stage_lds() { return NS * (32 * MSUB * 128 + 256 * 64 + 512 * 4); }

template <int MSUB, int MODE, int NS>
hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr int lds = stage_lds<MSUB, NS>();
    static bool attr_set = false;   // raise the dynamic LDS cap once per process
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute((const void*)k_gemm_q8<MSUB, MODE, NS>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    k_gemm_q8<MSUB, MODE, NS><<<grid, kThreads, lds, st>>>(a);
    return hipGetLastError();
}

template <int MSUB>
hipError_t launch_msub(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr int NS = MSUB == 2 ? 3 : 2;
    if (a.mode == 1) return launch_one<MSUB, 1, NS>(a, grid, st);
    return launch_one<MSUB, 0, NS>(a, grid, st);
}

}  // namespace

int gemm_pick_msub(double avg_rows) {
    if (avg_rows <= 64) return 2;
    return 4;
}
int gemm_tile_m(int msub) { return 32 * msub; }
int64_t gemm_n_tiles(int mode, int32_t N) {
    const int ntw = mode == 1 ? 128 : 256;
    return (N + ntw - 1) / ntw;
}

hipError_t launch_gemm_q8(const GemmArgs& a0, int msub, hipStream_t st) {
    GemmArgs a = a0;
    if (a.n_prob < 2) a.p[1] = GemmProblem{};
    int64_t total = 0;
    for (int i = 0; i < a.n_prob; i++)
        total += (int64_t)((a.p[i].m_tiles_max + 7) / 8 * 8) * gemm_n_tiles(a.mode, a.p[i].N);
    if (total <= 0) return hipSuccess;
    a.grid_real = (int32_t)total;
    const int grid = (int)total;
    switch (msub) {
        case 2: return launch_msub<2>(a, grid, st);
        case 4: return launch_msub<4>(a, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
