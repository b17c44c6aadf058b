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

template <int MSUB, int MODE>
__global__ __launch_bounds__(kThreads) void k_gemm_q8(GemmArgs args) {
    constexpr int BM = 32 * MSUB;
    constexpr int NTW = MODE == 1 ? 128 : 256;  // output columns per block
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * 128];

    // ---- logical tile (XCD-aware remap: the hardware deals blocks round-robin over 8 XCDs)
    const int G = gridDim.x;
    const int fb = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
    if (fb >= args.grid_real) return;
    int f = fb, pi = 0;
    {
        const GemmProblem& P0 = args.p[0];
        const int t0 = P0.m_tiles_max * ((P0.N + NTW - 1) / NTW);
        if (f >= t0) {
            pi = 1;
            f -= t0;
        }
    }
    const GemmProblem& P = args.p[pi];
    const int N = P.N, K = P.K;
    const int n_nt = (N + NTW - 1) / NTW;
    const int mt = f / n_nt, nt = f - mt * n_nt;
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

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int nsteps = (K + 63) >> 6;

    // ---- activation rows this thread stages: row r = tid/8 + 32*i, 16-byte chunk c = tid%8
    const int ac = tid & 7;
    const uint16_t* arow[MSUB];
    int a_lds_off[MSUB];
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
        const int r = (tid >> 3) + 32 * i;
        const int j = m0 + min(r, m_len - 1);
        const int64_t src = P.a_rows ? (int64_t)P.a_rows[j]
                                     : (int64_t)(P.a_row_mod ? j % P.a_row_mod : j);
        arow[i] = P.A + src * P.lda + ac * 8;
        a_lds_off[i] = r * 128 + ((ac ^ (r & 7)) << 4);
    }

    // ---- weight rows of this lane: column group 0 and 1
    int nB0, nB1;
    const int8_t* qb1;
    const uint16_t* db1;
    if (MODE == 1) {
        nB0 = nt * 128 + wv * 32 + l32;
        nB1 = nB0;
        qb1 = P.qs2;
        db1 = P.d2;
    } else {
        nB0 = nt * 256 + wv * 64 + l32;
        nB1 = nB0 + 32;
        qb1 = P.qs1;
        db1 = P.d1;
    }
    const int64_t KB = K >> 5;
    const int64_t r0 = (int64_t)e * N + min(nB0, N - 1);
    const int64_t r1 = (int64_t)e * N + min(nB1, N - 1);
    const int8_t* q0p = P.qs1 + r0 * K + 32 * h;
    const int8_t* q1p = qb1 + r1 * K + 32 * h;
    const uint16_t* s0p = P.d1 + r0 * KB + h;
    const uint16_t* s1p = db1 + r1 * KB + h;

    f32x16 acc[MSUB][2];
#pragma unroll
    for (int i = 0; i < MSUB; i++)
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][c][v] = 0.f;

    i32x4 ra[MSUB];
    i32x4 rb[2][2];
    uint16_t rs[2];

    auto load_a = [&](int s) {
        const int kk = s * 64 + ac * 8;
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            if (kk < K) ra[i] = *(const i32x4*)(arow[i] + s * 64);
            else ra[i] = i32x4{0, 0, 0, 0};
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < MSUB; i++) *(i32x4*)(&lds[buf][a_lds_off[i]]) = ra[i];
    };
    auto load_b = [&](int s) {
        if (s * 64 + 32 * h < K) {
            const int8_t* p0 = q0p + (int64_t)s * 64;
            const int8_t* p1 = q1p + (int64_t)s * 64;
            rb[0][0] = *(const i32x4*)(p0);
            rb[0][1] = *(const i32x4*)(p0 + 16);
            rb[1][0] = *(const i32x4*)(p1);
            rb[1][1] = *(const i32x4*)(p1 + 16);
            rs[0] = s0p[2 * s];
            rs[1] = s1p[2 * s];
        } else {
            rb[0][0] = rb[0][1] = rb[1][0] = rb[1][1] = i32x4{0, 0, 0, 0};
            rs[0] = rs[1] = 0;
        }
    };

    load_a(0);
    load_b(0);
    store_a(0);
    if (nsteps > 1) load_a(1);
    __syncthreads();

    for (int s = 0; s < nsteps; s++) {
        const int cur = s & 1;
        bf16x8 bf[2][4];
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const float d = half_bits_to_float(rs[c]);
            bf[c][0] = dequant8(rb[c][0][0], rb[c][0][1], d);
            bf[c][1] = dequant8(rb[c][0][2], rb[c][0][3], d);
            bf[c][2] = dequant8(rb[c][1][0], rb[c][1][1], d);
            bf[c][3] = dequant8(rb[c][1][2], rb[c][1][3], d);
        }
        if (s + 1 < nsteps) load_b(s + 1);
        const uint8_t* L = lds[cur];
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            if (i * 32 < m_len) {
                const int r = i * 32 + l32;
#pragma unroll
                for (int ss = 0; ss < 4; ss++) {
                    const int chunk = (4 * h + ss) ^ (r & 7);
                    const bf16x8 af = *(const bf16x8*)(L + r * 128 + (chunk << 4));
                    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[0][ss], acc[i][0], 0, 0, 0);
                    acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[1][ss], acc[i][1], 0, 0, 0);
                }
            }
        }
        if (s + 1 < nsteps) {
            store_a(cur ^ 1);
            if (s + 2 < nsteps) load_a(s + 2);
        }
        __syncthreads();
    }

    // ---- epilogue. Accumulator v of lane l holds row 8*(v/4) + 4*(l/32) + v%4 of
    // the 32x32 sub-tile and column l%32.
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
        if (i * 32 >= m_len) continue;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int row = i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (row >= m_len) continue;
            const int j = m0 + row;
            const int64_t orow = P.out_rows ? (int64_t)P.out_rows[j] : (int64_t)j;
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

template <int MSUB>
hipError_t launch_msub(const GemmArgs& a, int grid, hipStream_t st) {
    if (a.mode == 1) k_gemm_q8<MSUB, 1><<<grid, kThreads, 0, st>>>(a);
    else k_gemm_q8<MSUB, 0><<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
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
    int64_t total = 0;
    for (int i = 0; i < a.n_prob; i++) total += (int64_t)a.p[i].m_tiles_max * gemm_n_tiles(a.mode, a.p[i].N);
    if (a.n_prob < 2) a.p[1] = GemmProblem{};
    if (total <= 0) return hipSuccess;
    a.grid_real = (int32_t)total;
    const int grid = (int)((total + 7) / 8 * 8);
    switch (msub) {
        case 2: return launch_msub<2>(a, grid, st);
        case 4: return launch_msub<4>(a, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
