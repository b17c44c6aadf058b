// Internal declarations shared by the libmoe translation units (host dispatcher and
// the gfx950 kernels). Not part of the public ABI; see include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- limits
constexpr int kMaxExperts = 1024;          // row-id pass keeps per-wave counters in LDS
constexpr int kMaxBuckets = kMaxExperts + 1;  // + one bucket for out-of-range ids
constexpr int64_t kRowIdsOneBlockMax = 4096;   // entries handled by the single-workgroup pass
constexpr int kDecMaxSlots = 256;          // GEMV path: n_tokens * n_used
constexpr int64_t kDecMaxWidth = 16384;    // GEMV path: widest staged activation row
constexpr int kAlign = 256;                // workspace sub-buffer alignment

// ---------------------------------------------------------------- row ids (K1)
struct RowIdsArgs {
    const int32_t* ids;   // [n] flattened [T][k]
    int64_t n;            // T * k
    int32_t k, E, B;
    int32_t* ids_src1;    // [n]
    int32_t* ids_dst;     // [n]
    int32_t* bounds;      // [E + 1]
    int32_t* inv;         // optional [n]: position of entry i in the sorted order
    int32_t* tile_off[2]; // optional [E + 1]: exclusive prefix of ceil(count_e / tile_m[i])
    int32_t tile_m[2];
    // optional, with tile_off[i]: per M tile j, {expert e owning it, tile_off[e],
    // bounds[e], rows of e}; tile_cap[i] entries of room (an upper bound on the count)
    int32_t* tile_tab[2];
    int32_t tile_cap[2];
    int32_t* chunk_cnt;   // multi-block scratch [E + 1][n_chunks] (bucket-major)
    int32_t* bucket_tot;  // multi-block scratch [E + 1]
    int64_t n_chunks;
    int64_t chunk;        // entries per chunk (multi-block)
};
size_t row_ids_scratch_bytes(int64_t n, int32_t E);
hipError_t launch_row_ids(const RowIdsArgs& a, hipStream_t st, int* n_launches);

// ---------------------------------------------------------------- grouped GEMM (K3/K4)
// One "problem" = a set of expert segments that share weight shapes. Rows of the
// problem are indexed by a sorted position j; expert segment e owns
// [bounds[e], bounds[e+1]) (routed) or [e*seg_len, (e+1)*seg_len) (uniform: shared
// experts, every token in order).
struct GemmProblem {
    const int8_t* qs1;     // Q8_0 weights [n_mat][N][K] (gate, or the only matrix)
    const uint16_t* d1;    // fp16 scales [n_mat][N][K/32]
    const int8_t* qs2;     // gate/up mode: up weights, same shape
    const uint16_t* d2;
    int32_t N, K;
    const int32_t* bounds;    // routed: [n_seg + 1]; nullptr: uniform segments
    const int32_t* tile_off;  // routed: [n_seg + 1] M-tile prefix (tile height = block M)
    const int32_t* tile_tab;  // routed, optional: per M tile {expert, its first tile, first row, rows}
    int32_t n_seg;
    int32_t seg_len;          // uniform segments
    int32_t m_tiles_max;      // grid upper bound on M tiles of this problem
    const uint16_t* A;        // bf16 activations
    int64_t lda;
    const int32_t* a_rows;    // A row of position j, or nullptr: row (a_row_mod ? j % a_row_mod : j)
    int32_t a_row_mod;
    void* out;
    int64_t ldo;
    const int32_t* out_rows;  // nullptr: row j; else out_rows[j]
    // 1: segments average at most one M tile, so each weight slab is read once per
    // launch and the 64-row kernel's copies of it carry the non-temporal hint (they
    // leave L2 before the activation rows and scales that are read again). The 128-row
    // kernel ignores it: its segments usually share each slab between M tiles.
    int32_t w_once;
};
struct GemmArgs {
    GemmProblem p[2];
    int32_t n_prob;
    int32_t mode;             // 0: fp32 out = acc; 1: bf16 out = silu(acc_gate) * acc_up
    int32_t grid_real;        // blocks carrying tiles (before padding to a multiple of 8)
    // 0: Q8_0 experts; 1: MXFP4 -- qs1/qs2 hold two E2M1 codes per byte ([n_mat][N][K/2],
    // even column in the low nibble), d1/d2 the E8M0 scale bytes ([n_mat][N][K/32])
    int32_t fmt;
};
// Block tile height for a given average rows-per-expert (host heuristic).
int gemm_pick_msub(double avg_rows);
int gemm_tile_m(int msub);
hipError_t launch_gemm_q8(const GemmArgs& a, int msub, hipStream_t st);

// ---------------------------------------------------------------- fp32 grouped matmul (Tiny)
struct GemmF32Args {
    const float* W;        // [E][N][K]
    const float* A;        // [rows][K]
    const int32_t* ids;    // [T*k]
    const int32_t* ids_src1;
    const int32_t* ids_dst;
    const int32_t* bounds; // [E + 1]
    int64_t n_slots;       // T * k
    int32_t E, N, K;
    float* out;            // [T*k][N], row = ids_dst[j]
};
hipError_t launch_gemm_f32(const GemmF32Args& a, hipStream_t st);

// ---------------------------------------------------------------- decode GEMV (D1/D2)
struct DecWeights {
    const int8_t* qs1; const uint16_t* d1;   // [n_mat][N][K]
    const int8_t* qs2; const uint16_t* d2;   // gate/up mode: up weights
    int32_t n_mat, N, K;
    // 0: Q8_0 (int8 codes, fp16 scales); 1: MXFP4 -- qs holds two E2M1 codes per byte
    // ([n_mat][N][K/2], even column in the low nibble) and d the E8M0 scale bytes
    // ([n_mat][N][K/32]); the pointers are read as bytes
    int32_t fmt;
};
struct DecArgs {
    const int32_t* ids;     // [T][k]
    int32_t T, k, E;
    DecWeights rw;          // routed experts
    DecWeights sw;          // shared experts (n_mat = 0: none)
    // activation of routed slot i = (t, s): act + (t*act_B + s % act_B) * K
    const void* act; int32_t act_type; int32_t act_B;   // act_type: 1 bf16, 0 fp32
    // activation of shared expert j, token t: sact + (j*sact_jstride + t) * K
    const void* sact; int32_t sact_type; int64_t sact_jstride;
    float* out;             // routed: [T*k][N]
    float* sout;            // shared: [n_mat][T][N]
    int32_t mode;           // 0 raw, 1 silu(gate) * up
    int32_t d_max;          // upper bound on distinct experts (grid)
    int32_t rows_per_block;
    // down mode, optional: the weighted sum over each token's slots (route_w, or weight 1
    // when null) plus the shared experts, written to out_tok [T][N] by the GEMV itself
    const float* route_w;
    float* out_tok;
};
// *reduced (if given) tells whether out_tok was written (the reduction was fused); when
// false the per-slot rows are in out / sout and the reduce kernel still has to run.
hipError_t launch_decode(const DecArgs& a, hipStream_t st, bool* reduced = nullptr);

// ---------------------------------------------------------------- router top-k
struct RouterArgs {
    const float* logits;  // [T][E]
    int64_t T;
    int32_t E;            // <= kMaxExperts
    int32_t k;            // 1 <= k <= E
    int32_t* ids;         // [T][k]
    float* w;             // [T][k]
};
hipError_t launch_router(const RouterArgs& a, hipStream_t st);

// ---------------------------------------------------------------- reduce / scatter (K5)
struct ReduceArgs {
    const int32_t* ids;     // [T][k]
    const float* route_w;   // [T][k] or nullptr
    int32_t T, k, E, N;
    const float* y;         // per-slot rows [T*k][N] (slot order)
    const float* ysh;       // shared rows [S][T][N] or nullptr
    int32_t S;
    float* out;             // weighted: [T][N]; zero-fix mode: [T*k][N]
    int32_t mode;           // 0: weighted sum (+ shared), 1: zero rows of invalid slots
};
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st);

}  // namespace moe
