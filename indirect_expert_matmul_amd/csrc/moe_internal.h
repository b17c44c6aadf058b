// Internal declarations shared by the libmoe translation units (host dispatcher and
// the gfx950 kernels). Not part of the public ABI; see include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace moe {

// ---------------------------------------------------------------- per-device set-up
// One-time set-up that depends on the device (raising a kernel's dynamic LDS cap, an
// occupancy query): each kernel keeps one PerDeviceOnce. The first call on a device
// runs the set-up under the lock and stores its int result; later calls on that device
// read it without locking. Safe to call from several host threads at once.
constexpr int kMaxDevices = 64;
struct PerDeviceOnce {
    std::mutex mu;
    std::atomic<int> done[kMaxDevices];
    int value[kMaxDevices];
};
// f(int& value) -> hipError_t runs once per device (the current one); on success the
// stored value is returned through *value (if given). A failed set-up is retried by
// the next call.
template <class F>
hipError_t once_per_device(PerDeviceOnce& o, F&& f, int* value = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (o.done[dev].load(std::memory_order_acquire) == 0) {
        std::lock_guard<std::mutex> g(o.mu);
        if (o.done[dev].load(std::memory_order_relaxed) == 0) {
            int v = 0;
            e = f(v);
            if (e != hipSuccess) return e;
            o.value[dev] = v;
            o.done[dev].store(1, std::memory_order_release);
        }
    }
    if (value) *value = o.value[dev];
    return hipSuccess;
}
// Raise kern's dynamic LDS cap to bytes, once per device.
inline hipError_t set_lds_cap(PerDeviceOnce& o, const void* kern, int bytes) {
    return once_per_device(o, [&](int&) {
        return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    });
}

// ---------------------------------------------------------------- limits
constexpr int kMaxExperts = 1024;          // row-id pass keeps per-wave counters in LDS
constexpr int kMaxBuckets = kMaxExperts + 1;  // + one bucket for out-of-range ids
constexpr int64_t kRowIdsOneBlockMax = 4096;   // entries handled by the single-workgroup pass
constexpr int kDecMaxSlots = 256;          // GEMV path: n_tokens * n_used
constexpr int64_t kDecMaxWidth = 16384;    // GEMV path: widest staged activation row
constexpr int kDecAutoSlots = 48;          // automatic GEMV choice, wave kernels: n_tokens * n_used
constexpr int kAlign = 256;                // workspace sub-buffer alignment

// Sets the thread-local message moe_last_error() returns.
void set_last_error(const char* msg);

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
    // extra rows the last M tile of an expert may hold beyond tile_m (0, or 32 when the
    // GEMM's tiles have room for tile_m + 32 rows): an expert with up to tile_m + 32 rows
    // past its full tiles gets one tile fewer
    int32_t tile_x[2];
    // optional, with tile_off[i]: per M tile j, {expert e owning it, tile_off[e],
    // bounds[e], rows of e}; tile_cap[i] entries of room (an upper bound on the count)
    int32_t* tile_tab[2];
    int32_t tile_cap[2];
    // multi-block scratch (row_ids_carve_scratch places it in row_ids_scratch_bytes):
    int32_t* chunk_cnt;   // [E + 1][n_chunks] per-chunk counts, then their prefix over chunks
    int32_t* bucket_tot;  // [E + 1] bucket totals
    int32_t* wcnt;        // [n_chunks][waves][E + 1] per-wave counts of each chunk
    uint16_t* rank16;     // [n] rank of each entry among its wave's entries of its bucket
    int64_t n_chunks;
    int64_t chunk;        // entries per chunk (multi-block)
    uint32_t k_magic;     // ii / k == (ii * k_magic) >> k_shift for ii < 2^31
    int32_t k_shift;
};
size_t row_ids_scratch_bytes(int64_t n, int32_t E);
void row_ids_carve_scratch(RowIdsArgs& a, void* scratch);
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
    int32_t tile_x;           // extra rows of a segment's last M tile (as RowIdsArgs::tile_x)
    int32_t tile_m;           // 160-row wide kernel only: M-tile height (128 with tile_x = 32,
                              // or 160); 0 elsewhere
    const uint16_t* A;        // bf16 activations
    int64_t lda;
    // quantized-activation GEMM only: int8 activation codes [rows][K] and float32
    // scales [rows][K/32] (one per 32-column block); rows indexed as for A
    const int8_t* Aq;
    const float* Ad;
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
    // even column in the low nibble), d1/d2 the E8M0 scale bytes ([n_mat][N][K/32]);
    // 2: IQ4_NL -- codes packed as MXFP4's, d1/d2 fp16 scales as Q8_0's; 3: IQ4_XS --
    // codes as IQ4_NL's, d1/d2 8-byte super-block records ([n_mat][N][K/256][8])
    int32_t fmt;
};
// Block tile height for a given average rows-per-expert (host heuristic).
int gemm_pick_msub(double avg_rows);
int gemm_tile_m(int msub);
// Extra rows (0 or 32) the last M tile of an expert may hold on the GEMM path for this
// tile choice, weight format and K: 32 where the 128-row wide kernel runs, whose
// 160-row variant takes such tiles (MXFP4: when every scale tensor of the launch
// starts at an even address; IQ4_NL: at a 4-byte aligned one; IQ4_XS: 8-byte).
int gemm_tile_x(int msub, int fmt, int64_t K, bool scales_aligned);
// Puts routed problem p and tile table q of the row-id pass on the 160-row kernel's tiles.
void gemm_set_tall(GemmProblem& p, RowIdsArgs& r, int q);
// M tiles of a segment of `rows` rows: tiles of tm rows, the last one holding up to
// tm + tx (at least one tile for a non-empty segment).
inline __host__ __device__ int tiles_of(int rows, int tm, int tx) {
    if (rows <= 0) return 0;
    const int t = (rows - tx + tm - 1) / tm;
    return t > 1 ? t : 1;
}
hipError_t launch_gemm_q8(const GemmArgs& a, int msub, hipStream_t st);
// Upper bound on the work-items launch_gemm_q8 would launch for these arguments (a
// dispatch holds fewer than 2^32).
int64_t gemm_q8_max_threads(const GemmArgs& a, int msub);

// ---------------------------------------------------------------- quantized activations
// Rows of 32-column blocks -> int8 codes and one float32 scale per block:
// d = max|x| / 127, q = rint(x / d) (float32, ties to even), clamped to [-127, 127].
struct QuantPart {
    const void* src;   // [rows][K], bf16 bits (src_bf16) or float32
    int64_t rows, K;   // K % 32 == 0
    int8_t* q;         // [rows][K]
    float* d;          // [rows][K/32]
};
struct QuantArgs {
    QuantPart part[2]; // one launch quantizes up to two tensors (e.g. h and the shared h)
    int32_t n_part;
    int32_t src_bf16;
    int64_t blocks0;   // set by the launcher: thread blocks of part 0
};
hipError_t launch_quant_act(const QuantArgs& a, hipStream_t st);
// Grouped GEMM of Q8_0 experts with quantized activations (GemmProblem.Aq / Ad; fmt 0
// weights; tile_tab required for routed problems; 128-row tiles: m_tiles_max and the
// row-id pass's tile tables must use tile height 128).
hipError_t launch_gemm_q8a(const GemmArgs& a, hipStream_t st);
int64_t gemm_q8a_max_threads(const GemmArgs& a);
constexpr int kQ8aTileM = 128;

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
    // ([n_mat][N][K/32]); the pointers are read as bytes; 2: IQ4_NL -- codes as MXFP4's,
    // fp16 scales as Q8_0's; 3: IQ4_XS -- codes as MXFP4's, 8-byte super-block records
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
    // wave kernels: rows per shared-expert unit (0: rows_per_block). A shared unit serves
    // every token, so it streams its rows once per pass of P tokens; fewer rows per unit
    // keep its length near a routed unit's.
    int32_t rows_shared;
    // down mode, optional: the weighted sum over each token's slots (route_w, or weight 1
    // when null) plus the shared experts, written to out_tok [T][N] by the GEMV itself
    const float* route_w;
    float* out_tok;
};
// *reduced (if given) tells whether out_tok was written (the reduction was fused); when
// false the per-slot rows are in out / sout and the reduce kernel still has to run.
hipError_t launch_decode(const DecArgs& a, hipStream_t st, bool* reduced = nullptr);

// ---------------------------------------------------------------- row gather (K2)
struct GatherArgs {
    const void* src;      // [src_rows][row_bytes]
    int64_t src_rows;
    int64_t row_bytes;    // a multiple of 2
    const int32_t* idx;   // [n]
    int64_t n;
    void* dst;            // [n][row_bytes]
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t st);

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
