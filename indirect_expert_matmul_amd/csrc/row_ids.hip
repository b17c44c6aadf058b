// Row-id pass (K1): the three maps of the deterministic MoE path -- src1 rows
// reordered so every expert's rows are contiguous (ids_src1), the same order for
// dst (ids_dst) and each expert's bounds (expert_bounds) -- built without any
// atomic slot counter ("CUDA: better MoE implementation", sections 2 and 2.1: the
// old gather claimed destination slots with an atomic increment, which was slow
// and made the row order, hence the float summation order, change run to run).
//
// gfx950 design: a stable counting sort built from wavefront primitives.
//   * Each wave owns a contiguous range of entries (t*k + s order) and walks it 64
//     at a time. Lanes holding the same bucket find each other through a per-bucket
//     64-bit mask in LDS that every lane of the group ORs its bit into (OR is
//     order-independent, so the mask is the same on every run; the one-workgroup pass
//     with more than 512 buckets uses one ballot per bit of the bucket id instead);
//     the group's lowest lane adds the group size to the wave's LDS counter (one
//     writer per counter, no atomic counter), and a lane's rank inside its group is a
//     masked bit count (mbcnt).
//   * Per-bucket exclusive scans over waves (and, for large inputs, over
//     workgroups), then over buckets, give every (wave, bucket) its first output
//     position; a second walk over the same range places every entry. Entries keep
//     their (t, s) order inside a bucket, so the result is unique.
//   * Bucket E collects ids outside [0, E): they land after all expert segments.
//   * Inputs up to kRowIdsOneBlockMax entries run as one 1024-thread workgroup (one
//     launch); larger ones use count / scan-over-chunks / place, where every place
//     block scans the bucket totals itself (with at most kLocalScanChunks chunks it
//     also sums the per-chunk counts, and the scan over chunks is skipped).
//     The count pass already ranks every entry inside its (wave, bucket) group and
//     stores that rank (16 bits) and each wave's counts, so the place pass needs no
//     ballots: position = bucket start + chunk offset + wave offset + rank.
#include "moe_internal.h"

namespace moe {
namespace {

#ifndef MOE_ROWIDS_CHUNKS
#define MOE_ROWIDS_CHUNKS 1024   // chunks the multi-block pass aims at
#endif
#ifndef MOE_ROWIDS_MAXB
#define MOE_ROWIDS_MAXB 32       // batches of 64 per wave per chunk, at most
#endif
#ifndef MOE_ROWIDS_PRE
#define MOE_ROWIDS_PRE 8         // batches of ids loaded ahead of their use (one-workgroup pass)
#endif
#ifndef MOE_ROWIDS_COUNT_PRE
#define MOE_ROWIDS_COUNT_PRE 4   // batches per group in the count pass (two groups in flight)
#endif

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxBatchesPerWave = MOE_ROWIDS_MAXB;
static_assert(kMaxBatchesPerWave * 64 <= 65536, "ranks inside a wave's range are 16-bit");
constexpr int64_t kMaxChunk = (int64_t)kThreads * kMaxBatchesPerWave;   // 16384 entries

// Entries per chunk of the multi-block pass: about MOE_ROWIDS_CHUNKS chunks, each wave
// walking 2 to kMaxBatchesPerWave batches of 64 (long enough walks keep the id loads
// ahead of their use, and few chunks keep the per-chunk counts small).
int64_t chunk_len(int64_t n) {
    constexpr int64_t kTarget = MOE_ROWIDS_CHUNKS;
    int64_t bpw = (n + kTarget * (int64_t)kThreads - 1) / (kTarget * (int64_t)kThreads);
    bpw = bpw < 2 ? 2 : (bpw > kMaxBatchesPerWave ? kMaxBatchesPerWave : bpw);
    return bpw * kThreads;
}

__device__ __forceinline__ int bucket_of(int32_t e, int32_t E) {
    return (e >= 0 && e < E) ? e : E;
}

// Lanes (among `active`) whose bucket equals this lane's bucket: per bit of the bucket
// id, keep the lanes that agree with this lane on that bit (the bit's ballot, inverted
// where this lane's bit is 0).
__device__ __forceinline__ uint64_t match_bucket(int b, uint64_t active, int nbits) {
    uint32_t lo = (uint32_t)active, hi = (uint32_t)(active >> 32);
    for (int i = 0; i < nbits; i++) {
        const uint32_t bit = ((uint32_t)b >> i) & 1u;
        const uint64_t bal = __ballot(bit);
        const uint32_t flip = bit - 1u;   // 0 if the bit is set, all ones if not
        lo &= (uint32_t)bal ^ flip;
        hi &= (uint32_t)(bal >> 32) ^ flip;
    }
    return ((uint64_t)hi << 32) | lo;
}

// Number of set bits of m strictly below this lane.
__device__ __forceinline__ int rank_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The same lane set through this wave's LDS mask words (one per bucket): each active
// lane clears its bucket's word, ORs its own bit into it and reads it back. A wave's
// LDS instructions execute in order (every clear before any OR, every OR before any
// read) and OR does not depend on the order of the lanes, so the mask is exact and the
// same on every run. Three LDS instructions instead of one ballot per bucket-id bit.
__device__ __forceinline__ uint64_t match_bucket_lds(int b, bool act, uint64_t* msk_w) {
    uint64_t m = 0;
    if (act) {
        msk_w[b] = 0;
        __hip_atomic_fetch_or(msk_w + b, 1ull << (threadIdx.x & 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        m = __hip_atomic_load(msk_w + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    return m;
}

constexpr int kPre = MOE_ROWIDS_PRE;  // batches of ids loaded ahead of their use
constexpr int kCountPre = MOE_ROWIDS_COUNT_PRE;

// load_raw only issues the loads, every lane of every batch (past the end a lane
// re-reads entry end-1; the caller guarantees bb < end), so that no value is merged
// with a default and nothing waits for them until their group is ranked; to_buckets
// turns them into buckets.
template <int NP>
__device__ __forceinline__ void load_raw(const int32_t* __restrict__ ids, int64_t bb, int64_t end,
                                         int32_t (&raw)[NP]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < NP; q++) raw[q] = ids[min(bb + q * 64 + lane, end - 1)];
}
template <int NP>
__device__ __forceinline__ void to_buckets(const int32_t (&raw)[NP], int64_t bb, int64_t end, int32_t E,
                                           int (&b)[NP]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < NP; q++) b[q] = bb + q * 64 + lane < end ? bucket_of(raw[q], E) : -1;
}
// Loads of batches [bb, bb + NP*64) as buckets: one per lane per batch, -1 past the end.
// Only batches that start before the end are loaded (a wave-uniform test, so a wave
// with an empty range loads nothing), and in the last one every lane loads (past the
// end it re-reads entry end-1), so all the loads are in flight before the first
// result is used; a load under a lane condition would be waited for inside its
// branch, one round trip per batch.
template <int NP>
__device__ __forceinline__ void load_batches(const int32_t* __restrict__ ids, int64_t bb,
                                             int64_t end, int32_t E, int (&b)[NP]) {
    const int lane = threadIdx.x & 63;
    int32_t raw[NP];
#pragma unroll
    for (int q = 0; q < NP; q++) raw[q] = bb + q * 64 < end ? ids[min(bb + q * 64 + lane, end - 1)] : 0;
    to_buckets(raw, bb, end, E, b);
}

// Histogram of the loaded batches starting at entry b0 (entries from `end` on are
// skipped) into this wave's counter row. No atomics: each bucket present in a batch
// has exactly one leader lane. Lanes of a bucket are found through this wave's LDS mask
// words when msk_w is given, otherwise with ballots.
__device__ __forceinline__ void count_batches(const int (&bk)[kPre], int64_t b0, int64_t end, int nbits,
                                              int32_t* cnt_w, uint64_t* msk_w) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPre; q++) {
        if (b0 + q * 64 >= end) break;  // uniform
        const bool act = bk[q] >= 0;
        const int b = act ? bk[q] : 0;
        const uint64_t m = msk_w ? match_bucket_lds(b, act, msk_w) : match_bucket(b, __ballot(act), nbits);
        if (act && lane == __ffsll((unsigned long long)m) - 1) cnt_w[b] += __popcll(m);
    }
}

// Places the loaded batches starting at entry b0: position = base[b] + running[b] +
// rank in batch.
__device__ __forceinline__ void place_batches(const RowIdsArgs& a, const int (&bk)[kPre], int64_t b0,
                                              int64_t end, int nbits, const int32_t* base, int32_t* run_w,
                                              uint64_t* msk_w) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPre; q++) {
        const int64_t bb = b0 + q * 64;
        if (bb >= end) break;  // uniform
        const int64_t i = bb + lane;
        const bool act = bk[q] >= 0;
        const int b = act ? bk[q] : 0;
        const uint64_t m = msk_w ? match_bucket_lds(b, act, msk_w) : match_bucket(b, __ballot(act), nbits);
        int32_t prev = 0;
        if (act) {
            prev = run_w[b];
            const int32_t pos = base[b] + prev + rank_below(m);
            const int32_t ii = (int32_t)i;  // n < 2^31 is a validated limit
            // src1 row t*B + s % B: ii itself when B = k, t when B = 1
            int32_t src = ii;
            if (a.B != a.k) {   // uniform
                const int32_t t = ii / a.k;
                src = a.B == 1 ? t : t * a.B + (ii - t * a.k) % a.B;
            }
            a.ids_src1[pos] = src;
            a.ids_dst[pos] = ii;
            if (a.inv) a.inv[i] = pos;
        }
        // every lane has read its counter before the group's leader bumps it
        __builtin_amdgcn_wave_barrier();
        if (act && lane == __ffsll((unsigned long long)m) - 1) run_w[b] = prev + __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

// In-place exclusive scan of v[0, n) (LDS) by all NT threads of the block; returns the
// total. wsum: LDS scratch of NT / 64 ints.
template <int NT = kThreads>
__device__ int32_t block_scan(int32_t* v, int n, int32_t* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (n + NT - 1) / NT;
    const int beg = min(tid * per, n), end = min(beg + per, n);
    int32_t s = 0;
    for (int i = beg; i < end; i++) s += v[i];
    int32_t x = s;
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int32_t pre = 0, total = 0;
    for (int j = 0; j < NT / 64; j++) {
        if (j < w) pre += wsum[j];
        total += wsum[j];
    }
    int32_t run = pre + x - s;
    for (int i = beg; i < end; i++) {
        const int32_t t = v[i];
        v[i] = run;
        run += t;
    }
    __syncthreads();
    return total;
}

// bstart[0..NB) holds bucket starts: write bounds and the M-tile prefixes (NT threads).
// tmp[0..E] holds tile table q's exclusive M-tile prefix: one entry per M tile, so the
// GEMM finds its tile with a single load (NT threads).
template <int NT = kThreads>
__device__ void write_tile_tab(const RowIdsArgs& a, int q, const int32_t* bstart, const int32_t* tmp) {
    for (int b = threadIdx.x; b < a.E; b += NT) {
        const int32_t lo = bstart[b], hi = bstart[b + 1];
        for (int32_t j = tmp[b]; j < tmp[b + 1] && j < a.tile_cap[q]; j++) {
            int32_t* t = a.tile_tab[q] + 4 * (int64_t)j;
            t[0] = b;
            t[1] = tmp[b];
            t[2] = lo;
            t[3] = hi - lo;
        }
    }
}

// M-tile prefix and tile table q from the bucket starts (NT threads, tmp: LDS scratch).
template <int NT = kThreads>
__device__ void write_tiles(const RowIdsArgs& a, int q, const int32_t* bstart, int32_t* tmp, int32_t* wsum) {
    const int E = a.E, NB = E + 1;
    const int tm = a.tile_m[q], tx = a.tile_x[q];
    for (int b = threadIdx.x; b < NB; b += NT)
        tmp[b] = b < E ? tiles_of(bstart[b + 1] - bstart[b], tm, tx) : 0;
    __syncthreads();
    block_scan<NT>(tmp, NB, wsum);
    for (int b = threadIdx.x; b < NB; b += NT) a.tile_off[q][b] = tmp[b];
    if (a.tile_tab[q]) write_tile_tab<NT>(a, q, bstart, tmp);
    __syncthreads();
}

template <int NT = kThreads>
__device__ void write_bounds_and_tiles(const RowIdsArgs& a, const int32_t* bstart, int32_t* tmp,
                                       int32_t* wsum) {
    for (int b = threadIdx.x; b < a.E + 1; b += NT) a.bounds[b] = bstart[b];
    for (int q = 0; q < 2; q++)
        if (a.tile_off[q]) write_tiles<NT>(a, q, bstart, tmp, wsum);  // uniform across the block
}

__device__ __forceinline__ int bucket_bits(int NB) { return 32 - __clz(NB - 1); }

// ---------------------------------------------------------------- one workgroup
// 16 waves (the most one workgroup holds), so each wave walks at most four batches:
// with 8 waves the two serial walks (count, place) of 6 batches each took 3.3 and
// 3.6 us of an 11.8 us pass on 3072 entries; with 16 waves and the ids kept in
// registers between the walks, the pass takes about 7 us.
constexpr int kSingleWaves = 16;
static_assert(kRowIdsOneBlockMax <= (int64_t)kSingleWaves * 64 * kPre,
              "the one-workgroup pass keeps each wave's ids in kPre registers");

// LDS of the one-workgroup pass: with MASK, per-wave group mask words [kSingleWaves][NB]
// (64-bit) first; then per-wave counters [kSingleWaves][NB], bucket starts [NB + 1] and
// tile counts [NB + 1].
size_t single_lds_bytes(int NB, bool mask) {
    return (mask ? (size_t)kSingleWaves * NB * sizeof(uint64_t) : 0) +
           ((size_t)kSingleWaves * NB + 2 * ((size_t)NB + 1)) * sizeof(int32_t);
}
// The mask words are used up to this many buckets (about 100 KB of LDS); beyond, the
// lanes of a bucket are found with one ballot per bit of the bucket id.
constexpr int kSingleMaskBuckets = 512;

template <bool MASK>
__global__ __launch_bounds__(kSingleWaves * 64) void k_row_ids_single(RowIdsArgs a) {
    constexpr int NW = kSingleWaves, NT = NW * 64;
    extern __shared__ __attribute__((aligned(16))) uint64_t lds_single[];
    __shared__ int32_t wsum[NW];
    const int NB = a.E + 1, nbits = bucket_bits(NB);
    uint64_t* msk_w = MASK ? lds_single + (threadIdx.x >> 6) * NB : nullptr;
    int32_t* cnt = (int32_t*)(lds_single + (MASK ? NW * NB : 0));
    int32_t* bstart = cnt + NW * NB;
    int32_t* tmp = bstart + NB + 1;
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < NW * NB; i += NT) cnt[i] = 0;
    __syncthreads();
    const int64_t per = ((a.n + NW * 64 - 1) / (NW * 64)) * 64;
    const int64_t beg = min((int64_t)w * per, a.n), end = min(beg + per, a.n);
    int bk[kPre];   // this wave's ids (per <= kPre batches), kept for the placement
    load_batches(a.ids, beg, end, a.E, bk);
    count_batches(bk, beg, end, nbits, cnt + w * NB, msk_w);
    __syncthreads();
    // per bucket, exclusive scan of the wave counters: 16 consecutive lanes hold one
    // bucket's counters (wave order) and scan them with shuffles
    for (int idx = threadIdx.x; idx < NB * NW; idx += NT) {
        const int b = idx / NW, v = idx - b * NW;
        const int32_t c = cnt[v * NB + b];
        int32_t x = c;
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            const int32_t y = __shfl_up(x, d, NW);
            if (v >= d) x += y;
        }
        cnt[v * NB + b] = x - c;
        if (v == NW - 1) bstart[b] = x;
    }
    __syncthreads();
    // wave 0 alone: exclusive scans of the bucket counts (into bucket starts and bounds)
    // and, for the first tile table, of the experts' M-tile counts, with shuffles and no
    // block barrier (two block-wide scans took about 2 us of the pass)
    const int tm0 = a.tile_off[0] ? a.tile_m[0] : 0, tx0 = a.tile_x[0];
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = (NB + 63) >> 6;
        const int b0 = min(lane * per, NB), b1 = min(b0 + per, NB);
        int32_t sc = 0, stl = 0;
        for (int b = b0; b < b1; b++) {
            const int32_t c = bstart[b];
            sc += c;
            if (tm0 && b < a.E) stl += tiles_of(c, tm0, tx0);
        }
        int32_t xc = sc, xt = stl;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t yc = __shfl_up(xc, d), yt = __shfl_up(xt, d);
            if (lane >= d) {
                xc += yc;
                xt += yt;
            }
        }
        int32_t rc = xc - sc, rt = xt - stl;
        for (int b = b0; b < b1; b++) {
            const int32_t c = bstart[b];
            bstart[b] = rc;
            a.bounds[b] = rc;
            rc += c;
            if (tm0) {
                tmp[b] = rt;
                a.tile_off[0][b] = rt;
                if (b < a.E) rt += tiles_of(c, tm0, tx0);
            }
        }
    }
    __syncthreads();
    if (tm0 && a.tile_tab[0]) write_tile_tab<NT>(a, 0, bstart, tmp);
    if (a.tile_off[1]) {   // a second tile table: the block-wide path (tmp is reused)
        __syncthreads();
        write_tiles<NT>(a, 1, bstart, tmp, wsum);
    }
    place_batches(a, bk, beg, end, nbits, bstart, cnt + w * NB, msk_w);
}

// ---------------------------------------------------------------- multi-block
// Counts one chunk and ranks its entries: each wave walks its range, and every entry
// gets its rank among the wave's earlier entries of the same bucket (stored as 16 bits:
// a wave's range is at most kMaxBatchesPerWave * 64 entries). The wave's counts go to
// wcnt (chunk-major) for the place pass, the chunk's totals to chunk_cnt (bucket-major)
// for the scan over chunks. Registers are held to 64 per lane so that four blocks (eight
// waves per SIMD) fit a CU: 1024 chunks then run in one round instead of one and a third.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_row_ids_count(RowIdsArgs a) {
    // LDS, sized for this launch: per wave, a group mask per bucket [kWaves][NB] and the
    // running count per bucket [kWaves][NB]
    extern __shared__ __attribute__((aligned(16))) uint64_t count_lds[];
    const int NB = a.E + 1;
    uint64_t* msk = count_lds;
    int32_t* cnt = (int32_t*)(count_lds + kWaves * NB);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < kWaves * NB; i += kThreads) cnt[i] = 0;
    __syncthreads();
    uint64_t* msk_w = msk + w * NB;
    const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
    const int64_t per = a.chunk / kWaves;
    const int64_t beg = min(c0 + w * per, a.n), end = min(beg + per, a.n);
    int32_t* run_w = cnt + w * NB;
    // Ranks one group of kCountPre batches starting at entry b0 (ids past the range are -1),
    // in three phases whose LDS instructions are issued back to back, batch after
    // batch, with one wait per phase (a wave's LDS instructions execute in order):
    //   masks: the lanes of batch q holding bucket b each clear b's mask word, then OR
    //     their own bit into it and read it back; batch q's read precedes batch q+1's
    //     clear. OR does not depend on the order of the lanes, so the mask is the same
    //     on every run;
    //   counts: the group's lowest lane adds the group size to the wave's counter of b
    //     and gets the counter's previous value; the batches' adds to one counter run in
    //     batch order, and within a batch every counter has one adder;
    //   ranks: each lane takes that previous value from its group's lowest lane.
    auto rank_group = [&](const int32_t (&raw)[kCountPre], int64_t b0) {
        int bk[kCountPre];
        to_buckets(raw, b0, end, a.E, bk);
        uint64_t m[kCountPre];
#pragma unroll
        for (int q = 0; q < kCountPre; q++) {
            m[q] = 0;
            if (bk[q] >= 0) {
                msk_w[bk[q]] = 0;
                __hip_atomic_fetch_or(msk_w + bk[q], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                m[q] = __hip_atomic_load(msk_w + bk[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        int32_t prev[kCountPre];
#pragma unroll
        for (int q = 0; q < kCountPre; q++) {
            prev[q] = 0;
            if (bk[q] >= 0 && rank_below(m[q]) == 0)
                prev[q] = __hip_atomic_fetch_add(run_w + bk[q], __popcll(m[q]), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        int32_t base[kCountPre];
#pragma unroll
        for (int q = 0; q < kCountPre; q++)
            base[q] = __shfl(prev[q], bk[q] >= 0 ? __ffsll((unsigned long long)m[q]) - 1 : lane);
#pragma unroll
        for (int q = 0; q < kCountPre; q++)
            if (bk[q] >= 0) a.rank16[b0 + q * 64 + lane] = (uint16_t)(base[q] + rank_below(m[q]));
    };
    // two groups of batches in registers: the next group's ids load while this one is
    // ranked (they are turned into buckets only when their group is ranked). The loads
    // are issued without a condition (a group past the end re-reads entry end-1): a
    // path that skipped them would make the compiler wait for every load in flight
    // where the paths join.
    constexpr int64_t G = kCountPre * 64;
    if (beg < end) {   // uniform
        int32_t r0[kCountPre], r1[kCountPre];
        load_raw(a.ids, beg, end, r0);
        for (int64_t b0 = beg; b0 < end; b0 += 2 * G) {
            load_raw(a.ids, b0 + G, end, r1);
            rank_group(r0, b0);
            if (b0 + G >= end) break;
            load_raw(a.ids, b0 + 2 * G, end, r0);
            rank_group(r1, b0 + G);
        }
    }
    __syncthreads();
    int32_t* wc = a.wcnt + (int64_t)blockIdx.x * kWaves * NB;
    for (int i = threadIdx.x; i < kWaves * NB; i += kThreads) wc[i] = cnt[i];
    for (int b = threadIdx.x; b < NB; b += kThreads) {
        int32_t s = 0;
        for (int v = 0; v < kWaves; v++) s += cnt[v * NB + b];
        a.chunk_cnt[(int64_t)b * a.n_chunks + blockIdx.x] = s;
    }
}

// One block per bucket: exclusive scan of that bucket's per-chunk counts.
__global__ __launch_bounds__(kThreads) void k_row_ids_scan_chunks(RowIdsArgs a) {
    __shared__ int32_t wsum[kWaves];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t nc = a.n_chunks;
    const int64_t per = (nc + kThreads - 1) / kThreads;
    const int64_t beg = min((int64_t)tid * per, nc), end = min(beg + per, nc);
    int32_t* col = a.chunk_cnt + (int64_t)b * nc;   // this bucket's counts, chunk order
    int32_t s = 0;
    for (int64_t c = beg; c < end; c++) s += col[c];
    int32_t x = s;
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int32_t pre = 0, total = 0;
    for (int j = 0; j < kWaves; j++) {
        if (j < w) pre += wsum[j];
        total += wsum[j];
    }
    int32_t run = pre + x - s;
    for (int64_t c = beg; c < end; c++) {
        const int32_t t = col[c];
        col[c] = run;
        run += t;
    }
    if (tid == 0) a.bucket_tot[b] = total;
}

// Places one chunk from the count pass's ranks. The chunk's entries are first put in
// bucket order in LDS (position inside the chunk: the bucket's start in the chunk + the
// wave's offset + the entry's rank), then every bucket's run is written out
// contiguously: consecutive output positions come from consecutive threads, instead of
// each entry storing to a scattered position of its own.
// Every block turns the bucket totals into bucket starts itself (a block scan over
// E + 1 values), and block 0 also writes the bounds and tile tables, so no launch sits
// between the scan over chunks and this one. LOCAL: few chunks (kLocalScanChunks at
// most): each block also sums the per-chunk counts itself -- its bucket's prefix over
// the earlier chunks and the bucket totals -- so the scan over chunks is skipped too.
// Otherwise both come from the scan over chunks.
constexpr int64_t kLocalScanChunks = 128;

template <bool LOCAL>
__global__ __launch_bounds__(kThreads) void k_row_ids_place(RowIdsArgs a) {
    __shared__ int32_t wsum[kWaves];
    // LDS, sized for this launch: per-wave offsets [kWaves][NB], bucket starts inside the
    // chunk [NB + 1], global start of each bucket's run [NB] (then output position minus
    // position in the chunk), and the chunk in bucket order: bucket << 16 | index in the
    // chunk [chunk], the bucket starts [NB + 1] and a tile-count scratch [NB + 1]
    extern __shared__ __attribute__((aligned(16))) int32_t lds[];
    const int NB = a.E + 1;
    int32_t* woff = lds;
    int32_t* cstart = woff + kWaves * NB;
    int32_t* gbase = cstart + NB + 1;
    uint32_t* st = (uint32_t*)(gbase + NB);
    int32_t* bstart = (int32_t*)(st + a.chunk);
    int32_t* tmp = bstart + NB + 1;
    const int tid = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
    const int64_t per = a.chunk / kWaves;
    const int32_t* wc = a.wcnt + (int64_t)blockIdx.x * kWaves * NB;
    for (int b = tid; b < NB; b += kThreads) {
        int32_t run = 0;
        for (int v = 0; v < kWaves; v++) {
            const int32_t t = wc[v * NB + b];
            woff[v * NB + b] = run;
            run += t;
        }
        cstart[b] = run;
        if constexpr (LOCAL) {
            const int32_t* row = a.chunk_cnt + (int64_t)b * a.n_chunks;   // this bucket, chunk order
            int32_t pre = 0, tot = 0;
            const int nc = (int)a.n_chunks;
#pragma unroll 8
            for (int c = 0; c < nc; c++) {   // independent loads, kept in flight together
                const int32_t t = row[c];
                pre += c < (int)blockIdx.x ? t : 0;
                tot += t;
            }
            gbase[b] = pre;
            bstart[b] = tot;
        } else {   // from the scan over chunks: this chunk's prefix, the bucket total
            gbase[b] = a.chunk_cnt[(int64_t)b * a.n_chunks + blockIdx.x];
            bstart[b] = a.bucket_tot[b];
        }
    }
    __syncthreads();
    block_scan(bstart, NB, wsum);   // bucket totals -> bucket starts
    for (int b = tid; b < NB; b += kThreads) gbase[b] += bstart[b];
    if (blockIdx.x == 0) {   // block-uniform
        bstart[NB] = a.n;     // (bounds past the valid buckets are never read)
        write_bounds_and_tiles(a, bstart, tmp, wsum);
    }
    __syncthreads();
    const int32_t chunk_n = block_scan(cstart, NB, wsum);
    // gbase becomes the offset from a position in the chunk to its output position
    for (int b = tid; b < NB; b += kThreads) gbase[b] -= cstart[b];
    // Each wave puts the range the count pass ranked with it (so its offsets are one row
    // of woff) in bucket order, kPre batches of ids and ranks loaded together: unclamped
    // per-lane loads would be waited for one batch at a time.
    {
        const int w = tid >> 6, lane = tid & 63;
        const int32_t cn = (int32_t)min(a.chunk, a.n - c0);   // chunk-relative, < 2^16
        const int32_t wbeg = min(w * (int32_t)per, cn), wend = min(wbeg + (int32_t)per, cn);
        const int32_t* idc = a.ids + c0;
        const uint16_t* rkc = a.rank16 + c0;
        const int32_t* wo = woff + w * NB;
        for (int32_t e0 = wbeg; e0 < wend; e0 += kPre * 64) {
            int32_t id[kPre];
            uint32_t rk[kPre];
#pragma unroll
            for (int q = 0; q < kPre; q++) {
                id[q] = 0;
                rk[q] = 0;
                if (e0 + q * 64 < wend) {   // uniform; past the end a lane re-reads entry wend-1
                    const int32_t e = min(e0 + q * 64 + lane, wend - 1);
                    id[q] = idc[e];
                    rk[q] = rkc[e];
                }
            }
#pragma unroll
            for (int q = 0; q < kPre; q++) {
                const int32_t e = e0 + q * 64 + lane;
                if (e < wend) {
                    const int b = bucket_of(id[q], a.E);
                    st[cstart[b] + wo[b] + (int32_t)rk[q]] = ((uint32_t)b << 16) | (uint32_t)e;
                }
            }
        }
    }
    __syncthreads();
    for (int32_t p = tid; p < chunk_n; p += kThreads) {
        const uint32_t v = st[p];
        const int b = (int)(v >> 16);
        const int32_t g = gbase[b] + p;
        const uint32_t ii = (uint32_t)(c0 + (v & 0xffffu));   // n < 2^31 is a validated limit
        const uint32_t t = (uint32_t)(((uint64_t)ii * a.k_magic) >> a.k_shift);   // ii / k
        // src1 row t*B + s % B: ii itself when B = k, t when B = 1 (no division)
        uint32_t src;
        if (a.B == a.k) src = ii;         // block-uniform
        else if (a.B == 1) src = t;
        else src = t * a.B + (ii - t * (uint32_t)a.k) % a.B;
        a.ids_src1[g] = (int32_t)src;
        a.ids_dst[g] = (int32_t)ii;
        if (a.inv) a.inv[ii] = g;
    }
}

}  // namespace

namespace {
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
}  // namespace

// Multi-block scratch, in this order: chunk_cnt [NB][n_chunks], bucket_tot [NB],
// wcnt [n_chunks][kWaves][NB], rank16 [n].
size_t row_ids_scratch_bytes(int64_t n, int32_t E) {
    if (n <= kRowIdsOneBlockMax) return 0;
    const int64_t ch = chunk_len(n);
    const int64_t nc = (n + ch - 1) / ch;
    const size_t NB = (size_t)E + 1;
    return align_up((size_t)nc * NB * 4) + align_up(NB * 4) + align_up((size_t)nc * kWaves * NB * 4) +
           align_up((size_t)n * 2);
}

void row_ids_carve_scratch(RowIdsArgs& a, void* scratch) {
    const int64_t ch = chunk_len(a.n);
    const int64_t nc = (a.n + ch - 1) / ch;
    const size_t NB = (size_t)a.E + 1;
    char* p = (char*)scratch;
    a.chunk_cnt = (int32_t*)p;
    p += align_up((size_t)nc * NB * 4);
    a.bucket_tot = (int32_t*)p;
    p += align_up(NB * 4);
    a.wcnt = (int32_t*)p;
    p += align_up((size_t)nc * kWaves * NB * 4);
    a.rank16 = (uint16_t*)p;
}

hipError_t launch_row_ids(const RowIdsArgs& a0, hipStream_t st, int* n_launches) {
    RowIdsArgs a = a0;
    if (a.n <= kRowIdsOneBlockMax) {
        static PerDeviceOnce lds_cap_mask, lds_cap_ballot;   // dynamic LDS caps, once per device
        if (a.E + 1 <= kSingleMaskBuckets) {
            if (const hipError_t e = set_lds_cap(lds_cap_mask, (const void*)k_row_ids_single<true>,
                                                 (int)single_lds_bytes(kSingleMaskBuckets, true)))
                return e;
            k_row_ids_single<true><<<1, kSingleWaves * 64, single_lds_bytes(a.E + 1, true), st>>>(a);
        } else {
            if (const hipError_t e = set_lds_cap(lds_cap_ballot, (const void*)k_row_ids_single<false>,
                                                 (int)single_lds_bytes(kMaxBuckets, false)))
                return e;
            k_row_ids_single<false><<<1, kSingleWaves * 64, single_lds_bytes(a.E + 1, false), st>>>(a);
        }
        if (n_launches) *n_launches = 1;
        return hipGetLastError();
    }
    a.chunk = chunk_len(a.n);
    a.n_chunks = (a.n + a.chunk - 1) / a.chunk;
    const size_t count_lds = (size_t)kWaves * (a.E + 1) * (sizeof(uint64_t) + sizeof(int32_t));
    {
        static PerDeviceOnce cap;   // the count kernel's dynamic LDS cap, once per device
        if (const hipError_t e = set_lds_cap(cap, (const void*)k_row_ids_count,
                                             kWaves * kMaxBuckets * (int)(sizeof(uint64_t) + sizeof(int32_t))))
            return e;
    }
    // ii / k as a multiply-high: M = floor(2^(31 + l) / k) + 1 with l = ceil(log2 k) is
    // exact for every ii < 2^31
    {
        int l = 0;
        while ((1 << l) < a.k) l++;
        a.k_magic = (uint32_t)(((uint64_t)1 << (31 + l)) / (uint64_t)a.k + 1);
        a.k_shift = 31 + l;
    }
    // the place kernel's LDS: wave offsets and starts for NB buckets, then the chunk in
    // bucket order (one word per entry)
    const int64_t NB = a.E + 1;
    const size_t stage = (size_t)(kWaves * NB + 4 * NB + 3) * 4 + (size_t)a.chunk * 4;
    constexpr int kCap = (int)((kWaves * kMaxBuckets + 4 * kMaxBuckets + 3) * 4 + kMaxChunk * 4);
    if (a.n_chunks <= kLocalScanChunks) {
        static PerDeviceOnce lds_cap;
        if (const hipError_t e = set_lds_cap(lds_cap, (const void*)k_row_ids_place<true>, kCap)) return e;
        k_row_ids_count<<<(unsigned)a.n_chunks, kThreads, count_lds, st>>>(a);
        k_row_ids_place<true><<<(unsigned)a.n_chunks, kThreads, stage, st>>>(a);
        if (n_launches) *n_launches = 2;
        return hipGetLastError();
    }
    static PerDeviceOnce lds_cap;
    if (const hipError_t e = set_lds_cap(lds_cap, (const void*)k_row_ids_place<false>, kCap)) return e;
    k_row_ids_count<<<(unsigned)a.n_chunks, kThreads, count_lds, st>>>(a);
    k_row_ids_scan_chunks<<<(unsigned)(a.E + 1), kThreads, 0, st>>>(a);
    k_row_ids_place<false><<<(unsigned)a.n_chunks, kThreads, stage, st>>>(a);
    if (n_launches) *n_launches = 3;
    return hipGetLastError();
}

}  // namespace moe
