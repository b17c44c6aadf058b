// Row-id pass (K1): the three maps of the deterministic MoE path -- src1 rows
// reordered so every expert's rows are contiguous (ids_src1), the same order for
// dst (ids_dst) and each expert's bounds (expert_bounds) -- built without any
// atomic slot counter ("CUDA: better MoE implementation", sections 2 and 2.1: the
// old gather claimed destination slots with an atomic increment, which was slow
// and made the row order, hence the float summation order, change run to run).
//
// gfx950 design: a stable counting sort built from wavefront primitives.
//   * Each wave owns a contiguous range of entries (t*k + s order) and walks it 64
//     at a time. Lanes holding the same bucket find each other with one ballot per
//     bit of the bucket id; the group's lowest lane adds the group size to the
//     wave's LDS counter (one writer per counter, so no atomics), and a lane's rank
//     inside its group is a masked bit count (mbcnt).
//   * Per-bucket exclusive scans over waves (and, for large inputs, over
//     workgroups), then over buckets, give every (wave, bucket) its first output
//     position; a second walk over the same range places every entry. Entries keep
//     their (t, s) order inside a bucket, so the result is unique.
//   * Bucket E collects ids outside [0, E): they land after all expert segments.
//   * Inputs up to kRowIdsOneBlockMax entries run as one 1024-thread workgroup (one
//     launch); larger ones use count / scan-over-chunks / scan-over-buckets / place.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxBatchesPerWave = 16;
constexpr int64_t kMaxChunk = (int64_t)kThreads * kMaxBatchesPerWave;   // 8192 entries

// Entries per chunk of the multi-block pass: about 2048 chunks, each wave walking 2 to
// 16 batches of 64 (long enough walks keep the id loads ahead of their use, and few
// chunks keep the per-chunk counts small).
int64_t chunk_len(int64_t n) {
    int64_t bpw = (n + 2048 * (int64_t)kThreads - 1) / (2048 * (int64_t)kThreads);
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

constexpr int kPre = 8;  // batches of ids loaded ahead of their use

// Loads of batches [bb, bb + kPre*64): one id per lane per batch, bucket E past the end.
__device__ __forceinline__ void load_batches(const int32_t* __restrict__ ids, int64_t bb,
                                             int64_t end, int32_t E, int (&b)[kPre]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPre; q++) {
        const int64_t i = bb + q * 64 + lane;
        b[q] = i < end ? bucket_of(ids[i], E) : -1;
    }
}

// Histogram of the loaded batches starting at entry b0 (entries from `end` on are
// skipped) into this wave's counter row. No atomics: each bucket present in a batch
// has exactly one leader lane.
__device__ __forceinline__ void count_batches(const int (&bk)[kPre], int64_t b0, int64_t end, int nbits,
                                              int32_t* cnt_w) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPre; q++) {
        if (b0 + q * 64 >= end) break;  // uniform
        const bool act = bk[q] >= 0;
        const int b = act ? bk[q] : 0;
        const uint64_t m = match_bucket(b, __ballot(act), nbits);
        if (act && lane == __ffsll((unsigned long long)m) - 1) cnt_w[b] += __popcll(m);
    }
}

// Places the loaded batches starting at entry b0: position = base[b] + running[b] +
// rank in batch.
__device__ __forceinline__ void place_batches(const RowIdsArgs& a, const int (&bk)[kPre], int64_t b0,
                                              int64_t end, int nbits, const int32_t* base, int32_t* run_w) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPre; q++) {
        const int64_t bb = b0 + q * 64;
        if (bb >= end) break;  // uniform
        const int64_t i = bb + lane;
        const bool act = bk[q] >= 0;
        const int b = act ? bk[q] : 0;
        const uint64_t m = match_bucket(b, __ballot(act), nbits);
        int32_t prev = 0;
        if (act) {
            prev = run_w[b];
            const int32_t pos = base[b] + prev + rank_below(m);
            const int32_t ii = (int32_t)i;  // n < 2^31 is a validated limit
            const int32_t t = ii / a.k;
            const int32_t s = ii - t * a.k;
            a.ids_src1[pos] = t * a.B + s % a.B;
            a.ids_dst[pos] = ii;
            if (a.inv) a.inv[i] = pos;
        }
        // every lane has read its counter before the group's leader bumps it
        __builtin_amdgcn_wave_barrier();
        if (act && lane == __ffsll((unsigned long long)m) - 1) run_w[b] = prev + __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

// Histogram of entries [beg, end) into this wave's counter row.
__device__ void wave_count(const int32_t* __restrict__ ids, int64_t beg, int64_t end, int32_t E,
                           int nbits, int32_t* cnt_w) {
    for (int64_t b0 = beg; b0 < end; b0 += kPre * 64) {
        int bk[kPre];
        load_batches(ids, b0, end, E, bk);
        count_batches(bk, b0, end, nbits, cnt_w);
    }
}

// Places entries [beg, end).
__device__ void wave_place(const RowIdsArgs& a, int64_t beg, int64_t end, int nbits,
                           const int32_t* base, int32_t* run_w) {
    for (int64_t b0 = beg; b0 < end; b0 += kPre * 64) {
        int bk[kPre];
        load_batches(a.ids, b0, end, a.E, bk);
        place_batches(a, bk, b0, end, nbits, base, run_w);
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
    const int tm = a.tile_m[q];
    for (int b = threadIdx.x; b < NB; b += NT)
        tmp[b] = b < E ? (bstart[b + 1] - bstart[b] + tm - 1) / tm : 0;
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

// LDS of the one-workgroup pass: per-wave counters [kSingleWaves][NB], then bucket
// starts [NB + 1] and tile counts [NB + 1].
size_t single_lds_bytes(int NB) { return ((size_t)kSingleWaves * NB + 2 * ((size_t)NB + 1)) * sizeof(int32_t); }

__global__ __launch_bounds__(kSingleWaves * 64) void k_row_ids_single(RowIdsArgs a) {
    constexpr int NW = kSingleWaves, NT = NW * 64;
    extern __shared__ __attribute__((aligned(16))) int32_t lds_single[];
    __shared__ int32_t wsum[NW];
    const int NB = a.E + 1, nbits = bucket_bits(NB);
    int32_t* cnt = lds_single;
    int32_t* bstart = cnt + NW * NB;
    int32_t* tmp = bstart + NB + 1;
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < NW * NB; i += NT) cnt[i] = 0;
    __syncthreads();
    const int64_t per = ((a.n + NW * 64 - 1) / (NW * 64)) * 64;
    const int64_t beg = min((int64_t)w * per, a.n), end = min(beg + per, a.n);
    int bk[kPre];   // this wave's ids (per <= kPre batches), kept for the placement
    load_batches(a.ids, beg, end, a.E, bk);
    count_batches(bk, beg, end, nbits, cnt + w * NB);
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
    const int tm0 = a.tile_off[0] ? a.tile_m[0] : 0;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = (NB + 63) >> 6;
        const int b0 = min(lane * per, NB), b1 = min(b0 + per, NB);
        int32_t sc = 0, stl = 0;
        for (int b = b0; b < b1; b++) {
            const int32_t c = bstart[b];
            sc += c;
            if (tm0 && b < a.E) stl += (c + tm0 - 1) / tm0;
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
                if (b < a.E) rt += (c + tm0 - 1) / tm0;
            }
        }
    }
    __syncthreads();
    if (tm0 && a.tile_tab[0]) write_tile_tab<NT>(a, 0, bstart, tmp);
    if (a.tile_off[1]) {   // a second tile table: the block-wide path (tmp is reused)
        __syncthreads();
        write_tiles<NT>(a, 1, bstart, tmp, wsum);
    }
    place_batches(a, bk, beg, end, nbits, bstart, cnt + w * NB);
}

// ---------------------------------------------------------------- multi-block
__global__ __launch_bounds__(kThreads) void k_row_ids_count(RowIdsArgs a) {
    __shared__ int32_t cnt[kWaves * kMaxBuckets];
    const int NB = a.E + 1, nbits = bucket_bits(NB);
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kWaves * NB; i += kThreads) cnt[i] = 0;
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
    const int64_t per = a.chunk / kWaves;
    const int64_t beg = min(c0 + w * per, a.n), end = min(beg + per, a.n);
    wave_count(a.ids, beg, end, a.E, nbits, cnt + w * NB);
    __syncthreads();
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

// Single block: bucket starts, bounds, tile prefixes; bucket_tot becomes the starts.
__global__ __launch_bounds__(kThreads) void k_row_ids_scan_buckets(RowIdsArgs a) {
    __shared__ int32_t bstart[kMaxBuckets + 1];
    __shared__ int32_t tmp[kMaxBuckets + 1];
    __shared__ int32_t wsum[kWaves];
    const int NB = a.E + 1;
    for (int b = threadIdx.x; b < NB; b += kThreads) bstart[b] = a.bucket_tot[b];
    __syncthreads();
    block_scan(bstart, NB, wsum);
    write_bounds_and_tiles(a, bstart, tmp, wsum);
    for (int b = threadIdx.x; b < NB; b += kThreads) a.bucket_tot[b] = bstart[b];
}

// Places one chunk. The chunk's entries are first put in bucket order in LDS (their
// position inside the chunk: the bucket's start in the chunk + the wave's offset +
// the running count + the rank in the batch), then every bucket's run is written out
// contiguously: consecutive output positions come from consecutive threads, instead of
// each entry storing to a scattered position of its own.
__global__ __launch_bounds__(kThreads) void k_row_ids_place(RowIdsArgs a) {
    __shared__ int32_t wsum[kWaves];
    // LDS, sized for this launch: per-wave offsets (then running counts) [kWaves][NB],
    // bucket starts inside the chunk [NB + 1], global start of each bucket's run [NB],
    // and the chunk in bucket order: entry index [chunk], bucket [chunk]
    extern __shared__ __attribute__((aligned(16))) int32_t lds[];
    const int NB = a.E + 1, nbits = bucket_bits(NB);
    int32_t* cnt = lds;
    int32_t* cstart = cnt + kWaves * NB;
    int32_t* gbase = cstart + NB + 1;
    int32_t* st_i = gbase + NB;
    uint16_t* st_bk = (uint16_t*)(st_i + a.chunk);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kWaves * NB; i += kThreads) cnt[i] = 0;
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
    const int64_t per = a.chunk / kWaves;
    const int64_t beg = min(c0 + w * per, a.n), end = min(beg + per, a.n);
    wave_count(a.ids, beg, end, a.E, nbits, cnt + w * NB);
    __syncthreads();
    for (int b = tid; b < NB; b += kThreads) {
        int32_t run = 0;
        for (int v = 0; v < kWaves; v++) {
            const int32_t t = cnt[v * NB + b];
            cnt[v * NB + b] = run;
            run += t;
        }
        cstart[b] = run;
    }
    __syncthreads();
    const int32_t chunk_n = block_scan(cstart, NB, wsum);
    for (int b = tid; b < NB; b += kThreads)
        gbase[b] = a.bucket_tot[b] + a.chunk_cnt[(int64_t)b * a.n_chunks + blockIdx.x];
    __syncthreads();
    int32_t* run_w = cnt + w * NB;
    for (int64_t b0 = beg; b0 < end; b0 += kPre * 64) {
        int bk[kPre];
        load_batches(a.ids, b0, end, a.E, bk);
#pragma unroll
        for (int q = 0; q < kPre; q++) {
            const int64_t bb = b0 + q * 64;
            if (bb >= end) break;  // uniform
            const int64_t i = bb + lane;
            const bool act = bk[q] >= 0;
            const int b = act ? bk[q] : 0;
            const uint64_t m = match_bucket(b, __ballot(act), nbits);
            int32_t prev = 0;
            if (act) {
                prev = run_w[b];
                const int32_t lp = cstart[b] + prev + rank_below(m);   // position in the chunk
                st_i[lp] = (int32_t)i;  // n < 2^31 is a validated limit
                st_bk[lp] = (uint16_t)b;
                if (a.inv) a.inv[i] = gbase[b] + lp - cstart[b];
            }
            // every lane has read its counter before the group's leader bumps it
            __builtin_amdgcn_wave_barrier();
            if (act && lane == __ffsll((unsigned long long)m) - 1) run_w[b] = prev + __popcll(m);
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    for (int32_t p = tid; p < chunk_n; p += kThreads) {
        const int b = st_bk[p];
        const int32_t g = gbase[b] + p - cstart[b];
        const int32_t ii = st_i[p];
        const int32_t t = ii / a.k;
        const int32_t s = ii - t * a.k;
        a.ids_src1[g] = t * a.B + s % a.B;
        a.ids_dst[g] = ii;
    }
}

}  // namespace

size_t row_ids_scratch_bytes(int64_t n, int32_t E) {
    if (n <= kRowIdsOneBlockMax) return 0;
    const int64_t ch = chunk_len(n);
    const int64_t nc = (n + ch - 1) / ch;
    const size_t a = (size_t)nc * (size_t)(E + 1) * sizeof(int32_t);
    return ((a + kAlign - 1) / kAlign) * kAlign + (size_t)(E + 1) * sizeof(int32_t);
}

hipError_t launch_row_ids(const RowIdsArgs& a0, hipStream_t st, int* n_launches) {
    RowIdsArgs a = a0;
    if (a.n <= kRowIdsOneBlockMax) {
        static bool attr_set = false;   // raise the dynamic LDS cap once per process
        if (!attr_set) {
            const hipError_t e = hipFuncSetAttribute((const void*)k_row_ids_single,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)single_lds_bytes(kMaxBuckets));
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        k_row_ids_single<<<1, kSingleWaves * 64, single_lds_bytes(a.E + 1), st>>>(a);
        if (n_launches) *n_launches = 1;
        return hipGetLastError();
    }
    a.chunk = chunk_len(a.n);
    a.n_chunks = (a.n + a.chunk - 1) / a.chunk;
    // the place kernel's LDS: counters and starts for NB buckets, then the chunk in
    // bucket order (an int and a short per entry)
    const int64_t NB = a.E + 1;
    const size_t stage = (size_t)(kWaves * NB + 2 * NB + 1) * 4 + (size_t)a.chunk * 6;
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(
            (const void*)k_row_ids_place, hipFuncAttributeMaxDynamicSharedMemorySize,
            (int)((kWaves * kMaxBuckets + 2 * kMaxBuckets + 1) * 4 + kMaxChunk * 6));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    k_row_ids_count<<<(unsigned)a.n_chunks, kThreads, 0, st>>>(a);
    k_row_ids_scan_chunks<<<(unsigned)(a.E + 1), kThreads, 0, st>>>(a);
    k_row_ids_scan_buckets<<<1, kThreads, 0, st>>>(a);
    k_row_ids_place<<<(unsigned)a.n_chunks, kThreads, stage, st>>>(a);
    if (n_launches) *n_launches = 4;
    return hipGetLastError();
}

}  // namespace moe
