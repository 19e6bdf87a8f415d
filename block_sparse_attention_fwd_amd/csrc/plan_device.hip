// Device-side planning of BLOCK masks: the mask-to-tile mapping and the task
// organisation of the host planner, run as HIP kernels on a mask that is
// already in device memory (Tessera, arXiv 2609.25869, abstract: logical
// masks mapped to physical tiles and tasks, with preparation kept cheap; a
// dynamic mask produced on the GPU then needs no host round trip).
//
// The kernels produce the host planner's plan, record for record: per task
// (batch, head, query tile) the ordered key-tile records {k0, FULL/PARTIAL |
// sub-block keep bits}, and the task array in the same launch order (longest
// first, or longest first grouped for the XCDs: runs of one cost class split
// into X segments of neighbouring query tiles and interleaved). Only where
// the records sit differs: task t's records start at t * nkt (its worst
// case), so no pass over all tasks is needed before they are written.
//
//   map_tasks     one wave per task: records of the non-empty key tiles,
//                 compacted in key order; tile counts
//   slice_map     (SLICE masks, in place of map_tasks) one wave per list:
//                 gather records and the plan's copy of the keys
//   chunk_counts  one workgroup per chunk of tasks: tasks per sort key
//                 (cost class, highest first; tasks without tiles last)
//   scan_keys     one workgroup: exclusive prefix over (key, chunk), totals
//   place_tasks   one workgroup per chunk: stable rank of each task in its
//                 class -> launch slot (XCD interleave) -> task array
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_device.hpp"

namespace bsa {

namespace {

constexpr int kWave = 64;
constexpr int kChunk = kDevPlanChunk;
constexpr int kChunkWaves = kChunk / kWave;

// The host planner's rule for the sub-block keep bits of a (query tile, key
// tile) pair: every kept logical block sets the bit of the tile sub-block that
// holds its first query row and key column; the pair is FULL when every valid
// sub-block is kept and the key tile is whole. Block sides are powers of two
// and a query tile starts on a block boundary (or lies inside one block), so
// logical query block qb0 + j is sub-row j and, for bk <= 64, key block
// kb0 + i is sub-column i: NQ = BQ / min(bq, BQ) rows and NK = 64 / min(bk, 64)
// columns. Each lane loads its tile's NQ x NK mask entries for R key tiles at
// once (independent loads), then forms the bits.
template <int NQ, int NK, bool BITS, int R>
__device__ __forceinline__ void tile_bits(const DevPlanArgs &a, int64_t row0, int nq, int nsq_valid, int64_t tk0,
                                          int32_t L, uint32_t (&bits)[R], bool (&full)[R])
{
    uint32_t v[R][NQ];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t tk = tk0 + (int64_t)r * kWave;
        const int32_t k0 = (int32_t)(tk * kTileK);
        const int64_t kb0 = (int64_t)k0 >> a.lbk;
        const int64_t kb_last = (int64_t)(min(k0 + kTileK, L) - 1) >> a.lbk;
        const bool in = tk < a.nkt;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            uint32_t x = 0;
            if (in && j < nq) {
                const int64_t row = row0 + j;
                if (BITS) {
                    const uint64_t w = a.bits[row * a.words + (kb0 >> 6)];
                    x = (uint32_t)(w >> (kb0 & 63)) & ((1u << NK) - 1);
                    if (NK > 1) x &= (2u << (kb_last - kb0 < NK - 1 ? kb_last - kb0 : NK - 1)) - 1;
                } else {
                    const uint8_t *p = a.u8 + row * a.nkb + kb0;
#pragma unroll
                    for (int i = 0; i < NK; ++i)
                        if (kb0 + i <= kb_last) x |= (uint32_t)(p[i] != 0) << i;
                }
            }
            v[r][j] = x;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t tk = tk0 + (int64_t)r * kWave;
        const int32_t k0 = (int32_t)(tk * kTileK), k1 = min(k0 + kTileK, L);
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < NQ; ++j) acc |= v[r][j] << (j * NK);
        const int nsk_valid = min(NK, ((k1 - 1 - k0) >> a.lbke) + 1);
        const uint32_t row_want = (1u << nsk_valid) - 1;
        uint32_t want = 0;
#pragma unroll
        for (int j = 0; j < NQ; ++j)
            if (j < nsq_valid) want |= row_want << (j * NK);
        bits[r] = acc;
        full[r] = (acc & want) == want && k0 + kTileK <= L;
    }
}

__device__ __forceinline__ int key_of(const DevPlanArgs &a, int32_t cnt)
{
    const int c = a.cls_of[cnt];
    return c < 0 ? a.nclass : a.nclass - 1 - c;
}

// Exclusive prefix of v over the workgroup; *total gets the sum.
template <int NT>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t *red, int64_t *total)
{
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int64_t x = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const int64_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == kWave - 1) red[w] = x;
    __syncthreads();
    int64_t before = 0, all = 0;
    for (int i = 0; i < NT / kWave; ++i) {
        if (i < w) before += red[i];
        all += red[i];
    }
    *total = all;
    return before + x - v;
}

template <int NQ, int NK, bool BITS>
__global__ __launch_bounds__(kWave) void map_tasks(DevPlanArgs a)
{
    constexpr int R = 2;  // key tiles per lane and round
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.x, bh = t / a.nqt, tq = t % a.nqt;
    const int32_t L = (int32_t)a.L;
    const int32_t q0 = (int32_t)tq * a.BQ, q1 = min(q0 + a.BQ, L);
    const int64_t qb0 = (int64_t)q0 >> a.lbq;
    const int nq = (int)(((int64_t)(q1 - 1) >> a.lbq) - qb0 + 1);
    const int nsq_valid = min(NQ, ((q1 - 1 - q0) >> a.lbqe) + 1);
    const int64_t row0 = bh * a.nqb + qb0;
    TileRec *out = a.tiles + t * a.nkt;
    const uint64_t below = (1ull << lane) - 1;
    int c = 0, f = 0;
    for (int64_t start = 0; start < a.nkt; start += R * kWave) {
        uint32_t bits[R];
        bool full[R];
        tile_bits<NQ, NK, BITS, R>(a, row0, nq, nsq_valid, start + lane, L, bits, full);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint64_t kept = __ballot(bits[r] != 0), whole = __ballot(bits[r] != 0 && full[r]);
            if (bits[r]) {
                const int64_t tk = start + r * kWave + lane;
                out[c + __popcll(kept & below)] = TileRec{(int32_t)(tk * kTileK), bits[r] | (full[r] ? 0u : kPartial)};
            }
            c += __popcll(kept);
            f += __popcll(whole);
        }
    }
    if (lane == 0) {
        a.cnt[t] = c;
        a.full[t] = f;
    }
}

// SLICE masks (FG-Attn, arXiv 2509.16518, abstract: M x 1 slices whose keys
// are gathered into packed tiles): one wave per list. The list's keys become
// gather records of kTileK keys (the last one short and PARTIAL), and are
// copied into the plan clamped into [0, L), counting entries that are out of
// range or not increasing; a list whose bounds fall outside [0, nnz] or span
// more than L keys is taken as empty and counted once.
__global__ __launch_bounds__(kWave) void slice_map(DevPlanArgs a)
{
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.x;
    int64_t s = a.row_ptr[t], e = a.row_ptr[t + 1];
    int err = 0;
    if (s < 0 || e < s || e > a.nnz || e - s > a.L) {
        err = lane == 0;
        s = e = 0;
    }
    const int64_t n = e - s;
    const int ntile = (int)((n + kTileK - 1) / kTileK);
    TileRec *out = a.tiles + t * a.nkt;
    for (int i = lane; i < ntile; i += kWave) {
        const int cnt = (int)min((int64_t)kTileK, n - (int64_t)kTileK * i);
        out[i] = TileRec{(int32_t)(s + (int64_t)kTileK * i), (uint32_t)cnt | (cnt < kTileK ? kPartial : 0u)};
    }
    const int32_t last = (int32_t)a.L - 1;
    for (int64_t j = s + lane; j < e; j += kWave) {
        const int32_t k = a.col_idx[j];
        err += k < 0 || k > last || (j > s && k <= a.col_idx[j - 1]);
        a.gidx[j] = min(max(k, 0), last);
    }
    for (int o = 32; o > 0; o >>= 1) err += __shfl_xor(err, o, kWave);
    if (lane == 0) {
        a.cnt[t] = ntile;
        a.full[t] = (int)(n / kTileK);
        a.errs[t] = err;
    }
}

__global__ __launch_bounds__(kChunk) void chunk_counts(DevPlanArgs a)
{
    __shared__ int h[kDevPlanMaxKeys];
    __shared__ int64_t red[kChunkWaves];
    const int64_t chunk = blockIdx.x, i = chunk * kChunk + threadIdx.x;
    for (int k = threadIdx.x; k < a.nkeys; k += kChunk) h[k] = 0;
    __syncthreads();
    int c = 0, f = 0, e = 0;
    if (i < a.ntasks) {
        c = a.cnt[i];
        f = a.full[i];
        e = a.errs ? a.errs[i] : 0;
        atomicAdd(&h[key_of(a, c)], 1);  // LDS
    }
    int64_t sc = 0, sf = 0, se = 0;
    (void)block_exclusive_scan<kChunk>(c, red, &sc);
    (void)block_exclusive_scan<kChunk>(f, red, &sf);
    (void)block_exclusive_scan<kChunk>(e, red, &se);
    if (threadIdx.x == 0) {
        a.csum[3 * chunk] = sc;
        a.csum[3 * chunk + 1] = sf;
        a.csum[3 * chunk + 2] = se;
    }
    __syncthreads();
    for (int k = threadIdx.x; k < a.nkeys; k += kChunk) a.hist[(int64_t)k * a.nchunks + chunk] = h[k];
}

__global__ __launch_bounds__(kChunk) void scan_keys(DevPlanArgs a)
{
    __shared__ int64_t red[kChunkWaves];
    const int64_t n = (int64_t)a.nkeys * a.nchunks, per = (n + kChunk - 1) / kChunk;
    const int64_t lo = min(n, (int64_t)threadIdx.x * per), hi = min(n, lo + per);
    int64_t s = 0;
    for (int64_t i = lo; i < hi; ++i) s += a.hist[i];
    int64_t total = 0;
    int64_t run = block_exclusive_scan<kChunk>(s, red, &total);
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t v = a.hist[i];
        a.hist[i] = (int32_t)run;
        run += v;
    }
    // per-chunk record sums
    int64_t r = 0, f = 0, e = 0;
    for (int64_t ch = threadIdx.x; ch < a.nchunks; ch += kChunk) {
        r += a.csum[3 * ch];
        f += a.csum[3 * ch + 1];
        e += a.csum[3 * ch + 2];
    }
    int64_t rt = 0, ft = 0, et = 0;
    (void)block_exclusive_scan<kChunk>(r, red, &rt);
    (void)block_exclusive_scan<kChunk>(f, red, &ft);
    (void)block_exclusive_scan<kChunk>(e, red, &et);
    if (threadIdx.x == 0) {
        a.hist[n] = (int32_t)total;
        a.stats[0] = rt;
        a.stats[1] = ft;
        a.stats[2] = a.row_ptr ? 0 : a.ntasks * a.nkt - rt;  // gathered lists skip no tile
        a.stats[3] = et;
    }
}

// Launch order: keys ascending (cost classes from the highest down, tasks
// without tiles last); inside a class the tasks keep (head, query tile) order
// and rank r of m goes to slot X (r mod q) + r / q for r < X q (q = m / X),
// the remainder after them in order.
__global__ __launch_bounds__(kChunk) void place_tasks(DevPlanArgs a)
{
    __shared__ int run[kDevPlanMaxKeys];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t chunk = blockIdx.x, i = chunk * kChunk + threadIdx.x;
    for (int k = threadIdx.x; k < a.nkeys; k += kChunk) run[k] = 0;
    const bool valid = i < a.ntasks;
    const int32_t c = valid ? a.cnt[i] : 0;
    const int key = valid ? key_of(a, c) : -1;
    // lanes of this wave before this one with the same key, and all of them
    int before = 0, same = 0;
    for (int j = 0; j < kWave; ++j) {
        const int kj = __shfl(key, j, kWave);
        if (kj == key) {
            ++same;
            before += j < lane;
        }
    }
    __syncthreads();
    // waves in turn: a wave reads the running count of its keys, then the
    // last lane of each key adds the wave's tasks of that key
    int local = 0;
    for (int w = 0; w < kChunkWaves; ++w) {
        if (wave == w && valid) {
            local = run[key] + before;
            if (before == same - 1) run[key] = local + 1;
        }
        __syncthreads();
    }
    if (!valid) return;
    const int64_t kb = (int64_t)key * a.nchunks;
    const int64_t base = a.hist[kb], m = a.hist[kb + a.nchunks] - base;
    const int64_t r = a.hist[kb + chunk] - base + local;
    const int64_t q = m / a.X;
    const int64_t pos = base + (r < a.X * q ? (int64_t)a.X * (r % q) + r / q : r);
    Task tk;
    tk.bh = (int32_t)(i / a.nqt);
    tk.q0 = (int32_t)((i % a.nqt) * a.BQ);
    tk.tb = (int32_t)(i * a.nkt);
    tk.te = tk.tb + c;
    a.tasks[pos] = tk;
}

}  // namespace

hipError_t launch_device_plan(const DevPlanArgs &a, hipStream_t stream)
{
    if (a.ntasks <= 0) return hipSuccess;
    if (a.row_ptr) {
        hipLaunchKernelGGL(slice_map, dim3((unsigned)a.ntasks), dim3(kWave), 0, stream, a);
        hipLaunchKernelGGL(chunk_counts, dim3((unsigned)a.nchunks), dim3(kChunk), 0, stream, a);
        hipLaunchKernelGGL(scan_keys, dim3(1), dim3(kChunk), 0, stream, a);
        hipLaunchKernelGGL(place_tasks, dim3((unsigned)a.nchunks), dim3(kChunk), 0, stream, a);
        return hipGetLastError();
    }
    const int nq = a.BQ / a.bqe, nk = kTileK / a.bke;
    auto map = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3((unsigned)a.ntasks), dim3(kWave), 0, stream, a); };
#define BSA_MAP_CASE(Q, K)                                               \
    else if (nq == Q && nk == K) {                                       \
        if (a.bits) map(map_tasks<Q, K, true>);                          \
        else map(map_tasks<Q, K, false>);                                \
    }
    if (false) {
    }
    BSA_MAP_CASE(1, 1) BSA_MAP_CASE(2, 1) BSA_MAP_CASE(4, 1) BSA_MAP_CASE(8, 1)
    BSA_MAP_CASE(1, 2) BSA_MAP_CASE(2, 2) BSA_MAP_CASE(4, 2) BSA_MAP_CASE(8, 2)
    else return hipErrorInvalidValue;
#undef BSA_MAP_CASE
    hipLaunchKernelGGL(chunk_counts, dim3((unsigned)a.nchunks), dim3(kChunk), 0, stream, a);
    hipLaunchKernelGGL(scan_keys, dim3(1), dim3(kChunk), 0, stream, a);
    hipLaunchKernelGGL(place_tasks, dim3((unsigned)a.nchunks), dim3(kChunk), 0, stream, a);
    return hipGetLastError();
}

}  // namespace bsa
