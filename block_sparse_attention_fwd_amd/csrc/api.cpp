// Host side of the block-sparse attention library: the C ABI, logical-mask
// ingest and validation, physical mapping of logical blocks onto tiles, the
// profile-guided regime lookup, task organisation and the single upload of a
// plan to the device.
//
// Method sources (cited by title and section):
//  - Tessera (arXiv 2609.25869), abstract: logical masks decoupled from GPU
//    execution; a physical mapping layer that retains, combines or subdivides
//    logical blocks into physical tiles; a task organisation layer that groups
//    tiles into GPU tasks for data reuse, parallelism and load/compute
//    overlap; regime selection through a lookup table built by offline
//    profiling, to keep preparation cheap.
//  - Sparse VideoGen / Splash Attention summary ("Sparse VideoGen", "Splash
//    Attention"): spatial/temporal head patterns, empty tiles skipped, exact
//    coordinate masking on boundary tiles only, temporal-major token layout.
//  - FG-Attn (arXiv 2509.16518), abstract: M x 1 slices whose selected keys
//    are gathered into packed tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <memory>
#include <new>
#include <sstream>
#include <stdexcept>
#include <string>
#include <thread>

#include <emmintrin.h>  // SSE2 (x86-64 baseline): byte masks to keep bits
#include <sched.h>
#include <vector>

#include "../../include/bsa.h"
#include "mempool.hpp"
#include "plan_device.hpp"
#include "route_probe.hpp"
#include "plan_format.hpp"

namespace bsa {
hipError_t launch_forward(const KernelArgs &a, int waves, int rb, int d, int dtype, int nbuf, hipStream_t stream);
hipError_t launch_forward_f32(const KernelArgs &a, int waves, int d, hipStream_t stream);
}

using namespace bsa;

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------

static thread_local std::string g_last_error;

static int32_t fail(int32_t status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(bsa_status_str(status)) + ": " + buf;
    return status;
}

extern "C" const char *bsa_status_str(int32_t s)
{
    switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARGUMENT: return "BSA_ERR_INVALID_ARGUMENT";
    case BSA_ERR_INVALID_MASK: return "BSA_ERR_INVALID_MASK";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_OUT_OF_MEMORY: return "BSA_ERR_OUT_OF_MEMORY";
    case BSA_ERR_HIP: return "BSA_ERR_HIP";
    case BSA_ERR_INTERNAL: return "BSA_ERR_INTERNAL";
    default: return "BSA_ERR_UNKNOWN";
    }
}

extern "C" const char *bsa_last_error(void) { return g_last_error.c_str(); }

extern "C" int32_t bsa_abi_version(void) { return BSA_ABI_VERSION; }

// ---------------------------------------------------------------------------
// regimes and the lookup table
// ---------------------------------------------------------------------------

struct Regime {
    int family;  // 0 = contiguous / permuted key tiles, 1 = gathered key lists
    int tile_q;  // = 32 * waves * rb
    int waves;   // wavefronts per workgroup
    int rb;      // 32-row query blocks per wave
    int nbuf;    // LDS key/value buffers: 3 = two tiles in flight (0 = the kernel's default: 2, or 1 for two waves at d = 128)
};

static const Regime kRegimes[] = {
    {0, 128, 4, 1, 0},  // 0: 128 x 64 tiles, 4 waves of 32 rows
    {0, 64, 2, 1, 0},   // 1: 64 x 64 tiles, 2 waves of 32 rows (d = 128: one LDS buffer, four workgroups per CU)
    {1, 64, 2, 1, 0},   // 2: 64-query gather tiles (as regime 1)
    {1, 128, 4, 1, 0},  // 3: 128-query gather tiles
    {0, 256, 8, 1, 3},  // 4: 256 x 64 tiles, 8 waves of 32 rows, three LDS buffers (copies two tiles ahead)
};
static const int kNumRegimes = (int)(sizeof kRegimes / sizeof kRegimes[0]);

extern "C" int32_t bsa_regime_count(void) { return kNumRegimes; }

extern "C" int32_t bsa_regime_info(int32_t r, bsa_regime_desc_t *out)
{
    if (!out || r < 0 || r >= kNumRegimes) return fail(BSA_ERR_INVALID_ARGUMENT, "regime %d out of range", r);
    out->family = kRegimes[r].family;
    out->tile_q = kRegimes[r].tile_q;
    out->tile_k = kTileK;
    out->waves = kRegimes[r].waves;
    out->rows_per_wave = 32 * kRegimes[r].rb;
    return BSA_OK;
}

// Lookup-table rule: first matching line wins. Fields:
//   kind block_q block_k density_lo density_hi fill_lo fill_hi [fill2_lo fill2_hi] L_lo L_hi regime [order]
// kind is block|slice|video; block sizes may be '*'; order is xcd (the
// default) or lpt (BSA_ORDER_*); a line without the fill2 range matches any
// fill2. density, fill and fill2 are the mask features of mask_features()
// (-1 where a kind has none; such a feature matches any range).
struct LutRule {
    int kind;  // BSA_MASK_BLOCK_U8 (both block kinds), SLICE, VIDEO
    int bq, bk;  // 0 = any
    double dlo, dhi;
    double flo, fhi;
    double f2lo, f2hi;  // fill of 256-row tiles ([0, 1] when the line omits it)
    int64_t Llo, Lhi;
    int regime;
    int order;
};

#include "lut_default.inc"  // defines kDefaultLut (text of lut/gfx950.lut)

static bool parse_lut(const std::string &text, std::vector<LutRule> &rules, std::string &err)
{
    std::istringstream in(text);
    std::string line;
    int ln = 0;
    while (std::getline(in, line)) {
        ++ln;
        auto hash = line.find('#');
        if (hash != std::string::npos) line.resize(hash);
        // kind bq bk density_lo density_hi fill_lo fill_hi [fill2_lo fill2_hi] L_lo L_hi regime [order]
        std::istringstream ls(line);
        std::vector<std::string> tok;
        for (std::string t; ls >> t;) tok.push_back(t);
        if (tok.empty()) continue;
        LutRule r{};
        r.order = BSA_ORDER_XCD_GROUPED;
        if (tok.back() == "lpt" || tok.back() == "xcd") {
            if (tok.back() == "lpt") r.order = BSA_ORDER_LONGEST_FIRST;
            tok.pop_back();
        }
        const std::string &kind = tok[0];
        if (kind == "block") r.kind = BSA_MASK_BLOCK_U8;
        else if (kind == "slice") r.kind = BSA_MASK_SLICE_CSR;
        else if (kind == "video") r.kind = BSA_MASK_VIDEO;
        else { err = "lookup table line " + std::to_string(ln) + ": unknown kind " + kind; return false; }
        if (tok.size() == 11 || tok.size() == 13) {
            // one field more than a rule: an order name that is neither xcd nor lpt
            char *end = nullptr;
            (void)std::strtod(tok.back().c_str(), &end);
            if (end && *end != '\0') {
                err = "lookup table line " + std::to_string(ln) + ": unknown order " + tok.back();
                return false;
            }
        }
        if (tok.size() != 10 && tok.size() != 12) {
            err = "lookup table line " + std::to_string(ln) + " malformed";
            return false;
        }
        const bool has_f2 = tok.size() == 12;
        const std::string &bq = tok[1], &bk = tok[2];
        r.f2lo = 0.0;
        r.f2hi = 1.0;
        // every numeric field must be a whole number token
        auto real = [](const std::string &t) {
            size_t used = 0;
            const double v = std::stod(t, &used);
            if (used != t.size()) throw std::invalid_argument(t);
            return v;
        };
        auto whole = [](const std::string &t) {
            size_t used = 0;
            const long long v = std::stoll(t, &used);
            if (used != t.size()) throw std::invalid_argument(t);
            return v;
        };
        try {
            size_t i = 3;
            r.dlo = real(tok[i++]);
            r.dhi = real(tok[i++]);
            r.flo = real(tok[i++]);
            r.fhi = real(tok[i++]);
            if (has_f2) {
                r.f2lo = real(tok[i++]);
                r.f2hi = real(tok[i++]);
            }
            r.Llo = whole(tok[i++]);
            r.Lhi = whole(tok[i++]);
            const long long reg = whole(tok[i]);
            if (reg < 0 || reg >= kNumRegimes) {
                err = "lookup table line " + std::to_string(ln) + ": regime out of range";
                return false;
            }
            r.regime = (int)reg;
            r.bq = bq == "*" ? 0 : (int)whole(bq);
            r.bk = bk == "*" ? 0 : (int)whole(bk);
        } catch (const std::exception &) {
            err = "lookup table line " + std::to_string(ln) + " malformed";
            return false;
        }
        rules.push_back(r);
    }
    return true;
}

// ---------------------------------------------------------------------------
// the plan object
// ---------------------------------------------------------------------------

// A plan is one contiguous image -- tasks | tile records | gather indices |
// head flags, each section 256-byte aligned -- identical on the host (pinned
// memory from a recycling pool, or plain memory for host-only plans) and on
// the device (a block from a per-device recycling pool). It is uploaded once,
// asynchronously on a library stream; bsa_forward orders its launch after the
// upload with an event.
struct bsa_plan_s {
    int32_t B = 0, H = 0, d = 0, dtype = 0;
    int64_t L = 0;
    int32_t kind = 0, block_q = 0, block_k = 0;
    int32_t regime = 0;
    int32_t T = 0, Hg = 0, Wg = 0, anchor = 0, radius = 0;
    int32_t bq_shift = 0, bk_shift = 0, nsk = 1, sub_q = 0, sub_k = 0;
    int32_t mode = 0;
    int32_t task_order = BSA_ORDER_XCD_GROUPED;
    double mask_density = -1.0, mask_fill = -1.0, mask_fill2 = -1.0;  // regime-lookup features (-1: none for the kind)
    std::vector<uint8_t> head_layout, head_pattern;
    // image
    uint8_t *img = nullptr;
    size_t img_cap = 0, img_bytes = 0;
    bool img_pinned = false;
    std::unique_ptr<uint8_t[]> img_host;  // the image of a host-only plan, or a device plan read back (not zero-filled)
    size_t img_host_n = 0;
    size_t off_tasks = 0, off_tiles = 0, off_gidx = 0, off_flags = 0, off_coords = 0;
    int64_t coord_stride = 0;                   // words per video key-coordinate table
    std::vector<uint8_t> head_coord_table;      // per head: index of its table
    int64_t ntasks = 0, ntiles = 0, ngidx = 0;  // ntasks: tasks in the task array
    int64_t nreal_tasks = 0;                    // one per (batch, head, query tile)
    const Task *tasks() const { return (const Task *)(img + off_tasks); }
    const TileRec *tiles() const { return (const TileRec *)(img + off_tiles); }
    const int32_t *gidx() const { return (const int32_t *)(img + off_gidx); }
    // statistics
    int64_t tiles_full = 0, tiles_partial = 0, tiles_empty = 0, gather_rows = 0;
    int64_t plan_ns = 0;
    int64_t phase_ns[5] = {0, 0, 0, 0, 0};  // ingest, regime, mapping, tasks, upload
    // device copy
    int32_t device = -1;
    void *dev = nullptr;
    size_t dev_cap = 0;
    hipEvent_t uploaded = nullptr;
    std::atomic<bool> upload_seen{false};  // `uploaded` has completed (forwards need not wait on it)
    // Completes after every forward enqueued on this plan so far: bsa_forward
    // records it after each launch, so that destroying the plan waits for the
    // kernels that still read its device image before the image goes back to
    // the recycling pool (where the next plan may upload into it).
    hipEvent_t last_use = nullptr;
    hipStream_t last_stream = nullptr;
    bool used = false;
    std::mutex use_mu;
    // plans built on the device (bsa_plan_device): the image exists only in
    // device memory until a host query reads back its statistics (and, for
    // the coverage, the task and record sections)
    bool device_planned = false;
    bool stats_read = false;
    bool host_copy = false;
    size_t off_stats = 0;
    int64_t mask_errors = 0;   // invalid slice entries the planning kernels found
    uint8_t *small = nullptr;  // pinned upload source of the head flags and cost classes
    size_t small_cap = 0;
};

static int ilog2(int v)
{
    int s = 0;
    while ((1 << s) < v) ++s;
    return s;
}
static bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// ---------------------------------------------------------------------------
// video-pattern tile classification (exact-safe: EMPTY and FULL are claimed
// only when true for every pair; anything else is PARTIAL and masked exactly
// on the device)
// ---------------------------------------------------------------------------

namespace {

struct Geo {
    int64_t L, T, HW, W;
};

struct Rect {
    int64_t y0, y1, x0, x1;
};

// Frames covered by logical positions [lo, hi] of a head, as a 64-bit set
// (T <= 64) or as "all" when it cannot be represented exactly.
struct FrameSet {
    bool all;
    uint64_t bits;
};

inline FrameSet frames_of(const Geo &g, bool tm, int64_t lo, int64_t hi)
{
    FrameSet f{false, 0};
    if (g.T > 64) { f.all = true; return f; }
    if (!tm) {
        int64_t a = lo / g.HW, b = hi / g.HW;
        for (int64_t t = a; t <= b; ++t) f.bits |= 1ull << t;
        return f;
    }
    int64_t n = hi - lo + 1;
    if (n >= g.T) { f.bits = g.T == 64 ? ~0ull : ((1ull << g.T) - 1); return f; }
    for (int64_t i = 0; i < n; ++i) f.bits |= 1ull << ((lo + i) % g.T);
    return f;
}

// At most 6 rectangles: a raster range is <= 3, a range wrapping over the
// frame end is two raster ranges.
struct Rects {
    Rect r[6];
    int n = 0;
    void clear() { n = 0; }
    void push_back(const Rect &x) { r[n++] = x; }
    const Rect *begin() const { return r; }
    const Rect *end() const { return r + n; }
};

inline void range_rects(const Geo &g, int64_t p0, int64_t p1, Rects &out)
{
    int64_t y0 = p0 / g.W, x0 = p0 % g.W, y1 = p1 / g.W, x1 = p1 % g.W;
    if (y0 == y1) { out.push_back({y0, y0, x0, x1}); return; }
    out.push_back({y0, y0, x0, g.W - 1});
    if (y1 > y0 + 1) out.push_back({y0 + 1, y1 - 1, 0, g.W - 1});
    out.push_back({y1, y1, 0, x1});
}

// Pixels covered by logical positions [lo, hi] of a head.
inline void pixel_rects(const Geo &g, bool tm, int64_t lo, int64_t hi, Rects &out)
{
    out.clear();
    if (tm) { range_rects(g, lo / g.T, hi / g.T, out); return; }
    if (hi - lo + 1 >= g.HW) { range_rects(g, 0, g.HW - 1, out); return; }
    int64_t p0 = lo % g.HW, p1 = hi % g.HW;
    if (p0 <= p1) range_rects(g, p0, p1, out);
    else { range_rects(g, p0, g.HW - 1, out); range_rects(g, 0, p1, out); }
}

inline int64_t gap(int64_t a0, int64_t a1, int64_t b0, int64_t b1) { return std::max<int64_t>({0, b0 - a1, a0 - b1}); }
inline int64_t span(int64_t a0, int64_t a1, int64_t b0, int64_t b1) { return std::max(a1 - b0, b1 - a0); }

enum { kEmpty = 0, kFull = 1, kPart = 2 };

struct VideoTileSets {
    FrameSet f;
    Rects r;
};

inline int classify_video(int pattern, int64_t anchor, int64_t radius, const VideoTileSets &q, const VideoTileSets &k,
                          bool key_crop)
{
    bool any, all;
    if (pattern == BSA_PAT_DENSE) {
        any = all = true;
    } else if (pattern == BSA_PAT_SPATIAL) {
        if (q.f.all || k.f.all) {
            any = true;
            all = false;
        } else {
            bool a_in_k = anchor < 64 && ((k.f.bits >> anchor) & 1);
            any = (q.f.bits & k.f.bits) != 0 || a_in_k;
            // every key frame must be the anchor, or the single query frame
            all = true;
            uint64_t kb = k.f.bits;
            bool q_single = q.f.bits && !(q.f.bits & (q.f.bits - 1));
            while (kb) {
                int t = __builtin_ctzll(kb);
                kb &= kb - 1;
                if (t == anchor) continue;
                if (!(q_single && ((q.f.bits >> t) & 1))) { all = false; break; }
            }
        }
    } else {
        any = false;
        all = true;
        for (const Rect &a : q.r)
            for (const Rect &b : k.r) {
                if (std::max(gap(a.y0, a.y1, b.y0, b.y1), gap(a.x0, a.x1, b.x0, b.x1)) <= radius) any = true;
                if (std::max(span(a.y0, a.y1, b.y0, b.y1), span(a.x0, a.x1, b.x0, b.x1)) > radius) all = false;
            }
    }
    if (!any) return kEmpty;
    if (all && !key_crop) return kFull;
    return kPart;
}

// Per-head output of the mapping, later concatenated.
struct HeadOut {
    std::vector<Task> tasks;
    std::vector<TileRec> tiles;  // k0/offsets relative to this head's gidx block
    std::vector<int32_t> gidx;
    int64_t full = 0, part = 0, empty = 0, grows = 0;
    void clear()
    {
        tasks.clear();
        tiles.clear();
        gidx.clear();
        full = part = empty = grows = 0;
    }
};

// Persistent worker threads for the planner (creating threads on every
// bsa_plan call costs more than the mapping of a small mask). One parallel
// region runs at a time; a nested or concurrent region runs on the caller.
class WorkerPool {
  public:
    static WorkerPool &get()
    {
        static WorkerPool *pool = new WorkerPool();  // lives until process exit
        return *pool;
    }

    void run(int64_t n, const std::function<void(int64_t)> &f)
    {
        if (n <= 0) return;
        std::unique_lock<std::mutex> region(region_mu_, std::try_to_lock);
        if (n == 1 || in_worker_ || !region.owns_lock() || workers_.empty()) {
            for (int64_t i = 0; i < n; ++i) f(i);
            return;
        }
        {
            std::lock_guard<std::mutex> g(mu_);
            job_ = &f;
            n_ = n;
            next_.store(0);
            pending_ = (int)workers_.size();
            gen_.store(gen_.load(std::memory_order_relaxed) + 1, std::memory_order_release);
        }
        cv_.notify_all();
        drain();
        std::unique_lock<std::mutex> g(mu_);
        done_cv_.wait(g, [&] { return pending_ == 0; });
        job_ = nullptr;
    }

  private:
    WorkerPool()
    {
        // threads = the CPUs this process may run on (affinity mask), at most
        // OMP_NUM_THREADS when that is set, at most 32
        unsigned hc = std::thread::hardware_concurrency();
        cpu_set_t cs;
        if (sched_getaffinity(0, sizeof cs, &cs) == 0 && CPU_COUNT(&cs) > 0) hc = (unsigned)CPU_COUNT(&cs);
        if (const char *e = std::getenv("OMP_NUM_THREADS"); e && std::atoi(e) > 0) hc = std::min(hc, (unsigned)std::atoi(e));
        const int nt = (int)std::max(1u, std::min(hc, 32u)) - 1;
        for (int t = 0; t < nt; ++t) workers_.emplace_back([this] { loop(); });
        for (auto &w : workers_) w.detach();
    }

    void drain()
    {
        for (int64_t i; (i = next_.fetch_add(1)) < n_;) (*job_)(i);
    }

    void loop()
    {
        in_worker_ = true;
        uint64_t seen = 0;
        for (;;) {
            // a planner runs several parallel regions in a row, and plans often
            // follow each other closely: look for the next region for a short
            // while before sleeping (a wake-up costs tens of microseconds)
            const auto spin_end = std::chrono::steady_clock::now() + std::chrono::microseconds(kSpinUs);
            while (gen_.load(std::memory_order_acquire) == seen && std::chrono::steady_clock::now() < spin_end)
                std::this_thread::yield();
            {
                std::unique_lock<std::mutex> g(mu_);
                cv_.wait(g, [&] { return gen_.load(std::memory_order_acquire) != seen; });
                seen = gen_.load(std::memory_order_acquire);
            }
            drain();
            {
                std::lock_guard<std::mutex> g(mu_);
                if (--pending_ == 0) done_cv_.notify_one();
            }
        }
    }

    std::mutex region_mu_, mu_;
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> workers_;
    const std::function<void(int64_t)> *job_ = nullptr;
    int64_t n_ = 0;
    std::atomic<int64_t> next_{0};
    int pending_ = 0;
    std::atomic<uint64_t> gen_{0};
    static constexpr int kSpinUs = 300;
    static thread_local bool in_worker_;
};
thread_local bool WorkerPool::in_worker_ = false;

template <class F>
void parallel_for(int64_t n, F &&f)
{
    const std::function<void(int64_t)> fn = f;
    WorkerPool::get().run(n, fn);
}

}  // namespace

// ---------------------------------------------------------------------------
// physical mapping per head
// ---------------------------------------------------------------------------

// Keep bits of one BLOCK_U8 row (nkb bytes, nonzero = kept) as 64-bit words,
// bit j of word w = block 64 w + j; 16 bytes per SSE2 compare.
static void u8_row_bits(const uint8_t *row, int64_t nkb, uint64_t *out)
{
    const int64_t words = (nkb + 63) / 64;
    const __m128i zero = _mm_setzero_si128();
    for (int64_t w = 0; w < words; ++w) {
        const int64_t base = w * 64, n = std::min<int64_t>(64, nkb - base);
        uint64_t x = 0;
        if (n == 64) {
            for (int c = 0; c < 4; ++c) {
                const __m128i v = _mm_loadu_si128((const __m128i *)(row + base + 16 * c));
                const unsigned z = (unsigned)_mm_movemask_epi8(_mm_cmpeq_epi8(v, zero));
                x |= (uint64_t)(~z & 0xFFFFu) << (16 * c);
            }
        } else {
            for (int64_t j = 0; j < n; ++j) x |= (uint64_t)(row[base + j] != 0) << j;
        }
        out[w] = x;
    }
}

// Keep-bit row qb of head bh: BLOCK_BITS rows directly, BLOCK_U8 rows
// converted into `buf` (words entries).
static const uint64_t *block_row_bits(const bsa_mask_desc_t &m, int64_t bh, int64_t qb, int64_t nqb, int64_t nkb,
                                      uint64_t *buf)
{
    const int64_t words = (nkb + 63) / 64;
    if (m.kind == BSA_MASK_BLOCK_BITS) return (const uint64_t *)m.data + (bh * nqb + qb) * words;
    u8_row_bits((const uint8_t *)m.data + (bh * nqb + qb) * nkb, nkb, buf);
    return buf;
}

// BLOCK masks: retain (bq = tile_q, bk = tile_k), combine (smaller logical
// blocks merged into one tile, kept sub-blocks recorded as bits) or subdivide
// (larger logical blocks split over several tiles). Each logical row is read
// as keep-bit words and only its kept blocks are visited (ctz); a bitset of
// the key tiles the query tile touches yields the records in key order, so
// the work per query tile follows the kept blocks, not the row length.
static void map_block_head(const bsa_plan_s &p, const bsa_mask_desc_t &m, int b, int h, int BQ, int64_t tq_lo,
                           int64_t tq_hi, HeadOut &out)
{
    const int64_t L = p.L;
    const int64_t nqb = (L + p.block_q - 1) / p.block_q, nkb = (L + p.block_k - 1) / p.block_k;
    const int64_t nkt = (L + kTileK - 1) / kTileK;
    const int bqe = std::min(p.block_q, BQ), bke = std::min(p.block_k, kTileK);
    const int nsq = BQ / bqe, nsk = kTileK / bke;
    const int64_t bh = (int64_t)b * p.H + h;
    const int64_t words = (nkb + 63) / 64, twords = (nkt + 63) / 64;
    // key blocks of at most one tile (block_k <= 64): the key tiles are read
    // straight off the rows' bit words, one word (64 or 32 key tiles) at a
    // time; larger key blocks (split over several tiles) go through a per-tile
    // accumulator
    const bool word_path = p.block_k <= kTileK;
    std::vector<uint64_t> rowbuf((size_t)words * (word_path ? nsq : 1));
    std::vector<uint32_t> acc(word_path ? 0 : (size_t)nkt, 0u);
    std::vector<uint64_t> touched(word_path ? 0 : (size_t)twords, 0u);
    out.tasks.reserve((size_t)(tq_hi - tq_lo));
    for (int64_t tq = tq_lo; tq < tq_hi; ++tq) {
        const int64_t q0 = tq * BQ, q1 = std::min<int64_t>(q0 + BQ, L);
        const int64_t qb0 = q0 / p.block_q, qb1 = (q1 - 1) / p.block_q;
        const int nsq_valid = (int)std::min<int64_t>(nsq, (q1 - 1 - q0) / bqe + 1);
        Task t{(int32_t)bh, (int32_t)q0, (int32_t)out.tiles.size(), 0};
        int64_t n_tiles = 0;
        // a tile whose rows and keys all exist is FULL when every one of its
        // sub-blocks is kept; a cropped last key tile is always PARTIAL
        uint32_t want_full = 0;
        for (int sq = 0; sq < nsq_valid; ++sq)
            for (int sk = 0; sk < nsk; ++sk) want_full |= 1u << (sq * nsk + sk);
        auto emit = [&](int64_t tk, uint32_t bits) {
            const int64_t k0 = tk * kTileK;
            const bool full = k0 + kTileK <= L && (bits & want_full) == want_full;
            out.tiles.push_back({(int32_t)k0, bits | (full ? 0u : kPartial)});
            if (full) ++out.full; else ++out.part;
            ++n_tiles;
        };
        if (word_path) {
            // the logical rows of the tile (sub-row sq of each) as bit words
            const uint64_t *rows[32];
            int sqs[32];
            int nr = 0;
            for (int64_t qb = qb0; qb <= qb1; ++qb, ++nr) {
                sqs[nr] = qb * p.block_q <= q0 ? 0 : (int)((qb * p.block_q - q0) / bqe);
                rows[nr] = block_row_bits(m, bh, qb, nqb, nkb, rowbuf.data() + (size_t)nr * words);
            }
            for (int64_t w = 0; w < words; ++w) {
                uint64_t o = 0;
                for (int r = 0; r < nr; ++r) o |= rows[r][w];
                if (!o) continue;
                if (nsk == 1) {
                    // bit j of word w: key block = key tile 64 w + j
                    for (uint64_t x = o; x; x &= x - 1) {
                        const int j = __builtin_ctzll(x);
                        uint32_t bits = 0;
                        for (int r = 0; r < nr; ++r) bits |= (uint32_t)((rows[r][w] >> j) & 1u) << sqs[r];
                        emit(w * 64 + j, bits);
                    }
                } else {
                    // bits j, j + 1 (j even) of word w: the two 32-key blocks of
                    // key tile 32 w + j / 2
                    for (uint64_t x = (o | (o >> 1)) & 0x5555555555555555ull; x; x &= x - 1) {
                        const int j = __builtin_ctzll(x);
                        uint32_t bits = 0;
                        for (int r = 0; r < nr; ++r) bits |= (uint32_t)((rows[r][w] >> j) & 3u) << (2 * sqs[r]);
                        emit(w * 32 + j / 2, bits);
                    }
                }
            }
        } else {
            for (int64_t qb = qb0; qb <= qb1; ++qb) {
                const int sq = qb * p.block_q <= q0 ? 0 : (int)((qb * p.block_q - q0) / bqe);
                const uint64_t *row = block_row_bits(m, bh, qb, nqb, nkb, rowbuf.data());
                // a key block spans block_k / 64 tiles (the last one cropped at L)
                for (int64_t w = 0; w < words; ++w)
                    for (uint64_t x = row[w]; x; x &= x - 1) {
                        const int64_t kb = w * 64 + __builtin_ctzll(x);
                        const int64_t k_lo = kb * p.block_k, k_hi = std::min<int64_t>(k_lo + p.block_k, L) - 1;
                        for (int64_t tk = k_lo / kTileK; tk <= k_hi / kTileK; ++tk) {
                            acc[tk] |= 1u << (sq * nsk);
                            touched[tk >> 6] |= 1ull << (tk & 63);
                        }
                    }
            }
            for (int64_t tw = 0; tw < twords; ++tw) {
                for (uint64_t x = touched[tw]; x; x &= x - 1) {
                    const int64_t tk = tw * 64 + __builtin_ctzll(x);
                    emit(tk, acc[tk]);
                    acc[tk] = 0u;
                }
                touched[tw] = 0u;
            }
        }
        out.empty += nkt - n_tiles;
        t.te = (int32_t)out.tiles.size();
        out.tasks.push_back(t);
    }
}

// VIDEO masks: for each query tile, classify the key tiles of a candidate
// superset derived from the pattern (frames of the query tile and the anchor
// frame; key pixels within the window of the query pixels); every tile outside
// it is provably empty. Candidates are classified exactly. A PARTIAL tile is
// classified again for each wave's rows, with the same exact-safe test: a wave
// none of whose pairs is kept skips the tile, a wave all of whose pairs are
// kept runs it unmasked (Splash Attention's empty-tile skip and boundary-only
// masking, applied at the granularity one wavefront computes).
static void map_video_head(const bsa_plan_s &p, int b, int h, int BQ, int64_t tq_lo, int64_t tq_hi, HeadOut &out)
{
    const int64_t L = p.L;
    const Geo g{L, p.T, (int64_t)p.Hg * p.Wg, p.Wg};
    const bool tm = p.head_layout[h] == BSA_LAYOUT_TEMPORAL_MAJOR;
    const int pat = p.head_pattern[h];
    const int64_t nkt = (L + kTileK - 1) / kTileK;
    const int64_t bh = (int64_t)b * p.H + h;
    const int64_t r = p.radius, W = p.Wg, Hg = p.Hg, HW = g.HW;
    VideoTileSets ks;  // frames or pixels of the key tile being classified
    VideoTileSets qs;
    const int NWV = BQ / kWaveRows;
    VideoTileSets qw[8];                            // per-wave query sets (NWV <= 8)
    int64_t qw_rows[8];
    std::vector<std::pair<int64_t, int64_t>> cand;  // key-tile index ranges [t0, t1]
    auto add_keys = [&](int64_t lo, int64_t hi) {   // key positions [lo, hi]
        lo = std::max<int64_t>(lo, 0);
        hi = std::min<int64_t>(hi, L - 1);
        if (lo <= hi) cand.push_back({lo / kTileK, hi / kTileK});
    };
    out.tasks.reserve((size_t)(tq_hi - tq_lo));
    int64_t computed = 0;
    for (int64_t tq = tq_lo; tq < tq_hi; ++tq) {
        const int64_t q0 = tq * BQ, q1 = std::min<int64_t>(q0 + BQ, L);
        if (pat == BSA_PAT_SPATIAL) qs.f = frames_of(g, tm, q0, q1 - 1);
        if (pat == BSA_PAT_TEMPORAL) pixel_rects(g, tm, q0, q1 - 1, qs.r);
        for (int wv = 0; wv < NWV; ++wv) {
            const int64_t a = q0 + (int64_t)kWaveRows * wv, e = std::min<int64_t>(a + kWaveRows, q1);
            qw_rows[wv] = e - a;
            if (e <= a) continue;
            if (pat == BSA_PAT_SPATIAL) qw[wv].f = frames_of(g, tm, a, e - 1);
            if (pat == BSA_PAT_TEMPORAL) pixel_rects(g, tm, a, e - 1, qw[wv].r);
        }
        cand.clear();
        if (pat == BSA_PAT_SPATIAL && !tm) {
            const int64_t fa = q0 / HW, fb = (q1 - 1) / HW;
            add_keys(fa * HW, (fb + 1) * HW - 1);
            add_keys((int64_t)p.anchor * HW, ((int64_t)p.anchor + 1) * HW - 1);
        } else if (pat == BSA_PAT_TEMPORAL && tm) {
            // key pixels within the window of a query rectangle, one pixel range
            // per window row; a pixel owns T consecutive positions
            for (const Rect &rc : qs.r) {
                const int64_t xa = std::max<int64_t>(0, rc.x0 - r), xb = std::min<int64_t>(W - 1, rc.x1 + r);
                for (int64_t y = std::max<int64_t>(0, rc.y0 - r); y <= std::min<int64_t>(Hg - 1, rc.y1 + r); ++y)
                    add_keys((y * W + xa) * p.T, (y * W + xb + 1) * p.T - 1);
            }
        } else if (pat == BSA_PAT_TEMPORAL) {
            // frame-major: the band of window rows, once per frame
            int64_t ymin = Hg, ymax = -1;
            for (const Rect &rc : qs.r) { ymin = std::min(ymin, rc.y0); ymax = std::max(ymax, rc.y1); }
            const int64_t ya = std::max<int64_t>(0, ymin - r), yb = std::min<int64_t>(Hg - 1, ymax + r);
            for (int64_t t = 0; t < p.T; ++t) add_keys(t * HW + ya * W, t * HW + (yb + 1) * W - 1);
        } else {
            add_keys(0, L - 1);
        }
        std::sort(cand.begin(), cand.end());
        Task t{(int32_t)bh, (int32_t)q0, (int32_t)out.tiles.size(), 0};
        int64_t last = -1;
        for (const auto &c : cand) {
            for (int64_t tk = std::max(c.first, last + 1); tk <= c.second; ++tk) {
                const int64_t k0 = tk * kTileK, k1 = std::min<int64_t>(k0 + kTileK, L);
                const bool crop = k0 + kTileK > L;
                if (pat == BSA_PAT_SPATIAL) ks.f = frames_of(g, tm, k0, k1 - 1);
                if (pat == BSA_PAT_TEMPORAL) pixel_rects(g, tm, k0, k1 - 1, ks.r);
                int cl = classify_video(pat, p.anchor, p.radius, qs, ks, crop);
                if (cl == kEmpty) continue;
                uint32_t aux = 0;
                if (cl == kPart) {
                    aux = kPartial;
                    for (int wv = 0; wv < NWV; ++wv) {
                        const int wc = qw_rows[wv] <= 0 ? kEmpty : classify_video(pat, p.anchor, p.radius, qw[wv], ks, crop);
                        if (wc == kEmpty) aux |= 1u << wv;
                        if (wc == kFull) aux |= 1u << (kWaveFullShift + wv);
                    }
                }
                out.tiles.push_back({(int32_t)k0, aux});
                if (cl == kFull) ++out.full; else ++out.part;
            }
            last = std::max(last, c.second);
        }
        computed += (int64_t)out.tiles.size() - t.tb;
        t.te = (int32_t)out.tiles.size();
        out.tasks.push_back(t);
    }
    out.empty = (tq_hi - tq_lo) * nkt - computed;
}

// SLICE masks: each M-query block's sorted key list packed into gather tiles
// of kTileK keys; only the last tile of a list can be short (masked).
static void map_slice_head(const bsa_plan_s &p, const bsa_mask_desc_t &m, int b, int h, int64_t tq_lo, int64_t tq_hi,
                           HeadOut &out)
{
    const int64_t L = p.L, M = p.block_q, nqb = (L + M - 1) / M;
    const int64_t bh = (int64_t)b * p.H + h;
    const int64_t base = m.row_ptr[bh * nqb + tq_lo];
    const int64_t n_all = m.row_ptr[bh * nqb + tq_hi] - base;
    out.gidx.assign(m.col_idx + base, m.col_idx + base + n_all);
    out.grows = n_all;
    for (int64_t i = tq_lo; i < tq_hi; ++i) {
        const int64_t s = m.row_ptr[bh * nqb + i] - base, e = m.row_ptr[bh * nqb + i + 1] - base;
        Task t{(int32_t)bh, (int32_t)(i * M), (int32_t)out.tiles.size(), 0};
        for (int64_t o = s; o < e; o += kTileK) {
            uint32_t cnt = (uint32_t)std::min<int64_t>(kTileK, e - o);
            out.tiles.push_back({(int32_t)o, cnt | (cnt < (uint32_t)kTileK ? kPartial : 0u)});
            if (cnt < (uint32_t)kTileK) ++out.part; else ++out.full;
        }
        t.te = (int32_t)out.tiles.size();
        out.tasks.push_back(t);
    }
}

// ---------------------------------------------------------------------------
// validation (mask ingest)
// ---------------------------------------------------------------------------

static int32_t validate(const bsa_mask_desc_t *m, int32_t B, int32_t H, int64_t L, int32_t d, int32_t bq, int32_t bk,
                        const bsa_plan_opts_t &o, bool device_mask = false)
{
    if (!m) return fail(BSA_ERR_INVALID_ARGUMENT, "logical_mask is NULL");
    if (B < 1 || H < 1 || L < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "B, H, L must be >= 1 (got %d, %d, %lld)", B, H, (long long)L);
    if (L > (1ll << 30)) return fail(BSA_ERR_UNSUPPORTED, "L = %lld exceeds 2^30", (long long)L);
    if (d != 64 && d != 128) return fail(BSA_ERR_UNSUPPORTED, "head dim d = %d (supported: 64, 128)", d);
    if (o.dtype != BSA_DTYPE_BF16 && o.dtype != BSA_DTYPE_F32) return fail(BSA_ERR_INVALID_ARGUMENT, "dtype %d", o.dtype);
    const bool has_geo = o.T || o.Hg || o.Wg;
    if (has_geo) {
        if (o.T < 1 || o.Hg < 1 || o.Wg < 1 || (int64_t)o.T * o.Hg * o.Wg != L)
            return fail(BSA_ERR_INVALID_ARGUMENT, "video geometry %d x %d x %d does not match L = %lld", o.T, o.Hg, o.Wg, (long long)L);
        if (o.T > 2046 || o.Hg > 512 || o.Wg > 512)
            return fail(BSA_ERR_UNSUPPORTED, "video geometry beyond T <= 2046, Hg <= 512, Wg <= 512");
    }
    if (o.head_layout) {
        for (int h = 0; h < H; ++h) {
            if (o.head_layout[h] > 1) return fail(BSA_ERR_INVALID_ARGUMENT, "head_layout[%d] = %d", h, o.head_layout[h]);
            if (o.head_layout[h] == BSA_LAYOUT_TEMPORAL_MAJOR && !has_geo)
                return fail(BSA_ERR_INVALID_ARGUMENT, "temporal-major head %d needs the video geometry", h);
        }
    }
    if (o.force_regime < -1 || o.force_regime >= kNumRegimes)
        return fail(BSA_ERR_INVALID_ARGUMENT, "force_regime %d out of range", o.force_regime);
    if (o.task_order < -1 || o.task_order > BSA_ORDER_LONGEST_FIRST)
        return fail(BSA_ERR_INVALID_ARGUMENT, "task_order %d out of range", o.task_order);
    switch (m->kind) {
    case BSA_MASK_BLOCK_U8:
    case BSA_MASK_BLOCK_BITS:
        if (!m->data) return fail(BSA_ERR_INVALID_ARGUMENT, "block mask data is NULL");
        if (!is_pow2(bq) || !is_pow2(bk) || bq < 32 || bk < 32 || bq > 1024 || bk > 1024)
            return fail(BSA_ERR_UNSUPPORTED, "block shape %d x %d (supported: powers of two in [32, 1024])", bq, bk);
        if (m->kind == BSA_MASK_BLOCK_BITS && !device_mask) {
            const int64_t nqb = (L + bq - 1) / bq, nkb = (L + bk - 1) / bk, words = (nkb + 63) / 64;
            if (nkb % 64) {
                const uint64_t stray = ~0ull << (nkb % 64);
                const uint64_t *w = (const uint64_t *)m->data;
                for (int64_t r = 0; r < (int64_t)B * H * nqb; ++r)
                    if (w[r * words + words - 1] & stray)
                        return fail(BSA_ERR_INVALID_MASK, "bit row %lld has bits beyond key block %lld", (long long)r, (long long)nkb);
            }
        }
        return BSA_OK;
    case BSA_MASK_SLICE_CSR: {
        if (!m->row_ptr || !m->col_idx) return fail(BSA_ERR_INVALID_ARGUMENT, "slice row_ptr/col_idx is NULL");
        if (bk != 1) return fail(BSA_ERR_INVALID_ARGUMENT, "slice masks need block_k = 1 (got %d)", bk);
        if (bq != 64 && bq != 128) return fail(BSA_ERR_UNSUPPORTED, "slice block M = %d (supported: 64, 128)", bq);
        if (m->nnz < 0 || m->nnz > (1ll << 31) - 1) return fail(BSA_ERR_INVALID_ARGUMENT, "slice nnz = %lld", (long long)m->nnz);
        // a device mask is checked by the planning kernels (see bsa_plan_device)
        if (device_mask) return BSA_OK;
        const int64_t nl = (int64_t)B * H * ((L + bq - 1) / bq);
        if (m->nnz && m->nnz != m->row_ptr[nl])
            return fail(BSA_ERR_INVALID_MASK, "nnz = %lld but row_ptr ends at %lld", (long long)m->nnz, (long long)m->row_ptr[nl]);
        if (m->row_ptr[0] != 0) return fail(BSA_ERR_INVALID_MASK, "row_ptr[0] = %lld, expected 0", (long long)m->row_ptr[0]);
        for (int64_t i = 0; i < nl; ++i)
            if (m->row_ptr[i + 1] < m->row_ptr[i]) return fail(BSA_ERR_INVALID_MASK, "row_ptr decreases at %lld", (long long)i);
        if (m->row_ptr[nl] > (1ll << 31) - 1) return fail(BSA_ERR_UNSUPPORTED, "more than 2^31 - 1 slice keys");
        std::atomic<int64_t> bad{-1};
        parallel_for((nl + 1023) / 1024, [&](int64_t c) {
            for (int64_t i = c * 1024; i < std::min(nl, c * 1024 + 1024); ++i)
                for (int64_t e = m->row_ptr[i]; e < m->row_ptr[i + 1]; ++e) {
                    int32_t k = m->col_idx[e];
                    if (k < 0 || k >= L || (e > m->row_ptr[i] && k <= m->col_idx[e - 1])) {
                        int64_t x = -1;
                        bad.compare_exchange_strong(x, i);
                        return;
                    }
                }
        });
        if (bad.load() >= 0)
            return fail(BSA_ERR_INVALID_MASK, "slice list %lld is not strictly increasing within [0, L)", (long long)bad.load());
        return BSA_OK;
    }
    case BSA_MASK_VIDEO:
        if (!m->head_pattern) return fail(BSA_ERR_INVALID_ARGUMENT, "video head_pattern is NULL");
        if (bq != 1 || bk != 1) return fail(BSA_ERR_INVALID_ARGUMENT, "video masks need block 1 x 1 (got %d x %d)", bq, bk);
        if (!has_geo) return fail(BSA_ERR_INVALID_ARGUMENT, "video masks need the geometry T, Hg, Wg");
        for (int h = 0; h < H; ++h)
            if (m->head_pattern[h] > BSA_PAT_TEMPORAL)
                return fail(BSA_ERR_INVALID_MASK, "head_pattern[%d] = %d", h, m->head_pattern[h]);
        if (m->anchor_frame < 0 || m->anchor_frame >= o.T) return fail(BSA_ERR_INVALID_MASK, "anchor frame %d outside [0, %d)", m->anchor_frame, o.T);
        if (m->radius < 0 || m->radius > 256) return fail(BSA_ERR_INVALID_MASK, "radius %d outside [0, 256]", m->radius);
        return BSA_OK;
    default:
        return fail(BSA_ERR_INVALID_ARGUMENT, "unknown mask kind %d", m->kind);
    }
}

// ---------------------------------------------------------------------------
// regime selection
// ---------------------------------------------------------------------------

// Mask features for the regime lookup (Tessera, arXiv 2609.25869, abstract:
// the physical tiles that suit a mask depend on its shape, and the regime is
// looked up from offline profiling at low cost):
//  - density: kept logical blocks over all blocks (slices: listed keys over
//    all (query block, key) pairs);
//  - fill: kept pairs over the pairs of the non-empty 128 x 64 physical tiles
//    (regime 0's tiling), i.e. the share of computed pairs that are kept.
//    Banded and windowed layouts fill their tiles (near 1); a random layout
//    of blocks smaller than the tile leaves most of each non-empty tile
//    masked (about density / (1 - (1 - density)^k) for k blocks per tile),
//    where 64-row tiles waste less;
//  - fill2: the same over 256 x 64 tiles (the 8-wave regime's tiling). It is
//    at most fill, and near it where the two 128-row halves of a 256-row tile
//    keep the same key tiles (banded, windowed and frame-aligned video
//    layouts); a random layout of 128-row blocks fills 128-row tiles and
//    leaves half of each 256-row tile masked.
// BLOCK features come from a fixed sample: every kFeatureStride-th 128-row
// query tile of every head (all of them when a head has fewer tiles) for
// density and fill, and the 256-row tiles that start at those rows for fill2,
// read as keep-bit words, so the cost is a fraction of one mapping pass and
// the result is a deterministic function of the mask.
struct MaskFeatures {
    double density = -1.0;
    double fill = -1.0;
    double fill2 = -1.0;
};
constexpr int64_t kFeatureStride = 4;

static MaskFeatures mask_features(const bsa_mask_desc_t &m, int32_t B, int32_t H, int64_t L, int32_t bq, int32_t bk)
{
    MaskFeatures f;
    if (m.kind == BSA_MASK_SLICE_CSR) {
        const int64_t nl = (int64_t)B * H * ((L + bq - 1) / bq);
        f.density = (double)(m.nnz ? m.nnz : m.row_ptr[nl]) / ((double)nl * (double)L);
        return f;
    }
    if (m.kind == BSA_MASK_VIDEO) return f;
    const int64_t nqb = (L + bq - 1) / bq, nkb = (L + bk - 1) / bk;
    const int64_t nqt = (L + 127) / 128, nkt = (L + kTileK - 1) / kTileK;
    const int64_t words = (nkb + 63) / 64, twords = (nkt + 63) / 64;
    const int64_t stride = nqt >= 4 * kFeatureStride ? kFeatureStride : 1;
    const int64_t nqt2 = (L + 255) / 256, stride2 = stride == 1 ? 1 : stride / 2;
    const int64_t heads = (int64_t)B * H;
    const int64_t last_w = L - (nkb - 1) * bk;  // width of the (cropped) last key block
    struct Acc {
        int64_t blocks = 0, kept = 0;
        double kept_pairs = 0.0, exec_pairs = 0.0, kept_pairs2 = 0.0, exec_pairs2 = 0.0;
    };
    std::vector<Acc> acc((size_t)heads);
    parallel_for(heads, [&](int64_t bh) {
        std::vector<uint64_t> rowbuf((size_t)words), uni((size_t)words), uni2((size_t)words), tiles((size_t)twords);
        Acc a;
        // the non-empty 64-key tiles of a union of keep-bit rows
        auto count_tiles = [&](const std::vector<uint64_t> &u) -> int64_t {
            int64_t nt = 0;
            if (bk == 32 || bk == 64) {
                // a tile holds two key blocks (bit pairs) or one (bits)
                for (int64_t w = 0; w < words; ++w)
                    nt += __builtin_popcountll(bk == 64 ? u[w] : (u[w] | (u[w] >> 1)) & 0x5555555555555555ull);
                return nt;
            }
            if (bk % kTileK == 0) {
                // a block covers bk / 64 whole tiles; the last block only those before L
                for (int64_t w = 0; w < words; ++w) nt += __builtin_popcountll(u[w]);
                nt *= bk / kTileK;
                if ((u[(nkb - 1) >> 6] >> ((nkb - 1) & 63)) & 1)
                    nt -= bk / kTileK - (last_w + kTileK - 1) / kTileK;
                return nt;
            }
            std::fill(tiles.begin(), tiles.end(), 0ull);
            for (int64_t w = 0; w < words; ++w)
                for (uint64_t x = u[w]; x; x &= x - 1) {
                    const int64_t kb = w * 64 + __builtin_ctzll(x);
                    const int64_t k_lo = kb * bk, k_hi = std::min<int64_t>(k_lo + bk, L) - 1;
                    for (int64_t tk = k_lo / kTileK; tk <= k_hi / kTileK; ++tk) tiles[tk >> 6] |= 1ull << (tk & 63);
                }
            for (int64_t w = 0; w < twords; ++w) nt += __builtin_popcountll(tiles[w]);
            return nt;
        };
        // 256-row tile t2 = 128-row tiles 2 t2 and 2 t2 + 1; the first (both
        // when every 128-row tile is sampled) is also a density / fill sample
        for (int64_t t2 = 0; t2 < nqt2; t2 += stride2) {
            std::fill(uni2.begin(), uni2.end(), 0ull);
            for (int64_t tq = 2 * t2; tq < std::min<int64_t>(2 * t2 + 2, nqt); ++tq) {
                const bool sampled = tq == 2 * t2 || stride == 1;
                const int64_t q0 = tq * 128, q1 = std::min<int64_t>(q0 + 128, L);
                std::fill(uni.begin(), uni.end(), 0ull);
                for (int64_t qb = q0 / bq; qb <= (q1 - 1) / bq; ++qb) {
                    const uint64_t *row = block_row_bits(m, bh, qb, nqb, nkb, rowbuf.data());
                    int64_t k = 0;
                    for (int64_t w = 0; w < words; ++w) {
                        k += __builtin_popcountll(row[w]);
                        uni[w] |= row[w];
                    }
                    const bool last = (row[words - 1] >> ((nkb - 1) & 63)) & 1;
                    const int64_t r_in = std::min<int64_t>(q1, (qb + 1) * bq) - std::max<int64_t>(q0, qb * bq);
                    const double kp = (double)r_in * (double)(k * bk - (last ? bk - last_w : 0));
                    a.kept_pairs2 += kp;
                    if (sampled) {
                        a.kept_pairs += kp;
                        a.kept += k;
                        a.blocks += nkb;
                    }
                }
                for (int64_t w = 0; w < words; ++w) uni2[w] |= uni[w];
                if (sampled) a.exec_pairs += (double)count_tiles(uni) * (double)(q1 - q0) * (double)kTileK;
            }
            const int64_t r2 = std::min<int64_t>(256 * t2 + 256, L) - 256 * t2;
            a.exec_pairs2 += (double)count_tiles(uni2) * (double)r2 * (double)kTileK;
        }
        acc[bh] = a;
    });
    Acc t;
    for (const Acc &a : acc) {
        t.blocks += a.blocks;
        t.kept += a.kept;
        t.kept_pairs += a.kept_pairs;
        t.exec_pairs += a.exec_pairs;
        t.kept_pairs2 += a.kept_pairs2;
        t.exec_pairs2 += a.exec_pairs2;
    }
    f.density = t.blocks ? (double)t.kept / (double)t.blocks : 0.0;
    f.fill = t.exec_pairs > 0 ? std::min(1.0, t.kept_pairs / t.exec_pairs) : 1.0;
    f.fill2 = t.exec_pairs2 > 0 ? std::min(1.0, t.kept_pairs2 / t.exec_pairs2) : 1.0;
    return f;
}

static int32_t choose_regime(const bsa_mask_desc_t &m, int32_t B, int32_t H, int64_t L, int32_t bq, int32_t bk,
                             const bsa_plan_opts_t &o, int *regime, int *order, bool density_known = true,
                             MaskFeatures *feat_out = nullptr)
{
    *order = BSA_ORDER_XCD_GROUPED;
    if (o.force_regime >= 0 && o.task_order >= 0) {
        *regime = o.force_regime;
    } else {
        // the compiled-in table is parsed once; a table file on every call
        static const std::vector<LutRule> default_rules = [] {
            std::vector<LutRule> r;
            std::string e;
            if (!parse_lut(kDefaultLut, r, e)) r.clear();
            return r;
        }();
        std::vector<LutRule> file_rules;
        const std::vector<LutRule> *rules_p = &default_rules;
        if (o.lut_path) {
            std::ifstream f(o.lut_path);
            if (!f) return fail(BSA_ERR_INVALID_ARGUMENT, "cannot read lookup table %s", o.lut_path);
            std::stringstream ss;
            ss << f.rdbuf();
            std::string err;
            if (!parse_lut(ss.str(), file_rules, err)) return fail(BSA_ERR_INVALID_ARGUMENT, "%s", err.c_str());
            rules_p = &file_rules;
        }
        const std::vector<LutRule> &rules = *rules_p;
        const int kind = m.kind == BSA_MASK_BLOCK_BITS ? BSA_MASK_BLOCK_U8 : m.kind;
        const MaskFeatures feat = density_known ? mask_features(m, B, H, L, bq, bk) : MaskFeatures{};
        if (feat_out) *feat_out = feat;
        const double dens = feat.density, fill = feat.fill, fill2 = feat.fill2;
        *regime = -1;
        for (const LutRule &r : rules) {
            if (r.kind != kind) continue;
            if (r.bq && r.bq != bq) continue;
            if (r.bk && r.bk != bk) continue;
            // features not known (a mask in device memory): only a rule that
            // holds for every density and fill applies, not the first bin's
            if (!density_known &&
                (r.dlo > 0.0 || r.dhi < 1.0 || r.flo > 0.0 || r.fhi < 1.0 || r.f2lo > 0.0 || r.f2hi < 1.0))
                continue;
            if (dens >= 0 && (dens < r.dlo || dens > r.dhi)) continue;
            if (fill >= 0 && (fill < r.flo || fill > r.fhi)) continue;
            if (fill2 >= 0 && (fill2 < r.f2lo || fill2 > r.f2hi)) continue;
            if (L < r.Llo || L > r.Lhi) continue;
            *regime = r.regime;
            *order = r.order;
            break;
        }
        if (*regime < 0) *regime = m.kind == BSA_MASK_SLICE_CSR ? (bq == 128 ? 3 : 2) : 0;
        if (o.force_regime >= 0) *regime = o.force_regime;
    }
    if (o.task_order >= 0) *order = o.task_order;
    const Regime &R = kRegimes[*regime];
    const bool slice = m.kind == BSA_MASK_SLICE_CSR;
    if (slice != (R.family == 1))
        return fail(BSA_ERR_UNSUPPORTED, "regime %d (%s) cannot run %s masks", *regime, R.family ? "gather" : "tile",
                    slice ? "slice" : "block/video");
    if (slice && R.tile_q != bq) return fail(BSA_ERR_UNSUPPORTED, "gather regime %d has %d-query tiles, mask has M = %d", *regime, R.tile_q, bq);
    return BSA_OK;
}

// ---------------------------------------------------------------------------
// plan memory: pools and the per-device upload stream
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kPoolCap = (size_t)1 << 30;  // cached bytes per pool

BlockPool &pinned_pool()
{
    static BlockPool *pool = new BlockPool(
        [](size_t n) -> void * {
            void *p = nullptr;
            return hipHostMalloc(&p, n, hipHostMallocDefault) == hipSuccess ? p : nullptr;
        },
        [](void *p) { (void)hipHostFree(p); }, kPoolCap);
    return *pool;
}

struct DeviceRt {
    hipStream_t upload = nullptr;  // non-blocking: uploads never wait for other streams' work
    std::unique_ptr<BlockPool> pool;
};

// Per-device runtime, created on first use (the caller has the device current).
DeviceRt *device_rt(int dev, std::string &err)
{
    static std::mutex mu;
    static std::map<int, DeviceRt *> rts;
    std::lock_guard<std::mutex> g(mu);
    auto it = rts.find(dev);
    if (it != rts.end()) return it->second;
    DeviceRt *rt = new DeviceRt;
    hipError_t e = hipStreamCreateWithFlags(&rt->upload, hipStreamNonBlocking);
    if (e != hipSuccess) {
        err = std::string("hipStreamCreateWithFlags: ") + hipGetErrorString(e);
        delete rt;
        return nullptr;
    }
    rt->pool.reset(new BlockPool(
        [dev](size_t n) -> void * {
            int cur = 0;
            (void)hipGetDevice(&cur);
            (void)hipSetDevice(dev);
            void *p = nullptr;
            hipError_t e2 = hipMalloc(&p, n);
            (void)hipSetDevice(cur);
            return e2 == hipSuccess ? p : nullptr;
        },
        [dev](void *p) {
            int cur = 0;
            (void)hipGetDevice(&cur);
            (void)hipSetDevice(dev);
            (void)hipFree(p);
            (void)hipSetDevice(cur);
        },
        kPoolCap));
    rts[dev] = rt;
    return rt;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// ---------------------------------------------------------------------------
// task organisation
// ---------------------------------------------------------------------------

// One task per (batch, head, query tile) -- also for query tiles without any
// key tile, so that every output row is written; workgroup i of the launch
// runs task i. The heads' outputs are copied in parallel into the plan image,
// then ordered for the device: longest first (a stable counting sort on the
// tile count, so that the tail of the launch holds the cheapest work) and, by
// default, grouped for the XCDs (below).
static int xcd_count()
{
    if (const char *e = std::getenv("BSA_XCDS")) return std::max(1, std::atoi(e));
    return 8;
}

// XCD grouping of a longest-first order. The order is cut into runs of
// tasks of similar cost (tile counts within a factor kCostClass); inside a
// run the tasks are put back in (head, query tile) order, split into X equal
// segments, and interleaved: slot s + X i + x of the run takes task i of
// segment x (the remainder of an uneven split forms the run's last, partial
// round). Workgroup j of a launch goes to XCD j mod X, so every segment --
// neighbouring query tiles of a head, which share most of their key tiles --
// runs on one XCD and shares its L2, while at every point of the launch all
// XCDs are handed tasks of the same cost, as in the plain longest-first
// order (the hardware hands workgroups to the XCDs in turn, so an XCD that
// is handed longer tasks than the others would hold them up).
constexpr double kCostClass = 1.3;

static void group_for_xcds(Task *tasks, int64_t n, int X, int32_t max_cost)
{
    std::vector<int> cls_of((size_t)max_cost + 1, -1);  // cost class of each tile count
    for (int32_t c = 1; c <= max_cost; ++c) cls_of[(size_t)c] = (int)(std::log((double)c) / std::log(kCostClass));
    auto cls = [&](const Task &t) { return cls_of[(size_t)std::max(0, t.te - t.tb)]; };
    std::vector<Task> run;
    for (int64_t a = 0; a < n;) {
        int64_t b = a + 1;
        while (b < n && cls(tasks[b]) == cls(tasks[a])) ++b;
        run.assign(tasks + a, tasks + b);
        std::stable_sort(run.begin(), run.end(),
                         [](const Task &u, const Task &v) { return u.bh != v.bh ? u.bh < v.bh : u.q0 < v.q0; });
        const int64_t m = b - a, q = m / X;
        int64_t pos = a;
        for (int64_t i = 0; i < q; ++i)
            for (int x = 0; x < X; ++x) tasks[pos++] = run[(size_t)(x * q + i)];
        for (int64_t k = X * q; k < m; ++k) tasks[pos++] = run[(size_t)k];
        a = b;
    }
}

static int32_t organise_tasks(bsa_plan_s &p, const std::vector<HeadOut *> &heads, const std::vector<int32_t> &head_bh)
{
    const size_t nh = heads.size();
    std::vector<int64_t> t_off(nh + 1, 0), r_off(nh + 1, 0), g_off(nh + 1, 0);
    int32_t max_cost = 0;
    for (size_t i = 0; i < nh; ++i) {
        const HeadOut &h = *heads[i];
        t_off[i + 1] = t_off[i] + (int64_t)h.tasks.size();
        r_off[i + 1] = r_off[i] + (int64_t)h.tiles.size();
        g_off[i + 1] = g_off[i] + (int64_t)h.gidx.size();
        p.tiles_full += h.full;
        p.tiles_partial += h.part;
        p.tiles_empty += h.empty;
        p.gather_rows += h.grows;
        for (const Task &t : h.tasks) max_cost = std::max(max_cost, t.te - t.tb);
    }
    const int64_t nreal = t_off[nh];
    p.ntiles = r_off[nh];
    p.ngidx = g_off[nh];
    p.ntasks = nreal;
    p.nreal_tasks = nreal;
    p.off_tasks = 0;
    p.off_tiles = align_up(std::max<int64_t>(1, p.ntasks) * sizeof(Task));
    p.off_gidx = p.off_tiles + align_up(std::max<int64_t>(1, p.ntiles) * sizeof(TileRec));
    p.off_flags = p.off_gidx + align_up(std::max<int64_t>(1, p.ngidx) * sizeof(int32_t));
    p.off_coords = p.off_flags + align_up((size_t)p.H * sizeof(uint32_t));
    // video masks: one key-coordinate table per (pattern, layout) pair the heads use
    int ntables = 0;
    int table_of[3][2] = {{-1, -1}, {-1, -1}, {-1, -1}};
    p.head_coord_table.assign(p.H, 0);
    if (p.mode == kModeVideo) {
        p.coord_stride = (p.L + kTileK - 1) / kTileK * kTileK;
        for (int h = 0; h < p.H; ++h) {
            int &t = table_of[p.head_pattern[h]][p.head_layout[h] ? 1 : 0];
            if (t < 0) t = ntables++;
            p.head_coord_table[h] = (uint8_t)t;
        }
    }
    p.img_bytes = p.off_coords + align_up((size_t)std::max(1, ntables) * (size_t)std::max<int64_t>(1, p.coord_stride) * sizeof(int32_t));
    if (p.device >= 0) {
        p.img = (uint8_t *)pinned_pool().acquire(p.img_bytes, &p.img_cap);
        if (!p.img) return fail(BSA_ERR_OUT_OF_MEMORY, "pinned host allocation of %zu bytes failed", p.img_bytes);
        p.img_pinned = true;
    } else {
        p.img_host.reset(new uint8_t[p.img_bytes]);
        p.img_host_n = p.img_bytes;
        p.img = p.img_host.get();
        p.img_cap = p.img_bytes;
    }
    // tiles and gather indices, per head in parallel; tasks unsorted into a scratch list
    std::vector<Task> unsorted((size_t)nreal);
    TileRec *tiles = (TileRec *)(p.img + p.off_tiles);
    int32_t *gidx = (int32_t *)(p.img + p.off_gidx);
    const bool gather = p.mode == kModeGather;
    parallel_for((int64_t)nh, [&](int64_t i) {
        const HeadOut &h = *heads[i];
        const int32_t toff = (int32_t)r_off[i], goff = (int32_t)g_off[i];
        Task *td = unsorted.data() + t_off[i];
        for (size_t k = 0; k < h.tasks.size(); ++k) {
            Task t = h.tasks[k];
            t.bh = head_bh[i];  // (a head may share its mapping with another)
            t.tb += toff;
            t.te += toff;
            td[k] = t;
        }
        TileRec *rd = tiles + r_off[i];
        if (gather) {
            for (size_t k = 0; k < h.tiles.size(); ++k) rd[k] = {h.tiles[k].k0 + goff, h.tiles[k].aux};
        } else if (!h.tiles.empty()) {
            std::memcpy(rd, h.tiles.data(), h.tiles.size() * sizeof(TileRec));
        }
        if (!h.gidx.empty()) std::memcpy(gidx + g_off[i], h.gidx.data(), h.gidx.size() * sizeof(int32_t));
    });
    Task *tasks = (Task *)(p.img + p.off_tasks);
    // longest first: a stable counting sort on the tile count, descending
    std::vector<int64_t> bucket((size_t)max_cost + 2, 0);
    for (const Task &t : unsorted) ++bucket[(size_t)(max_cost - (t.te - t.tb)) + 1];
    for (size_t c = 1; c < bucket.size(); ++c) bucket[c] += bucket[c - 1];
    for (const Task &t : unsorted) tasks[bucket[(size_t)(max_cost - (t.te - t.tb))]++] = t;
    if (p.task_order == BSA_ORDER_XCD_GROUPED) group_for_xcds(tasks, nreal, xcd_count(), max_cost);
    uint32_t *flags = (uint32_t *)(p.img + p.off_flags);
    for (int h = 0; h < p.H; ++h)
        flags[h] = (p.head_layout[h] ? kHeadTemporalMajor : 0u) | ((uint32_t)p.head_pattern[h] << kHeadPatShift) |
                   ((uint32_t)p.head_coord_table[h] << kHeadCoordShift);
    // Key-coordinate word of each logical position of a head, as the exact
    // video predicates compare it (Sparse VideoGen / Splash Attention summary,
    // "Splash Attention": coordinate masking on boundary tiles): the frame
    // (spatial pattern) or (y << 16) | x (temporal pattern) of the position's
    // token; positions past the sequence end hold a word no predicate keeps.
    if (p.mode == kModeVideo) {
        int32_t *coords = (int32_t *)(p.img + p.off_coords);
        for (int pat = 0; pat < 3; ++pat)
            for (int lay = 0; lay < 2; ++lay) {
                if (table_of[pat][lay] < 0) continue;
                int32_t *c = coords + table_of[pat][lay] * p.coord_stride;
                // chunks of positions in parallel; inside a chunk, running
                // coordinates (no divisions)
                constexpr int64_t kChunk = 4096;
                parallel_for((p.L + kChunk - 1) / kChunk, [&, pat, lay, c](int64_t ci) {
                    const int64_t k0 = ci * kChunk, k1 = std::min<int64_t>(p.L, k0 + kChunk);
                    const int64_t HWp = (int64_t)p.Hg * p.Wg;
                    int32_t t, y, x;
                    if (lay) {
                        t = (int32_t)(k0 % p.T);
                        const int64_t px = k0 / p.T;
                        y = (int32_t)(px / p.Wg);
                        x = (int32_t)(px % p.Wg);
                    } else {
                        t = (int32_t)(k0 / HWp);
                        y = (int32_t)((k0 % HWp) / p.Wg);
                        x = (int32_t)(k0 % p.Wg);
                    }
                    for (int64_t k = k0; k < k1; ++k) {
                        c[k] = pat == BSA_PAT_SPATIAL ? t : (pat == BSA_PAT_TEMPORAL ? ((y << 16) | x) : 0);
                        if (lay) {  // j = pixel * T + frame: frame first, then the pixel
                            if (++t == p.T) { t = 0; if (++x == p.Wg) { x = 0; ++y; } }
                        } else {    // token = frame * HW + y * Wg + x
                            if (++x == p.Wg) { x = 0; if (++y == p.Hg) { y = 0; ++t; } }
                        }
                    }
                });
                for (int64_t k = p.L; k < p.coord_stride; ++k) c[k] = 0x7FFF7FFF;
            }
    }
    return BSA_OK;
}

// ---------------------------------------------------------------------------
// device upload (asynchronous, on the device's upload stream)
// ---------------------------------------------------------------------------

// The plan's two events: its upload (or device planning) has run; its last
// enqueued forward has run. On failure neither is left set.
static hipError_t create_plan_events(bsa_plan_s *p)
{
    hipError_t e = hipEventCreateWithFlags(&p->uploaded, hipEventDisableTiming);
    if (e != hipSuccess) {
        p->uploaded = nullptr;
        return e;
    }
    e = hipEventCreateWithFlags(&p->last_use, hipEventDisableTiming);
    if (e != hipSuccess) {
        p->last_use = nullptr;
        (void)hipEventDestroy(p->uploaded);
        p->uploaded = nullptr;
    }
    return e;
}

static int32_t upload(bsa_plan_s &p)
{
    if (p.device < 0) return BSA_OK;
    int cur = 0;
    (void)hipGetDevice(&cur);
    hipError_t e = hipSetDevice(p.device);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "hipSetDevice(%d): %s", p.device, hipGetErrorString(e));
    std::string err;
    DeviceRt *rt = device_rt(p.device, err);
    int32_t st = BSA_OK;
    if (!rt) {
        st = fail(BSA_ERR_HIP, "%s", err.c_str());
    } else if (!(p.dev = rt->pool->acquire(p.img_bytes, &p.dev_cap))) {
        st = fail(BSA_ERR_OUT_OF_MEMORY, "device allocation of %zu bytes failed", p.img_bytes);
    } else if ((e = create_plan_events(&p)) != hipSuccess) {
        st = fail(BSA_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
    } else if ((e = hipMemcpyAsync(p.dev, p.img, p.img_bytes, hipMemcpyHostToDevice, rt->upload)) != hipSuccess ||
               (e = hipEventRecord(p.uploaded, rt->upload)) != hipSuccess) {
        st = fail(BSA_ERR_HIP, "plan upload: %s", hipGetErrorString(e));
    }
    (void)hipSetDevice(cur);
    return st;
}

// Give the plan's memory back to the pools (after its upload has completed).
static void release_plan_memory(bsa_plan_s *p)
{
    if (p->last_use) {
        // the forwards enqueued on this plan have finished reading it
        if (p->used) (void)hipEventSynchronize(p->last_use);
        (void)hipEventDestroy(p->last_use);
        p->last_use = nullptr;
    }
    if (p->uploaded) {
        (void)hipEventSynchronize(p->uploaded);
        (void)hipEventDestroy(p->uploaded);
        p->uploaded = nullptr;
    }
    if (p->dev) {
        std::string err;
        if (DeviceRt *rt = device_rt(p->device, err)) rt->pool->release(p->dev, p->dev_cap);
        p->dev = nullptr;
    }
    if (p->img && p->img_pinned) pinned_pool().release(p->img, p->img_cap);
    p->img = nullptr;
    if (p->small) pinned_pool().release(p->small, p->small_cap);
    p->small = nullptr;
}

// Reused per-head mapping buffers (their capacity survives across plans).
namespace {
struct Builder {
    std::vector<HeadOut> heads;
};
std::mutex g_builder_mu;
std::vector<Builder *> g_builders;

Builder *take_builder()
{
    std::lock_guard<std::mutex> g(g_builder_mu);
    if (g_builders.empty()) return new Builder;
    Builder *b = g_builders.back();
    g_builders.pop_back();
    return b;
}

void give_builder(Builder *b)
{
    std::lock_guard<std::mutex> g(g_builder_mu);
    g_builders.push_back(b);
}
}  // namespace

// ---------------------------------------------------------------------------
// C entry points
// ---------------------------------------------------------------------------

extern "C" void bsa_plan_opts_default(bsa_plan_opts_t *o)
{
    if (!o) return;
    std::memset(o, 0, sizeof *o);
    o->dtype = BSA_DTYPE_BF16;
    o->force_regime = -1;
    o->device = 0;
    o->task_order = -1;
}

extern "C" int32_t bsa_plan(const bsa_mask_desc_t *logical_mask, int32_t B, int32_t H, int64_t L, int32_t d,
                            int32_t block_q, int32_t block_k, const bsa_plan_opts_t *opts, bsa_plan_t *out_plan)
{
    if (!out_plan) return fail(BSA_ERR_INVALID_ARGUMENT, "out_plan is NULL");
    *out_plan = nullptr;
    const auto t_start = std::chrono::steady_clock::now();
    auto now_ns = [&] {
        return (int64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t_start).count();
    };
    int64_t t_ingest = 0, t_regime = 0, t_map = 0, t_tasks = 0;
    try {
        bsa_plan_opts_t o;
        bsa_plan_opts_default(&o);
        if (opts) o = *opts;
        int32_t st = validate(logical_mask, B, H, L, d, block_q, block_k, o);
        if (st != BSA_OK) return st;
        t_ingest = now_ns();
        if (std::getenv("BSA_TEST_FAIL_ALLOC")) return fail(BSA_ERR_OUT_OF_MEMORY, "simulated allocation failure");
        const bsa_mask_desc_t &m = *logical_mask;
        int regime = 0, order = 0;
        MaskFeatures feat;
        st = choose_regime(m, B, H, L, block_q, block_k, o, &regime, &order, true, &feat);
        if (st != BSA_OK) return st;
        t_regime = now_ns();

        std::unique_ptr<bsa_plan_s> p(new bsa_plan_s);
        p->mask_density = feat.density;
        p->mask_fill = feat.fill;
        p->mask_fill2 = feat.fill2;
        p->B = B; p->H = H; p->L = L; p->d = d; p->dtype = o.dtype;
        p->kind = m.kind; p->block_q = block_q; p->block_k = block_k;
        p->regime = regime;
        p->T = o.T; p->Hg = o.Hg; p->Wg = o.Wg;
        p->anchor = m.anchor_frame; p->radius = m.radius;
        p->device = o.device;
        p->task_order = order;
        p->head_layout.assign(H, 0);
        if (o.head_layout) p->head_layout.assign(o.head_layout, o.head_layout + H);
        p->head_pattern.assign(H, 0);
        if (m.kind == BSA_MASK_VIDEO) p->head_pattern.assign(m.head_pattern, m.head_pattern + H);
        const Regime &R = kRegimes[regime];
        p->mode = m.kind == BSA_MASK_VIDEO ? kModeVideo : (m.kind == BSA_MASK_SLICE_CSR ? kModeGather : kModeBlock);
        if (p->mode == kModeBlock) {
            p->sub_q = std::min(block_q, R.tile_q);
            p->sub_k = std::min(block_k, kTileK);
            p->bq_shift = ilog2(p->sub_q);
            p->bk_shift = ilog2(p->sub_k);
            p->nsk = kTileK / p->sub_k;
        }
        Builder *builder = take_builder();
        std::unique_ptr<Builder, void (*)(Builder *)> builder_guard(builder, give_builder);
        std::vector<HeadOut> &heads = builder->heads;
        if (heads.size() < (size_t)B * H) heads.resize((size_t)B * H);
        // Heads with identical logical masks share one mapping: video heads of
        // one pattern and layout (in every batch), and BLOCK heads whose mask
        // bytes equal the previous head's (a mask broadcast over heads). Only
        // the first of each group is mapped; the task array takes the others'
        // tasks and tiles from it.
        const int64_t NBH = (int64_t)B * H;
        std::vector<int64_t> src((size_t)NBH);
        const int64_t nqb_m = (L + block_q - 1) / block_q, nkb_m = (L + block_k - 1) / block_k;
        const size_t head_bytes = m.kind == BSA_MASK_BLOCK_U8 ? (size_t)(nqb_m * nkb_m)
                                  : m.kind == BSA_MASK_BLOCK_BITS ? (size_t)(nqb_m * ((nkb_m + 63) / 64)) * 8 : 0;
        // BLOCK: each head's mask bytes against the previous head's, in parallel
        // (a small-block mask holds megabytes per head)
        std::vector<uint8_t> same_as_prev((size_t)NBH, 0);
        if (p->mode == kModeBlock && NBH > 1) {
            const uint8_t *d = (const uint8_t *)m.data;
            parallel_for(NBH - 1, [&](int64_t i) {
                const int64_t bh = i + 1;
                same_as_prev[(size_t)bh] = std::memcmp(d + (size_t)(bh - 1) * head_bytes, d + (size_t)bh * head_bytes, head_bytes) == 0;
            });
        }
        for (int64_t bh = 0; bh < NBH; ++bh) {
            src[(size_t)bh] = bh;
            if (p->mode == kModeVideo) {
                const int h = (int)(bh % H);
                for (int64_t o = 0; o < bh; ++o) {
                    const int ho = (int)(o % H);
                    if (src[(size_t)o] == o && p->head_pattern[ho] == p->head_pattern[h] && p->head_layout[ho] == p->head_layout[h]) {
                        src[(size_t)bh] = o;
                        break;
                    }
                }
            } else if (p->mode == kModeBlock && same_as_prev[(size_t)bh]) {
                src[(size_t)bh] = src[(size_t)(bh - 1)];
            }
        }
        // work items: chunks of kMapChunk query tiles of the heads to map, so
        // that a few distinct heads still spread over all worker threads
        constexpr int64_t kMapChunk = 16;
        const int64_t nqt = p->mode == kModeGather ? (L + block_q - 1) / block_q : (L + R.tile_q - 1) / R.tile_q;
        const int64_t per_head = (nqt + kMapChunk - 1) / kMapChunk;
        std::vector<int64_t> first_item((size_t)NBH, -1);
        int64_t nitems = 0;
        for (int64_t bh = 0; bh < NBH; ++bh)
            if (src[(size_t)bh] == bh) { first_item[(size_t)bh] = nitems; nitems += per_head; }
        if (heads.size() < (size_t)nitems) heads.resize((size_t)nitems);
        std::vector<int64_t> item_head((size_t)nitems);
        for (int64_t bh = 0; bh < NBH; ++bh)
            for (int64_t c = 0; first_item[(size_t)bh] >= 0 && c < per_head; ++c) item_head[(size_t)(first_item[(size_t)bh] + c)] = bh;
        parallel_for(nitems, [&](int64_t it) {
            HeadOut &out = heads[(size_t)it];
            out.clear();
            const int64_t bh = item_head[(size_t)it], c = it - first_item[(size_t)bh];
            const int64_t lo = c * kMapChunk, hi = std::min(nqt, lo + kMapChunk);
            const int b = (int)(bh / H), h = (int)(bh % H);
            if (p->mode == kModeBlock) map_block_head(*p, m, b, h, R.tile_q, lo, hi, out);
            else if (p->mode == kModeVideo) map_video_head(*p, b, h, R.tile_q, lo, hi, out);
            else map_slice_head(*p, m, b, h, lo, hi, out);
        });
        size_t total_tiles = 0;
        for (int64_t i = 0; i < NBH; ++i)
            for (int64_t c = 0; c < per_head; ++c) total_tiles += heads[(size_t)(first_item[(size_t)src[(size_t)i]] + c)].tiles.size();
        if (total_tiles >= (size_t)INT32_MAX) return fail(BSA_ERR_UNSUPPORTED, "plan has more than 2^31 tiles");
        t_map = now_ns();
        // the task array takes every head's chunks in (head, query tile) order
        std::vector<HeadOut *> hp;
        std::vector<int32_t> hp_bh;
        hp.reserve((size_t)(NBH * per_head));
        hp_bh.reserve((size_t)(NBH * per_head));
        for (int64_t i = 0; i < NBH; ++i)
            for (int64_t c = 0; c < per_head; ++c) {
                hp.push_back(&heads[(size_t)(first_item[(size_t)src[(size_t)i]] + c)]);
                hp_bh.push_back((int32_t)i);
            }
        st = organise_tasks(*p, hp, hp_bh);
        t_tasks = now_ns();
        if (st == BSA_OK) st = upload(*p);
        if (st != BSA_OK) {
            release_plan_memory(p.get());
            return st;
        }
        p->plan_ns = now_ns();
        const int64_t marks[6] = {0, t_ingest, t_regime, t_map, t_tasks, p->plan_ns};
        for (int i = 0; i < 5; ++i) p->phase_ns[i] = marks[i + 1] - marks[i];
        if (const char *lg = std::getenv("BSA_LOG"); lg && std::atoi(lg) >= 1)
            std::fprintf(stderr, "[bsa] plan %.3f ms: ingest %.3f, regime %.3f (r%d), mapping %.3f, tasks %.3f, upload %.3f; "
                                 "tiles full %lld partial %lld empty %lld\n",
                         p->plan_ns * 1e-6, p->phase_ns[0] * 1e-6, p->phase_ns[1] * 1e-6, p->regime, p->phase_ns[2] * 1e-6,
                         p->phase_ns[3] * 1e-6, p->phase_ns[4] * 1e-6, (long long)p->tiles_full,
                         (long long)p->tiles_partial, (long long)p->tiles_empty);
        *out_plan = p.release();
        return BSA_OK;
    } catch (const std::bad_alloc &) {
        return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation failed while planning");
    } catch (const std::exception &ex) {
        return fail(BSA_ERR_INTERNAL, "%s", ex.what());
    }
}

// ---------------------------------------------------------------------------
// device-side planning (BLOCK masks in device memory)
// ---------------------------------------------------------------------------

extern "C" int32_t bsa_plan_device(const bsa_mask_desc_t *logical_mask, int32_t B, int32_t H, int64_t L, int32_t d,
                                   int32_t block_q, int32_t block_k, const bsa_plan_opts_t *opts, void *stream,
                                   bsa_plan_t *out_plan)
{
    if (!out_plan) return fail(BSA_ERR_INVALID_ARGUMENT, "out_plan is NULL");
    *out_plan = nullptr;
    const auto t_start = std::chrono::steady_clock::now();
    try {
        bsa_plan_opts_t o;
        bsa_plan_opts_default(&o);
        if (opts) o = *opts;
        if (!logical_mask) return fail(BSA_ERR_INVALID_ARGUMENT, "logical_mask is NULL");
        const bool slice = logical_mask->kind == BSA_MASK_SLICE_CSR;
        if (logical_mask->kind != BSA_MASK_BLOCK_U8 && logical_mask->kind != BSA_MASK_BLOCK_BITS && !slice)
            return fail(BSA_ERR_UNSUPPORTED, "device planning takes BLOCK and SLICE masks (kind %d)", logical_mask->kind);
        if (o.device < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "device planning needs a device (opts.device = %d)", o.device);
        int32_t st = validate(logical_mask, B, H, L, d, block_q, block_k, o, true);
        if (st != BSA_OK) return st;
        const bsa_mask_desc_t &m = *logical_mask;
        int regime = 0, order = 0;
        // a slice mask's density is nnz / (lists * L): known without reading it
        MaskFeatures feat;
        st = choose_regime(m, B, H, L, block_q, block_k, o, &regime, &order, slice, &feat);
        if (st != BSA_OK) return st;
        const Regime &R = kRegimes[regime];

        std::unique_ptr<bsa_plan_s> p(new bsa_plan_s);
        p->mask_density = feat.density;
        p->mask_fill = feat.fill;
        p->mask_fill2 = feat.fill2;
        p->B = B; p->H = H; p->L = L; p->d = d; p->dtype = o.dtype;
        p->kind = m.kind; p->block_q = block_q; p->block_k = block_k;
        p->regime = regime;
        p->T = o.T; p->Hg = o.Hg; p->Wg = o.Wg;
        p->device = o.device;
        p->task_order = order;
        p->head_layout.assign(H, 0);
        if (o.head_layout) p->head_layout.assign(o.head_layout, o.head_layout + H);
        p->head_pattern.assign(H, 0);
        p->mode = slice ? kModeGather : kModeBlock;
        if (!slice) {
            p->sub_q = std::min(block_q, R.tile_q);
            p->sub_k = std::min(block_k, kTileK);
            p->bq_shift = ilog2(p->sub_q);
            p->bk_shift = ilog2(p->sub_k);
            p->nsk = kTileK / p->sub_k;
        }
        p->gather_rows = p->ngidx = slice ? m.nnz : 0;
        p->device_planned = true;

        const int64_t nqt = (L + R.tile_q - 1) / R.tile_q, nkt = (L + kTileK - 1) / kTileK;
        const int64_t NT = (int64_t)B * H * nqt, cap = NT * nkt;
        if (cap >= (int64_t)INT32_MAX) return fail(BSA_ERR_UNSUPPORTED, "device plan capacity above 2^31 tiles");
        if (NT >= ((int64_t)1 << 24)) return fail(BSA_ERR_UNSUPPORTED, "device planning of more than 2^24 tasks");
        p->ntasks = p->nreal_tasks = NT;
        p->ntiles = -1;  // known once read back

        // cost classes of tile counts: the same table as the host's XCD grouping;
        // plain longest first is the class = count case on one XCD
        const bool grouped = order == BSA_ORDER_XCD_GROUPED;
        const int64_t nchunks = (NT + kDevPlanChunk - 1) / kDevPlanChunk;
        const size_t small_bytes = (size_t)H * sizeof(uint32_t) + (size_t)(nkt + 1) * sizeof(int32_t);
        p->small = (uint8_t *)pinned_pool().acquire(small_bytes, &p->small_cap);
        if (!p->small) return fail(BSA_ERR_OUT_OF_MEMORY, "pinned host allocation of %zu bytes failed", small_bytes);
        uint32_t *flags = (uint32_t *)p->small;
        for (int h = 0; h < H; ++h) flags[h] = p->head_layout[h] ? kHeadTemporalMajor : 0u;
        int32_t *cls_of = (int32_t *)(p->small + (size_t)H * sizeof(uint32_t));
        cls_of[0] = -1;
        int32_t nclass = 0;
        for (int64_t c = 1; c <= nkt; ++c) {
            cls_of[c] = grouped ? (int32_t)(std::log((double)c) / std::log(kCostClass)) : (int32_t)c;
            nclass = std::max(nclass, cls_of[c] + 1);
        }
        const int32_t nkeys = nclass + 1;
        if (nkeys > kDevPlanMaxKeys) {
            release_plan_memory(p.get());
            return fail(BSA_ERR_UNSUPPORTED, "device planning in longest-first order of more than %d key tiles",
                        kDevPlanMaxKeys - 2);
        }

        // device image: the host plan's sections (each task's tile records at
        // its worst-case size, task t's from record t * nkt), then the
        // planner's scratch
        p->off_tasks = 0;
        p->off_tiles = align_up((size_t)std::max<int64_t>(1, NT) * sizeof(Task));
        p->off_gidx = p->off_tiles + align_up((size_t)std::max<int64_t>(1, cap) * sizeof(TileRec));
        p->off_flags = p->off_gidx + align_up((size_t)std::max<int64_t>(1, p->ngidx) * sizeof(int32_t));
        p->off_coords = p->off_flags + align_up((size_t)H * sizeof(uint32_t));
        const size_t off_cnt = p->off_coords + align_up(sizeof(int32_t));
        const size_t off_full = off_cnt + align_up((size_t)NT * sizeof(int32_t));
        const size_t off_errs = off_full + align_up((size_t)NT * sizeof(int32_t));
        const size_t off_hist = off_errs + align_up((size_t)NT * sizeof(int32_t));
        const size_t off_csum = off_hist + align_up((size_t)(nkeys * nchunks + 1) * sizeof(int32_t));
        const size_t off_cls = off_csum + align_up((size_t)nchunks * 3 * sizeof(int64_t));
        p->off_stats = off_cls + align_up((size_t)(nkt + 1) * sizeof(int32_t));
        p->img_bytes = p->off_stats + align_up(4 * sizeof(int64_t));

        int cur = 0;
        (void)hipGetDevice(&cur);
        hipError_t e = hipSetDevice(p->device);
        if (e != hipSuccess) return fail(BSA_ERR_HIP, "hipSetDevice(%d): %s", p->device, hipGetErrorString(e));
        std::string err;
        DeviceRt *rt = device_rt(p->device, err);
        if (!rt) st = fail(BSA_ERR_HIP, "%s", err.c_str());
        else if (!(p->dev = rt->pool->acquire(p->img_bytes, &p->dev_cap)))
            st = fail(BSA_ERR_OUT_OF_MEMORY, "device allocation of %zu bytes failed", p->img_bytes);
        else if ((e = create_plan_events(p.get())) != hipSuccess)
            st = fail(BSA_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
        if (st == BSA_OK) {
            uint8_t *dv = (uint8_t *)p->dev;
            const hipStream_t s = (hipStream_t)stream;
            DevPlanArgs a{};
            a.u8 = m.kind == BSA_MASK_BLOCK_U8 ? (const uint8_t *)m.data : nullptr;
            a.bits = m.kind == BSA_MASK_BLOCK_BITS ? (const uint64_t *)m.data : nullptr;
            if (slice) {
                a.row_ptr = m.row_ptr;
                a.col_idx = m.col_idx;
                a.nnz = m.nnz;
                a.gidx = (int32_t *)(dv + p->off_gidx);
                a.errs = (int32_t *)(dv + off_errs);
            }
            a.L = L;
            a.BQ = R.tile_q;
            a.bq = block_q;
            a.bk = block_k;
            a.bqe = p->sub_q;
            a.bke = p->sub_k;
            a.nsq = slice ? 0 : R.tile_q / p->sub_q;
            a.nsk = p->nsk;
            a.lbq = ilog2(block_q);
            a.lbk = ilog2(block_k);
            a.lbqe = p->bq_shift;
            a.lbke = p->bk_shift;
            a.nqb = (L + block_q - 1) / block_q;
            a.nkb = (L + block_k - 1) / block_k;
            a.words = (a.nkb + 63) / 64;
            a.nqt = nqt;
            a.nkt = nkt;
            a.ntasks = NT;
            a.nchunks = nchunks;
            a.cnt = (int32_t *)(dv + off_cnt);
            a.full = (int32_t *)(dv + off_full);
            a.hist = (int32_t *)(dv + off_hist);
            a.csum = (int64_t *)(dv + off_csum);
            a.tasks = (Task *)(dv + p->off_tasks);
            a.tiles = (TileRec *)(dv + p->off_tiles);
            a.cls_of = (const int32_t *)(dv + off_cls);
            a.nclass = nclass;
            a.nkeys = nkeys;
            a.X = grouped ? xcd_count() : 1;
            a.stats = (int64_t *)(dv + p->off_stats);
            if ((e = hipMemcpyAsync(dv + p->off_flags, flags, (size_t)H * sizeof(uint32_t), hipMemcpyHostToDevice, s)) != hipSuccess ||
                (e = hipMemcpyAsync(dv + off_cls, cls_of, (size_t)(nkt + 1) * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess ||
                (e = launch_device_plan(a, s)) != hipSuccess || (e = hipEventRecord(p->uploaded, s)) != hipSuccess)
                st = fail(BSA_ERR_HIP, "device planning: %s", hipGetErrorString(e));
        }
        (void)hipSetDevice(cur);
        if (st != BSA_OK) {
            release_plan_memory(p.get());
            return st;
        }
        p->plan_ns = (int64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t_start).count();
        *out_plan = p.release();
        return BSA_OK;
    } catch (const std::bad_alloc &) {
        return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation failed while planning");
    } catch (const std::exception &ex) {
        return fail(BSA_ERR_INTERNAL, "%s", ex.what());
    }
}

// Host view of a device-built plan: waits for the planning kernels, then
// reads back the statistics and, with `image`, the task and record sections.
static int32_t read_back_device_plan(bsa_plan_s *p, bool image)
{
    if (!p->device_planned || (p->stats_read && (!image || p->host_copy))) return BSA_OK;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(p->device);
    hipError_t e = hipEventSynchronize(p->uploaded);
    if (e == hipSuccess && !p->stats_read) {
        int64_t stats[4] = {0, 0, 0, 0};
        e = hipMemcpy(stats, (uint8_t *)p->dev + p->off_stats, sizeof stats, hipMemcpyDeviceToHost);
        if (e == hipSuccess) {
            p->ntiles = stats[0];
            p->tiles_full = stats[1];
            p->tiles_partial = stats[0] - stats[1];
            p->tiles_empty = stats[2];
            p->mask_errors = stats[3];
            p->stats_read = true;
        }
    }
    if (e == hipSuccess && image && !p->host_copy) {
        // tasks and records, and the gathered keys of a slice plan
        const size_t n = p->mode == kModeGather ? p->off_flags : p->off_gidx;
        p->img_host.reset(new uint8_t[std::max<size_t>(n, 1)]);
        p->img_host_n = n;
        e = hipMemcpy(p->img_host.get(), p->dev, n, hipMemcpyDeviceToHost);
        if (e == hipSuccess) {
            p->img = p->img_host.get();
            p->img_cap = n;
            p->host_copy = true;
        }
    }
    (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "reading back a device plan: %s", hipGetErrorString(e));
    return BSA_OK;
}

extern "C" void bsa_plan_destroy(bsa_plan_t p)
{
    if (!p) return;
    release_plan_memory(p);
    delete p;
}

// Division by a runtime constant d in [1, 2^30] for numerators 0 <= n < 2^31:
// n / d == (umulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (round-up multiplier; the sum cannot
// overflow 32 bits because umulhi(n, m) < n).
static void magic_div(uint32_t d, uint32_t *m, int32_t *s)
{
    int l = 0;
    while ((1ull << l) < d) ++l;
    *m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    *s = l;
}

static int32_t forward_impl(bsa_plan_t p, const void *Q, const void *K, const void *V, void *O, uint64_t *stamps,
                            void *stream)
{
    if (!p) return fail(BSA_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (p->device < 0 || !p->dev) return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built host-only (device = -1)");
    if (!Q || !K || !V || !O) return fail(BSA_ERR_INVALID_ARGUMENT, "Q, K, V and O must be non-NULL device pointers");
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15)
        return fail(BSA_ERR_INVALID_ARGUMENT, "Q, K, V and O must be 16-byte aligned");
    if (p->ntasks == 0) return BSA_OK;
    KernelArgs a{};
    a.Q = Q; a.K = K; a.V = V; a.O = O;
    const uint8_t *dev = (const uint8_t *)p->dev;
    a.tasks = (const Task *)(dev + p->off_tasks);
    a.tiles = (const TileRec *)(dev + p->off_tiles);
    a.gidx = (const int32_t *)(dev + p->off_gidx);
    a.head_flags = (const uint32_t *)(dev + p->off_flags);
    a.coords = (const int32_t *)(dev + p->off_coords);
    a.coords_stride = (int32_t)p->coord_stride;
    a.ntasks = (int32_t)p->ntasks;
    a.H = p->H;
    a.L = (int32_t)p->L;
    a.T = p->T; a.HW = p->Hg * p->Wg; a.W = p->Wg;
    magic_div((uint32_t)std::max(a.T, 1), &a.magic_T, &a.shift_T);
    magic_div((uint32_t)std::max(a.HW, 1), &a.magic_HW, &a.shift_HW);
    magic_div((uint32_t)std::max(a.W, 1), &a.magic_W, &a.shift_W);
    a.anchor = p->anchor; a.radius = p->radius;
    a.mode = p->mode;
    a.bq_shift = p->bq_shift; a.bk_shift = p->bk_shift; a.nsk = p->nsk;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->d));
    a.stamps = stamps;
    int cur = 0;
    (void)hipGetDevice(&cur);
    if (cur != p->device) (void)hipSetDevice(p->device);
    // the launch is ordered after the plan's upload; once the upload is seen
    // complete, no wait goes into the stream any more
    hipError_t e = hipSuccess;
    if (!p->upload_seen.load(std::memory_order_acquire)) {
        e = hipEventQuery(p->uploaded);
        if (e == hipSuccess) p->upload_seen.store(true, std::memory_order_release);
        else if (e == hipErrorNotReady) e = hipStreamWaitEvent((hipStream_t)stream, p->uploaded, 0);
    }
    if (e == hipSuccess) {
        const Regime &R = kRegimes[p->regime];
        e = p->dtype == BSA_DTYPE_F32 ? launch_forward_f32(a, R.tile_q / 32, p->d, (hipStream_t)stream)
                                      : launch_forward(a, R.waves, R.rb, p->d, p->dtype, R.nbuf, (hipStream_t)stream);
    }
    if (e == hipSuccess) {
        // last_use completes after this forward and after every earlier one:
        // a forward on another stream than the previous one first makes the
        // record wait for the previous record (later work on this stream then
        // also waits for the other stream's forward of this plan)
        std::lock_guard<std::mutex> g(p->use_mu);
        const hipStream_t s = (hipStream_t)stream;
        if (p->used && s != p->last_stream) e = hipStreamWaitEvent(s, p->last_use, 0);
        if (e == hipSuccess) e = hipEventRecord(p->last_use, s);
        if (e == hipSuccess) {
            p->used = true;
            p->last_stream = s;
        }
    }
    if (cur != p->device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return BSA_OK;
}

extern "C" int32_t bsa_forward(bsa_plan_t p, const void *Q, const void *K, const void *V, void *O, void *stream)
{
    return forward_impl(p, Q, K, V, O, nullptr, stream);
}

extern "C" int32_t bsa_forward_stamped(bsa_plan_t p, const void *Q, const void *K, const void *V, void *O,
                                       uint64_t *stamps, void *stream)
{
    if (!stamps || ((uintptr_t)stamps & 7)) return fail(BSA_ERR_INVALID_ARGUMENT, "stamps must be an 8-byte aligned device pointer");
    if (p && p->dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_UNSUPPORTED, "clock stamps are written by the bf16 kernel only");
    return forward_impl(p, Q, K, V, O, stamps, stream);
}

extern "C" int32_t bsa_plan_info(bsa_plan_t p, bsa_plan_info_t *out)
{
    if (!p || !out) return fail(BSA_ERR_INVALID_ARGUMENT, "plan or out is NULL");
    if (int32_t st = read_back_device_plan(p, false); st != BSA_OK) return st;
    const Regime &R = kRegimes[p->regime];
    out->regime = p->regime;
    out->tile_q = R.tile_q;
    out->tile_k = kTileK;
    out->gather = R.family;
    out->tasks = p->nreal_tasks;
    out->workgroups = p->ntasks;
    out->tiles_full = p->tiles_full;
    out->tiles_partial = p->tiles_partial;
    out->tiles_empty = p->tiles_empty;
    out->gather_rows = p->gather_rows;
    out->executed_pairs = (double)(p->tiles_full + p->tiles_partial) * R.tile_q * kTileK;
    out->device_bytes = (int64_t)p->dev_cap;
    out->plan_ns = p->plan_ns;
    for (int i = 0; i < 5; ++i) out->phase_ns[i] = p->phase_ns[i];
    out->task_order = p->task_order;
    out->mask_density = p->mask_density;
    out->mask_fill = p->mask_fill;
    out->mask_fill2 = p->mask_fill2;
    if (p->mask_errors)
        return fail(BSA_ERR_INVALID_MASK, "the device mask had %lld invalid slice entries or lists (clamped or dropped)",
                    (long long)p->mask_errors);
    return BSA_OK;
}

extern "C" int32_t bsa_plan_coverage(bsa_plan_t p, int32_t b, int32_t h, bsa_cov_sink_t sink, void *user)
{
    if (!p || !sink) return fail(BSA_ERR_INVALID_ARGUMENT, "plan or sink is NULL");
    if (b < 0 || b >= p->B || h < 0 || h >= p->H) return fail(BSA_ERR_INVALID_ARGUMENT, "head (%d, %d) out of range", b, h);
    if (int32_t st = read_back_device_plan(p, true); st != BSA_OK) return st;
    const Regime &R = kRegimes[p->regime];
    const int32_t bh = b * p->H + h;
    const Task *tasks = p->tasks();
    const TileRec *tiles = p->tiles();
    for (int64_t ti = 0; ti < p->ntasks; ++ti) {
        const Task &t = tasks[ti];
        if (t.bh != bh) continue;
        for (int32_t i = t.tb; i < t.te; ++i) {
            const TileRec &r = tiles[i];
            bsa_tile_record_t rec{};
            rec.task = ti;
            rec.q0 = t.q0;
            rec.q1 = std::min<int64_t>(t.q0 + R.tile_q, p->L);
            rec.kind = (r.aux & kPartial) ? BSA_TILE_PARTIAL : BSA_TILE_FULL;
            if (p->mode == kModeGather) {
                rec.predicate = BSA_PRED_LIST;
                rec.keys = p->gidx() + r.k0;
                rec.nkeys = r.aux & kAuxMask;
            } else {
                rec.predicate = p->mode == kModeBlock ? BSA_PRED_SUBBLOCK : BSA_PRED_VIDEO;
                rec.k0 = r.k0;
                rec.k1 = std::min<int64_t>((int64_t)r.k0 + kTileK, p->L);
                rec.sub_bits = r.aux & kAuxMask;
                rec.sub_q = p->sub_q;
                rec.sub_k = p->sub_k;
            }
            if (p->mode == kModeVideo && (r.aux & kPartial)) {
                // one record per wave that runs the tile: FULL or PARTIAL rows
                rec.sub_bits = 0;
                const int64_t tq1 = rec.q1;
                for (int wv = 0; wv < R.tile_q / kWaveRows; ++wv) {
                    rec.q0 = t.q0 + (int64_t)kWaveRows * wv;
                    rec.q1 = std::min<int64_t>(rec.q0 + kWaveRows, tq1);
                    if (rec.q0 >= rec.q1 || ((r.aux >> wv) & 1u)) continue;
                    rec.kind = ((r.aux >> (kWaveFullShift + wv)) & 1u) ? BSA_TILE_FULL : BSA_TILE_PARTIAL;
                    if (sink(user, &rec)) return BSA_OK;
                }
                continue;
            }
            if (sink(user, &rec)) return BSA_OK;
        }
    }
    return BSA_OK;
}

// ---------------------------------------------------------------------------
// requests: plan + forward over a sequence of masks, pipelined
// ---------------------------------------------------------------------------

struct bsa_request_s {
    bsa_request_desc_t desc{};
    std::vector<uint8_t> head_layout;  // owned copies of the option pointers
    std::string lut_path;
    struct Slot {
        bsa_plan_t plan = nullptr;
        hipEvent_t done = nullptr;  // recorded after the plan's forward
    };
    std::vector<Slot> ring;  // circular, `depth` slots
    int64_t oldest = 0, inflight = 0;
    bsa_request_stats_t stats{};
};

namespace {

struct DeviceScope {
    int prev = 0;
    explicit DeviceScope(int dev)
    {
        (void)hipGetDevice(&prev);
        if (prev != dev) (void)hipSetDevice(dev);
    }
    ~DeviceScope() { (void)hipSetDevice(prev); }
};

// Wait for the oldest in-flight forward, then destroy its plan.
int32_t retire_oldest(bsa_request_s *r)
{
    bsa_request_s::Slot &s = r->ring[(size_t)(r->oldest % r->desc.depth)];
    hipError_t e;
    {
        DeviceScope ds(r->desc.opts.device);
        e = hipEventSynchronize(s.done);
    }
    bsa_plan_destroy(s.plan);
    s.plan = nullptr;
    ++r->oldest;
    --r->inflight;
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "waiting for a request's forward: %s", hipGetErrorString(e));
    return BSA_OK;
}

}  // namespace

extern "C" int32_t bsa_request_create(const bsa_request_desc_t *desc, bsa_request_t *out)
{
    if (!out) return fail(BSA_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    if (!desc) return fail(BSA_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (desc->depth < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "request depth %d (at least 1)", desc->depth);
    if (desc->opts.device < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "a request runs forwards: opts.device must be a device");
    if (desc->B < 1 || desc->H < 1 || desc->L < 1 || (desc->d != 64 && desc->d != 128))
        return fail(BSA_ERR_INVALID_ARGUMENT, "request shape B=%d H=%d L=%lld d=%d", desc->B, desc->H, (long long)desc->L,
                    desc->d);
    try {
        std::unique_ptr<bsa_request_s> r(new bsa_request_s);
        r->desc = *desc;
        if (desc->opts.head_layout) {
            r->head_layout.assign(desc->opts.head_layout, desc->opts.head_layout + desc->H);
            r->desc.opts.head_layout = r->head_layout.data();
        }
        if (desc->opts.lut_path) {
            r->lut_path = desc->opts.lut_path;
            r->desc.opts.lut_path = r->lut_path.c_str();
        }
        r->ring.resize((size_t)desc->depth);
        DeviceScope ds(desc->opts.device);
        for (auto &s : r->ring) {
            const hipError_t e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
            if (e != hipSuccess) {
                s.done = nullptr;
                for (auto &t : r->ring)
                    if (t.done) (void)hipEventDestroy(t.done);
                return fail(BSA_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
            }
        }
        *out = r.release();
        return BSA_OK;
    } catch (const std::bad_alloc &) {
        return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
}

extern "C" int32_t bsa_request_submit(bsa_request_t r, const bsa_mask_desc_t *mask, int32_t block_q, int32_t block_k,
                                      int32_t mask_on_device, const void *Q, const void *K, const void *V, void *O)
{
    if (!r || !mask) return fail(BSA_ERR_INVALID_ARGUMENT, "request or mask is NULL");
    const bsa_request_desc_t &d = r->desc;
    const auto t0 = std::chrono::steady_clock::now();
    if (r->inflight >= d.depth)
        if (int32_t st = retire_oldest(r); st != BSA_OK) return st;
    const auto t1 = std::chrono::steady_clock::now();
    bsa_plan_t p = nullptr;
    int32_t st = mask_on_device
                     ? bsa_plan_device(mask, d.B, d.H, d.L, d.d, block_q, block_k, &d.opts,
                                       d.plan_stream ? d.plan_stream : d.stream, &p)
                     : bsa_plan(mask, d.B, d.H, d.L, d.d, block_q, block_k, &d.opts, &p);
    const auto t2 = std::chrono::steady_clock::now();
    r->stats.wait_ns += (int64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(t1 - t0).count();
    r->stats.plan_ns += (int64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(t2 - t1).count();
    if (st != BSA_OK) return st;
    st = bsa_forward(p, Q, K, V, O, d.stream);
    if (st != BSA_OK) {
        bsa_plan_destroy(p);  // nothing of it was launched
        return st;
    }
    bsa_request_s::Slot &s = r->ring[(size_t)((r->oldest + r->inflight) % d.depth)];
    hipError_t e;
    {
        DeviceScope ds(d.opts.device);
        e = hipEventRecord(s.done, (hipStream_t)d.stream);
        if (e != hipSuccess) (void)hipStreamSynchronize((hipStream_t)d.stream);
    }
    if (e != hipSuccess) {
        bsa_plan_destroy(p);
        return fail(BSA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
    }
    s.plan = p;
    ++r->inflight;
    ++r->stats.submitted;
    return BSA_OK;
}

extern "C" int32_t bsa_request_finish(bsa_request_t r)
{
    if (!r) return fail(BSA_ERR_INVALID_ARGUMENT, "request is NULL");
    int32_t first = BSA_OK;
    while (r->inflight > 0) {
        const int32_t st = retire_oldest(r);
        if (first == BSA_OK) first = st;
    }
    return first;
}

extern "C" int32_t bsa_request_stats(bsa_request_t r, bsa_request_stats_t *out)
{
    if (!r || !out) return fail(BSA_ERR_INVALID_ARGUMENT, "request or out is NULL");
    *out = r->stats;
    return BSA_OK;
}

extern "C" void bsa_request_destroy(bsa_request_t r)
{
    if (!r) return;
    (void)bsa_request_finish(r);
    {
        DeviceScope ds(r->desc.opts.device);
        for (auto &s : r->ring)
            if (s.done) (void)hipEventDestroy(s.done);
    }
    delete r;
}

// ---------------------------------------------------------------------------
// head routing probe
// ---------------------------------------------------------------------------

// probe workgroups per call, read from BSA_PROBE_WGS when set (a tuning knob)
static int64_t probe_workgroups()
{
    const char *e = std::getenv("BSA_PROBE_WGS");
    return e ? std::max(1, std::atoi(e)) : 256;
}

// Argument checks shared by both routing entry points.
static int32_t check_route_args(const void *Q, const void *K, const void *V, int32_t B, int32_t H, int64_t L,
                                int32_t d, const bsa_route_desc_t *desc, const uint8_t *head_pattern)
{
    if (!Q || !K || !V || !desc || !head_pattern || !desc->rows)
        return fail(BSA_ERR_INVALID_ARGUMENT, "Q, K, V, desc, desc->rows and head_pattern must be non-NULL");
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V) & 15)
        return fail(BSA_ERR_INVALID_ARGUMENT, "Q, K and V must be 16-byte aligned");
    const bsa_route_desc_t &r = *desc;
    if (B < 1 || H < 1 || L < 1 || L >= ((int64_t)1 << 31) || (d != 64 && d != 128))
        return fail(BSA_ERR_INVALID_ARGUMENT, "routing shape B=%d H=%d L=%lld d=%d", B, H, (long long)L, d);
    if (r.T < 1 || r.Hg < 1 || r.Wg < 1 || r.Hg >= 32768 || r.Wg >= 32768 || (int64_t)r.T * r.Hg * r.Wg != L)
        return fail(BSA_ERR_INVALID_ARGUMENT, "geometry T=%d Hg=%d Wg=%d does not give L=%lld", r.T, r.Hg, r.Wg,
                    (long long)L);
    if (r.anchor_frame < 0 || r.anchor_frame >= r.T || r.radius < 0 || r.radius > 256)
        return fail(BSA_ERR_INVALID_ARGUMENT, "anchor frame %d / radius %d out of range", r.anchor_frame, r.radius);
    if (r.n_rows < 1 || r.n_rows > 4096) return fail(BSA_ERR_INVALID_ARGUMENT, "n_rows %d (1 .. 4096)", r.n_rows);
    for (int32_t i = 0; i < r.n_rows; ++i)
        if (r.rows[i] < 0 || r.rows[i] >= L) return fail(BSA_ERR_INVALID_ARGUMENT, "row %d = %d out of range", i, r.rows[i]);
    if (r.device < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "routing needs a device (desc->device = %d)", r.device);
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || r.device >= ndev)
        return fail(BSA_ERR_INVALID_ARGUMENT, "device %d does not exist (%d devices)", r.device, ndev);
    return BSA_OK;
}

// The probe's arguments other than its device buffers (rows, part, err_rows).
static RouteArgs route_args(const void *Q, const void *K, const void *V, int32_t B, int32_t H, int64_t L, int32_t d,
                            const bsa_route_desc_t &r, int32_t nchunk)
{
    RouteArgs a{};
    a.Q = Q; a.K = K; a.V = V;
    a.BH = B * H;
    a.L = (int32_t)L;
    a.HW = r.Hg * r.Wg;
    a.W = r.Wg;
    a.anchor = r.anchor_frame;
    a.radius = r.radius;
    magic_div((uint32_t)a.HW, &a.magic_HW, &a.shift_HW);
    magic_div((uint32_t)a.W, &a.magic_W, &a.shift_W);
    a.S = r.n_rows;
    a.nsb = (r.n_rows + 31) / 32;
    a.nkt = (int32_t)((L + kTileK - 1) / kTileK);
    a.nchunk = nchunk;
    a.tiles_per_chunk = (a.nkt + nchunk - 1) / nchunk;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    return a;
}

// Key chunks of the probe: about probe_workgroups() workgroups of six waves
// (two blocks of 32 sampled rows x three variants), at most one per key tile.
static int32_t route_chunks(int32_t BH, int32_t S, int64_t L)
{
    const int32_t nsb = (S + 31) / 32;
    const int64_t nkt = (L + kTileK - 1) / kTileK;
    const int64_t units = (int64_t)BH * ((nsb + 1) / 2);
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(nkt, probe_workgroups() / units));
}

extern "C" int32_t bsa_route_heads(const void *Q, const void *K, const void *V, int32_t B, int32_t H, int64_t L,
                                   int32_t d, const bsa_route_desc_t *desc, void *stream, uint8_t *head_pattern,
                                   double *err)
{
    if (int32_t st = check_route_args(Q, K, V, B, H, L, d, desc, head_pattern); st != BSA_OK) return st;
    const bsa_route_desc_t &r = *desc;
    try {
        const int32_t BH = B * H, S = r.n_rows, nsb = (S + 31) / 32;
        const int32_t nchunk = route_chunks(BH, S, L);
        const size_t part_floats = (size_t)BH * nsb * nchunk * 3 * (64 + 32 * (size_t)d);
        const size_t off_rows = 0;
        const size_t off_err = align_up((size_t)S * sizeof(int32_t));
        const size_t off_part = off_err + align_up((size_t)BH * S * 2 * sizeof(float));
        const size_t bytes = off_part + part_floats * sizeof(float);
        const size_t host_bytes = align_up((size_t)S * sizeof(int32_t)) + (size_t)BH * S * 2 * sizeof(float);

        DeviceScope ds(r.device);
        std::string e_str;
        DeviceRt *rt = device_rt(r.device, e_str);
        if (!rt) return fail(BSA_ERR_HIP, "%s", e_str.c_str());
        size_t dev_cap = 0, host_cap = 0;
        uint8_t *dev = (uint8_t *)rt->pool->acquire(bytes, &dev_cap);
        if (!dev) return fail(BSA_ERR_OUT_OF_MEMORY, "device allocation of %zu bytes failed", bytes);
        uint8_t *host = (uint8_t *)pinned_pool().acquire(host_bytes, &host_cap);
        if (!host) {
            rt->pool->release(dev, dev_cap);
            return fail(BSA_ERR_OUT_OF_MEMORY, "pinned host allocation of %zu bytes failed", host_bytes);
        }
        std::memcpy(host, r.rows, (size_t)S * sizeof(int32_t));
        float *err_host = (float *)(host + align_up((size_t)S * sizeof(int32_t)));

        RouteArgs a = route_args(Q, K, V, B, H, L, d, r, nchunk);
        a.rows = (const int32_t *)(dev + off_rows);
        a.part = (float *)(dev + off_part);
        a.err_rows = (float *)(dev + off_err);
        const hipStream_t s = (hipStream_t)stream;
        hipEvent_t done = nullptr;
        hipError_t e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
        if (e == hipSuccess) e = hipMemcpyAsync(dev + off_rows, host, (size_t)S * sizeof(int32_t), hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = launch_route_probe(a, d, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(err_host, dev + off_err, (size_t)BH * S * 2 * sizeof(float), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipEventRecord(done, s);
        if (e == hipSuccess) e = hipEventSynchronize(done);
        else (void)hipStreamSynchronize(s);  // nothing may still use the scratch memory
        if (done) (void)hipEventDestroy(done);
        int32_t st = BSA_OK;
        if (e != hipSuccess) {
            st = fail(BSA_ERR_HIP, "routing probe: %s", hipGetErrorString(e));
        } else {
            // per head: mean over the batch, the sampled rows and the dims
            for (int h = 0; h < H; ++h) {
                double es = 0.0, et = 0.0;
                for (int b = 0; b < B; ++b)
                    for (int i = 0; i < S; ++i) {
                        const float *er = err_host + ((size_t)(b * H + h) * S + i) * 2;
                        es += er[0];
                        et += er[1];
                    }
                const double n = (double)B * S * d;
                es /= n;
                et /= n;
                head_pattern[h] = es <= et ? BSA_PAT_SPATIAL : BSA_PAT_TEMPORAL;
                if (err) {
                    err[2 * h] = es;
                    err[2 * h + 1] = et;
                }
            }
        }
        pinned_pool().release(host, host_cap);
        rt->pool->release(dev, dev_cap);
        return st;
    } catch (const std::bad_alloc &) {
        return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
}

// ---------------------------------------------------------------------------
// allocation-free head routing
// ---------------------------------------------------------------------------

// Scratch of bsa_route_heads_noalloc: a fixed array in each device's memory,
// held for the life of the process, shared by every call on that device. In
// host code `scratch` names a host-side stand-in: the array's device address
// comes from hipGetSymbolAddress (per device) and only that address is used.
constexpr size_t kRouteScratchBytes = (size_t)32 << 20;  // 32 MiB
constexpr int32_t kRouteMaxHeads = 1024;                 // B * H
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu[kMaxDevices];  // one routing call at a time per device
void *g_scratch_ptr[kMaxDevices];      // device address of `scratch`, per device (set once)

// The device address of this device's scratch array; called with the device
// current and g_scratch_mu[device] held.
hipError_t scratch_address(int device, uint8_t **out)
{
    if (!g_scratch_ptr[device]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = ptr;
    }
    *out = (uint8_t *)g_scratch_ptr[device];
    return hipSuccess;
}
}  // namespace

extern "C" int32_t bsa_route_heads_noalloc(const void *Q, const void *K, const void *V, int32_t B, int32_t H,
                                           int64_t L, int32_t d, const bsa_route_desc_t *desc, void *stream,
                                           uint8_t *head_pattern, double *err)
{
    if (int32_t st = check_route_args(Q, K, V, B, H, L, d, desc, head_pattern); st != BSA_OK) return st;
    const bsa_route_desc_t &r = *desc;
    if (r.device >= kMaxDevices) return fail(BSA_ERR_INVALID_ARGUMENT, "device %d (at most %d)", r.device, kMaxDevices - 1);
    if ((int64_t)B * H > kRouteMaxHeads)
        return fail(BSA_ERR_UNSUPPORTED, "B * H = %lld exceeds the allocation-free limit of %d heads", (long long)B * H,
                    kRouteMaxHeads);
    const int32_t BH = B * H, S = r.n_rows, nsb = (S + 31) / 32;
    // layout of the scratch: rows | per-row errors | per-head sums | partials
    const size_t off_err = align_up((size_t)S * sizeof(int32_t));
    const size_t off_sums = off_err + align_up((size_t)BH * S * 2 * sizeof(float));
    const size_t off_part = off_sums + align_up((size_t)H * 2 * sizeof(double));
    const size_t chunk_bytes = (size_t)BH * nsb * 3 * (64 + 32 * (size_t)d) * sizeof(float);
    if (off_part + chunk_bytes > kRouteScratchBytes)
        return fail(BSA_ERR_UNSUPPORTED, "routing %d heads x %d rows at d = %d needs %zu bytes of scratch, more than the "
                    "allocation-free limit of %zu", BH, S, d, off_part + chunk_bytes, kRouteScratchBytes);
    // as many key chunks as the scratch holds (fewer chunks: less parallelism, same result up to rounding)
    const int32_t nchunk = std::max<int32_t>(
        1, std::min<int32_t>(route_chunks(BH, S, L), (int32_t)((kRouteScratchBytes - off_part) / chunk_bytes)));

    std::lock_guard<std::mutex> lock(g_scratch_mu[r.device]);
    DeviceScope ds(r.device);
    uint8_t *dev = nullptr;
    hipError_t e = scratch_address(r.device, &dev);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    RouteArgs a = route_args(Q, K, V, B, H, L, d, r, nchunk);
    a.rows = (const int32_t *)dev;
    a.err_rows = (float *)(dev + off_err);
    a.part = (float *)(dev + off_part);
    double sums[2 * kRouteMaxHeads];
    const hipStream_t s = (hipStream_t)stream;
    // every scratch element the kernels read is written earlier in this call:
    // nothing needs clearing
    e = hipMemcpyAsync(dev, r.rows, (size_t)S * sizeof(int32_t), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_route_probe(a, d, s);
    if (e == hipSuccess) e = launch_route_head_sums(a.err_rows, B, H, S, (double *)(dev + off_sums), s);
    if (e == hipSuccess) e = hipMemcpyAsync(sums, dev + off_sums, (size_t)H * 2 * sizeof(double), hipMemcpyDeviceToHost, s);
    const hipError_t es = hipStreamSynchronize(s);  // the scratch and `sums` are free again after this
    if (e == hipSuccess) e = es;
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "routing probe: %s", hipGetErrorString(e));
    const double n = (double)B * S * d;
    for (int h = 0; h < H; ++h) {
        const double e_sp = sums[2 * h] / n, e_tp = sums[2 * h + 1] / n;
        head_pattern[h] = e_sp <= e_tp ? BSA_PAT_SPATIAL : BSA_PAT_TEMPORAL;
        if (err) {
            err[2 * h] = e_sp;
            err[2 * h + 1] = e_tp;
        }
    }
    return BSA_OK;
}
