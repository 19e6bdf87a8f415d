// Device plan format shared by the host planner and the gfx950 kernels.
//
// A plan is a list of workgroup tasks, one per (batch, head, query tile), and
// per task an ordered run of key-tile records. Empty (query tile, key tile)
// pairs never appear; a record is either FULL (every pair of the tile is
// kept: no mask work) or PARTIAL (the kernel evaluates the exact predicate on
// that tile only). This is the physical tile layer of Tessera (arXiv
// 2609.25869, abstract) with Splash Attention's empty-tile skipping and
// boundary-only exact masking (Sparse VideoGen / Splash Attention summary,
// "Splash Attention").
#pragma once
#include <cstdint>

namespace bsa {

constexpr int kTileK = 64;         // keys per physical key tile
constexpr uint32_t kPartial = 0x80000000u;
constexpr uint32_t kAuxMask = 0x0000FFFFu;
// Video PARTIAL tiles refine their class per wave (a wave owns kWaveRows
// consecutive query rows of the tile): aux bit w set = wave w keeps no pair
// of the tile and skips it; bit kWaveFullShift + w set = wave w keeps every
// pair of the tile and runs it without the mask.
constexpr int kWaveRows = 32;
constexpr int kWaveFullShift = 8;

// Which predicate PARTIAL tiles evaluate.
enum MaskMode : int32_t {
    kModeBlock = 0,   // sub-block keep bits of the record, plus key < L
    kModeVideo = 1,   // per-head spatial / temporal coordinate predicate, plus key < L
    kModeGather = 2,  // key slot < record count (gathered key lists)
};

// Per-head flags (kernel reads head_flags[h]).
constexpr uint32_t kHeadTemporalMajor = 1u;   // bit 0: logical j = p*T + t
constexpr uint32_t kHeadPatShift = 1;         // bits 1..2: video pattern
constexpr uint32_t kHeadCoordShift = 3;       // bits 3..4: video key-coordinate table of the head

struct Task {        // 16 bytes
    int32_t bh;      // b * H + h; -1 = no-op padding task
    int32_t q0;      // first logical query position of the tile
    int32_t tb, te;  // key-tile records [tb, te)
};

struct TileRec {     // 8 bytes
    int32_t k0;      // first logical key (tile families) or offset into gidx (gather)
    uint32_t aux;    // kPartial | sub-block bits (block) | valid count (gather) | per-wave bits (video)
};

struct KernelArgs {
    const void *Q, *K, *V;
    void *O;
    const Task *tasks;
    const TileRec *tiles;
    const int32_t *gidx;
    const uint32_t *head_flags;
    const int32_t *coords;     // video key-coordinate tables, coords_stride words each
    int32_t ntasks;
    int32_t coords_stride;     // padded to whole 64-key tiles
    int32_t H;
    int32_t L;
    int32_t T, HW, W;          // video geometry (0 if unused)
    uint32_t magic_T, magic_HW, magic_W;  // n / d == (umulhi(n, magic) + n) >> shift for 0 <= n < 2^31
    int32_t shift_T, shift_HW, shift_W;
    int32_t anchor, radius;
    int32_t mode;              // MaskMode
    int32_t bq_shift, bk_shift, nsk;  // block sub-block geometry (log2 sizes, sub-blocks per key tile)
    float scale_log2;          // log2(e) / sqrt(d)
    uint64_t *stamps;          // per-task clock stamps (instrumented launches), else null
};

}  // namespace bsa
