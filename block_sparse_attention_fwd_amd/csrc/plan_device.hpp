// Arguments of the device-side planning kernels (plan_device.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_format.hpp"

namespace bsa {

// Tasks per ordering workgroup, and the most sort keys (cost classes plus
// the class of tasks without tiles) the ordering kernels hold in LDS.
constexpr int kDevPlanChunk = 1024;
constexpr int kDevPlanMaxKeys = 8192;

struct DevPlanArgs {
    const uint8_t *u8;      // BLOCK_U8 mask [B][H][nqb][nkb] (device), or
    const uint64_t *bits;   // BLOCK_BITS mask [B][H][nqb][words] (device), or
    const int64_t *row_ptr; // SLICE_CSR lists [B*H*nqb + 1] and
    const int32_t *col_idx; // their keys [nnz] (device)
    int64_t nnz;
    int32_t *gidx;          // [nnz] the plan's copy of the slice keys (clamped into [0, L))
    int32_t *errs;          // [ntasks] slice entries found invalid per list
    int64_t L;
    int32_t BQ;             // physical query tile (rows per task)
    int32_t bq, bk;         // logical block shape
    int32_t bqe, bke;       // sub-block shape inside a tile: min(bq, BQ), min(bk, 64)
    int32_t nsq, nsk;       // sub-blocks per tile: BQ / bqe, 64 / bke
    int32_t lbq, lbk, lbqe, lbke;  // log2 of bq, bk, bqe, bke
    int64_t nqb, nkb, words;
    int64_t nqt, nkt;       // query tiles per head, key tiles per head
    int64_t ntasks;         // B * H * nqt, in (head, query tile) order
    int64_t nchunks;        // ceil(ntasks / kDevPlanChunk)
    int32_t *cnt;           // [ntasks] non-empty key tiles of each task
    int32_t *full;          // [ntasks] FULL key tiles of each task
    int32_t *hist;          // [nkeys * nchunks + 1] tasks per (key, chunk), then its exclusive prefix
    int64_t *csum;          // [nchunks][3] records, FULL records and invalid slice entries of each chunk
    Task *tasks;            // [ntasks] launch order
    TileRec *tiles;         // [ntasks][nkt]: the records of task t start at t * nkt
    const int32_t *cls_of;  // [nkt + 1] cost class of a tile count (-1 for 0)
    int32_t nclass;         // classes are 0 .. nclass - 1
    int32_t nkeys;          // nclass + 1: key nclass - 1 - class, tasks without tiles last
    int32_t X;              // XCDs the launch is dealt over
    int64_t *stats;         // [4] records, FULL records, empty (task, key tile) pairs, invalid slice entries
};

hipError_t launch_device_plan(const DevPlanArgs &a, hipStream_t stream);

}  // namespace bsa
