// Arguments of the head routing probe kernels (route_probe.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsa {

struct RouteArgs {
    const void *Q, *K, *V;    // bf16 [B][H][L][d], frame-major tokens
    int32_t BH, L;
    int32_t HW, W, anchor, radius;
    uint32_t magic_HW, magic_W;
    int32_t shift_HW, shift_W;
    const int32_t *rows;      // [S] sampled query tokens (device)
    int32_t S, nsb;           // samples, blocks of 32 samples
    int32_t nkt, nchunk, tiles_per_chunk;
    float scale_log2;         // log2(e) / sqrt(d)
    float *part;              // [BH * nsb][nchunk][3][64 + 32 d] partial softmax states
    float *err_rows;          // [BH][S][2] squared differences (spatial, temporal) per sampled row
};

hipError_t launch_route_probe(const RouteArgs &a, int d, hipStream_t stream);

// Per head h: sums[2 h] and sums[2 h + 1] = the spatial and temporal squared
// differences of err_rows summed over the batch and the sampled rows, in fp64
// and in the order b = 0..B-1, i = 0..S-1 (the order the host sums them in).
hipError_t launch_route_head_sums(const float *err_rows, int32_t B, int32_t H, int32_t S, double *sums,
                                  hipStream_t stream);

}  // namespace bsa
