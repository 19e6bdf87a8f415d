// gfx950 fp32 forward kernel of block-sparse attention (validation build).
//
// Same plans, same task/tile walk and the same exact predicates as the bf16
// kernel, with fp32 Q, K, V, O and fp32 MFMAs (v_mfma_f32_32x32x2_f32), and P
// kept in fp32. It exists to check the method's arithmetic at a precision
// where the remaining error is rounding of fp32 sums: its output agrees with
// an fp64 evaluation to ~1e-6 relative per row.
// Sums over tens of thousands of keys would lose that in fp32 alone (the
// rounding of a running sum grows with the square root of its length, to
// ~1e-5 at 20,000 keys), so each key tile's products and weights are summed
// in fp32 (the MFMA accumulates one tile, from zero) and the tile results are
// added in fp64: the output, the row sum and their rescaling run in double.
//
// Operand layout of v_mfma_f32_32x32x2_f32 (wave64): lane l supplies
// A[l % 32][l / 32] and B[l / 32][l % 32]; the 32x32 result uses the same
// register layout as the bf16 kernel's (key 8*(r/4) + 4*(l/32) + r%4 of the
// lane's query in register r).
//  - S^T = K Q^T: step kk contracts dims kdim(kk, 0) and kdim(kk, 1), one per
//    lane half, where kdim(kk, h) = kk % 32 + 32 h + 64 (kk / 32); any
//    bijection of the dims gives the same dot product, and this one puts the
//    two halves' LDS reads 32 banks apart.
//  - O^T += V^T P^T: step r contracts the two keys the lane halves hold in
//    score register r, so P feeds the MFMA straight from the registers.
// K rows are padded to D + 1 floats (consecutive keys one bank apart), V rows
// to D + 8 (rows 4 apart land 32 banks apart).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.hpp"

namespace bsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NW, int D>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void bsa_fwd_f32(KernelArgs a)
{
    constexpr int BK = kTileK;
    constexpr int KS = D + 1;  // K row stride in floats
    constexpr int VS = D + 8;  // V row stride in floats
    constexpr int NT = NW * 64;
    __shared__ float ksm[BK * KS];
    __shared__ __attribute__((aligned(16))) float vsm[BK * VS];
    __shared__ __attribute__((aligned(16))) int kcoord[BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Task task = a.tasks[blockIdx.x];
    if (task.bh < 0) return;
    const int bh = task.bh;
    const int h = bh % a.H;
    const uint32_t hflag = a.head_flags[h];
    const bool tm = (hflag & kHeadTemporalMajor) != 0;
    const int pat = (int)((hflag >> kHeadPatShift) & 3u);
    const int L = a.L;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    const float *Qh = (const float *)a.Q + head_off;
    const float *Kh = (const float *)a.K + head_off;
    const float *Vh = (const float *)a.V + head_off;
    float *Oh = (float *)a.O + head_off;
    const bool gather = a.mode == kModeGather;
    const bool video = a.mode == kModeVideo;

    int q[1], qt[1] = {0};
    unsigned qwin[1] = {0u};
    q[0] = task.q0 + 32 * w + l32;
    const bool qvalid = q[0] < L;
    const int qtok = head_token(qvalid ? q[0] : L - 1, tm, a);
    if (video) video_query_coords(qtok, a, qt[0], qwin[0]);

    double oacc[D / 32][16];  // output sums across tiles, fp64
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[n][r] = 0.0;
    float m_ref = -INFINITY;
    double l_run = 0.0;
    const int ntile = task.te - task.tb;

    if (ntile > 0) {
        // this lane's query row at the dims it contracts: kdim(kk, hf) for kk < D/2
        float qreg[D / 2];
#pragma unroll
        for (int c = 0; c < D / 64; ++c)
#pragma unroll
            for (int i = 0; i < 32; i += 4) {
                const f32x4 v = *(const f32x4 *)(Qh + (size_t)qtok * D + 64 * c + 32 * hf + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) qreg[32 * c + i + e] = v[e];
            }
        const f32x16 zero16 = {};

        RecordStream rs;
        rs.init(a.tiles, task.tb, task.te, lane);
        for (int j = 0; j < ntile; ++j) {
            if ((j & 63) == 0 && j > 0) rs.advance();
            const TileRec rec = rs.get(j);
            const int cnt = (int)(rec.aux & kAuxMask);
            __syncthreads();  // the previous tile's LDS readers are done
            // ---- K/V tile -> LDS (rows past the sequence / list end repeat a
            // valid row; their scores are masked)
            for (int idx = tid; idx < BK * D / 4; idx += NT) {
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                const int kpos = gather ? a.gidx[rec.k0 + (row < cnt ? row : cnt - 1)] : min(rec.k0 + row, L - 1);
                const size_t g = (size_t)head_token(kpos, tm, a) * D + 4 * c4;
                const f32x4 kv = *(const f32x4 *)(Kh + g);
                const f32x4 vv = *(const f32x4 *)(Vh + g);
#pragma unroll
                for (int e = 0; e < 4; ++e) ksm[row * KS + 4 * c4 + e] = kv[e];
                *(f32x4 *)&vsm[row * VS + 4 * c4] = vv;
            }
            if (video && tid < BK) kcoord[tid] = video_key_word(rec.k0 + tid, tm, pat, a);
            __syncthreads();

            // a PARTIAL tile may keep no pair of this wave's rows
            if (wave_skips_tile(a, a.mode, rec.aux, w)) continue;
            // ---- S^T = K Q^T for keys 0..31 (s0) and 32..63 (s1)
            f32x16 s0[1], s1[1];
            s0[0] = zero16;
            s1[0] = zero16;
#pragma unroll
            for (int kk = 0; kk < D / 2; ++kk) {
                const int dim = kk % 32 + 32 * hf + 64 * (kk / 32);
                const float k0v = ksm[l32 * KS + dim];
                const float k1v = ksm[(32 + l32) * KS + dim];
                s0[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0v, qreg[kk], s0[0], 0, 0, 0);
                s1[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1v, qreg[kk], s1[0], 0, 0, 0);
            }

            // ---- exact mask on PARTIAL tiles only
            if (wave_masks_tile(a.mode, rec.aux, w))
                mask_partial_tile<1>(s0, s1, a, a.mode, rec.k0, rec.aux, pat, LDS_PTR(const int, &kcoord[4 * hf]), qt,
                                     qwin, 32 * w, hf);

            // ---- online softmax (reference max moves only by more than kSlack)
            float mx = fmaxf(s0[0][0], s1[0][0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = max3f(mx, s0[0][r], s1[0][r]);
            mx = swap_halves_max(mx) * a.scale_log2;
            const bool need = mx > m_ref + kSlack;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const double alpha = need ? (double)__builtin_amdgcn_exp2f(m_ref - mx) : 1.0;
                m_ref = need ? mx : m_ref;
                l_run *= alpha;
#pragma unroll
                for (int n = 0; n < D / 32; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[n][r] *= alpha;
            }
            const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
            float psum[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s0[0][r] = __builtin_amdgcn_exp2f(fmaf(s0[0][r], a.scale_log2, -m_use));
                s1[0][r] = __builtin_amdgcn_exp2f(fmaf(s1[0][r], a.scale_log2, -m_use));
                psum[r] = s0[0][r] + s1[0][r];
            }
            // the tile's weights: a pairwise sum, then added in fp64
#pragma unroll
            for (int st = 8; st >= 1; st /= 2)
#pragma unroll
                for (int r = 0; r < st; ++r) psum[r] += psum[r + st];
            l_run += (double)psum[0];

            // ---- O^T += V^T P^T for this tile (from zero), added to the fp64 sums
            f32x16 otile[D / 32];
#pragma unroll
            for (int n = 0; n < D / 32; ++n) otile[n] = zero16;
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                const int key = 32 * (r / 16) + 8 * ((r % 16) / 4) + 4 * hf + r % 4;
                const float p = r < 16 ? s0[0][r] : s1[0][r - 16];
#pragma unroll
                for (int n = 0; n < D / 32; ++n)
                    otile[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(vsm[key * VS + 32 * n + l32], p, otile[n], 0, 0, 0);
            }
#pragma unroll
            for (int n = 0; n < D / 32; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[n][r] += (double)otile[n][r];
        }
    }

    // ---- epilogue: O = O / l (0 for rows without a kept key), in fp64
    const uint64_t lb = (uint64_t)__double_as_longlong(l_run);
    const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)lb, (unsigned)lb, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(lb >> 32), (unsigned)(lb >> 32), false, false);
    // each lane holds its own half's sum in one of the swapped pair and the
    // other half's in the other; their sum is the row's
    const double l_a = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0]));
    const double l_b = __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
    const double l_tot = l_a + l_b;
    const double inv = l_tot > 0.0 ? 1.0 / l_tot : 0.0;
    if (qvalid) {
        float *orow = Oh + (size_t)qtok * D;
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 o4 = {(float)(oacc[n][4 * rr] * inv), (float)(oacc[n][4 * rr + 1] * inv),
                                  (float)(oacc[n][4 * rr + 2] * inv), (float)(oacc[n][4 * rr + 3] * inv)};
                *(f32x4 *)(orow + 32 * n + 8 * rr + 4 * hf) = o4;
            }
    }
}

template <int NW, int D>
static hipError_t launch_f32(const KernelArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL((bsa_fwd_f32<NW, D>), dim3(a.ntasks), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_forward_f32(const KernelArgs &a, int waves, int d, hipStream_t stream)
{
    if (waves == 8 && d == 128) return launch_f32<8, 128>(a, stream);
    if (waves == 8 && d == 64) return launch_f32<8, 64>(a, stream);
    if (waves == 4 && d == 128) return launch_f32<4, 128>(a, stream);
    if (waves == 4 && d == 64) return launch_f32<4, 64>(a, stream);
    if (waves == 2 && d == 128) return launch_f32<2, 128>(a, stream);
    if (waves == 2 && d == 64) return launch_f32<2, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace bsa
