// Head routing probe: for a sample of query rows of every (batch, head), the
// dense attention output and the outputs under the spatial and the temporal
// video patterns (Sparse VideoGen / Splash Attention summary, "Sparse
// VideoGen": each head is routed on the fly to a spatial or a temporal sparse
// pattern). The host turns the per-row squared differences into the routing.
//
//   probe_partial  one workgroup of three waves per (batch, head, 32 sampled
//                  rows, key chunk); the waves share each staged K/V tile and
//                  run the online softmax of those rows under one of the three
//                  masks each (dense, spatial, temporal), written as (max,
//                  sum, unnormalised output) partials
//   probe_combine  one workgroup per (batch, head, 8 sampled rows): the
//                  partials merged per variant, and per row the squared
//                  differences of the two patterns' outputs from the dense one
//
// Layout on the MFMA units as in the forward kernel: S^T = K Q^T with one query
// per lane column (lane l: query l % 32, keys 8*(r/4) + 4*(l/32) + r%4 of a
// 32-key half), O^T += V^T P^T with V^T read from row-major V in LDS by the
// transposing read. Key tokens are processed in frame-major order: the video
// patterns are defined on token coordinates, so a head's memory layout does
// not change what the probe computes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.hpp"
#include "route_probe.hpp"

namespace bsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kVariants = 3;  // dense, spatial, temporal

template <int V>
struct IntC {
    static constexpr int value = V;
};
constexpr int kGroups = 2;    // blocks of 32 sampled rows per workgroup (they share the staged tiles)

__device__ __forceinline__ bf16x8 load8(const __bf16 *p) { return __builtin_bit_cast(bf16x8, *(const i32x4 *)p); }

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l writes its 16 bytes to LDS [lds + 16 l); M0 carries the LDS address.
// Issued through inline assembly, so that the compiler does not make the LDS
// reads of the current tile wait for it; completion is awaited explicitly.
__device__ __forceinline__ void copy16_lds(const void *g, uint32_t lds)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// LDS layouts without bank conflicts: K row r stores 16-byte chunk c at
// position c ^ (r % (D/8)); V row k stores chunk c at c ^ vswz(k % 4), so the
// transposing read of 4 consecutive keys x 32 contiguous bytes hits distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int key_mod4)
{
    return D == 128 ? (int)((0xAC60u >> (4 * key_mod4)) & 15u) : 2 * key_mod4;
}

template <int D>
__global__ __launch_bounds__(64 * kVariants * kGroups) __attribute__((amdgpu_waves_per_eu(2))) void probe_partial(RouteArgs a)
{
    constexpr int ROWB = 2 * D;
    // double-buffered: tile t + 1 lands while tile t is computed
    __shared__ __attribute__((aligned(1024))) unsigned char ksm[2][kTileK * ROWB];  // row r: chunk c at c ^ (r % (D/8))
    __shared__ __attribute__((aligned(1024))) unsigned char vsm[2][kTileK * ROWB];  // row k: chunk c at c ^ vswz(k % 4)
    __shared__ __attribute__((aligned(16))) int kframe[2][kTileK];  // -1 past the sequence end
    __shared__ __attribute__((aligned(16))) int kyx[2][kTileK];     // (y << 16) | x

    const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
    // wave wv: variant wv % 3 (0 dense, 1 spatial, 2 temporal) of sample
    // block g = wv / 3 of the workgroup's group
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int v = wv % kVariants, g = wv / kVariants;
    const int nsg = (a.nsb + kGroups - 1) / kGroups;
    const int bh = blockIdx.x / nsg, sb = (blockIdx.x % nsg) * kGroups + g, chunk = blockIdx.y;
    const bool active = sb < a.nsb;  // a missing last block still stages tiles
    const int unit = bh * a.nsb + min(sb, a.nsb - 1);
    const int L = a.L;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    const __bf16 *Qh = (const __bf16 *)a.Q + head_off;
    const __bf16 *Kh = (const __bf16 *)a.K + head_off;
    const __bf16 *Vh = (const __bf16 *)a.V + head_off;

    // this lane's sampled query (rows past the sample repeat the last one;
    // their partials are never read)
    const int qi = min(sb * 32 + l32, a.S - 1);
    const int qtok = a.rows[qi];
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qreg[s] = load8(Qh + (size_t)qtok * D + 16 * s + 8 * hf);
    const int qf = fdiv(qtok, a.magic_HW, a.shift_HW);
    const int qp = qtok - qf * a.HW;
    const int qy = fdiv(qp, a.magic_W, a.shift_W), qx = qp - qy * a.W;

    // V^T operand offsets: keys 4*hf + key_sub (+16c, +8; all the same row
    // mod 4), dims dd_base + 32n
    const int grp = lane >> 4, jl = lane & 15;
    const int dd_base = 16 * (grp & 1) + 4 * (jl & 3);
    const int key_sub = jl >> 2;
    const int sv = vswz<D>(key_sub);
    int voff[D / 32];
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
        voff[n] = (4 * hf + key_sub) * ROWB + 16 * (((32 * n + dd_base) >> 3) ^ sv) + 2 * (dd_base & 7);

    f32x16 oacc[D / 32];
    float m_ref = -INFINITY, l_run = 0.f;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;

    const int t0 = chunk * a.tiles_per_chunk, t1 = min(t0 + a.tiles_per_chunk, a.nkt);
    // K and V tiles -> LDS by direct copies, shared out over the waves (rows
    // past L repeat row L-1: finite values, weight 0); chunks land in the
    // swizzled positions. Wave 0 writes the tile's key coordinates.
    auto stage = [&](int t, int buf) {
        const int k0 = t * kTileK;
        constexpr int NI = kTileK * ROWB / 1024;  // wave-wide copies per tensor
        for (int idx = wv; idx < 2 * NI; idx += kVariants * kGroups) {
            const int i = idx % NI;
            const int byte = 1024 * i + 16 * lane;
            const int r = byte / ROWB, pos = (byte % ROWB) / 16;
            const size_t grow = (size_t)min(k0 + r, L - 1) * D;
            const uint32_t off = (uint32_t)(1024 * i);
            if (idx < NI)
                copy16_lds(Kh + grow + 8 * (pos ^ (r & (D / 8 - 1))),
                           __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&ksm[buf][0] + off));
            else
                copy16_lds(Vh + grow + 8 * (pos ^ vswz<D>(r & 3)),
                           __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&vsm[buf][0] + off));
        }
        if (wv == 0) {
            const int kt = k0 + lane;
            int f = -1, yx = 0;
            if (kt < L) {
                f = fdiv(kt, a.magic_HW, a.shift_HW);
                const int p = kt - f * a.HW;
                const int y = fdiv(p, a.magic_W, a.shift_W);
                yx = (y << 16) | (p - y * a.W);
            }
            kframe[buf][lane] = f;
            kyx[buf][lane] = yx;
        }
    };
    if (t0 < t1) stage(t0, 0);
    for (int t = t0; t < t1; ++t) {
        const int cur = (t - t0) & 1;
        // tile t has landed (each wave waits for its own copies), and every
        // wave is done with tile t - 1, whose buffer tile t + 1 now takes
        wait_copies();
        __syncthreads();
        if (t + 1 < t1) stage(t + 1, cur ^ 1);
        if (!active) continue;
        const unsigned char *kt_lds = &ksm[cur][0];
        const unsigned char *vt_lds = &vsm[cur][0];

        // ---- S^T = K Q^T
        f32x16 sc[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int r = 32 * h2 + l32;
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const bf16x8 kv = *LDS_PTR(const bf16x8, kt_lds + r * ROWB + 16 * ((2 * s + hf) ^ (r & (D / 8 - 1))));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qreg[s], acc, 0, 0, 0);
            }
            sc[h2] = acc;
        }

        // the variant's mask on this lane's 32 scores, in place: kept scores
        // become s*c, the others -inf. Dense: key inside the sequence;
        // spatial: key in the query's frame or the anchor frame; temporal: key
        // pixel within the radius of the query pixel (Chebyshev), any frame.
        // One code path per variant (v is wave-uniform).
        auto apply_mask = [&](auto vc) {
            constexpr int V = decltype(vc)::value;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int kbase = 32 * h2 + 8 * g + 4 * hf;
                    const i32x4 f4 = *LDS_PTR(const i32x4, &kframe[cur][kbase]);
                    i32x4 w4 = {};
                    if (V == 2) w4 = *LDS_PTR(const i32x4, &kyx[cur][kbase]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        bool k = f4[j] >= 0;
                        if (V == 1) k = k & ((f4[j] == qf) | (f4[j] == a.anchor));
                        // |dy| <= r as one unsigned compare of dy + r against 2r
                        if (V == 2)
                            k = k & ((unsigned)((w4[j] >> 16) - qy + a.radius) <= 2u * (unsigned)a.radius) &
                                ((unsigned)((w4[j] & 0xFFFF) - qx + a.radius) <= 2u * (unsigned)a.radius);
                        sc[h2][4 * g + j] = k ? sc[h2][4 * g + j] * a.scale_log2 : -INFINITY;
                    }
                }
        };
        if (v == 0) apply_mask(IntC<0>{});
        else if (v == 1) apply_mask(IntC<1>{});
        else apply_mask(IntC<2>{});
        float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = max3f(mx, sc[0][r], sc[1][r]);
        mx = swap_halves_max(mx);
        // the reference moves only when a tile's maximum exceeds it by more than kSlack
        const bool need = mx > m_ref + kSlack;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.0f;
            m_ref = need ? mx : m_ref;
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < D / 32; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[n][r] *= alpha;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        u32x4 pk[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(sc[c / 2][8 * (c % 2) + e] - m_use);
                const float p1 = __builtin_amdgcn_exp2f(sc[c / 2][8 * (c % 2) + e + 1] - m_use);
                const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
                pk[c][e / 2] = __builtin_bit_cast(unsigned, pp);
            }
        // ---- O^T += V^T P^T
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int n = 0; n < D / 32; ++n) {
                const unsigned char *pa = vt_lds + voff[n] + 16 * c * ROWB;
                const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, pa));
                const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, pa + 8 * ROWB));
                const bf16x4 a4 = __builtin_bit_cast(bf16x4, va), b4 = __builtin_bit_cast(bf16x4, vb);
                const bf16x8 vop = {a4[0], a4[1], a4[2], a4[3], b4[0], b4[1], b4[2], b4[3]};
                oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, __builtin_bit_cast(bf16x8, pk[c]), oacc[n], 0, 0, 0);
            }
    }

    // ---- partial of this variant: the row maximum, the row sum and the
    // unnormalised output rows [32][D]
    if (!active) return;
    float *pv = a.part + ((size_t)(unit * a.nchunk + chunk) * kVariants + v) * (size_t)(64 + 32 * D);
    const float lt = swap_halves_sum(l_run);
    if (hf == 0) {
        pv[l32] = m_ref;
        pv[32 + l32] = lt;
    }
    float *orow = pv + 64 + (size_t)l32 * D;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int dd = 32 * n + 8 * rr + 4 * hf;
            *(float4 *)(orow + dd) = make_float4(oacc[n][4 * rr], oacc[n][4 * rr + 1], oacc[n][4 * rr + 2], oacc[n][4 * rr + 3]);
        }
}

// One workgroup of 256 threads per (batch, head, 8 sampled rows): thread t
// takes row t / 32 of the group and dims [D/32 * (t % 32), +D/32).
template <int D>
__global__ __launch_bounds__(256) void probe_combine(RouteArgs a)
{
    constexpr int DPT = D / 32;
    const int unit = blockIdx.x >> 2, bh = unit / a.nsb, sb = unit % a.nsb;
    const int row = 8 * (blockIdx.x & 3) + (threadIdx.x >> 5), part32 = threadIdx.x & 31;
    const size_t stride_v = 64 + 32 * (size_t)D, stride_c = kVariants * stride_v;
    const float *base = a.part + (size_t)unit * a.nchunk * stride_c;
    float o[kVariants][DPT];
#pragma unroll
    for (int v = 0; v < kVariants; ++v) {
        float M = -INFINITY;
        for (int c = 0; c < a.nchunk; ++c) M = fmaxf(M, base[c * stride_c + v * stride_v + row]);
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < DPT; ++j) o[v][j] = 0.f;
        for (int c = 0; c < a.nchunk; ++c) {
            const float *pv = base + c * stride_c + v * stride_v;
            const float mc = pv[row];
            if (mc == -INFINITY) continue;  // no key of this variant in the chunk
            const float w = __builtin_amdgcn_exp2f(mc - M);
            lsum += pv[32 + row] * w;
            const float *orow = pv + 64 + (size_t)row * D + DPT * part32;
#pragma unroll
            for (int j = 0; j < DPT; ++j) o[v][j] += orow[j] * w;
        }
        const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
        for (int j = 0; j < DPT; ++j) o[v][j] *= inv;
    }
    float e_sp = 0.f, e_tp = 0.f;
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const float ds = o[1][j] - o[0][j], dt = o[2][j] - o[0][j];
        e_sp = fmaf(ds, ds, e_sp);
        e_tp = fmaf(dt, dt, e_tp);
    }
    // sum over the 32 threads of the row (one half of a wave)
    for (int off = 1; off < 32; off <<= 1) {
        e_sp += __shfl_xor(e_sp, off, 64);
        e_tp += __shfl_xor(e_tp, off, 64);
    }
    const int qi = sb * 32 + row;
    if (part32 == 0 && qi < a.S) {
        float *er = a.err_rows + ((size_t)bh * a.S + qi) * 2;
        er[0] = e_sp;
        er[1] = e_tp;
    }
}

// One thread per head: the head's squared differences summed over the batch
// and the sampled rows, sequentially, in fp64.
__global__ __launch_bounds__(64) void route_head_sums(const float *err_rows, int B, int H, int S, double *sums)
{
    const int h = blockIdx.x * 64 + threadIdx.x;
    if (h >= H) return;
    double es = 0.0, et = 0.0;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < S; ++i) {
            const float *er = err_rows + ((size_t)(b * H + h) * S + i) * 2;
            es += er[0];
            et += er[1];
        }
    sums[2 * h] = es;
    sums[2 * h + 1] = et;
}

}  // namespace

hipError_t launch_route_head_sums(const float *err_rows, int32_t B, int32_t H, int32_t S, double *sums,
                                  hipStream_t stream)
{
    hipLaunchKernelGGL(route_head_sums, dim3((unsigned)((H + 63) / 64)), dim3(64), 0, stream, err_rows, B, H, S, sums);
    return hipGetLastError();
}

hipError_t launch_route_probe(const RouteArgs &a, int d, hipStream_t stream)
{
    const dim3 grid_p((unsigned)(a.BH * ((a.nsb + kGroups - 1) / kGroups)), (unsigned)a.nchunk),
        grid_c((unsigned)(a.BH * a.nsb * 4));
    if (d == 128) {
        hipLaunchKernelGGL(probe_partial<128>, grid_p, dim3(64 * kVariants * kGroups), 0, stream, a);
        hipLaunchKernelGGL(probe_combine<128>, grid_c, dim3(256), 0, stream, a);
    } else if (d == 64) {
        hipLaunchKernelGGL(probe_partial<64>, grid_p, dim3(64 * kVariants * kGroups), 0, stream, a);
        hipLaunchKernelGGL(probe_combine<64>, grid_c, dim3(256), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bsa
