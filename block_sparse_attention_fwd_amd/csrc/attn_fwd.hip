// gfx950 (CDNA4) forward kernel of block-sparse attention.
//
// One workgroup runs one task: a tile of 32*NW query rows of one (batch,
// head) against the ordered key tiles the plan lists for it (Tessera, arXiv
// 2609.25869, abstract: physical tiles grouped into GPU tasks for data reuse
// and load/compute overlap). Every key tile of 64 keys is staged in LDS once
// and shared by all waves; the next tile's load is in flight while the current
// tile is computed (double-buffered LDS). Empty tiles never reach the kernel;
// FULL tiles run with no mask code; PARTIAL tiles evaluate the exact predicate
// (Sparse VideoGen / Splash Attention summary, "Splash Attention": empty tiles
// bypassed, exact coordinate masking only on boundary tiles). Gathered tiles
// load the listed key rows into packed LDS tiles (FG-Attn, arXiv 2509.16518,
// abstract: asynchronous-gather load of a sparse key/value set).
//
// Matrix layout on the MFMA units (v_mfma_f32_32x32x16_bf16, wave64):
//  - S^T = K Q^T: A = 32 keys x 16 dims from LDS, B = Q^T from registers.
//    The result puts one query per lane column: lane l holds query l%32 and
//    keys 8*(r/4) + 4*(l/32) + r%4 for r = 0..15, so a row maximum / sum is
//    an in-lane reduction plus one exchange with lane l^32.
//  - O^T += V^T P^T: A = V^T (32 dims x 16 keys) read from row-major V with
//    the transposing LDS read, B = P^T straight from the score registers.
//    O^T again has one query per lane column, so the online-softmax rescale
//    is per lane.
// Online softmax in fp32 with base-2 exponentials: m' = max(m, rowmax(s)*c),
// p = 2^(s*c - m'), l' = 2^(m - m') l + sum p, O' = 2^(m - m') O + P V with
// c = log2(e)/sqrt(d); P is rounded to bf16 once and the same rounded values
// feed both the PV product and the row sum. Rows with no kept key output 0.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_format.hpp"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

template <int NW, int D>
struct Cfg {
    static constexpr int BQ = 32 * NW;
    static constexpr int BK = kTileK;
    static constexpr int ROWB = D * 2;                 // bytes per bf16 row
    static constexpr int TILEB = BK * ROWB;            // bytes per K or V tile
    static constexpr int CHUNKS = ROWB / 16;           // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROWB;            // rows per wave-wide 1 KiB copy
    static constexpr int INSTS = BK / RPI / NW;        // copies per wave per tensor per tile
    static_assert(INSTS >= 1, "tile too small for the workgroup");
};

// XOR swizzles of the 16-byte chunks within a row (conflict-free LDS access):
// K rows are read 8 or 16 rows at a time at one chunk; V is read through the
// transposing read 4 consecutive keys at a time.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : (row & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int row)
{
    if (D == 128) {
        const int r = row & 3;
        return r == 0 ? 0 : (r == 1 ? 6 : (r == 2 ? 12 : 10));
    }
    return 2 * (row & 3);
}

__device__ __forceinline__ float swap_halves_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16 *p)
{
    i32x4 v = *(const i32x4 *)p;
    return __builtin_bit_cast(bf16x8, v);
}

template <int NW, int D>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void bsa_fwd_bf16(KernelArgs a)
{
    using C = Cfg<NW, D>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][C::TILEB];  // [buffer][K, V][tile]
    __shared__ __attribute__((aligned(16))) int kcoord[2][C::BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const Task task = a.tasks[blockIdx.x];
    const int bh = task.bh;
    const int h = bh % a.H;
    const uint32_t hflag = a.head_flags[h];
    const bool tm = (hflag & kHeadTemporalMajor) != 0;
    const int pat = (int)((hflag >> kHeadPatShift) & 3u);
    const int L = a.L;
    const int T = a.T, HW = a.HW, W = a.W;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    const __bf16 *Qh = (const __bf16 *)a.Q + head_off;
    const __bf16 *Kh = (const __bf16 *)a.K + head_off;
    const __bf16 *Vh = (const __bf16 *)a.V + head_off;
    __bf16 *Oh = (__bf16 *)a.O + head_off;

    auto token = [&](int j) -> int { return tm ? (j % T) * HW + j / T : j; };

    // ---- this lane's query row (logical position q, frame-major token qtok)
    const int q = task.q0 + 32 * w + l32;
    const bool qvalid = q < L;
    const int qtok = token(qvalid ? q : L - 1);

    const int ntile = task.te - task.tb;
    const bool gather = a.mode == kModeGather;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    if (ntile > 0) {
        bf16x8 qreg[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qreg[s] = load_bf16x8(Qh + (size_t)qtok * D + 16 * s + 8 * hf);

        // query coordinates for the video predicates
        int qt = 0, qy = 0, qx = 0;
        if (a.mode == kModeVideo) {
            qt = qtok / HW;
            qy = (qtok % HW) / W;
            qx = qtok % W;
        }

        // rows this lane copies for each tile: slot = (w*INSTS + i)*RPI + lane/CHUNKS
        const int pos = lane % C::CHUNKS;
        int idx_nxt[C::INSTS];  // gathered logical key positions of the next tile to fetch

        auto load_indices = [&](int rec_i, int *dst) {
            const TileRec r = a.tiles[rec_i];
            const int cnt = (int)(r.aux & kAuxMask);
#pragma unroll
            for (int i = 0; i < C::INSTS; ++i) {
                int slot = (w * C::INSTS + i) * C::RPI + lane / C::CHUNKS;
                dst[i] = a.gidx[r.k0 + (slot < cnt ? slot : cnt - 1)];
            }
        };

        // global -> registers (in flight while the current tile is computed)
        i32x4 stage_k[C::INSTS], stage_v[C::INSTS];
        int stage_c = -1;
        auto fetch_tile = [&](int rec_i, const int *idx) {
            const TileRec r = a.tiles[rec_i];
#pragma unroll
            for (int i = 0; i < C::INSTS; ++i) {
                const int slot = (w * C::INSTS + i) * C::RPI + lane / C::CHUNKS;
                const int kpos = gather ? idx[i] : min(r.k0 + slot, L - 1);
                const int ktok = token(kpos);
                stage_k[i] = *(const i32x4 *)(Kh + (size_t)ktok * D + 8 * (pos ^ swz_k<D>(slot)));
                stage_v[i] = *(const i32x4 *)(Vh + (size_t)ktok * D + 8 * (pos ^ swz_v<D>(slot)));
            }
            if (a.mode == kModeVideo && w == 0) {
                // packed (t, y, x) of each key slot; slots past the sequence end
                // get a value no query coordinate can match
                const int kp = r.k0 + lane;
                int v = -1;
                if (kp < L) {
                    const int kt = token(kp);
                    v = ((kt / HW) << 20) | (((kt % HW) / W) << 10) | (kt % W);
                }
                stage_c = v;
            }
        };
        // registers -> LDS buffer `buf`
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int i = 0; i < C::INSTS; ++i) {
                *LDS_PTR(i32x4, &smem[buf][0][(w * C::INSTS + i) * 1024 + 16 * lane]) = stage_k[i];
                *LDS_PTR(i32x4, &smem[buf][1][(w * C::INSTS + i) * 1024 + 16 * lane]) = stage_v[i];
            }
            if (a.mode == kModeVideo && w == 0) kcoord[buf][lane] = stage_c;
        };

        // prologue: tile 0 into buffer 0
        if (gather) load_indices(task.tb, idx_nxt);
        fetch_tile(task.tb, idx_nxt);
        if (gather && ntile > 1) load_indices(task.tb + 1, idx_nxt);
        store_tile(0);
        __syncthreads();

        const int krow0 = l32, krow1 = 32 + l32;
        const int fk0 = swz_k<D>(krow0), fk1 = swz_k<D>(krow1);

        for (int j = 0; j < ntile; ++j) {
            const int cur = j & 1;
            const TileRec rec = a.tiles[task.tb + j];
            const bool more = j + 1 < ntile;
            if (more) {
                fetch_tile(task.tb + j + 1, idx_nxt);
                if (gather && j + 2 < ntile) load_indices(task.tb + j + 2, idx_nxt);
            }

            // ---- S^T = K Q^T
            f32x16 sacc[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) { sacc[0][r] = 0.f; sacc[1][r] = 0.f; }
            const unsigned char *kt = smem[cur][0];
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const int c = 2 * s + hf;
                bf16x8 k0v = *LDS_PTR(bf16x8, kt + krow0 * C::ROWB + 16 * (c ^ fk0));
                bf16x8 k1v = *LDS_PTR(bf16x8, kt + krow1 * C::ROWB + 16 * (c ^ fk1));
                sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0v, qreg[s], sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1v, qreg[s], sacc[1], 0, 0, 0);
            }
            // keep LDS reads next to the MFMAs that consume them (bounds register use)
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }

            // ---- exact mask on PARTIAL tiles only
            if (rec.aux & kPartial) {
                if (a.mode == kModeVideo) {
                    const int *kc = kcoord[cur];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const i32x4 c4 = *LDS_PTR(i32x4, kc + 32 * kb + 8 * g + 4 * hf);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int v = c4[e];
                                bool keep;
                                if (pat == 1) {
                                    const int kt2 = (int)((unsigned)v >> 20);
                                    keep = kt2 == qt || kt2 == a.anchor;
                                } else if (pat == 2) {
                                    const int ky = (v >> 10) & 1023, kx = v & 1023;
                                    keep = abs(ky - qy) <= a.radius && abs(kx - qx) <= a.radius;
                                } else {
                                    keep = v != -1;
                                }
                                if (!keep) sacc[kb][4 * g + e] = -INFINITY;
                            }
                        }
                } else {
                    // keep bits of key slots 0..31 (lo) and 32..63 (hi) for this lane's query
                    uint32_t lo, hi;
                    int kmax;  // slots >= kmax are not kept (sequence end / list end)
                    if (a.mode == kModeBlock) {
                        const int sq = (q - task.q0) >> a.bq_shift;
                        const uint32_t rowbits = rec.aux >> (sq * a.nsk);
                        lo = (rowbits & 1u) ? ~0u : 0u;
                        hi = ((rowbits >> (a.nsk - 1)) & 1u) ? ~0u : 0u;
                        kmax = L - rec.k0;
                    } else {
                        lo = hi = ~0u;
                        kmax = (int)(rec.aux & kAuxMask);
                    }
                    if (kmax < 64) {
                        lo &= kmax >= 32 ? ~0u : ((1u << max(kmax, 0)) - 1u);
                        hi &= kmax <= 32 ? 0u : ((1u << (kmax - 32)) - 1u);
                    }
                    lo >>= 4 * hf;
                    hi >>= 4 * hf;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int bit = 8 * (r / 4) + (r % 4);
                        if (!((lo >> bit) & 1u)) sacc[0][r] = -INFINITY;
                        if (!((hi >> bit) & 1u)) sacc[1][r] = -INFINITY;
                    }
                }
            }

            // ---- online softmax
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[1][r]));
            mx = swap_halves_max(mx);
            const float m_new = fmaxf(m_run, mx * a.scale_log2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;

            bf16x8 pk[4];
            float psum = 0.f;
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float s0 = sacc[c / 2][8 * (c % 2) + e], s1 = sacc[c / 2][8 * (c % 2) + e + 1];
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s0, a.scale_log2, -m_use));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s1, a.scale_log2, -m_use));
                    const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
                    psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
                    pk[c][e] = pp[0];
                    pk[c][e + 1] = pp[1];
                }
            }
            l_run = l_run * alpha + psum;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
                for (int n = 0; n < D / 32; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[n][r] *= alpha;
            }

            // ---- O^T += V^T P^T
            const unsigned char *vt = smem[cur][1];
            const int grp = lane >> 4, jl = lane & 15;
            const int dd_base = 16 * (grp & 1) + 4 * (jl & 3);  // dim offset this lane addresses
            const int key_sub = jl >> 2;                         // key within the group of 4
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int n = 0; n < D / 32; ++n) {
                    const int dd = 32 * n + dd_base;
                    const int ka = 16 * c + 4 * hf + key_sub, kb2 = ka + 8;
                    const unsigned char *pa = vt + ka * C::ROWB + 16 * ((dd >> 3) ^ swz_v<D>(ka)) + 2 * (dd & 7);
                    const unsigned char *pb = vt + kb2 * C::ROWB + 16 * ((dd >> 3) ^ swz_v<D>(kb2)) + 2 * (dd & 7);
                    const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, pa));
                    const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, pb));
                    const bf16x4 a4 = __builtin_bit_cast(bf16x4, va), b4 = __builtin_bit_cast(bf16x4, vb);
                    const bf16x8 vop = {a4[0], a4[1], a4[2], a4[3], b4[0], b4[1], b4[2], b4[3]};
                    oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pk[c], oacc[n], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4 * (D / 32); ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            }

            if (more) store_tile(cur ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: O = O / l (0 for rows without a kept key), bf16 RNE
    const float l_tot = swap_halves_sum(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qvalid) {
        __bf16 *orow = Oh + (size_t)qtok * D;
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int dd = 32 * n + 8 * rr + 4 * hf;
                const bf16x4 o4 = {(__bf16)(oacc[n][4 * rr] * inv), (__bf16)(oacc[n][4 * rr + 1] * inv),
                                   (__bf16)(oacc[n][4 * rr + 2] * inv), (__bf16)(oacc[n][4 * rr + 3] * inv)};
                *(bf16x4 *)(orow + dd) = o4;
            }
    }
}

template <int NW, int D>
static hipError_t launch(const KernelArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL((bsa_fwd_bf16<NW, D>), dim3(a.ntasks), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_forward(const KernelArgs &a, int waves, int d, int dtype, hipStream_t stream)
{
    if (dtype != 0) return hipErrorInvalidValue;
    if (waves == 4 && d == 128) return launch<4, 128>(a, stream);
    if (waves == 4 && d == 64) return launch<4, 64>(a, stream);
    if (waves == 2 && d == 128) return launch<2, 128>(a, stream);
    if (waves == 2 && d == 64) return launch<2, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace bsa
