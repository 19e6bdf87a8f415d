// gfx950 (CDNA4) forward kernel of block-sparse attention.
//
// One workgroup runs one task: a tile of 32*NW query rows of one (batch,
// head) against the ordered key tiles the plan lists for it (Tessera, arXiv
// 2609.25869, abstract: physical tiles grouped into GPU tasks for data reuse
// and load/compute overlap). Every key tile of 64 keys is staged in LDS once
// and shared by all waves; the next tile's global loads are in flight while
// the current tile is computed, and land in the other half of a
// double-buffered LDS tile (the 8-wave kernel keeps two tiles in flight in a
// ring of three buffers). Empty tiles never reach the kernel; FULL tiles
// run with no mask code; PARTIAL tiles evaluate the exact predicate (Sparse
// VideoGen / Splash Attention summary, "Splash Attention": empty tiles
// bypassed, exact coordinate masking only on boundary tiles). Gathered tiles
// load the listed key rows into packed LDS tiles (FG-Attn, arXiv 2509.16518,
// abstract: gather a sparse set of key/value vectors into packed tiles).
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
// Online softmax in fp32 with base-2 exponentials and c = log2(e)/sqrt(d):
// p = 2^(s*c - m), l = sum p, O = sum p V, O / l at the end. The reference m
// only moves when a tile's maximum exceeds it by more than kSlack (then O and
// l are rescaled by 2^(m_old - m_new)); p therefore stays below 2^kSlack and
// the result, O / l, does not depend on where m sits. P is rounded to bf16
// once and the same rounded values feed both the PV product and the row sum.
// Rows with no kept key output 0.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.hpp"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct IntC {
    static constexpr int value = V;
};

template <int NW, int RB, int D>
struct Cfg {
    static constexpr int BQ = 32 * NW * RB;            // query rows per task
    static constexpr int BK = kTileK;
    static constexpr int ROWB = D * 2;                 // bytes per bf16 row
    static constexpr int TILEB = BK * ROWB;            // bytes per K or V tile
    static constexpr int CHUNKS = ROWB / 16;           // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROWB;            // rows per wave-wide 1 KiB copy
    static constexpr int INSTS = BK / RPI / NW;        // copies per wave per tensor per tile
    static_assert(INSTS >= 1, "tile too small for the workgroup");
};

// Conflict-free LDS layouts; rows keep their natural 256/128-byte stride and
// the 16-byte chunks of a row are XOR-swizzled. K row r stores chunk c at
// position c ^ swz_k(r): one chunk read from 8 or 16 consecutive rows hits
// distinct banks. V row k stores chunk c at c ^ swz_v(k & 3): the transposing
// read of 4 consecutive keys x 32 contiguous bytes hits distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return row & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int key_mod4)
{
    return D == 128 ? (int)((0xAC60u >> (4 * key_mod4)) & 15u) : 2 * key_mod4;  // {0,6,12,10} / {0,2,4,6}
}

// Direct global -> LDS copy (global_load_lds_dwordx4): lane l writes the 16
// bytes at its global address to LDS bytes [lds + 16 l, +16). It is issued
// through inline assembly so that the compiler does not make every later LDS
// read wait for it (it cannot tell that the reads use the other buffer);
// completion is awaited explicitly (s_waitcnt vmcnt) before the barrier that
// hands the buffer to the other waves. M0 carries the LDS address; no
// compiler-generated code of this kernel uses M0.
__device__ __forceinline__ void copy16_to_lds(const void *g, uint32_t lds)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
}
// The same copy with a wave-uniform base address in SGPRs and a 32-bit
// per-lane byte offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void copy16_to_lds_s(const void *base, uint32_t off, uint32_t lds)
{
    // the base is wave-uniform; make that explicit so it lives in an SGPR pair
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
}
// One dword per lane (global_load_lds_dword): lane l writes LDS bytes
// [lds + 4 l, +4); scalar base, 32-bit lane offsets, as copy16_to_lds_s.
__device__ __forceinline__ void copy4_to_lds_s(const void *base, uint32_t off, uint32_t lds)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(sb), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
}
// All vector-memory operations issued so far (the copies included) have
// completed: s_waitcnt vmcnt(0), written with the compiler builtin so that the
// compiler's own wait bookkeeping sees it and does not wait again, later, for
// loads it issued before this point (with copies in flight, such a wait would
// stall on the copies).
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16 *p)
{
    i32x4 v = *(const i32x4 *)p;
    return __builtin_bit_cast(bf16x8, v);
}

// Kernel: NW waves per workgroup, each wave owns RB consecutive blocks of 32
// query rows. Every K operand read from LDS feeds RB score MFMAs and every V
// operand read feeds RB output MFMAs, so LDS bytes per MFMA fall as 1/RB.
// MODE is the plan's MaskMode: each mode gets its own build, free of the
// others' record, copy and mask code.
template <int NW, int RB, int D, int NB, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RB == 1 && (NW >= 4 || NB == 1) ? 2 : 1, RB == 1 ? 2 : 1))) void bsa_fwd_bf16(KernelArgs a)
{
    using C = Cfg<NW, RB, D>;
    // NB = 2: tile j + 1 lands in the other buffer while tile j is computed;
    // NB = 1: one buffer, filled after each tile (other workgroups on the CU
    // cover the copy), so that twice as many workgroups fit in LDS;
    // NB = 3: tile j + 2 is issued while tile j is computed, so a copy has two
    // tiles of compute to land. The two halves of the workgroup copy
    // alternate tiles (waves 0..NW/2-1 the even ones), so that each wave only
    // ever waits for all of its own copies: the half that issued tile j + 1
    // waits at the end of tile j, while the other half's tile j + 2 stays in
    // flight.
    static_assert(NB != 3 || NW >= 4, "three buffers need two copy groups");
    constexpr int CW = NB == 3 ? NW / 2 : NW;       // waves that copy one tile
    constexpr int CI = C::BK / C::RPI / CW;          // copies per copying wave per tensor
    __shared__ __attribute__((aligned(16))) int kcoord[NB][C::BK];  // [buffer] video key coordinates
    __shared__ __attribute__((aligned(1024))) unsigned char ksm[NB][C::TILEB];  // [buffer] swizzled K tile
    __shared__ __attribute__((aligned(1024))) unsigned char vsm[NB][C::TILEB];  // [buffer] swizzled V tile

    const int tid = threadIdx.x;
    const int lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    // task fields and head flags are workgroup-uniform: scalar registers
    const Task tl = a.tasks[blockIdx.x];
    const Task task{__builtin_amdgcn_readfirstlane(tl.bh), __builtin_amdgcn_readfirstlane(tl.q0),
                    __builtin_amdgcn_readfirstlane(tl.tb), __builtin_amdgcn_readfirstlane(tl.te)};
    if (task.bh < 0) return;  // padding task of an XCD segment
    // instrumented launches: thread 0 stamps the task's start and end with the
    // shader clock counter and the constant 100 MHz counter
    if (a.stamps && tid == 0) {
        a.stamps[4 * blockIdx.x] = __builtin_amdgcn_s_memtime();
        a.stamps[4 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
    }
    const int bh = task.bh;
    const int h = bh % a.H;
    const uint32_t hflag = (uint32_t)__builtin_amdgcn_readfirstlane((int)a.head_flags[h]);
    const bool tm = (hflag & kHeadTemporalMajor) != 0;
    const int pat = (int)((hflag >> kHeadPatShift) & 3u);
    const int L = a.L;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    const __bf16 *Qh = (const __bf16 *)a.Q + head_off;
    const __bf16 *Kh = (const __bf16 *)a.K + head_off;
    const __bf16 *Vh = (const __bf16 *)a.V + head_off;
    __bf16 *Oh = (__bf16 *)a.O + head_off;

    auto token = [&](int j) -> int { return head_token(j, tm, a); };

    // ---- this lane's query rows: one per 32-row block rb (logical q, frame-major token qtok)
    int q[RB], qtok[RB];
    bool qvalid[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        q[rb] = task.q0 + 32 * (w * RB + rb) + l32;
        qvalid[rb] = q[rb] < L;
        qtok[rb] = token(qvalid[rb] ? q[rb] : L - 1);
    }

    const int ntile = task.te - task.tb;
    constexpr bool gather = MODE == kModeGather;
    constexpr bool video = MODE == kModeVideo;

    // Softmax reference: a row takes the maximum of its first kept scores as
    // reference and keeps it; the per-tile row maximum is computed only while
    // some row of the wave has no reference yet. Scores more than 64 (base 2)
    // above the reference would make sums overflow: a row whose sum ends above
    // 2^64, or not finite, makes the whole task run again in careful mode,
    // where every tile computes its row maximum and the reference follows it
    // (moving only when a tile's maximum exceeds it by more than kSlack).
    bool careful = false;
    f32x16 oacc[RB][D / 32];
    float m_ref[RB], l_run[RB];
    for (;;) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[rb][n][r] = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) { m_ref[rb] = -INFINITY; l_run[rb] = 0.f; }

    if (ntile > 0) {
        bf16x8 qreg[RB][D / 16];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int s = 0; s < D / 16; ++s) qreg[rb][s] = load_bf16x8(Qh + (size_t)qtok[rb] * D + 16 * s + 8 * hf);

        // query coordinates for the video predicates: frame (spatial) or the
        // packed window origin ((y - r) << 16) + (x - r) (temporal)
        int qt[RB];
        unsigned qwin[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            qt[rb] = 0;
            qwin[rb] = 0;
            if (video) video_query_coords(qtok[rb], a, qt[rb], qwin[rb]);
        }

        // rows this lane copies for each tile: slot = (wc*CI + i)*RPI + lane/CHUNKS,
        // wc = the wave's index among the waves that copy the tile
        const int pos = lane % C::CHUNKS;
        const int wc = w % CW;
        const bool odd_copier = w >= CW;  // NB = 3: this wave copies the odd tiles
        int idx_nxt[CI];  // gathered logical key positions of the next tile to fetch

        RecordStream rs;
        rs.init(a.tiles, task.tb, task.te, lane);

        auto load_indices = [&](const TileRec r, int *dst) {
            const int cnt = (int)(r.aux & kAuxMask);
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                int slot = (wc * CI + i) * C::RPI + lane / C::CHUNKS;
                dst[i] = a.gidx[r.k0 + (slot < cnt ? slot : cnt - 1)];
            }
        };

        // global -> LDS copies of a tile (in flight while the previous tile is
        // computed), the video key coordinates included
        const int32_t *ctab = a.coords + (int)((hflag >> kHeadCoordShift) & 3u) * a.coords_stride;
        // per-lane byte offsets of the copied chunks within a contiguous tile
        uint32_t kgoff[CI], vgoff[CI];
#pragma unroll
        for (int i = 0; i < CI; ++i) {
            const int slot = (wc * CI + i) * C::RPI + lane / C::CHUNKS;
            kgoff[i] = (uint32_t)(slot * C::ROWB + 16 * (pos ^ swz_k<D>(slot)));
            vgoff[i] = (uint32_t)(slot * C::ROWB + 16 * (pos ^ swz_v<D>(slot & 3)));
        }
        auto fetch_tile = [&](const TileRec r, const int *idx, int buf) {
            const uint32_t kl = (uint32_t)(uintptr_t)&ksm[buf][0], vl = (uint32_t)(uintptr_t)&vsm[buf][0];
            if (!tm && !gather && r.k0 + C::BK <= L) {
                // 64 consecutive rows: scalar base + loop-invariant lane offsets
                const __bf16 *kb = Kh + (size_t)r.k0 * D, *vb = Vh + (size_t)r.k0 * D;
#pragma unroll
                for (int i = 0; i < CI; ++i) {
                    const uint32_t off = (uint32_t)((wc * CI + i) * 1024);
                    copy16_to_lds_s(kb, kgoff[i], __builtin_amdgcn_readfirstlane(kl + off));
                    copy16_to_lds_s(vb, vgoff[i], __builtin_amdgcn_readfirstlane(vl + off));
                }
            } else {
                // listed rows (gather) or rows of a temporal-major head: one
                // address per lane, all computed before the copies are issued
                int ktok[CI];
#pragma unroll
                for (int i = 0; i < CI; ++i) {
                    const int slot = (wc * CI + i) * C::RPI + lane / C::CHUNKS;
                    ktok[i] = token(gather ? idx[i] : min(r.k0 + slot, L - 1));
                }
#pragma unroll
                for (int i = 0; i < CI; ++i) {
                    const int slot = (wc * CI + i) * C::RPI + lane / C::CHUNKS;
                    const uint32_t off = (uint32_t)((wc * CI + i) * 1024);
                    copy16_to_lds(Kh + (size_t)ktok[i] * D + 8 * (pos ^ swz_k<D>(slot)), __builtin_amdgcn_readfirstlane(kl + off));
                    copy16_to_lds(Vh + (size_t)ktok[i] * D + 8 * (pos ^ swz_v<D>(slot & 3)), __builtin_amdgcn_readfirstlane(vl + off));
                }
            }
            if (video && wc == 0) {
                // the tile's 64 key-coordinate words, copied from the head's
                // table in the plan (frame, or (y << 16) | x; kNoKey past the end)
                copy4_to_lds_s(ctab + r.k0, 4u * (uint32_t)lane, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&kcoord[buf][0]));
            }
        };
        // publish a fetched tile: its copies have landed
        auto finish_tile = [&](int) { wait_copies(); };

        // prologue: tile 0 into buffer 0 (NB = 3: and tile 1 into buffer 1, by
        // the odd half, which waits for it at the end of tile 0)
        if constexpr (NB == 3) {
            if (!odd_copier) {
                fetch_tile(rs.get(0), idx_nxt, 0);
                finish_tile(0);
            } else if (ntile > 1) {
                fetch_tile(rs.get(1), idx_nxt, 1);
            }
        } else {
            if (gather) load_indices(rs.get(0), idx_nxt);
            fetch_tile(rs.get(0), idx_nxt, 0);
            if (gather && ntile > 1) load_indices(rs.get(1), idx_nxt);
            finish_tile(0);
        }
        __syncthreads();

        // per-lane LDS read offsets (loop-invariant; tile-relative parts are immediates)
        int koff[D / 16];  // K rows l32 (+32: same swizzle), chunk 2s + hf
#pragma unroll
        for (int s = 0; s < D / 16; ++s) koff[s] = l32 * C::ROWB + 16 * ((2 * s + hf) ^ swz_k<D>(l32));
        const int grp = lane >> 4, jl = lane & 15;
        const int dd_base = 16 * (grp & 1) + 4 * (jl & 3);  // first dim this lane addresses
        const int key_sub = jl >> 2;                         // key within a group of 4
        const int sv = swz_v<D>(key_sub);
        int voff[D / 32];  // V^T operand of dim block n: keys 4*hf + key_sub (+16c, +8)
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
            voff[n] = (4 * hf + key_sub) * C::ROWB + 16 * (((32 * n + dd_base) >> 3) ^ sv) + 2 * (dd_base & 7);
        const f32x16 zero16 = {};

        // one key tile; the LDS buffer index is a compile-time constant (the loop
        // below is unrolled by NB), so every LDS operand address is a
        // loop-invariant register plus an immediate offset
        auto tile_step = [&](const int j, auto cur_c) {
            constexpr int cur = NB == 1 ? 0 : decltype(cur_c)::value;
            if ((j & 63) == 0 && j > 0) rs.advance();
            const TileRec rec = rs.get(j);
            const bool more = j + 1 < ntile;
            if (NB == 2 && more) {
                fetch_tile(rs.get(j + 1), idx_nxt, cur ^ 1);
                if (gather && j + 2 < ntile) load_indices(rs.get(j + 2), idx_nxt);
            }
            // NB = 3: tile j + 2 goes to the buffer tile j - 1 left (its reads
            // ended before the barrier that closed tile j - 1); the half that
            // copies it is the one that copied tile j, whose copies have landed
            if (NB == 3 && j + 2 < ntile && odd_copier == ((j & 1) != 0))
                fetch_tile(rs.get(j + 2), idx_nxt, (cur + 2) % 3);

            // A PARTIAL tile may keep no pair of this wave's rows: the wave
            // skips it (and still takes its part in the copies and barriers)
            if (!wave_skips_tile(a, MODE, rec.aux, w)) {
            // ---- S^T = K Q^T: s0 = keys 0..31, s1 = keys 32..63 of each row block
            const unsigned char *kt = ksm[cur];
            f32x16 s0[RB], s1[RB];
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const bf16x8 k0v = *LDS_PTR(bf16x8, kt + koff[s]);
                const bf16x8 k1v = *LDS_PTR(bf16x8, kt + koff[s] + 32 * C::ROWB);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    s0[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0v, qreg[rb][s], s == 0 ? zero16 : s0[rb], 0, 0, 0);
                    s1[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1v, qreg[rb][s], s == 0 ? zero16 : s1[rb], 0, 0, 0);
                }
            }
            // LDS reads run two read pairs ahead of the MFMAs that consume them
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int s = 0; s < D / 16 - 2; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * RB, 0);

            // ---- exact mask on PARTIAL tiles only
            if (wave_masks_tile(MODE, rec.aux, w)) mask_partial_tile<RB>(s0, s1, a, MODE, rec.k0, rec.aux, pat, LDS_PTR(const int, &kcoord[cur][4 * hf]), qt, qwin, 32 * w * RB, hf);

            // ---- online softmax per row block
            u32x4 pk[RB][4];  // bf16 pairs, one cvt_pk each
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                if (careful || __builtin_amdgcn_ballot_w64(m_ref[rb] == -INFINITY)) {
                    float mx = fmaxf(s0[rb][0], s1[rb][0]);
#pragma unroll
                    for (int r = 1; r < 16; ++r) mx = max3f(mx, s0[rb][r], s1[rb][r]);
                    mx = swap_halves_max(mx) * a.scale_log2;
                    const bool need = mx > m_ref[rb] + kSlack;
                    if (__builtin_amdgcn_ballot_w64(need)) {
                        // lanes that keep their reference (also those still at -inf) scale by exactly 1
                        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref[rb] - mx) : 1.0f;
                        m_ref[rb] = need ? mx : m_ref[rb];
                        l_run[rb] *= alpha;
#pragma unroll
                        for (int n = 0; n < D / 32; ++n)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[rb][n][r] *= alpha;
                    }
                }
                const float m_use = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
                const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const float x0 = (c < 2 ? s0[rb] : s1[rb])[8 * (c % 2) + e];
                        const float x1 = (c < 2 ? s0[rb] : s1[rb])[8 * (c % 2) + e + 1];
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(x0, a.scale_log2, -m_use));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(x1, a.scale_log2, -m_use));
                        const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
                        l_run[rb] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run[rb], false);
                        pk[rb][c][e / 2] = __builtin_bit_cast(unsigned, pp);
                    }
                }
            }

            // ---- O^T += V^T P^T (one V operand read feeds RB MFMAs)
            const unsigned char *vt = vsm[cur];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int n = 0; n < D / 32; ++n) {
                    const unsigned char *pa = vt + voff[n] + 16 * c * C::ROWB;  // keys 16c + 4hf + key_sub
                    const unsigned char *pb = pa + 8 * C::ROWB;                  // ... + 8
                    const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, pa));
                    const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, pb));
                    const bf16x4 a4 = __builtin_bit_cast(bf16x4, va), b4 = __builtin_bit_cast(bf16x4, vb);
                    const bf16x8 vop = {a4[0], a4[1], a4[2], a4[3], b4[0], b4[1], b4[2], b4[3]};
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        oacc[rb][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, __builtin_bit_cast(bf16x8, pk[rb][c]), oacc[rb][n], 0, 0, 0);
                }
            }
            // transposing reads run two operand reads ahead
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
            for (int i = 0; i < 4 * (D / 32) - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, RB, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 1);
            }

            if constexpr (NB == 2) {
                if (more) finish_tile(cur ^ 1);
                __syncthreads();
            } else if constexpr (NB == 3) {
                // tile j + 1 has landed: its copying half waits for its copies
                if (more && odd_copier == (((j + 1) & 1) != 0)) finish_tile(0);
                __syncthreads();
            } else {
                __syncthreads();  // every wave is done with the buffer
                if (more) {
                    fetch_tile(rs.get(j + 1), idx_nxt, 0);
                    if (gather && j + 2 < ntile) load_indices(rs.get(j + 2), idx_nxt);
                    finish_tile(0);
                    __syncthreads();
                }
            }
        };
        int j = 0;
        if constexpr (NB == 3) {
            for (; j + 2 < ntile; j += 3) {
                tile_step(j, IntC<0>{});
                tile_step(j + 1, IntC<1>{});
                tile_step(j + 2, IntC<2>{});
            }
            if (j < ntile) tile_step(j, IntC<0>{});
            if (j + 1 < ntile) tile_step(j + 1, IntC<1>{});
        } else {
            for (; j + 1 < ntile; j += 2) {
                tile_step(j, IntC<0>{});
                tile_step(j + 1, IntC<1>{});
            }
            if (j < ntile) tile_step(j, IntC<0>{});
        }
    }
    bool bad = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) bad |= !(l_run[rb] <= 0x1p64f);
    if (careful || !__syncthreads_or(bad)) break;
    careful = true;
    }

    // ---- epilogue: O = O / l (0 for rows without a kept key), bf16 RNE
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = swap_halves_sum(l_run[rb]);
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        if (qvalid[rb]) {
            __bf16 *orow = Oh + (size_t)qtok[rb] * D;
#pragma unroll
            for (int n = 0; n < D / 32; ++n)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int dd = 32 * n + 8 * rr + 4 * hf;
                    const bf16x4 o4 = {(__bf16)(oacc[rb][n][4 * rr] * inv), (__bf16)(oacc[rb][n][4 * rr + 1] * inv),
                                       (__bf16)(oacc[rb][n][4 * rr + 2] * inv), (__bf16)(oacc[rb][n][4 * rr + 3] * inv)};
                    *(bf16x4 *)(orow + dd) = o4;
                }
        }
    }
    if (a.stamps && tid == 0) {
        a.stamps[4 * blockIdx.x + 2] = __builtin_amdgcn_s_memtime();
        a.stamps[4 * blockIdx.x + 3] = __builtin_amdgcn_s_memrealtime();
    }
}

// one kernel build per (NW, RB, D, NB, mask mode); the plan's mode picks it
template <int NW, int RB, int D, int NB = 2>
static hipError_t launch(const KernelArgs &a, hipStream_t stream)
{
    const dim3 grid(a.ntasks), block(NW * 64);
    if (a.mode == kModeVideo) {
        hipLaunchKernelGGL((bsa_fwd_bf16<NW, RB, D, NB, kModeVideo>), grid, block, 0, stream, a);
    } else if (a.mode == kModeGather) {
        if constexpr (NB == 3) return hipErrorInvalidValue;  // gathered tiles keep two buffers at most
        else hipLaunchKernelGGL((bsa_fwd_bf16<NW, RB, D, NB, kModeGather>), grid, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL((bsa_fwd_bf16<NW, RB, D, NB, kModeBlock>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_forward(const KernelArgs &a, int waves, int rb, int d, int dtype, int nbuf, hipStream_t stream)
{
    if (dtype != 0) return hipErrorInvalidValue;
    if (nbuf == 3) {
        // contiguous / permuted key tiles only (the gather regimes keep their
        // own buffering)
        if (a.mode == kModeGather || rb != 1) return hipErrorInvalidValue;
        if (waves == 8 && d == 128) return launch<8, 1, 128, 3>(a, stream);
        if (waves == 8 && d == 64) return launch<8, 1, 64, 3>(a, stream);
        return hipErrorInvalidValue;
    }
    if (rb == 1) {
        if (waves == 4 && d == 128) return launch<4, 1, 128>(a, stream);
        if (waves == 4 && d == 64) return launch<4, 1, 64>(a, stream);
        // two waves, d = 128: single-buffered, so that four workgroups (two
        // waves per SIMD) fit in LDS; measured faster than double-buffered
        // with one wave per SIMD (FG-Attn M = 64: 4.42 -> 4.03 ms)
        if (waves == 2 && d == 128) return launch<2, 1, 128, 1>(a, stream);
        if (waves == 2 && d == 64) return launch<2, 1, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace bsa
