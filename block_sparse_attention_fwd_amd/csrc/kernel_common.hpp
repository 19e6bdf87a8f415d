// Device helpers shared by the bf16 and fp32 forward kernels: token
// addressing of temporal-major heads, video key coordinates, the exact
// predicate of PARTIAL tiles and the lane-pair reductions of the score
// layout.
//
// Score layout (both kernels): a 32x32 MFMA result S^T holds keys in rows and
// queries in columns; lane l owns query l % 32 and, in register r, key
// 8*(r/4) + 4*(l/32) + r%4 of the 32-key block.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_format.hpp"

namespace bsa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr float kSlack = 8.0f;  // log2 headroom before the softmax reference moves

// Key-coordinate word of a slot past the sequence end: no frame equals it, and
// (kNoKey - window origin) has both 16-bit halves far above any 2*radius
// (radius <= 256, coordinates < 512), so no video predicate keeps it.
constexpr int kNoKey = 0x7FFF7FFF;

// n / d for 0 <= n < 2^31 with the host-computed multiplier (round-up method)
__device__ __forceinline__ int fdiv(int n, uint32_t m, int s)
{
    return (int)((__umulhi((unsigned)n, m) + (unsigned)n) >> s);
}

// Logical position j of a head -> frame-major token. Temporal-major heads
// (Sparse VideoGen / Splash Attention summary, "Splash Attention": token
// layouts permuted into temporal-major order) use j = p*T + t for the token
// t*HW + p; the permutation lives only in addresses.
__device__ __forceinline__ int head_token(int j, bool tm, const KernelArgs &a)
{
    if (!tm) return j;
    const int p = fdiv(j, a.magic_T, a.shift_T);
    return (j - p * a.T) * a.HW + p;
}

// Video coordinate word of key position kp: its frame (spatial pattern) or
// (y << 16) | x (temporal pattern); kNoKey past the sequence end.
__device__ __forceinline__ int video_key_word(int kp, bool tm, int pat, const KernelArgs &a)
{
    if (kp >= a.L) return kNoKey;
    const int kt = head_token(kp, tm, a);
    const int t = fdiv(kt, a.magic_HW, a.shift_HW);
    const int p = kt - t * a.HW;
    const int y = fdiv(p, a.magic_W, a.shift_W), x = p - y * a.W;
    return pat == 1 ? t : (pat == 2 ? ((y << 16) | x) : 0);
}

// Query side of the video predicates: the frame, and the packed window origin
// ((y - r) << 16) + (x - r), of frame-major token qtok.
__device__ __forceinline__ void video_query_coords(int qtok, const KernelArgs &a, int &qt, unsigned &qwin)
{
    qt = fdiv(qtok, a.magic_HW, a.shift_HW);
    const int p = qtok - qt * a.HW;
    const int y = fdiv(p, a.magic_W, a.shift_W), x = p - y * a.W;
    qwin = ((unsigned)(y - a.radius) << 16) + (unsigned)(x - a.radius);
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

// three-input maximum on one VALU op (scores are never NaN, so no quieting of
// the inputs is needed)
__device__ __forceinline__ float max3f(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// The key-tile records of one task, as a wave reads them: 64 records per
// vector load (lane l holds record 64 c + l of chunk c), one chunk ahead of
// use, and a record is taken out with two lane reads into scalar registers.
// A per-tile load of each record would put a memory round trip in front of
// every tile. get(j) serves records j in [64*chunk, 64*chunk + 128) of the
// task; advance() is called at the top of the tile step that enters a new
// chunk, where no tile copies are in flight, so the wait for the chunk loaded
// 64 tiles earlier costs nothing. Lanes past the task's end repeat its last
// record (no branch, so the loads land straight in their registers).
struct RecordStream {
    const TileRec *tiles;
    int tb, te, lane, chunk;
    uint32_t cur_k0, cur_aux, nxt_k0, nxt_aux;

    __device__ __forceinline__ void load(int c, uint32_t &k0, uint32_t &aux) const
    {
        const TileRec r = tiles[min(tb + 64 * c + lane, te - 1)];
        k0 = (uint32_t)r.k0;
        aux = r.aux;
    }
    __device__ __forceinline__ void init(const TileRec *t, int b, int e, int ln)
    {
        tiles = t;
        tb = b;
        te = e;
        lane = ln;
        chunk = 0;
        load(0, cur_k0, cur_aux);
        load(1, nxt_k0, nxt_aux);
    }
    __device__ __forceinline__ void advance()
    {
        cur_k0 = nxt_k0;
        cur_aux = nxt_aux;
        ++chunk;
        load(chunk + 1, nxt_k0, nxt_aux);
    }
    __device__ __forceinline__ TileRec get(int j) const
    {
        const bool in_cur = (j >> 6) == chunk;
        const int l = j & 63;
        const uint32_t k0c = __builtin_amdgcn_readlane(cur_k0, l), k0n = __builtin_amdgcn_readlane(nxt_k0, l);
        const uint32_t axc = __builtin_amdgcn_readlane(cur_aux, l), axn = __builtin_amdgcn_readlane(nxt_aux, l);
        // (the fields are wave-uniform; readfirstlane keeps them, and all the
        // address arithmetic on them, in scalar registers)
        TileRec r;
        r.k0 = __builtin_amdgcn_readfirstlane((int32_t)(in_cur ? k0c : k0n));
        r.aux = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(in_cur ? axc : axn));
        return r;
    }
};

// Per-wave refinement of a PARTIAL tile for wave w (query rows 32w..32w+31 of
// the task); both are wave-uniform. `mode` is the plan's MaskMode (a
// compile-time constant where the kernel is built for one mode).
//  - skip: the wave's rows keep no pair of the tile. Video tiles carry the bit
//    from the plan; block tiles whose sub-block rows are at least 32 queries
//    tall read it from the sub-block keep bits of the wave's sub-block row.
//  - mask: the wave's rows need the exact predicate (video tiles carry a bit
//    for rows that keep every pair).
__device__ __forceinline__ bool wave_skips_tile(const KernelArgs &a, int mode, uint32_t aux, int w)
{
    if (!(aux & kPartial)) return false;
    if (mode == kModeVideo) return (aux >> w) & 1u;
    if (mode == kModeBlock && a.bq_shift >= 5) {
        const int sq = (kWaveRows * w) >> a.bq_shift;
        return ((aux >> (sq * a.nsk)) & ((1u << a.nsk) - 1u)) == 0u;
    }
    return false;
}
__device__ __forceinline__ bool wave_masks_tile(int mode, uint32_t aux, int w)
{
    if (!(aux & kPartial)) return false;
    if (mode == kModeVideo) return !((aux >> (kWaveFullShift + w)) & 1u);
    return true;
}

// Exact predicate of a PARTIAL 64-key tile (Sparse VideoGen / Splash
// Attention summary, "Splash Attention": exact coordinate masking on boundary
// tiles only). s0 / s1 are the scores of keys 0..31 / 32..63 of each 32-row
// block rb; unkept scores become -inf.
//  - video: per-key coordinate words in LDS (kc = the tile's 64 words + 4*hf)
//    against the query's frame
//    (spatial: same frame or the anchor frame) or window (temporal: packed
//    |dy| <= r and |dx| <= r through one unsigned compare per half);
//  - block: keep bits of the logical sub-blocks merged into the tile, plus
//    key < L;
//  - gather: key slot < the record's count.
template <int RB>
__device__ __forceinline__ void mask_partial_tile(f32x16 (&s0)[RB], f32x16 (&s1)[RB], const KernelArgs &a, int mode,
                                                  int rec_k0, uint32_t rec_aux, int pat, const __attribute__((address_space(3))) int *kc,
                                                  const int (&qt)[RB], const unsigned (&qwin)[RB], int wrow0, int hf)
{
    if (mode == kModeVideo) {
        const unsigned win2 = 2u * (unsigned)a.radius;
        if (pat == 1) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const i32x4 c0 = *(const __attribute__((address_space(3))) i32x4 *)(kc + 8 * g);
                const i32x4 c1 = *(const __attribute__((address_space(3))) i32x4 *)(kc + 32 + 8 * g);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s0[rb][4 * g + e] = (c0[e] == qt[rb] || c0[e] == a.anchor) ? s0[rb][4 * g + e] : -INFINITY;
                        s1[rb][4 * g + e] = (c1[e] == qt[rb] || c1[e] == a.anchor) ? s1[rb][4 * g + e] : -INFINITY;
                    }
            }
        } else if (pat == 2) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const i32x4 c0 = *(const __attribute__((address_space(3))) i32x4 *)(kc + 8 * g);
                const i32x4 c1 = *(const __attribute__((address_space(3))) i32x4 *)(kc + 32 + 8 * g);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned d0 = (unsigned)c0[e] - qwin[rb], d1 = (unsigned)c1[e] - qwin[rb];
                        s0[rb][4 * g + e] = max(d0 & 0xffffu, d0 >> 16) <= win2 ? s0[rb][4 * g + e] : -INFINITY;
                        s1[rb][4 * g + e] = max(d1 & 0xffffu, d1 >> 16) <= win2 ? s1[rb][4 * g + e] : -INFINITY;
                    }
            }
        } else {  // dense: only slots past the sequence end
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const i32x4 c0 = *(const __attribute__((address_space(3))) i32x4 *)(kc + 8 * g);
                const i32x4 c1 = *(const __attribute__((address_space(3))) i32x4 *)(kc + 32 + 8 * g);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s0[rb][4 * g + e] = c0[e] != kNoKey ? s0[rb][4 * g + e] : -INFINITY;
                        s1[rb][4 * g + e] = c1[e] != kNoKey ? s1[rb][4 * g + e] : -INFINITY;
                    }
            }
        }
        return;
    }
    // keep bits of key slots 0..31 (lo) and 32..63 (hi) for each row block
    const int kmax = mode == kModeBlock ? a.L - rec_k0 : (int)(rec_aux & kAuxMask);
    uint32_t vlo = ~0u, vhi = ~0u;  // slots >= kmax: past the sequence / list end
    if (kmax < 64) {
        vlo = kmax >= 32 ? ~0u : ((1u << max(kmax, 0)) - 1u);
        vhi = kmax <= 32 ? 0u : ((1u << (kmax - 32)) - 1u);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        uint32_t lo = vlo, hi = vhi;
        if (mode == kModeBlock) {
            // logical blocks are at least 32 queries tall, so a 32-row block
            // (rows wrow0 + 32 rb .. + 31 of the task) lies in one sub-block row
            const int sq = (wrow0 + 32 * rb) >> a.bq_shift;
            const uint32_t rowbits = rec_aux >> (sq * a.nsk);
            lo &= (rowbits & 1u) ? ~0u : 0u;
            hi &= ((rowbits >> (a.nsk - 1)) & 1u) ? ~0u : 0u;
        }
        lo >>= 4 * hf;
        hi >>= 4 * hf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int bit = 8 * (r / 4) + (r % 4);
            s0[rb][r] = ((lo >> bit) & 1u) ? s0[rb][r] : -INFINITY;
            s1[rb][r] = ((hi >> bit) & 1u) ? s1[rb][r] : -INFINITY;
        }
    }
}

}  // namespace bsa
