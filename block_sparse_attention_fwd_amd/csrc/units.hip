// Unit microbenchmarks of the gfx950 resources the forward kernel leans on,
// measured on the device itself: the denominators its roofline fractions are
// quoted against, and the co-issue behaviour that decides how the softmax
// overlaps the matrix products.
//
//  - MFMA rate: v_mfma_f32_32x32x16_bf16 on independent accumulators, every
//    SIMD busy, optionally with exponentials (v_exp_f32) or fused
//    multiply-adds issued between the MFMAs of the same wave, or by a second
//    wave of the same SIMD.
//  - Vector unit rates: v_exp_f32 and v_fma_f32 per wave instruction.
//  - LDS read rate: ds_read_b128 and ds_read_b64_tr_b16 (the operand reads of
//    the forward kernel).
//  - HBM rate: a streaming read and a copy of a large device buffer.
//
// Every kernel records the shader clock (s_memtime) and the constant 100 MHz
// clock (s_memrealtime) of wave 0 of block 0, so the host can turn the
// kernel's event time into clock cycles at the clock the device actually ran.
// Results are written to a small device array the caller passes in and reads
// back; the kernels read no other memory except the streaming buffers.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsa_units {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// stamps[0..3]: shader clock and real-time clock at start and end (block 0, wave 0)
__device__ __forceinline__ void stamp(uint64_t *stamps, int slot)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        stamps[2 * slot] = __builtin_amdgcn_s_memtime();
        stamps[2 * slot + 1] = __builtin_amdgcn_s_memrealtime();
    }
}

// MFMA loop. MODE 0: MFMAs only; 1: NE exponentials after each MFMA in the
// same wave; 2: NE fused multiply-adds after each MFMA in the same wave;
// 3: waves 0-3 of the 8-wave block issue MFMAs only and waves 4-7 (one on
// each SIMD beside them) issue NE exponentials per MFMA of their partner.
template <int MODE, int NE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mfma(int iters, uint64_t *stamps,
                                                                                          float *sink)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    stamp(stamps, 0);
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = 0.01f * (float)(lane + i);
    const bool mfma_wave = MODE != 3 || w < 4;
    const bool vec_wave = MODE == 1 || MODE == 2 || (MODE == 3 && w >= 4);
    auto vec = [&](int k0) {
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            float &x = e[(k0 + k) & 7];
            if (MODE == 2) x = fmaf(x, 0.999f, 0.001f);
            else x = __builtin_amdgcn_exp2f(-x);
        }
    };
    if (mfma_wave && MODE != 3) {
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            if (vec_wave) vec(0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            if (vec_wave) vec(NE);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            if (vec_wave) vec(2 * NE);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
            if (vec_wave) vec(3 * NE);
            // keep the issue order: each MFMA, then its NE vector instructions
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (NE > 0) __builtin_amdgcn_sched_group_barrier(MODE == 2 ? 0x002 : 0x400, NE, 0);
            }
        }
    } else if (mfma_wave) {
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
            vec(0);
            vec(NE);
            vec(2 * NE);
            vec(3 * NE);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += e[i];
    stamp(stamps, 1);
    if (s == 12345.678f) sink[threadIdx.x] = s;  // keeps the work; never true for these inputs
}

// Vector-unit rate: each wave issues `iters` x 16 instructions on 16
// independent registers. OP 0: v_exp_f32; 1: v_fma_f32.
template <int OP>
__global__ __launch_bounds__(256) void k_valu(int iters, uint64_t *stamps, float *sink)
{
    const int lane = threadIdx.x & 63;
    stamp(stamps, 0);
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.01f * (float)(lane + i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = OP == 0 ? __builtin_amdgcn_exp2f(-x[i]) : fmaf(x[i], 0.999f, 0.001f);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i];
    stamp(stamps, 1);
    if (s == 12345.678f) sink[threadIdx.x] = s;
}

// LDS read rate: 64 KiB of LDS read over and over by every wave of the block.
// OP 0: ds_read_b128 (16 bytes per lane); 1: ds_read_b64_tr_b16 (8 bytes per
// lane). Addresses stay inside the array.
template <int OP>
__global__ __launch_bounds__(512) void k_lds(int iters, uint64_t *stamps, float *sink)
{
    __shared__ __attribute__((aligned(16))) unsigned char buf[65536];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 65536 / 4; i += blockDim.x) ((int *)buf)[i] = i;
    __syncthreads();
    stamp(stamps, 0);
    i32x4 acc = {0, 0, 0, 0};
    const int stride = OP == 0 ? 1024 : 512;  // bytes per wave instruction
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int off = ((it * 8 + k + w * 8) * stride + lane * (stride / 64)) & 65535;
            if (OP == 0) {
                const i32x4 v = *(const __attribute__((address_space(3))) i32x4 *)(buf + off);
                acc ^= v;
            } else {
                const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(buf + off));
                acc[0] ^= (int)v[0] ^ ((int)v[1] << 16);
                acc[1] ^= (int)v[2] ^ ((int)v[3] << 16);
            }
        }
    }
    stamp(stamps, 1);
    if (acc[0] + acc[1] + acc[2] + acc[3] == 0x7EADBEEF) sink[threadIdx.x] = 1.f;
}

// Streaming HBM read (OP 0) or copy (OP 1) of n16 16-byte words.
template <int OP>
__global__ __launch_bounds__(256) void k_stream(const i32x4 *src, i32x4 *dst, int64_t n16, uint64_t *stamps, float *sink)
{
    stamp(stamps, 0);
    i32x4 acc = {0, 0, 0, 0};
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += step) {
        const i32x4 v = __builtin_nontemporal_load(src + i);
        if (OP == 1) __builtin_nontemporal_store(v, dst + i);
        else acc ^= v;
    }
    stamp(stamps, 1);
    if (OP == 0 && acc[0] + acc[1] + acc[2] + acc[3] == 0x7EADBEEF) sink[threadIdx.x] = 1.f;
}

}  // namespace bsa_units

using namespace bsa_units;

// Launch one unit benchmark and time it with events on the null stream.
// which: 0 = MFMA only, 1 = MFMA + exp same wave, 2 = MFMA + fma same wave,
// 3 = MFMA wave + exp wave on each SIMD (param = instructions per MFMA, 0..4);
// 10 = v_exp_f32, 11 = v_fma_f32; 20 = ds_read_b128, 21 = ds_read_b64_tr_b16;
// 30 = HBM read, 31 = HBM copy (param = MiB). blocks: workgroups of the launch.
// out[0] = event ms, out[1] = shader clock ticks and out[2] = 100 MHz ticks of
// block 0, wave 0, between its start and end stamps. Returns a hipError_t.
extern "C" int bsa_units_run(int which, int param, int iters, int blocks, double *out)
{
    hipError_t e;
    uint64_t *stamps = nullptr;
    float *sink = nullptr;
    i32x4 *buf = nullptr;
    hipEvent_t t0, t1;
    if ((e = hipMalloc(&stamps, 8 * sizeof(uint64_t))) != hipSuccess) return e;
    if ((e = hipMalloc(&sink, 1024 * sizeof(float))) != hipSuccess) return e;
    const int64_t n16 = (int64_t)param * (1 << 20) / 16;
    if (which >= 30) {
        if ((e = hipMalloc(&buf, (size_t)(which == 31 ? 2 : 1) * (size_t)n16 * 16)) != hipSuccess) return e;
        (void)hipMemset(buf, 1, (size_t)(which == 31 ? 2 : 1) * (size_t)n16 * 16);
    }
    (void)hipEventCreate(&t0);
    (void)hipEventCreate(&t1);
    for (int rep = 0; rep < 2; ++rep) {  // the first launch warms up clocks and code
        (void)hipEventRecord(t0, nullptr);
#define MF(M, N) hipLaunchKernelGGL((k_mfma<M, N>), dim3(blocks), dim3(512), 0, nullptr, iters, stamps, sink)
        switch (which) {
        case 0: MF(0, 0); break;
        case 1: switch (param) { case 1: MF(1, 1); break; case 2: MF(1, 2); break; case 3: MF(1, 3); break; case 4: MF(1, 4); break; default: MF(0, 0); } break;
        case 2: switch (param) { case 1: MF(2, 1); break; case 2: MF(2, 2); break; case 3: MF(2, 3); break; case 4: MF(2, 4); break; default: MF(0, 0); } break;
        case 3: switch (param) { case 1: MF(3, 1); break; case 2: MF(3, 2); break; case 3: MF(3, 3); break; case 4: MF(3, 4); break; default: MF(0, 0); } break;
        case 10: hipLaunchKernelGGL((k_valu<0>), dim3(blocks), dim3(256), 0, nullptr, iters, stamps, sink); break;
        case 11: hipLaunchKernelGGL((k_valu<1>), dim3(blocks), dim3(256), 0, nullptr, iters, stamps, sink); break;
        case 20: hipLaunchKernelGGL((k_lds<0>), dim3(blocks), dim3(512), 0, nullptr, iters, stamps, sink); break;
        case 21: hipLaunchKernelGGL((k_lds<1>), dim3(blocks), dim3(512), 0, nullptr, iters, stamps, sink); break;
        case 30: hipLaunchKernelGGL((k_stream<0>), dim3(blocks), dim3(256), 0, nullptr, buf, buf, n16, stamps, sink); break;
        case 31: hipLaunchKernelGGL((k_stream<1>), dim3(blocks), dim3(256), 0, nullptr, buf, buf + n16, n16, stamps, sink); break;
        default: e = hipErrorInvalidValue;
        }
#undef MF
        if (e != hipSuccess) break;
        if ((e = hipGetLastError()) != hipSuccess) break;
        (void)hipEventRecord(t1, nullptr);
        if ((e = hipEventSynchronize(t1)) != hipSuccess) break;
    }
    float ms = 0.f;
    uint64_t h[4] = {0, 0, 0, 0};
    if (e == hipSuccess) {
        (void)hipEventElapsedTime(&ms, t0, t1);
        e = hipMemcpy(h, stamps, sizeof h, hipMemcpyDeviceToHost);
    }
    out[0] = ms;
    out[1] = (double)(h[2] - h[0]);
    out[2] = (double)(h[3] - h[1]);
    (void)hipEventDestroy(t0);
    (void)hipEventDestroy(t1);
    (void)hipFree(stamps);
    (void)hipFree(sink);
    if (buf) (void)hipFree(buf);
    return e;
}
