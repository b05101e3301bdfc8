// fa_clock_probe.hip -- measurement helpers for the benchmark (libfa_clock.so),
// not part of the attention library: the shader clock probe, and reference
// kernels that give the ceilings the attention kernels are judged against
// on this part -- a register-only stream of fp16 matrix instructions, a
// streaming read of device memory, and the issue rate of the vector
// instructions the softmax is made of.
//
// The shader clock the GPU actually runs at while a workload executes: one
// wavefront, launched on a side stream while the workload's kernels are in
// flight, spins for a window of the 100 MHz real-time counter and counts
// shader clock cycles (s_memtime) over the same window.  Under a board power
// limit the clock sits below the frequency the published peak assumes, so
// the benchmark reports both.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void clock_probe_kernel(unsigned long long *out, unsigned long long window)
{
    if (threadIdx.x != 0) return;
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1 = r0;
    while (r1 - r0 < window) r1 = __builtin_amdgcn_s_memrealtime();  // ends: the counter always advances
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    out[0] = t1 - t0;
    out[1] = r1 - r0;
}

typedef _Float16 half8p __attribute__((ext_vector_type(8)));
typedef float floatx16p __attribute__((ext_vector_type(16)));
typedef unsigned int uint4p __attribute__((ext_vector_type(4)));

// Four independent accumulator chains of v_mfma_f32_32x32x16_f16 per
// wavefront, operands held in registers, eight wavefronts per workgroup and
// two per SIMD (the occupancy of the attention kernels at D = 128): the
// matrix unit's sustained fp16 rate with no memory traffic at all.  The
// matrix unit's power, and so the clock the part holds under its power
// limit, depends on the operand bits.  Operand patterns (MODE):
//   0  every operand an fp16 value with a random sign, a random 10-bit
//      fraction and a magnitude in [1/4, 4) (an xorshift stream per lane);
//      the four chains rotate through eight such A and B fragments, as a
//      kernel multiplying Gaussian data sees;
//   1  few distinct small values (many zeros);
//   2  as 0, but four consecutive MFMAs share their B fragment (operand
//      reuse between neighbouring instructions);
//   3  as 0 with the 5 low fraction bits zero (fewer bits that toggle).
// Each thread writes one sum at the end so the chains are not removed.
__device__ __forceinline__ unsigned int xorshift(unsigned int &x)
{
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
}

// sign, exponent 13..16 (2^-2 .. 2^1), fraction under `mask`: binary16 bits
__device__ __forceinline__ _Float16 random_half(unsigned int &x, unsigned int mask)
{
    const unsigned int r = xorshift(x);
    const unsigned short h =
        (unsigned short)(((r >> 15) & 0x8000u) | ((13u + (r & 3u)) << 10) | ((r >> 2) & mask));
    return __builtin_bit_cast(_Float16, h);
}

template <int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void
mfma_stream_kernel(float *out, int iters)
{
    const int t = threadIdx.x;
    half8p A[8], B[8];
    unsigned int x = 0x9e3779b9u ^ (unsigned int)((blockIdx.x * blockDim.x + t) * 2654435761u);
    constexpr unsigned int kMask = MODE == 3 ? 0x3e0u : 0x3ffu;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (MODE == 1) {
                A[j][i] = (_Float16)(((t + i + j) & 7) * 0.0625f);
                B[j][i] = (_Float16)(((t * 3 + i + j) & 7) * 0.0625f);
            } else {
                A[j][i] = random_half(x, kMask);
                B[j][i] = random_half(x, kMask);
            }
        }
    floatx16p c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (MODE == 2) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[j], B[j], c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[(j + 3) & 7], B[j], c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[(j + 5) & 7], B[j], c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[(j + 2) & 7], B[j], c3, 0, 0, 0);
            } else {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[j], B[j], c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[j], B[(j + 3) & 7], c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[(j + 5) & 7], B[j], c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[(j + 2) & 7], B[(j + 6) & 7], c3, 0, 0, 0);
            }
        }
    }
    float s = 0.0f;
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// Streaming read: every thread loads 16 bytes per step, grid-strided over
// n16 16-byte elements (the whole buffer, once), and writes one word.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void
read_stream_kernel(const uint4p *buf, size_t n16, unsigned int *out)
{
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t step = (size_t)gridDim.x * blockDim.x;
    uint4p acc = {0u, 0u, 0u, 0u};
    for (size_t i = gid; i < n16; i += step) acc ^= buf[i];
    out[gid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Vector-ALU issue rate of one instruction kind: eight independent chains per
// wavefront of v_exp_f32 (mode 0), v_exp_f16 (mode 1) or v_fma_f32 (mode 2)
// on registers, 512 threads per workgroup.  The chains stay bounded (x <-
// 2^-x converges to about 0.64, x <- x/2 + 1/4 to 1/2), so no operand is ever
// infinite or denormal.  Each thread writes one sum so the chains are kept.
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512))) void
valu_stream_kernel(float *out, int iters, int mode)
{
    const int t = threadIdx.x;
    float x[8];
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[i] = 1e-3f * (float)((t & 63) + i);
        h[i] = (_Float16)x[i];
    }
    const float half_ = 0.5f, quarter = 0.25f;
    if (mode == 0) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 8; ++i) __asm__ volatile("v_exp_f32 %0, -%0" : "+v"(x[i]));
    } else if (mode == 1) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 8; ++i) __asm__ volatile("v_exp_f16 %0, -%0" : "+v"(h[i]));
    } else {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __asm__ volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(half_), "v"(quarter));
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += x[i] + (float)h[i];
    out[(size_t)blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

// Vector-ALU rate: `workgroups` workgroups of 512 threads, each wavefront
// issuing 8 * iters instructions of the kind `mode` selects (0 v_exp_f32,
// 1 v_exp_f16, 2 v_fma_f32).  out: device buffer of at least workgroups *
// 512 floats.  Returns 0, or 1 on bad arguments or a rejected launch.
extern "C" __attribute__((visibility("default"))) int fa_probe_valu_stream(void *out, long long out_floats,
                                                                            int workgroups, int iters, int mode,
                                                                            void *stream)
{
    if (!out || workgroups <= 0 || iters <= 0 || mode < 0 || mode > 2 ||
        out_floats < (long long)workgroups * 512)
        return 1;
    hipLaunchKernelGGL(valu_stream_kernel, dim3(workgroups), dim3(512), 0, (hipStream_t)stream,
                       (float *)out, iters, mode);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Matrix-unit ceiling: `workgroups` workgroups of 512 threads, each wavefront
// issuing 32 * iters v_mfma_f32_32x32x16_f16 (32768 flops each) on the
// operand pattern `mode` (0 random, 1 structured, 2 random with B shared by
// four consecutive MFMAs, 3 random with the 5 low fraction bits zero).  out:
// device buffer of at least workgroups * 512 floats.  Returns 0, or 1 on bad
// arguments or a rejected launch.
extern "C" __attribute__((visibility("default"))) int fa_probe_mfma_stream(void *out, long long out_floats,
                                                                            int workgroups, int iters,
                                                                            int mode, void *stream)
{
    if (!out || workgroups <= 0 || iters <= 0 || mode < 0 || mode > 3 ||
        out_floats < (long long)workgroups * 512)
        return 1;
    const dim3 grid(workgroups), block(512);
    hipStream_t s = (hipStream_t)stream;
    switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_stream_kernel<0>, grid, block, 0, s, (float *)out, iters); break;
    case 1: hipLaunchKernelGGL(mfma_stream_kernel<1>, grid, block, 0, s, (float *)out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_stream_kernel<2>, grid, block, 0, s, (float *)out, iters); break;
    default: hipLaunchKernelGGL(mfma_stream_kernel<3>, grid, block, 0, s, (float *)out, iters); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Read ceiling: `workgroups` workgroups of 256 threads read the `bytes` bytes
// at buf (a multiple of 16, 16-byte aligned) once; out: device buffer of at
// least workgroups * 256 words.  Returns 0, or 1 on bad arguments or a
// rejected launch.
extern "C" __attribute__((visibility("default"))) int fa_probe_read_stream(const void *buf, long long bytes,
                                                                            void *out, long long out_words,
                                                                            int workgroups, void *stream)
{
    if (!buf || !out || bytes <= 0 || (bytes & 15) || ((uintptr_t)buf & 15) || workgroups <= 0 ||
        out_words < (long long)workgroups * 256)
        return 1;
    hipLaunchKernelGGL(read_stream_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       (const uint4p *)buf, (size_t)(bytes / 16), (unsigned int *)out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// out: device buffer of 2 uint64 (shader cycles, 100 MHz ticks) written by
// the probe; window_ticks: window length in 100 MHz ticks (>= 1); stream:
// hipStream_t to launch on.  Returns 0, or 1 if the launch was rejected.
extern "C" __attribute__((visibility("default"))) int fa_clock_probe(void *out,
                                                                      unsigned long long window_ticks,
                                                                      void *stream)
{
    if (!out || window_ticks == 0) return 1;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (unsigned long long *)out, window_ticks);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
