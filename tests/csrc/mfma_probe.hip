// mfma_probe.hip -- tiny single-wavefront kernels that expose, lane by lane,
// the register layouts the attention kernel relies on, so a test can check
// them against a matrix product computed on the host:
//   * v_mfma_f32_32x32x16_f16: what each lane holds of A, B and the result;
//   * v_permlane32_swap: the two results for the same value given twice;
//   * fp32 -> fp16 packed conversion: rounding mode;
//   * v_mfma_f32_32x32x64_f8f6f4 (fp8 e4m3 operands): which A byte meets
//     which B byte, the result layout, the decoding of every fp8 code;
//   * ds_read_b64_tr_b8: which LDS bytes each lane receives;
//   * fp32 -> fp8 e4m3 packed conversion: rounding and byte placement;
//   * v_mfma_f32_4x4x4_16b_f16 (16 independent 4x4x4 blocks): which lanes'
//     halves meet which, and where each result lands.
// Test support only; not part of libfa.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef int int8v __attribute__((ext_vector_type(8)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

#define PROBE_API extern "C" __attribute__((visibility("default")))

// a, b: [64 lanes][8 halves] as the lanes' operand registers; c: [64][16].
__global__ void mfma_kernel(const half8 *a, const half8 *b, floatx16 *c)
{
    int l = threadIdx.x;
    floatx16 acc = {};
    c[l] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[l], b[l], acc, 0, 0, 0);
}

// out[0][l], out[1][l]: the two results of swapping x with itself.
__global__ void permlane_kernel(const float *x, float *out)
{
    int l = threadIdx.x;
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[l]), __float_as_uint(x[l]), false,
                                              false);
    out[l] = __uint_as_float(r[0]);
    out[64 + l] = __uint_as_float(r[1]);
}

__global__ void cvt_kernel(const float *x, _Float16 *y, int n)
{
    int i = 2 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (i + 1 < n) {
        float2v f = {x[i], x[i + 1]};
        half2v h = __builtin_convertvector(f, half2v);
        y[i] = h[0];
        y[i + 1] = h[1];
    }
}

PROBE_API int probe_mfma_32x32x16_f16(const void *a, const void *b, void *c, hipStream_t s)
{
    hipLaunchKernelGGL(mfma_kernel, dim3(1), dim3(64), 0, s, (const half8 *)a, (const half8 *)b,
                       (floatx16 *)c);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// n independent f16 MFMAs, one wavefront each: block i takes a[i], b[i]
// ([64 lanes][8 halves]) and the accumulator input cin[i] ([64][16]).
__global__ void mfma_f16_batch_kernel(const half8 *a, const half8 *b, const floatx16 *cin, floatx16 *c)
{
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    c[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[i], cin[i], 0, 0, 0);
}

PROBE_API int probe_mfma_32x32x16_f16_batch(const void *a, const void *b, const void *cin, void *c, int n,
                                            hipStream_t s)
{
    if (n <= 0) return 2;
    hipLaunchKernelGGL(mfma_f16_batch_kernel, dim3(n), dim3(64), 0, s, (const half8 *)a, (const half8 *)b,
                       (const floatx16 *)cin, (floatx16 *)c);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

PROBE_API int probe_permlane32_swap(const void *x, void *out, hipStream_t s)
{
    hipLaunchKernelGGL(permlane_kernel, dim3(1), dim3(64), 0, s, (const float *)x, (float *)out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// n must be even; x: n floats, y: n halves.
PROBE_API int probe_cvt_f16(const void *x, void *y, int n, hipStream_t s)
{
    if (n <= 0 || (n & 1)) return 2;
    int pairs = n / 2;
    hipLaunchKernelGGL(cvt_kernel, dim3((pairs + 255) / 256), dim3(256), 0, s, (const float *)x,
                       (_Float16 *)y, n);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// a, b: [64 lanes][32 fp8 bytes] as the lanes' operand registers; c: [64][16].
// scaled != 0: the scaled form with unit (E8M0 127) scales on both operands.
__global__ void mfma_f8_kernel(const int8v *a, const int8v *b, floatx16 *c, int scaled)
{
    int l = threadIdx.x;
    floatx16 acc = {};
    if (scaled)
        c[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], acc, 0, 0, 0, 127, 0, 127);
    else
        c[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], acc, 0, 0, 0, 0, 0, 0);
}

// n independent MFMAs, one wavefront each: block i takes its operands from
// a[i], b[i] ([64 lanes][32 fp8 bytes]) and its accumulator input from
// cin[i] ([64][16]), and writes c[i].  Unscaled form.
__global__ void mfma_f8_batch_kernel(const int8v *a, const int8v *b, const floatx16 *cin, floatx16 *c)
{
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    c[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[i], cin[i], 0, 0, 0, 0, 0, 0);
}

PROBE_API int probe_mfma_32x32x64_f8_batch(const void *a, const void *b, const void *cin, void *c, int n,
                                           hipStream_t s)
{
    if (n <= 0) return 2;
    hipLaunchKernelGGL(mfma_f8_batch_kernel, dim3(n), dim3(64), 0, s, (const int8v *)a, (const int8v *)b,
                       (const floatx16 *)cin, (floatx16 *)c);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// LDS[0..1023] = src; lane l reads 8 bytes with ds_read_b64_tr_b8 at byte
// offset addr[l] (a multiple of 8, at most 1016: checked on the host).
__global__ void tr8_kernel(const int *src, const int *addr, int2v *out)
{
    __shared__ int lds[256];
    int l = threadIdx.x;
    for (int i = l; i < 256; i += 64) lds[i] = src[i];
    __syncthreads();
    typedef __attribute__((address_space(3))) int2v lds_int2v;
    lds_int2v *p = (lds_int2v *)((__attribute__((address_space(3))) char *)lds + addr[l]);
    out[l] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(p);
}

// y[4i..4i+3]: x[4i], x[4i+1] packed into the low half of a dword and
// x[4i+2], x[4i+3] into its high half.
__global__ void cvt_fp8_kernel(const float *x, int *y, int n4)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4) {
        int r = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i], x[4 * i + 1], 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i + 2], x[4 * i + 3], r, true);
        y[i] = r;
    }
}

PROBE_API int probe_mfma_32x32x64_f8(const void *a, const void *b, void *c, int scaled, hipStream_t s)
{
    hipLaunchKernelGGL(mfma_f8_kernel, dim3(1), dim3(64), 0, s, (const int8v *)a, (const int8v *)b,
                       (floatx16 *)c, scaled);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// src: 1024 bytes (device); addr: 64 ints (host and device copies: the host
// copy is checked); out: 64 x 8 bytes.
PROBE_API int probe_ds_read_tr8(const void *src, const int *addr_host, const void *addr_dev, void *out,
                                hipStream_t s)
{
    for (int l = 0; l < 64; ++l)
        if (addr_host[l] < 0 || addr_host[l] > 1016 || (addr_host[l] & 7)) return 2;
    hipLaunchKernelGGL(tr8_kernel, dim3(1), dim3(64), 0, s, (const int *)src, (const int *)addr_dev,
                       (int2v *)out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// n must be a positive multiple of 4; x: n floats, y: n bytes.
PROBE_API int probe_cvt_fp8(const void *x, void *y, int n, hipStream_t s)
{
    if (n <= 0 || (n & 3)) return 2;
    int n4 = n / 4;
    hipLaunchKernelGGL(cvt_fp8_kernel, dim3((n4 + 255) / 256), dim3(256), 0, s, (const float *)x,
                       (int *)y, n4);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// a, b: [64 lanes][4 halves] as the lanes' operand registers; c: [64][4].
__global__ void mfma4_kernel(const half4 *a, const half4 *b, float4v *c)
{
    int l = threadIdx.x;
    float4v acc = {};
    c[l] = __builtin_amdgcn_mfma_f32_4x4x4f16(a[l], b[l], acc, 0, 0, 0);
}

PROBE_API int probe_mfma_4x4x4_16b_f16(const void *a, const void *b, void *c, hipStream_t s)
{
    hipLaunchKernelGGL(mfma4_kernel, dim3(1), dim3(64), 0, s, (const half4 *)a, (const half4 *)b,
                       (float4v *)c);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
