// mfma_probe.hip -- tiny single-wavefront kernels that expose, lane by lane,
// the register layouts the attention kernel relies on, so a test can check
// them against a matrix product computed on the host:
//   * v_mfma_f32_32x32x16_f16: what each lane holds of A, B and the result;
//   * v_permlane32_swap: the two results for the same value given twice;
//   * fp32 -> fp16 packed conversion: rounding mode.
// Test support only; not part of libfa.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));

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
