// Device evaluation of the library's fixed-sequence math (exp_fixed,
// sigmoid_fixed, silu_fixed from common.h) over an array, so that the tests can
// compare it bit for bit with the CPU oracle's definitions on a dense sample.
// Test support only: built into libmoe_probe.so, outside the layer's ABI.
#include "common.h"

namespace {
__global__ __launch_bounds__(256) void math_kernel(const float* __restrict__ x, int64_t n,
                                                   float* __restrict__ e, float* __restrict__ sg,
                                                   float* __restrict__ sl) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float v = x[i];
    e[i] = moe::exp_fixed(v);
    sg[i] = moe::sigmoid_fixed(v);
    sl[i] = moe::silu_fixed(v);
}
}  // namespace

// e[i] = exp_fixed(x[i]), sg[i] = sigmoid_fixed(x[i]), sl[i] = silu_fixed(x[i]);
// device pointers of n floats each
extern "C" int moe_probe_math(const float* x, int64_t n, float* e, float* sg, float* sl, void* stream) {
    if (n < 0 || (n > 0 && (!x || !e || !sg || !sl))) return -2;
    if (n == 0) return 0;
    hipLaunchKernelGGL(math_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       x, n, e, sg, sl);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
