// hadamard.hip -- the normalized Hadamard rotation of K, V, q (and back of the
// output) for the 2-bit cache: every row of dim values becomes x H / sqrt(dim),
// H of Sylvester's construction ("OSCAR2 KV Cache benchmark", rotation model
// conversion: the pages bake a Hadamard rotation per head into the model so
// that the 2-bit cache holds rotated K and V).  H / sqrt(dim) is orthogonal
// and symmetric: scores of rotated q and k are unchanged, and one more
// rotation undoes the rotated output.
//
// One workgroup per row, dim / 2 threads: the fast Walsh-Hadamard transform in
// LDS, log2(dim) butterfly stages (a, b) -> (a + b, a - b) over pairs h apart,
// then one product by the fp32 value of 1/sqrt(dim).  Every thread owns one
// pair per stage, so a barrier between stages is the only synchronisation.
// The order of the fp32 operations is fixed (deterministic).
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(512) void hadamard_kernel(float* __restrict__ x, int dim, int log2dim, float scale) {
#pragma clang fp contract(off)
    extern __shared__ float buf[];
    float* row = x + (size_t)blockIdx.x * dim;
    const int t = threadIdx.x, half = dim >> 1;
    buf[t] = row[t];
    buf[t + half] = row[t + half];
    __syncthreads();
    for (int s = 0; s < log2dim; ++s) {
        const int h = 1 << s;
        const int i = ((t >> s) << (s + 1)) | (t & (h - 1)), j = i + h;
        const float a = buf[i], b = buf[j];
        buf[i] = a + b;
        buf[j] = a - b;
        __syncthreads();
    }
    row[t] = buf[t] * scale;
    row[t + half] = buf[t + half] * scale;
}

}  // namespace

hipError_t launch_hadamard(float* x, int64_t n_rows, int dim, hipStream_t stream) {
    int log2dim = 0;
    while ((1 << log2dim) < dim) ++log2dim;
    const float scale = (float)(1.0 / sqrt((double)dim));
    hipLaunchKernelGGL(hadamard_kernel, dim3((unsigned)n_rows), dim3(dim / 2), dim * sizeof(float), stream, x, dim,
                       log2dim, scale);
    return hipGetLastError();
}

}  // namespace kvq
