// read_probe.hip -- a plain HBM read kernel, the ceiling the decode kernels'
// streaming is compared with.  Measurement infrastructure for bench.py; not
// part of the libkvq ABI.
//
// Every wave reads whole 1 KiB pieces (16 bytes per lane, one contiguous wave
// request), sweeping the buffer with a stride of all waves, UNROLL pieces in
// flight per wave, and folds them with xor into one word per thread (written
// out, so no load is dead).  With 8 waves per workgroup and one workgroup
// per CU this is the access pattern of the decode kernels without their math.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int UNROLL>
__global__ __launch_bounds__(512) void read_probe_kernel(const uint4* __restrict__ src, long n_pieces,
                                                          uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const long n_waves = (long)gridDim.x * (blockDim.x >> 6);
    long p = (long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    uint4 acc = {0u, 0u, 0u, 0u};
    for (; p + (UNROLL - 1) * n_waves < n_pieces; p += UNROLL * n_waves) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = src[(p + u * n_waves) * 64 + lane];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            acc.x ^= v[u].x;
            acc.y ^= v[u].y;
            acc.z ^= v[u].z;
            acc.w ^= v[u].w;
        }
    }
    for (; p < n_pieces; p += n_waves) {
        const uint4 v = src[p * 64 + lane];
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

// Reads `bytes` (a multiple of 1024, 16-byte aligned) of d_src once on
// `stream` with n_wg workgroups of waves * 64 threads; d_out holds
// n_wg * waves * 64 words.  unroll: 2, 4, 8 or 16 pieces in flight per wave.
// Returns 0, or -1 on a bad argument, or the HIP error of the launch.
extern "C" int kvq_probe_read(const void* d_src, size_t bytes, uint32_t* d_out, int n_wg, int waves, int unroll,
                              void* stream) {
    if (d_src == nullptr || d_out == nullptr || bytes % 1024 != 0 || ((uintptr_t)d_src & 15) != 0 || n_wg < 1 ||
        waves < 1 || waves > 8)
        return -1;
    const long n = (long)(bytes / 1024);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(n_wg), block(waves * 64);
    const uint4* src = static_cast<const uint4*>(d_src);
    switch (unroll) {
        case 2: hipLaunchKernelGGL(read_probe_kernel<2>, grid, block, 0, s, src, n, d_out); break;
        case 4: hipLaunchKernelGGL(read_probe_kernel<4>, grid, block, 0, s, src, n, d_out); break;
        case 8: hipLaunchKernelGGL(read_probe_kernel<8>, grid, block, 0, s, src, n, d_out); break;
        case 16: hipLaunchKernelGGL(read_probe_kernel<16>, grid, block, 0, s, src, n, d_out); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}
