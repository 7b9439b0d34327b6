// read_probe.hip -- a plain HBM read kernel, the ceiling the decode kernels'
// streaming is compared with.  Measurement infrastructure for bench.py; not
// part of the libkvq ABI.
//
// Every wave reads whole 1 KiB pieces (16 bytes per lane, one contiguous wave
// request), sweeping the buffer with a stride of all waves, UNROLL pieces in
// flight per wave, with or without the non-temporal hint, and folds them with
// xor into one word per thread (written out, so no load is dead).  With 8 waves per workgroup and one workgroup
// per CU this is the access pattern of the decode kernels without their math.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// NT: non-temporal loads (the cache-policy hint of data read once).
template <int UNROLL, bool NT>
__global__ __launch_bounds__(512) void read_probe_kernel(const u32x4* __restrict__ src, long n_pieces,
                                                          uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const long n_waves = (long)gridDim.x * (blockDim.x >> 6);
    long p = (long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    auto load = [&](long piece) { return NT ? __builtin_nontemporal_load(src + piece * 64 + lane) : src[piece * 64 + lane]; };
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; p + (UNROLL - 1) * n_waves < n_pieces; p += UNROLL * n_waves) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = load(p + u * n_waves);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
    }
    for (; p < n_pieces; p += n_waves) acc ^= load(p);
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

template <bool NT>
int launch_probe(const u32x4* src, long n, uint32_t* d_out, dim3 grid, dim3 block, int unroll, hipStream_t s) {
    switch (unroll) {
        case 2: hipLaunchKernelGGL((read_probe_kernel<2, NT>), grid, block, 0, s, src, n, d_out); break;
        case 4: hipLaunchKernelGGL((read_probe_kernel<4, NT>), grid, block, 0, s, src, n, d_out); break;
        case 8: hipLaunchKernelGGL((read_probe_kernel<8, NT>), grid, block, 0, s, src, n, d_out); break;
        case 16: hipLaunchKernelGGL((read_probe_kernel<16, NT>), grid, block, 0, s, src, n, d_out); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 1024, 16-byte aligned) of d_src once on
// `stream` with n_wg workgroups of waves * 64 threads; d_out holds
// n_wg * waves * 64 words.  unroll: 2, 4, 8 or 16 pieces in flight per wave;
// nontemporal: 1 for loads with the non-temporal hint, 0 for plain loads.
// Returns 0, or -1 on a bad argument, or the HIP error of the launch.
extern "C" int kvq_probe_read(const void* d_src, size_t bytes, uint32_t* d_out, int n_wg, int waves, int unroll,
                              int nontemporal, void* stream) {
    if (d_src == nullptr || d_out == nullptr || bytes % 1024 != 0 || ((uintptr_t)d_src & 15) != 0 || n_wg < 1 ||
        waves < 1 || waves > 8)
        return -1;
    const long n = (long)(bytes / 1024);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(n_wg), block(waves * 64);
    const u32x4* src = static_cast<const u32x4*>(d_src);
    return nontemporal ? launch_probe<true>(src, n, d_out, grid, block, unroll, s)
                       : launch_probe<false>(src, n, d_out, grid, block, unroll, s);
}
