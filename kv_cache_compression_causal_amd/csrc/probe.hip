// Measurement probes: the matrix-core and HBM-read rates this chip delivers
// in practice, reported next to the published peaks that the kernels'
// roofline fractions are taken against.  Not part of the attention path.
//
// mfma_probe_kernel: every wave runs 8 independent accumulator chains of
// v_mfma_f32_16x16x32_bf16 on register operands (each product depends on the
// previous one of its chain, so nothing can be hoisted out of the loop).
// read_probe_kernel: each workgroup streams its contiguous share with 16-byte
// loads, 16 in flight per lane, folded with xor so the loads are live.
#include "lt_internal.h"

namespace lt {
namespace {

// (No launch bounds: with them the compiler put the accumulators in AGPRs and
// moved them around every iteration.)
__global__ void mfma_probe_kernel(int iters, float *sink) {
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (bf16)(0.001f * (float)((t + e) & 31));
        b[e] = (bf16)(0.002f * (float)((t * 3 + e) & 15));
    }
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
        c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
        c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
        c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
    }
    const f32x4 cs = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    const float acc = cs[0] + cs[1] + cs[2] + cs[3];
    sink[(size_t)blockIdx.x * 256 + t] = acc;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                         unsigned *sink) {
    // Workgroup w reads its contiguous share of the buffer, UNR loads in
    // flight per lane.
    constexpr int UNR = 16;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * per;
    const size_t end = beg + per < n16 ? beg + per : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t i = beg + threadIdx.x; i < end; i += 256 * UNR) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const size_t j = i + (size_t)u * 256;
            v[u] = j < end ? p[j] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= v[u];
    }
    const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u) sink[blockIdx.x] = x;  // almost never taken; keeps the loads live
}

}  // namespace

hipError_t launch_mfma_probe(int blocks, int iters, float *sink, hipStream_t st) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, st, iters, sink);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *buf, size_t bytes, int blocks, unsigned *sink, hipStream_t st) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, st, (const u32x4 *)buf, bytes / 16,
                       sink);
    return hipGetLastError();
}

}  // namespace lt
