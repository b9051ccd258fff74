// Matrix-core throughput probe: the MFMA shapes the path uses, issued back to
// back with no memory traffic, so a timed launch gives the rate this GPU
// actually sustains for them (the published peaks assume the top clock).
//   kind 0: v_mfma_f32_16x16x32_f16 (the attention's QK and PV), 16,384 flop
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 x E2M1 (the prefill
//           indexer), 131,072 flop
// Each wave runs four independent accumulator chains so the matrix core never
// waits on a result; operands come from the lane index so nothing is constant
// folded, and each lane writes one sum so nothing is dead.
#include <hip/hip_runtime.h>

#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void k_mfma_probe(int64_t iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    if constexpr (KIND == 0) {
        v8h a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (_Float16)(0.001f * (lane + i));
            b[i] = (_Float16)(0.002f * (lane - i));
        }
        // distinct starting values keep the compiler from merging the chains
        v4f c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {1.f, 1.f, 1.f, 1.f}, c2 = {2.f, 2.f, 2.f, 2.f}, c3 = {3.f, 3.f, 3.f, 3.f};
        for (int64_t it = 0; it < iters; it += 4) {  // iters: a multiple of 4
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c3, 0, 0, 0);
            }
        }
        const v4f t = c0 + c1 + c2 + c3;
        s = t[0] + t[1] + t[2] + t[3];
    } else {
        v8i a = {lane * 0x01010101, lane ^ 0x3c3c3c3c, 0, 0, 0, 0, 0, 0};
        a[2] = a[0] ^ 0x11111111;
        a[3] = a[1] ^ 0x22222222;
        v8i b = {lane * 0x00ff00ff, lane ^ 0x5a5a5a5a, 0, 0, 0, 0, 0, 0};
        b[2] = b[0] ^ 0x44444444;
        b[3] = b[1] ^ 0x77777777;
        v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            c1[i] = 1.f;
            c2[i] = 2.f;
            c3[i] = 3.f;
        }
        for (int64_t it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 4, 4, 0, 127, 0, 127);
            c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 4, 4, 0, 127, 0, 127);
            c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 4, 4, 0, 127, 0, 127);
            c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 4, 4, 0, 127, 0, 127);
        }
        const v16f t = c0 + c1 + c2 + c3;
#pragma unroll
        for (int i = 0; i < 16; ++i) s += t[i];
    }
    sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

hipError_t launch_mfma_probe(int kind, int blocks, int64_t iters, float* sink, hipStream_t st) {
    if (kind == 0)
        hipLaunchKernelGGL(k_mfma_probe<0>, dim3(blocks), dim3(kProbeThreads), 0, st, iters, sink);
    else
        hipLaunchKernelGGL(k_mfma_probe<1>, dim3(blocks), dim3(kProbeThreads), 0, st, iters, sink);
    return hipGetLastError();
}

}  // namespace csa
