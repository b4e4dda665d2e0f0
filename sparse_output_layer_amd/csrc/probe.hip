// probe.hip -- a measurement utility, not a step of the layer: a dense loop
// of bf16 MFMAs on register operands, with no memory traffic, whose rate is
// the attainable matrix-core peak of the GPU it runs on (reported beside the
// datasheet peak in the roofline figures).
#include "common.h"
#include "kernels.h"

namespace haste {

constexpr int PROBE_CHAINS = 16;   // independent accumulators per wave

__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float *sink) {
    const int lane = threadIdx.x & 63;
    u32x4 ra, rb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // small bf16 values that depend on the lane
        ra[e] = 0x3c003c00u + (unsigned)((lane + e) & 7);
        rb[e] = 0x3b803b80u + (unsigned)((lane * 3 + e) & 7);
    }
    const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
    f32x4 acc[PROBE_CHAINS];
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = mfma32(a, b, acc[c]);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    // never true in practice; keeps the loop from being removed
    if (s == 12345.0f && blockIdx.x == 0 && threadIdx.x == 0) sink[0] = s;
}

hipError_t launch_probe_mfma(int blocks, int iters, float *sink, hipStream_t st) {
    hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
    return hipGetLastError();
}

}  // namespace haste
