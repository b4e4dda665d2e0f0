// f32path.hip -- fp32 kernels for small problems where fp32 inputs must be
// kept at full precision (one thread per output, VALU fp32 FMAs), plus the
// index-check and top-K merge utilities.
//
// Same definitions as the bf16 path (HASTE summary page, section "Method",
// items 1 and 2): z[b][t] = sum_f X[b][idx[t/G][f]] * W[t][f]; the head is a
// dense classifier; sigmoid-BCE against the row's positives.
#include "common.h"
#include "kernels.h"

namespace haste {

__device__ __forceinline__ float is_positive(const int32_t *row_ptr, const int32_t *labels, int b,
                                             int64_t gid) {
    for (int k = row_ptr[b]; k < row_ptr[b + 1]; ++k)
        if ((int64_t)labels[k] == gid) return 1.f;
    return 0.f;
}

// accurate fp32 BCE (libm-quality expf / log1pf)
__device__ __forceinline__ void bce_f32(float z, float y, float s, float &dz, float &l) {
    const float e = expf(-fabsf(z));
    const float sig = z >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
    dz = s * (sig - y);
    l = s * ((fmaxf(z, 0.f) - y * z) + log1pf(e));
}

__global__ void k_f32_tail_logits(F32Args a, int store_z, int bce, int loss) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    float l = 0.f;
    if (i < (int64_t)a.B * a.L) {
        const int b = (int)(i / a.L);
        const int64_t t = i % a.L;
        const int32_t *ix = a.idx + (t / a.G) * a.F;
        const float *wr = a.W + t * a.F;
        const float *xr = a.X + (int64_t)b * a.D;
        float z = 0.f;
        for (int f = 0; f < a.F; ++f) z = fmaf(xr[ix[f]], wr[f], z);
        if (store_z) a.Z[i] = z;
        if (bce) {
            float dz;
            bce_f32(z, is_positive(a.row_ptr, a.labels, b, a.label_offset + t), a.s, dz, l);
            if (a.dZ) a.dZ[i] = dz;
        }
    }
    if (loss && a.loss) {
        __shared__ float s_loss[16];
        block_loss_add(l, s_loss, a.loss);
    }
}

__global__ void k_f32_tail_dw(F32Args a) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t rows = a.Ng * a.G;
    if (i >= rows * a.F) return;
    const int64_t t = i / a.F;
    const int f = (int)(i % a.F);
    float acc = 0.f;
    if (t < a.L) {
        const int d = a.idx[(t / a.G) * a.F + f];
        for (int b = 0; b < a.B; ++b) acc = fmaf(a.X[(int64_t)b * a.D + d], a.dZ[(int64_t)b * a.L + t], acc);
    }
    a.dW[i] = acc;
}

// one thread per (row b, group g, slot f): dX[b][idx[g][f]] += sum_j dz*w
__global__ void k_f32_tail_dx(F32Args a) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= (int64_t)a.B * a.Ng * a.F) return;
    const int f = (int)(i % a.F);
    const int64_t g = (i / a.F) % a.Ng;
    const int b = (int)(i / (a.F * a.Ng));
    float acc = 0.f;
    for (int j = 0; j < a.G; ++j) {
        const int64_t t = g * a.G + j;
        if (t >= a.L) break;
        acc = fmaf(a.dZ[(int64_t)b * a.L + t], a.W[t * a.F + f], acc);
    }
    atomicAdd(a.dX + (int64_t)b * a.D + a.idx[g * a.F + f], acc);
}

// head: W is Wh (H x D), L is H, G/F unused
__global__ void k_f32_head_logits(F32Args a, int store_z, int bce, int loss) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    float l = 0.f;
    if (i < (int64_t)a.B * a.L) {
        const int b = (int)(i / a.L);
        const int64_t h = i % a.L;
        const float *wr = a.W + h * a.D;
        const float *xr = a.X + (int64_t)b * a.D;
        float z = 0.f;
        for (int d = 0; d < a.D; ++d) z = fmaf(xr[d], wr[d], z);
        if (store_z) a.Z[i] = z;
        if (bce) {
            float dz;
            bce_f32(z, is_positive(a.row_ptr, a.labels, b, a.label_offset + h), a.s, dz, l);
            if (a.dZ) a.dZ[i] = dz;
        }
    }
    if (loss && a.loss) {
        __shared__ float s_loss[16];
        block_loss_add(l, s_loss, a.loss);
    }
}

__global__ void k_f32_head_dw(F32Args a) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= a.L * a.D) return;
    const int64_t h = i / a.D;
    const int d = (int)(i % a.D);
    float acc = 0.f;
    for (int b = 0; b < a.B; ++b) acc = fmaf(a.dZ[(int64_t)b * a.L + h], a.X[(int64_t)b * a.D + d], acc);
    a.dW[i] = acc;
}

__global__ void k_f32_head_dx(F32Args a) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= (int64_t)a.B * a.D) return;
    const int b = (int)(i / a.D), d = (int)(i % a.D);
    float acc = 0.f;
    for (int64_t h = 0; h < a.L; ++h) acc = fmaf(a.dZ[(int64_t)b * a.L + h], a.W[h * a.D + d], acc);
    a.dX[i] += acc;
}

static dim3 blocks_for(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

hipError_t launch_f32_tail_logits(const F32Args &a, bool store_z, bool bce, bool loss,
                                  hipStream_t st) {
    const int64_t n = (int64_t)a.B * a.L;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_f32_tail_logits, blocks_for(n), dim3(256), 0, st, a, (int)store_z,
                       (int)bce, (int)loss);
    return hipGetLastError();
}
hipError_t launch_f32_tail_dw(const F32Args &a, hipStream_t st) {
    const int64_t n = a.Ng * a.G * a.F;
    hipLaunchKernelGGL(k_f32_tail_dw, blocks_for(n), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_f32_tail_dx(const F32Args &a, hipStream_t st) {
    const int64_t n = (int64_t)a.B * a.Ng * a.F;
    hipLaunchKernelGGL(k_f32_tail_dx, blocks_for(n), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_f32_head_logits(const F32Args &a, bool store_z, bool bce, bool loss,
                                  hipStream_t st) {
    const int64_t n = (int64_t)a.B * a.L;
    hipLaunchKernelGGL(k_f32_head_logits, blocks_for(n), dim3(256), 0, st, a, (int)store_z,
                       (int)bce, (int)loss);
    return hipGetLastError();
}
hipError_t launch_f32_head_dw(const F32Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_f32_head_dw, blocks_for(a.L * a.D), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_f32_head_dx(const F32Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_f32_head_dx, blocks_for((int64_t)a.B * a.D), dim3(256), 0, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------ utilities
// first_bad = min over groups whose index row is not strictly increasing
// inside [0, D); caller presets it to INT_MAX and maps INT_MAX -> -1.
__global__ void k_validate(const int32_t *idx, int64_t Ng, int F, int D, int32_t *first_bad) {
    const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (g >= Ng) return;
    const int32_t *r = idx + g * F;
    bool bad = false;
    for (int f = 0; f < F; ++f) {
        const int v = r[f];
        if (v < 0 || v >= D) bad = true;
        if (f > 0 && v <= r[f - 1]) bad = true;
    }
    if (bad) atomicMin(first_bad, (int32_t)(g < 0x7fffffff ? g : 0x7ffffffe));
}

__global__ void k_validate_fix(int32_t *first_bad) {
    if (*first_bad == 0x7fffffff) *first_bad = -1;
}

hipError_t launch_validate(const int32_t *idx, int64_t Ng, int F, int D, int32_t *first_bad,
                           hipStream_t st) {
    hipError_t e = launch_fill_u32(first_bad, 0x7fffffffu, 1, st);
    if (e != hipSuccess) return e;
    if (Ng > 0) {
        hipLaunchKernelGGL(k_validate, blocks_for(Ng), dim3(256), 0, st, idx, Ng, F, D, first_bad);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_validate_fix, dim3(1), dim3(1), 0, st, first_bad);
    return hipGetLastError();
}

// (value desc, id asc) order
__device__ __forceinline__ bool before(float va, int32_t ia, float vb, int32_t ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ void k_topk_merge(int B, int K, const float *av, const int32_t *ai, const float *bv,
                             const int32_t *bi, float *ov, int32_t *oi) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    int x = 0, y = 0;
    for (int k = 0; k < K; ++k) {
        const bool ha = x < K, hb = y < K;  // K picks from 2K: one side always has one
        const float va = ha ? av[b * K + x] : 0.f, vb = hb ? bv[b * K + y] : 0.f;
        const int32_t ia = ha ? ai[b * K + x] : 0, ib = hb ? bi[b * K + y] : 0;
        const bool takea = ha && (!hb || before(va, ia, vb, ib));
        if (takea) {
            ov[b * K + k] = va;
            oi[b * K + k] = ia;
            ++x;
        } else {
            ov[b * K + k] = vb;
            oi[b * K + k] = ib;
            ++y;
        }
    }
}

hipError_t launch_topk_merge(int B, int K, const float *av, const int32_t *ai, const float *bv,
                             const int32_t *bi, float *ov, int32_t *oi, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_topk_merge, blocks_for(B), dim3(256), 0, st, B, K, av, ai, bv, bi, ov, oi);
    return hipGetLastError();
}

}  // namespace haste
