// common.h -- device helpers shared by the gfx950 kernels of libhaste.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace haste {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

#define HASTE_LDS(T, p) ((__attribute__((address_space(3))) T *)(p))

// 16x16 output, K = 32 bf16 per instruction.  Operand lane layout (both A
// and B): lane l holds row/col (l % 16) and K slots 8*(l/16) .. +7.
// Output: lane l holds rows 4*(l/16)+i (i = 0..3) of column l % 16.
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32 output, K = 16 bf16 per instruction.  A / B: lane l holds row / col
// (l % 32) and K slots 8*(l/32) .. +7.  Output: register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4 of column l % 32.
__device__ __forceinline__ f32x16 mfma32x32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16 output, K = 16: lane l holds K slots 4*(l/16) .. +3.
__device__ __forceinline__ f32x4 mfma16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each block of 16
// lanes, lane i receives, for k = 0..3, element (i % 4) of the 4-element
// run addressed by lane 4*k + i/4 of its block.
__device__ __forceinline__ i16x4 lds_read_tr(const void *lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(HASTE_LDS(i16x4, lds_ptr));
}

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
    return __uint_as_float(((unsigned)b) << 16);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ unsigned short f32_to_bf16(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(unsigned short, h);
}

// Two floats to a bf16 pair (lo in bits 0-15), one packed conversion.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

// Sigmoid-BCE on one logit, fp32, scaled by s.  e = exp(-|z|) is shared by
// the sigmoid and the softplus.  Hardware exp/log/rcp via the device math
// intrinsics (__expf, __logf).
struct BceOut {
    float dz;
    float loss;
};

__device__ __forceinline__ float bce_dz(float z, float y, float s) {
    float e = __expf(-fabsf(z));
    float r = __frcp_rn(1.0f + e);
    float sig = z >= 0.f ? r : e * r;
    return s * (sig - y);
}

__device__ __forceinline__ BceOut bce_both(float z, float y, float s) {
    float e = __expf(-fabsf(z));
    float r = __frcp_rn(1.0f + e);
    float sig = z >= 0.f ? r : e * r;
    float lin = fmaxf(z, 0.f) - y * z;
    // log(1+e) for e in (0, 1]: use log1p-accurate form for small e
    float l1p = (e < 1e-4f) ? e * (1.0f - 0.5f * e) : __logf(1.0f + e);
    BceOut o;
    o.dz = s * (sig - y);
    o.loss = s * (lin + l1p);
    return o;
}

// Fast forms for the fused epilogue (hardware v_exp_f32 / v_rcp_f32 /
// v_log_f32, about 1 ulp each).  sigmoid(z) from e = exp(-|z|):
// r = 1/(1+e) is sigmoid(|z|); sigmoid(z) = r for z >= 0, 1 - r otherwise.
// softplus(z) = max(z,0) + log(1+e); the log of a product of (1+e) factors
// (each in [1, 2]) replaces one log per logit (prod1p, log1p_pos below).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp_neg_abs(float z) {
    return __builtin_amdgcn_exp2f(fabsf(z) * -kLog2e);
}
__device__ __forceinline__ float fast_sigmoid(float z, float e, float &den) {
    den = 1.0f + e;
    const float r = __builtin_amdgcn_rcpf(den);
    return z >= 0.f ? r : 1.0f - r;
}
__device__ __forceinline__ float fast_log(float x) {
    return __builtin_amdgcn_logf(x) * kLn2;
}
// Products of (1 + e) factors are kept as q = product - 1: the small e of a
// large |z| would otherwise be rounded away against the 1 (an absolute error
// of 2^-24 on a term of size e), which dominates the loss when most logits
// are far below zero.  (1 + q)(1 + t) - 1 = q + t + q*t:
__device__ __forceinline__ float prod1p(float q, float t) { return __builtin_fmaf(q, t, q + t); }
// log(1 + q) for q >= 0 within a few ulps: with u = 1 + q rounded,
// log(u) * q / (u - 1) cancels the rounding of u (exact q when u = 1)
__device__ __forceinline__ float log1p_pos(float q) {
    const float u = 1.0f + q;
    const float d = u - 1.0f;
    return d == 0.f ? q : fast_log(u) * (q * __builtin_amdgcn_rcpf(d));
}

// Workgroup barrier that waits only for this wave's LDS operations.  Global
// loads, including global->LDS copies, stay in flight (__syncthreads would
// wait for those copies too).  Also a compiler memory barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// DPP lane exchange inside a row of 16 lanes (all lanes active).
// Controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned v) {
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
// Order-preserving map of a float to an unsigned key: a larger float has a
// larger key, -0 is taken as +0 (so that key order is the float order), and
// key 0 lies below every mapped number (-inf maps to 0x007fffff).  Integer
// max folds into one DPP instruction; a float max over a DPP operand does
// not (its operands are first quieted).
__device__ __forceinline__ unsigned f32_order_key(float v) {
    const unsigned b = __float_as_uint(v + 0.0f);
    return b ^ ((unsigned)((int)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(unsigned u) {
    return __uint_as_float(u ^ (~(unsigned)((int)u >> 31) | 0x80000000u));
}

// Over the 16 lanes of the row: the largest value, and the smallest key among
// the lanes holding it (every lane receives both); the max runs on order keys
__device__ __forceinline__ void row16_argmax(float &v, unsigned &key) {
    const unsigned u0 = f32_order_key(v);
    unsigned u = u0;
    u = max(u, dpp_u32<0xB1>(u));
    u = max(u, dpp_u32<0x4E>(u));
    u = max(u, dpp_u32<0x141>(u));
    u = max(u, dpp_u32<0x140>(u));
    unsigned k = u0 == u ? key : 0xffffffffu;
    k = min(k, dpp_u32<0xB1>(k));
    k = min(k, dpp_u32<0x4E>(k));
    k = min(k, dpp_u32<0x141>(k));
    k = min(k, dpp_u32<0x140>(k));
    v = f32_from_order_key(u);
    key = k;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Adds the workgroup's sum of v (any value per lane) to *loss with a single
// atomic add.  Called by every thread of the workgroup; part is LDS room for
// one float per wave that no wave reads any more.  Thousands of adds to one
// address at the end of a launch queue up one behind another: one per wave
// cost 10 us of a 29 us head launch and 7% of the dW pass at c2.
__device__ __forceinline__ void block_loss_add(float v, float *part, float *loss) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += part[i];
        atomicAdd(loss, t);
    }
}

}  // namespace haste
