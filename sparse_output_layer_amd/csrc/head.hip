// head.hip -- the dense head classifier (HASTE summary page, section
// "Method", item 2: the frequent labels use a standard dense classifier) as
// bf16 MFMA GEMMs on gfx950.
//
// One templated GEMM covers the three contractions of a training step:
//   forward  Zh  = X  Wh^T   (A = X [b][d],  K-major; B = Wh [h][d], K-major)
//   weights  dWh = dZh^T X   (A = dZh [b][h] M-major; B = X [b][d], N-major)
//   input    dX += dZh Wh    (A = dZh [b][h] K-major; B = Wh [h][d], N-major)
// K-major tiles are read from LDS with 16-byte reads; M/N-major tiles with
// the transposing ds_read_b64_tr_b16, so no operand is ever transposed in
// HBM.  128x128 output tile, K step 32, 4 waves of 64x64, LDS double
// buffered.  Epilogues: fused sigmoid-BCE (loss + dz), bf16 store, fp32
// atomic add (split-K).
#include "common.h"
#include "kernels.h"

namespace haste {

constexpr int TM = 128, TN = 128, TK = 32;
constexpr int KROW = TK + 8;    // K-major LDS row (shorts): 80 B, 16 B aligned
constexpr int MROW = TM + 8;    // M/N-major LDS row (shorts): 272 B

// Load one 128 x 32 operand tile from HBM into registers (2 x 16 B per
// thread), masked to zero outside [0, rows) x [0, K).
template <bool KMAJ>
__device__ __forceinline__ void load_tile(const unsigned short *__restrict__ P, int ld, int r0,
                                          int rows, int k0, int K, u32x4 (&v)[2]) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int i = threadIdx.x + it * 256;
        int r, k;
        if (KMAJ) {  // row r (M), 4 segments of 8 along K
            r = i >> 2;
            k = (i & 3) * 8;
        } else {     // row k (32 rows), 16 segments of 8 along M
            k = i >> 4;
            r = (i & 15) * 8;
        }
        const int gr = r0 + r, gk = k0 + k;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (KMAJ) {
            if (gr < rows && gk < K) {
                if (gk + 8 <= K) {
                    x = *(const u32x4 *)(P + (int64_t)gr * ld + gk);
                } else {
                    unsigned short tmp[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) tmp[e] = gk + e < K ? P[(int64_t)gr * ld + gk + e] : 0;
                    x = __builtin_bit_cast(u32x4, tmp);
                }
            }
        } else {
            if (gk < K && gr < rows) {
                if (gr + 8 <= rows) {
                    x = *(const u32x4 *)(P + (int64_t)gk * ld + gr);
                } else {
                    unsigned short tmp[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) tmp[e] = gr + e < rows ? P[(int64_t)gk * ld + gr + e] : 0;
                    x = __builtin_bit_cast(u32x4, tmp);
                }
            }
        }
        v[it] = x;
    }
}

template <bool KMAJ>
__device__ __forceinline__ void store_tile(unsigned short *S, const u32x4 (&v)[2]) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int i = threadIdx.x + it * 256;
        if (KMAJ) {
            *(u32x4 *)(S + (i >> 2) * KROW + (i & 3) * 8) = v[it];
        } else {
            *(u32x4 *)(S + (i >> 4) * MROW + (i & 15) * 8) = v[it];
        }
    }
}

// MFMA operand (16 rows of the tile starting at r, K slots 8q..8q+7).
template <bool KMAJ>
__device__ __forceinline__ bf16x8 read_operand(const unsigned short *S, int r, int q, int m) {
    if (KMAJ) {
        return *(const bf16x8 *)(S + (r + m) * KROW + 8 * q);
    } else {
        // transposed read: lane (q, m) points at K row 8q+4h+m/4, columns r+4(m%4)
        i16x4 a0 = lds_read_tr(S + (8 * q + (m >> 2)) * MROW + r + 4 * (m & 3));
        i16x4 a1 = lds_read_tr(S + (8 * q + 4 + (m >> 2)) * MROW + r + 4 * (m & 3));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

template <bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs g) {
    constexpr int ASZ = A_KMAJ ? TM * KROW : TK * MROW;
    constexpr int BSZ = B_KMAJ ? TN * KROW : TK * MROW;
    __shared__ __attribute__((aligned(16))) unsigned short sm[2 * (ASZ + BSZ)];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q = lane >> 4, m = lane & 15;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
    const int kbeg = blockIdx.z * g.k_split;
    int kend = kbeg + g.k_split;
    if (kend > g.K) kend = g.K;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    u32x4 ra[2], rb[2];
    const int nk = (kend - kbeg + TK - 1) / TK;
    if (nk > 0) {
        load_tile<A_KMAJ>(g.A, g.lda, m0, g.M, kbeg, kend, ra);
        load_tile<B_KMAJ>(g.Bm, g.ldb, n0, g.N, kbeg, kend, rb);
        store_tile<A_KMAJ>(sm, ra);
        store_tile<B_KMAJ>(sm + ASZ, rb);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        unsigned short *SA = sm + cur * (ASZ + BSZ);
        unsigned short *SB = SA + ASZ;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = kbeg + (kt + 1) * TK;
            load_tile<A_KMAJ>(g.A, g.lda, m0, g.M, k0, kend, ra);
            load_tile<B_KMAJ>(g.Bm, g.ldb, n0, g.N, k0, kend, rb);
        }
        bf16x8 av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = read_operand<A_KMAJ>(SA, wm + 16 * i, q, m);
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = read_operand<B_KMAJ>(SB, wn + 16 * j, q, m);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
        if (more) {
            unsigned short *NA = sm + (cur ^ 1) * (ASZ + BSZ);
            store_tile<A_KMAJ>(NA, ra);
            store_tile<B_KMAJ>(NA + ASZ, rb);
        }
        __syncthreads();
    }

    // epilogue: lane owns C[m0+wm+16i+4q+e][n0+wn+16j+m]
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn + 16 * j + m;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm + 16 * i + 4 * q + e;
                if (row >= g.M || col >= g.N) continue;
                const float v = acc[i][j][e];
                const int64_t o = (int64_t)row * g.N + col;
                if (EPI == EPI_BCE) {
                    if (g.bitmap) {
                        const float y = (float)((g.bitmap[(int64_t)row * g.bm_words + (col >> 5)] >>
                                                 (col & 31)) & 1u);
                        BceOut r = bce_both(v, y, g.s);
                        lsum += r.loss;
                        if (g.dZout) g.dZout[o] = f32_to_bf16(r.dz);
                    }
                    if (g.Zout) g.Zout[o] = f32_to_bf16(v);
                } else if (EPI == EPI_STORE16) {
                    g.C16[o] = f32_to_bf16(v);
                } else {
                    atomicAdd(g.C32 + o, v);
                }
            }
        }
    if (EPI == EPI_BCE && g.loss) {
        float v = wave_sum(lsum);
        if (lane == 0) atomicAdd(g.loss, v);
    }
}

hipError_t launch_gemm(bool a_kmaj, bool b_kmaj, int epi, const GemmArgs &g, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
    const int splits = (g.K + g.k_split - 1) / g.k_split;
    dim3 grid((g.N + TN - 1) / TN, (g.M + TM - 1) / TM, splits);
#define GL(AK, BK, E) \
    hipLaunchKernelGGL((k_gemm<AK, BK, E>), grid, dim3(256), 0, st, g)
    if (epi == EPI_BCE && a_kmaj && b_kmaj) GL(true, true, EPI_BCE);
    else if (epi == EPI_STORE16 && !a_kmaj && !b_kmaj) GL(false, false, EPI_STORE16);
    else if (epi == EPI_ATOMIC32 && a_kmaj && !b_kmaj) GL(true, false, EPI_ATOMIC32);
    else return hipErrorInvalidValue;
#undef GL
    return hipGetLastError();
}

// bm[b][h/32] |= bit(h%32) for every positive of row b with global id in
// [off, off+H).  bm must be zeroed first.
__global__ void k_head_bitmap(const int32_t *row_ptr, const int32_t *labels, int nnz, int B,
                              int64_t off, int H, uint32_t *bm, int words) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    const int64_t h = (int64_t)labels[k] - off;
    if (h < 0 || h >= H) return;
    int lo = 0, hi = B;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (row_ptr[mid] <= k) lo = mid; else hi = mid;
    }
    atomicOr(bm + (int64_t)lo * words + (h >> 5), 1u << (h & 31));
}

hipError_t launch_head_bitmap(const int32_t *row_ptr, const int32_t *labels, int nnz, int B,
                              int64_t off, int H, uint32_t *bm, int words, hipStream_t st) {
    hipError_t e = launch_fill_u32(bm, 0u, (size_t)B * words, st);
    if (e != hipSuccess || nnz <= 0) return e;
    hipLaunchKernelGGL(k_head_bitmap, dim3((nnz + 255) / 256), dim3(256), 0, st, row_ptr, labels,
                       nnz, B, off, H, bm, words);
    return hipGetLastError();
}

}  // namespace haste
