// tail.hip -- gfx950 kernels of the sparse tail: group-shared fixed fan-in
// (HASTE summary page, gist.science, section "Method", item 1: the labels of
// a group share one fan-in index set and keep their own weights; the
// group's features are gathered once into on-chip memory and reused by all
// G labels through a dense matrix-core contraction).
//
// Data layout in HBM (all row-major):
//   XT  : D x Bp bf16, the transpose of X, zero-padded to Bp columns, so the
//         features a group gathers are contiguous rows of B values
//   idx : Ng x F int32, W / dW : (Ng*G) x F bf16 (label-major), dX : B x D f32
//
// Kernel T1 ("gather + contract + epilogue + dW"): one workgroup per run of
//   4*RW consecutive groups, every row of the batch.  The batch is streamed
//   in chunks of BC rows: the chunk XT[:, c*BC:(c+1)*BC] is staged once in
//   LDS and every group of the run gathers its F rows from it with
//   transposing LDS reads (ds_read_b64_tr_b16) straight into MFMA operands.
//   Z_g = X_g W_g runs on bf16 MFMA with W_g held in VGPRs for the whole
//   run; the sigmoid-BCE epilogue turns Z into dz in registers, and
//   dW_g += X_g^T dz accumulates in AGPRs across chunks, so dW_g is written
//   once, in bf16, with no cross-workgroup reduction.
// Kernel T2 ("dX"): one workgroup per (chunk of BC2 rows, range of groups).
//   It recomputes Z_g for its rows from the LDS-resident chunk, turns it
//   into dz, and accumulates dX_chunk += dz_g * W~_g in MFMA registers,
//   where W~_g is the group's weight slice expanded over all D features
//   (zero outside idx_g; built per group in LDS from an inverse index).
//   This keeps the scatter-add of the pages' backward pass out of LDS
//   atomics: dX is flushed to HBM once per workgroup with global atomics.
#include "common.h"
#include "kernels.h"

namespace haste {

// ------------------------------------------------------------------ prep
// XT[d][b] = X[b][d] for b < B, 0 for B <= b < Bp.  64x64 tiles via LDS.
__global__ __launch_bounds__(256) void k_transpose_x(const unsigned short *__restrict__ X,
                                                     unsigned short *__restrict__ XT,
                                                     int B, int D, int Bp) {
    __shared__ unsigned short t[64][66];
    const int b0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int bb = i / 64, dd = i % 64;
        int b = b0 + bb, d = d0 + dd;
        t[bb][dd] = (b < B && d < D) ? X[(int64_t)b * D + d] : (unsigned short)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int dd = i / 64, bb = i % 64;
        int b = b0 + bb, d = d0 + dd;
        if (d < D && b < Bp) XT[(int64_t)d * Bp + b] = t[bb][dd];
    }
}

hipError_t launch_transpose_x(const unsigned short *X, unsigned short *XT, int B,
                              int D, int Bp, hipStream_t st) {
    dim3 grid((Bp + 63) / 64, (D + 63) / 64);
    hipLaunchKernelGGL(k_transpose_x, grid, dim3(256), 0, st, X, XT, B, D, Bp);
    return hipGetLastError();
}

__global__ void k_fill_u32(uint32_t *p, uint32_t v, size_t n) {
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill_u32(void *p, uint32_t v, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st,
                       (uint32_t *)p, v, n);
    return hipGetLastError();
}

// ---------------------------------------------------- group-major positives
// The fused epilogue walks, per group, the list of (row b, slot j) pairs
// whose label is a positive.  Built deterministically without atomics or
// scans: every tail positive gets the key (g << 32) | (b*G + j); the entry
// of a positive lands at the number of keys smaller than its own, and
// grp_ptr[g] is the number of keys smaller than (g << 32).  The keys are
// few (one per positive), so each workgroup keeps them all in LDS.
__device__ __forceinline__ int row_of(const int32_t *row_ptr, int B, int k) {
    int lo = 0, hi = B;  // row_ptr[lo] <= k < row_ptr[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (row_ptr[mid] <= k) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ void k_gpos_keys(const int32_t *row_ptr, const int32_t *labels, int nnz, int B,
                            int64_t off, int64_t L, int G, long long *keys) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    const int64_t t = (int64_t)labels[k] - off;
    long long key = -1;
    if (t >= 0 && t < L)
        key = ((long long)(t / G) << 32) | (long long)(row_of(row_ptr, B, k) * G + (int)(t % G));
    keys[k] = key;
}

__global__ __launch_bounds__(256) void k_gpos_place(const long long *keys, int nnz, int64_t Ng,
                                                    int32_t *grp_ptr, int32_t *ent) {
    constexpr int CH = 2048;
    __shared__ long long sk[CH];
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const bool roleA = t <= Ng;                      // grp_ptr[t]
    const long long thrA = roleA ? (long long)(t << 32) : 0;
    long long thrB = -1;                             // own key (role B)
    if (t < nnz) thrB = keys[t];
    int cA = 0, cB = 0;
    for (int c0 = 0; c0 < nnz; c0 += CH) {
        __syncthreads();
        for (int i = threadIdx.x; i < CH; i += blockDim.x)
            sk[i] = c0 + i < nnz ? keys[c0 + i] : -1;
        __syncthreads();
        const int lim = nnz - c0 < CH ? nnz - c0 : CH;
        for (int i = 0; i < lim; ++i) {
            const long long v = sk[i];
            cA += (v >= 0 && v < thrA) ? 1 : 0;
            cB += (v >= 0 && v < thrB) ? 1 : 0;
        }
    }
    if (roleA) grp_ptr[t] = cA;
    if (thrB >= 0) ent[cB] = (int32_t)(thrB & 0xffffffffLL);
}

// Up to 16384 positives: one workgroup sorts the keys in LDS (bitonic), then
// grp_ptr[g] is a binary search for (g << 32) and the entries are the low
// words of the sorted keys.  Non-tail positives carry the largest key.
constexpr int GPOS_SORT_MAX = 16384;

__global__ __launch_bounds__(1024) void k_gpos_sort(long long *keys, int nnz, int *nvalid) {
    extern __shared__ unsigned long long sk[];
    int N = 2;
    while (N < nnz) N <<= 1;
    const int tid = threadIdx.x;
    for (int i = tid; i < N; i += 1024)
        sk[i] = (i < nnz && keys[i] >= 0) ? (unsigned long long)keys[i] : ~0ull;
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < N; i += 1024) {
                const int p = i ^ j;
                if (p > i) {
                    const unsigned long long x = sk[i], y = sk[p];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) {
                        sk[i] = y;
                        sk[p] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < nnz; i += 1024) {
        keys[i] = (long long)sk[i];
        const bool last = sk[i] != ~0ull && (i + 1 == N || sk[i + 1] == ~0ull);
        if (last) *nvalid = i + 1;
    }
    if (tid == 0 && sk[0] == ~0ull) *nvalid = 0;
}

__global__ void k_gpos_index(const long long *sorted, const int *nvalid, int64_t Ng,
                             int32_t *grp_ptr, int32_t *ent) {
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int n = *nvalid;
    if (t <= Ng) {
        const unsigned long long thr = (unsigned long long)t << 32;
        int lo = 0, hi = n;  // first index with sorted >= thr
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((unsigned long long)sorted[mid] < thr) lo = mid + 1; else hi = mid;
        }
        grp_ptr[t] = lo;
    }
    if (t < n) ent[t] = (int32_t)(sorted[t] & 0xffffffffLL);
}

hipError_t launch_group_positives(const int32_t *row_ptr, const int32_t *labels, int nnz,
                                  int B, int64_t off, int64_t L, int G, int64_t Ng,
                                  long long *keys, int32_t *grp_ptr, int32_t *ent,
                                  hipStream_t st) {
    hipError_t e;
    if (nnz > 0) {
        hipLaunchKernelGGL(k_gpos_keys, dim3((nnz + 255) / 256), dim3(256), 0, st, row_ptr,
                           labels, nnz, B, off, L, G, keys);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t n = (Ng + 1 > nnz ? Ng + 1 : nnz);
    if (nnz <= GPOS_SORT_MAX) {
        int N = 2;
        while (N < nnz) N <<= 1;
        int *nvalid = (int *)(keys + (nnz > 0 ? nnz : 1));
        const size_t lds = (size_t)N * 8;
        (void)hipFuncSetAttribute((const void *)k_gpos_sort,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k_gpos_sort, dim3(1), dim3(1024), lds, st, keys, nnz, nvalid);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_gpos_index, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           keys, nvalid, Ng, grp_ptr, ent);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_gpos_place, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, keys,
                       nnz, Ng, grp_ptr, ent);
    return hipGetLastError();
}

// ------------------------------------------------------------ epilogue
// Positives of group g that fall in rows [r0, r0 + nrows): sets bit
// ((bt*JT + jt)*4 + i) of the returned mask for each (row, slot) owned by
// this lane.  Layout "rows in 4-groups": the lane owns rows r0+16bt+4q+i of
// slot 16jt+m (T1's Z layout).
template <int BT, int JT>
__device__ __forceinline__ uint64_t pos_mask_rows4(const int32_t *grp_ptr, const int32_t *ent,
                                                   int64_t g, int G, int r0, int q, int m) {
    uint64_t mask = 0;
    const int e0 = grp_ptr[g], e1 = grp_ptr[g + 1];
    for (int e = e0; e < e1; ++e) {
        const int v = ent[e];
        const int lb = v / G - r0, j = v % G;
        if (lb < 0 || lb >= 16 * BT) continue;
        const int bt = lb >> 4, qq = (lb >> 2) & 3, ii = lb & 3;
        const int jt = j >> 4, mm = j & 15;
        if (qq == q && mm == m) mask |= 1ull << ((bt * JT + jt) * 4 + ii);
    }
    return mask;
}

// Z^T layout (T2): the lane owns slots 16jt+4q+i of row r0+16bt+m.
template <int BT, int JT>
__device__ __forceinline__ uint64_t pos_mask_slots4(const int32_t *grp_ptr, const int32_t *ent,
                                                    int64_t g, int G, int r0, int q, int m) {
    uint64_t mask = 0;
    const int e0 = grp_ptr[g], e1 = grp_ptr[g + 1];
    for (int e = e0; e < e1; ++e) {
        const int v = ent[e];
        const int lb = v / G - r0, j = v % G;
        if (lb < 0 || lb >= 16 * BT) continue;
        const int bt = lb >> 4, mm = lb & 15;
        const int jt = j >> 4, qq = (j >> 2) & 3, ii = j & 3;
        if (qq == q && mm == m) mask |= 1ull << ((bt * JT + jt) * 4 + ii);
    }
    return mask;
}

// ------------------------------------------------------------------- T1
// Groups per run = 4 waves * RW; the batch is streamed in chunks of 32 rows.
// Chunk tiles are double-buffered in LDS and filled with asynchronous
// direct global->LDS loads (global_load_lds_dwordx4): while the waves
// contract chunk c, chunk c+1 is already in flight, at no register cost.
constexpr int T1_BC = 32;
constexpr int T1_BCP = T1_BC + 8;          // padded row: 80 B = 5 slots of 16 B

// bytes of one chunk buffer: 5 slots per feature row, whole 1 KB wave blocks
__host__ __device__ inline int t1_nblk(int D) { return (5 * D + 63) / 64; }   // 1 KB blocks
__host__ __device__ inline int t1_blk_per_wave(int D, int NW) { return (t1_nblk(D) + NW - 1) / NW; }
__host__ __device__ inline size_t t1_buf_bytes(int D, int NW) {
    return (size_t)NW * t1_blk_per_wave(D, NW) * 1024;
}

// Issue this wave's share of the asynchronous copy of chunk ch into buf.
template <int NW>
__device__ __forceinline__ void t1_stage_async(const TailArgs &a, unsigned short *buf, int ch,
                                               int w, int lane) {
    const int nbw = t1_blk_per_wave(a.D, NW);
    for (int i = 0; i < nbw; ++i) {
        const int blk = w * nbw + i;
        const int s = blk * 64 + lane;            // 16-byte slot of the padded tile
        int row = s / 5, seg = s % 5;
        if (seg == 4) seg = 3;                    // pad slot: harmless duplicate
        if (row >= a.D) { row = 0; seg = 0; }     // beyond the tile: dummy source
        const unsigned short *src = a.XT + (int64_t)row * a.Bp + ch * T1_BC + seg * 8;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(
                                                  (char *)buf + (size_t)blk * 1024), 16, 0, 0);
    }
}

template <int G, int F, int RW, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, 1) void k_tail_t1(TailArgs a, int store_z, int do_loss) {
    constexpr int JT = G / 16, KS = F / 32, FT = F / 16;
    constexpr int BC = T1_BC, BCP = T1_BCP;
    constexpr bool DO_Z = (MODE != T1_DW_MEM);
    constexpr bool DO_DW = (MODE != T1_FWD);
    extern __shared__ __attribute__((aligned(16))) unsigned short tiles[];
    const size_t bstride = t1_buf_bytes(a.D, NW) / 2;   // in shorts

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q = lane >> 4, m = lane & 15;
    const int nch = a.Bp / BC;
    const int64_t n_runs = (a.Ng + NW * RW - 1) / (NW * RW);
    const bool need_pos = MODE != T1_DW_MEM && (do_loss || DO_DW);
    float lsum = 0.f;

    for (int64_t run = blockIdx.x; run < n_runs; run += gridDim.x) {
        const int64_t gw = run * (NW * RW) + (int64_t)w * RW;
        bf16x8 wreg[RW][KS][JT];
        unsigned zrow[RW][KS];            // tr-gather rows: lo16 = h 0, hi16 = h 1
        unsigned frow[RW][FT / 2];        // dW rows, two f-tiles per word
        int gp0[RW], gp1[RW];             // positives range per group
        f32x4 dwacc[RW][FT][JT];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int64_t g = gw + r;
            const bool ok = g < a.Ng;
            const int32_t *ix = a.idx + (ok ? g : 0) * (int64_t)F;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const unsigned lo = (unsigned)ix[32 * s + 8 * q + (m >> 2)];
                const unsigned hi = (unsigned)ix[32 * s + 8 * q + 4 + (m >> 2)];
                zrow[r][s] = lo | (hi << 16);
                if (DO_Z) {
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const unsigned short *wp =
                            a.W + (((ok ? g : 0) * G + 16 * jt + m) * (int64_t)F + 32 * s + 8 * q);
                        wreg[r][s][jt] = *(const bf16x8 *)wp;
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < FT / 2; ++p)
                frow[r][p] = (unsigned)ix[32 * p + m] | ((unsigned)ix[32 * p + 16 + m] << 16);
            gp0[r] = gp1[r] = 0;
            if (need_pos && ok) {
                gp0[r] = a.grp_ptr[g];
                gp1[r] = a.grp_ptr[g + 1];
            }
#pragma unroll
            for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) dwacc[r][ft][jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        __syncthreads();                  // previous run's readers are done with buffer 0
        t1_stage_async<NW>(a, tiles, 0, w, lane);
        for (int ch = 0; ch < nch; ++ch) {
            __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of chunk ch have landed
            __syncthreads();                 // ... and everyone's; chunk ch-1 is consumed
            if (ch + 1 < nch)
                t1_stage_async<NW>(a, tiles + ((ch + 1) & 1) * bstride, ch + 1, w, lane);
            const unsigned short *tile = tiles + (ch & 1) * bstride;
            const int r0 = ch * BC;

#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int64_t g = gw + r;
                if (g >= a.Ng) continue;  // wave-uniform
                // positives of group g in rows [r0, r0+32): lane owns rows r0+16h2+4q+i, slot 16jt+m
                uint64_t ymask = 0;
                bool has_pos = false;             // wave-uniform
                for (int e = gp0[r]; e < gp1[r]; ++e) {
                    const int v = a.grp_ent[e];
                    const int lb = v / G - r0, j = v % G;
                    if (lb < 0 || lb >= BC) continue;
                    has_pos = true;
                    if (((lb >> 2) & 3) == q && (j & 15) == m)
                        ymask |= 1ull << (((lb >> 4) * JT + (j >> 4)) * 4 + (lb & 3));
                }
                f32x4 zacc[2][JT];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) zacc[h2][jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                if (DO_Z) {
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const unsigned rlo = zrow[r][s] & 0xffffu, rhi = zrow[r][s] >> 16;
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const int col = 16 * h2 + 4 * (m & 3);
                            i16x4 a0 = lds_read_tr(tile + rlo * BCP + col);
                            i16x4 a1 = lds_read_tr(tile + rhi * BCP + col);
                            bf16x8 A = __builtin_bit_cast(
                                bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                            for (int jt = 0; jt < JT; ++jt)
                                zacc[h2][jt] = mfma32(A, wreg[r][s][jt], zacc[h2][jt]);
                        }
                    }
                }
                // ---- epilogue: lane owns (row r0+16h2+4q+i, slot 16jt+m)
                unsigned dzp[2][JT][2];
                const bool tile_live = (r0 + BC <= a.B) && ((g + 1) * G <= a.L);
                if (MODE != T1_DW_MEM && tile_live && !has_pos && !(MODE == T1_FWD && store_z)) {
                    // fast path: every element live, no positive, no logits to store
                    float lin = 0.f, prod = 1.f;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            float dzv[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float z = zacc[h2][jt][i];
                                const float e = fast_exp_neg_abs(z);
                                float den;
                                dzv[i] = a.s * fast_sigmoid(z, e, den);
                                prod *= den;
                                lin += fmaxf(z, 0.f);
                            }
                            dzp[h2][jt][0] = pack_bf16x2(dzv[0], dzv[1]);
                            dzp[h2][jt][1] = pack_bf16x2(dzv[2], dzv[3]);
                        }
                    // at most 8*JT <= 32 factors in [1, 2]: the product stays below 2^32
                    if (do_loss) lsum += a.s * (lin + fast_log(prod));
                } else {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            float dzv[4];
                            const int64_t t = g * G + 16 * jt + m;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int row = r0 + 16 * h2 + 4 * q + i;
                                const bool live = row < a.B && t < a.L;
                                const float z = zacc[h2][jt][i];
                                float dz = 0.f;
                                if (MODE == T1_DW_MEM) {
                                    if (live) dz = bf16_to_f32(a.dZ[(int64_t)row * a.L + t]);
                                } else {
                                    const float y =
                                        (float)((ymask >> ((h2 * JT + jt) * 4 + i)) & 1ull);
                                    if (live && (do_loss || DO_DW)) {
                                        const float e = fast_exp_neg_abs(z);
                                        float den;
                                        dz = a.s * (fast_sigmoid(z, e, den) - y);
                                        if (do_loss)
                                            lsum += a.s * ((fmaxf(z, 0.f) - y * z) + fast_log(den));
                                    }
                                    if (MODE == T1_FWD && store_z && live)
                                        a.Z[(int64_t)row * a.L + t] = f32_to_bf16(z);
                                }
                                dzv[i] = dz;
                            }
                            dzp[h2][jt][0] = pack_bf16x2(dzv[0], dzv[1]);
                            dzp[h2][jt][1] = pack_bf16x2(dzv[2], dzv[3]);
                        }
                }
                if (DO_DW) {
                    bf16x8 Bj[JT];
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        u32x4 v = {dzp[0][jt][0], dzp[0][jt][1], dzp[1][jt][0], dzp[1][jt][1]};
                        Bj[jt] = __builtin_bit_cast(bf16x8, v);
                    }
#pragma unroll
                    for (int ft = 0; ft < FT; ++ft) {
                        const unsigned row =
                            (ft & 1) ? (frow[r][ft >> 1] >> 16) : (frow[r][ft >> 1] & 0xffffu);
                        const unsigned short *p = tile + row * BCP + 4 * q;
                        u32x2 lo = *(const u32x2 *)p;
                        u32x2 hi = *(const u32x2 *)(p + 16);
                        u32x4 v = {lo.x, lo.y, hi.x, hi.y};
                        bf16x8 A = __builtin_bit_cast(bf16x8, v);
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt)
                            dwacc[r][ft][jt] = mfma32(A, Bj[jt], dwacc[r][ft][jt]);
                    }
                }
            }
        }
        if (DO_DW) {
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int64_t g = gw + r;
                if (g >= a.Ng) continue;
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const f32x4 v = dwacc[r][ft][jt];
                        const int64_t t = g * G + 16 * jt + m;  // padded rows get dz = 0
                        u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *(u32x2 *)(a.dW + t * F + 16 * ft + 4 * q) = o;
                    }
            }
        }
    }
    if (do_loss && a.loss) {
        float v = wave_sum(lsum);
        if (lane == 0) atomicAdd(a.loss, v);
    }
}

// Dynamic LDS above the default per-kernel limit must be allowed per kernel.
static void allow_lds(const void *fn, size_t bytes) {
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int G, int F, int RW, int NW>
static hipError_t t1_launch(int mode, const TailArgs &a, bool store_z, bool do_loss,
                            hipStream_t st) {
    const size_t lds = t1_buf_bytes(a.D, NW) * 2;
    const int64_t n_runs = (a.Ng + NW * RW - 1) / (NW * RW);
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t grid = n_runs < ncu ? n_runs : ncu;
    if (grid <= 0) return hipSuccess;
    const dim3 blk(64 * NW);
    switch (mode) {
    case T1_FWD:
        allow_lds((const void *)k_tail_t1<G, F, RW, NW, T1_FWD>, lds);
        hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_FWD>), dim3((unsigned)grid), blk, lds, st,
                           a, (int)store_z, (int)do_loss);
        break;
    case T1_DW_BCE:
        allow_lds((const void *)k_tail_t1<G, F, RW, NW, T1_DW_BCE>, lds);
        hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_BCE>), dim3((unsigned)grid), blk, lds,
                           st, a, 0, (int)do_loss);
        break;
    default:
        allow_lds((const void *)k_tail_t1<G, F, RW, NW, T1_DW_MEM>, lds);
        hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_MEM>), dim3((unsigned)grid), blk, lds,
                           st, a, 0, 0);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_tail_t1(int mode, int G, const TailArgs &a, bool store_z, bool do_loss,
                          hipStream_t st) {
#define T1CASE(GG, FF, RR, NN) \
    if (G == GG && a.F == FF) return t1_launch<GG, FF, RR, NN>(mode, a, store_z, do_loss, st);
    T1CASE(16, 32, 4, 8)
    T1CASE(16, 64, 3, 8)
    T1CASE(16, 128, 2, 8)
    T1CASE(32, 32, 3, 8)
    T1CASE(32, 64, 2, 8)
    T1CASE(32, 128, 1, 8)
    T1CASE(64, 32, 2, 8)
    T1CASE(64, 64, 1, 8)
    T1CASE(64, 128, 1, 4)
#undef T1CASE
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------- T2
// Workgroup = (row chunk of BC2 rows) x (range of groups), 8 waves.  Each
// wave owns NTW32 tiles of 32 features of the dX accumulator (32x32 MFMA
// tiles, rows x features).
//
// Per group g, the dense product dX_chunk += dz_g (rows x G) * W~_g (G x D)
// runs on v_mfma_f32_32x32x16_bf16 (K = 16 labels per instruction), where
// W~_g is W_g^T scattered to the rows idx_g and zero elsewhere: the B
// operand of feature d is row f of W_g^T when idx_g[f] = d, else a zero row.
//
// Software pipeline, one barrier per group.  W_g and idx_g arrive in an LDS
// ring of R slots through asynchronous direct global->LDS loads issued R-1
// groups ahead (no registers held).  Iteration g:
//   issue the loads of group g+R,
//   (1) recompute Z^T of group g+1 for the chunk (A operand from the raw
//       W_{g+1} rows, B operand gathered from the chunk with transposing
//       reads at rows idx_{g+1}), sigmoid-BCE -> dz, published in LDS in the
//       A-operand layout of the 32x32x16 product,
//   (2) build W_{g+1}^T ([f][j]) and the inverse index feature -> f,
//   (3) dense product of group g,
//   wait for the loads of group g+2, barrier.
constexpr int T2_NW = 8;

struct T2Lds {  // byte offsets of the LDS regions (host and device agree)
    int ring, ring_slot, ring_idx, wts, wts_slot, inv, exch, total;
};

__host__ __device__ inline T2Lds t2_layout(int D, int F, int G, int BC2, int NTW32, int R) {
    T2Lds L;
    const int BCP = BC2 + 8, RT = BC2 / 32, JT = G / 16;
    const int wbytes = G * F * 2;                  // multiple of 1 KB
    int o = ((D * BCP * 2) + 1023) / 1024 * 1024;  // X^T chunk
    L.ring = o;
    L.ring_idx = wbytes;                           // idx_g, then grp_ptr[g], grp_ptr[g+1]
    L.ring_slot = wbytes + 1024;                   // both fit in one 1 KB block (F <= 128)
    o += R * L.ring_slot;
    L.wts = o;
    L.wts_slot = (F + 1) * G * 2;                  // row F = zeros
    o += 2 * L.wts_slot;
    L.inv = o;
    o += 2 * (T2_NW * NTW32 * 32) * 2;
    o = (o + 15) / 16 * 16;
    L.exch = o;
    o += 2 * RT * JT * 64 * 16;
    o = (o + 1023) / 1024 * 1024;                  // + one scratch block for dummy copies
    L.total = o + 1024;
    return L;
}

__device__ __forceinline__ void vm_wait(int n) {
    // s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

template <int G, int BC2, int NTW32>
__global__ __launch_bounds__(64 * T2_NW, 1) void k_tail_t2(TailArgs a, int dz_mem, int n_granges,
                                                           int R) {
    constexpr int NW = T2_NW, NT = 64 * NW;
    constexpr int JT = G / 16, BT = BC2 / 16, RT = BC2 / 32, BCP = BC2 + 8;
    constexpr int NDP = NW * NTW32 * 32;
    const int F = a.F, KS = F / 32;
    const T2Lds LY = t2_layout(a.D, F, G, BC2, NTW32, R);
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned short *tile = (unsigned short *)lds;
    unsigned char *ring = lds + LY.ring;
    unsigned short *wts0 = (unsigned short *)(lds + LY.wts);
    short *inv0 = (short *)(lds + LY.inv);
    unsigned char *exch0 = lds + LY.exch;
    unsigned char *scratch = lds + LY.total - 1024;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int q = lane >> 4, m = lane & 15;
    const int gr = blockIdx.x % n_granges, bch = blockIdx.x / n_granges;
    const int64_t gA = (int64_t)gr * a.Ng / n_granges, gB = (int64_t)(gr + 1) * a.Ng / n_granges;
    const int ng = (int)(gB - gA);
    const int r0 = bch * BC2;
    const int nq = (G / 4) * (F / 4);
    const int dbase = w * NTW32 * 32;
    const int wblk = G * F * 2 / 1024;               // 1 KB blocks of raw W per group
    const int nblk = wblk + 1;                       // + idx
    const int NB = (nblk + NW - 1) / NW;             // copies per wave per group

    // Asynchronous copy of W_g, idx_g (and grp_ptr[g], grp_ptr[g+1] after it)
    // into ring slot (g - gA) % R.  The pointer read covers 4 entries; the
    // workspace holds 3 spare entries past grp_ptr[Ng].
    auto issue = [&](int k) {  // k = g - gA
        unsigned char *slot = ring + (k % R) * LY.ring_slot;
        const int64_t g = gA + k;
        for (int i = 0; i < NB; ++i) {
            const int blk = w + NW * i;
            if (blk < wblk) {
                const unsigned short *src = a.W + g * G * (int64_t)F + blk * 512 + lane * 8;
                __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(
                                                          slot + blk * 1024), 16, 0, 0);
            } else if (blk == wblk) {
                const int32_t *src = a.idx + g * (int64_t)F + (lane < F / 4 ? lane * 4 : 0);
                if (lane == F / 4 && !dz_mem) src = a.grp_ptr + g;
                __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(
                                                          slot + LY.ring_idx), 16, 0, 0);
            } else {  // keep the per-wave copy count uniform
                __builtin_amdgcn_global_load_lds(a.W + lane * 8, (__attribute__((address_space(3))) void *)(
                                                          scratch), 16, 0, 0);
            }
        }
    };

    {   // stage the chunk, reset the inverse maps, zero rows
        constexpr int SEG = BC2 / 8;
        const unsigned short *src = a.XT + r0;
        for (int i = tid; i < a.D * SEG; i += NT) {
            const int d = i / SEG, sg = i % SEG;
            *(u32x4 *)(tile + d * BCP + sg * 8) = *(const u32x4 *)(src + (int64_t)d * a.Bp + sg * 8);
        }
        for (int i = tid; i < 2 * NDP; i += NT) inv0[i] = (short)F;
        for (int i = tid; i < 2 * G; i += NT)
            wts0[(i / G) * (LY.wts_slot / 2) + F * G + i % G] = 0;
    }
    f32x16 acc[RT][NTW32];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NTW32; ++nt) acc[rt][nt] = (f32x16){};

    // (1) Z^T of group k -> dz -> exch slot k & 1
    auto zt = [&](int k) {
        const unsigned char *slot = ring + (k % R) * LY.ring_slot;
        const unsigned short *rw = (const unsigned short *)slot;
        const int *ri = (const int *)(slot + LY.ring_idx);
        unsigned char *exch = exch0 + (k & 1) * (RT * JT * 64 * 16);
        const int64_t g = gA + k;
        int gp0 = 0, gp1 = 0;
        if (!dz_mem) {
            gp0 = ri[F];
            gp1 = ri[F + 1];
        }
        for (int tl = w; tl < JT * BT; tl += NW) {   // label tile jt, row tile bt
            const int jt = tl / BT, bt = tl % BT;
            float dzv[4];
            const int row = r0 + 16 * bt + m;
            if (!dz_mem) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const int col = 16 * bt + 4 * (m & 3);
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 Av = *(const bf16x8 *)(rw + (16 * jt + m) * F + 32 * s + 8 * q);
                    const int fa = 32 * s + 8 * q + (m >> 2);
                    i16x4 b0 = lds_read_tr(tile + ri[fa] * BCP + col);
                    i16x4 b1 = lds_read_tr(tile + ri[fa + 4] * BCP + col);
                    bf16x8 Bv = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
                    z = mfma32(Av, Bv, z);
                }
                // positives of this group inside the tile (lane owns slots 16jt+4q+i of row)
                unsigned ymask = 0;
                bool has_pos = false;            // wave-uniform
                for (int e = gp0; e < gp1; ++e) {
                    const int v = a.grp_ent[e];
                    const int lb = v / G - (r0 + 16 * bt), j = v % G;
                    if (lb < 0 || lb >= 16 || (j >> 4) != jt) continue;
                    has_pos = true;
                    if (lb == m && ((j >> 2) & 3) == q) ymask |= 1u << (j & 3);
                }
                if (!has_pos && r0 + 16 * bt + 16 <= a.B && (g + 1) * G <= a.L) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float den;
                        dzv[i] = a.s * fast_sigmoid(z[i], fast_exp_neg_abs(z[i]), den);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t t = g * G + 16 * jt + 4 * q + i;
                        const bool live = row < a.B && t < a.L;
                        float den;
                        dzv[i] = live ? a.s * (fast_sigmoid(z[i], fast_exp_neg_abs(z[i]), den) -
                                               (float)((ymask >> i) & 1u))
                                      : 0.f;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t t = g * G + 16 * jt + 4 * q + i;
                    const bool live = row < a.B && t < a.L;
                    dzv[i] = live ? bf16_to_f32(a.dZ[(int64_t)row * a.L + t]) : 0.f;
                }
            }
            // element (row 16bt+m, label 16jt+4q+i) -> 32x32x16 A operand of row tile bt/2:
            // lane 16(bt%2)+m+32(q/2), K slots 4(q%2)+i
            const int lane2 = 16 * (bt & 1) + m + 32 * (q >> 1);
            *(u32x2 *)(exch + (((bt >> 1) * JT + jt) * 64 + lane2) * 16 + 8 * (q & 1)) =
                (u32x2){pack_bf16x2(dzv[0], dzv[1]), pack_bf16x2(dzv[2], dzv[3])};
        }
    };

    // (2) W_g^T ([f][j]) and the inverse index, for group k
    auto build = [&](int k) {
        const unsigned char *slot = ring + (k % R) * LY.ring_slot;
        const unsigned short *rw = (const unsigned short *)slot;
        const int *ri = (const int *)(slot + LY.ring_idx);
        unsigned short *wts = wts0 + (k & 1) * (LY.wts_slot / 2);
        short *inv = inv0 + (k & 1) * NDP;
        for (int u = tid; u < nq; u += NT) {
            const int ja = u % (G / 4), fc = u / (G / 4);
            u32x2 rr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rr[e] = *(const u32x2 *)(rw + (4 * ja + e) * F + 4 * fc);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int word = kk >> 1, sh = (kk & 1) * 16;
                const unsigned v0 = (rr[0][word] >> sh) & 0xffffu, v1 = (rr[1][word] >> sh) & 0xffffu;
                const unsigned v2 = (rr[2][word] >> sh) & 0xffffu, v3 = (rr[3][word] >> sh) & 0xffffu;
                *(u32x2 *)(wts + (4 * fc + kk) * G + 4 * ja) = (u32x2){v0 | (v1 << 16), v2 | (v3 << 16)};
            }
        }
        if (tid < F) inv[ri[tid]] = (short)tid;
    };

    // (3) dense product of group k
    auto dense = [&](int k) {
        const unsigned short *wts = wts0 + (k & 1) * (LY.wts_slot / 2) + 8 * (lane >> 5);
        short *inv = inv0 + (k & 1) * NDP;
        const unsigned char *exch = exch0 + (k & 1) * (RT * JT * 64 * 16);
        const unsigned short *brow[NTW32];
#pragma unroll
        for (int nt = 0; nt < NTW32; ++nt) brow[nt] = wts + inv[dbase + 32 * nt + (lane & 31)] * G;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            bf16x8 Am[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                Am[rt] = *(const bf16x8 *)(exch + ((rt * JT + jt) * 64 + lane) * 16);
#pragma unroll
            for (int nt = 0; nt < NTW32; ++nt) {
                const bf16x8 Bv = *(const bf16x8 *)(brow[nt] + 16 * jt);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = mfma32x32(Am[rt], Bv, acc[rt][nt]);
            }
        }
        // reset this wave's slice of the inverse map (only this wave reads it)
        for (int i = lane; i < NTW32 * 32; i += 64) inv[dbase + i] = (short)F;
    };

    // Ring: groups 0..R-1 are loaded up front; iteration k refills the slot of
    // group k (last read by zt/build of group k in iteration k-1, before the
    // barrier that closed it) with group k+R.
    __syncthreads();
    for (int k = 0; k < R && k < ng; ++k) issue(k);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ng > 0) {
        zt(0);
        build(0);
    }
    __syncthreads();
    for (int k = 0; k < ng; ++k) {
        if (k + R < ng) issue(k + R);
        if (k + 1 < ng) {
            zt(k + 1);
            build(k + 1);
        }
        dense(k);
        // iteration k+1 reads group k+2: wait for its loads (vector-memory
        // results return in issue order), leaving the later groups in flight
        const int last = k + R < ng ? k + R : ng - 1;
        const int after = (k + 2 < ng) ? last - (k + 2) : 0;
        vm_wait(after > 0 ? after * NB : 0);
        lds_barrier();
    }

    // flush: reg r of tile (rt, nt) = row 32rt+8(r/4)+4(lane/32)+r%4, feature dbase+32nt+lane%32
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NTW32; ++nt) {
            const int d = dbase + 32 * nt + (lane & 31);
            if (d >= a.D) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = r0 + 32 * rt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < a.B) atomicAdd(a.dX + (int64_t)row * a.D + d, acc[rt][nt][r]);
            }
        }
}

static T2Lds t2_plan(int D, int F, int G, int BC2, int NTW32, int &R) {
    for (R = 4; R >= 2; --R) {
        T2Lds L = t2_layout(D, F, G, BC2, NTW32, R);
        if (L.total <= 160 * 1024) return L;
    }
    R = 0;
    return t2_layout(D, F, G, BC2, NTW32, 2);
}

static int64_t t2_granges(int nbch, int64_t Ng) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    // group ranges: a multiple of 8 (so the row chunks of one range share an
    // XCD and its L2 for W_g), about one workgroup per CU overall
    int64_t ngr = (ncu + nbch - 1) / nbch;
    ngr = (ngr + 7) / 8 * 8;
    if (ngr > Ng) ngr = Ng;
    return ngr;
}

template <int G, int BC2, int NTW32>
static hipError_t t2_go(bool dz_mem, const TailArgs &a, hipStream_t st) {
    const int nbch = a.Bp / BC2;
    const int64_t ngr = t2_granges(nbch, a.Ng);
    if (ngr < 1) return hipSuccess;
    int R = 0;
    const T2Lds L = t2_plan(a.D, a.F, G, BC2, NTW32, R);
    if (R < 2) return hipErrorInvalidValue;
    allow_lds((const void *)k_tail_t2<G, BC2, NTW32>, L.total);
    hipLaunchKernelGGL((k_tail_t2<G, BC2, NTW32>), dim3((unsigned)(ngr * nbch)), dim3(64 * T2_NW),
                       L.total, st, a, (int)dz_mem, (int)ngr, R);
    return hipGetLastError();
}

static bool t2_fits(int D, int F, int G, int BC2, int NTW32) {
    int R = 0;
    t2_plan(D, F, G, BC2, NTW32, R);
    return R >= 2;
}

template <int G, int NTW32>
static hipError_t t2_pick_bc(bool dz_mem, const TailArgs &a, hipStream_t st) {
    if (t2_fits(a.D, a.F, G, 64, NTW32)) return t2_go<G, 64, NTW32>(dz_mem, a, st);
    return t2_go<G, 32, NTW32>(dz_mem, a, st);
}

template <int G>
static hipError_t t2_pick(bool dz_mem, const TailArgs &a, hipStream_t st) {
    const int nd = (a.D + 31) / 32, need = (nd + T2_NW - 1) / T2_NW;
    if (need <= 1) return t2_pick_bc<G, 1>(dz_mem, a, st);
    if (need <= 2) return t2_pick_bc<G, 2>(dz_mem, a, st);
    if (need <= 3) return t2_pick_bc<G, 3>(dz_mem, a, st);
    return t2_pick_bc<G, 4>(dz_mem, a, st);
}

hipError_t launch_tail_t2(int G, bool dz_mem, const TailArgs &a, hipStream_t st) {
    switch (G) {
    case 16: return t2_pick<16>(dz_mem, a, st);
    case 32: return t2_pick<32>(dz_mem, a, st);
    case 64: return t2_pick<64>(dz_mem, a, st);
    }
    return hipErrorInvalidValue;
}

bool tail_bf16_supported(int G, int F, int D) {
    if (!(G == 16 || G == 32 || G == 64)) return false;
    if (!(F == 32 || F == 64 || F == 128)) return false;
    if (D < F || D > 1024) return false;
    // T1: two chunk buffers; T2: chunk + pipeline buffers with BC2 = 32 at least
    if (t1_buf_bytes(D, 8) * 2 > 160 * 1024 || t1_buf_bytes(D, 4) * 2 > 160 * 1024) return false;
    const int nd = (D + 31) / 32, need = (nd + T2_NW - 1) / T2_NW;
    const int ntw = need <= 1 ? 1 : need <= 2 ? 2 : need <= 3 ? 3 : 4;
    if (t2_layout(D, F, G, 32, ntw, 2).total > 160 * 1024) return false;
    return true;
}

}  // namespace haste
