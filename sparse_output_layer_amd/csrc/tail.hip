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
// Also zeroes the dW/logits pass's run counters (sched, 2 words) when given.
__global__ __launch_bounds__(256) void k_transpose_x(const unsigned short *__restrict__ X,
                                                     unsigned short *__restrict__ XT,
                                                     int B, int D, int Bp, unsigned *sched) {
    __shared__ unsigned short t[64][66];
    const int b0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
    if (sched && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 2) sched[threadIdx.x] = 0u;
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

hipError_t launch_transpose_x(const unsigned short *X, unsigned short *XT, int B, int D, int Bp,
                              unsigned *sched, hipStream_t st) {
    dim3 grid((Bp + 63) / 64, (D + 63) / 64);
    hipLaunchKernelGGL(k_transpose_x, grid, dim3(256), 0, st, X, XT, B, D, Bp, sched);
    return hipGetLastError();
}

// ------------------------------------------------- given dZ -> dz tiles
// The backward from a caller's dZ (B x L bf16, row-major) reuses the step's
// dz tiles: tile ((g * nch + ch) * JT + jt) holds 1 KB, lane (q, m) the rows
// 32ch + 16h2 + 4q + i (i = 0..3, h2 = 0..1) of label gG + 16jt + m, zero past
// B and past L.  A workgroup reads 32 rows x 256 labels (512-byte row
// pieces) into LDS and writes 16 tiles, each by one wave in 16-byte stores.
constexpr int DZT_LAB = 256;
__global__ __launch_bounds__(256) void k_dz_tiles(const unsigned short *__restrict__ dZ, int B, int64_t L,
                                                  int G, int nch, int64_t ntiles16,
                                                  unsigned short *__restrict__ dzt) {
    __shared__ unsigned short s[32][DZT_LAB + 2];
    const int t = threadIdx.x, ch = blockIdx.y;
    const int64_t l0 = (int64_t)blockIdx.x * DZT_LAB;
    for (int r = 0; r < 32; ++r) {
        const int row = 32 * ch + r;
        const int64_t lab = l0 + t;
        s[r][t] = row < B && lab < L ? dZ[(int64_t)row * L + lab] : (unsigned short)0;
    }
    __syncthreads();
    const int lane = t & 63, w = t >> 6, q = lane >> 4, m = lane & 15;
    const int JT = G / 16;
    for (int k = w; k < DZT_LAB / 16; k += 4) {
        const int64_t lt = l0 / 16 + k;            // 16-label tile: group lt / JT, slot block lt % JT
        if (lt >= ntiles16) break;
        const int64_t g = lt / JT, jt = lt % JT;
        unsigned v[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {             // pairs (h2, i), (h2, i + 1)
            const int h2 = h >> 1, i = 2 * (h & 1);
            const int r = 16 * h2 + 4 * q + i;
            v[h] = (unsigned)s[r][16 * k + m] | ((unsigned)s[r + 1][16 * k + m] << 16);
        }
        *(u32x4 *)(dzt + (((g * nch + ch) * JT + jt) << 9) + lane * 8) = (u32x4){v[0], v[1], v[2], v[3]};
    }
}

hipError_t launch_dz_tiles(const unsigned short *dZ, int B, int64_t L, int G, int Bp, int64_t Ng,
                           unsigned short *dzt, hipStream_t st) {
    if (B <= 0 || L <= 0) return hipSuccess;
    if (G % 16 != 0 || Bp % 32 != 0) return hipErrorInvalidValue;
    const int nch = Bp / 32;
    const int64_t nlab = Ng * G;                   // padded label count: whole tiles
    const dim3 grid((unsigned)((nlab + DZT_LAB - 1) / DZT_LAB), (unsigned)nch);
    hipLaunchKernelGGL(k_dz_tiles, grid, dim3(256), 0, st, dZ, B, L, G, nch, Ng * (G / 16), dzt);
    return hipGetLastError();
}

// ------------------------------------------------------- feature order
// Order of each group's F features in which T1 reads the gathered rows, so
// that its LDS reads hit distinct banks.  A chunk row (feature d) is 80 bytes
// long, so its bank position depends on d mod 16 (its class).  T1 reads, per
// instruction, the 16 features of 16 consecutive positions (dW operands: each
// 16 bytes of a row, conflict-free when the 16 classes differ) and, per half
// wave, the 8 features of positions {0-3, 8-11} or {4-7, 12-15} of a block of
// 16 (transposing reads: 32 bytes of a row, conflict-free when the classes
// are distinct and of one parity).  So position k of a block takes class
// c(k mod 16): even classes at slots 0-3 and 8-11, odd ones at 4-7, 12-15.
// Per group (one wave, features f = lane and lane + 64): the r-th feature of
// class c (in f order) takes block r at its class's slot while r < F/16; the
// features left over (classes with more than F/16 members) fill the empty
// positions, those of their own parity first, in order.  perm[g][k] is the
// position's feature f, idxp[g][k] = idx[g][perm[g][k]].  Any order is a
// correct contraction; this one only removes bank conflicts.
__device__ __forceinline__ int fo_slot_of(int c) {
    const int j = c >> 1;
    return (c & 1) ? (j < 4 ? 4 + j : 8 + j) : (j < 4 ? j : 4 + j);
}
__device__ __forceinline__ int fo_class_of_slot(int s) {
    return 2 * ((s & 3) + 4 * (s >> 3)) + ((s >> 2) & 1);
}

constexpr int FO_WAVES = 4;   // waves per block
constexpr int FO_GPW = 4;     // groups per wave, their loads issued together

__global__ __launch_bounds__(64 * FO_WAVES) void k_feature_order(const int32_t *idx, int64_t Ng,
                                                                 int F, unsigned short *idxp,
                                                                 unsigned char *perm) {
    __shared__ unsigned char s_pos[FO_WAVES][128], s_ovf[FO_WAVES][2][128];
    __shared__ unsigned short s_ix[FO_WAVES][128];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nb = F >> 4;
    const unsigned long long lt = (1ull << lane) - 1;
    const int64_t g0 = (blockIdx.x * (int64_t)FO_WAVES + w) * FO_GPW;
    int ixr[FO_GPW][2];
#pragma unroll
    for (int u = 0; u < FO_GPW; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int f = lane + 64 * h;
            ixr[u][h] = g0 + u < Ng && f < F ? idx[(g0 + u) * F + f] : -1;
        }
    const int ssl = fo_class_of_slot(lane & 15);   // class of this lane's positions
#pragma unroll
    for (int u = 0; u < FO_GPW; ++u) {
        const int64_t g = g0 + u;
        const bool ok = g < Ng;
        int cls[2], rank[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) cls[h] = ixr[u][h] >= 0 ? (ixr[u][h] & 15) : -1;
        // bit-sliced ballots: the features of class c in half h are the valid
        // ones whose four class bits match c
        unsigned long long vm[2], bm[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            vm[h] = __ballot(cls[h] >= 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) bm[h][k] = __ballot(cls[h] >= 0 && ((cls[h] >> k) & 1));
        }
        auto members = [&](int c, int h) {
            unsigned long long mk = vm[h];
#pragma unroll
            for (int k = 0; k < 4; ++k) mk &= ((c >> k) & 1) ? bm[h][k] : ~bm[h][k];
            return mk;
        };
        // rank of each feature within its class; the count of this lane's
        // position class
        if (cls[0] >= 0) rank[0] = __popcll(members(cls[0], 0) & lt);
        if (cls[1] >= 0) rank[1] = __popcll(members(cls[1], 0)) + __popcll(members(cls[1], 1) & lt);
        const int scnt = __popcll(members(ssl, 0)) + __popcll(members(ssl, 1));
        // overflow features: index among those of their parity
        bool ov[2];
        int oi[2] = {0, 0}, on[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) ov[h] = cls[h] >= 0 && rank[h] >= nb;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const bool s0 = ov[0] && (cls[0] & 1) == qq, s1 = ov[1] && (cls[1] & 1) == qq;
            const unsigned long long m0 = __ballot(s0), m1 = __ballot(s1);
            const int n0 = __popcll(m0);
            on[qq] = n0 + __popcll(m1);
            if (s0) oi[0] = __popcll(m0 & lt);
            if (s1) oi[1] = n0 + __popcll(m1 & lt);
        }
        // empty positions: index among those of their parity
        bool em[2];
        int ei[2] = {0, 0}, en[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = lane + 64 * h;
            em[h] = ok && k < F && scnt <= (k >> 4);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const bool s0 = em[0] && (ssl & 1) == p, s1 = em[1] && (ssl & 1) == p;
            const unsigned long long m0 = __ballot(s0), m1 = __ballot(s1);
            const int n0 = __popcll(m0);
            en[p] = n0 + __popcll(m1);
            if (s0) ei[0] = __popcll(m0 & lt);
            if (s1) ei[1] = n0 + __popcll(m1 & lt);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int f = lane + 64 * h;
            if (cls[h] < 0) continue;
            s_ix[w][f] = (unsigned short)ixr[u][h];
            if (ov[h]) s_ovf[w][cls[h] & 1][oi[h]] = (unsigned char)f;
            else s_pos[w][16 * rank[h] + fo_slot_of(cls[h])] = (unsigned char)f;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = lane + 64 * h;
            if (!ok || k >= F) continue;
            int f;
            if (!em[h]) {
                f = s_pos[w][k];
            } else {
                // own parity while its overflow lasts, then the other parity's
                // surplus (the part its own empty positions leave over)
                const int p = ssl & 1;
                f = ei[h] < on[p] ? s_ovf[w][p][ei[h]] : s_ovf[w][p ^ 1][en[p ^ 1] + ei[h] - on[p]];
            }
            perm[g * F + k] = (unsigned char)f;
            idxp[g * F + k] = s_ix[w][f];
        }
        __syncthreads();   // the next group reuses the wave's LDS
    }
}

hipError_t launch_feature_order(const int32_t *idx, int64_t Ng, int F, unsigned short *idxp,
                                unsigned char *perm, hipStream_t st) {
    if (Ng <= 0) return hipSuccess;
    if (F % 16 != 0 || F > 128) return hipErrorInvalidValue;
    const int64_t per_block = FO_WAVES * FO_GPW;
    hipLaunchKernelGGL(k_feature_order, dim3((unsigned)((Ng + per_block - 1) / per_block)),
                       dim3(64 * FO_WAVES), 0, st, idx, Ng, F, idxp, perm);
    return hipGetLastError();
}

__global__ void k_fill_u32(uint32_t *p, uint32_t v, size_t n) {
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

// SGD update after a step: out = fma(-lr, dW, W) (bf16: both read as bf16,
// one fp32 fma, one rounding to bf16)
__global__ void k_sgd(const void *W, const void *dW, float lr, void *out, int64_t n, int bf16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        if (bf16) {
            const float w = __uint_as_float((unsigned)((const unsigned short *)W)[i] << 16);
            const float g = __uint_as_float((unsigned)((const unsigned short *)dW)[i] << 16);
            ((unsigned short *)out)[i] = f32_to_bf16(__builtin_fmaf(-lr, g, w));
        } else {
            ((float *)out)[i] = __builtin_fmaf(-lr, ((const float *)dW)[i], ((const float *)W)[i]);
        }
    }
}

hipError_t launch_sgd(const void *W, const void *dW, float lr, void *out, int64_t n, bool bf16,
                      hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_sgd, dim3((unsigned)blocks), dim3(256), 0, st, W, dW, lr, out, n, (int)bf16);
    return hipGetLastError();
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
// whose label is a positive.  Built deterministically without a sort network:
// every tail positive gets the key (g << 32) | (b*G + j); a key's rank (the
// valid keys below it, plus equal keys at smaller input positions, so a label
// listed twice in a row keeps both entries in input order) is its place in
// the group-major order, and the list is written directly (sorted[rank] =
// key).  grp_ptr[g] is a binary search for (g << 32); entries are the keys'
// low words.  Ranking is nnz^2 comparisons, spread over a 2-D grid of
// 256 x 256 key tiles.
__device__ __forceinline__ int row_of(const int32_t *row_ptr, int B, int k) {
    int lo = 0, hi = B;  // row_ptr[lo] <= k < row_ptr[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (row_ptr[mid] <= k) lo = mid; else hi = mid;
    }
    return lo;
}

// Invalid key: all ones (compares above every valid key as unsigned).
__global__ void k_gpos_keys(const int32_t *row_ptr, const int32_t *labels, int nnz, int B,
                            int64_t off, int64_t L, int G, unsigned long long *keys, int *rank,
                            int *nvalid) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k == 0) *nvalid = 0;
    if (k >= nnz) return;
    const int64_t t = (int64_t)labels[k] - off;
    unsigned long long key = ~0ull;
    if (t >= 0 && t < L)
        key = ((unsigned long long)(t / G) << 32) |
              (unsigned long long)(unsigned)(row_of(row_ptr, B, k) * G + (int)(t % G));
    keys[k] = key;
    rank[k] = 0;
}

constexpr int GPOS_TILE = 256;

// Block (x, y): keys of tile x counted against the keys of tile y.
__global__ __launch_bounds__(GPOS_TILE) void k_gpos_rank(const unsigned long long *keys, int nnz,
                                                          int *rank, int *nvalid) {
    __shared__ unsigned long long sk[GPOS_TILE];
    const int k = blockIdx.x * GPOS_TILE + threadIdx.x;
    const int j0 = blockIdx.y * GPOS_TILE;
    const int jj = j0 + threadIdx.x;
    sk[threadIdx.x] = jj < nnz ? keys[jj] : ~0ull;
    const unsigned long long own = k < nnz ? keys[k] : ~0ull;
    __syncthreads();
    if (own == ~0ull) return;
    // equal keys count only at positions before k
    const int before = k - j0 < 0 ? 0 : (k - j0 > GPOS_TILE ? GPOS_TILE : k - j0);
    int r = 0;
#pragma unroll 16
    for (int i = 0; i < GPOS_TILE; ++i) {
        const unsigned long long v = sk[i];
        r += (v < own || (v == own && i < before)) ? 1 : 0;
    }
    if (r) atomicAdd(rank + k, r);
    if (blockIdx.y == 0) atomicAdd(nvalid, 1);
}

__global__ void k_gpos_scatter(const unsigned long long *keys, const int *rank, int nnz,
                               unsigned long long *sorted) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    const unsigned long long key = keys[k];
    if (key != ~0ull) sorted[rank[k]] = key;
}

__global__ void k_gpos_index(const unsigned long long *sorted, const int *nvalid, int64_t Ng,
                             int32_t *grp_ptr, int32_t *ent) {
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int n = *nvalid;
    if (t <= Ng) {
        const unsigned long long thr = (unsigned long long)t << 32;
        int lo = 0, hi = n;  // first index with sorted >= thr
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sorted[mid] < thr) lo = mid + 1; else hi = mid;
        }
        grp_ptr[t] = lo;
    }
    if (t < n) ent[t] = (int32_t)(sorted[t] & 0xffffffffull);
}

// keys: workspace of 20*max(nnz,1) + 8 bytes, 8-byte aligned (keys, sorted
// keys, ranks, count)
hipError_t launch_group_positives(const int32_t *row_ptr, const int32_t *labels, int nnz,
                                  int B, int64_t off, int64_t L, int G, int64_t Ng,
                                  long long *keys_ws, int32_t *grp_ptr, int32_t *ent,
                                  hipStream_t st) {
    hipError_t e;
    if (nnz <= 0) return launch_fill_u32(grp_ptr, 0u, (size_t)(Ng + 1), st);
    unsigned long long *keys = (unsigned long long *)keys_ws;
    unsigned long long *sorted = keys + nnz;
    int *rank = (int *)(sorted + nnz);
    int *nvalid = rank + nnz;
    const unsigned nt = (unsigned)((nnz + GPOS_TILE - 1) / GPOS_TILE);
    hipLaunchKernelGGL(k_gpos_keys, dim3(nt), dim3(GPOS_TILE), 0, st, row_ptr, labels, nnz, B,
                       off, L, G, keys, rank, nvalid);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_gpos_rank, dim3(nt, nt), dim3(GPOS_TILE), 0, st, keys, nnz, rank,
                       nvalid);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_gpos_scatter, dim3(nt), dim3(GPOS_TILE), 0, st, keys, rank, nnz, sorted);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = Ng + 1 > nnz ? Ng + 1 : nnz;
    hipLaunchKernelGGL(k_gpos_index, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sorted,
                       nvalid, Ng, grp_ptr, ent);
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

// bytes of one chunk buffer: 5 slots of 16 bytes per feature row
__host__ __device__ inline size_t t1_buf_bytes(int D, int NW) {
    (void)NW;
    return (size_t)D * T1_BCP * 2;
}
constexpr int T1_BUF_BYTES = 80 * 1024;    // one chunk buffer, static: D <= 1024
constexpr int T1_ROWS_PER_COPY = 12;       // feature rows per copy instruction (60 lanes)

// Source offset (bytes) of this lane's 16-byte slot within a block of 12
// feature rows: row lane/5, segment lane%5 (the pad slot repeats segment 3).
// It does not depend on the block or the chunk, so the copies need no
// per-lane arithmetic.
__device__ __forceinline__ unsigned t1_copy_voff(int lane, int Bp) {
    const int row = lane / 5, seg = lane % 5;
    return (unsigned)(row * Bp + 8 * (seg == 4 ? 3 : seg)) * 2u;
}

// Issue this wave's share of the asynchronous copy of chunk ch into buf: one
// direct global->LDS copy per block of 12 rows (lanes 60..63 idle); the last
// block is moved back to end at row D (its overlap rewrites equal data).
template <int NW>
__device__ __forceinline__ void t1_stage_async(const TailArgs &a, unsigned short *buf, int ch,
                                               int w, int lane, unsigned voff) {
    const int nblk = (a.D + T1_ROWS_PER_COPY - 1) / T1_ROWS_PER_COPY;
    for (int b = w; b < nblk; b += NW) {
        const int r0 = min(T1_ROWS_PER_COPY * b, a.D - T1_ROWS_PER_COPY);
        const char *src = (const char *)(a.XT + (int64_t)r0 * a.Bp + ch * T1_BC);
        if (lane < 5 * T1_ROWS_PER_COPY)
            __builtin_amdgcn_global_load_lds(src + voff, (__attribute__((address_space(3))) void *)(
                                                             buf + r0 * T1_BCP), 16, 0, 0);
    }
}

// How T1's groups are dealt out.  A run gives each of the NW waves RW
// groups.  Whole runs fill `n_full` tickets, a whole number of rounds of the
// grid; the groups left over are spread over the grid in smaller tickets of
// `k` waves each (the other waves of the workgroup idle), so the last round
// is not a few full runs on a few CUs while the others wait.  A ticket's time
// is set by its chunk loop, which is shorter with fewer waves at work.
struct T1Tickets {
    int64_t n_full;     // tickets of whole runs
    int64_t n_tickets;  // all tickets
    int k;              // waves at work in a ticket past n_full
};

__host__ inline T1Tickets t1_tickets(int64_t Ng, int RW, int NW, int ncu) {
    T1Tickets t{};
    const int64_t slots = (Ng + RW - 1) / RW, runs = (slots + NW - 1) / NW;
    t.n_full = runs / ncu * ncu;
    const int64_t left = slots - t.n_full * NW;
    int64_t k = (left + ncu - 1) / ncu;
    k = k < 1 ? 1 : k > NW ? NW : k;
    t.k = (int)k;
    t.n_tickets = t.n_full + (left + k - 1) / k;
    return t;
}

// Whether every logit of the wave's chunk tile has |z| <= 2 (wave-uniform)
template <int JT>
__device__ __forceinline__ bool t1_small_logits(const f32x4 (&zacc)[2][JT]) {
    float mz = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mz = fmaxf(mz, fabsf(zacc[h2][jt][i]));
    return __all(mz <= 2.0f);
}

// TK: the fused top-K stage 1 (one bucket per group, K' = 1) is compiled in:
// 1 with the maximum's own id, 2 with the group's first label as the id.
// GS: the layer's group size when a wave owns a slice of G labels of a
// larger group (GS = G: a wave owns whole groups).  The GS / G slices of a
// group share its index set and feature order and go to different waves, so
// a wave of a wide group needs no more registers than one of a group of G.
template <int G, int F, int RW, int NW, int MODE, int TK = 0, int GS = G>
__global__ __launch_bounds__(64 * NW, 1) void k_tail_t1(TailArgs a, T1Tickets tix, int store_z,
                                                        int do_loss) {
    constexpr int JT = G / 16, KS = F / 32, FT = F / 16;
    constexpr int NSL = GS / G;            // label slices per group
    constexpr int JTS = GS / 16;           // 16-label tiles per group (dz tile index)
    static_assert(GS % G == 0 && (NSL == 1 || (RW == 1 && TK == 0)), "slices: one per wave, no top-K");
    const int64_t Nu = a.Ng * NSL;         // work units: (group, slice)
    constexpr int BC = T1_BC, BCP = T1_BCP;
    // a group's W / dW slab (G x F) passes through LDS, one row per WSP
    // elements (16 bytes of padding: rows 4 banks apart), to turn the feature
    // order into full-width global accesses; WPL 16-byte pieces per lane
    constexpr int WSP = F + 8, WPL = G * F / 8 / 64;
    static_assert(G * F % 512 == 0, "slab pieces must fill whole waves");
    static_assert(NW * G * WSP * 2 <= T1_BUF_BYTES, "slab staging exceeds a chunk buffer");
    constexpr bool DO_Z = (MODE != T1_DW_MEM);
    constexpr bool DO_DW = (MODE != T1_FWD);
    // The two chunk buffers are distinct LDS objects and the chunk loop is
    // unrolled by two, so every access names its buffer statically: the
    // compiler then sees that the copy into one buffer cannot alias the
    // reads of the other and does not wait for the copy before them.
    __shared__ __attribute__((aligned(16))) unsigned short buf0[T1_BUF_BYTES / 2];
    __shared__ __attribute__((aligned(16))) unsigned short buf1[T1_BUF_BYTES / 2];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);   // wave index in a scalar register
    const unsigned voff = t1_copy_voff(lane, a.Bp);
    const int q = lane >> 4, m = lane & 15;
    const int nch = a.Bp / BC;
    const bool need_pos = MODE != T1_DW_MEM && (do_loss || DO_DW);
    float lsum = 0.f;

    // Runs in a dynamic order: a workgroup's first run is its index, the next
    // ones come from a ticket counter (so that workgroups which start late,
    // behind other work on their CU, take fewer runs); the last workgroup to
    // finish resets the counters for the next launch.  The ticket reaches the
    // waves through the padding of row 0 of buffer 1 (never read; at the end
    // of a run no copy into buffer 1 is pending and the next run's W staging
    // comes after its first barrier).
    int *const s_ticket = (int *)(buf1 + 32);
    for (int64_t run = blockIdx.x; run < tix.n_tickets;) {
        // first group of this wave; a.Ng (no group) for the idle waves of a small ticket
        // (wave-uniform: from the scalar wave index, so the group's
        // addresses are formed in scalar registers)
        const int64_t gw = run < tix.n_full ? (run * NW + wu) * RW
                           : wu < tix.k     ? (tix.n_full * NW + (run - tix.n_full) * tix.k + wu) * RW
                                            : Nu;
        bf16x8 wreg[RW][KS][JT];
        u32x2 pwz[DO_Z ? RW : 1][KS];     // perm bytes of positions 32s + 8q .. + 7
        // LDS byte offsets within a chunk buffer, fixed for a run: the two
        // transposing gathers of each K step (this lane's column included),
        // and the two 8-byte halves of each dW operand row.  The second half's
        // offset is made opaque here, so the compiler neither fuses the two
        // reads into one paired read (about twice the LDS cycles) nor spends
        // instructions per chunk on keeping them apart.
        unsigned zoff[RW][KS][2];
        unsigned dwo[RW][FT][2];
        int gp0[RW], pn[RW], pe[RW];      // positives per group: first, count, entry per lane
        int pc[RW];                       // next positive of the group not yet below the chunk
        f32x4 dwacc[RW][FT][JT];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const bool ok = gw + r < Nu;
            const int64_t g = (gw + r) / NSL;
            // features in the bank-aware order: position k reads feature
            // perm[g][k] (row idxp[g][k] of the chunk, column perm[g][k] of W)
            const int64_t gs = ok ? g : 0;
            const unsigned short *ix = a.idxp + gs * (int64_t)F;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const unsigned lo = (unsigned)ix[32 * s + 8 * q + (m >> 2)];
                const unsigned hi = (unsigned)ix[32 * s + 8 * q + 4 + (m >> 2)];
                zoff[r][s][0] = (lo * BCP + 4 * (m & 3)) * 2u;
                zoff[r][s][1] = (hi * BCP + 4 * (m & 3)) * 2u;
                if (DO_Z) pwz[r][s] = *(const u32x2 *)(a.perm + gs * F + 32 * s + 8 * q);
            }
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
                dwo[r][ft][0] = ((unsigned)ix[16 * ft + m] * BCP + 4 * q) * 2u;
                dwo[r][ft][1] = dwo[r][ft][0] + 32u;
                asm volatile("" : "+v"(dwo[r][ft][1]));
            }
            gp0[r] = pn[r] = pe[r] = pc[r] = 0;
            if (need_pos && ok) {
                gp0[r] = __builtin_amdgcn_readfirstlane(a.grp_ptr[g]);
                pn[r] = __builtin_amdgcn_readfirstlane(a.grp_ptr[g + 1]) - gp0[r];
                pe[r] = lane < pn[r] ? a.grp_ent[gp0[r] + lane] : 0;
            }
#pragma unroll
            for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) dwacc[r][ft][jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        // one chunk of BC rows, staged in `tile`
        auto chunk = [&](const unsigned short *tile, const int ch) {
            const int r0 = ch * BC;

#pragma unroll
            for (int r = 0; r < RW; ++r) {
                if (gw + r >= Nu) continue;  // wave-uniform
                const int64_t g = (gw + r) / NSL;
                const int sl = (int)((gw + r) % NSL);
                const int64_t t0 = g * GS + G * sl;   // this wave's first label
                // positives of group g in rows [r0, r0+32): lane owns rows r0+16h2+4q+i, slot 16jt+m
                uint64_t ymask = 0;
                bool has_pos = false;             // wave-uniform
                auto add_pos = [&](const int v) {
                    const int lb = v / GS - r0, j = v % GS - G * sl;
                    if (lb < 0 || lb >= BC || j < 0 || j >= G) return;
                    has_pos = true;
                    if (((lb >> 2) & 3) == q && (j & 15) == m)
                        ymask |= 1ull << (((lb >> 4) * JT + (j >> 4)) * 4 + (lb & 3));
                };
                // The group's entries are sorted by row, and chunks come in row
                // order: a cursor walks the list once per run, taking the
                // entries of this chunk's rows.  Entries 0..63 come from
                // registers; the rest (a label with more than 64 positives in the
                // batch) from memory, in a loop of its own so that the register
                // path carries no wait for loads in flight.
                {
                    int e = pc[r];
                    const int n1 = pn[r] < 64 ? pn[r] : 64;
                    for (; e < n1; ++e) {
                        const int v = __builtin_amdgcn_readlane(pe[r], e);
                        if (v / GS >= r0 + BC) break;
                        add_pos(v);
                    }
                    if (e >= 64)
                        for (; e < pn[r]; ++e) {
                            const int v = a.grp_ent[gp0[r] + e];
                            if (v / GS >= r0 + BC) break;
                            add_pos(v);
                        }
                    pc[r] = e;
                }
                f32x4 zacc[2][JT];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) zacc[h2][jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                if (DO_Z) {
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const char *tb = (const char *)tile + 32 * h2;
                            i16x4 a0 = lds_read_tr(tb + zoff[r][s][0]);
                            i16x4 a1 = lds_read_tr(tb + zoff[r][s][1]);
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
                const bool tile_live = (r0 + BC <= a.B) && (t0 + G <= a.L);
                if (MODE == T1_DW_MEM && a.dzt) {
                    // the caller's dZ, already in the tile layout (zero past B and L)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const u32x4 v =
                            *(const u32x4 *)(a.dzt + ((((int64_t)g * nch + ch) * JTS + JT * sl + jt) << 9) + lane * 8);
                        dzp[0][jt][0] = v[0];
                        dzp[0][jt][1] = v[1];
                        dzp[1][jt][0] = v[2];
                        dzp[1][jt][1] = v[3];
                    }
                } else if (MODE != T1_DW_MEM && tile_live && !has_pos && !(MODE == T1_FWD && store_z) &&
                           t1_small_logits<JT>(zacc)) {
                    // fastest path: as below, and every |z| <= 2 in the wave, so
                    // t = e^-z needs no sign split: s*sigmoid(z) = s / (1 + t), and
                    // softplus(z) = z + log(1 + t) with eight factors 1 + t <= 8.4
                    // a product (below 2^25); the sum of z and the log cancel to
                    // at most 2e-6 of the terms' value at |z| <= 2
                    float sumz = 0.f, logs = 0.f;
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        float prod = 1.f;
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            float dzv[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float z = zacc[h2][jt][i];
                                const float den = 1.0f + __builtin_amdgcn_exp2f(z * -kLog2e);
                                dzv[i] = a.s * __builtin_amdgcn_rcpf(den);
                                prod *= den;
                                sumz += z;
                            }
                            dzp[h2][jt][0] = pack_bf16x2(dzv[0], dzv[1]);
                            dzp[h2][jt][1] = pack_bf16x2(dzv[2], dzv[3]);
                            if (a.Z32) {   // fp32 logits for the top-K
                                const int64_t t = t0 + 16 * jt + m;
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    a.Z32[(int64_t)(r0 + 16 * h2 + 4 * q + i) * a.L + t] = zacc[h2][jt][i];
                            }
                        }
                        logs += fast_log(prod);
                    }
                    if (do_loss) lsum += a.s * (sumz + logs);
                } else if (MODE != T1_DW_MEM && tile_live && !has_pos && !(MODE == T1_FWD && store_z)) {
                    // fast path: every element live, no positive, no logits to store;
                    // lin2 = sum of z + |z| = twice the sum of max(z, 0), exactly;
                    // the (1 + e) factors' product kept as product - 1
                    float lin2 = 0.f, prod = 0.f;
                    const float hs = 0.5f * a.s;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            float dzv[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                // r = 1/(1 + exp(-|z|)) is sigmoid(|z|); s*sigmoid(z)
                                // = s/2 + sign(z) * (s*r - s/2)
                                const float z = zacc[h2][jt][i];
                                const float e = fast_exp_neg_abs(z);
                                const float r = __builtin_amdgcn_rcpf(1.0f + e);
                                dzv[i] = hs + __builtin_copysignf(__builtin_fmaf(a.s, r, -hs), z);
                                prod = prod1p(prod, e);
                                lin2 += z + fabsf(z);
                            }
                            dzp[h2][jt][0] = pack_bf16x2(dzv[0], dzv[1]);
                            dzp[h2][jt][1] = pack_bf16x2(dzv[2], dzv[3]);
                            if (a.Z32) {   // fp32 logits for the top-K
                                const int64_t t = t0 + 16 * jt + m;
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    a.Z32[(int64_t)(r0 + 16 * h2 + 4 * q + i) * a.L + t] = zacc[h2][jt][i];
                            }
                        }
                    // at most 8*JT <= 32 factors in [1, 2]: the product stays below 2^32
                    if (do_loss) lsum += a.s * (0.5f * lin2 + log1p_pos(prod));
                } else {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            float dzv[4];
                            const int64_t t = t0 + 16 * jt + m;
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
                                            lsum += a.s * ((fmaxf(z, 0.f) - y * z) + log1p_pos(e));
                                    }
                                    if (MODE == T1_FWD && store_z && live)
                                        a.Z[(int64_t)row * a.L + t] = f32_to_bf16(z);
                                    if (a.Z32 && live) a.Z32[(int64_t)row * a.L + t] = z;
                                }
                                dzv[i] = dz;
                            }
                            dzp[h2][jt][0] = pack_bf16x2(dzv[0], dzv[1]);
                            dzp[h2][jt][1] = pack_bf16x2(dzv[2], dzv[3]);
                        }
                }
                if constexpr (TK == 2) {
                    // the exact top-K needs only each (group, row)'s largest
                    // logit: the group is its candidate, and a later pass
                    // recomputes the K best groups of the row.  Ties between
                    // groups go to the smaller group, as they would to the
                    // smaller label id.  The max runs on order keys over the
                    // lane's slots, then over the 16 lanes of the row.
                    const bool all_live = (g + 1) * G <= a.L;   // wave-uniform
                    unsigned ku[2][4];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if (all_live) {
                                float v = zacc[h2][0][i];
#pragma unroll
                                for (int jt = 1; jt < JT; ++jt) v = fmaxf(v, zacc[h2][jt][i]);
                                ku[h2][i] = f32_order_key(v);
                            } else {
                                unsigned u = 0u;   // key 0: no live label
#pragma unroll
                                for (int jt = 0; jt < JT; ++jt)
                                    if (g * G + 16 * jt + m < a.L) u = max(u, f32_order_key(zacc[h2][jt][i]));
                                ku[h2][i] = u;
                            }
                        }
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int i = 0; i < 4; ++i) ku[h2][i] = max(ku[h2][i], dpp_u32<0xB1>(ku[h2][i]));
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int i = 0; i < 4; ++i) ku[h2][i] = max(ku[h2][i], dpp_u32<0x4E>(ku[h2][i]));
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int i = 0; i < 4; ++i) ku[h2][i] = max(ku[h2][i], dpp_u32<0x141>(ku[h2][i]));
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int i = 0; i < 4; ++i) ku[h2][i] = max(ku[h2][i], dpp_u32<0x140>(ku[h2][i]));
                    if (m == 0) {
                        const unsigned gid = (unsigned)(a.tk_off + g * G);
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            f32x4 cv;
                            u32x4 ci;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const unsigned u = ku[h2][i];
                                cv[i] = u == 0u ? -INFINITY : f32_from_order_key(u);
                                ci[i] = u == 0u ? 0xffffffffu : gid;
                            }
                            const int64_t o = g * (int64_t)a.Bp + r0 + 16 * h2 + 4 * q;
                            __builtin_nontemporal_store(cv, (f32x4 *)(a.tk_v + o));
                            __builtin_nontemporal_store(ci, (u32x4 *)(a.tk_i + o));
                        }
                    }
                } else if constexpr (TK == 1) {
                    // top-K stage 1 fused here, one bucket per group and K' = 1:
                    // per row, the group's largest logit (ties: smaller id), into
                    // group-major lists (Ng x Bp); lane m = 0 of each q stores rows
                    // 4q..4q+3 and 16+4q.. of the chunk, 16 bytes each.  The max
                    // runs on order keys (key 0: label past L).  Groups of 16: the
                    // lane's 8 rows (h2, i) reduce over the 16 lanes side by side;
                    // larger groups: the lane's own slots first, then row by row
                    // (the faster form for each, measured).
                    if constexpr (JT == 1) {
                        unsigned ku[8], k0[8], kj[8];
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) {
                            ku[r8] = k0[r8] =
                                g * G + m < a.L ? f32_order_key(zacc[r8 >> 2][0][r8 & 3]) : 0u;
                            kj[r8] = (unsigned)m;
                        }
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) ku[r8] = max(ku[r8], dpp_u32<0xB1>(ku[r8]));
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) ku[r8] = max(ku[r8], dpp_u32<0x4E>(ku[r8]));
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) ku[r8] = max(ku[r8], dpp_u32<0x141>(ku[r8]));
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) ku[r8] = max(ku[r8], dpp_u32<0x140>(ku[r8]));
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) kj[r8] = k0[r8] == ku[r8] ? kj[r8] : 0xffffffffu;
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) kj[r8] = min(kj[r8], dpp_u32<0xB1>(kj[r8]));
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) kj[r8] = min(kj[r8], dpp_u32<0x4E>(kj[r8]));
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) kj[r8] = min(kj[r8], dpp_u32<0x141>(kj[r8]));
#pragma unroll
                        for (int r8 = 0; r8 < 8; ++r8) kj[r8] = min(kj[r8], dpp_u32<0x140>(kj[r8]));
                        if (m == 0) {
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                f32x4 cv;
                                u32x4 ci;
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const unsigned u = ku[4 * h2 + i];
                                    cv[i] = u == 0u ? -INFINITY : f32_from_order_key(u);
                                    ci[i] = u == 0u ? 0xffffffffu
                                                    : (unsigned)(a.tk_off + g * G + kj[4 * h2 + i]);
                                }
                                const int64_t o = g * (int64_t)a.Bp + r0 + 16 * h2 + 4 * q;
                                __builtin_nontemporal_store(cv, (f32x4 *)(a.tk_v + o));
                                __builtin_nontemporal_store(ci, (u32x4 *)(a.tk_i + o));
                            }
                        }
                    } else {
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            f32x4 cv;
                            u32x4 ci;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                float bv = -INFINITY;
                                unsigned bj = 0xffffffffu;
#pragma unroll
                                for (int jt = 0; jt < JT; ++jt) {   // ascending slots: ties keep the first
                                    const unsigned j = 16 * jt + m;
                                    const float z = zacc[h2][jt][i];
                                    if (g * G + j < a.L && (bj == 0xffffffffu || z > bv)) {
                                        bv = z;
                                        bj = j;
                                    }
                                }
                                row16_argmax(bv, bj);
                                cv[i] = bj == 0xffffffffu ? -INFINITY : bv;
                                ci[i] = bj == 0xffffffffu ? 0xffffffffu : (unsigned)(a.tk_off + g * G + bj);
                            }
                            if (m == 0) {
                                const int64_t o = g * (int64_t)a.Bp + r0 + 16 * h2 + 4 * q;
                                __builtin_nontemporal_store(cv, (f32x4 *)(a.tk_v + o));
                                __builtin_nontemporal_store(ci, (u32x4 *)(a.tk_i + o));
                            }
                        }
                    }
                }
                if (DO_DW) {
                    bf16x8 Bj[JT];
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        u32x4 v = {dzp[0][jt][0], dzp[0][jt][1], dzp[1][jt][0], dzp[1][jt][1]};
                        Bj[jt] = __builtin_bit_cast(bf16x8, v);
                        // dz tile (g, chunk, jt) for the dX pass, in this register layout:
                        // lane (q, m) holds rows 4q+i and 16+4q+i (i = 0..3) of label 16jt+m.
                        // Streams written once here and read once later (dz tiles, dW,
                        // top-K lists) and W read once go with the non-temporal hint,
                        // which leaves the cache to the chunks of X^T (measured: 6% less
                        // time for this pass on the 670K workload)
                        if (MODE == T1_DW_BCE && a.dzt)
                            __builtin_nontemporal_store(v, (u32x4 *)(a.dzt + ((((int64_t)g * nch + ch) * JTS + JT * sl + jt) << 9) + lane * 8));
                    }
                    auto dw_read = [&](int ft) {
                        u32x2 lo = *(const u32x2 *)((const char *)tile + dwo[r][ft][0]);
                        u32x2 hi = *(const u32x2 *)((const char *)tile + dwo[r][ft][1]);
                        u32x4 v = {lo.x, lo.y, hi.x, hi.y};
                        return __builtin_bit_cast(bf16x8, v);
                    };
                    // the reads of step ft+1 are issued before the products of
                    // step ft, so a step waits for its own reads only
                    bf16x8 Acur = dw_read(0);
#pragma unroll
                    for (int ft = 0; ft < FT; ++ft) {
                        bf16x8 Anext = Acur;
                        if (ft + 1 < FT) Anext = dw_read(ft + 1);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt)
                            dwacc[r][ft][jt] = mfma32(Acur, Bj[jt], dwacc[r][ft][jt]);
                        Acur = Anext;
                    }
                }
            }
        };
        // nch is even (Bp is a multiple of 64)
        __syncthreads();                  // previous run's readers are done with both buffers
        t1_stage_async<NW>(a, buf0, 0, wu, lane, voff);
        if (DO_Z) {
            // W operands in the feature order, through this wave's slab in
            // buffer 1 (free until the loop's first barrier; groups in turn)
            unsigned short *ws = buf1 + w * (G * WSP);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                // this wave's G label rows (slice of its group), or group 0's
                const int64_t ls = gw + r < Nu ? ((gw + r) / NSL) * GS + G * ((gw + r) % NSL) : 0;
                u32x4 wraw[WPL];
#pragma unroll
                for (int i = 0; i < WPL; ++i)
                    wraw[i] = __builtin_nontemporal_load((const u32x4 *)(a.W + ls * (int64_t)F + 8 * (64 * i + lane)));
#pragma unroll
                for (int i = 0; i < WPL; ++i) {
                    const int pc16 = 64 * i + lane;
                    *(u32x4 *)(ws + (pc16 / (F / 8)) * WSP + 8 * (pc16 % (F / 8))) = wraw[i];
                }
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const unsigned short *wr = ws + (16 * jt + m) * WSP;
                        unsigned short e8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            e8[e] = wr[(pwz[r][s][e >> 2] >> (8 * (e & 3))) & 255u];
                        wreg[r][s][jt] = __builtin_bit_cast(bf16x8, e8);
                    }
            }
        }
        for (int ch = 0; ch < nch; ch += 2) {
            __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of chunk ch have landed
            __syncthreads();                 // ... and everyone's; chunk ch-1 is consumed
            t1_stage_async<NW>(a, buf1, ch + 1, wu, lane, voff);
            chunk(buf0, ch);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (ch + 2 < nch) t1_stage_async<NW>(a, buf0, ch + 2, wu, lane, voff);
            chunk(buf1, ch + 1);
        }
        if (DO_DW) {
            // dW back to the natural feature order through this wave's slab in
            // buffer 0 (no copy into it is pending and every wave has read
            // its last chunk), then full-width stores; groups in turn
            unsigned short *ws = buf0 + w * (G * WSP);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                if (gw + r >= Nu) continue;   // wave-uniform
                const int64_t g = (gw + r) / NSL;
                const int64_t t0 = g * GS + G * ((gw + r) % NSL);
                unsigned pw[FT];           // perm bytes of positions 16ft + 4q .. + 3
#pragma unroll
                for (int ft = 0; ft < FT; ++ft) pw[ft] = *(const unsigned *)(a.perm + g * F + 16 * ft + 4 * q);
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const f32x4 v = dwacc[r][ft][jt];   // padded rows get dz = 0
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            ws[(16 * jt + m) * WSP + ((pw[ft] >> (8 * i)) & 255u)] = f32_to_bf16(v[i]);
                    }
#pragma unroll
                for (int i = 0; i < WPL; ++i) {
                    const int pc16 = 64 * i + lane;
                    const u32x4 v = *(const u32x4 *)(ws + (pc16 / (F / 8)) * WSP + 8 * (pc16 % (F / 8)));
                    const int64_t o = t0 * (int64_t)F + 8 * pc16;
                    if (!a.Wout) {
                        __builtin_nontemporal_store(v, (u32x4 *)(a.dW + o));
                    } else {
                        // fused SGD: Wout = fma(-lr, dW, W) with dW as it would be
                        // stored (bf16): the same arithmetic as k_sgd after a step
                        const u32x4 w = __builtin_nontemporal_load((const u32x4 *)(a.W + o));
                        u32x4 r;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float w0 = __uint_as_float(w[e] << 16), w1 = __uint_as_float(w[e] & 0xffff0000u);
                            const float g0 = __uint_as_float(v[e] << 16), g1 = __uint_as_float(v[e] & 0xffff0000u);
                            r[e] = pack_bf16x2(__builtin_fmaf(-a.lr, g0, w0), __builtin_fmaf(-a.lr, g1, w1));
                        }
                        __builtin_nontemporal_store(r, (u32x4 *)(a.Wout + o));
                    }
                }
            }
        }
        if (a.sched) {
            if (threadIdx.x == 0) *s_ticket = (int)gridDim.x + (int)atomicAdd(a.sched, 1u);
            __syncthreads();
            run = __builtin_amdgcn_readfirstlane(*s_ticket);
        } else {
            run += gridDim.x;
        }
    }
    if (a.sched && threadIdx.x == 0) {
        // a workgroup counts itself out after its last ticket: the last one
        // out knows that every ticket is taken
        __threadfence();
        if (atomicAdd(a.sched + 1, 1u) == gridDim.x - 1) {
            atomicExch(a.sched, 0u);
            atomicExch(a.sched + 1, 0u);
        }
    }
    // one add per workgroup; the waves' sums meet in buffer 0, where no copy
    // is pending after the last run
    if (do_loss && a.loss) block_loss_add(lsum, (float *)buf0, a.loss);
}

// Dynamic LDS above the default per-kernel limit must be allowed per kernel.
static void allow_lds(const void *fn, size_t bytes) {
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int G, int F, int RW, int NW, int GS = G>
static hipError_t t1_launch(int mode, const TailArgs &a, bool store_z, bool do_loss,
                            hipStream_t st) {
    if (t1_buf_bytes(a.D, NW) > (size_t)T1_BUF_BYTES) return hipErrorInvalidValue;
    const size_t lds = 0;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const T1Tickets tix = t1_tickets(a.Ng * (GS / G), RW, NW, ncu);
    const int64_t grid = tix.n_tickets < ncu ? tix.n_tickets : ncu;
    if (grid <= 0) return hipSuccess;
    const dim3 blk(64 * NW);
    const int tk = a.tk_v == nullptr ? 0 : a.tk_max_only ? 2 : 1;
    if constexpr (GS != G) {
        // label slices: no fused top-K
        if (tk) return hipErrorInvalidValue;
        switch (mode) {
        case T1_FWD:
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_FWD, 0, GS>), dim3((unsigned)grid), blk, lds,
                               st, a, tix, (int)store_z, (int)do_loss);
            break;
        case T1_DW_BCE:
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_BCE, 0, GS>), dim3((unsigned)grid), blk,
                               lds, st, a, tix, 0, (int)do_loss);
            break;
        default:
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_MEM, 0, GS>), dim3((unsigned)grid), blk,
                               lds, st, a, tix, 0, 0);
            break;
        }
        return hipGetLastError();
    }
    switch (mode) {
    case T1_FWD:
        if (tk == 2)
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_FWD, 2>), dim3((unsigned)grid), blk, lds,
                               st, a, tix, (int)store_z, (int)do_loss);
        else if (tk == 1)
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_FWD, 1>), dim3((unsigned)grid), blk, lds,
                               st, a, tix, (int)store_z, (int)do_loss);
        else
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_FWD>), dim3((unsigned)grid), blk, lds, st,
                               a, tix, (int)store_z, (int)do_loss);
        break;
    case T1_DW_BCE:
        if (tk == 2)
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_BCE, 2>), dim3((unsigned)grid), blk,
                               lds, st, a, tix, 0, (int)do_loss);
        else if (tk == 1)
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_BCE, 1>), dim3((unsigned)grid), blk,
                               lds, st, a, tix, 0, (int)do_loss);
        else
            hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_BCE>), dim3((unsigned)grid), blk, lds,
                               st, a, tix, 0, (int)do_loss);
        break;
    default:
        if (tk) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_tail_t1<G, F, RW, NW, T1_DW_MEM>), dim3((unsigned)grid), blk, lds,
                           st, a, tix, 0, 0);
        break;
    }
    return hipGetLastError();
}

// ------------------------------------------------------- fixed fan-in, G = 1
// Every label keeps its own F indices (the per-label layout that the HASTE
// page compares against, section "Results"): the forward has to gather F
// rows of X for every label instead of every group.  Logits and the
// sigmoid-BCE loss only.  Workgroup = FF_R labels over the whole batch: their
// tables of (row offset, weight) pairs are built once in LDS; 32-row chunks
// of X^T (rows of 64 bytes) stream through LDS, double-buffered with direct
// global->LDS copies; each wave owns eight labels, four at a time (one per
// quarter-wave; a lane per two adjacent rows, read as one 4-byte word), and
// reads the table four entries at a time.
constexpr int FF_NW = 8;                   // waves per workgroup
constexpr int FF_R = 64;                   // labels per workgroup (eight per wave)
constexpr int FF_BUF_BYTES = 64 * 1024;    // one chunk buffer: D <= 1024 rows of 64 bytes

// This wave's share of the copy of chunk ch: one copy instruction per 16 rows
// (lane: row lane/4, 16-byte segment lane%4); the last block moved back to
// end at row D (its overlap rewrites equal data).
__device__ __forceinline__ void ff_stage_async(const TailArgs &a, unsigned short *buf, int ch, int w,
                                               unsigned voff) {
    const int nblk = (a.D + 15) / 16;
    for (int b = w; b < nblk; b += FF_NW) {
        const int r0 = min(16 * b, a.D - 16);
        const char *src = (const char *)(a.XT + (int64_t)r0 * a.Bp + ch * 32);
        __builtin_amdgcn_global_load_lds(src + voff, (__attribute__((address_space(3))) void *)(
                                                         buf + r0 * 32), 16, 0, 0);
    }
}

template <int F>
__global__ __launch_bounds__(64 * FF_NW, 1) void k_fanin1_fwd(TailArgs a, int store_z, int do_loss) {
    __shared__ __attribute__((aligned(16))) unsigned short fbuf0[FF_BUF_BYTES / 2];
    __shared__ __attribute__((aligned(16))) unsigned short fbuf1[FF_BUF_BYTES / 2];
    __shared__ __attribute__((aligned(16))) unsigned tab[FF_R][F];  // row offset | bf16 weight << 16
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int qd = lane >> 4, rp = lane & 15;      // label of the quad, row pair
    const unsigned voff = (unsigned)((lane >> 2) * a.Bp + 8 * (lane & 3)) * 2u;
    const int nch = a.Bp / 32;
    const int64_t t_begin = (int64_t)blockIdx.x * FF_R;
    float lsum = 0.f;

    ff_stage_async(a, fbuf0, 0, wu, voff);
    // the workgroup's tables (labels past L: offset 0, weight 0)
    for (int e = threadIdx.x; e < FF_R * F; e += 64 * FF_NW) {
        const int64_t t = t_begin + e / F;
        unsigned v = 0;
        if (t < a.L) v = (unsigned)a.idx[t * F + e % F] * 64u | (unsigned)a.W[t * F + e % F] << 16;
        tab[e / F][e % F] = v;
    }
    // this lane's two labels (quads 8w..8w+3 and 8w+4..8w+7) and their positives
    int p0[2], p1[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int64_t t = t_begin + 8 * wu + 4 * k + qd;
        p0[k] = p1[k] = 0;
        if (t < a.L) {
            p0[k] = a.grp_ptr[t];
            p1[k] = a.grp_ptr[t + 1];
        }
    }

    auto chunk = [&](const unsigned short *tile, const int ch) {
        const int row0 = ch * 32 + 2 * rp;
        const unsigned char *tb = (const unsigned char *)tile + 4 * rp;
        // both quads of the wave in one loop: two independent chains of LDS
        // round trips (table entries, then the rows they point at)
        float z[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
        const int lt0 = 8 * wu + qd;
#pragma unroll 2
        for (int f4 = 0; f4 < F; f4 += 4) {
            u32x4 v4[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) v4[k] = *(const u32x4 *)&tab[lt0 + 4 * k][f4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const unsigned x2 = *(const unsigned *)(tb + (v4[k][j] & 0xffffu));
                    const float wf = __uint_as_float(v4[k][j] & 0xffff0000u);
                    z[k][0] = __builtin_fmaf(__uint_as_float(x2 << 16), wf, z[k][0]);
                    z[k][1] = __builtin_fmaf(__uint_as_float(x2 & 0xffff0000u), wf, z[k][1]);
                }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t t = t_begin + lt0 + 4 * k;
            if (t >= a.L) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = row0 + i;
                if (row >= a.B) continue;
                if (store_z) a.Z[(int64_t)row * a.L + t] = f32_to_bf16(z[k][i]);
                if (do_loss) {
                    float y = 0.f;
                    for (int e = p0[k]; e < p1[k]; ++e) y = a.grp_ent[e] == row ? 1.f : y;
                    lsum += a.s * ((fmaxf(z[k][i], 0.f) - y * z[k][i]) + log1p_pos(fast_exp_neg_abs(z[k][i])));
                }
            }
        }
    };
    // nch is even (Bp is a multiple of 64); the first barrier also publishes the tables
    for (int ch = 0; ch < nch; ch += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        ff_stage_async(a, fbuf1, ch + 1, wu, voff);
        chunk(fbuf0, ch);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (ch + 2 < nch) ff_stage_async(a, fbuf0, ch + 2, wu, voff);
        chunk(fbuf1, ch + 1);
    }
    // no copy into buffer 0 is pending after the last chunk pair
    if (do_loss && a.loss) block_loss_add(lsum, (float *)fbuf0, a.loss);
}

hipError_t launch_fanin1_fwd(const TailArgs &a, bool store_z, bool do_loss, hipStream_t st) {
    if (a.D > FF_BUF_BYTES / 64 || a.D < 16) return hipErrorInvalidValue;
    const int64_t grid = (a.L + FF_R - 1) / FF_R;
    if (grid <= 0) return hipSuccess;
#define FFCASE(FF)                                                                                 \
    if (a.F == FF) {                                                                               \
        hipLaunchKernelGGL((k_fanin1_fwd<FF>), dim3((unsigned)grid), dim3(64 * FF_NW), 0, st, a,   \
                           (int)store_z, (int)do_loss);                                            \
        return hipGetLastError();                                                                  \
    }
    FFCASE(32)
    FFCASE(64)
    FFCASE(128)
#undef FFCASE
    return hipErrorInvalidValue;
}

// Training step of the per-label layer (G = 1): the forward's logits and
// loss, then dz = s (sigmoid(z) - y) (zero past B and L) and dW[t][f] =
// sum_b X[b][idx[t][f]] dz[b][t] over the batch.  dz also goes to HBM
// label-major (dzt: L x Bp bf16) for the dX pass.  Workgroup = FS_R labels
// over the whole batch, four per wave (a quarter-wave per label, a lane per
// two adjacent rows, as in the forward).  Per chunk the wave's four labels'
// dz pass through LDS (fp32, 4 x 32); then each lane takes one label
// (lane / 16) and every sixteenth of its features (lane % 16 + 16j): 32 FMAs
// per feature over the chunk's rows, read as four 16-byte pieces of the
// feature's X^T row.  A row's pieces fall in four bank groups that depend on
// the feature, so the lanes of a label start at different pieces (the same
// rotation picks the dz they multiply, which keeps every register index
// static).  The chunk buffers are 60 KB (D <= 960).
constexpr int FS_BUF_BYTES = 60 * 1024;
constexpr int FS_R = 32;                   // labels per workgroup (four per wave)

template <int F>
__global__ __launch_bounds__(64 * FF_NW, 1) void k_fanin1_step(TailArgs a, int do_loss) {
    constexpr int FJ = F / 16;   // features per lane
    __shared__ __attribute__((aligned(16))) unsigned short fbuf0[FS_BUF_BYTES / 2];
    __shared__ __attribute__((aligned(16))) unsigned short fbuf1[FS_BUF_BYTES / 2];
    __shared__ __attribute__((aligned(16))) unsigned tab[FS_R][F];  // row offset | bf16 weight << 16
    __shared__ __attribute__((aligned(16))) float dzl[FF_NW][4][32];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int qd = lane >> 4, rp = lane & 15;      // the label of the quarter-wave, row pair / first feature
    const int rot = rp & 3;                        // phase B: first 16-byte piece
    const unsigned voff = (unsigned)((lane >> 2) * a.Bp + 8 * (lane & 3)) * 2u;
    const int nch = a.Bp / 32;
    const int64_t t_begin = (int64_t)blockIdx.x * FS_R;
    const int lt = 4 * wu + qd;                    // this lane's label in the workgroup
    const int64_t t = t_begin + lt;
    float lsum = 0.f;

    ff_stage_async(a, fbuf0, 0, wu, voff);
    for (int e = threadIdx.x; e < FS_R * F; e += 64 * FF_NW) {
        const int64_t te = t_begin + e / F;
        unsigned v = 0;
        if (te < a.L) v = (unsigned)a.idx[te * F + e % F] * 64u | (unsigned)a.W[te * F + e % F] << 16;
        tab[e / F][e % F] = v;
    }
    int p0 = 0, p1 = 0;
    if (t < a.L) {
        p0 = a.grp_ptr[t];
        p1 = a.grp_ptr[t + 1];
    }
    float acc[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[j] = 0.f;
    unsigned offs[FJ];   // phase B: byte offsets of this lane's feature rows (after the first barrier)

    auto chunk = [&](const unsigned short *tile, const int ch) {
        const int row0 = ch * 32 + 2 * rp;
        const unsigned char *tb = (const unsigned char *)tile + 4 * rp;
        float z0 = 0.f, z1 = 0.f;
#pragma unroll 4
        for (int f4 = 0; f4 < F; f4 += 4) {
            const u32x4 v4 = *(const u32x4 *)&tab[lt][f4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned x2 = *(const unsigned *)(tb + (v4[j] & 0xffffu));
                const float wf = __uint_as_float(v4[j] & 0xffff0000u);
                z0 = __builtin_fmaf(__uint_as_float(x2 << 16), wf, z0);
                z1 = __builtin_fmaf(__uint_as_float(x2 & 0xffff0000u), wf, z1);
            }
        }
        // phase A: dz and the loss; dz to LDS (this wave's labels) and to HBM
        float dz[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float z = i ? z1 : z0;
            const int row = row0 + i;
            dz[i] = 0.f;
            if (t < a.L && row < a.B) {
                float y = 0.f;
                for (int e = p0; e < p1; ++e) y = a.grp_ent[e] == row ? 1.f : y;
                const float ex = fast_exp_neg_abs(z);
                float den;
                dz[i] = a.s * (fast_sigmoid(z, ex, den) - y);
                if (do_loss) lsum += a.s * ((fmaxf(z, 0.f) - y * z) + log1p_pos(ex));
            }
        }
        *(float2 *)&dzl[wu][qd][2 * rp] = make_float2(dz[0], dz[1]);
        if (t < a.L) *(unsigned *)(a.dzt + t * a.Bp + row0) = pack_bf16x2(dz[0], dz[1]);
        // the wave's own LDS writes are in order before its reads below
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // phase B: dW over the chunk's rows, one 16-byte piece (8 rows) of
        // every feature row at a time, the pieces in the lane's rotated order
        const unsigned char *tt = (const unsigned char *)tile;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int pp = (p + rot) & 3;
            const f32x4 lo = *(const f32x4 *)&dzl[wu][qd][8 * pp];
            const f32x4 hi = *(const f32x4 *)&dzl[wu][qd][8 * pp + 4];
            const float dr[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const u32x4 x = *(const u32x4 *)(tt + offs[j] + 16 * pp);
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s0 = __builtin_fmaf(__uint_as_float(x[e] << 16), dr[2 * e], s0);
                    s1 = __builtin_fmaf(__uint_as_float(x[e] & 0xffff0000u), dr[2 * e + 1], s1);
                }
                acc[j] += s0 + s1;
            }
        }
    };
    for (int ch = 0; ch < nch; ch += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (ch == 0) {   // the tables are complete after the first barrier
#pragma unroll
            for (int j = 0; j < FJ; ++j) offs[j] = tab[lt][rp + 16 * j] & 0xffffu;
        }
        ff_stage_async(a, fbuf1, ch + 1, wu, voff);
        chunk(fbuf0, ch);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (ch + 2 < nch) ff_stage_async(a, fbuf0, ch + 2, wu, voff);
        chunk(fbuf1, ch + 1);
    }
    if (t < a.L) {
#pragma unroll
        for (int j = 0; j < FJ; ++j) a.dW[t * F + rp + 16 * j] = f32_to_bf16(acc[j]);
    }
    // no copy into buffer 0 is pending after the last chunk pair
    if (do_loss && a.loss) block_loss_add(lsum, (float *)fbuf0, a.loss);
}

// dX of the per-label layer from the step's label-major dz: dX[b][d] +=
// dz[b][t] W[t][f] for every (t, f) with idx[t][f] = d.  Workgroup = 32 rows
// x a range of labels; its dX^T tile (D x 32 fp32) stays in LDS, the four
// rows 4w..4w+3 of feature d in the 16 bytes at d*128 + 16 (w ^ (d & 7)) (so
// that the lanes' 16-byte pieces spread over the banks).  The range's labels
// come through LDS in batches of FX_NB (idx, W, dz), loaded into registers
// one batch ahead.  Wave w owns rows 4w..4w+3; per label a lane takes a
// feature (lane, lane + 64) and adds dz[rows][t] W[t][f] to its four rows of
// feature idx[t][f]: one 16-byte read, four FMAs, one 16-byte write.  The
// features of a label are distinct and the waves' rows are, so no two lanes
// touch one element at once.  The tile is flushed once with coalesced fp32
// atomics.
constexpr int FX_NW = 8, FX_NB = 16;

template <int F>
struct FxBatch {
    static constexpr int IDX = FX_NB * F * 4 / 16;      // 16-byte pieces of idx
    static constexpr int WP = FX_NB * F * 2 / 16;       // of W
    static constexpr int DZ = FX_NB * 32 * 2 / 16;      // of dz
    static constexpr int N = IDX + WP + DZ;
    static constexpr int PPT = (N + 64 * FX_NW - 1) / (64 * FX_NW);   // pieces per thread
    static constexpr int BYTES = N * 16;
};

__host__ __device__ inline size_t fx_lds_bytes(int D, int F) {
    return (size_t)D * 128 + (size_t)FX_NB * (F * 6 + 64);
}

template <int F>
__global__ __launch_bounds__(64 * FX_NW, 1) void k_fanin1_dx(TailArgs a, int nrc, int64_t per) {
    using Bt = FxBatch<F>;
    extern __shared__ __attribute__((aligned(16))) unsigned char fx_lds[];
    float *const dxt = (float *)fx_lds;
    unsigned char *const bat = fx_lds + (size_t)a.D * 128;   // idx, then W, then dz
    const int32_t *const bidx = (const int32_t *)bat;
    const unsigned short *const bw = (const unsigned short *)(bat + Bt::IDX * 16);
    const unsigned short *const bdz = (const unsigned short *)(bat + (Bt::IDX + Bt::WP) * 16);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
    // blocks: the row chunks of one label range run on one XCD (block b on XCD b % 8)
    const int k8 = blockIdx.x >> 3, xcd = blockIdx.x & 7;
    const int rc = k8 % nrc;
    const int64_t rg = (int64_t)(k8 / nrc) * 8 + xcd;
    const int r0 = rc * 32;
    const int64_t t0 = rg * per;
    const int64_t t1 = t0 + per < a.L ? t0 + per : a.L;
    if (t0 >= t1) return;   // an empty range (workgroup-uniform)
    for (int i = tid; i < a.D * 32; i += 64 * FX_NW) dxt[i] = 0.f;

    auto load = [&](int64_t tb, u32x4 (&r)[Bt::PPT]) {
#pragma unroll
        for (int n = 0; n < Bt::PPT; ++n) {
            const int pc = tid + 64 * FX_NW * n;
            const char *src;
            if (pc < Bt::IDX) {
                const int64_t e = tb * F + 4 * (int64_t)pc;    // F ints a label, contiguous
                src = (const char *)(a.idx + (e < a.L * F ? e : a.L * F - 4));
            } else if (pc < Bt::IDX + Bt::WP) {
                const int64_t e = tb * F + 8 * (int64_t)(pc - Bt::IDX);
                src = (const char *)(a.W + (e < a.L * F ? e : a.L * F - 8));
            } else {
                const int q = pc - Bt::IDX - Bt::WP, l = q >> 2;   // four pieces a label
                const int64_t t = tb + l < a.L ? tb + l : a.L - 1;
                src = (const char *)(a.dzt + t * a.Bp + r0 + 8 * (q & 3));
            }
            r[n] = pc < Bt::N ? *(const u32x4 *)src : (u32x4){0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](const u32x4 (&r)[Bt::PPT]) {
#pragma unroll
        for (int n = 0; n < Bt::PPT; ++n) {
            const int pc = tid + 64 * FX_NW * n;
            if (pc < Bt::N) *(u32x4 *)(bat + 16 * pc) = r[n];
        }
    };
    u32x4 pf[Bt::PPT];
    load(t0, pf);
    for (int64_t tb = t0; tb < t1; tb += FX_NB) {
        __syncthreads();           // the previous batch is consumed (and the tile zeroed)
        store(pf);
        if (tb + FX_NB < t1) load(tb + FX_NB, pf);
        __syncthreads();
        const int nl = t1 - tb < FX_NB ? (int)(t1 - tb) : FX_NB;
        // a label's operands are read one label ahead; its two features'
        // read-modify-writes are issued together (the features of a label
        // are distinct, so their pieces are too)
        constexpr int KF = (F + 63) / 64;
        struct Ops {
            int d[KF];
            float wt[KF];
            u32x2 dz2;
        };
        auto ops = [&](int l) {
            Ops o;
            o.dz2 = *(const u32x2 *)(bdz + l * 32 + 4 * w);   // rows 4w..4w+3 (broadcast)
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int f = lane + 64 * k < F ? lane + 64 * k : F - 1;
                o.d[k] = bidx[l * F + f];
                o.wt[k] = __uint_as_float((unsigned)bw[l * F + f] << 16);
            }
            return o;
        };
        Ops nx = ops(0);
        for (int l = 0; l < nl; ++l) {
            const Ops o = nx;
            if (l + 1 < nl) nx = ops(l + 1);
            const float dz[4] = {__uint_as_float(o.dz2.x << 16), __uint_as_float(o.dz2.x & 0xffff0000u),
                                 __uint_as_float(o.dz2.y << 16), __uint_as_float(o.dz2.y & 0xffff0000u)};
            f32x4 *e[KF];
            f32x4 v[KF];
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                e[k] = (f32x4 *)(dxt + o.d[k] * 32 + 4 * (w ^ (o.d[k] & 7)));
                v[k] = *e[k];
            }
#pragma unroll
            for (int k = 0; k < KF; ++k) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[k][i] = __builtin_fmaf(dz[i], o.wt[k], v[k][i]);
                if (lane + 64 * k < F) *e[k] = v[k];
            }
        }
    }
    __syncthreads();
    // flush: lanes over consecutive features of one row
    for (int i = tid; i < a.D * 32; i += 64 * FX_NW) {
        const int rr = i / a.D, d = i - rr * a.D;
        if (r0 + rr < a.B)
            atomicAdd(a.dX + (int64_t)(r0 + rr) * a.D + d, dxt[d * 32 + 4 * ((rr >> 2) ^ (d & 7)) + (rr & 3)]);
    }
}

bool fanin1_step_supported(int F, int D) {
    return (F == 32 || F == 64 || F == 128) && D >= 16 && D <= FS_BUF_BYTES / 64 &&
           fx_lds_bytes(D, F) <= 160 * 1024;
}

hipError_t launch_fanin1_step(const TailArgs &a, bool do_loss, hipStream_t st) {
    if (!fanin1_step_supported(a.F, a.D) || !a.dzt || !a.dW || !a.dX || a.Bp % 64) return hipErrorInvalidValue;
    const int64_t grid = (a.L + FS_R - 1) / FS_R;
    if (grid <= 0) return hipSuccess;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const int nrc = a.Bp / 32;
    int ngr = (ncu + nrc - 1) / nrc;
    ngr = (ngr + 7) / 8 * 8;
    const int64_t per = ((a.L + ngr - 1) / ngr + FX_NB - 1) / FX_NB * FX_NB;
    const size_t lds = fx_lds_bytes(a.D, a.F);
#define FSCASE(FF)                                                                                 \
    if (a.F == FF) {                                                                               \
        hipLaunchKernelGGL((k_fanin1_step<FF>), dim3((unsigned)grid), dim3(64 * FF_NW), 0, st, a,  \
                           (int)do_loss);                                                          \
        allow_lds((const void *)k_fanin1_dx<FF>, lds);                                             \
        hipLaunchKernelGGL((k_fanin1_dx<FF>), dim3((unsigned)(nrc * ngr)), dim3(64 * FX_NW), lds,  \
                           st, a, nrc, per);                                                       \
        return hipGetLastError();                                                                  \
    }
    FSCASE(32)
    FSCASE(64)
    FSCASE(128)
#undef FSCASE
    return hipErrorInvalidValue;
}

hipError_t launch_tail_t1(int mode, int G, const TailArgs &a, bool store_z, bool do_loss,
                          hipStream_t st) {
    // Groups of 64 at F = 128 without a fused top-K: each wave takes a
    // 32-label slice of a group (8 waves of 256 registers, as for groups of
    // 32); a whole group per wave needs 512 registers, four waves per
    // workgroup, too few to hide the chunk loop's latencies.  Measured on the
    // 670K-label workload (c3 shape): 433 us against 562 us whole-group and
    // 451 us with 16-label slices (16 waves); groups of 32 kept whole ran
    // 1,019 us against 1,105 us in 16-label slices on the 3M-label workload.
    if (a.tk_v == nullptr && G == 64 && a.F == 128)
        return t1_launch<32, 128, 1, 8, 64>(mode, a, store_z, do_loss, st);
#define T1CASE(GG, FF, RR, NN) \
    if (G == GG && a.F == FF) return t1_launch<GG, FF, RR, NN>(mode, a, store_z, do_loss, st);
    T1CASE(16, 32, 2, 16)
    T1CASE(16, 64, 1, 16)
    T1CASE(16, 128, 1, 16)
    T1CASE(32, 32, 1, 16)
    T1CASE(32, 64, 1, 16)
    T1CASE(32, 128, 1, 8)
    T1CASE(64, 32, 2, 8)
    T1CASE(64, 64, 1, 8)
    T1CASE(64, 128, 1, 4)
#undef T1CASE
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------- T2
// Workgroup = (row chunk of BC2 rows) x (range of groups), 16 waves in three
// roles, each SIMD hosting two consumers, one Z^T wave and one builder:
//   consumers (8): own all BC2 rows x NTW32 32-feature tiles of the dX
//     accumulator, in 32x32 MFMA accumulators for the whole group range, and
//     run only the dense product;
//   Z^T waves (4): recompute Z^T and dz;
//   builders (4): build W^T and the inverse index.
//
// Per group g the dense product dX_chunk += dz_g (rows x G) * W~_g (G x D)
// runs on v_mfma_f32_32x32x16_bf16 (K = 16 labels per instruction), where
// W~_g is W_g^T scattered to the rows idx_g and zero elsewhere: the B
// operand of feature d is row f of W_g^T when idx_g[f] = d, else a zero row
// (the inverse index d -> f is rebuilt per group).
//
// Groups are processed GPI at a time ("steps"), so that the recompute of
// Z^T has at least eight 16x16 tiles per step.  One barrier per step.  The
// Z^T waves and builders load their operands (idx_g, W_g rows, the pointer
// pair of the group-major positives) straight from global memory into
// registers, four steps ahead of use, and work two steps ahead of the
// consumers, so that none of their memory or MFMA latencies is on the path
// of a step.  Iteration k:
//   consumers: dense product of step k;
//   Z^T waves: sigmoid-BCE epilogue of step k+1 (from the Z^T accumulators
//     of the previous iteration) -> dz, stored in LDS in the A-operand layout
//     of the 32x32x16 product; gather (transposing reads of the chunk at rows
//     idx) and MFMAs of step k+2 and the load of its positives; load the
//     operands of step k+4;
//   builders: W^T ([f][j]) and the inverse index of step k+2; load step k+4;
//   all: clear the inverse index of step k-1, barrier.
//
// Bank spreading: the chunk's 16-byte units are rotated by the row index,
// W^T rows are padded by 8 bytes.
constexpr int T2_NC = 8, T2_NZ = 4, T2_NB = 4;   // consumer, Z^T and W^T waves
constexpr int T2_NW = T2_NC + T2_NZ + T2_NB;

__host__ __device__ constexpr int t2_gpi(int G, int BC2) {
    return (G / 16) * (BC2 / 16) * 2 <= 8 ? 2 : 1;
}

struct T2Lds {  // byte offsets and sizes of the LDS regions (host and device agree)
    int wts, wts_grp, inv, ndp, exch, exch_grp, total;
};

__host__ __device__ inline T2Lds t2_layout(int D, int F, int G, int BC2, int NTW32) {
    T2Lds L;
    const int GPI = t2_gpi(G, BC2);
    L.ndp = T2_NC * NTW32 * 32;
    int o = (D * BC2 * 2 + 15) & ~15;            // X^T chunk, rows of BC2 bf16
    L.wts = o;
    L.wts_grp = (F + 1) * (G * 2 + 16);          // W_g^T (padded rows) + zero row F
    o += 3 * GPI * L.wts_grp;                    // three steps
    L.inv = o;
    o += (4 * GPI * L.ndp + 15) & ~15;           // u8 inverse index, four steps
    L.exch = o;
    L.exch_grp = BC2 * G * 2;                    // dz of one group, MFMA A layout
    o += 2 * GPI * L.exch_grp;
    L.total = o;
    return L;
}

template <int G, int BC2, int NTW32>
__global__ __launch_bounds__(64 * T2_NW, 1) void k_tail_t2(TailArgs a, int dz_mode, int n_granges) {
    constexpr int NT = 64 * T2_NW;
    constexpr int GPI = t2_gpi(G, BC2);
    constexpr int JT = G / 16, BT = BC2 / 16, RT = BC2 / 32;
    constexpr int NU = BC2 / 8;                // 16-byte units per chunk row
    constexpr int GPR = G / 4, LGPR = G == 16 ? 2 : G == 32 ? 3 : 4;
    // W^T row stride, bytes: 16 bytes of padding keep every operand read one
    // aligned 16-byte read (a pair of 8-byte reads costs about twice as much)
    constexpr int WTS = G * 2 + 16;
    constexpr int NDP = T2_NC * NTW32 * 32;    // features covered by the consumer waves
    constexpr int LROW = BC2 == 64 ? 7 : 6;    // log2 of a chunk row in bytes
    constexpr int NTILE = GPI * JT * BT;       // 16x16 Z^T tiles per step
    constexpr int TPW = NTILE / T2_NZ;         // tiles per Z^T wave (same group and label tile)
    static_assert(NTILE % T2_NZ == 0 && BT % TPW == 0, "Z^T tile split");
    constexpr int NB_T = T2_NB * 64;           // builder threads
    constexpr int UPT = (GPI * GPR * 32 + NB_T - 1) / NB_T;   // W^T units per builder thread (F <= 128)
    const int F = a.F, KS = F / 32;
    const int lf4 = F == 128 ? 5 : F == 64 ? 4 : 3;        // log2(F/4)
    const int lnq = LGPR + lf4;                             // log2(W^T units per group)
    const T2Lds LY = t2_layout(a.D, F, G, BC2, NTW32);
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *tile = lds;
    unsigned char *wts0 = lds + LY.wts;
    unsigned char *inv0 = lds + LY.inv;
    unsigned char *exch0 = lds + LY.exch;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hq = lane >> 4, m = lane & 15;
    const int gr = blockIdx.x % n_granges, bch = blockIdx.x / n_granges;
    const int64_t gA = (int64_t)gr * a.Ng / n_granges, gB = (int64_t)(gr + 1) * a.Ng / n_granges;
    const int ng = (int)(gB - gA);
    // labels from the range's first one on, at most INT_MAX: bounds in 32-bit
    // arithmetic (gA is below the unit count, so this is positive)
    const int lrem = (int)(a.L - gA * G < 0x7fffffff ? a.L - gA * G : 0x7fffffff);
    const int nsteps = (ng + GPI - 1) / GPI;
    const int r0 = bch * BC2;
    // wave roles (uniform): consumers 0..7, Z^T waves 8..11, builders 12..15
    const int role = w < T2_NC ? 0 : w < T2_NC + T2_NZ ? 1 : 2;
    auto live = [&](int k, int q) { return k * GPI + q < ng; };   // 32-bit, scalar

    const int dz_mem = dz_mode;             // dz not recomputed (modes 1, 2)
    {   // stage the chunk (units rotated by row), reset the inverse maps, zero rows
        const unsigned short *src = a.XT + r0;
        for (int i = tid; i < (dz_mode == 0 ? a.D * NU : 0); i += NT) {
            const int d = i / NU, u = i % NU;
            *(u32x4 *)(tile + (d << LROW) + (((u + d) & (NU - 1)) << 4)) =
                *(const u32x4 *)(src + (int64_t)d * a.Bp + u * 8);
        }
        const unsigned fill = (unsigned)F * 0x01010101u;
        for (int i = tid; i < 4 * GPI * NDP / 4; i += NT) ((unsigned *)inv0)[i] = fill;
        for (int i = tid; i < 3 * GPI * (G / 2); i += NT)
            ((unsigned *)(wts0 + (i / (G / 2)) * LY.wts_grp + F * WTS))[i % (G / 2)] = 0u;
    }
    __syncthreads();

    // Per-iteration tail shared by all roles: clear the inverse index of step
    // k-1 (no longer read), barrier.  Each role runs its own loop so that its
    // registers are not live in the other roles' code; every loop passes the
    // same number of barriers.
    const unsigned fill = (unsigned)F * 0x01010101u;
    auto close_step = [&](int k) {
        unsigned *ivp = (unsigned *)(inv0 + ((k + 3) & 3) * GPI * NDP);
        for (int i = tid; i < GPI * NDP / 4; i += NT) ivp[i] = fill;
        lds_barrier();
    };

    if (role == 0) {
        // ---------------------------------------------------------- consumers
        const int dbase = w * NTW32 * 32;      // first feature of this wave
        f32x16 acc[RT][NTW32];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < NTW32; ++nt) acc[rt][nt] = (f32x16){};
        __syncthreads();                       // prologue of the other roles
        int sw = 0;                            // W^T buffer of step k (k mod 3)
        for (int k = 0; k < nsteps; ++k) {
            const unsigned char *wts = wts0 + sw * GPI * LY.wts_grp;
            const unsigned char *inv = inv0 + (k & 3) * GPI * NDP;
            const unsigned char *exch = exch0 + (k & 1) * GPI * LY.exch_grp;
#pragma unroll
            for (int q = 0; q < GPI; ++q) {
                if (!live(k, q)) break;
                const unsigned char *wt = wts + q * LY.wts_grp + 16 * (lane >> 5);
                const unsigned char *iv = inv + q * NDP + dbase + (lane & 31);
                const unsigned char *brow[NTW32];
#pragma unroll
                for (int nt = 0; nt < NTW32; ++nt) brow[nt] = wt + iv[32 * nt] * WTS;
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) {
                    bf16x8 Am[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        Am[rt] = *(const bf16x8 *)(exch + q * LY.exch_grp + ((rt * JT + jt) * 64 + lane) * 16);
#pragma unroll
                    for (int nt = 0; nt < NTW32; ++nt) {   // labels 16jt + 8(lane/32) .. +7 of row f
                        const bf16x8 Bv = *(const bf16x8 *)(brow[nt] + 32 * jt);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = mfma32x32(Am[rt], Bv, acc[rt][nt]);
                    }
                }
            }
            close_step(k);
            sw = sw == 2 ? 0 : sw + 1;
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
    } else if (role == 1 && dz_mode == 2) {
        // --------------------------------------------------- dz tile loaders
        // dz comes from the tiles of the dW pass: wave p copies tile p of a
        // step (group q, 32-row block rt, label tile jt; at most four per
        // step) into exch, transposed from the dW pass's layout (lane (qq, mm):
        // rows 4qq+i and 16+4qq+i of label mm) into the A-operand layout
        // (lane: one row, eight consecutive labels).  Loads run four steps
        // ahead.
        constexpr int NBLK = GPI * RT * JT;
        static_assert(NBLK <= T2_NZ, "one dz tile per loader wave");
        const int blk = w - T2_NC;
        const bool act = blk < NBLK;
        const int q = blk / (RT * JT), rt = (blk / JT) % RT, jt = blk % JT;
        const int64_t nch32 = a.Bp / 32;
        const int mm = lane & 15, qq = lane >> 4;
        auto fetch = [&](int k, u32x4 &v) {
            if (!act || !live(k, q)) return;
            const int64_t g = gA + (int64_t)k * GPI + q;
            v = *(const u32x4 *)(a.dzt + (((g * nch32 + (r0 >> 5) + rt) * JT + jt) << 9) + lane * 8);
        };
        auto put = [&](int k, const u32x4 &v) {
            if (!act || !live(k, q)) return;
            unsigned char *ex = exch0 + ((k & 1) * GPI + q) * LY.exch_grp + (rt * JT + jt) * 1024 +
                                (32 * (mm >> 3)) * 16 + 2 * (mm & 7);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int rho = 16 * (e >> 2) + 4 * qq + (e & 3);
                const unsigned wv = v[e >> 1];
                *(unsigned short *)(ex + rho * 16) = (unsigned short)((e & 1) ? (wv >> 16) : (wv & 0xffffu));
            }
        };
        u32x4 s0 = {}, s1 = {}, s2 = {}, s3 = {};
        fetch(0, s0);
        fetch(1, s1);
        fetch(2, s2);
        fetch(3, s3);
        put(0, s0);
        fetch(4, s0);
        __syncthreads();
        // iteration k: step k+1 is in set (k+1) mod 4; it then receives step k+5
        auto iter = [&](int k, u32x4 &v) {
            put(k + 1, v);
            fetch(k + 5, v);
            close_step(k);
        };
        for (int k = 0; k < nsteps; k += 4) {
            iter(k, s1);
            if (k + 1 < nsteps) iter(k + 1, s2);
            if (k + 2 < nsteps) iter(k + 2, s3);
            if (k + 3 < nsteps) iter(k + 3, s0);
        }
    } else if (role == 1) {
        // ------------------------------------------------------------ Z^T waves
        // Wave p takes tiles p*TPW .. +TPW-1 of a step: one group q and label
        // tile jt, TPW consecutive 16-row tiles bt0.. (lane (hq, m) owns labels
        // 16jt + 4hq .. +3 of row 16bt + m in each).
        const int tl0 = (w - T2_NC) * TPW;
        const int q = tl0 / (JT * BT), jt = (tl0 % (JT * BT)) / BT, bt0 = tl0 % BT;
        const int ch = (m & 1) * 8;
        struct Ops {            // operands of one step, loaded four steps ahead
            int d[8];           // idx[32s + 8hq + m/4] and idx[.. + 4], s < KS
            u32x4 A[4];         // W row 16jt+m, features 32s + 8hq .. +7
            int gp0, gp1;       // group-major positives of the group
        };
        auto fetch = [&](int k, Ops &o) {
            if (!live(k, q) || dz_mem) return;
            const int64_t g = gA + (int64_t)k * GPI + q;
            const int32_t *ix = a.idx + g * F + 8 * hq + (m >> 2);
            const unsigned short *wr = a.W + (g * G + 16 * jt + m) * (int64_t)F + 8 * hq;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s >= KS) break;
                o.d[2 * s] = ix[32 * s];
                o.d[2 * s + 1] = ix[32 * s + 4];
                o.A[s] = *(const u32x4 *)(wr + 32 * s);
            }
            o.gp0 = a.grp_ptr[g];
            o.gp1 = a.grp_ptr[g + 1];
        };
        f32x4 z[TPW];           // Z^T of the step in flight (from the MFMAs of the previous iteration)
        int zg0 = 0, zn = 0;    // its positives: first entry and count (uniform)
        int pe = 0;             // entry zg0 + lane, lane < min(zn, 64)
        // transposing reads of the chunk at rows idx, then the MFMAs, of step
        // k into z; and the load of its positives
        auto part1 = [&](int k, const Ops &o) {
            if (!live(k, q) || dz_mem) return;
            i16x4 b[4][TPW][2];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s >= KS) break;
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    // chunk address of (row d, columns 16bt + 4(m%4) .. +3)
                    const int cu16 = (2 * (bt0 + t) + ((m & 3) >> 1)) << 4;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int d = o.d[2 * s + h];
                        b[s][t][h] = lds_read_tr(tile + ((d << LROW) | ((((d << 4) + cu16) & ((NU - 1) << 4)) | ch)));
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TPW; ++t) z[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s >= KS) break;
                const bf16x8 Av = __builtin_bit_cast(bf16x8, o.A[s]);
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const bf16x8 Bv = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(b[s][t][0], b[s][t][1], 0, 1, 2, 3, 4, 5, 6, 7));
                    z[t] = mfma32(Av, Bv, z[t]);
                }
            }
            zg0 = __builtin_amdgcn_readfirstlane(o.gp0);
            zn = __builtin_amdgcn_readfirstlane(o.gp1) - zg0;
            pe = lane < zn ? a.grp_ent[zg0 + lane] : 0;
        };
        // sigmoid-BCE of step k (Z^T in z) -> dz -> exch
        auto epilogue = [&](int k) {
            if (!live(k, q)) return;
            const int64_t g = gA + (int64_t)k * GPI + q;
            float dzv[TPW][4];
            if (!dz_mem) {
                // positives of this group inside the wave's rows
                unsigned ymask[TPW];
                bool has_pos = false;                // wave-uniform
#pragma unroll
                for (int t = 0; t < TPW; ++t) ymask[t] = 0;
                auto add_pos = [&](const int v) {
                    const int lb = v / G - (r0 + 16 * bt0), j = v % G;
                    if (lb < 0 || lb >= 16 * TPW || (j >> 4) != jt) return;
                    has_pos = true;
#pragma unroll
                    for (int t = 0; t < TPW; ++t)
                        if (lb == 16 * t + m && ((j >> 2) & 3) == hq) ymask[t] |= 1u << (j & 3);
                };
                const int n1 = zn < 64 ? zn : 64;   // registers first, then memory
                for (int e = 0; e < n1; ++e) add_pos(__builtin_amdgcn_readlane(pe, e));
                for (int e = 64; e < zn; ++e) add_pos(a.grp_ent[zg0 + e]);
                // sigmoid(z) = 1 / (1 + 2^(-z log2 e)); saturates cleanly at both ends
                if (!has_pos && r0 + 16 * (bt0 + TPW) <= a.B && (g + 1) * G <= a.L) {
#pragma unroll
                    for (int t = 0; t < TPW; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            dzv[t][i] = a.s * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z[t][i] * -kLog2e));
                } else {
#pragma unroll
                    for (int t = 0; t < TPW; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int64_t lt = g * G + 16 * jt + 4 * hq + i;
                            const bool on = r0 + 16 * (bt0 + t) + m < a.B && lt < a.L;
                            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z[t][i] * -kLog2e));
                            dzv[t][i] = on ? a.s * (sg - (float)((ymask[t] >> i) & 1u)) : 0.f;
                        }
                }
            } else {
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = r0 + 16 * (bt0 + t) + m;
                        const int64_t lt = g * G + 16 * jt + 4 * hq + i;
                        const bool on = row < a.B && lt < a.L;
                        dzv[t][i] = on ? bf16_to_f32(a.dZ[(int64_t)row * a.L + lt]) : 0.f;
                    }
            }
            // (row 16bt+m, label 16jt+4hq+i) -> A operand of the 32-row block bt/2:
            // lane 16(bt%2)+m+32(hq/2), K slots 4(hq%2)+i
            unsigned char *ex = exch0 + (k & 1) * GPI * LY.exch_grp + q * LY.exch_grp;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int bt = bt0 + t;
                const int lane2 = 16 * (bt & 1) + m + 32 * (hq >> 1);
                *(u32x2 *)(ex + (((bt >> 1) * JT + jt) * 64 + lane2) * 16 + 8 * (hq & 1)) =
                    (u32x2){pack_bf16x2(dzv[t][0], dzv[t][1]), pack_bf16x2(dzv[t][2], dzv[t][3])};
            }
        };
        Ops oA, oB;
        fetch(0, oA);
        fetch(1, oB);
        part1(0, oA);
        epilogue(0);
        fetch(2, oA);
        part1(1, oB);
        fetch(3, oB);
        __syncthreads();
        // iteration k: z holds step k+1; oA (k even) / oB (k odd) holds step k+2
        // and then receives step k+4
        auto iter = [&](int k, Ops &o) {
            __builtin_amdgcn_s_setprio(2);     // short chain: issue ahead of the MFMA stream
            epilogue(k + 1);
            part1(k + 2, o);
            __builtin_amdgcn_s_setprio(0);
            fetch(k + 4, o);
            close_step(k);
        };
        for (int k = 0; k < nsteps; k += 2) {   // unrolled by two: the operand sets alternate
            iter(k, oA);
            if (k + 1 < nsteps) iter(k + 1, oB);
        }
    } else {
        // ------------------------------------------------------------- builders
        // Thread = 4 labels x 4 features of W_g.  Four consecutive lanes take
        // consecutive feature quads, then the label quads, then the next
        // features: with the 8-byte row padding the W^T writes of 16 lanes
        // hit distinct banks.
        const int bth = tid - (T2_NC + T2_NZ) * 64;
        struct Ops {
            u32x2 r[UPT][4];    // rows 4ja+e, features 4fc .. +3, per unit
            int fi;             // idx[f] of the inverse-index entry of this thread
        };
        auto unit = [&](int i, int &q, int &fc, int &ja) {
            const int u = bth + NB_T * i;
            q = u >> lnq;
            const int rest = u & ((1 << lnq) - 1), r2 = rest >> 2;
            ja = r2 & (GPR - 1);
            fc = ((r2 >> LGPR) << 2) | (rest & 3);
        };
        auto fetch = [&](int k, Ops &o) {
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                int q, fc, ja;
                unit(i, q, fc, ja);
                if (bth + NB_T * i >= (GPI << lnq) || !live(k, q)) continue;
                const int64_t g = gA + (int64_t)k * GPI + q;
                const unsigned short *wr = a.W + (g * G + 4 * ja) * (int64_t)F + 4 * fc;
#pragma unroll
                for (int e = 0; e < 4; ++e) o.r[i][e] = *(const u32x2 *)(wr + e * F);
            }
            if (bth < GPI * F) {
                const int q = bth / F;
                if (live(k, q)) o.fi = a.idx[(gA + (int64_t)k * GPI + q) * F + (bth - q * F)];
            }
        };
        auto build = [&](int k, const Ops &o) {
            unsigned char *wts = wts0 + (k % 3) * GPI * LY.wts_grp;
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                int q, fc, ja;
                unit(i, q, fc, ja);
                if (bth + NB_T * i >= (GPI << lnq) || !live(k, q)) continue;
                unsigned char *wt = wts + q * LY.wts_grp + (4 * fc) * WTS + 8 * ja;
                // rows of labels past L (a ragged last group) go in as zeros:
                // their dz is zero, and 0 times whatever the caller left in
                // those rows (NaN included) must not reach dX.  Masks on the
                // permuted words (label 4ja + e in half e % 2 of word e / 2),
                // so no loaded register is rewritten before its use
                const int lab0 = (k * GPI + q) * G + 4 * ja;   // from the range's first label
                const unsigned m01 = (lab0 < lrem ? 0x0000ffffu : 0u) | (lab0 + 1 < lrem ? 0xffff0000u : 0u);
                const unsigned m23 = (lab0 + 2 < lrem ? 0x0000ffffu : 0u) | (lab0 + 3 < lrem ? 0xffff0000u : 0u);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {   // feature 4fc+kk: element kk of each row
                    const unsigned sel = (kk & 1) ? 0x07060302u : 0x05040100u;
                    const int wd = kk >> 1;
                    const u32x2 v = {__builtin_amdgcn_perm(o.r[i][1][wd], o.r[i][0][wd], sel) & m01,
                                     __builtin_amdgcn_perm(o.r[i][3][wd], o.r[i][2][wd], sel) & m23};
                    *(u32x2 *)(wt + kk * WTS) = v;
                }
            }
            if (bth < GPI * F) {
                const int q = bth / F;
                if (live(k, q)) inv0[((k & 3) * GPI + q) * NDP + o.fi] = (unsigned char)(bth - q * F);
            }
        };
        Ops oA, oB;
        fetch(0, oA);
        fetch(1, oB);
        build(0, oA);
        build(1, oB);
        fetch(2, oA);
        fetch(3, oB);
        __syncthreads();
        auto iter = [&](int k, Ops &o) {
            build(k + 2, o);
            fetch(k + 4, o);
            close_step(k);
        };
        for (int k = 0; k < nsteps; k += 2) {
            iter(k, oA);
            if (k + 1 < nsteps) iter(k + 1, oB);
        }
    }
}

// ------------------------------------------------------------------ T2d
// dX from the dz tiles of the dW pass (no recompute, no X^T chunk in LDS).
// Workgroup = (row chunk of BC2 rows) x (range of groups), 12 waves:
//   consumers (8): dX_chunk += dz_g * W~_g on 32x32x16 MFMAs as in T2, but
//     the operands of step k+1 (inverse-index lookups, W^T rows, dz) are
//     loaded into registers right behind the MFMAs of step k, so no LDS
//     latency sits between a barrier and the next MFMA;
//   builders (4): per step, W^T and the inverse index of the GPI groups,
//     and the dz tiles transposed from the dW pass's layout into the
//     A-operand layout; their operands (W rows, idx, dz) are loaded from
//     global memory six steps ahead, four iterations before use.
// Buffers of step s: W^T and dz in ring slot s mod 3, the inverse index in
// slot s mod 4.  Iteration k: builders clear the inverse index of step k-1
// and fill step k+2; consumers run step k, loading its later groups and the
// first groups of step k+1 as they go; one barrier.  The barrier is __syncthreads(): with no
// global->LDS copies in flight it waits for LDS operations only, and the
// compiler knows that the loads of step k+1 have landed, so it puts no
// wait for them in front of the MFMAs of step k+1.
constexpr int T2D_NB = 4, T2D_NW = T2_NC + T2D_NB;

// groups per step: for groups of 16 on 64-row chunks and D > 256, twice the
// Z^T-recompute kernel's (half as many barriers; the builders' operand sets
// still fit in registers without spilling); otherwise the same
__host__ __device__ constexpr int t2d_gpi(int G, int BC2, int NTW32) {
    return G == 16 && BC2 == 64 && NTW32 > 1 ? 2 * t2_gpi(G, BC2) : t2_gpi(G, BC2);
}

struct T2dLds {  // byte offsets and sizes of the LDS regions (host and device agree)
    int wts, wts_grp, inv, ndp, exch, exch_grp, total;
};

__host__ __device__ inline T2dLds t2d_layout(int F, int G, int BC2, int NTW32) {
    T2dLds L;
    const int GPI = t2d_gpi(G, BC2, NTW32);
    L.ndp = T2_NC * NTW32 * 32;
    int o = 0;
    L.wts = o;
    L.wts_grp = (F + 1) * (G * 2 + 16);                // W_g^T (padded rows) + zero row F
    o += 3 * GPI * L.wts_grp;
    L.inv = o;
    o += (4 * GPI * L.ndp * 2 + 15) & ~15;            // u16 inverse index (byte offsets)
    L.exch = o;
    L.exch_grp = BC2 * G * 2;                          // dz of one group, MFMA A layout
    o += 3 * GPI * L.exch_grp;
    L.total = o;
    return L;
}

// GS: the layer's group size when each unit of work is a slice of G labels of
// a larger group (GS = G: whole groups).  Unit u is slice u % (GS/G) of group
// u / (GS/G); its weight rows start at u * G, its index row is its group's.
template <int G, int BC2, int NTW32, int GS = G>
__global__ __launch_bounds__(64 * T2D_NW, 1) void k_tail_t2d(TailArgs a, int n_granges) {
    constexpr int NT = 64 * T2D_NW;
    constexpr int NSL = GS / G, JTS = GS / 16;
    static_assert(GS % G == 0, "slices of whole label tiles");
    const int64_t Nu = a.Ng * NSL;
    constexpr int GPI = t2d_gpi(G, BC2, NTW32);
    constexpr int JT = G / 16, RT = BC2 / 32;
    constexpr int GPR = G / 4, LGPR = G == 16 ? 2 : G == 32 ? 3 : 4;
    // W^T row stride, bytes: 16 bytes of padding keep every operand read one
    // aligned 16-byte read (a pair of 8-byte reads costs about twice as much)
    constexpr int WTS = G * 2 + 16;
    constexpr int NDP = T2_NC * NTW32 * 32;    // features covered by the consumer waves
    constexpr int NB_T = T2D_NB * 64;          // builder threads
    constexpr int UPT = (GPI * GPR * 32 + NB_T - 1) / NB_T;   // W^T units per builder thread (F <= 128)
    constexpr int NBLK = GPI * RT * JT;        // 1 KB dz tiles per step
    constexpr int TPB = (NBLK + T2D_NB - 1) / T2D_NB;       // dz tiles per builder wave
    constexpr int FPT = (GPI * 128 + NB_T - 1) / NB_T;      // inverse entries per builder thread (F <= 128)
    const int F = a.F;
    const int lf4 = F == 128 ? 5 : F == 64 ? 4 : 3;        // log2(F/4)
    const int lnq = LGPR + lf4;                             // log2(W^T units per group)
    const T2dLds LY = t2d_layout(F, G, BC2, NTW32);
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *wts0 = lds + LY.wts;
    // inverse index: per feature the byte offset of its W^T row (f * WTS),
    // F * WTS (the zero row) for a feature the group lacks
    unsigned short *inv0 = (unsigned short *)(lds + LY.inv);
    unsigned char *exch0 = lds + LY.exch;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int gr = blockIdx.x % n_granges, bch = blockIdx.x / n_granges;
    const int64_t gA = (int64_t)gr * Nu / n_granges, gB = (int64_t)(gr + 1) * Nu / n_granges;
    const int ng = (int)(gB - gA);
    // labels from the range's first one on, at most INT_MAX: bounds in 32-bit
    // arithmetic (gA is below the unit count, so this is positive)
    const int lrem = (int)(a.L - gA * G < 0x7fffffff ? a.L - gA * G : 0x7fffffff);
    const int nsteps = (ng + GPI - 1) / GPI;
    // iterations: a multiple of four, so the builders' loop body (unrolled
    // by four) has no exits; the extra iterations only pass the barrier
    const int niter = (nsteps + 3) & ~3;
    const int r0 = bch * BC2;
    auto live = [&](int k, int q) { return k * GPI + q < ng; };   // 32-bit, scalar
    const unsigned fill = (unsigned)(F * WTS) * 0x00010001u;

    // inverse maps to "no feature" (row F), zero rows of the W^T buffers
    for (int i = tid; i < 4 * GPI * NDP / 2; i += NT) ((unsigned *)inv0)[i] = fill;
    for (int i = tid; i < 3 * GPI * (G / 2); i += NT)
        ((unsigned *)(wts0 + (i / (G / 2)) * LY.wts_grp + F * WTS))[i % (G / 2)] = 0u;
    __syncthreads();

    if (w < T2_NC) {
        // ---------------------------------------------------------- consumers
        const int dbase = w * NTW32 * 32;      // first feature of this wave
        f32x16 acc[RT][NTW32];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < NTW32; ++nt) acc[rt][nt] = (f32x16){};
        struct Opd {
            bf16x8 A[RT][JT];                  // dz: row 32rt + lane%32, labels 16jt + 8(lane/32) ..
            bf16x8 Bv[JT][NTW32];              // W~: feature dbase + 32nt + lane%32, same labels
        };
        // Operand sets: with two or more groups per step, group q in set q % 2,
        // the set just used taking group q+2 (of this step, or one of the
        // first two of the next, complete since the previous iteration); with
        // one group per step, one set taking the next step's group.
        constexpr int NS = GPI >= 2 ? 2 : 1;
        // With at least NS + 2 groups per step, the inverse-index entries of a
        // load's group are read one load earlier (that group is then at most
        // in step k+1, whose index is complete), so the W~ row reads do not
        // wait for them.  Steps with fewer groups look them up in the load.
        constexpr bool IVPF = GPI >= NS + 2;
        Opd R[NS];
        unsigned ivn[NTW32];
        auto load_iv = [&](int k, int q) {
            const unsigned short *iv = inv0 + ((k & 3) * GPI + q) * NDP + dbase + (lane & 31);
#pragma unroll
            for (int nt = 0; nt < NTW32; ++nt) ivn[nt] = iv[32 * nt];
        };
        // A (dz: row 32rt + lane%32, labels 16jt + 8(lane/32) .. + 7) from the
        // tile as the dW pass wrote it, by two transposing reads of four
        // labels each: in a block of 16 lanes (rows 16h .. 16h + 15, labels
        // 8lh ..), lane 4k + j points at the four rows 16h + 4j .. of label
        // 8lh + 4t + k, which the dW pass's lane (j, label) holds at bytes
        // 8h .. 8h + 7 of its piece (slot 16j + (label ^ 4j))
        const int tr_k = (lane & 15) >> 2, tr_j = lane & 3, tr_h = (lane >> 4) & 1, tr_lh = lane >> 5;
        unsigned tr_off[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int lab = 8 * tr_lh + 4 * t + tr_k;
            tr_off[t] = 16 * (16 * tr_j + (lab ^ (4 * tr_j))) + 8 * tr_h;
        }
        auto load = [&](int k, int q) {
            const unsigned char *wt = wts0 + ((k % 3) * GPI + q) * LY.wts_grp + 16 * (lane >> 5);
            const unsigned char *ex = exch0 + ((k % 3) * GPI + q) * LY.exch_grp;
            if (!IVPF) load_iv(k, q);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) {
                    const unsigned char *tb = ex + (rt * JT + jt) * 1024;
                    const i16x4 a0 = lds_read_tr(tb + tr_off[0]);
                    const i16x4 a1 = lds_read_tr(tb + tr_off[1]);
                    R[q % NS].A[rt][jt] =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
            for (int nt = 0; nt < NTW32; ++nt) {
                const unsigned char *br = wt + ivn[nt];
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) R[q % NS].Bv[jt][nt] = *(const bf16x8 *)(br + 32 * jt);
            }
        };
        __syncthreads();                       // builders have filled steps 0 and 1
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            if (IVPF) load_iv(0, q);
            if (live(0, q)) load(0, q);
        }
        if (IVPF) load_iv(0, NS);
        __syncthreads();                       // step 0 looked up before its inverse index is cleared
        for (int k = 0; k < niter; ++k) {
#pragma unroll
            for (int q = 0; q < GPI; ++q) {
                if (live(k, q)) {
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
                        for (int nt = 0; nt < NTW32; ++nt)
#pragma unroll
                            for (int rt = 0; rt < RT; ++rt)
                                acc[rt][nt] = mfma32x32(R[q % NS].A[rt][jt], R[q % NS].Bv[jt][nt], acc[rt][nt]);
                }
                // operands of group q + NS (this step or the next), then the
                // inverse-index entries of the group after it
                if (q + NS < GPI) {
                    if (live(k, q + NS)) load(k, q + NS);
                } else if (live(k + 1, q + NS - GPI)) {
                    load(k + 1, q + NS - GPI);
                }
                if (IVPF) {
                    if (q + NS + 1 < GPI) load_iv(k, q + NS + 1);
                    else load_iv(k + 1, q + NS + 1 - GPI);
                }
            }
            __syncthreads();
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
    } else {
        // ------------------------------------------------------------- builders
        // W^T: thread = 4 labels x 4 features of W_g (as in T2).  dz: wave p
        // takes tiles p, p+4, .. of a step (group q, 32-row block rt, label
        // tile jt); lane (qq, mm) holds rows 4qq+i and 16+4qq+i of label mm.
        const int bw = w - T2_NC;
        const int bth = tid - T2_NC * 64;
        const int mm = lane & 15, qq = lane >> 4;
        const int64_t nch32 = a.Bp / 32;
        struct Ops {
            u32x2 r[UPT][4];    // rows 4ja+e, features 4fc .. +3, per unit
            int fi[FPT];        // idx[f] of the inverse-index entries bth, bth + NB_T, ..
            u32x4 dz[TPB];      // dz tiles
        };
        auto unit = [&](int i, int &q, int &fc, int &ja) {
            const int u = bth + NB_T * i;
            q = u >> lnq;
            const int rest = u & ((1 << lnq) - 1), r2 = rest >> 2;
            ja = r2 & (GPR - 1);
            fc = ((r2 >> LGPR) << 2) | (rest & 3);
        };
        auto tile_of = [&](int t, int &q, int &rt, int &jt) {
            const int blk = bw + T2D_NB * t;
            q = blk / (RT * JT);
            rt = (blk / JT) % RT;
            jt = blk % JT;
            return blk < NBLK;
        };
        // Every load is issued on every path, from a clamped address where
        // the group, unit or tile does not exist (the value is then unused):
        // with no load skipped, the compiler can wait for exactly the set it
        // needs instead of for all loads in flight.
        // unit (group slice) of step k's slot q, clamped to the last one; the
        // clamp in 32-bit arithmetic (gA < Nu, so the bound is >= 0)
        const int ulast = (int)(Nu - 1 - gA < 0x7fffffff ? Nu - 1 - gA : 0x7fffffff);
        auto gsafe = [&](int k, int q) {
            const int r = k * GPI + q;
            return gA + (int64_t)(r < ulast ? r : ulast);
        };
        auto fetch = [&](int k, Ops &o) {
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                int q, fc, ja;
                unit(i, q, fc, ja);
                if (bth + NB_T * i >= (GPI << lnq)) q = fc = ja = 0;
                const unsigned short *wr = a.W + (gsafe(k, q) * G + 4 * ja) * (int64_t)F + 4 * fc;
#pragma unroll
                for (int e = 0; e < 4; ++e) o.r[i][e] = *(const u32x2 *)(wr + e * F);
            }
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                const int e = bth + NB_T * i;
                const int q = e < GPI * F ? e / F : 0;
                const int f = e < GPI * F ? e - q * F : 0;
                o.fi[i] = a.idx[gsafe(k, q) / NSL * F + f];
            }
#pragma unroll
            for (int t = 0; t < TPB; ++t) {
                int q, rt, jt;
                if (!tile_of(t, q, rt, jt)) q = rt = jt = 0;
                const int64_t u = gsafe(k, q);
                o.dz[t] = *(const u32x4 *)(a.dzt + (((u / NSL * nch32 + (r0 >> 5) + rt) * JTS + u % NSL * JT + jt) << 9) +
                                           lane * 8);
            }
        };
        auto build = [&](int k, const Ops &o) {
            unsigned char *wts = wts0 + (k % 3) * GPI * LY.wts_grp;
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                int q, fc, ja;
                unit(i, q, fc, ja);
                if (bth + NB_T * i >= (GPI << lnq) || !live(k, q)) continue;
                unsigned char *wt = wts + q * LY.wts_grp + (4 * fc) * WTS + 8 * ja;
                // rows of labels past L (a ragged last group) go in as zeros:
                // their dz is zero, and 0 times whatever the caller left in
                // those rows (NaN included) must not reach dX.  Masks on the
                // permuted words (label 4ja + e in half e % 2 of word e / 2),
                // so no loaded register is rewritten before its use
                const int lab0 = (k * GPI + q) * G + 4 * ja;   // from the range's first label
                const unsigned m01 = (lab0 < lrem ? 0x0000ffffu : 0u) | (lab0 + 1 < lrem ? 0xffff0000u : 0u);
                const unsigned m23 = (lab0 + 2 < lrem ? 0x0000ffffu : 0u) | (lab0 + 3 < lrem ? 0xffff0000u : 0u);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {   // feature 4fc+kk: element kk of each row
                    const unsigned sel = (kk & 1) ? 0x07060302u : 0x05040100u;
                    const int wd = kk >> 1;
                    const u32x2 v = {__builtin_amdgcn_perm(o.r[i][1][wd], o.r[i][0][wd], sel) & m01,
                                     __builtin_amdgcn_perm(o.r[i][3][wd], o.r[i][2][wd], sel) & m23};
                    *(u32x2 *)(wt + kk * WTS) = v;
                }
            }
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                const int e = bth + NB_T * i;
                if (e >= GPI * F) break;
                const int q = e / F;
                if (live(k, q)) inv0[((k & 3) * GPI + q) * NDP + o.fi[i]] = (unsigned short)((e - q * F) * WTS);
            }
#pragma unroll
            for (int t = 0; t < TPB; ++t) {
                int q, rt, jt;
                if (!tile_of(t, q, rt, jt) || !live(k, q)) continue;
                // the tile as the dW pass wrote it, lane (qq, mm)'s piece at
                // slot 16qq + (mm ^ 4qq): the consumers' transposing reads of
                // one 16-lane block then fall on distinct banks
                unsigned char *ex = exch0 + ((k % 3) * GPI + q) * LY.exch_grp + (rt * JT + jt) * 1024;
                *(u32x4 *)(ex + 16 * (16 * qq + (mm ^ (4 * qq)))) = o.dz[t];
            }
        };
        // operand sets: step s in set s mod 4, loaded four iterations ahead
        Ops o0, o1, o2, o3;
        fetch(0, o0);
        fetch(1, o1);
        fetch(2, o2);
        fetch(3, o3);
        build(0, o0);
        fetch(4, o0);
        build(1, o1);
        fetch(5, o1);
        __syncthreads();
        __syncthreads();
        auto iter = [&](int k, Ops &o) {
            unsigned *ivp = (unsigned *)(inv0 + ((k + 3) & 3) * GPI * NDP);   // step k-1
            for (int i = bth; i < GPI * NDP / 2; i += NB_T) ivp[i] = fill;
            build(k + 2, o);
            fetch(k + 6, o);
            __syncthreads();
        };
        for (int k = 0; k < niter; k += 4) {
            iter(k, o2);
            iter(k + 1, o3);
            iter(k + 2, o0);
            iter(k + 3, o1);
        }
    }
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

static bool t2_fits(int D, int F, int G, int BC2, int NTW32) {
    return t2_layout(D, F, G, BC2, NTW32).total <= 160 * 1024;
}

static int t2_ntw(int D, int BC2) {   // 32-feature tiles per consumer wave
    (void)BC2;
    return ((D + 31) / 32 + T2_NC - 1) / T2_NC;
}

template <int G, int BC2, int NTW32>
static hipError_t t2_go(int dz_mode, const TailArgs &a, hipStream_t st) {
    const int nbch = a.Bp / BC2;
    const int64_t ngr = t2_granges(nbch, a.Ng);
    if (ngr < 1) return hipSuccess;
    const T2Lds L = t2_layout(a.D, a.F, G, BC2, NTW32);
    if (L.total > 160 * 1024) return hipErrorInvalidValue;
    allow_lds((const void *)k_tail_t2<G, BC2, NTW32>, L.total);
    hipLaunchKernelGGL((k_tail_t2<G, BC2, NTW32>), dim3((unsigned)(ngr * nbch)), dim3(64 * T2_NW),
                       L.total, st, a, dz_mode, (int)ngr);
    return hipGetLastError();
}

template <int G, int BC2>
static hipError_t t2_pick_ntw(int dz_mode, const TailArgs &a, hipStream_t st) {
    switch (t2_ntw(a.D, BC2)) {
    case 1: return t2_go<G, BC2, 1>(dz_mode, a, st);
    case 2: return t2_go<G, BC2, 2>(dz_mode, a, st);
    case 3: return t2_go<G, BC2, 3>(dz_mode, a, st);
    }
    if constexpr (BC2 == 32)
        if (t2_ntw(a.D, BC2) == 4) return t2_go<G, BC2, 4>(dz_mode, a, st);
    return hipErrorInvalidValue;
}

template <int G, int BC2, int NTW32, int GS = G>
static hipError_t t2d_go(const TailArgs &a, hipStream_t st) {
    const int nbch = a.Bp / BC2;
    const int64_t ngr = t2_granges(nbch, a.Ng * (GS / G));
    if (ngr < 1) return hipSuccess;
    const T2dLds L = t2d_layout(a.F, G, BC2, NTW32);
    if (L.total > 160 * 1024) return hipErrorInvalidValue;
    allow_lds((const void *)k_tail_t2d<G, BC2, NTW32, GS>, L.total);
    hipLaunchKernelGGL((k_tail_t2d<G, BC2, NTW32, GS>), dim3((unsigned)(ngr * nbch)), dim3(64 * T2D_NW),
                       L.total, st, a, (int)ngr);
    return hipGetLastError();
}

template <int G, int BC2, int GS = G>
static hipError_t t2d_pick_ntw(const TailArgs &a, hipStream_t st) {
    switch (t2_ntw(a.D, BC2)) {
    case 1: return t2d_go<G, BC2, 1, GS>(a, st);
    case 2: return t2d_go<G, BC2, 2, GS>(a, st);
    case 3: return t2d_go<G, BC2, 3, GS>(a, st);
    }
    if constexpr (BC2 == 32)
        if (t2_ntw(a.D, BC2) == 4) return t2d_go<G, BC2, 4, GS>(a, st);
    return hipErrorInvalidValue;
}

// 64-row chunks when the batch is larger than 32 rows and the accumulator
// (2 x NTW32 32x32 tiles per consumer) stays within 96 registers
template <int G>
static hipError_t t2d_pick(const TailArgs &a, hipStream_t st) {
    if constexpr (G < 64)
        if (a.B > 32 && t2_ntw(a.D, 64) <= 3) return t2d_pick_ntw<G, 64>(a, st);
    return t2d_pick_ntw<G, 32>(a, st);
}

// Groups of GS > 16 as GS/16 slices of 16 labels (each slice its own unit of
// the dense product, with the operand sets and 64-row chunks of groups of 16)
template <int GS>
static hipError_t t2d_pick_sliced(const TailArgs &a, hipStream_t st) {
    if (a.B > 32 && t2_ntw(a.D, 64) <= 3) return t2d_pick_ntw<16, 64, GS>(a, st);
    return t2d_pick_ntw<16, 32, GS>(a, st);
}

// 64-row chunks when they fit in LDS, the batch is larger than 32 rows and
// the accumulator (2 x NTW32 32x32 tiles per consumer) stays within 96 registers
static int t2_bc(int G, int F, int D, int B) {
    if (G < 64 && B > 32 && t2_ntw(D, 64) <= 3 && t2_fits(D, F, G, 64, t2_ntw(D, 64))) return 64;
    return 32;
}

template <int G>
static hipError_t t2_pick(int dz_mode, const TailArgs &a, hipStream_t st) {
    if constexpr (G < 64)   // G = 64 always takes 32-row chunks (16 Z^T tiles per 64 rows)
        if (t2_bc(G, a.F, a.D, a.B) == 64) return t2_pick_ntw<G, 64>(dz_mode, a, st);
    return t2_pick_ntw<G, 32>(dz_mode, a, st);
}

hipError_t launch_tail_t2(int G, int dz_mode, const TailArgs &a, hipStream_t st) {
    if (dz_mode < 0 || dz_mode > 2 || (dz_mode == 1 && !a.dZ) || (dz_mode == 2 && !a.dzt))
        return hipErrorInvalidValue;
    if (dz_mode == 2) {
        // The dense form runs D/F times the layer's flops; the scatter form
        // runs the layer's own but pays a fixed cost per group and row chunk.
        // Measured on gfx950: the scatter form is ahead only where the dense
        // form's excess is large and groups are wide (D = 16F, G = 64: 1.18
        // against 1.79 ms); at D = 6F it is behind for G = 16, 32 and 64.
        if (G >= 32 && a.D >= 12 * a.F && tail_dxs_supported(G, a.F, a.D))
            return launch_tail_dxs(G, a, st);
        // Groups of 64 as four slices of 16 labels (measured on the 670K-label
        // workload with groups of 64: 435-440 us against 479-486 us with whole
        // groups in 32-row chunks); groups of 32 stay whole (the same either
        // way on the 3M-label workload)
        if (G == 64) return t2d_pick_sliced<64>(a, st);
        switch (G) {
        case 16: return t2d_pick<16>(a, st);
        case 32: return t2d_pick<32>(a, st);
        case 64: return t2d_pick<64>(a, st);
        }
        return hipErrorInvalidValue;
    }
    switch (G) {
    case 16: return t2_pick<16>(dz_mode, a, st);
    case 32: return t2_pick<32>(dz_mode, a, st);
    case 64: return t2_pick<64>(dz_mode, a, st);
    }
    return hipErrorInvalidValue;
}

bool tail_bf16_supported(int G, int F, int D) {
    if (G == 1) return (F == 32 || F == 64 || F == 128) && D >= F && D >= 16 && D <= 1024;
    if (!(G == 16 || G == 32 || G == 64)) return false;
    if (!(F == 32 || F == 64 || F == 128)) return false;
    if (D < F || D > 1024) return false;
    // T1: two chunk buffers; T2: chunk + pipeline buffers with 32-row chunks at least
    if (t1_buf_bytes(D, 8) > (size_t)T1_BUF_BYTES || t1_buf_bytes(D, 4) > (size_t)T1_BUF_BYTES) return false;
    if (!t2_fits(D, F, G, 32, t2_ntw(D, 32))) return false;
    return true;
}

}  // namespace haste
