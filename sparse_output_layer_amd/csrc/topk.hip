// topk.hip -- per-row top-K of fp32 logits on gfx950 (top-K page, section
// "Method": stage 1 takes the top-K' of every bucket of a row, stage 2
// merges the buckets' lists; with K' = K the result is exact, with K' < K it
// is the page's approximate two-stage top-K).
//
// Order: value descending, ties by smaller id (the same total order as the
// merge of two lists).  A row with fewer than K entries is padded with
// (-inf, -1).
//
// Stage 1 (k_topk_stage1): one workgroup per (row, bucket of TOPK_SEG
// consecutive columns).  Every thread keeps a sorted list of K entries in
// registers over a strided share of the bucket (coalesced reads; a value
// enters only if it beats the thread's K-th entry), then the 256 lists are
// merged pairwise in LDS (eight rounds).  Stage 2 (k_topk_stage2): one
// workgroup per row over the rows' bucket lists, same merge.
#include "common.h"
#include "kernels.h"

namespace haste {

constexpr int TOPK_MAX = 8;
constexpr int TOPK_THREADS = 256;

__device__ __forceinline__ bool tk_before(float va, int32_t ia, float vb, int32_t ib) {
    return va > vb || (va == vb && ia < ib);
}

// Insert (v, id) into the sorted list (l_v, l_i) of K entries if it belongs.
template <int K>
__device__ __forceinline__ void tk_insert(float (&l_v)[K], int32_t (&l_i)[K], float v, int32_t id) {
    if (!tk_before(v, id, l_v[K - 1], l_i[K - 1])) return;
    float cv = v;
    int32_t ci = id;
#pragma unroll
    for (int k = 0; k < K; ++k) {   // bubble the new entry into place
        const bool sw = tk_before(cv, ci, l_v[k], l_i[k]);
        const float tv = l_v[k];
        const int32_t ti = l_i[k];
        l_v[k] = sw ? cv : tv;
        l_i[k] = sw ? ci : ti;
        cv = sw ? tv : cv;
        ci = sw ? ti : ci;
    }
}

// Merge the 256 per-thread lists held in LDS (s_v/s_i, K per thread) and
// write the first K entries of the union to out_v/out_i (thread 0).
template <int K>
__device__ __forceinline__ void tk_block_merge(float *s_v, int32_t *s_i, float (&l_v)[K],
                                               int32_t (&l_i)[K], float *out_v, int32_t *out_i) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        s_v[t * K + k] = l_v[k];
        s_i[t * K + k] = l_i[k];
    }
    __syncthreads();
    for (int half = TOPK_THREADS / 2; half > 0; half >>= 1) {
        if (t < half) {
            // two sorted lists -> first K of their union
            const float *av = s_v + t * K, *bv = s_v + (t + half) * K;
            const int32_t *ai = s_i + t * K, *bi = s_i + (t + half) * K;
            int x = 0, y = 0;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float va = av[x < K ? x : K - 1], vb = bv[y < K ? y : K - 1];
                const int32_t ia = ai[x < K ? x : K - 1], ib = bi[y < K ? y : K - 1];
                const bool takea = y >= K || (x < K && tk_before(va, ia, vb, ib));
                l_v[k] = takea ? va : vb;
                l_i[k] = takea ? ia : ib;
                x += takea ? 1 : 0;
                y += takea ? 0 : 1;
            }
        }
        __syncthreads();
        if (t < half) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                s_v[t * K + k] = l_v[k];
                s_i[t * K + k] = l_i[k];
            }
        }
        __syncthreads();
    }
    if (t == 0) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            out_v[k] = s_v[k];
            out_i[k] = s_i[k];
        }
    }
}

// Stage 1: z is rows x n (row stride ld), ids id_offset + column; bucket
// `seg` covers columns [seg*seg_len, min((seg+1)*seg_len, n)).  Each thread
// keeps its top-KP (a bucket's top-KP lies in the union of those lists).
template <int KP>
__global__ __launch_bounds__(TOPK_THREADS) void k_topk_stage1(const float *__restrict__ z, int64_t ld,
                                                              int64_t n, int64_t id_offset, int nseg,
                                                              int64_t seg_len, float *cand_v,
                                                              int32_t *cand_i) {
    __shared__ float s_v[TOPK_THREADS * KP];
    __shared__ int32_t s_i[TOPK_THREADS * KP];
    const int seg = blockIdx.x, row = blockIdx.y;
    const int64_t c0 = (int64_t)seg * seg_len;
    const int64_t c1 = c0 + seg_len < n ? c0 + seg_len : n;
    float l_v[KP];
    int32_t l_i[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        l_v[k] = -INFINITY;
        l_i[k] = -1;
    }
    const float *zr = z + (int64_t)row * ld;
    // scalar up to a 16-byte boundary, then four 16-byte loads in flight per
    // thread, then the scalar remainder
    int64_t a0 = c0 + ((4 - (int64_t)(((uintptr_t)(zr + c0) >> 2) & 3)) & 3);
    if (a0 > c1) a0 = c1;
    const int64_t nv = (c1 - a0) >> 2;
    const int64_t a1 = a0 + (nv << 2);
    for (int64_t c = c0 + threadIdx.x; c < a0; c += TOPK_THREADS)
        tk_insert<KP>(l_v, l_i, zr[c], (int32_t)(id_offset + c));
    const f32x4 *zv = (const f32x4 *)(zr + a0);
    constexpr int U = 4;
    for (int64_t v0 = threadIdx.x; v0 < nv; v0 += (int64_t)TOPK_THREADS * U) {
        f32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + (int64_t)u * TOPK_THREADS;
            x[u] = zv[v < nv ? v : nv - 1];   // clamped: no load is skipped
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + (int64_t)u * TOPK_THREADS;
            if (v >= nv) break;
            const int32_t id = (int32_t)(id_offset + a0 + 4 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) tk_insert<KP>(l_v, l_i, x[u][e], id + e);
        }
    }
    for (int64_t c = a1 + threadIdx.x; c < c1; c += TOPK_THREADS)
        tk_insert<KP>(l_v, l_i, zr[c], (int32_t)(id_offset + c));
    const int64_t o = ((int64_t)row * nseg + seg) * KP;
    tk_block_merge<KP>(s_v, s_i, l_v, l_i, cand_v + o, cand_i + o);
}

// Stage 2: per row, ncand candidates (the buckets' lists) -> K entries.
template <int K>
__global__ __launch_bounds__(TOPK_THREADS) void k_topk_stage2(const float *cand_v, const int32_t *cand_i,
                                                              int64_t ncand, float *out_v, int32_t *out_i) {
    __shared__ float s_v[TOPK_THREADS * K];
    __shared__ int32_t s_i[TOPK_THREADS * K];
    const int row = blockIdx.x;
    float l_v[K];
    int32_t l_i[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        l_v[k] = -INFINITY;
        l_i[k] = -1;
    }
    const int64_t base = (int64_t)row * ncand;
    for (int64_t e = threadIdx.x; e < ncand; e += TOPK_THREADS) {
        const int32_t id = cand_i[base + e];
        if (id >= 0) tk_insert<K>(l_v, l_i, cand_v[base + e], id);
    }
    tk_block_merge<K>(s_v, s_i, l_v, l_i, out_v + (int64_t)row * K, out_i + (int64_t)row * K);
}

// Buckets of a row of n logits: nbuckets buckets of ceil(n / nbuckets)
// consecutive labels (fewer when that length leaves the last ones empty);
// nbuckets == 0 -> about TOPK_WG / rows buckets (at least one), so that
// stage 1 has about TOPK_WG workgroups over all rows.
TopkBuckets topk_buckets(int64_t n, int64_t nbuckets, int64_t rows) {
    TopkBuckets b{};
    if (n <= 0) return b;
    if (nbuckets <= 0) {
        nbuckets = rows > 0 ? (TOPK_WG + rows - 1) / rows : 1;
        if (nbuckets > 65535) nbuckets = 65535;
    }
    if (nbuckets > n) nbuckets = n;
    b.seg_len = (n + nbuckets - 1) / nbuckets;
    b.nseg = (n + b.seg_len - 1) / b.seg_len;
    return b;
}

template <int KP>
static hipError_t topk_stage1_go(const float *z, int64_t ld, int rows, int64_t n, int64_t id_offset,
                                 const TopkBuckets &b, float *cand_v, int32_t *cand_i, hipStream_t st) {
    hipLaunchKernelGGL(k_topk_stage1<KP>, dim3((unsigned)b.nseg, (unsigned)rows), dim3(TOPK_THREADS), 0,
                       st, z, ld, n, id_offset, (int)b.nseg, b.seg_len, cand_v, cand_i);
    return hipGetLastError();
}

template <int K>
static hipError_t topk_stage2_go(int rows, int64_t ncand, const float *cand_v, const int32_t *cand_i,
                                 float *out_v, int32_t *out_i, hipStream_t st) {
    hipLaunchKernelGGL(k_topk_stage2<K>, dim3((unsigned)rows), dim3(TOPK_THREADS), 0, st, cand_v,
                       cand_i, ncand, out_v, out_i);
    return hipGetLastError();
}

// Group-major candidates (ngroups x ld, entry (g, row) at g*ld + row, ld a
// multiple of 4, both arrays 16-byte aligned): a workgroup takes 4*LPG rows x
// one segment of groups.  Lane l of wave w keeps a K-list for each of rows
// 4(l % LPG) .. +3 of the block over groups seg0 + GPW*w + l / LPG, + 4*GPW,
// .. (GPW = 64 / LPG groups per wave and load: a block of fewer than 256 rows
// still fills the wave).  Every load is 16 bytes, LPG lanes read consecutive
// rows of one group, and TOPK_GM_UNROLL loads are in flight per lane.  The
// 4*GPW lists of a row then merge in LDS, one thread per row.
constexpr int TOPK_GM_UNROLL = 8;

template <int K>
__global__ __launch_bounds__(256) void k_topk_group_major(const float *gv, const int32_t *gi, int64_t ld,
                                                          int rows, int lpg, int64_t ngroups,
                                                          int64_t seg_groups, int nseg, float *mid_v,
                                                          int32_t *mid_i) {
    __shared__ float s_v[1024 * K];
    __shared__ int32_t s_i[1024 * K];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gpw = 64 / lpg, sub = lane / lpg, lr = lane % lpg;
    const int64_t rb = (int64_t)blockIdx.x * (4 * lpg);
    const int64_t r4 = rb + 4 * lr;   // this lane's first row; r4 + 4 <= ld when r4 < rows
    const int seg = blockIdx.y;
    const int64_t g0 = (int64_t)seg * seg_groups;
    const int64_t g1 = g0 + seg_groups < ngroups ? g0 + seg_groups : ngroups;
    float l_v[4][K];
    int32_t l_i[4][K];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            l_v[e][k] = -INFINITY;
            l_i[e][k] = -1;
        }
    if (r4 < rows) {
        constexpr int U = TOPK_GM_UNROLL;
        const int64_t step = 4 * gpw;
        for (int64_t gb = g0 + gpw * w + sub; gb < g1; gb += step * U) {
            f32x4 xv[U];
            u32x4 xi[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t g = gb + step * u < g1 ? gb + step * u : gb;   // clamped: no load is skipped
                xv[u] = *(const f32x4 *)(gv + g * ld + r4);
                xi[u] = *(const u32x4 *)(gi + g * ld + r4);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (gb + step * u >= g1) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int32_t id = (int32_t)xi[u][e];
                    if (id >= 0 && r4 + e < rows) tk_insert<K>(l_v[e], l_i[e], xv[u][e], id);
                }
            }
        }
    }
    // list (w, sub) of block row 4*lr + e at slot ((w*64 + lane)*4 + e)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            s_v[((w * 64 + lane) * 4 + e) * K + k] = l_v[e][k];
            s_i[((w * 64 + lane) * 4 + e) * K + k] = l_i[e][k];
        }
    __syncthreads();
    const int t = threadIdx.x;
    const int64_t row = rb + t;
    if (t < 4 * lpg && row < rows) {
        float m_v[K];
        int32_t m_i[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            m_v[k] = -INFINITY;
            m_i[k] = -1;
        }
        for (int ww = 0; ww < 4; ++ww)
            for (int sb = 0; sb < gpw; ++sb) {
                const int base = ((ww * 64 + sb * lpg + (t >> 2)) * 4 + (t & 3)) * K;
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (s_i[base + k] >= 0) tk_insert<K>(m_v, m_i, s_v[base + k], s_i[base + k]);
            }
        const int64_t o = (row * nseg + seg) * K;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            mid_v[o + k] = m_v[k];
            mid_i[o + k] = m_i[k];
        }
    }
}

// Lanes per group of the group-major merge: 64 (256 rows a block), or the
// fewest power of two whose 4 rows a lane cover all rows (at least 8)
static int topk_gm_lpg(int64_t rows) {
    int lpg = 8;
    while (lpg < 64 && 4 * lpg < rows) lpg *= 2;
    return lpg;
}

// Segments of the group-major merge: about TOPK_GM_BLOCKS workgroups over
// all row blocks, at least 16 groups per wave and row
TopkGmSegs topk_gm_segments(int64_t ngroups, int64_t rows) {
    TopkGmSegs s{};
    if (ngroups <= 0 || rows <= 0) return s;
    const int lpg = topk_gm_lpg(rows);
    const int64_t rblocks = (rows + 4 * lpg - 1) / (4 * lpg);
    const int64_t want = (TOPK_GM_BLOCKS + rblocks - 1) / rblocks;
    const int64_t minseg = 16 * 4 * (64 / lpg);
    s.seg_groups = (ngroups + want - 1) / want;
    if (s.seg_groups < minseg) s.seg_groups = minseg;
    s.nseg = (ngroups + s.seg_groups - 1) / s.seg_groups;
    return s;
}

template <int K>
static hipError_t topk_gm_go(const float *gv, const int32_t *gi, int64_t ld, int rows, int64_t ngroups,
                             float *mid_v, int32_t *mid_i, float *out_v, int32_t *out_i,
                             hipStream_t st) {
    const TopkGmSegs s = topk_gm_segments(ngroups, rows);
    const int lpg = topk_gm_lpg(rows);
    hipLaunchKernelGGL(k_topk_group_major<K>,
                       dim3((unsigned)((rows + 4 * lpg - 1) / (4 * lpg)), (unsigned)s.nseg), dim3(256), 0,
                       st, gv, gi, ld, rows, lpg, ngroups, s.seg_groups, (int)s.nseg, mid_v, mid_i);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return topk_stage2_go<K>(rows, s.nseg * K, mid_v, mid_i, out_v, out_i, st);
}

hipError_t launch_topk_group_major(const float *gv, const int32_t *gi, int64_t ld, int rows,
                                   int64_t ngroups, int K, float *mid_v, int32_t *mid_i,
                                   float *out_v, int32_t *out_i, hipStream_t st) {
    if (rows <= 0 || ngroups <= 0) return hipSuccess;
    if ((ld & 3) || ld < rows || (((uintptr_t)gv | (uintptr_t)gi) & 15)) return hipErrorInvalidValue;
    if (topk_gm_segments(ngroups, rows).nseg > 65535) return hipErrorInvalidValue;
    switch (K) {
    case 1: return topk_gm_go<1>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    case 2: return topk_gm_go<2>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    case 3: return topk_gm_go<3>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    case 4: return topk_gm_go<4>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    case 5: return topk_gm_go<5>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    case 6: return topk_gm_go<6>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    case 7: return topk_gm_go<7>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    case 8: return topk_gm_go<8>(gv, gi, ld, rows, ngroups, mid_v, mid_i, out_v, out_i, st);
    }
    return hipErrorInvalidValue;
}

// Stage 2 alone, over candidate lists written elsewhere (rows x ncand)
hipError_t launch_topk_merge_cands(const float *cand_v, const int32_t *cand_i, int rows,
                                   int64_t ncand, int K, float *out_v, int32_t *out_i,
                                   hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    switch (K) {
    case 1: return topk_stage2_go<1>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 2: return topk_stage2_go<2>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 3: return topk_stage2_go<3>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 4: return topk_stage2_go<4>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 5: return topk_stage2_go<5>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 6: return topk_stage2_go<6>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 7: return topk_stage2_go<7>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 8: return topk_stage2_go<8>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_row_topk(const float *z, int64_t ld, int rows, int64_t n, int64_t id_offset,
                           int K, int KP, int64_t nbuckets, float *cand_v, int32_t *cand_i,
                           float *out_v, int32_t *out_i, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (KP == 0) KP = K;
    if (K < 1 || K > TOPK_MAX || KP < 1 || KP > K || nbuckets < 0) return hipErrorInvalidValue;
    const TopkBuckets b = topk_buckets(n, nbuckets, rows);
    if (b.nseg < 1 || b.nseg > (1 << 24)) return hipErrorInvalidValue;
    hipError_t e = hipErrorInvalidValue;
    switch (KP) {
    case 1: e = topk_stage1_go<1>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    case 2: e = topk_stage1_go<2>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    case 3: e = topk_stage1_go<3>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    case 4: e = topk_stage1_go<4>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    case 5: e = topk_stage1_go<5>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    case 6: e = topk_stage1_go<6>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    case 7: e = topk_stage1_go<7>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    case 8: e = topk_stage1_go<8>(z, ld, rows, n, id_offset, b, cand_v, cand_i, st); break;
    }
    if (e != hipSuccess) return e;
    const int64_t ncand = b.nseg * KP;
    switch (K) {
    case 1: return topk_stage2_go<1>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 2: return topk_stage2_go<2>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 3: return topk_stage2_go<3>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 4: return topk_stage2_go<4>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 5: return topk_stage2_go<5>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 6: return topk_stage2_go<6>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 7: return topk_stage2_go<7>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    case 8: return topk_stage2_go<8>(rows, ncand, cand_v, cand_i, out_v, out_i, st);
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------------ exact top-K, second step
// With the logits pass's one-maximum-per-group lists merged into each row's
// K best groups (value, id of the group's largest logit, ties to the smaller
// id), the row's exact top-K lies inside those K groups: a label of the true
// top-K has a logit at least that of every label after it, so its group's
// maximum ranks before the maxima of all groups holding only later labels,
// and fewer than K groups can rank before it.  This pass recomputes the K
// groups' logits of the row exactly as the logits pass forms them -- the
// same bf16 operands in the same feature order, the same sequence of
// 16x16x32 MFMAs from a zero accumulator, so the same fp32 values bit for
// bit -- and keeps the K best of the K*G.  Workgroup = one row, wave w = its
// w-th group; A operand: the row's X values at the group's features (every
// MFMA row the same), B operand: W_g in that order.
template <int G, int F>
__global__ __launch_bounds__(64 * TOPK_MAX) void k_topk_refine(const unsigned short *__restrict__ X, int D,
                                                               const unsigned short *__restrict__ W,
                                                               const unsigned short *__restrict__ idxp,
                                                               const unsigned char *__restrict__ perm,
                                                               int64_t L, int64_t tk_off, int K,
                                                               float *out_v, int32_t *out_i) {
    constexpr int JT = G / 16, KS = F / 32;
    __shared__ float lv[TOPK_MAX * G];
    __shared__ int32_t li[TOPK_MAX * G];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q = lane >> 4, m = lane & 15;
    // the w-th group of the row (wave-uniform); -1: fewer than K candidates
    const int32_t cid = w < K ? out_i[(int64_t)b * K + w] : -1;
    if (cid >= 0) {
        const int64_t g = ((int64_t)cid - tk_off) / G;
        const unsigned short *xr = X + (int64_t)b * D;
        bf16x8 A[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            unsigned short e8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) e8[e] = xr[idxp[g * F + 32 * s + 8 * q + e]];
            A[s] = __builtin_bit_cast(bf16x8, e8);
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const unsigned short *wr = W + (g * G + 16 * jt + m) * (int64_t)F;
            f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                unsigned short e8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) e8[e] = wr[perm[g * F + 32 * s + 8 * q + e]];
                acc = mfma32(A[s], __builtin_bit_cast(bf16x8, e8), acc);
            }
            if (q == 0) {   // lanes 0..15 hold label 16jt + m (every row is row b)
                const int64_t t = g * G + 16 * jt + m;
                lv[w * G + 16 * jt + m] = t < L ? acc[0] : -INFINITY;
                li[w * G + 16 * jt + m] = t < L ? (int32_t)(tk_off + t) : -1;
            }
        }
    } else if (w < TOPK_MAX) {
        for (int j = lane; j < G; j += 64) {
            lv[w * G + j] = -INFINITY;
            li[w * G + j] = -1;
        }
    }
    __syncthreads();
    if (w != 0) return;
    // wave 0: K rounds of an arg-max over the K * G entries (ties: smaller id)
    const int n = K * G;
    for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int32_t bi = -1;
        int bp = -1;
        for (int p = lane; p < n; p += 64) {
            const int32_t id = li[p];
            if (id >= 0 && (bi < 0 || tk_before(lv[p], id, bv, bi))) {
                bv = lv[p];
                bi = id;
                bp = p;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int32_t oi = __shfl_xor(bi, off, 64);
            const int op = __shfl_xor(bp, off, 64);
            if (oi >= 0 && (bi < 0 || tk_before(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
                bp = op;
            }
        }
        if (lane == 0) {
            out_v[(int64_t)b * K + k] = bi >= 0 ? bv : -INFINITY;
            out_i[(int64_t)b * K + k] = bi;
            if (bp >= 0) li[bp] = -1;   // taken
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
    }
}

template <int G, int F>
static hipError_t topk_refine_go(const unsigned short *X, int B, int D, const unsigned short *W,
                                 const unsigned short *idxp, const unsigned char *perm, int64_t L,
                                 int64_t tk_off, int K, float *out_v, int32_t *out_i, hipStream_t st) {
    hipLaunchKernelGGL((k_topk_refine<G, F>), dim3((unsigned)B), dim3(64 * TOPK_MAX), 0, st, X, D, W, idxp,
                       perm, L, tk_off, K, out_v, out_i);
    return hipGetLastError();
}

hipError_t launch_topk_refine(const unsigned short *X, int B, int D, const unsigned short *W,
                              const unsigned short *idxp, const unsigned char *perm, int G, int F,
                              int64_t L, int64_t tk_off, int K, float *out_v, int32_t *out_i,
                              hipStream_t st) {
    if (B <= 0) return hipSuccess;
    if (K < 1 || K > TOPK_MAX) return hipErrorInvalidValue;
    switch (G * 1000 + F) {
    case 16032: return topk_refine_go<16, 32>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 16064: return topk_refine_go<16, 64>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 16128: return topk_refine_go<16, 128>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 32032: return topk_refine_go<32, 32>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 32064: return topk_refine_go<32, 64>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 32128: return topk_refine_go<32, 128>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 64032: return topk_refine_go<64, 32>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 64064: return topk_refine_go<64, 64>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    case 64128: return topk_refine_go<64, 128>(X, B, D, W, idxp, perm, L, tk_off, K, out_v, out_i, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace haste
