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
// whose label is a positive.  Built deterministically: counts, one exclusive
// scan, then each positive finds its rank among the positives of its group
// ordered by (b, j) -- no atomic append, so the lists are reproducible.
__device__ __forceinline__ int row_of(const int32_t *row_ptr, int B, int k) {
    int lo = 0, hi = B;  // row_ptr[lo] <= k < row_ptr[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (row_ptr[mid] <= k) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ void k_gpos_count(const int32_t *row_ptr, const int32_t *labels, int nnz,
                             int64_t off, int64_t L, int G, int32_t *cnt) {
    int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= nnz) return;
    int64_t t = (int64_t)labels[k] - off;
    if (t >= 0 && t < L) atomicAdd(&cnt[t / G], 1);
}

// Single-workgroup exclusive scan of cnt[0..n) into ptr[0..n].
__global__ __launch_bounds__(1024) void k_scan(const int32_t *cnt, int32_t *ptr, int64_t n) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int64_t per = (n + 1023) / 1024;
    const int64_t a = tid * per, b = a + per < n ? a + per : n;
    int32_t s = 0;
    for (int64_t i = a; i < b; ++i) s += cnt[i];
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t run = part[tid] - s;  // exclusive prefix of this thread's segment
    for (int64_t i = a; i < b; ++i) {
        ptr[i] = run;
        run += cnt[i];
    }
    if (tid == 1023) ptr[n] = part[1023];
}

__global__ __launch_bounds__(256) void k_gpos_fill(const int32_t *row_ptr, const int32_t *labels,
                                                   int nnz, int B, int64_t off, int64_t L,
                                                   int G, const int32_t *ptr, int32_t *ent) {
    __shared__ long long keys[2048];
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    long long mykey = -1;
    int myg = 0, myb = 0, myj = 0;
    if (k < nnz) {
        int64_t t = (int64_t)labels[k] - off;
        if (t >= 0 && t < L) {
            myb = row_of(row_ptr, B, k);
            myg = (int)(t / G);
            myj = (int)(t % G);
            mykey = ((long long)myg * B + myb) * G + myj;
        }
    }
    int rank = 0;
    for (int c0 = 0; c0 < nnz; c0 += 2048) {
        __syncthreads();
        for (int i = threadIdx.x; i < 2048; i += blockDim.x) {
            int kk = c0 + i;
            long long key = -1;
            if (kk < nnz) {
                int64_t t = (int64_t)labels[kk] - off;
                if (t >= 0 && t < L)
                    key = ((long long)(t / G) * B + row_of(row_ptr, B, kk)) * G + (t % G);
            }
            keys[i] = key;
        }
        __syncthreads();
        if (mykey >= 0) {
            int lim = nnz - c0 < 2048 ? nnz - c0 : 2048;
            long long gbase = (long long)myg * B * G;
            for (int i = 0; i < lim; ++i) {
                long long kv = keys[i];
                rank += (kv >= gbase && kv < mykey) ? 1 : 0;
            }
        }
    }
    if (mykey >= 0) ent[ptr[myg] + rank] = myb * G + myj;
}

hipError_t launch_group_positives(const int32_t *row_ptr, const int32_t *labels, int nnz,
                                  int B, int64_t off, int64_t L, int G, int64_t Ng,
                                  int32_t *cnt, int32_t *grp_ptr, int32_t *ent,
                                  hipStream_t st) {
    hipError_t e = launch_fill_u32(cnt, 0u, (size_t)Ng, st);
    if (e != hipSuccess) return e;
    if (nnz > 0) {
        hipLaunchKernelGGL(k_gpos_count, dim3((nnz + 255) / 256), dim3(256), 0, st, row_ptr,
                           labels, nnz, off, L, G, cnt);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, cnt, grp_ptr, Ng);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (nnz > 0) {
        hipLaunchKernelGGL(k_gpos_fill, dim3((nnz + 255) / 256), dim3(256), 0, st, row_ptr,
                           labels, nnz, B, off, L, G, grp_ptr, ent);
        e = hipGetLastError();
    }
    return e;
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
// Groups per run = 4 waves * RW.  BC = rows per chunk (64 or 32).
template <int G, int F, int RW, int BC, int MODE>
__global__ __launch_bounds__(256, 1) void k_tail_t1(TailArgs a, int store_z, int do_loss) {
    constexpr int JT = G / 16, KS = F / 32, FT = F / 16, BT = BC / 16, KB = BC / 32;
    constexpr int BCP = BC + 8;  // padded LDS row (shorts); 16-byte aligned rows
    constexpr bool DO_Z = (MODE != T1_DW_MEM);
    constexpr bool DO_DW = (MODE != T1_FWD);
    extern __shared__ __attribute__((aligned(16))) unsigned short tile[];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q = lane >> 4, m = lane & 15;
    const int nch = a.Bp / BC;
    const int64_t n_runs = (a.Ng + 4 * RW - 1) / (4 * RW);
    float lsum = 0.f;

    for (int64_t run = blockIdx.x; run < n_runs; run += gridDim.x) {
        const int64_t gw = run * (4 * RW) + (int64_t)w * RW;
        bf16x8 wreg[RW][KS][JT];
        unsigned zrow[RW][KS];        // tr-gather rows: lo16 = h 0, hi16 = h 1
        unsigned frow[RW][(FT + 1) / 2];  // dW rows, two f-tiles per word
        f32x4 dwacc[RW][FT][JT];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int64_t g = gw + r;
            const bool ok = g < a.Ng;
            const int32_t *ix = a.idx + (ok ? g : 0) * (int64_t)F;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                unsigned lo = ok ? (unsigned)ix[32 * s + 8 * q + (m >> 2)] : 0u;
                unsigned hi = ok ? (unsigned)ix[32 * s + 8 * q + 4 + (m >> 2)] : 0u;
                zrow[r][s] = lo | (hi << 16);
                if (DO_Z) {
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        if (ok) {
                            const unsigned short *wp =
                                a.W + ((g * G + 16 * jt + m) * (int64_t)F + 32 * s + 8 * q);
                            wreg[r][s][jt] = *(const bf16x8 *)wp;
                        } else {
                            wreg[r][s][jt] = (bf16x8){};
                        }
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < (FT + 1) / 2; ++p) {
                unsigned lo = ok ? (unsigned)ix[16 * (2 * p) + m] : 0u;
                unsigned hi = (ok && 2 * p + 1 < FT) ? (unsigned)ix[16 * (2 * p + 1) + m] : 0u;
                frow[r][p] = lo | (hi << 16);
            }
#pragma unroll
            for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) dwacc[r][ft][jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        for (int ch = 0; ch < nch; ++ch) {
            __syncthreads();
            {   // stage XT[:, ch*BC .. +BC) in LDS
                constexpr int SEG = BC / 8;
                const unsigned short *src = a.XT + (int64_t)ch * BC;
                for (int i = threadIdx.x; i < a.D * SEG; i += 256) {
                    const int d = i / SEG, sg = i % SEG;
                    u32x4 v = *(const u32x4 *)(src + (int64_t)d * a.Bp + sg * 8);
                    *(u32x4 *)(tile + d * BCP + sg * 8) = v;
                }
            }
            __syncthreads();
            const int r0 = ch * BC;

#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int64_t g = gw + r;
                if (g >= a.Ng) continue;  // wave-uniform
                uint64_t ymask = 0;
                if (MODE != T1_DW_MEM && (do_loss || DO_DW))
                    ymask = pos_mask_rows4<BT, JT>(a.grp_ptr, a.grp_ent, g, G, r0, q, m);
                // 32 rows at a time: Z for b-tiles 2kb, 2kb+1 -> epilogue -> dW
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
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
                                const int col = 16 * (2 * kb + h2) + 4 * (m & 3);
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
                    // ---- epilogue: lane owns (row r0+16bt+4q+i, slot 16jt+m)
                    unsigned dzp[2][JT][2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            const int bt = 2 * kb + h2;
                            float dzv[4];
                            const int64_t t = g * G + 16 * jt + m;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int row = r0 + 16 * bt + 4 * q + i;
                                const bool live = row < a.B && t < a.L;
                                const float z = zacc[h2][jt][i];
                                float dz = 0.f;
                                if (MODE == T1_DW_MEM) {
                                    if (live) dz = bf16_to_f32(a.dZ[(int64_t)row * a.L + t]);
                                } else {
                                    const float y =
                                        (float)((ymask >> ((bt * JT + jt) * 4 + i)) & 1ull);
                                    if (do_loss || DO_DW) {
                                        BceOut o = bce_both(z, y, a.s);
                                        if (live) {
                                            dz = o.dz;
                                            if (do_loss) lsum += o.loss;
                                        }
                                    }
                                    if (MODE == T1_FWD && store_z && live)
                                        a.Z[(int64_t)row * a.L + t] = f32_to_bf16(z);
                                }
                                dzv[i] = dz;
                            }
                            dzp[h2][jt][0] = pack_bf16x2(dzv[0], dzv[1]);
                            dzp[h2][jt][1] = pack_bf16x2(dzv[2], dzv[3]);
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
                            const unsigned short *p = tile + row * BCP + 32 * kb + 4 * q;
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

static int t1_bc(int D) { return D * (64 + 8) * 2 <= 160 * 1024 ? 64 : 32; }

// Dynamic LDS above the default per-kernel limit must be allowed per kernel.
static void allow_lds(const void *fn, size_t bytes) {
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int G, int F, int RW, int BC>
static hipError_t t1_launch_bc(int mode, const TailArgs &a, bool store_z, bool do_loss,
                               hipStream_t st) {
    const size_t lds = (size_t)a.D * (BC + 8) * 2;
    const int64_t n_runs = (a.Ng + 4 * RW - 1) / (4 * RW);
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t grid = n_runs < ncu ? n_runs : ncu;
    if (grid <= 0) return hipSuccess;
    switch (mode) {
    case T1_FWD:
        allow_lds((const void *)k_tail_t1<G, F, RW, BC, T1_FWD>, lds);
        hipLaunchKernelGGL((k_tail_t1<G, F, RW, BC, T1_FWD>), dim3((unsigned)grid), dim3(256),
                           lds, st, a, (int)store_z, (int)do_loss);
        break;
    case T1_DW_BCE:
        allow_lds((const void *)k_tail_t1<G, F, RW, BC, T1_DW_BCE>, lds);
        hipLaunchKernelGGL((k_tail_t1<G, F, RW, BC, T1_DW_BCE>), dim3((unsigned)grid), dim3(256),
                           lds, st, a, 0, (int)do_loss);
        break;
    default:
        allow_lds((const void *)k_tail_t1<G, F, RW, BC, T1_DW_MEM>, lds);
        hipLaunchKernelGGL((k_tail_t1<G, F, RW, BC, T1_DW_MEM>), dim3((unsigned)grid), dim3(256),
                           lds, st, a, 0, 0);
        break;
    }
    return hipGetLastError();
}

template <int G, int F, int RW>
static hipError_t t1_launch(int mode, const TailArgs &a, bool store_z, bool do_loss,
                            hipStream_t st) {
    if (t1_bc(a.D) == 64) return t1_launch_bc<G, F, RW, 64>(mode, a, store_z, do_loss, st);
    return t1_launch_bc<G, F, RW, 32>(mode, a, store_z, do_loss, st);
}

hipError_t launch_tail_t1(int mode, int G, const TailArgs &a, bool store_z, bool do_loss,
                          hipStream_t st) {
#define T1CASE(GG, FF, RR) \
    if (G == GG && a.F == FF) return t1_launch<GG, FF, RR>(mode, a, store_z, do_loss, st);
    T1CASE(16, 32, 8)
    T1CASE(16, 64, 6)
    T1CASE(16, 128, 4)
    T1CASE(32, 32, 6)
    T1CASE(32, 64, 3)
    T1CASE(32, 128, 2)
    T1CASE(64, 32, 3)
    T1CASE(64, 64, 1)
    T1CASE(64, 128, 1)
#undef T1CASE
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------- T2
// Workgroup = (row chunk of BC2 rows) x (range of groups).  NTW = d-tiles of
// 16 features owned by each of the 4 waves for the dX accumulator.
template <int G, int BC2, int NTW>
__global__ __launch_bounds__(256, 1) void k_tail_t2(TailArgs a, int dz_mem, int n_granges) {
    constexpr int JT = G / 16, BT = BC2 / 16, BCP = BC2 + 8;
    constexpr int NDP = 4 * NTW * 16;              // inverse-map entries
    const int F = a.F, KS = F / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned short smem[];
    unsigned short *tile = smem;                                  // D x BCP
    unsigned short *wts0 = tile + (size_t)a.D * BCP;              // [2][F][G]
    short *inv0 = (short *)(wts0 + 2 * F * G);                    // [2][NDP]
    u32x2 *exch0 = (u32x2 *)(inv0 + 2 * NDP);                      // [2][BT][JT][64]

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q = lane >> 4, m = lane & 15;
    const int gr = blockIdx.x % n_granges, bch = blockIdx.x / n_granges;
    const int64_t gA = (int64_t)gr * a.Ng / n_granges, gB = (int64_t)(gr + 1) * a.Ng / n_granges;
    const int r0 = bch * BC2;

    {   // stage the chunk, reset both inverse maps
        constexpr int SEG = BC2 / 8;
        const unsigned short *src = a.XT + r0;
        for (int i = threadIdx.x; i < a.D * SEG; i += 256) {
            const int d = i / SEG, sg = i % SEG;
            *(u32x4 *)(tile + d * BCP + sg * 8) = *(const u32x4 *)(src + (int64_t)d * a.Bp + sg * 8);
        }
        for (int i = threadIdx.x; i < 2 * NDP; i += 256) inv0[i] = (short)-1;
    }
    f32x4 acc[BT][NTW];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[bt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    for (int64_t g = gA; g < gB; ++g) {
        const int p = (int)((g - gA) & 1);
        unsigned short *wts = wts0 + p * F * G;
        short *inv = inv0 + p * NDP;
        u32x2 *exch = exch0 + p * (BT * JT * 64);
        const int32_t *ix = a.idx + g * (int64_t)F;

        // (a) W_g^T into LDS ([f][j]) via 4x4 register transposes; inverse map
        {
            const int nq = (G / 4) * (F / 4);
            for (int u = threadIdx.x; u < nq; u += 256) {
                const int ja = u % (G / 4), fc = u / (G / 4);
                u32x2 rw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rw[e] = *(const u32x2 *)(a.W + (g * G + 4 * ja + e) * (int64_t)F + 4 * fc);
                // rw[e] holds W[j=4ja+e][f=4fc..4fc+3]; emit out[k] = W[4ja..+3][4fc+k]
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int word = k >> 1, sh = (k & 1) * 16;
                    unsigned v0 = (rw[0][word] >> sh) & 0xffffu, v1 = (rw[1][word] >> sh) & 0xffffu;
                    unsigned v2 = (rw[2][word] >> sh) & 0xffffu, v3 = (rw[3][word] >> sh) & 0xffffu;
                    u32x2 o = {v0 | (v1 << 16), v2 | (v3 << 16)};
                    *(u32x2 *)(wts + (4 * fc + k) * G + 4 * ja) = o;
                }
            }
            for (int f = threadIdx.x; f < F; f += 256) inv[ix[f]] = (short)f;
        }
        __syncthreads();

        // (b) recompute Z^T for the chunk, BCE -> dz, publish dz as MFMA A operands
        for (int tl = w; tl < JT * BT; tl += 4) {
            const int jt = tl / BT, bt = tl % BT;
            uint64_t ymask = 0;
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            if (!dz_mem) {
                const unsigned short *wrow = a.W + (g * G + 16 * jt + m) * (int64_t)F + 8 * q;
                const int col = 16 * bt + 4 * (m & 3);
                for (int s = 0; s < KS; ++s) {
                    bf16x8 A = *(const bf16x8 *)(wrow + 32 * s);
                    const int rlo = ix[32 * s + 8 * q + (m >> 2)];
                    const int rhi = ix[32 * s + 8 * q + 4 + (m >> 2)];
                    i16x4 b0 = lds_read_tr(tile + rlo * BCP + col);
                    i16x4 b1 = lds_read_tr(tile + rhi * BCP + col);
                    bf16x8 Bv = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
                    z = mfma32(A, Bv, z);
                }
                ymask = pos_mask_slots4<BT, JT>(a.grp_ptr, a.grp_ent, g, G, r0, q, m);
            }
            // lane owns slots j = 16jt+4q+i of row r0+16bt+m
            const int row = r0 + 16 * bt + m;
            float dzv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t t = g * G + 16 * jt + 4 * q + i;
                const bool live = row < a.B && t < a.L;
                float dz = 0.f;
                if (live) {
                    if (dz_mem) {
                        dz = bf16_to_f32(a.dZ[(int64_t)row * a.L + t]);
                    } else {
                        const float y = (float)((ymask >> ((bt * JT + jt) * 4 + i)) & 1ull);
                        dz = bce_dz(z[i], y, a.s);
                    }
                }
                dzv[i] = dz;
            }
            exch[(bt * JT + jt) * 64 + lane] = (u32x2){pack_bf16x2(dzv[0], dzv[1]),
                                                        pack_bf16x2(dzv[2], dzv[3])};
        }
        __syncthreads();

        // (c) dX_chunk[:, wave's d-range] += dz (BC2 x G) * W~_g (G x d-range)
        const int dbase = w * NTW * 16;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            i16x4 Am[BT];
#pragma unroll
            for (int bt = 0; bt < BT; ++bt)
                Am[bt] = __builtin_bit_cast(i16x4, exch[(bt * JT + jt) * 64 + lane]);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int d = dbase + 16 * nt + m;
                const int f = inv[d];
                i16x4 Bv = {0, 0, 0, 0};
                if (f >= 0) Bv = *(const i16x4 *)(wts + f * G + 16 * jt + 4 * q);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) acc[bt][nt] = mfma16(Am[bt], Bv, acc[bt][nt]);
            }
        }
        // reset this wave's slice of the inverse map (only this wave reads it)
        for (int i = lane; i < NTW * 16; i += 64) inv[dbase + i] = (short)-1;
    }

    // flush: lane owns rows r0+16bt+4q+i, feature dbase+16nt+m
    const int dbase = w * NTW * 16;
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int d = dbase + 16 * nt + m;
            if (d >= a.D) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = r0 + 16 * bt + 4 * q + i;
                if (row < a.B) atomicAdd(a.dX + (int64_t)row * a.D + d, acc[bt][nt][i]);
            }
        }
}

static size_t t2_lds(int D, int F, int G, int BC2, int NTW) {
    const int BT = BC2 / 16, JT = G / 16, NDP = 4 * NTW * 16;
    return (size_t)D * (BC2 + 8) * 2 + 2 * (size_t)F * G * 2 + 2 * (size_t)NDP * 2 +
           2 * (size_t)BT * JT * 64 * 8;
}

template <int G, int BC2, int NTW>
static hipError_t t2_go(bool dz_mem, const TailArgs &a, hipStream_t st) {
    const size_t lds = t2_lds(a.D, a.F, G, BC2, NTW);
    const int nbch = a.Bp / BC2;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    // group ranges: a multiple of 8 (so the b-chunks of one range share an
    // XCD and its L2 for W_g), about one workgroup per CU overall
    int64_t ngr = (ncu + nbch - 1) / nbch;
    ngr = (ngr + 7) / 8 * 8;
    if (ngr > a.Ng) ngr = a.Ng;
    if (ngr < 1) return hipSuccess;
    allow_lds((const void *)k_tail_t2<G, BC2, NTW>, lds);
    hipLaunchKernelGGL((k_tail_t2<G, BC2, NTW>), dim3((unsigned)(ngr * nbch)), dim3(256), lds,
                       st, a, (int)dz_mem, (int)ngr);
    return hipGetLastError();
}

template <int G, int NTW>
static hipError_t t2_pick_bc(bool dz_mem, const TailArgs &a, hipStream_t st) {
    if (t2_lds(a.D, a.F, G, 64, NTW) <= 160 * 1024) return t2_go<G, 64, NTW>(dz_mem, a, st);
    return t2_go<G, 32, NTW>(dz_mem, a, st);
}

template <int G>
static hipError_t t2_pick(bool dz_mem, const TailArgs &a, hipStream_t st) {
    const int nd = (a.D + 15) / 16, need = (nd + 3) / 4;
    if (need <= 2) return t2_pick_bc<G, 2>(dz_mem, a, st);
    if (need <= 4) return t2_pick_bc<G, 4>(dz_mem, a, st);
    if (need <= 8) return t2_pick_bc<G, 8>(dz_mem, a, st);
    if (need <= 12) return t2_pick_bc<G, 12>(dz_mem, a, st);
    if (need <= 16) return t2_go<G, 32, 16>(dz_mem, a, st);
    return t2_go<G, 32, 24>(dz_mem, a, st);
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
    if (D < F || D > 1536) return false;
    // T2 needs the chunk + buffers in LDS with BC2 = 32 at least
    const int nd = (D + 15) / 16, need = (nd + 3) / 4;
    int ntw = need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 12 ? 12 : need <= 16 ? 16 : 24;
    if (t2_lds(D, F, G, 32, ntw) > 160 * 1024) return false;
    if ((size_t)D * (32 + 8) * 2 > 160 * 1024) return false;
    return true;
}

}  // namespace haste
