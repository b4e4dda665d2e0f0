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
                    if (g.Z32) g.Z32[o] = v;
                } else if (EPI == EPI_STORE16) {
                    g.C16[o] = f32_to_bf16(v);
                } else {
                    atomicAdd(g.C32 + o, v);
                }
            }
        }
    if (EPI == EPI_BCE && g.loss) {
        __shared__ float s_loss[4];
        block_loss_add(lsum, s_loss, g.loss);
    }
}

// ------------------------------------------------------------ pipelined GEMM
// Same contractions and epilogues as k_gemm, for shapes whose M, N, K and
// split length are multiples of 8 (every head of the workloads): M tile of
// TMT = 64 or 128 rows, N tile 128, K step 64.  Operand tiles go from global
// memory straight into LDS (16 bytes a lane, 1 KB a wave instruction) through
// a ring of GEMM_NS stages, so the copies of the next GEMM_NS - 1 steps are in
// flight while one step is computed.  Each stage is an LDS array of its own
// and the K loop is unrolled by GEMM_NS, so every access names its stage and
// the compiler sees that a read of one stage does not need the copies into
// the others.  Addresses are clamped into the matrix (nothing is skipped);
// K slots past the split's end are zeroed in the operand registers.
constexpr int TK2 = 64;
constexpr int GEMM_NS = 3;

// LDS layouts (no padding: the copies write 1 KB contiguous).
// K-major tile, ROWS rows x 64 K (128 B a row): the 16-byte segment s of row r
// sits at s ^ ((r >> 1) & 7), so the 16 consecutive rows of an operand read
// fall on 16 different 16-byte bank groups.
__device__ __forceinline__ int kmaj_seg(int r, int s) { return s ^ ((r >> 1) & 7); }
// M-major tile, 64 K rows x ROWS (2 ROWS bytes a row): the 32-byte chunk of a
// K row is permuted by bits of the row, so that the 16 K rows a transposing
// read covers (8q + j, q and j in 0..3) spread over all chunks, two apiece.
template <int ROWS>
__device__ __forceinline__ int mmaj_seg(int k, int s) {
    if (ROWS == 128) return s ^ (2 * ((k & 3) | (((k >> 3) & 1) << 2)));
    return s ^ (2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1)));
}

// Copies of one ROWS x 64 operand tile of step k0 into S: ROWS/32 one-KB
// blocks per wave.
template <bool KMAJ, int ROWS>
__device__ __forceinline__ void copy_tile3(const unsigned short *P, int ld, int r0, int rows, int k0,
                                           int K, unsigned short *S, int w, int lane) {
    constexpr int NC = ROWS / 32;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int blk = w * NC + c;
        const unsigned short *src;
        if (KMAJ) {   // 8 rows of 128 B per block
            const int row = 8 * blk + (lane >> 3);
            const int sg = kmaj_seg(row, lane & 7);
            const int gr = r0 + row < rows ? r0 + row : rows - 1;
            const int gk = k0 + 8 * sg <= K - 8 ? k0 + 8 * sg : K - 8;
            src = P + (int64_t)gr * ld + gk;
        } else {      // ROWS/8 lanes per K row
            constexpr int LPR = ROWS / 8;
            const int kr = blk * (64 / LPR) + lane / LPR;
            const int sg = mmaj_seg<ROWS>(kr, lane % LPR);
            const int gk = k0 + kr < K ? k0 + kr : K - 1;
            const int gc = r0 + 8 * sg <= rows - 8 ? r0 + 8 * sg : rows - 8;
            src = P + (int64_t)gk * ld + gc;
        }
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(S + blk * 512), 16,
                                         0, 0);
    }
}

// operand of the 16 rows from r, K slots 32ks + 8q .. +7
template <bool KMAJ, int ROWS>
__device__ __forceinline__ bf16x8 read_operand3(const unsigned short *S, int r, int ks, int q, int m) {
    if (KMAJ) {
        const int row = r + m;
        return *(const bf16x8 *)(S + row * TK2 + 8 * kmaj_seg(row, 4 * ks + q));
    }
    const int col = r + 4 * (m & 3), sg = col >> 3, within = col & 7;
    const int k0 = 32 * ks + 8 * q + (m >> 2);
    i16x4 a0 = lds_read_tr(S + k0 * ROWS + 8 * mmaj_seg<ROWS>(k0, sg) + within);
    i16x4 a1 = lds_read_tr(S + (k0 + 4) * ROWS + 8 * mmaj_seg<ROWS>(k0 + 4, sg) + within);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// s_waitcnt with only the vector-memory count constrained
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool A_KMAJ, bool B_KMAJ, int EPI, int TMT>
__global__ __launch_bounds__(256, 2) void k_gemm2(GemmArgs g) {
    constexpr int MI = TMT / 32;      // 16-row MFMA tiles per wave (waves: 2 along M, 2 along N)
    constexpr int ASZ = TMT * TK2, BSZ = TN * TK2;   // shorts
    constexpr int LPS = TMT / 32 + TN / 32;          // copies per wave and step
    __shared__ __attribute__((aligned(1024))) unsigned short st0[ASZ + BSZ];
    __shared__ __attribute__((aligned(1024))) unsigned short st1[ASZ + BSZ];
    __shared__ __attribute__((aligned(1024))) unsigned short st2[ASZ + BSZ];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q = lane >> 4, m = lane & 15;
    const int wm = (w >> 1) * (TMT / 2), wn = (w & 1) * 64;
    // Workgroups go round-robin over the 8 XCDs.  Tile t = (split, n, m),
    // m fastest, goes to workgroup slot (t mod T/8)*8 + t/(T/8), so that the
    // M tiles sharing one B tile (and split) run on one XCD and its L2.
    const int gx = gridDim.x, gy = gridDim.y;
    const int T = gx * gy * gridDim.z;
    const int L = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const int t = (T & 7) == 0 ? (L & 7) * (T >> 3) + (L >> 3) : L;
    const int by = t % gy, bx = (t / gy) % gx, bz = t / (gx * gy);
    const int m0 = by * TMT, n0 = bx * TN;
    const int kbeg = bz * g.k_split;
    int kend = kbeg + g.k_split;
    if (kend > g.K) kend = g.K;
    const int nk = (kend - kbeg + TK2 - 1) / TK2;
    // BCE: the positives of the tile (TMT rows x 4 bitmap words) go to LDS
    // first, so the epilogue reads them there instead of once per logit.
    // From the row CSR: a thread per row builds the row's four words (no two
    // threads share a word); the K loop's barriers publish them.
    __shared__ __attribute__((aligned(16))) uint32_t bm_tile[EPI == EPI_BCE ? TMT * 4 : 1];
    const bool has_pos = g.bitmap || g.pos_ptr;
    if (EPI == EPI_BCE && g.pos_ptr) {
        for (int r = threadIdx.x; r < TMT; r += 256) {
            const int row = m0 + r;
            uint32_t w0 = 0u, w1 = 0u, w2 = 0u, w3 = 0u;
            if (row < g.M) {
                const int e1 = min(g.pos_ptr[row + 1], g.pos_nnz);
                for (int e = max(g.pos_ptr[row], 0); e < e1; ++e) {
                    const int64_t c = (int64_t)g.pos_lab[e] - g.pos_off - n0;
                    if (c < 0 || c >= TN || n0 + c >= g.N) continue;
                    const uint32_t bit = 1u << (c & 31);
                    const int wd = (int)(c >> 5);
                    w0 |= wd == 0 ? bit : 0u;
                    w1 |= wd == 1 ? bit : 0u;
                    w2 |= wd == 2 ? bit : 0u;
                    w3 |= wd == 3 ? bit : 0u;
                }
            }
            *(u32x4 *)(bm_tile + 4 * r) = (u32x4){w0, w1, w2, w3};
        }
    } else if (EPI == EPI_BCE) {
        for (int i = threadIdx.x; i < TMT * 4; i += 256) {
            const int row = m0 + (i >> 2), wd = (n0 >> 5) + (i & 3);
            bm_tile[i] = g.bitmap && row < g.M && wd < g.bm_words
                             ? g.bitmap[(int64_t)row * g.bm_words + wd] : 0u;
        }
    }

    f32x4 acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int kt, unsigned short *S) {
        const int k0 = kbeg + kt * TK2;
        copy_tile3<A_KMAJ, TMT>(g.A, g.lda, m0, g.M, k0, g.K, S, w, lane);
        copy_tile3<B_KMAJ, TN>(g.Bm, g.ldb, n0, g.N, k0, g.K, S + ASZ, w, lane);
    };
    auto compute = [&](int kt, const unsigned short *S) {
        const int k0 = kbeg + kt * TK2;
        const bool tail = k0 + TK2 > kend;   // wave-uniform
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 av[MI], bv[4];
#pragma unroll
            for (int i = 0; i < MI; ++i) av[i] = read_operand3<A_KMAJ, TMT>(S, wm + 16 * i, ks, q, m);
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = read_operand3<B_KMAJ, TN>(S + ASZ, wn + 16 * j, ks, q, m);
            if (tail && k0 + 32 * ks + 8 * q >= kend) {
                // K slots past the split: zero on both sides
#pragma unroll
                for (int i = 0; i < MI; ++i) av[i] = (bf16x8){};
#pragma unroll
                for (int j = 0; j < 4; ++j) bv[j] = (bf16x8){};
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
        }
    };
    // Step kt: wait for this wave's copies of step kt (those of step kt+1 stay
    // in flight), then a barrier: everyone's copies have landed, and every
    // wave is done with step kt-1, whose stage the copies of step kt+2 then
    // overwrite.  No __syncthreads: its fence would wait for every copy in
    // flight.  The barrier waits for this wave's LDS reads instead: the
    // compiler may move the MFMAs that consume the reads of step kt-1 below
    // the barrier, and its own wait for those reads with them, and a read
    // still in flight there would race with the copies that overwrite its
    // stage right after the barrier.  The loop has no exit but its end (the
    // steps run up to a multiple of GEMM_NS; those past the split's end see
    // zeroed operands and add nothing) and copies are issued unconditionally (clamped
    // addresses), so the compiler's own count of copies in flight is the same
    // on every path and it does not wait for the other stages; an exit in the
    // middle costs a full wait there and twice the registers.  All copies are
    // drained after the loop.
    auto sync = [&]() {
        wait_vm<LPS>();
        lds_barrier();
    };
    issue(0, st0);
    issue(1, st1);
    for (int kt = 0; kt < nk; kt += GEMM_NS) {
        sync();
        issue(kt + 2, st2);
        compute(kt, st0);
        sync();
        issue(kt + 3, st0);
        compute(kt + 1, st1);
        sync();
        issue(kt + 4, st1);
        compute(kt + 2, st2);
    }
    wait_vm<0>();

    // epilogue: lane owns C[m0+wm+16i+4q+e][n0+wn+16j+m].  BCE with the
    // hardware exp / rcp / log: sigmoid(z) from e = exp(-|z|), and
    // softplus(z) = max(z, 0) + log(1 + e), the logs taken of products of
    // sixteen (1 + e) factors (each in [1, 2]), kept as product - 1.  Whole
    // tiles take a path with no per-element branches.
    float lsum = 0.f, lin = 0.f, prod = 0.f;
    uint32_t bw[MI][4][2];   // bitmap words of the lane's rows: columns wn .. wn+31, wn+32 .. wn+63
    if (EPI == EPI_BCE) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    bw[i][e][h] = bm_tile[(wm + 16 * i + 4 * q + e) * 4 + (wn >> 5) + h];
    }
    const bool whole = m0 + TMT <= g.M && n0 + TN <= g.N;
    if (EPI == EPI_BCE && whole && has_pos && g.dZout && !g.Zout && !g.Z32) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn + 16 * j + m;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = m0 + wm + 16 * i + 4 * q + e;
                    const float v = acc[i][j][e];
                    const float y = (float)((bw[i][e][j >> 1] >> ((16 * j + m) & 31)) & 1u);
                    const float ex = fast_exp_neg_abs(v);
                    float den;
                    const float sg = fast_sigmoid(v, ex, den);
                    prod = prod1p(prod, ex);
                    lin += fmaxf(v, 0.f) - y * v;
                    g.dZout[(int64_t)row * g.N + col] = f32_to_bf16(g.s * (sg - y));
                }
            }
            lsum += log1p_pos(prod);
            prod = 0.f;
        }
    } else if (EPI != EPI_BCE && whole) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn + 16 * j + m;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t o = (int64_t)(m0 + wm + 16 * i + 4 * q + e) * g.N + col;
                    if (EPI == EPI_STORE16) g.C16[o] = f32_to_bf16(acc[i][j][e]);
                    else atomicAdd(g.C32 + o, acc[i][j][e]);
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
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
                        if (has_pos) {
                            const float y = (float)((bw[i][e][j >> 1] >> ((16 * j + m) & 31)) & 1u);
                            const float ex = fast_exp_neg_abs(v);
                            float den;
                            const float sg = fast_sigmoid(v, ex, den);
                            prod = prod1p(prod, ex);
                            lin += fmaxf(v, 0.f) - y * v;
                            if (g.dZout) g.dZout[o] = f32_to_bf16(g.s * (sg - y));
                        }
                        if (g.Zout) g.Zout[o] = f32_to_bf16(v);
                        if (g.Z32) g.Z32[o] = v;
                    } else if (EPI == EPI_STORE16) {
                        g.C16[o] = f32_to_bf16(v);
                    } else {
                        atomicAdd(g.C32 + o, v);
                    }
                }
            }
            if (EPI == EPI_BCE) {   // sixteen factors per i
                lsum += log1p_pos(prod);
                prod = 0.f;
            }
        }
    }
    if (EPI == EPI_BCE && g.loss) {
        __shared__ float s_loss[4];
        block_loss_add(g.s * (lin + lsum), s_loss, g.loss);
    }
}

bool gemm2_shape(const GemmArgs &g) {
    return g.M % 8 == 0 && g.N % 8 == 0 && g.K % 8 == 0 && g.k_split % 8 == 0;
}

hipError_t launch_gemm(bool a_kmaj, bool b_kmaj, int epi, const GemmArgs &g, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
    const int splits = (g.K + g.k_split - 1) / g.k_split;
    dim3 grid((g.N + TN - 1) / TN, (g.M + TM - 1) / TM, splits);
    if (gemm2_shape(g)) {
        // 64-row M tiles (4 waves of 32 x 64, LDS-bound) only when 128-row
        // tiles (4 waves of 64 x 64) would leave CUs idle
        const int t128 = ((g.N + TN - 1) / TN) * ((g.M + 127) / 128) * splits;
        const bool small = t128 < 256;
        const dim3 grid2((g.N + TN - 1) / TN, (g.M + (small ? 63 : 127)) / (small ? 64 : 128), splits);
#define GL2(AK, BK, E)                                                                    \
    if (small) hipLaunchKernelGGL((k_gemm2<AK, BK, E, 64>), grid2, dim3(256), 0, st, g);  \
    else hipLaunchKernelGGL((k_gemm2<AK, BK, E, 128>), grid2, dim3(256), 0, st, g)
        if (epi == EPI_BCE && a_kmaj && b_kmaj) { GL2(true, true, EPI_BCE); }
        else if (epi == EPI_STORE16 && !a_kmaj && !b_kmaj) { GL2(false, false, EPI_STORE16); }
        else if (epi == EPI_ATOMIC32 && a_kmaj && !b_kmaj) { GL2(true, false, EPI_ATOMIC32); }
        else return hipErrorInvalidValue;
#undef GL2
        return hipGetLastError();
    }
#define GL(AK, BK, E) \
    hipLaunchKernelGGL((k_gemm<AK, BK, E>), grid, dim3(256), 0, st, g)
    if (epi == EPI_BCE && g.pos_ptr) return hipErrorInvalidValue;   // k_gemm reads the bitmap
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
