// dxs.hip -- the tail's dX pass at the layer's own arithmetic (HASTE page,
// section "Method", item 1: the backward scatters each group's product back
// through its shared index set).
//
// For a row chunk of 32 rows and one label group g,
//     Y_g = dz_g (32 x G) . W_g (G x F)                 (MFMA, K = G)
//     dX[r][idx[g][f]] += Y_g[r][f]
// The scatter goes into a dX^T tile of the chunk that lives in LDS (D feature
// rows of 32 fp32 values) for the whole range of groups a workgroup takes, and
// the tile is added into dX with one fp32 atomic per element at the end.
// Unlike the dense form (dz_g times W_g scattered to all D features, D/F times
// the flops), the contraction here is exactly 2 * 32 * G * F flops per group
// and chunk, and the scatter moves 32 * F values.
//
// dz comes from the tiles the dW/logits pass stored (1 KB per 32 rows x 16
// labels, lane (q, m) of that pass holding label m, rows 4q..4q+3 and
// 16+4q..16+4q+3).
//
// Workgroup: 4 waves (F = 32) or 8 (F >= 64: two per SIMD).  Wave w = P t + h,
// P = waves / 2, takes rows 16t..16t+15 of the chunk and the feature part h of
// every group, so within a group the waves touch disjoint (row, feature) cells; one barrier per group keeps the
// groups apart (two groups may share features).  The barrier also hands over
// a two-stage ring of operands that direct global->LDS copies fill one group
// ahead: the group's dz tiles and W_g (16-byte pieces permuted on the way so
// that the transposing operand reads hit distinct banks).  In iteration g a
// wave forms Y of group g + 1 on the matrix cores while it adds Y of group g
// into the tile.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace haste {

constexpr int DXS_R = 32;      // rows per chunk (one dz tile row block)

// waves per workgroup: two row halves x NW/2 feature parts of 16-feature tiles
__host__ __device__ constexpr int dxs_nw(int F) { return F >= 64 ? 8 : 4; }

template <int G, int F, int NW = dxs_nw(F)>
struct DxsShape {
    static constexpr int JT = G / 16;                // dz tiles per group and chunk
    static constexpr int DZB = JT * 1024;            // their bytes
    static constexpr int WB = G * F * 2;             // W_g bytes
    static constexpr int IXB = F * 4;                // idx_g bytes
    static constexpr int STAGE = DZB + WB + IXB;     // one stage: dz tiles, W_g, idx_g
    static constexpr int NP = STAGE / 16;            // its 16-byte pieces
    static constexpr int NPW = (NP + 64 * NW - 1) / (64 * NW);   // pieces per lane
    // groups in flight from global memory: a register ring of DPF * NPW * 4
    // VGPRs, at most 128 of a wave's 256
    static constexpr int DPF = 32 / NPW > 8 ? 8 : 32 / NPW;
    static constexpr int NFP = NW / 2;               // feature parts
    static constexpr int FTW = F / 16 / NFP;         // 16-feature tiles per wave
    static constexpr int KS = G >= 32 ? G / 32 : 1;  // K steps of 32 labels (G = 16: one K = 16 step)
    static constexpr int QB = G >= 32 ? 3 : 2;       // label bit that tells the paired lane blocks apart
    static constexpr int P = F / 8;                  // 16-byte pieces per W_g row
};

// dz tile: the piece of lane (qq, m) of the dW pass sits at slot
// qq*16 + (m ^ 4qq) (an involution), so the transposing reads of one 16-lane
// block fall on distinct banks.
__device__ __forceinline__ int dxs_dz_slot(int qq, int m) { return qq * 16 + (m ^ (4 * qq)); }

// W_g row j: piece p sits at p ^ sigma(j); sigma separates the four labels
// one transposing read covers and the two lane blocks serviced together.
template <int F, int QB>
__device__ __forceinline__ int dxs_w_sigma(int j) {
    if constexpr (F == 128) return ((j & 3) << 1) | (((j >> QB) & 1) << 3);
    else if constexpr (F == 64) return (((j >> 1) & 1) << 1) | (((j >> QB) & 1) << 2);
    else return ((j >> QB) & 1) << 1;
}


// f(integral_constant<int, K>) for K = 0, 1, ..., in order
template <typename Fn, int... K>
__device__ __forceinline__ void dxs_unroll(Fn &&f, std::integer_sequence<int, K...>) {
    (f(std::integral_constant<int, K>{}), ...);
}

// dX^T tile: feature d is a row of 32 floats (8 slots of 16 bytes); slot s of
// row d is stored at s ^ ((d >> 1) & 7), so that 16 lanes writing rows with
// distinct d mod 16 hit distinct banks.  Returns the float offset.
__device__ __forceinline__ int dxs_tile_off(int d, int slot) {
    return d * 32 + ((slot ^ ((d >> 1) & 7)) << 2);
}

template <int G, int F>
__global__ __launch_bounds__(64 * dxs_nw(F), 1) void k_tail_dxs(TailArgs a, int nrc, int ngr) {
    using S = DxsShape<G, F>;
    constexpr int DXS_NW = dxs_nw(F);
    constexpr int FTW = S::FTW, KS = S::KS, QB = S::QB, NPW = S::NPW;
    constexpr int DPF = S::DPF;
    // the two stages are distinct LDS objects, each named statically in every
    // (unrolled) iteration
    __shared__ __attribute__((aligned(16))) unsigned char st0[S::STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char st1[S::STAGE];
    extern __shared__ __attribute__((aligned(16))) float dxt[];   // D x 32, swizzled slots

    const int lane = threadIdx.x & 63;
    const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, m = lane & 15;
    const int t = wu / S::NFP, hf = wu % S::NFP;
    // block -> (row chunk, group range); blocks b, b + 8, ... share an XCD, and
    // the nrc row chunks of one group range are among them, so W_g comes from
    // HBM once and from that XCD's L2 for the others
    const int bid = blockIdx.x, xcd = bid & 7, k8 = bid >> 3;
    const int rc = k8 % nrc, gr = (k8 / nrc) * 8 + xcd;
    const int64_t g0 = (int64_t)gr * a.Ng / ngr, g1 = (int64_t)(gr + 1) * a.Ng / ngr;
    if (g0 >= g1) return;   // workgroup-uniform: no barrier is skipped by part of it

    for (int i = threadIdx.x; i < a.D * 8; i += 64 * DXS_NW)
        *(f32x4 *)(dxt + 4 * i) = (f32x4){0.f, 0.f, 0.f, 0.f};

    // ---- per-lane constant parts of the operand addresses (bytes within a stage)
    const int kk = m >> 2, cc = m & 3;   // addressing role of this lane in its block
    // A (dz, rows 16t + m, K = labels): tile 2ks + (q >> 1), labels j0 .. j0 + 3
    int offA[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int j0 = G >= 32 ? 8 * (q & 1) + 4 * r : 4 * q;
        const int jt = G >= 32 ? (q >> 1) : 0;
        offA[r] = jt * 1024 + 16 * dxs_dz_slot(cc, j0 + kk) + 8 * t;
    }
    // B (W_g, features 16ft + m, K = labels): label j = 32ks + 8q + 4r + kk
    // (G = 16: 4q + kk); sigma(j) depends on kk and q only
    const int jb = G >= 32 ? 8 * q + kk : 4 * q + kk;
    const int sig = dxs_w_sigma<F, QB>(jb);
    int offB[FTW];
#pragma unroll
    for (int u = 0; u < FTW; ++u) {
        const int ft = hf * FTW + u;
        const int p = 2 * ft + (cc >> 1);
        offB[u] = S::DZB + jb * (2 * F) + 16 * (p ^ sig) + 8 * (cc & 1);
    }
    const int live_last = (int)(a.L - (a.Ng - 1) * G);   // live labels of the last group

    // ---- a group's stage as 16-byte pieces: dz tiles (piece of lane (qq, m')
    // of a tile at slot dxs_dz_slot), W_g (piece p of row j at p ^ sigma(j)),
    // idx_g.  Wave w moves the 1 KB blocks 4n + w, n < NPW (blocks past the
    // stage repeat the last one: the same bytes to the same place), so every
    // wave loads exactly NPW pieces per lane and group and the compiler can
    // count its outstanding loads.  A block lies in one region, so its source
    // is a wave-uniform base plus a per-lane offset.
    constexpr int NB = (S::NP + 63) / 64;   // 1 KB blocks of a stage (the last one partial)
    int blk[NPW], srcoff[NPW], wrow[NPW];
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
        blk[n] = min(n * DXS_NW + wu, NB - 1);   // wave-uniform
        const int pc = min(blk[n] * 64 + lane, S::NP - 1);
        wrow[n] = -1;
        if (pc < S::DZB / 16) {
            const int tile = pc >> 6, sl = pc & 63;
            srcoff[n] = tile * 1024 + 16 * dxs_dz_slot(sl >> 4, sl & 15);   // involution
        } else if (pc < (S::DZB + S::WB) / 16) {
            const int sp = pc - S::DZB / 16, j = sp / S::P, pp = sp % S::P;
            srcoff[n] = j * (2 * F) + 16 * (pp ^ dxs_w_sigma<F, QB>(j));
            wrow[n] = j;
        } else {
            srcoff[n] = 16 * (pc - (S::DZB + S::WB) / 16);
        }
    }
    auto gload = [&](int64_t g, u32x4 (&r)[NPW]) {
#pragma unroll
        for (int n = 0; n < NPW; ++n) {
            const int b0 = blk[n] * 64;   // first piece of the block (wave-uniform)
            const char *base = b0 < S::DZB / 16 ? (const char *)(a.dzt + ((g * nrc + rc) * S::JT << 9))
                             : b0 < (S::DZB + S::WB) / 16 ? (const char *)(a.W + g * G * (int64_t)F)
                                                          : (const char *)(a.idx + g * F);
            r[n] = *(const u32x4 *)(base + srcoff[n]);
        }
    };
    auto lwrite = [&](int64_t g, u32x4 (&r)[NPW], unsigned char *stg) {
        if (g == a.Ng - 1 && live_last < G) {   // wave-uniform, the last group only
            // labels past L: their W rows are never read for a result; zero
#pragma unroll
            for (int n = 0; n < NPW; ++n)
                if (wrow[n] >= live_last) r[n] = (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int n = 0; n < NPW; ++n)
            *(u32x4 *)(stg + 16 * min(blk[n] * 64 + lane, S::NP - 1)) = r[n];
    };
    // Y of a group from its stage: lane (q, m) gets feature 16ft + m, rows
    // 16t + 4q .. + 3
    auto product = [&](const unsigned char *stg, f32x4 (&y)[FTW]) {
#pragma unroll
        for (int u = 0; u < FTW; ++u) y[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (G >= 32) {
                const i16x4 a0 = lds_read_tr(stg + offA[0] + ks * 2048);
                const i16x4 a1 = lds_read_tr(stg + offA[1] + ks * 2048);
                const bf16x8 A = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int u = 0; u < FTW; ++u) {
                    const i16x4 b0 = lds_read_tr(stg + offB[u] + ks * 32 * 2 * F);
                    const i16x4 b1 = lds_read_tr(stg + offB[u] + ks * 32 * 2 * F + 4 * 2 * F);
                    const bf16x8 Bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
                    y[u] = mfma32(A, Bv, y[u]);
                }
            } else {
                const i16x4 A = lds_read_tr(stg + offA[0]);
#pragma unroll
                for (int u = 0; u < FTW; ++u) y[u] = mfma16(A, lds_read_tr(stg + offB[u]), y[u]);
            }
        }
    };
    // this lane's features of the group in a stage (one per tile)
    auto read_idx = [&](const unsigned char *stg, int (&ix)[FTW]) {
#pragma unroll
        for (int u = 0; u < FTW; ++u)
            ix[u] = *(const int *)(stg + S::DZB + S::WB + 4 * (16 * (hf * FTW + u) + m));
    };
    // tile += Y of one group (all reads, then all writes: the group's features are distinct)
    auto scatter = [&](const f32x4 (&y)[FTW], const int (&ix)[FTW]) {
        f32x4 *p[FTW];
        f32x4 old[FTW];
#pragma unroll
        for (int u = 0; u < FTW; ++u) p[u] = (f32x4 *)(dxt + dxs_tile_off(ix[u], 4 * t + q));
#pragma unroll
        for (int u = 0; u < FTW; ++u) old[u] = *p[u];
#pragma unroll
        for (int u = 0; u < FTW; ++u) *p[u] = old[u] + y[u];
    };

    // Pipeline.  Before iteration g: ycur = Y of g, icur = features of g, the
    // stage of g + 1 written; register slot (h - g0) mod DPF holds group h for
    // h = g + 2 .. g + DPF + 1 (loads past the range repeat the last group).
    // Iteration g: barrier (the stage of g + 1 written by every wave, the
    // stage of g read by every wave, the scatter of g - 1 done), scatter Y of
    // g, read the features of g + 1 and form Y of g + 1 from its stage, write
    // group g + 2 from its register slot into the stage of g, load group
    // g + 2 + DPF into that slot.
    u32x4 pf[DPF][NPW];
    f32x4 ycur[FTW], ynext[FTW] = {};
    int icur[FTW], inext[FTW] = {};
    // groups counted from g0 in 32-bit scalar arithmetic (64-bit compares
    // would be vector instructions)
    const int nrg = (int)(g1 - g0);
    auto clampg = [&](int r) { return g0 + (r < nrg ? r : nrg - 1); };
#pragma unroll
    for (int k = 0; k < DPF; ++k) gload(clampg(k), pf[k]);
    lwrite(g0, pf[0], st0);
    lwrite(clampg(1), pf[1], st1);
    gload(clampg(DPF), pf[0]);
    gload(clampg(DPF + 1), pf[1]);
    lds_barrier();                    // stages of g0, g0 + 1 written; tile zeroed
    read_idx(st0, icur);
    product(st0, ycur);

    auto iter = [&](auto kslot, int r) {          // group g0 + r
        constexpr int K = decltype(kslot)::value;   // r mod DPF
        constexpr int K2 = (K + 2) % DPF;           // slot of r + 2
        // stage of r (and r + 2) and of r + 1: parity of r (DPF is even or
        // the parity is taken from r itself)
        const bool odd = (DPF % 2 == 0) ? (K & 1) : (r & 1);
        unsigned char *const sa = odd ? st1 : st0;
        unsigned char *const sb = odd ? st0 : st1;
        lds_barrier();
        scatter(ycur, icur);
        if (r + 1 < nrg) {
            read_idx(sb, inext);
            product(sb, ynext);
        }
        if (r + 2 < nrg) lwrite(g0 + r + 2, pf[K2], sa);
        gload(clampg(r + 2 + DPF), pf[K2]);
#pragma unroll
        for (int u = 0; u < FTW; ++u) {
            ycur[u] = ynext[u];
            icur[u] = inext[u];
        }
    };
    // unrolled DPF times, so that every register slot is named statically
    for (int r = 0; r < nrg; r += DPF)
        dxs_unroll([&](auto k) {
            if (r + decltype(k)::value < nrg) iter(k, r + decltype(k)::value);
        }, std::make_integer_sequence<int, DPF>{});

    // ---- flush: one fp32 atomic per live element; lanes run over consecutive
    // features of one 4-row slot, so each atomic instruction is coalesced
    lds_barrier();
    const int r0 = rc * DXS_R;
    for (int i = threadIdx.x; i < a.D * 8; i += 64 * DXS_NW) {
        const int sl = i / a.D, d = i - sl * a.D;
        const f32x4 v = *(const f32x4 *)(dxt + dxs_tile_off(d, sl));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = r0 + 4 * sl + e;
            if (row < a.B && v[e] != 0.f) atomicAdd(a.dX + (int64_t)row * a.D + d, v[e]);
        }
    }
}

static void dxs_allow_lds(const void *fn, size_t bytes) {
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int G, int F>
static bool dxs_fits_t(int D) {
    return 2 * (size_t)DxsShape<G, F>::STAGE + (size_t)D * DXS_R * 4 <= 160 * 1024;
}

template <int G, int F>
static hipError_t dxs_go(const TailArgs &a, hipStream_t st) {
    if (!dxs_fits_t<G, F>(a.D) || !a.dzt || a.Bp % DXS_R) return hipErrorInvalidValue;
    const int nrc = a.Bp / DXS_R;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    // group ranges: a multiple of 8 (the row chunks of a range share an XCD),
    // about one workgroup per CU in all (the tile fills most of a CU's LDS)
    int ngr = (ncu + nrc - 1) / nrc;
    ngr = (ngr + 7) / 8 * 8;
    if (a.Ng / ngr + 1 > 0x7fffffff) return hipErrorInvalidValue;   // groups of a range: 32-bit
    const size_t dyn = (size_t)a.D * DXS_R * 4;
    dxs_allow_lds((const void *)k_tail_dxs<G, F>, dyn);
    hipLaunchKernelGGL((k_tail_dxs<G, F>), dim3((unsigned)(nrc * ngr)), dim3(64 * dxs_nw(F)), dyn, st, a, nrc, ngr);
    return hipGetLastError();
}

bool tail_dxs_supported(int G, int F, int D) {
    switch (G * 1000 + F) {
    case 16032: return dxs_fits_t<16, 32>(D);
    case 16064: return dxs_fits_t<16, 64>(D);
    case 16128: return dxs_fits_t<16, 128>(D);
    case 32032: return dxs_fits_t<32, 32>(D);
    case 32064: return dxs_fits_t<32, 64>(D);
    case 32128: return dxs_fits_t<32, 128>(D);
    case 64032: return dxs_fits_t<64, 32>(D);
    case 64064: return dxs_fits_t<64, 64>(D);
    case 64128: return dxs_fits_t<64, 128>(D);
    }
    return false;
}

hipError_t launch_tail_dxs(int G, const TailArgs &a, hipStream_t st) {
    switch (G * 1000 + a.F) {
    case 16032: return dxs_go<16, 32>(a, st);
    case 16064: return dxs_go<16, 64>(a, st);
    case 16128: return dxs_go<16, 128>(a, st);
    case 32032: return dxs_go<32, 32>(a, st);
    case 32064: return dxs_go<32, 64>(a, st);
    case 32128: return dxs_go<32, 128>(a, st);
    case 64032: return dxs_go<64, 32>(a, st);
    case 64064: return dxs_go<64, 64>(a, st);
    case 64128: return dxs_go<64, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace haste
