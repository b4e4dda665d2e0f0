// rewire.hip -- dynamic rewiring of the tail's fan-in sets (prune and
// regrow at group granularity).
//
// HASTE page ("HASTE: Hardware-Aware Dynamic Sparse Training for Large Output
// Spaces"): the title names dynamic sparse training, and section "Method",
// item 1 ("Structure") fixes one fan-in index set per label group, each label
// keeping its own weights.  The page gives no prune or regrow rule; the one
// built here is the plainest form of that training at group granularity:
//   - a position f of group g scores the L1 norm of its weight column over the
//     group's live labels, sum_j |W[gG+j][f]|, added in fp32 in ascending j;
//   - the k positions first in (score, feature id) order are pruned;
//   - k features outside the kept set are regrown from the caller's candidate
//     list (in list order; values outside [0, D), kept features and repeats
//     are skipped), then from the smallest features left;
//   - the new set is stored sorted; a kept feature's weight column moves with
//     it on every row of the group, a regrown feature's column is zero.
//
// One workgroup of one wave per group (G <= 64, F <= 256).  The wave copies
// the group's weights into LDS (one read of W from global memory), scores its
// positions from there, ranks them by counting over the keys in LDS, marks
// the kept features in a D-bit LDS bitmap, takes candidates 64 at a time
// (first occurrences only, so the choice is that of the list order), scans
// the bitmap in order for the sorted new set and writes the moved columns
// from LDS.  Bound: HBM (W read and written once, idx read and written, the
// candidates read); the ranking is O(F^2 / 64) VALU per group.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace haste {

namespace {

constexpr int RW_MAX_F = 256;
constexpr int RW_MAX_G = 64;

__device__ __forceinline__ float rw_abs(unsigned short v) { return __uint_as_float(((unsigned)v & 0x7fffu) << 16); }
__device__ __forceinline__ float rw_abs(float v) { return fabsf(v); }

// LDS regions of one workgroup (host and device agree): keys (8F), old and
// new features (4F each), pruned flags (F), the group's weights (G*F*es,
// 16-byte aligned), the feature bitmap (4 * ceil(D/32))
struct RwLds {
    size_t w, bits, total;
};
__host__ __device__ inline RwLds rw_layout(int G, int F, int D, int es) {
    RwLds l;
    l.w = ((size_t)F * 17 + 15) / 16 * 16;
    l.bits = l.w + ((size_t)G * F * es + 15) / 16 * 16;
    l.total = l.bits + (size_t)((D + 31) >> 5) * 4;
    return l;
}

// PPL: positions per lane (F <= 64 * PPL)
template <typename T, int PPL>
__global__ __launch_bounds__(64) void k_rewire(const int32_t *idx, const T *W, int64_t Ng, int G,
                                               int F, int D, int64_t L, int k, const int32_t *cand,
                                               int R, int32_t *idx_out, T *W_out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const RwLds ly = rw_layout(G, F, D, (int)sizeof(T));
    unsigned long long *keys = (unsigned long long *)smem;   // F: score bits << 32 | feature
    int32_t *oldf = (int32_t *)(keys + F);                   // F: old features, ascending
    int32_t *newf = oldf + F;                                // F: new features, ascending
    unsigned char *gone = (unsigned char *)(newf + F);       // F: 1 = pruned position
    T *wl = (T *)(smem + ly.w);                              // G x F: the group's weights
    unsigned *bits = (unsigned *)(smem + ly.bits);           // ceil(D/32) words
    const int nwords = (D + 31) >> 5;

    const int lane = threadIdx.x;
    const int64_t g = blockIdx.x;
    if (g >= Ng) return;   // whole workgroup (one wave)
    const int64_t row0 = g * (int64_t)G;
    const int live = (int)(L - row0 < G ? L - row0 : G);

    // 1. the group's weights into LDS (every load issued before any use; the
    //    weights are read from global memory once), its features, a clear bitmap
    const T *wg = W + row0 * F;
    const int nw = G * F;
    for (int e = lane; e < nw; e += 64) wl[e] = wg[e];
    for (int p = lane; p < F; p += 64) oldf[p] = idx[g * F + p];
    for (int i = lane; i < nwords; i += 64) bits[i] = 0u;
    __syncthreads();

    // 2. scores (fp32, rows in ascending order) and keys; rank = number of
    //    smaller keys (keys are distinct: the features are); the k smallest
    //    are pruned, the other features go into the bitmap
    unsigned long long mine[PPL];
#pragma unroll
    for (int t = 0; t < PPL; ++t) {
        const int p = lane + 64 * t;
        mine[t] = ~0ull;
        if (p < F) {
            float s = 0.f;
            for (int j = 0; j < live; ++j) s += rw_abs(wl[j * F + p]);
            // scores are >= +0, so their bit patterns order like the values
            mine[t] = ((unsigned long long)__float_as_uint(s) << 32) | (unsigned)oldf[p];
            keys[p] = mine[t];
        }
    }
    __syncthreads();
    unsigned rank[PPL] = {};
#pragma unroll 4
    for (int q = 0; q < F; ++q) {
        const unsigned long long kq = keys[q];   // same address for every lane
#pragma unroll
        for (int t = 0; t < PPL; ++t) rank[t] += kq < mine[t] ? 1u : 0u;
    }
#pragma unroll
    for (int t = 0; t < PPL; ++t) {
        const int p = lane + 64 * t;
        if (p < F) {
            const bool pr = rank[t] < (unsigned)k;
            gone[p] = pr ? 1 : 0;
            const int d = oldf[p];
            if (!pr && d >= 0 && d < D) atomicOr(&bits[d >> 5], 1u << (d & 31));
        }
    }
    __syncthreads();

    // 3. regrow: candidates in list order, 64 at a time
    int need = k;
    for (int base = 0; base < R && need > 0; base += 64) {
        const int c = base + lane < R ? cand[g * R + base + lane] : -1;
        const bool in_range = c >= 0 && c < D;
        const int cs = in_range ? c : 0;
        bool ok = in_range && !((bits[cs >> 5] >> (cs & 31)) & 1u);
        if (__ballot(ok) != 0ull) {
            // only the first occurrence of a value in this batch counts
            for (int i = 0; i < 63; ++i) {
                const int ci = __builtin_amdgcn_readlane(c, i);
                if (i < lane && ci == c) ok = false;
            }
            const unsigned long long bal = __ballot(ok);
            const int before = __popcll(bal & ((1ull << lane) - 1ull));
            if (ok && before < need) atomicOr(&bits[cs >> 5], 1u << (cs & 31));
            const int got = __popcll(bal);
            need -= got < need ? got : need;
        }
        __syncthreads();
    }
    // the list ran out: the smallest features left, in order
    for (int wb = 0; need > 0 && wb < nwords; wb += 64) {
        const int wi = wb + lane;
        unsigned freeb = 0u;
        if (wi < nwords) {
            freeb = ~bits[wi];
            const int hi = D - 32 * wi;   // valid bits in this word
            if (hi < 32) freeb &= (1u << hi) - 1u;
        }
        const int cnt = __popc(freeb);
        int incl = cnt;   // inclusive prefix over the lanes
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
        }
        int t = need - (incl - cnt);   // how many this lane takes
        unsigned setb = 0u;
        while (t > 0 && freeb) {
            const unsigned low = freeb & (0u - freeb);
            setb |= low;
            freeb ^= low;
            --t;
        }
        if (setb) bits[wi] |= setb;   // one lane per word
        const int total = __shfl(incl, 63);
        need -= total < need ? total : need;
        __syncthreads();
    }

    // 4. the new set in ascending order: one bitmap word per lane, rounds of 64
    int out = 0;
    for (int wb = 0; wb < nwords; wb += 64) {
        const int wi = wb + lane;
        unsigned b = wi < nwords ? bits[wi] : 0u;
        const int cnt = __popc(b);
        int incl = cnt;
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
        }
        int pos = out + incl - cnt;
        while (b) {
            const int bit = __builtin_ctz(b);
            b &= b - 1u;
            if (pos < F) newf[pos] = 32 * wi + bit;
            ++pos;
        }
        out += __shfl(incl, 63);
    }
    __syncthreads();

    // 5. sources of the new positions: the old position of a kept feature
    //    (binary search in the sorted old set), -1 for a regrown one; then the
    //    new index row and the moved columns (from LDS: the group's weights
    //    were read in full before any store, so idx_out / W_out may be idx / W)
    int src[PPL];
#pragma unroll
    for (int t = 0; t < PPL; ++t) {
        const int p = lane + 64 * t;
        src[t] = -1;
        if (p < F) {
            const int d = newf[p];
            int lo = 0, hi = F - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (oldf[mid] < d) lo = mid + 1;
                else hi = mid;
            }
            if (oldf[lo] == d && !gone[lo]) src[t] = lo;
            idx_out[g * F + p] = d;
        }
    }
    T *wo = W_out + row0 * F;
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int t = 0; t < PPL; ++t) {
            const int p = lane + 64 * t;
            if (p < F) wo[j * F + p] = src[t] >= 0 ? wl[j * F + src[t]] : T(0);
        }
}

template <typename T>
hipError_t rw_go(const int32_t *idx, const void *W, int64_t Ng, int G, int F, int D, int64_t L,
                 int k, const int32_t *cand, int R, int32_t *idx_out, void *W_out, hipStream_t st) {
    const size_t lds = rw_layout(G, F, D, (int)sizeof(T)).total;
    auto launch = [&](auto kern) {
        if (lds > 64 * 1024)
            (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(kern, dim3((unsigned)Ng), dim3(64), lds, st, idx, (const T *)W, Ng, G, F, D,
                           L, k, cand, R, idx_out, (T *)W_out);
    };
    if (F <= 64) launch(k_rewire<T, 1>);
    else if (F <= 128) launch(k_rewire<T, 2>);
    else launch(k_rewire<T, 4>);
    return hipGetLastError();
}

}  // namespace

bool rewire_supported(int G, int F, int D) {
    return G >= 1 && G <= RW_MAX_G && F >= 1 && F <= RW_MAX_F && D >= F && D <= 65536;
}

hipError_t launch_rewire(const int32_t *idx, const void *W, bool bf16, int64_t Ng, int G, int F,
                         int D, int64_t L, int k, const int32_t *cand, int R, int32_t *idx_out,
                         void *W_out, hipStream_t st) {
    if (Ng == 0) return hipSuccess;
    return bf16 ? rw_go<unsigned short>(idx, W, Ng, G, F, D, L, k, cand, R, idx_out, W_out, st)
                : rw_go<float>(idx, W, Ng, G, F, D, L, k, cand, R, idx_out, W_out, st);
}

}  // namespace haste
