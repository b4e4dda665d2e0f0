// abi.hip -- the extern "C" entry points of libhaste (declared and
// documented in include/haste.h): host-side argument checks, workspace
// layout and kernel dispatch.  Nothing here allocates device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/haste.h"
#include "kernels.h"

using namespace haste;

namespace {

thread_local std::string g_err;

haste_status fail(haste_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
haste_status fail(haste_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

haste_status hip_ok(hipError_t e, const char *what) {
    if (e == hipSuccess) return HASTE_OK;
    return fail(HASTE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TRY_HIP(expr, what)                                  \
    do {                                                     \
        haste_status _s = hip_ok((expr), (what));            \
        if (_s != HASTE_OK) return _s;                       \
    } while (0)
#define TRY(expr)                                            \
    do {                                                     \
        haste_status _s = (expr);                            \
        if (_s != HASTE_OK) return _s;                       \
    } while (0)

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// bytes of the top-K bucket lists (value + id per entry) for B rows of n logits
size_t topk_cand_bytes(int B, int64_t n, const haste_bce *bce) {
    const int K = bce->topk;
    const int KP = bce->topk_kprime > 0 && bce->topk_kprime <= K ? bce->topk_kprime : K;
    const int64_t nb = bce->topk_buckets > 0 ? bce->topk_buckets : 0;
    return (size_t)B * (size_t)topk_buckets(n, nb, B).nseg * (size_t)KP * 8;
}
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline int64_t n_groups(const haste_tail_desc *d) { return (d->L + d->G - 1) / d->G; }
inline int pad_rows(int B) { return (B + 63) / 64 * 64; }

// ----------------------------------------------------------- workspace maps
struct TailWs {
    size_t xt, cnt, ptr, ent, idxp, perm, sched, dz, dzt, z32, cand, fwd_total, total;
    bool has_dzt, has_topk, tk_fused, tk_exact;
};

// The exact top-K (K' = K) of bf16 groups of 16 and more: the logits pass
// keeps each (group, row)'s largest logit, a merge takes each row's K best
// groups, and a last pass recomputes those groups' logits and keeps the K
// best -- exact for any bucketing, without the fp32 logits.
bool topk_exact_fused(const haste_tail_desc *d, const haste_bce *bce) {
    if (!bce || bce->topk <= 0 || d->dtype != HASTE_BF16 || d->G < 16) return false;
    return bce->topk_kprime == 0 || bce->topk_kprime == bce->topk;
}

// The top-K's stage 1 runs inside the logits pass when its buckets are the
// label groups and K' = 1 (bf16, groups of 16 and more): same buckets, same
// K', same result as the separate stage 1, without the fp32 logits; and for
// the exact top-K (above).
bool topk_fused(const haste_tail_desc *d, const haste_bce *bce) {
    if (topk_exact_fused(d, bce)) return true;
    if (!bce || bce->topk <= 0 || d->dtype != HASTE_BF16 || d->G < 16) return false;
    if (bce->topk_kprime != 1 || bce->topk_buckets <= 0) return false;
    return topk_buckets(d->L, bce->topk_buckets, d->B).seg_len == d->G;
}

TailWs tail_ws(const haste_tail_desc *d, const haste_bce *bce) {
    TailWs w{};
    const int64_t ng = n_groups(d);
    const int nnz = bce ? (bce->nnz > 0 ? bce->nnz : 0) : 0;
    size_t o = 0;
    if (d->dtype == HASTE_BF16) {
        // first the dW/logits pass's feature order: idx reordered, and the
        // order (groups of 16 and more; G = 1 gathers per label).  It depends
        // on the shape and idx alone, so it sits at the same offset for every
        // call and haste_tail_prepare_layout can form it once.
        if (d->G > 1) {
            w.idxp = o; o += al256((size_t)ng * d->F * 2);
            w.perm = o; o += al256((size_t)ng * d->F);
        }
        w.xt = o;  o += al256((size_t)d->D * pad_rows(d->B) * 2);
        w.cnt = o; o += al256((size_t)(nnz > 0 ? nnz : 1) * 20 + 8);  // keys, sorted, ranks, count
        w.ptr = o; o += al256((size_t)(ng + 4) * 4);   // +3: 16-byte reads of a pair
        w.ent = o; o += al256((size_t)(nnz > 0 ? nnz : 1) * 4);
        w.sched = o; o += 256;   // the dW/logits pass's run counters
        // dz of the dW pass, kept for the dX pass unless the caller asks for
        // the lean form (which recomputes it): Bp x (Ng*G) bf16 in 1 KB tiles
        // (also without bce: the backward from a given dZ forms the same tiles)
        // (G = 1: the step's dz, label-major, L x B_p bf16: the same size)
        w.has_dzt = !(d->flags & HASTE_TAIL_LEAN);
    } else {
        // per-group counts; also the key space of haste_tail_group_positives
        const size_t keys = (size_t)(nnz > 0 ? nnz : 1) * 20 + 8;
        w.cnt = o; o += al256((size_t)ng * 4 > keys ? (size_t)ng * 4 : keys);
        w.dz = o;  o += al256((size_t)d->B * d->L * 4);
    }
    // top-K: fp32 logits B x L and the per-bucket lists; when stage 1 is fused,
    // the group-major lists (N_g x B_pad) and the merge's segment lists instead
    w.has_topk = bce && bce->topk > 0;
    w.tk_fused = topk_fused(d, bce);
    w.tk_exact = topk_exact_fused(d, bce);
    if (w.has_topk && !w.tk_fused) {
        w.z32 = o;  o += al256((size_t)d->B * d->L * 4);
        w.cand = o; o += al256(topk_cand_bytes(d->B, d->L, bce));
    } else if (w.has_topk) {
        w.cand = o;
        o += al256((size_t)ng * pad_rows(d->B) * 8 +
                   (size_t)d->B * topk_gm_segments(ng, d->B).nseg * bce->topk * 8);
    }
    // the dz tiles last: the forward, which never uses them, needs only what
    // comes before (fwd_total)
    w.fwd_total = o;
    if (w.has_dzt) { w.dzt = o; o += al256((size_t)ng * d->G * pad_rows(d->B) * 2); }
    w.total = o;
    return w;
}

struct HeadWs {
    size_t bm, dz, z32, cand, total;
    int words;
    bool has_topk;
};

HeadWs head_ws(const haste_head_desc *d, const haste_bce *bce) {
    HeadWs w{};
    size_t o = 0;
    w.words = (d->H + 31) / 32;
    w.bm = o; o += al256((size_t)d->B * w.words * 4);
    w.dz = o; o += al256((size_t)d->B * d->H * (d->dtype == HASTE_BF16 ? 2 : 4));
    w.has_topk = bce && bce->topk > 0;
    if (w.has_topk) {
        w.z32 = o;  o += al256((size_t)d->B * d->H * 4);
        w.cand = o; o += al256(topk_cand_bytes(d->B, d->H, bce));
    }
    w.total = o;
    return w;
}

// ------------------------------------------------------------- validation
haste_status check_tail(const haste_tail_desc *d) {
    if (!d) return fail(HASTE_ERR_INVALID, "tail descriptor is NULL");
    if (d->B < 1 || d->D < 1 || d->L < 1 || d->G < 1 || d->F < 1)
        return fail(HASTE_ERR_INVALID, "tail sizes must be >= 1 (B=%d D=%d L=%lld G=%d F=%d)",
                    d->B, d->D, (long long)d->L, d->G, d->F);
    if (d->F > d->D) return fail(HASTE_ERR_INVALID, "F=%d exceeds D=%d", d->F, d->D);
    if (d->dtype != HASTE_F32 && d->dtype != HASTE_BF16)
        return fail(HASTE_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (d->flags & ~(HASTE_TAIL_LEAN | HASTE_TAIL_LAYOUT_READY))
        return fail(HASTE_ERR_INVALID, "unknown tail flags 0x%x", d->flags);
    if (d->dtype == HASTE_BF16) {
        if (!tail_bf16_supported(d->G, d->F, d->D))
            return fail(HASTE_ERR_UNSUPPORTED,
                        "bf16 tail supports G in {16,32,64}, F in {32,64,128}, F <= D <= 1024 "
                        "(got G=%d F=%d D=%d)", d->G, d->F, d->D);
        if ((int64_t)d->B * d->G > (1 << 30))
            return fail(HASTE_ERR_UNSUPPORTED, "B*G too large");
    }
    if (d->L > ((int64_t)1 << 40)) return fail(HASTE_ERR_UNSUPPORTED, "L too large");
    return HASTE_OK;
}

haste_status check_head(const haste_head_desc *d) {
    if (!d) return fail(HASTE_ERR_INVALID, "head descriptor is NULL");
    if (d->B < 1 || d->D < 1 || d->H < 1)
        return fail(HASTE_ERR_INVALID, "head sizes must be >= 1 (B=%d D=%d H=%d)", d->B, d->D, d->H);
    if (d->dtype != HASTE_F32 && d->dtype != HASTE_BF16)
        return fail(HASTE_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (d->dtype == HASTE_BF16 && (d->D % 8 != 0 || d->H % 8 != 0))
        return fail(HASTE_ERR_UNSUPPORTED, "bf16 head needs D and H multiples of 8 (D=%d H=%d)",
                    d->D, d->H);
    return HASTE_OK;
}

// n: the call's label count (ids label_offset .. label_offset + n - 1)
haste_status check_bce(const haste_bce *b, int B, bool topk_ok, int64_t n) {
    if (!b) return HASTE_OK;
    if (b->nnz < 0) return fail(HASTE_ERR_INVALID, "bce.nnz < 0");
    if (!b->row_ptr) return fail(HASTE_ERR_INVALID, "bce.row_ptr is NULL");
    if (b->nnz > 0 && !b->labels) return fail(HASTE_ERR_INVALID, "bce.labels is NULL");
    if (b->label_offset < 0) return fail(HASTE_ERR_INVALID, "bce.label_offset < 0");
    if (b->topk < 0 || b->topk > 8) return fail(HASTE_ERR_INVALID, "bce.topk=%d outside [0, 8]", b->topk);
    if (b->topk != 0) {
        if (!topk_ok) return fail(HASTE_ERR_UNSUPPORTED, "bce.topk is not supported by this call");
        if (b->topk_kprime < 0 || b->topk_kprime > b->topk)
            return fail(HASTE_ERR_INVALID, "bce.topk_kprime=%d outside [0, topk=%d]", b->topk_kprime, b->topk);
        if (b->topk_buckets < 0 || b->topk_buckets > (1 << 24))
            return fail(HASTE_ERR_INVALID, "bce.topk_buckets=%d outside [0, 2^24]", b->topk_buckets);
        if (b->topk_kprime > 0 && b->topk_kprime < b->topk && b->topk_buckets == 0)
            return fail(HASTE_ERR_INVALID, "an approximate top-K (K' < K) needs bce.topk_buckets > 0");
        if (!b->topk_val || !aligned(b->topk_val, 4)) return fail(HASTE_ERR_INVALID, "bce.topk_val NULL or misaligned");
        if (!b->topk_idx || !aligned(b->topk_idx, 4)) return fail(HASTE_ERR_INVALID, "bce.topk_idx NULL or misaligned");
        if (b->label_offset + n - 1 > (int64_t)INT32_MAX)
            return fail(HASTE_ERR_UNSUPPORTED, "top-K ids are int32: label_offset + labels - 1 = %lld exceeds 2^31 - 1",
                        (long long)(b->label_offset + n - 1));
    }
    (void)B;
    return HASTE_OK;
}

haste_status need(const void *p, const char *name) {
    if (!p) return fail(HASTE_ERR_INVALID, "%s is NULL", name);
    return HASTE_OK;
}

haste_status need_al(const void *p, size_t a, const char *name) {
    if (!p) return fail(HASTE_ERR_INVALID, "%s is NULL", name);
    if (!aligned(p, a)) return fail(HASTE_ERR_INVALID, "%s is not %zu-byte aligned", name, a);
    return HASTE_OK;
}

haste_status check_ws(void *ws, size_t ws_bytes, size_t need_bytes) {
    if (need_bytes == 0) return HASTE_OK;
    if (!ws) return fail(HASTE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need_bytes);
    if (!aligned(ws, 256)) return fail(HASTE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (ws_bytes < need_bytes)
        return fail(HASTE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need_bytes);
    return HASTE_OK;
}

hipStream_t S(void *st) { return (hipStream_t)st; }
char *B8(void *p, size_t off) { return (char *)p + off; }

// ---------------------------------------------------------- bf16 tail core
TailArgs tail_args(const haste_tail_desc *d, const void *X, const int32_t *idx, const void *W,
                   void *ws, const TailWs &m) {
    (void)X;
    TailArgs a{};
    a.XT = (const unsigned short *)B8(ws, m.xt);
    a.idx = idx;
    a.W = (const unsigned short *)W;
    a.grp_ptr = (const int32_t *)B8(ws, m.ptr);
    a.grp_ent = (const int32_t *)B8(ws, m.ent);
    a.idxp = (const unsigned short *)B8(ws, m.idxp);
    a.perm = (const unsigned char *)B8(ws, m.perm);
    a.dzt = m.has_dzt ? (unsigned short *)B8(ws, m.dzt) : nullptr;
    a.sched = (unsigned *)B8(ws, m.sched);
    a.Z32 = m.has_topk && !m.tk_fused ? (float *)B8(ws, m.z32) : nullptr;
    if (m.tk_fused) {   // the group-major bucket lists, written by the logits pass (K' = 1)
        a.tk_v = (float *)B8(ws, m.cand);
        a.tk_i = (int32_t *)(a.tk_v + n_groups(d) * pad_rows(d->B));
        a.tk_max_only = m.tk_exact ? 1 : 0;
    }
    a.B = d->B;
    a.D = d->D;
    a.Bp = pad_rows(d->B);
    a.F = d->F;
    a.L = d->L;
    a.Ng = n_groups(d);
    return a;
}

haste_status bf16_prep(const haste_tail_desc *d, const void *X, const haste_bce *bce, void *ws,
                       const TailWs &m, hipStream_t st) {
    TRY_HIP(launch_transpose_x((const unsigned short *)X, (unsigned short *)B8(ws, m.xt), d->B,
                               d->D, pad_rows(d->B), (unsigned *)B8(ws, m.sched), st),
            "transpose X");
    if (bce) {
        TRY_HIP(launch_group_positives(bce->row_ptr, bce->labels, bce->nnz, d->B, bce->label_offset,
                                       d->L, d->G, n_groups(d), (long long *)B8(ws, m.cnt),
                                       (int32_t *)B8(ws, m.ptr), (int32_t *)B8(ws, m.ent), st),
                "group positives");
    }
    return HASTE_OK;
}

// The order in which the dW/logits pass reads each group's features; it
// depends on idx alone and is formed before every such pass.
haste_status feature_order(const haste_tail_desc *d, const int32_t *idx, void *ws, const TailWs &m,
                           hipStream_t st) {
    if (d->flags & HASTE_TAIL_LAYOUT_READY) return HASTE_OK;   // formed by an earlier call
    TRY_HIP(launch_feature_order(idx, n_groups(d), d->F, (unsigned short *)B8(ws, m.idxp),
                                 (unsigned char *)B8(ws, m.perm), st),
            "feature order");
    return HASTE_OK;
}

F32Args f32_tail_args(const haste_tail_desc *d, const void *X, const int32_t *idx, const void *W,
                      const haste_bce *bce) {
    F32Args a{};
    a.X = (const float *)X;
    a.idx = idx;
    a.W = (const float *)W;
    a.B = d->B;
    a.D = d->D;
    a.G = d->G;
    a.F = d->F;
    a.L = d->L;
    a.Ng = n_groups(d);
    if (bce) {
        a.row_ptr = bce->row_ptr;
        a.labels = bce->labels;
        a.label_offset = bce->label_offset;
        a.s = bce->grad_scale;
        a.loss = bce->loss;
    }
    return a;
}

// per-row top-K of the fp32 logits z (B x n) into bce->topk_val / topk_idx
haste_status run_topk(const haste_bce *bce, const float *z, int B, int64_t n, void *ws, size_t cand,
                      hipStream_t st) {
    const int K = bce->topk, KP = bce->topk_kprime ? bce->topk_kprime : K;
    const int64_t nc = (int64_t)B * topk_buckets(n, bce->topk_buckets, B).nseg * KP;
    float *cv = (float *)B8(ws, cand);
    int32_t *ci = (int32_t *)(cv + nc);
    TRY_HIP(launch_row_topk(z, n, B, n, bce->label_offset, K, KP, bce->topk_buckets, cv, ci,
                            bce->topk_val, bce->topk_idx, st),
            "top-K");
    return HASTE_OK;
}

// the tail's top-K after its logits pass: stage 2 alone when stage 1 was
// fused (one maximum per group); for the exact top-K, then the recomputation
// of each row's K best groups
haste_status tail_topk(const haste_tail_desc *d, const void *X, const haste_bce *bce, const TailWs &m,
                       const TailArgs &a, void *ws, hipStream_t st) {
    if (!m.has_topk) return HASTE_OK;
    if (!m.tk_fused) return run_topk(bce, a.Z32, d->B, d->L, ws, m.cand, st);
    const int64_t ng = n_groups(d);
    float *mid_v = (float *)(a.tk_i + ng * pad_rows(d->B));
    int32_t *mid_i = (int32_t *)(mid_v + (int64_t)d->B * topk_gm_segments(ng, d->B).nseg * bce->topk);
    TRY_HIP(launch_topk_group_major(a.tk_v, a.tk_i, pad_rows(d->B), d->B, ng, bce->topk, mid_v, mid_i,
                                    bce->topk_val, bce->topk_idx, st),
            "top-K merge");
    if (topk_exact_fused(d, bce))
        TRY_HIP(launch_topk_refine((const unsigned short *)X, d->B, d->D, a.W, a.idxp, a.perm, d->G, d->F,
                                   d->L, bce->label_offset, bce->topk, bce->topk_val, bce->topk_idx, st),
                "top-K refine");
    return HASTE_OK;
}

haste_status zero_dx(float *dX, int B, int D, int accumulate, hipStream_t st) {
    if (!accumulate) TRY_HIP(launch_fill_u32(dX, 0u, (size_t)B * D, st), "zero dX");
    return HASTE_OK;
}

// common argument checks of tail compute calls
// bf16 with G = 1 (per-label fan-in) has the forward and the one-call step
haste_status not_g1(const haste_tail_desc *d) {
    if (d->dtype == HASTE_BF16 && d->G == 1)
        return fail(HASTE_ERR_UNSUPPORTED, "bf16 with G = 1 supports haste_tail_fwd and haste_tail_step only");
    return HASTE_OK;
}

haste_status tail_common(const haste_tail_desc *d, const void *X, const int32_t *idx,
                         const void *W) {
    TRY(check_tail(d));
    const size_t al = d->dtype == HASTE_BF16 ? 16 : 4;
    TRY(need_al(X, al, "X"));
    TRY(need_al(idx, 4, "idx"));
    TRY(need_al(W, al, "W"));
    return HASTE_OK;
}

}  // namespace

// =================================================================== C ABI
extern "C" {

int haste_abi_version(void) { return HASTE_ABI_VERSION; }

const char *haste_status_string(int s) {
    switch (s) {
    case HASTE_OK: return "ok";
    case HASTE_ERR_INVALID: return "invalid argument";
    case HASTE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case HASTE_ERR_WORKSPACE: return "workspace missing or too small";
    case HASTE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *haste_last_error(void) { return g_err.c_str(); }

haste_status haste_tail_layout(const haste_tail_desc *d, int64_t *out) {
    g_err.clear();
    if (!d) return fail(HASTE_ERR_INVALID, "tail descriptor is NULL");
    if (!out) return fail(HASTE_ERR_INVALID, "out is NULL");
    if (d->L < 1 || d->G < 1 || d->F < 1) return fail(HASTE_ERR_INVALID, "L, G, F must be >= 1");
    const int64_t ng = n_groups(d);
    out[0] = ng;
    out[1] = ng * d->F;
    out[2] = ng * d->G;
    out[3] = d->L - (ng - 1) * d->G;
    return HASTE_OK;
}

size_t haste_tail_workspace_bytes(const haste_tail_desc *d, const haste_bce *bce) {
    if (check_tail(d) != HASTE_OK) return 0;
    return tail_ws(d, bce).total;
}

size_t haste_tail_fwd_workspace_bytes(const haste_tail_desc *d, const haste_bce *bce) {
    if (check_tail(d) != HASTE_OK) return 0;
    return tail_ws(d, bce).fwd_total;
}

haste_status haste_tail_prepare_layout(const haste_tail_desc *d, const int32_t *idx, void *ws,
                                       size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(check_tail(d));
    TRY(need_al(idx, 4, "idx"));
    if (d->dtype != HASTE_BF16 || d->G == 1) return HASTE_OK;   // no feature order on these paths
    const TailWs m = tail_ws(d, nullptr);
    TRY(check_ws(ws, ws_bytes, m.fwd_total));
    haste_tail_desc dd = *d;
    dd.flags &= ~HASTE_TAIL_LAYOUT_READY;
    return feature_order(&dd, idx, ws, m, S(stream));
}

size_t haste_head_workspace_bytes(const haste_head_desc *d, const haste_bce *bce) {
    (void)bce;
    if (check_head(d) != HASTE_OK) return 0;
    return head_ws(d, bce).total;
}

haste_status haste_tail_fwd(const haste_tail_desc *d, const void *X, const int32_t *idx,
                            const void *W, void *Z, const haste_bce *bce, void *ws,
                            size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(tail_common(d, X, idx, W));
    TRY(check_bce(bce, d->B, true, d->L));
    if (!Z && !bce) return fail(HASTE_ERR_INVALID, "nothing to compute: Z and bce are both NULL");
    if (Z && !aligned(Z, d->dtype == HASTE_BF16 ? 2 : 4)) return fail(HASTE_ERR_INVALID, "Z misaligned");
    const TailWs m = tail_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, m.fwd_total));
    hipStream_t st = S(stream);
    if (d->dtype == HASTE_BF16 && d->G == 1) {
        if (m.has_topk) return fail(HASTE_ERR_UNSUPPORTED, "no top-K with G = 1");
        TRY(bf16_prep(d, X, bce, ws, m, st));
        TailArgs a = tail_args(d, X, idx, W, ws, m);
        a.tk_off = bce ? bce->label_offset : 0;
        a.Z = (unsigned short *)Z;
        if (bce) {
            a.loss = bce->loss;
            a.s = bce->grad_scale;
        }
        TRY_HIP(launch_fanin1_fwd(a, Z != nullptr, bce && bce->loss, st), "tail fwd (G = 1)");
    } else if (d->dtype == HASTE_BF16) {
        TRY(bf16_prep(d, X, bce, ws, m, st));
        TailArgs a = tail_args(d, X, idx, W, ws, m);
        a.tk_off = bce ? bce->label_offset : 0;
        a.Z = (unsigned short *)Z;
        if (bce) {
            a.loss = bce->loss;
            a.s = bce->grad_scale;
        }
        TRY(feature_order(d, idx, ws, m, st));
        TRY_HIP(launch_tail_t1(T1_FWD, d->G, a, Z != nullptr, bce && bce->loss, st), "tail fwd");
        TRY(tail_topk(d, X, bce, m, a, ws, st));
    } else {
        F32Args a = f32_tail_args(d, X, idx, W, bce);
        a.Z = Z ? (float *)Z : m.has_topk ? (float *)B8(ws, m.z32) : nullptr;
        TRY_HIP(launch_f32_tail_logits(a, a.Z != nullptr, bce != nullptr, bce && bce->loss, st),
                "tail fwd f32");
        if (m.has_topk) TRY(run_topk(bce, a.Z, d->B, d->L, ws, m.cand, st));
    }
    return HASTE_OK;
}

haste_status haste_tail_bwd(const haste_tail_desc *d, const void *X, const int32_t *idx,
                            const void *W, const void *dZ, const haste_bce *bce, void *dW,
                            float *dX, int accumulate_dX, void *ws, size_t ws_bytes,
                            void *stream) {
    g_err.clear();
    TRY(tail_common(d, X, idx, W));
    TRY(not_g1(d));
    if (!dZ && !bce) return fail(HASTE_ERR_INVALID, "need dZ or bce to form the gradient");
    if (!dZ) TRY(check_bce(bce, d->B, false, d->L));
    TRY(need_al(dW, d->dtype == HASTE_BF16 ? 8 : 4, "dW"));
    TRY(need_al(dX, 4, "dX"));
    if (dZ && !aligned(dZ, d->dtype == HASTE_BF16 ? 2 : 4)) return fail(HASTE_ERR_INVALID, "dZ misaligned");
    const haste_bce *b = dZ ? nullptr : bce;
    const TailWs m = tail_ws(d, b);
    TRY(check_ws(ws, ws_bytes, m.total));
    hipStream_t st = S(stream);
    TRY(zero_dx(dX, d->B, d->D, accumulate_dX, st));
    if (d->dtype == HASTE_BF16) {
        TRY(bf16_prep(d, X, b, ws, m, st));
        TailArgs a = tail_args(d, X, idx, W, ws, m);
        a.dW = (unsigned short *)dW;
        a.dX = dX;
        a.dZ = (const unsigned short *)dZ;
        if (b) a.s = b->grad_scale;
        TRY(feature_order(d, idx, ws, m, st));
        if (dZ && a.dzt)   // the given dZ in the tile layout: both passes then read it coalesced
            TRY_HIP(launch_dz_tiles((const unsigned short *)dZ, d->B, d->L, d->G, a.Bp, a.Ng, a.dzt, st),
                    "dZ tiles");
        TRY_HIP(launch_tail_t1(dZ ? T1_DW_MEM : T1_DW_BCE, d->G, a, false, false, st), "tail dW");
        TRY_HIP(launch_tail_t2(d->G, a.dzt ? 2 : dZ ? 1 : 0, a, st), "tail dX");
    } else {
        F32Args a = f32_tail_args(d, X, idx, W, b);
        a.loss = nullptr;
        a.dW = (float *)dW;
        a.dX = dX;
        if (dZ) {
            a.dZ = (float *)dZ;
        } else {
            a.dZ = (float *)B8(ws, m.dz);
            TRY_HIP(launch_f32_tail_logits(a, false, true, false, st), "tail dz f32");
        }
        TRY_HIP(launch_f32_tail_dw(a, st), "tail dW f32");
        TRY_HIP(launch_f32_tail_dx(a, st), "tail dX f32");
    }
    return HASTE_OK;
}

haste_status haste_tail_step(const haste_tail_desc *d, const void *X, const int32_t *idx,
                             const void *W, const haste_bce *bce, void *dW, float *dX,
                             int accumulate_dX, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(tail_common(d, X, idx, W));
    const bool g1 = d->dtype == HASTE_BF16 && d->G == 1;
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->L));
    TRY(need_al(dW, d->dtype == HASTE_BF16 ? (g1 ? 2 : 8) : 4, "dW"));
    TRY(need_al(dX, 4, "dX"));
    const TailWs m = tail_ws(d, bce);
    if (g1) {
        if (m.has_topk) return fail(HASTE_ERR_UNSUPPORTED, "no top-K with G = 1");
        if (d->flags & HASTE_TAIL_LEAN)
            return fail(HASTE_ERR_UNSUPPORTED, "the G = 1 step keeps dz; HASTE_TAIL_LEAN is not taken");
        if (!fanin1_step_supported(d->F, d->D))
            return fail(HASTE_ERR_UNSUPPORTED, "the G = 1 step takes F in {32,64,128} and D <= 960 (F=%d D=%d)",
                        d->F, d->D);
    }
    TRY(check_ws(ws, ws_bytes, m.total));
    hipStream_t st = S(stream);
    TRY(zero_dx(dX, d->B, d->D, accumulate_dX, st));
    if (g1) {
        TRY(bf16_prep(d, X, bce, ws, m, st));
        TailArgs a = tail_args(d, X, idx, W, ws, m);
        a.tk_off = bce->label_offset;
        a.dW = (unsigned short *)dW;
        a.dX = dX;
        a.s = bce->grad_scale;
        a.loss = bce->loss;
        TRY_HIP(launch_fanin1_step(a, bce->loss != nullptr, st), "tail step (G = 1)");
    } else if (d->dtype == HASTE_BF16) {
        TRY(bf16_prep(d, X, bce, ws, m, st));
        TailArgs a = tail_args(d, X, idx, W, ws, m);
        a.tk_off = bce ? bce->label_offset : 0;
        a.dW = (unsigned short *)dW;
        a.dX = dX;
        a.s = bce->grad_scale;
        a.loss = bce->loss;
        TRY(feature_order(d, idx, ws, m, st));
        TRY_HIP(launch_tail_t1(T1_DW_BCE, d->G, a, false, bce->loss != nullptr, st), "tail step dW");
        TRY(tail_topk(d, X, bce, m, a, ws, st));
        TRY_HIP(launch_tail_t2(d->G, a.dzt ? 2 : 0, a, st), "tail step dX");
    } else {
        F32Args a = f32_tail_args(d, X, idx, W, bce);
        a.dW = (float *)dW;
        a.dX = dX;
        a.dZ = (float *)B8(ws, m.dz);
        a.Z = m.has_topk ? (float *)B8(ws, m.z32) : nullptr;
        TRY_HIP(launch_f32_tail_logits(a, m.has_topk, true, bce->loss != nullptr, st), "tail step f32");
        if (m.has_topk) TRY(run_topk(bce, a.Z, d->B, d->L, ws, m.cand, st));
        TRY_HIP(launch_f32_tail_dw(a, st), "tail dW f32");
        TRY_HIP(launch_f32_tail_dx(a, st), "tail dX f32");
    }
    return HASTE_OK;
}

haste_status haste_tail_step_sgd(const haste_tail_desc *d, const void *X, const int32_t *idx,
                                 const void *W, const haste_bce *bce, float lr, void *W_out,
                                 float *dX, int accumulate_dX, void *ws, size_t ws_bytes,
                                 void *stream) {
    g_err.clear();
    TRY(tail_common(d, X, idx, W));
    TRY(not_g1(d));
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->L));
    TRY(need_al(W_out, 16, "W_out"));
    TRY(need_al(dX, 4, "dX"));
    if (d->dtype != HASTE_BF16)
        return fail(HASTE_ERR_UNSUPPORTED, "the fused SGD step is a bf16 path; fp32 takes "
                                           "haste_tail_step + haste_sgd_update");
    if (!(lr == lr)) return fail(HASTE_ERR_INVALID, "lr is NaN");
    const size_t wbytes = (size_t)n_groups(d) * d->G * d->F * 2;
    const char *w0 = (const char *)W, *o0 = (const char *)W_out;
    if (o0 < w0 + wbytes && w0 < o0 + wbytes)
        return fail(HASTE_ERR_INVALID, "W_out overlaps W (the dX pass reads W after the update is written)");
    const TailWs m = tail_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, m.total));
    hipStream_t st = S(stream);
    TRY(zero_dx(dX, d->B, d->D, accumulate_dX, st));
    TRY(bf16_prep(d, X, bce, ws, m, st));
    TailArgs a = tail_args(d, X, idx, W, ws, m);
    a.tk_off = bce->label_offset;
    a.Wout = (unsigned short *)W_out;
    a.lr = lr;
    a.dX = dX;
    a.s = bce->grad_scale;
    a.loss = bce->loss;
    TRY(feature_order(d, idx, ws, m, st));
    TRY_HIP(launch_tail_t1(T1_DW_BCE, d->G, a, false, bce->loss != nullptr, st), "tail SGD step dW");
    TRY(tail_topk(d, X, bce, m, a, ws, st));
    TRY_HIP(launch_tail_t2(d->G, a.dzt ? 2 : 0, a, st), "tail SGD step dX");
    return HASTE_OK;
}

haste_status haste_sgd_update(int64_t n, int32_t dtype, const void *W, const void *dW, float lr,
                              void *W_out, void *stream) {
    g_err.clear();
    if (n < 0) return fail(HASTE_ERR_INVALID, "n < 0");
    if (dtype != HASTE_BF16 && dtype != HASTE_F32) return fail(HASTE_ERR_INVALID, "dtype %d", dtype);
    if (n == 0) return HASTE_OK;
    const size_t es = dtype == HASTE_BF16 ? 2 : 4;
    TRY(need_al(W, es, "W"));
    TRY(need_al(dW, es, "dW"));
    TRY(need_al(W_out, es, "W_out"));
    TRY_HIP(launch_sgd(W, dW, lr, W_out, n, dtype == HASTE_BF16, S(stream)), "SGD update");
    return HASTE_OK;
}

haste_status haste_tail_rewire(const haste_tail_desc *d, const int32_t *idx, const void *W,
                               int32_t k_prune, const int32_t *cand, int32_t n_cand,
                               int32_t *idx_out, void *W_out, void *stream) {
    g_err.clear();
    if (!d) return fail(HASTE_ERR_INVALID, "tail descriptor is NULL");
    if (d->D < 1 || d->L < 1 || d->G < 1 || d->F < 1)
        return fail(HASTE_ERR_INVALID, "tail sizes must be >= 1 (D=%d L=%lld G=%d F=%d)", d->D,
                    (long long)d->L, d->G, d->F);
    if (d->F > d->D) return fail(HASTE_ERR_INVALID, "F=%d exceeds D=%d", d->F, d->D);
    if (d->dtype != HASTE_BF16 && d->dtype != HASTE_F32) return fail(HASTE_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (!rewire_supported(d->G, d->F, d->D))
        return fail(HASTE_ERR_UNSUPPORTED, "rewiring takes G <= 64, F <= 256 and D <= 65536 (G=%d F=%d D=%d)",
                    d->G, d->F, d->D);
    if (k_prune < 0 || k_prune > d->F) return fail(HASTE_ERR_INVALID, "k_prune=%d outside [0, F=%d]", k_prune, d->F);
    if (n_cand < 0) return fail(HASTE_ERR_INVALID, "n_cand < 0");
    const int64_t ng = n_groups(d);
    if (ng > 0x7fffffffLL) return fail(HASTE_ERR_UNSUPPORTED, "more than 2^31 - 1 groups");
    const size_t es = d->dtype == HASTE_BF16 ? 2 : 4;
    TRY(need_al(idx, 4, "idx"));
    TRY(need_al(W, es, "W"));
    TRY(need_al(idx_out, 4, "idx_out"));
    TRY(need_al(W_out, es, "W_out"));
    if (n_cand > 0) TRY(need_al(cand, 4, "cand"));
    const size_t ibytes = (size_t)ng * d->F * 4, wbytes = (size_t)ng * d->G * d->F * es;
    const char *i0 = (const char *)idx, *io = (const char *)idx_out;
    const char *w0 = (const char *)W, *wo = (const char *)W_out;
    if (io != i0 && io < i0 + ibytes && i0 < io + ibytes)
        return fail(HASTE_ERR_INVALID, "idx_out overlaps idx without being it");
    if (wo != w0 && wo < w0 + wbytes && w0 < wo + wbytes)
        return fail(HASTE_ERR_INVALID, "W_out overlaps W without being it");
    TRY_HIP(launch_rewire(idx, W, d->dtype == HASTE_BF16, ng, d->G, d->F, d->D, d->L, k_prune, cand,
                          n_cand, idx_out, W_out, S(stream)),
            "rewire");
    return HASTE_OK;
}

haste_status haste_tail_prepare(const haste_tail_desc *d, const void *X, const haste_bce *bce,
                                void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(check_tail(d));
    TRY(not_g1(d));
    TRY(need_al(X, d->dtype == HASTE_BF16 ? 16 : 4, "X"));
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->L));
    const TailWs m = tail_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, m.total));
    if (d->dtype == HASTE_BF16) TRY(bf16_prep(d, X, bce, ws, m, S(stream)));
    return HASTE_OK;  // the fp32 path needs no preparation
}

haste_status haste_tail_step_dw(const haste_tail_desc *d, const void *X, const int32_t *idx,
                                const void *W, const haste_bce *bce, void *dW, void *ws,
                                size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(tail_common(d, X, idx, W));
    TRY(not_g1(d));
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->L));
    TRY(need_al(dW, d->dtype == HASTE_BF16 ? 8 : 4, "dW"));
    const TailWs m = tail_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, m.total));
    hipStream_t st = S(stream);
    if (d->dtype == HASTE_BF16) {
        TailArgs a = tail_args(d, X, idx, W, ws, m);
        a.tk_off = bce ? bce->label_offset : 0;
        a.dW = (unsigned short *)dW;
        a.s = bce->grad_scale;
        a.loss = bce->loss;
        TRY(feature_order(d, idx, ws, m, st));
        TRY_HIP(launch_tail_t1(T1_DW_BCE, d->G, a, false, bce->loss != nullptr, st), "tail step dW");
        TRY(tail_topk(d, X, bce, m, a, ws, st));
    } else {
        F32Args a = f32_tail_args(d, X, idx, W, bce);
        a.dW = (float *)dW;
        a.dZ = (float *)B8(ws, m.dz);
        a.Z = m.has_topk ? (float *)B8(ws, m.z32) : nullptr;
        TRY_HIP(launch_f32_tail_logits(a, m.has_topk, true, bce->loss != nullptr, st), "tail step f32");
        if (m.has_topk) TRY(run_topk(bce, a.Z, d->B, d->L, ws, m.cand, st));
        TRY_HIP(launch_f32_tail_dw(a, st), "tail dW f32");
    }
    return HASTE_OK;
}

haste_status haste_tail_step_dx(const haste_tail_desc *d, const void *X, const int32_t *idx,
                                const void *W, const haste_bce *bce, float *dX,
                                int accumulate_dX, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(tail_common(d, X, idx, W));
    TRY(not_g1(d));
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->L));
    TRY(need_al(dX, 4, "dX"));
    const TailWs m = tail_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, m.total));
    hipStream_t st = S(stream);
    TRY(zero_dx(dX, d->B, d->D, accumulate_dX, st));
    if (d->dtype == HASTE_BF16) {
        TailArgs a = tail_args(d, X, idx, W, ws, m);
        a.dX = dX;
        a.s = bce->grad_scale;
        TRY_HIP(launch_tail_t2(d->G, a.dzt ? 2 : 0, a, st), "tail step dX");
    } else {
        F32Args a = f32_tail_args(d, X, idx, W, bce);
        a.loss = nullptr;
        a.dX = dX;
        a.dZ = (float *)B8(ws, m.dz);
        TRY_HIP(launch_f32_tail_dx(a, st), "tail dX f32");
    }
    return HASTE_OK;
}

// ------------------------------------------------------------------- head
namespace {

haste_status head_common(const haste_head_desc *d, const void *X, const void *Wh) {
    TRY(check_head(d));
    const size_t al = d->dtype == HASTE_BF16 ? 16 : 4;
    TRY(need_al(X, al, "X"));
    TRY(need_al(Wh, al, "Wh"));
    return HASTE_OK;
}

// logits + (optional) BCE.  dz_out: where dz goes (NULL: nowhere).
haste_status head_logits(const haste_head_desc *d, const void *X, const void *Wh, void *Zh,
                         const haste_bce *bce, bool want_loss, void *dz_out, void *ws,
                         const HeadWs &m, hipStream_t st) {
    if (d->dtype == HASTE_BF16) {
        GemmArgs g{};
        g.A = (const unsigned short *)X;
        g.Bm = (const unsigned short *)Wh;
        g.M = d->B;
        g.N = d->H;
        g.K = d->D;
        g.lda = d->D;
        g.ldb = d->D;
        g.k_split = d->D;
        g.Zout = (unsigned short *)Zh;
        if (bce) {
            if (gemm2_shape(g)) {   // the GEMM reads the positives per tile
                g.pos_ptr = bce->row_ptr;
                g.pos_lab = bce->labels;
                g.pos_off = bce->label_offset;
                g.pos_nnz = bce->nnz;
            } else {
                TRY_HIP(launch_head_bitmap(bce->row_ptr, bce->labels, bce->nnz, d->B, bce->label_offset,
                                           d->H, (uint32_t *)B8(ws, m.bm), m.words, st),
                        "head bitmap");
                g.bitmap = (const uint32_t *)B8(ws, m.bm);
                g.bm_words = m.words;
            }
            g.s = bce->grad_scale;
            g.loss = want_loss ? bce->loss : nullptr;
            g.dZout = (unsigned short *)dz_out;
            if (m.has_topk) g.Z32 = (float *)B8(ws, m.z32);
        }
        TRY_HIP(launch_gemm(true, true, EPI_BCE, g, st), "head logits");
        if (bce && m.has_topk) TRY(run_topk(bce, g.Z32, d->B, d->H, ws, m.cand, st));
    } else {
        F32Args a{};
        a.X = (const float *)X;
        a.W = (const float *)Wh;
        a.Z = (float *)Zh;
        a.B = d->B;
        a.D = d->D;
        a.L = d->H;
        if (bce) {
            a.row_ptr = bce->row_ptr;
            a.labels = bce->labels;
            a.label_offset = bce->label_offset;
            a.s = bce->grad_scale;
            a.loss = want_loss ? bce->loss : nullptr;
            a.dZ = (float *)dz_out;
        }
        if (!a.Z && bce && m.has_topk) a.Z = (float *)B8(ws, m.z32);
        TRY_HIP(launch_f32_head_logits(a, a.Z != nullptr, bce != nullptr, want_loss, st),
                "head logits f32");
        if (bce && m.has_topk) TRY(run_topk(bce, a.Z, d->B, d->H, ws, m.cand, st));
    }
    return HASTE_OK;
}

haste_status head_grads(const haste_head_desc *d, const void *X, const void *Wh, const void *dz,
                        void *dWh, float *dX, hipStream_t st) {
    if (d->dtype == HASTE_BF16) {
        GemmArgs g{};  // dWh[h][d] = sum_b dz[b][h] X[b][d]
        g.A = (const unsigned short *)dz;
        g.Bm = (const unsigned short *)X;
        g.M = d->H;
        g.N = d->D;
        g.K = d->B;
        g.lda = d->H;
        g.ldb = d->D;
        g.k_split = d->B;
        g.C16 = (unsigned short *)dWh;
        TRY_HIP(launch_gemm(false, false, EPI_STORE16, g, st), "head dW");
        GemmArgs x{};  // dX[b][d] += sum_h dz[b][h] Wh[h][d]
        x.A = (const unsigned short *)dz;
        x.Bm = (const unsigned short *)Wh;
        x.M = d->B;
        x.N = d->D;
        x.K = d->H;
        x.lda = d->H;
        x.ldb = d->D;
        x.C32 = dX;
        // split K so that about 256 (64-row) tiles run, each split adding
        // its partial sums with fp32 atomics
        const int tiles = ((d->B + 63) / 64) * ((d->D + 127) / 128);
        int splits = (256 + tiles - 1) / tiles;
        int ks = (d->H + splits - 1) / splits;
        ks = (ks + 63) / 64 * 64;
        if (ks < 256) ks = 256;
        x.k_split = ks;
        TRY_HIP(launch_gemm(true, false, EPI_ATOMIC32, x, st), "head dX");
    } else {
        F32Args a{};
        a.X = (const float *)X;
        a.W = (const float *)Wh;
        a.dZ = (float *)dz;
        a.dW = (float *)dWh;
        a.dX = dX;
        a.B = d->B;
        a.D = d->D;
        a.L = d->H;
        TRY_HIP(launch_f32_head_dw(a, st), "head dW f32");
        TRY_HIP(launch_f32_head_dx(a, st), "head dX f32");
    }
    return HASTE_OK;
}

}  // namespace

haste_status haste_head_fwd(const haste_head_desc *d, const void *X, const void *Wh, void *Zh,
                            const haste_bce *bce, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(head_common(d, X, Wh));
    TRY(check_bce(bce, d->B, true, d->H));
    if (!Zh && !bce) return fail(HASTE_ERR_INVALID, "nothing to compute: Zh and bce are both NULL");
    const HeadWs m = head_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, bce ? m.total : 0));
    return head_logits(d, X, Wh, Zh, bce, bce && bce->loss, nullptr, ws, m, S(stream));
}

haste_status haste_head_bwd(const haste_head_desc *d, const void *X, const void *Wh,
                            const void *dZh, const haste_bce *bce, void *dWh, float *dX,
                            int accumulate_dX, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(head_common(d, X, Wh));
    if (!dZh && !bce) return fail(HASTE_ERR_INVALID, "need dZh or bce to form the gradient");
    if (!dZh) TRY(check_bce(bce, d->B, false, d->H));
    TRY(need_al(dWh, d->dtype == HASTE_BF16 ? 2 : 4, "dWh"));
    TRY(need_al(dX, 4, "dX"));
    if (dZh && !aligned(dZh, 16)) return fail(HASTE_ERR_INVALID, "dZh is not 16-byte aligned");
    const HeadWs m = head_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, dZh ? 0 : m.total));
    hipStream_t st = S(stream);
    TRY(zero_dx(dX, d->B, d->D, accumulate_dX, st));
    const void *dz = dZh;
    if (!dz) {
        TRY(head_logits(d, X, Wh, nullptr, bce, false, B8(ws, m.dz), ws, m, st));
        dz = B8(ws, m.dz);
    }
    return head_grads(d, X, Wh, dz, dWh, dX, st);
}

// ------------------------------------------- the entry point that allocates nothing
// Its workspace is this file-scope device array (each GPU holds its own
// copy, from module load until the process ends).  In host code `scratch`
// names a host-side stand-in, not device memory: the device address comes
// from hipGetSymbolAddress, taken once per device with that device current,
// and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[HASTE_HEAD_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

haste_status scratch_ptr(void **out) {
    int dev = -1;
    TRY_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(HASTE_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p) return fail(HASTE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return HASTE_OK;
}
}  // namespace

haste_status haste_head_step_noalloc(const haste_head_desc *d, const void *X, const void *Wh,
                                     const haste_bce *bce, void *dWh, float *dX, int accumulate_dX,
                                     void *stream) {
    g_err.clear();
    TRY(head_common(d, X, Wh));
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->H));
    const size_t need_bytes = head_ws(d, bce).total;
    if (need_bytes > HASTE_HEAD_SCRATCH_BYTES)
        return fail(HASTE_ERR_WORKSPACE, "this head step needs %zu workspace bytes; the static scratch holds %zu",
                    need_bytes, (size_t)HASTE_HEAD_SCRATCH_BYTES);
    void *ws = nullptr;
    TRY(scratch_ptr(&ws));
    return haste_head_step(d, X, Wh, bce, dWh, dX, accumulate_dX, ws, HASTE_HEAD_SCRATCH_BYTES, stream);
}

haste_status haste_head_step(const haste_head_desc *d, const void *X, const void *Wh,
                             const haste_bce *bce, void *dWh, float *dX, int accumulate_dX,
                             void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(head_common(d, X, Wh));
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->H));
    TRY(need_al(dWh, d->dtype == HASTE_BF16 ? 2 : 4, "dWh"));
    TRY(need_al(dX, 4, "dX"));
    const HeadWs m = head_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, m.total));
    hipStream_t st = S(stream);
    TRY(zero_dx(dX, d->B, d->D, accumulate_dX, st));
    TRY(head_logits(d, X, Wh, nullptr, bce, bce->loss != nullptr, B8(ws, m.dz), ws, m, st));
    return head_grads(d, X, Wh, B8(ws, m.dz), dWh, dX, st);
}

// -------------------------------------------------------------- utilities
haste_status haste_tail_group_positives(const haste_tail_desc *d, const haste_bce *bce,
                                        int32_t *grp_ptr, int32_t *entries, void *ws,
                                        size_t ws_bytes, void *stream) {
    g_err.clear();
    TRY(check_tail(d));
    TRY(need(bce, "bce"));
    TRY(check_bce(bce, d->B, true, d->L));   // top-K settings do not matter here
    TRY(need_al(grp_ptr, 4, "grp_ptr"));
    if (bce->nnz > 0) TRY(need_al(entries, 4, "entries"));
    const TailWs m = tail_ws(d, bce);
    TRY(check_ws(ws, ws_bytes, m.total));
    TRY_HIP(launch_group_positives(bce->row_ptr, bce->labels, bce->nnz, d->B, bce->label_offset,
                                   d->L, d->G, n_groups(d), (long long *)B8(ws, m.cnt), grp_ptr,
                                   entries, S(stream)),
            "group positives");
    return HASTE_OK;
}

haste_status haste_probe_mfma(int blocks, int iters, float *sink, void *stream) {
    g_err.clear();
    if (blocks < 1 || iters < 1) return fail(HASTE_ERR_INVALID, "blocks and iters must be >= 1");
    TRY(need_al(sink, 4, "sink"));
    TRY_HIP(launch_probe_mfma(blocks, iters, sink, S(stream)), "MFMA probe");
    return HASTE_OK;
}

haste_status haste_tail_validate(const haste_tail_desc *d, const int32_t *idx,
                                 int32_t *first_bad_group, void *stream) {
    g_err.clear();
    if (!d) return fail(HASTE_ERR_INVALID, "tail descriptor is NULL");
    if (d->L < 1 || d->G < 1 || d->F < 1 || d->D < 1) return fail(HASTE_ERR_INVALID, "bad sizes");
    TRY(need_al(idx, 4, "idx"));
    TRY(need_al(first_bad_group, 4, "first_bad_group"));
    TRY_HIP(launch_validate(idx, n_groups(d), d->F, d->D, first_bad_group, S(stream)), "validate");
    return HASTE_OK;
}

// ------------------------------------------------------ top-K parameters
// Expected min(X, K') for X the number of the K largest of n items that land
// in a bucket of m items under a uniformly random placement: X is
// hypergeometric, P(X = x) = C(m, x) C(n - m, K - x) / C(n, K); with K <= 8
// every product below has at most eight factors.
static double topk_bucket_expect(int64_t n, int K, int kp, int64_t m) {
    double e = 0.0;
    for (int x = 1; x <= K && x <= m; ++x) {
        if (K - x > n - m) continue;
        double p = 1.0;
        for (int i = 0; i < x; ++i) p *= (double)(m - i) / (double)(x - i);        // C(m, x)
        for (int i = 0; i < K - x; ++i) p *= (double)(n - m - i) / (double)(K - x - i);  // C(n-m, K-x)
        for (int i = 0; i < K; ++i) p *= (double)(K - i) / (double)(n - i);        // / C(n, K)
        e += p * (double)(x < kp ? x : kp);
    }
    return e;
}

// Expected recall for buckets of seg consecutive items (the last one shorter)
static double topk_recall_seg(int64_t n, int K, int kp, int64_t seg) {
    const int64_t nseg = (n + seg - 1) / seg, last = n - (nseg - 1) * seg;
    if (K >= n)   // all n items are the top; a bucket keeps min(its size, K') of them
        return ((double)(nseg - 1) * (double)(seg < kp ? seg : kp) + (double)(last < kp ? last : kp)) /
               (double)n;
    const double s = (double)(nseg - 1) * topk_bucket_expect(n, K, kp, seg) +
                     topk_bucket_expect(n, K, kp, last);
    return s / (double)K;
}

double haste_topk_expected_recall(int64_t n, int K, int kprime, int64_t buckets) {
    if (n < 1 || K < 1 || K > 8 || kprime < 1 || kprime > K || buckets < 1) return -1.0;
    const int64_t seg = topk_buckets(n, buckets, 1).seg_len;
    return topk_recall_seg(n, K, kprime, seg);
}

haste_status haste_topk_plan(int64_t n, int K, double target, int64_t min_buckets, int32_t *out) {
    g_err.clear();
    if (!out) return fail(HASTE_ERR_INVALID, "out is NULL");
    if (n < 1 || K < 1 || K > 8) return fail(HASTE_ERR_INVALID, "n=%lld K=%d", (long long)n, K);
    if (!(target > 0.0 && target <= 1.0)) return fail(HASTE_ERR_INVALID, "target %g outside (0, 1]", target);
    const int64_t bmax = n < 65535 ? n : 65535;
    if (min_buckets < 1 || min_buckets > bmax)
        return fail(HASTE_ERR_INVALID, "min_buckets=%lld outside [1, %lld]", (long long)min_buckets, (long long)bmax);
    int64_t best_cost = -1;
    for (int kp = 1; kp <= K; ++kp) {
        // smallest bucket count reaching the target; counts with the same
        // bucket length give the same buckets, so each length is tried once
        int64_t prev_seg = -1;
        for (int64_t b = min_buckets; b <= bmax; ++b) {
            if (best_cost >= 0 && b * kp >= best_cost) break;   // cannot beat the best
            const int64_t seg = (n + b - 1) / b;
            if (seg == prev_seg) continue;
            prev_seg = seg;
            if (topk_recall_seg(n, K, kp, seg) >= target) {
                best_cost = b * kp;
                out[0] = kp;
                out[1] = (int32_t)b;
                break;
            }
        }
    }
    if (best_cost < 0) return fail(HASTE_ERR_UNSUPPORTED, "no K' <= %d and at most %lld buckets reach recall %g",
                                   K, (long long)bmax, target);
    return HASTE_OK;
}

haste_status haste_topk_merge(int32_t B, int32_t K, const float *a_val, const int32_t *a_idx,
                              const float *b_val, const int32_t *b_idx, float *out_val,
                              int32_t *out_idx, void *stream) {
    g_err.clear();
    if (B < 0 || K < 1 || K > 64) return fail(HASTE_ERR_INVALID, "need B >= 0 and 1 <= K <= 64");
    TRY(need(a_val, "a_val"));
    TRY(need(a_idx, "a_idx"));
    TRY(need(b_val, "b_val"));
    TRY(need(b_idx, "b_idx"));
    TRY(need(out_val, "out_val"));
    TRY(need(out_idx, "out_idx"));
    TRY_HIP(launch_topk_merge(B, K, a_val, a_idx, b_val, b_idx, out_val, out_idx, S(stream)),
            "topk merge");
    return HASTE_OK;
}

}  // extern "C"
