/*
 * haste.h -- C ABI of the MI355X (gfx950) group-shared fixed fan-in output
 * layer: a sparse "tail" over many rare labels plus a dense "head" over the
 * frequent ones, with a fused sigmoid binary cross-entropy over sparse
 * positives.  One shared library, libhaste.so; HIP kernels only.
 *
 * The method (HASTE summary page, gist.science, "HASTE: Hardware-Aware
 * Dynamic Sparse Training for Large Output Spaces"):
 *   - section "Method", item 1 (group-shared fixed fan-in): tail labels are
 *     split into groups of G; every label of group g reads the same F input
 *     features idx[g][0..F) but owns its weights.  The group's features are
 *     gathered once into on-chip memory and reused by all G labels through a
 *     dense matrix-core contraction; indices are stored once per group.
 *   - section "Method", item 2 (head-tail decomposition): the frequent head
 *     labels use a standard dense classifier.
 * The loss and the backward formulas are not printed on the pages; this
 * library computes the exact gradients of
 *   z[b][t] = sum_f X[b][idx[t/G][f]] * W[t][f]            (tail)
 *   zh[b][h] = sum_d X[b][d] * Wh[h][d]                    (head)
 *   loss = s * sum_{b,label} softplus(z) - y*z,  dz = s * (sigmoid(z) - y)
 * with y = 1 exactly at the listed positives.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers (hipMalloc / torch CUDA
 *     memory) unless a parameter says "host".  The caller owns every buffer,
 *     including the workspace; the library never allocates, keeps no state
 *     between calls and is safe to call from several host threads.
 *   - Every call only enqueues work on `stream` (a hipStream_t, or NULL for
 *     the default stream) and never synchronises.
 *   - Layouts are row-major and densely packed:
 *       X   : B x D                 (dtype)
 *       idx : N_g x F  int32, N_g = ceil(L/G); each row strictly increasing,
 *                      values in [0, D)
 *       W   : (N_g*G) x F           (dtype) label-major: row t = g*G + j is
 *                      label t's weights over idx[g][0..F).  Rows t >= L
 *                      (padding of a ragged last group) are never read for
 *                      a result and their gradient rows are written as 0.
 *       Z,dZ: B x L                 (dtype), tail label t in column t
 *       Wh  : H x D                 (dtype)  Zh, dZh: B x H (dtype)
 *       dX  : B x D  float32
 *   - dtype HASTE_BF16: inputs are bf16, products accumulate in fp32 on the
 *     matrix cores (MFMA), dz is rounded to bf16 before it feeds the backward
 *     contractions, bf16 outputs are rounded to nearest even.
 *     dtype HASTE_F32: fp32 throughout (VALU kernels; small problems).
 *   - Errors: arguments are checked on the host before anything is
 *     enqueued; a failing check returns a status and enqueues nothing.
 *     Index contents are not checked by the compute calls (an index outside
 *     [0, D) reads or writes out of bounds); check them once with
 *     haste_tail_validate.  A failed HIP launch returns HASTE_ERR_HIP.
 *     haste_last_error() gives a message for the calling thread's last
 *     failure.
 */
#ifndef HASTE_H
#define HASTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HASTE_ABI_VERSION 5

typedef enum {
    HASTE_OK = 0,
    HASTE_ERR_INVALID = 1,     /* null pointer, bad size, misalignment      */
    HASTE_ERR_UNSUPPORTED = 2, /* valid, but outside the implemented shapes */
    HASTE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than needed  */
    HASTE_ERR_HIP = 4          /* a HIP runtime / launch error               */
} haste_status;

typedef enum { HASTE_F32 = 0, HASTE_BF16 = 1 } haste_dtype;

/* Tail shape.  Supported: B >= 1, D >= F, F >= 1, L >= 1, G >= 1.
 * bf16 kernels additionally need G in {16, 32, 64}, F a multiple of 32 with
 * F <= 128 (F in {32, 64, 128}), D <= 1024; other shapes
 * return HASTE_ERR_UNSUPPORTED.  G = 1 (every label its own F indices: the
 * per-label fixed fan-in layout the HASTE page compares against, section
 * "Results") is taken in bf16 by haste_tail_fwd (logits and loss, no top-K,
 * D >= 16) and by haste_tail_step (loss, dW, dX; no top-K, not
 * HASTE_TAIL_LEAN, 16 <= D <= 960: its dz is kept label-major in the
 * workspace, L x B_pad bf16); the other bf16 tail calls return
 * HASTE_ERR_UNSUPPORTED for it.  fp32 accepts any G and F. */
typedef struct {
    int32_t B;      /* rows in the batch                    */
    int32_t D;      /* input feature width                  */
    int64_t L;      /* live tail labels                     */
    int32_t G;      /* labels per group                     */
    int32_t F;      /* fan-in indices per group             */
    int32_t dtype;  /* haste_dtype of X, W, Z, dZ, dW       */
    int32_t flags;  /* HASTE_TAIL_LEAN | HASTE_TAIL_LAYOUT_READY, or 0 */
} haste_tail_desc;

/* Tail flag.  By default the bf16 training calls that form dz from the
 * positives (haste_tail_step, its split form, haste_tail_bwd with dZ NULL)
 * keep dz of the dW pass in the workspace as bf16 tiles, B_pad x (N_g*G)
 * x 2 bytes (B_pad = B rounded up to 64), and the dX pass reads them back;
 * haste_tail_bwd with a given dZ first copies dZ into the same tiles, which
 * both of its passes then read.  The workspace size includes the tiles
 * whether or not bce is given.  HASTE_TAIL_LEAN drops that buffer: the dX
 * pass recomputes Z and dz from X, W and the positives (or reads the given
 * dZ in place), and nothing of size B x L is stored.  Both forms give the
 * same results up to the summation order of Z. */
#define HASTE_TAIL_LEAN 1

/* Tail flag.  The bf16 calls that form logits read every group's features in
 * an order chosen for the LDS banks (a permutation of idx[g], formed from idx
 * alone, kept in the workspace at an offset that depends on the shape only).
 * Without this flag every such call forms it first.  With it the call takes
 * it from the workspace as haste_tail_prepare_layout (or an earlier call on
 * the same workspace and idx) left it: for training with a fixed idx, form it
 * once.  Calling with the flag on a workspace that does not hold the order
 * of this idx gives wrong results. */
#define HASTE_TAIL_LAYOUT_READY 2

/* Head shape (dense classifier).  bf16 needs D a multiple of 32. */
typedef struct {
    int32_t B;
    int32_t D;
    int32_t H;
    int32_t dtype;
} haste_head_desc;

/* Sigmoid-BCE over sparse positives, fused into the logit epilogue.
 * Positives are one row-CSR list for the whole output space in GLOBAL label
 * ids (head labels [0, H), tail label t has id H + t); each call uses the
 * ids in [label_offset, label_offset + its label count) and ignores the
 * rest.  Ids must be unique within a row. */
typedef struct {
    const int32_t *row_ptr;   /* device, B+1 entries, row_ptr[0] = 0          */
    const int32_t *labels;    /* device, nnz entries, global label ids        */
    int32_t nnz;              /* host copy of row_ptr[B]                      */
    int32_t reserved0;
    int64_t label_offset;     /* global id of this branch's label 0           */
    float grad_scale;         /* s: dz = s*(sigmoid(z) - y); usually 1/B      */
    int32_t topk_buckets;     /* buckets per row, in [1, 2^24]; 0: the
                                 library's choice (only with K' = K)          */
    float *loss;              /* device fp32 scalar; this call ADDS its loss,
                                 or NULL for no loss                          */
    int32_t topk;             /* 0, or K in [1, 8]: per-row top-K logits (see
                                 below)                                       */
    int32_t topk_kprime;      /* 0: K' = K (exact); else K' in [1, topk]      */
    float *topk_val;          /* device B x K, descending                     */
    int32_t *topk_idx;        /* device B x K global ids; ties -> smaller id  */
} haste_bce;

/* Top-K (top-K page, section "Method": the top-K' of every bucket, then a
 * merge of the buckets' lists).  With topk = K > 0 the calls that form
 * logits -- haste_tail_fwd, haste_tail_step, haste_tail_step_dw,
 * haste_head_fwd, haste_head_step -- write to topk_val / topk_idx K logits of
 * every row over this call's labels (ids = label_offset + label), value
 * descending, ties to the smaller id, rows with fewer than K candidates
 * padded with (-inf, -1).  A bucket is a run of consecutive labels:
 * topk_buckets runs of ceil(labels / topk_buckets) (fewer if that leaves the
 * last ones empty).  With topk_kprime = 0 (K' = K) the result is the exact
 * top-K of the kernels' fp32 logits for any bucket count, and
 * topk_buckets = 0 lets the library pick one (about 1024 / B, at least one:
 * enough stage-1 workgroups over all rows).  With K' < K it is the page's
 * approximate two-stage top-K (a logit of the true top-K is missed when more
 * than K' of them share its bucket) and topk_buckets must be given;
 * haste_topk_plan picks K' and the bucket count for a recall target.  When
 * the buckets are exactly the tail's label groups (ceil(L / topk_buckets)
 * = G, bf16) and K' = 1, stage 1 runs inside the logits pass (the top-K
 * page's matmul-fused stage 1): the same result without the fp32 logits in
 * the workspace.  The exact top-K (K' = K) of a bf16 tail with G >= 16 runs
 * the same fused stage over the label groups, merges each row's K best
 * groups, and recomputes those K groups' logits bit for bit as the logits
 * pass forms them to keep the K best: the exact top-K of the kernels' fp32
 * logits (a label of the row's top K lies in one of its K best groups),
 * again without the fp32 logits.  The head's and the tail's lists combine with
 * haste_topk_merge.  The workspace then also holds the call's fp32 logits
 * (B x labels x 4 bytes) and the bucket lists (B x buckets x K' x 8 bytes),
 * or, for the fused forms, the per-group lists (N_g x B_pad x 8 bytes).
 * haste_tail_bwd and haste_head_bwd reject topk > 0; the other calls ignore
 * it.  Ids are int32: a call whose label_offset + labels - 1 exceeds
 * 2^31 - 1 returns HASTE_ERR_UNSUPPORTED when topk > 0. */

/* Expected recall of the two-stage top-K (top-K page, "Theoretical
 * analysis": the K largest of n items fall into the buckets as a uniformly
 * random placement, so the number in a bucket of m items is hypergeometric,
 * and a bucket contributes min(that number, K')).  Buckets as the calls form
 * them for `buckets` buckets.  Host only; returns the expected fraction of
 * the true top-K that the result holds, or -1 for invalid arguments (n < 1,
 * K outside [1, 8], K' outside [1, K], buckets < 1). */
double haste_topk_expected_recall(int64_t n, int K, int kprime, int64_t buckets);

/* Automatic parameter choice (top-K page, "automatic parameter selection"):
 * among K' in [1, K] and bucket counts in [min_buckets, min(n, 65535)], the
 * pair whose expected recall is at least `target` with the fewest stage-2
 * candidates buckets * K' (ties: the smaller K').  min_buckets is the least
 * number of buckets the caller wants for stage 1's parallelism (with 1 the
 * answer is always the exact K' = K over one bucket: K candidates).  Host
 * only.  out = {K', buckets}.  Returns HASTE_ERR_INVALID for bad arguments
 * (target outside (0, 1], min_buckets outside [1, min(n, 65535)]) and
 * HASTE_ERR_UNSUPPORTED when no pair reaches the target. */
haste_status haste_topk_plan(int64_t n, int K, double target, int64_t min_buckets, int32_t *out);

int haste_abi_version(void);
const char *haste_status_string(int status);
/* Message of the calling thread's last failed call ("" if none). */
const char *haste_last_error(void);

/* Storage of the tail (Method item 1, "memory efficiency": one index set per
 * group).  out (host, 4 entries) = { N_g, stored index count N_g*F,
 * stored weight rows N_g*G, live labels in the last group }. */
haste_status haste_tail_layout(const haste_tail_desc *d, int64_t *out);

/* Workspace bytes needed by the tail / head calls for this shape and BCE
 * setup (bce may be NULL).  Pass a 256-byte aligned device buffer at least
 * this large as `ws`.  haste_tail_fwd needs only
 * haste_tail_fwd_workspace_bytes (the training calls' dz tiles excluded; the
 * regions they share sit at the same offsets). */
size_t haste_tail_workspace_bytes(const haste_tail_desc *d, const haste_bce *bce);
size_t haste_tail_fwd_workspace_bytes(const haste_tail_desc *d, const haste_bce *bce);
size_t haste_head_workspace_bytes(const haste_head_desc *d, const haste_bce *bce);

/* Forms in ws the feature order of idx that the logits calls read with
 * HASTE_TAIL_LAYOUT_READY (see there).  ws: at least
 * haste_tail_fwd_workspace_bytes(d, NULL) bytes, the workspace the later
 * calls use.  Nothing to do for fp32 or G = 1 (returns HASTE_OK).  Errors as
 * for the compute calls; the order depends on idx alone, so it stays valid
 * until idx changes. */
haste_status haste_tail_prepare_layout(const haste_tail_desc *d, const int32_t *idx, void *ws,
                                       size_t ws_bytes, void *stream);

/* Tail forward (Method item 1: gather X[:, idx[g]] once per group into LDS,
 * then a dense per-group contraction).  Writes Z (B x L) if Z != NULL;
 * adds the BCE loss and writes the top-K if bce asks for them.  At least one
 * of Z, bce must be given. */
haste_status haste_tail_fwd(const haste_tail_desc *d, const void *X,
                            const int32_t *idx, const void *W, void *Z,
                            const haste_bce *bce, void *ws, size_t ws_bytes,
                            void *stream);

/* Tail backward (HASTE page, "Method" item 1: the exact gradients of the
 * group-shared layer; the pages print no formulas, the reading is that the
 * backward is the exact gradient of the forward: dW_g = dZ_g^T X_g, dX the
 * scatter-add of dZ_g W_g through idx[g]).  dW (same shape/dtype as W,
 * padded rows zeroed) and dX (B x D fp32; overwritten, or added to when
 * accumulate_dX != 0).
 * dZ != NULL: use the given B x L gradient.  dZ == NULL: recompute z and
 * dz = s*(sigmoid(z)-y) from bce (dz kept in ws between the dW and dX
 * passes unless HASTE_TAIL_LEAN; bce->loss is NOT added here, so a separate
 * forward can own the loss). */
haste_status haste_tail_bwd(const haste_tail_desc *d, const void *X,
                            const int32_t *idx, const void *W, const void *dZ,
                            const haste_bce *bce, void *dW, float *dX,
                            int accumulate_dX, void *ws, size_t ws_bytes,
                            void *stream);

/* Fused tail training step (HASTE page, "Method" item 1; the loss is the
 * sigmoid binary cross-entropy over the listed positives, summed over
 * labels and scaled by s, and the gradients are its exact ones): loss
 * (+= into bce->loss), dW and dX in one call; no logits are stored, and with HASTE_TAIL_LEAN no B x L buffer of
 * any kind (see HASTE_TAIL_LEAN). */
haste_status haste_tail_step(const haste_tail_desc *d, const void *X,
                             const int32_t *idx, const void *W,
                             const haste_bce *bce, void *dW, float *dX,
                             int accumulate_dX, void *ws, size_t ws_bytes,
                             void *stream);

/* Fused tail training step with the optimizer update in the dW pass's
 * epilogue (plain SGD, no momentum; the pages name no optimizer): as
 * haste_tail_step, but instead of dW it writes W_out = W - lr * dW, where
 * dW is rounded to bf16 as haste_tail_step would store it and the update is
 * one fp32 fma rounded to bf16 -- bit for bit what haste_sgd_update gives
 * after haste_tail_step, without the dW write and the second pass.  dX is
 * computed with the old W, so W_out must not overlap W (swap the two
 * buffers between steps); HASTE_ERR_INVALID if it does.  bf16 only (fp32:
 * HASTE_ERR_UNSUPPORTED).  Caller-owned W_out, 16-byte aligned, same shape
 * as W; padded rows get W's values. */
haste_status haste_tail_step_sgd(const haste_tail_desc *d, const void *X,
                                 const int32_t *idx, const void *W,
                                 const haste_bce *bce, float lr, void *W_out,
                                 float *dX, int accumulate_dX, void *ws,
                                 size_t ws_bytes, void *stream);

/* SGD update after a step (the unfused form): W_out[i] = W[i] - lr * dW[i]
 * for n elements of dtype (bf16: fp32 fma of the bf16 values, rounded to
 * bf16).  W_out may equal W (in place).  Asynchronous on `stream`. */
haste_status haste_sgd_update(int64_t n, int32_t dtype, const void *W,
                              const void *dW, float lr, void *W_out,
                              void *stream);

/* Split form of haste_tail_step, for callers that time or overlap its
 * parts.  haste_tail_prepare writes into ws the transposed X and the
 * group-major positives.  haste_tail_step_dw (one kernel) then adds the
 * loss and writes dW (gather + contraction + fused BCE + weight gradient);
 * haste_tail_step_dx (one kernel, plus a fill of dX unless accumulating)
 * adds the tail's dX.  Both read what haste_tail_prepare left in ws, and
 * unless HASTE_TAIL_LEAN haste_tail_step_dx also reads the dz tiles that
 * haste_tail_step_dw left there: call the three on one stream, in this
 * order, with the same descriptor, X, idx, W, bce and workspace; together
 * they produce what haste_tail_step produces.  ws must not be reused by
 * another call in between. */
haste_status haste_tail_prepare(const haste_tail_desc *d, const void *X,
                                const haste_bce *bce, void *ws,
                                size_t ws_bytes, void *stream);
haste_status haste_tail_step_dw(const haste_tail_desc *d, const void *X,
                                const int32_t *idx, const void *W,
                                const haste_bce *bce, void *dW, void *ws,
                                size_t ws_bytes, void *stream);
haste_status haste_tail_step_dx(const haste_tail_desc *d, const void *X,
                                const int32_t *idx, const void *W,
                                const haste_bce *bce, float *dX,
                                int accumulate_dX, void *ws, size_t ws_bytes,
                                void *stream);

/* Head forward (Method item 2: dense classifier).  Zh (B x H) and/or the
 * fused BCE (loss, top-K). */
haste_status haste_head_fwd(const haste_head_desc *d, const void *X,
                            const void *Wh, void *Zh, const haste_bce *bce,
                            void *ws, size_t ws_bytes, void *stream);

/* Head backward (HASTE page, "Method" item 2: the dense classifier over the
 * frequent labels; exact gradients dWh = dZh^T X, dX += dZh Wh): dWh (H x D,
 * dtype) and dX (B x D fp32, overwritten or accumulated).  dZh != NULL uses it; NULL recomputes from bce. */
haste_status haste_head_bwd(const haste_head_desc *d, const void *X,
                            const void *Wh, const void *dZh,
                            const haste_bce *bce, void *dWh, float *dX,
                            int accumulate_dX, void *ws, size_t ws_bytes,
                            void *stream);

/* Fused head step (HASTE page, "Method" item 2, with the same loss as the
 * tail's): loss (+=), top-K (if asked), dWh, dX. */
haste_status haste_head_step(const haste_head_desc *d, const void *X,
                             const void *Wh, const haste_bce *bce, void *dWh,
                             float *dX, int accumulate_dX, void *ws,
                             size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same as
 * haste_head_step, but its workspace is a static device array of the library,
 * HASTE_HEAD_SCRATCH_BYTES per GPU, held by each GPU the library runs on
 * from module load until the process ends; the call allocates nothing.  The
 * caller still passes every input and output.  HASTE_ERR_WORKSPACE when the
 * step needs more than the array (haste_head_workspace_bytes(d, bce) >
 * HASTE_HEAD_SCRATCH_BYTES).  Every call on one GPU uses that GPU's one
 * array and keeps nothing in it for the next: calls that overlap on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Other errors as haste_head_step. */
#define HASTE_HEAD_SCRATCH_BYTES ((size_t)64 << 20)
haste_status haste_head_step_noalloc(const haste_head_desc *d, const void *X,
                                     const void *Wh, const haste_bce *bce,
                                     void *dWh, float *dX, int accumulate_dX,
                                     void *stream);

/* Group-major view of the tail positives (the list the fused epilogue
 * walks; the positives are the labels y = 1 of the sigmoid-BCE, and the
 * order is fixed so that it can be compared bit for bit): grp_ptr (N_g + 1 entries) and entries (<= nnz), entry = b*G + j,
 * ordered by group, then row b, then slot j.  Deterministic. */
haste_status haste_tail_group_positives(const haste_tail_desc *d,
                                        const haste_bce *bce, int32_t *grp_ptr,
                                        int32_t *entries, void *ws,
                                        size_t ws_bytes, void *stream);

/* Index check (HASTE page, "Method" item 1: one set of F distinct input
 * features per group; the reading here is that each set is stored sorted,
 * strictly increasing, inside [0, D)): writes to *first_bad_group (a DEVICE
 * int32, so the call stays asynchronous) the smallest group whose row of idx
 * breaks that, or -1. */
haste_status haste_tail_validate(const haste_tail_desc *d, const int32_t *idx,
                                 int32_t *first_bad_group, void *stream);

/* Dynamic rewiring of the tail's fan-in sets: one prune-and-regrow step of
 * every group (HASTE page: the title's dynamic sparse training; "Method"
 * item 1, "Structure": one fan-in set per group, own weights per label).
 * The page gives no rule; this call applies the plainest one at group
 * granularity:
 *   - position f of group g scores the L1 norm of its weight column over the
 *     group's live labels, sum_{j < min(G, L - gG)} |W[gG+j][f]|, added in
 *     fp32 in ascending j;
 *   - the k_prune positions first in (score, feature id) order are pruned;
 *   - k_prune features outside the kept set are regrown: cand[g][0..n_cand)
 *     in order (the caller's random draws; values outside [0, D), kept
 *     features and repeats are skipped, a feature pruned by this call may
 *     come back), then the smallest features left;
 *   - idx_out[g] is the new set, ascending; in W_out a kept feature's column
 *     is its column of W (every row of the group, padded rows too) and a
 *     regrown feature's column is zero.
 * idx: N_g x F int32, each row valid (strictly increasing in [0, D); see
 * haste_tail_validate); W, W_out: (N_g*G) x F of d->dtype; cand: N_g x n_cand
 * int32 (may be NULL when n_cand = 0); idx_out: N_g x F int32.  idx_out and
 * W_out may be idx and W (in place) but must not overlap them otherwise.
 * d->B and d->flags are not used.  After a rewiring, a feature order formed
 * for HASTE_TAIL_LAYOUT_READY belongs to the old idx: form it again.
 * Supported: G <= 64, F <= 256, D <= 65536.  Errors: HASTE_ERR_INVALID
 * (NULL or misaligned pointers, sizes < 1, F > D, k_prune outside [0, F],
 * n_cand < 0, partial overlap), HASTE_ERR_UNSUPPORTED (G > 64, F > 256,
 * D > 65536), HASTE_ERR_HIP.  Asynchronous on `stream`. */
haste_status haste_tail_rewire(const haste_tail_desc *d, const int32_t *idx,
                               const void *W, int32_t k_prune,
                               const int32_t *cand, int32_t n_cand,
                               int32_t *idx_out, void *W_out, void *stream);

/* Merge two per-row top-K lists (e.g. head and tail) into one: B x K each,
 * descending, ties broken toward the smaller id (second stage of the
 * two-stage top-K on the top-K page, with K' = K so the result is exact). */
haste_status haste_topk_merge(int32_t B, int32_t K, const float *a_val,
                              const int32_t *a_idx, const float *b_val,
                              const int32_t *b_idx, float *out_val,
                              int32_t *out_idx, void *stream);

/* Measurement utility, not a step of the layer: `blocks` workgroups of four
 * waves each run `iters` rounds of 16 independent 16x16x32 bf16 MFMA
 * accumulations on register operands (16*16*32*2 flops each; 4 * 16 * iters
 * per workgroup), with no memory traffic.  Timed by the caller, the rate is
 * the matrix cores' attainable bf16 peak.  sink: one device float, 4-byte
 * aligned, caller-owned, written only if the sum of the accumulators happens
 * to equal 12345 (that test keeps the loop).  Errors:
 * HASTE_ERR_INVALID for blocks < 1, iters < 1 or a NULL / misaligned sink;
 * HASTE_ERR_HIP for a failed launch.  Asynchronous on `stream`. */
haste_status haste_probe_mfma(int blocks, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* HASTE_H */
